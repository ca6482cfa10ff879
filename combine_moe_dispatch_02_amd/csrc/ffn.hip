// A3 + A4 -- the expert FFN as a persistent grouped GEMM on CDNA4 MFMA.
//
// StreamEP README, "How it works": the forward grouped GEMMs "A" and "Y" read
// the pool as it stands (dispatch's output is their input) and claim pool
// tiles as dispatch signals them. Reading taken for the math the page leaves
// open: w1[e] is [2I, H] with gate rows first, h = silu(gate) * up with
// silu(z) = z / (1 + exp(-z)), y = h . w2[e]^T, fp32 accumulation.
//
// Work unit = (pool tile m, N block j): a BM x BN output block of one expert
// (BM = pool tile, so a unit never spans two experts). GEMM A's unit takes BN/2
// gate rows and the matching BN/2 up rows of w1, so SwiGLU happens in the
// registers of the lanes that hold both accumulators. A persistent grid walks
// the units; GEMM A waits (acquire) until its tile's ready flag equals the
// epoch of the dispatch call.
//
// Two kernels, one K step = 128 bytes of each row (64 bf16 or 128 e4m3 / e2m1 pairs):
//  * ffn_gemm_kernel (4 waves, any BN of 128/256, row-major weights): A and B tiles
//    through a double-buffered LDS, loaded one step ahead via registers; one
//    barrier per step. fp8 there: each block's product leaves the MFMA on its own
//    (zero accumulator input), then acc += product * a_scale[row] * b_scale[block].
//  * ffn_big_kernel (8 waves, BM x 512 units, each wave BM x 64): the weights
//    stream straight into registers one step ahead (the MFMA-tiled layout of
//    moe_pack_weights makes each 16-byte lane load part of 1 KiB of contiguous
//    memory); the pool rows come through LDS, either two stages loaded through
//    registers (bf16) or by LDS-DMA (fp8), or a four-stage LDS-DMA ring three steps
//    ahead (bf16, mxfp4); the output leaves through LDS in whole row segments. fp8
//    there keeps acc in units of the current block's scales and rescales it by
//    old / new before each block's MFMAs.
// LDS rows are 128 bytes, 16-byte chunks XOR-swizzled by (row & 7), so the 8
// lanes that read one chunk column from 8 consecutive rows hit 8 different
// bank groups.
// bf16: v_mfma_f32_16x16x32_bf16, A/B fragments = 8 consecutive K values of one
// row per lane (lane l: row l%16, K chunk l/16).
// fp8: v_mfma_scale_f32_16x16x128_f8f6f4 with unit scales (E8M0 127), one per
// 128-wide K block.
// mxfp4: the same instruction with e2m1 weights (format 4) and e4m3 activations,
// its per-lane E8M0 operands carrying the 1x32 block scales of both sides.
#include <algorithm>
#include <type_traits>

#include "combine.h"
#include "common.h"
#include "ffn_sq.h"
#include "kernels.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x8_t __attribute__((ext_vector_type(8)));

struct FfnArgs {
  const uint8_t* A;          // pool (GEMM A) or h (GEMM Y): [rows][Kdim] elements
  const float* A_s;          // fp8: activation group scales, tile-major words (scale_word)
  const uint8_t* B;          // w1 or w2, expert-major
  const float* B_s;          // fp8: weight block scales, expert-major
  uint8_t* out;              // h (GEMM A) or y_pool (GEMM Y)
  float* out_s;              // fp8 GEMM A: h group scales, tile-major words
  int32_t ksteps;            // K steps of 128 bytes
  int64_t lda;               // bytes per A row
  int64_t b_expert;          // bytes per expert of B
  int64_t ldb;               // bytes per B row
  int32_t up_row0;           // GEMM A: first up row of w1 (= I)
  int64_t ldo;               // bytes per out row
  int32_t n_units;           // N blocks per tile
  int32_t s_kblocks;         // fp8, mxfp4: Kdim / 128 (scale words per row)
  int32_t bs_ld;             // fp8: B scale row stride (= Kdim / 128)
  int64_t bs_expert;         // fp8: B scale entries per expert
  int32_t out_groups;        // fp8 GEMM A: I / 128
  int32_t ktiles;            // tiled weights: K tiles per 16-row block (K/32 bf16, K/128 fp8)
  int32_t tile_shift;
  int32_t max_tiles;         // pool_rows / tile: tiles the buffers hold
  int32_t unit_order;        // 1: tile-major (m, j); 2: expert, N block, tile; 3: expert, N pair, tile
  int32_t n_experts;
  const int32_t* offsets;
  const int32_t* num_tiles;
  const int32_t* tile_expert;
  const uint32_t* tile_ready;
  uint32_t epoch;
  uint32_t* err;
  uint32_t* abort_epoch;     // epoch of a call whose ready-flag wait timed out (its other waits end)
  uint64_t timeout;
  int32_t wait_ready;
  // dispatch's count of raised ready flags (reset by the plan), or null: when it already
  // equals the tile count as the big-tile kernel starts, one acquire covers every tile
  const uint32_t* tiles_done;
  const uint8_t* A_e8;       // mxfp4: activation E8M0 scales, tile-major 4-byte words
  const uint8_t* B_e8;       // mxfp4: weight E8M0 scales in tile order, expert-major
  uint8_t* out_e8;           // mxfp4 GEMM A: h E8M0 scales, tile-major 4-byte words
  int64_t b_e8_expert;       // mxfp4: bytes per expert of B_e8
  // combine on completion (GEMM Y on the big-tile kernel; null ydone = off)
  uint32_t* ydone;           // per tile: GEMM Y units finished (GEMM A zeroes them)
  uint32_t* cq;              // next combine item to claim (GEMM A zeroes it)
  const int32_t* pos;        // plan: pool row of pair t*K+k
  const float* topk_w;       // [T][K]
  uint8_t* comb_out;         // out [T][H] bf16
  int32_t T, K;
  int32_t pool_rows;
  // training: GEMM A stores G = [gate | up] (bf16 [rows][2I]) before the activation;
  // the backward GEMM Y's SwiGLU-backward epilogue reads G there and writes dG over it
  uint8_t* g_save;
  int64_t g_ld;              // bytes per row of g_save (2I * 2)
  int32_t a_stages;          // 2: two A stages; else the four-stage ring where the kernel has it
  int32_t select;            // GEMM A, 1: return at once if the 256-row units win (sel)
  SqSelect sel;
};

__device__ inline uint32_t swz(int row, int chunk) { return (uint32_t)(row * 128 + ((chunk ^ (row & 7)) << 4)); }

// silu(g) * u with the hardware reciprocal (about 1 ulp) in place of a division
__device__ inline float silu_mul(float g, float u) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u; }

// ----------------------------------------------------------------------------
// Unit schedule shared by the kernels
// ----------------------------------------------------------------------------
// Unit u -> (pool tile m, N block j). Order 1 walks tiles, N blocks inside a
// tile (the pool tile is reused from L2 by its N blocks). Order 2 walks
// experts, then N blocks, then the expert's tiles, so units that run together
// stream the same weight panel. Order k >= 3 walks experts, then groups of k-1 N
// blocks, then the expert's tiles with the group's blocks back to back (order 3:
// pairs). Persistent workgroups are dealt to XCDs
// round-robin by the dispatcher (workgroup g runs on XCD g % 8), so slot(g)
// gives each XCD a contiguous run of units and its L2 sees the shared panel.
// units of a big-tile workgroup whose coordinates are found up front (later ones one by one)
constexpr int kBigUnitSlots = 64;

__device__ inline void unit_coords(const FfnArgs& a, int u, int order, int& m, int& j) {
  if (order == 1) {
    m = u / a.n_units;
    j = u - m * a.n_units;
    return;
  }
  int lo = 0, hi = a.n_experts - 1;
  while (lo < hi) {  // largest e whose first unit is <= u (empty experts share a start)
    const int mid = (lo + hi + 1) >> 1;
    if ((a.offsets[mid] >> a.tile_shift) * a.n_units <= u) lo = mid;
    else hi = mid - 1;
  }
  const int t0 = a.offsets[lo] >> a.tile_shift;
  const int te = (a.offsets[lo + 1] >> a.tile_shift) - t0;
  const int local = u - t0 * a.n_units;
  const int g = order - 1;  // order >= 3: N blocks in groups of order - 1
  if (order == 2 || a.n_units % g != 0) {
    j = local / te;
    m = t0 + (local - j * te);
  } else {
    // N blocks in groups of g, every tile of the expert inside a group, the group's
    // blocks back to back; with g = 2 (the default) a run of 32 units holds ~16
    // tiles x 2 weight panels
    const int jp = local / (g * te);
    const int r = local - jp * g * te;
    m = t0 + r / g;
    j = g * jp + (r - (r / g) * g);
  }
}


// wait until tile m's ready flag equals the epoch; false when the unit is skipped.
// A wait that times out records MOE_ERR_TIMEOUT and marks this call's epoch aborted,
// which ends the other waits of the same call at once; a later call (another epoch)
// is not affected by it, whether or not the error word has been read since.
__device__ inline bool wait_tile_ready(const FfnArgs& a, int m, int* s_go) {
  if (threadIdx.x == 0) {
    int go = 1;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while (__hip_atomic_load(&a.tile_ready[m], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != a.epoch) {
      if (__hip_atomic_load(a.abort_epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == a.epoch) {
        go = 0;
        break;
      }
      if (__builtin_amdgcn_s_memrealtime() - t0 > a.timeout) {
        record_error(a.err, MOE_ERR_TIMEOUT);
        __hip_atomic_store(a.abort_epoch, a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        go = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(4);
    }
    *s_go = go;
  }
  __syncthreads();
  const int go = *s_go;
  __syncthreads();  // s_go is rewritten for the next unit only after everyone read it
  if (go) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return go != 0;
}


template <int BM, int BN, int WM, int WN, bool FP8, bool GEMM_A>
struct Gemm {
  static constexpr int kWTM = BM / WM;
  static constexpr int kWTN = BN / WN;
  static constexpr int kTM = kWTM / 16;
  static constexpr int kTN = kWTN / 16;
  static constexpr int kABytes = BM * 128;
  static constexpr int kBBytes = BN * 128;
  static constexpr int kStage = kABytes + kBBytes;
  static constexpr int kAChunks = BM * 8;
  static constexpr int kBChunks = BN * 8;
  static constexpr int kALoads = (kAChunks + 255) / 256;
  static constexpr int kBLoads = kBChunks / 256;
  static_assert(WM * WN == 4, "four waves");
  static_assert(kTN % 2 == 0, "each wave holds matched halves of its columns");
  static_assert(kBChunks % 256 == 0, "B tile loads");
  static_assert(!FP8 || (GEMM_A ? BN == 256 : BN % 256 == 0 || BN == 128), "fp8 scale blocks");

  // local B row (0..BN) of MFMA tile tn's first column for wave column wn
  __device__ static inline int brow(int wn, int tn) {
    return tn < kTN / 2 ? wn * (kWTN / 2) + tn * 16 : BN / 2 + wn * (kWTN / 2) + (tn - kTN / 2) * 16;
  }
};

template <int BM, int BN, int WM, int WN, bool FP8, bool GEMM_A>
__global__ __launch_bounds__(256, 1) void ffn_gemm_kernel(FfnArgs a) {
  using G = Gemm<BM, BN, WM, WN, FP8, GEMM_A>;
  __shared__ __attribute__((aligned(16))) uint8_t s_tile[2][G::kStage];
  __shared__ float s_as[2][FP8 ? BM : 1];
  __shared__ float s_red[FP8 && GEMM_A ? WN : 1][FP8 && GEMM_A ? BM : 1];
  __shared__ int s_go;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN;
  const int wn = wave % WN;
  const int l16 = lane & 15;
  const int lhi = lane >> 4;

  int ntiles = a.num_tiles[0];
  if (ntiles > a.max_tiles) {
    // the plan needs more rows than the pool holds: compute what fits, report the rest
    if (blockIdx.x == 0 && tid == 0) record_error(a.err, MOE_ERR_INVALID);
    ntiles = a.max_tiles;
  }
  const int total = ntiles * a.n_units;
  if (GEMM_A && a.cq != nullptr && blockIdx.x == 0 && tid == 0) *a.cq = 0u;
  for (int u = blockIdx.x; u < total; u += gridDim.x) {
    const int m = u / a.n_units;
    const int j = u - m * a.n_units;
    const int m0 = m * BM;
    const int e = a.tile_expert[m];

    if (a.wait_ready && !wait_tile_ready(a, m, &s_go)) continue;
    if (GEMM_A && a.ydone != nullptr && j == 0 && tid == 0) a.ydone[m] = 0u;  // for GEMM Y's combine

    // sources of this unit
    const uint8_t* Arow0 = a.A + (int64_t)m0 * a.lda;
    const uint8_t* Bexp = a.B + (int64_t)e * a.b_expert;
    // global row of B for local row r
    auto b_global_row = [&](int r) -> int64_t {
      if constexpr (GEMM_A)
        return r < BN / 2 ? (int64_t)j * (BN / 2) + r : (int64_t)a.up_row0 + j * (BN / 2) + (r - BN / 2);
      else
        return (int64_t)j * BN + r;
    };

    u32x4 ra[G::kALoads];
    u32x4 rb[G::kBLoads];
    float ras = 0.f;

    auto load_stage = [&](int kt) {
#pragma unroll
      for (int i = 0; i < G::kALoads; ++i) {
        const int c = tid + i * 256;
        if (c < G::kAChunks) {
          const int r = c >> 3, ch = c & 7;
          ra[i] = *reinterpret_cast<const u32x4*>(Arow0 + (int64_t)r * a.lda + kt * 128 + ch * 16);
        }
      }
#pragma unroll
      for (int i = 0; i < G::kBLoads; ++i) {
        const int c = tid + i * 256;
        const int r = c >> 3, ch = c & 7;
        rb[i] = *reinterpret_cast<const u32x4*>(Bexp + b_global_row(r) * a.ldb + kt * 128 + ch * 16);
      }
      if constexpr (FP8) {
        if (tid < BM) ras = a.A_s[((int64_t)m * a.s_kblocks + kt) * BM + tid];
      }
    };
    auto store_stage = [&](int buf) {
      uint8_t* sa = s_tile[buf];
      uint8_t* sb = s_tile[buf] + G::kABytes;
#pragma unroll
      for (int i = 0; i < G::kALoads; ++i) {
        const int c = tid + i * 256;
        if (c < G::kAChunks) *reinterpret_cast<u32x4*>(sa + swz(c >> 3, c & 7)) = ra[i];
      }
#pragma unroll
      for (int i = 0; i < G::kBLoads; ++i) {
        const int c = tid + i * 256;
        *reinterpret_cast<u32x4*>(sb + swz(c >> 3, c & 7)) = rb[i];
      }
      if constexpr (FP8) {
        if (tid < BM) s_as[buf][tid] = ras;
      }
    };

    f32x4_t acc[G::kTM][G::kTN];
#pragma unroll
    for (int i = 0; i < G::kTM; ++i)
#pragma unroll
      for (int k = 0; k < G::kTN; ++k) acc[i][k] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    load_stage(0);
    store_stage(0);
    __syncthreads();

    for (int kt = 0; kt < a.ksteps; ++kt) {
      const int buf = kt & 1;
      if (kt + 1 < a.ksteps) load_stage(kt + 1);
      const uint8_t* sa = s_tile[buf];
      const uint8_t* sb = s_tile[buf] + G::kABytes;
      if constexpr (!FP8) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          bf16x8_t fa[G::kTM], fb[G::kTN];
#pragma unroll
          for (int tm = 0; tm < G::kTM; ++tm) {
            const int r = wm * G::kWTM + tm * 16 + l16;
            fa[tm] = *reinterpret_cast<const bf16x8_t*>(sa + swz(r, kk * 4 + lhi));
          }
#pragma unroll
          for (int tn = 0; tn < G::kTN; ++tn) {
            const int r = G::brow(wn, tn) + l16;
            fb[tn] = *reinterpret_cast<const bf16x8_t*>(sb + swz(r, kk * 4 + lhi));
          }
#pragma unroll
          for (int tm = 0; tm < G::kTM; ++tm)
#pragma unroll
            for (int tn = 0; tn < G::kTN; ++tn)
              acc[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[tm], fb[tn], acc[tm][tn], 0, 0, 0);
        }
      } else {
        // per-tile B block scales (uniform): the two column halves of this wave
        const float* bs = a.B_s + (int64_t)e * a.bs_expert;
        const float sb0 = bs[(b_global_row(G::brow(wn, 0)) >> 7) * a.bs_ld + kt];
        const float sb1 = bs[(b_global_row(G::brow(wn, G::kTN / 2)) >> 7) * a.bs_ld + kt];
        i32x8_t fa[G::kTM], fb[G::kTN];
#pragma unroll
        for (int tm = 0; tm < G::kTM; ++tm) {
          const int r = wm * G::kWTM + tm * 16 + l16;
          const u32x4 lo = *reinterpret_cast<const u32x4*>(sa + swz(r, 2 * lhi));
          const u32x4 hi = *reinterpret_cast<const u32x4*>(sa + swz(r, 2 * lhi + 1));
          fa[tm] = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
#pragma unroll
        for (int tn = 0; tn < G::kTN; ++tn) {
          const int r = G::brow(wn, tn) + l16;
          const u32x4 lo = *reinterpret_cast<const u32x4*>(sb + swz(r, 2 * lhi));
          const u32x4 hi = *reinterpret_cast<const u32x4*>(sb + swz(r, 2 * lhi + 1));
          fb[tn] = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
#pragma unroll
        for (int tm = 0; tm < G::kTM; ++tm) {
          float sa4[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) sa4[i] = s_as[buf][wm * G::kWTM + tm * 16 + lhi * 4 + i];
#pragma unroll
          for (int tn = 0; tn < G::kTN; ++tn) {
            const f32x4_t part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                fa[tm], fb[tn], f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
            const float sbt = tn < G::kTN / 2 ? sb0 : sb1;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[tm][tn][i] += part[i] * (sa4[i] * sbt);
          }
        }
      }
      if (kt + 1 < a.ksteps) store_stage(buf ^ 1);
      __syncthreads();
    }

    // ---------------- epilogue ----------------
    if constexpr (GEMM_A) {
      const int hcol0 = j * (BN / 2) + wn * (G::kWTN / 2);
      if constexpr (!FP8) {
#pragma unroll
        for (int tm = 0; tm < G::kTM; ++tm)
#pragma unroll
          for (int tn = 0; tn < G::kTN / 2; ++tn)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float h = silu_mul(acc[tm][tn][i], acc[tm][tn + G::kTN / 2][i]);
              const int row = m0 + wm * G::kWTM + tm * 16 + lhi * 4 + i;
              const int col = hcol0 + tn * 16 + l16;
              *reinterpret_cast<__bf16*>(a.out + (int64_t)row * a.ldo + col * 2) = (__bf16)h;
            }
      } else {
        float hv[G::kTM][G::kTN / 2][4];
        float rmax[G::kTM][4];
#pragma unroll
        for (int tm = 0; tm < G::kTM; ++tm)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float mx = 0.f;
#pragma unroll
            for (int tn = 0; tn < G::kTN / 2; ++tn) {
              const float h = silu_mul(acc[tm][tn][i], acc[tm][tn + G::kTN / 2][i]);
              hv[tm][tn][i] = h;
              mx = fmaxf(mx, fabsf(h));
            }
            rmax[tm][i] = row16_max(mx);
          }
        if (l16 == 0) {
#pragma unroll
          for (int tm = 0; tm < G::kTM; ++tm)
#pragma unroll
            for (int i = 0; i < 4; ++i) s_red[wn][wm * G::kWTM + tm * 16 + lhi * 4 + i] = rmax[tm][i];
        }
        __syncthreads();
#pragma unroll
        for (int tm = 0; tm < G::kTM; ++tm)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int rl = wm * G::kWTM + tm * 16 + lhi * 4 + i;
            float mx = 0.f;
#pragma unroll
            for (int w2 = 0; w2 < WN; ++w2) mx = fmaxf(mx, s_red[w2][rl]);
            const float sc = mx > 0.f ? mx / 448.0f : 1.0f;
            const float inv = 1.0f / sc;  // h codes: h * (1/scale), one division per row
            const int row = m0 + rl;
#pragma unroll
            for (int tn = 0; tn < G::kTN / 2; ++tn) {
              const int col = hcol0 + tn * 16 + l16;
              a.out[(int64_t)row * a.ldo + col] = (uint8_t)e4m3_from_f32(hv[tm][tn][i] * inv);
            }
            if (wn == 0 && l16 == 0) a.out_s[((int64_t)m * a.out_groups + ((j * (BN / 2)) >> 7)) * BM + rl] = sc;
          }
        __syncthreads();
      }
    } else {
#pragma unroll
      for (int tm = 0; tm < G::kTM; ++tm)
#pragma unroll
        for (int tn = 0; tn < G::kTN; ++tn)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = m0 + wm * G::kWTM + tm * 16 + lhi * 4 + i;
            const int col = j * BN + G::brow(wn, tn) + l16;
            *reinterpret_cast<__bf16*>(a.out + (int64_t)row * a.ldo + col * 2) = (__bf16)acc[tm][tn][i];
          }
    }
  }
}

// ----------------------------------------------------------------------------
// Big-tile kernel: BM x 512 output per workgroup, NW waves of BM x (512/NW).
//   A (the pool tile or h, shared by all waves) is loaded two K steps ahead
//   into registers and goes through a two-stage LDS ring; B (weights: each
//   wave owns 512/NW output columns that no other wave reads) streams from
//   global memory straight into registers, already in MFMA fragment layout,
//   one K step ahead of the one being multiplied. (A is the stream that misses
//   L2 -- a pool tile is used by one unit per N block, far apart in time --
//   while a weight panel is shared by the units running side by side on an XCD.)
//   A K step is 128 bytes of a row: 64 bf16 (two 16x16x32 MFMAs per tile) or
//   128 e4m3 (one 16x16x128 MFMA per tile = one scale block). In fp8 the
//   accumulator is kept in units of the current block's scale a_s[row] *
//   b_s[block]: each block first rescales it by old/new scale, then the MFMA
//   accumulates the block's code product in place; the epilogue applies the
//   last scale. (No second set of partial-sum registers.) The kernel is
//   used when the K extents are whole pairs of steps, so every step issues
//   the same loads and the compiler's load counters stay exact.
//   The MFMA runs transposed (weight fragment first), so a lane holds one
//   output row and 4 consecutive output columns: 8-byte stores, one fp8 row
//   scale per lane. (Staging the block through LDS for full-line stores was
//   measured slower: its barriers cost more than the partial lines.)
// ----------------------------------------------------------------------------
template <int BM, int NW, bool FP8, bool GEMM_A>
struct Big {
  static constexpr int kThreads = 64 * NW;
  static constexpr int kBN = 512;
  static constexpr int kWCols = kBN / NW;       // output columns per wave
  static constexpr int kHalf = kWCols / 2;      // gate (or first-half) columns per wave
  static constexpr int kTN = kWCols / 16;       // 16-wide tiles per wave
  static constexpr int kTM = BM / 16;
  static constexpr int kKB = 128;               // bytes of a row per K step
  static constexpr int kCH = 8;                 // 16-byte chunks of a row per K step
  static constexpr int kKS = FP8 ? 1 : 2;       // MFMAs per tile per K step
  static constexpr int kAStage = BM * kKB;
  static constexpr int kAChunks = BM * kCH;
  static constexpr int kALoads = (kAChunks + kThreads - 1) / kThreads;
};

// Combine on completion (StreamEP README, "How it works": a token's combine need not
// wait for the whole FFN, only for the expert outputs it reads). After its last GEMM Y unit, a workgroup claims
// items of one token per wave from a device-wide counter. A wave waits until every
// pool tile holding one of its token's pairs has all its GEMM Y units counted (an
// acquire after the counts), then does the token's weighted gather-sum exactly as
// the combine kernel does. Items are claimed only after the claimer's own units,
// and a unit never waits, so the waits end whenever the grid's workgroups can all be
// resident at once (the launch keeps the grid at or below the CU count). A wait that
// outlasts the timeout records MOE_ERR_TIMEOUT and writes the token's row as zeros.
__device__ inline void combine_tail(const FfnArgs& a, int* s_item) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int nw = blockDim.x >> 6;
  const int items = (a.T + nw - 1) / nw;
  const int H = (int)(a.ldo >> 1);
  const uint32_t target = (uint32_t)a.n_units;
  for (;;) {
    __syncthreads();
    if (tid == 0) *s_item = (int)__hip_atomic_fetch_add(a.cq, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int item = *s_item;
    if (item >= items) break;
    const int t = item * nw + (tid >> 6);
    if (t >= a.T) continue;
    const int64_t pair0 = (int64_t)t * a.K;
    int p = lane < a.K ? a.pos[pair0 + lane] : -1;
    if (p >= a.pool_rows) p = -1;  // past the allocation: dispatch has reported it
    const float wt = lane < a.K ? a.topk_w[pair0 + lane] : 0.f;
    uint64_t have = ballot(p >= 0);
    if (have != 0) {
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      for (;;) {
        const bool done =
            p < 0 || __hip_atomic_load(&a.ydone[p >> a.tile_shift], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target;
        if (ballot(!done) == 0) break;
        if (__builtin_amdgcn_s_memrealtime() - t0 > a.timeout) {
          if (lane == 0) record_error(a.err, MOE_ERR_TIMEOUT);
          have = 0;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    uint8_t* orow = a.comb_out + (int64_t)t * H * 2;
    if (a.K <= 8)
      combine_token_wide<2, 8>(a.out, p, wt, have, a.K, H, orow, lane);
    else
      combine_token<4>(a.out, p, wt, have, a.K, H, orow, lane);
  }
}


// Slot of chunk c of pool row r in an A stage (128-byte rows). bf16 (16-byte fragment
// reads): the chunk moves by r % 8, so 8 consecutive rows reading one chunk column hit 8
// distinct 16-byte bank groups. fp8 / mxfp4 (32-byte fragment reads, two chunks per lane):
// rows r and r + 8 also differ in the slot's low bit -- with r % 8 alone these reads spent
// 9-11% of CU cycles in bank conflicts, and the extra bit gives the bf16 reads 11-17%.
template <bool FP8>
__device__ inline uint32_t swz_a(int r, int c) {
  return (uint32_t)(r * 128 + ((c ^ (r & 7) ^ (FP8 ? (r >> 3) & 1 : 0)) << 4));
}

// MX (mxfp4): A is MXFP8 (e4m3 rows as in fp8, plus one E8M0 byte per 32 K), B is
// tiled MXFP4 (a 16 x 128 tile = 1 KiB, lane l's 16 bytes = 32 consecutive K of
// row l%16) with its E8M0 bytes in tile order (64 per tile, byte l = lane l's).
// The scaled MFMA takes, per lane, the scale of its row and of K block l/16 of the
// step, and pairs K [16b, 16b+16) + [64+16b, 64+16b+16) of an e4m3 operand lane
// block b with K [32b, 32b+32) of an e2m1 one: A fragments are therefore 16-byte
// chunks b and b+4 of the row's 128-byte step.
// EPI (GEMM Y only): 0 stores y; 1 is the backward GEMM Y's epilogue -- the product
// is dh, and with g, u from G it writes dG = [dh u silu'(g) | dh silu(g)] in place of G.
// RING (K steps a multiple of 4; used for bf16 and mxfp4): the pool rows come by LDS-DMA
// into a ring of four stages, three K steps ahead (registers hold none of them), instead
// of two stages (bf16: through registers, two steps ahead; fp8 / mxfp4: by LDS-DMA, one
// step ahead). The activation scales of fp8 / mxfp4 stay one step ahead, in two stages. The stages are separate LDS objects used with
// constant indices (the loop runs four steps per round), so the compiler can tell a
// step's reads from the DMA writes in flight and adds no wait of its own; each step ends
// with a vmcnt wait that leaves the two newer steps' DMAs outstanding and a bare barrier.
template <int BM, int NW, bool FP8, bool GEMM_A, bool PACKED, bool MX = false, int EPI = 0, bool RING = false>
__global__ __launch_bounds__(64 * NW, 1) void ffn_big_kernel(FfnArgs a) {
  static_assert(EPI == 0 || (!GEMM_A && !FP8), "the SwiGLU-backward epilogue is a bf16 GEMM Y one");
  static_assert(!MX || (FP8 && PACKED), "mxfp4 runs on the tiled e4m3 path");
  using C = Big<BM, NW, FP8, GEMM_A>;
  constexpr int TN = C::kTN, TM = C::kTM, KS = C::kKS, HALF = C::kHalf;
  static_assert(!MX || (TM >= TN && HALF % 32 == 0), "mxfp4 step and h block layout");
  // A stages: s_a for the register-staged bf16 path; separate objects s_r0..s_r3 where
  // A arrives by LDS-DMA (fp8 / mxfp4 use two of them, the bf16 ring four), so that the
  // compiler can tell a step's LDS reads from the DMA writes in flight to another stage
  // and does not wait for those
  constexpr bool kDmaA = RING || FP8;
  __shared__ __attribute__((aligned(16))) uint8_t s_a[2][kDmaA ? 16 : C::kAStage];
  __shared__ __attribute__((aligned(16))) uint8_t s_r0[kDmaA ? C::kAStage : 16];
  __shared__ __attribute__((aligned(16))) uint8_t s_r1[kDmaA ? C::kAStage : 16];
  __shared__ __attribute__((aligned(16))) uint8_t s_r2[RING ? C::kAStage : 16];
  __shared__ __attribute__((aligned(16))) uint8_t s_r3[RING ? C::kAStage : 16];
  auto ring = [&](auto ST) -> uint8_t* {
    constexpr int k = decltype(ST)::value;
    if constexpr (k == 0) return s_r0;
    else if constexpr (k == 1) return s_r1;
    else if constexpr (k == 2) return s_r2;
    else return s_r3;
  };
  __shared__ float s_as[2][FP8 && !MX ? BM : 1];
  __shared__ uint32_t s_ax[2][MX ? BM : 1];          // mxfp4: a row's 4 E8M0 bytes of a step
  __shared__ float s_rt[2][FP8 && PACKED && !MX ? BM : 1];  // fp8: a_s(previous step) / a_s(this step) per row
  // GEMM Y: each wave's 64 rows x 64 columns of bf16 output on their way out
  __shared__ __attribute__((aligned(16))) uint8_t s_ystage[GEMM_A ? 16 : NW * 8192];
  // GEMM A: the block's BM x 256 tile of h on its way out
  __shared__ __attribute__((aligned(16))) uint8_t s_hstage[GEMM_A ? BM * (FP8 ? 256 : 512) : 16];
  __shared__ float s_red[FP8 && GEMM_A && !MX ? NW : 1][FP8 && GEMM_A && !MX ? BM : 1];
  __shared__ int s_go;
  __shared__ int s_sel;
  __shared__ int4 s_uc[kBigUnitSlots];   // (tile, N block, expert) of this workgroup's first units
  __shared__ int s_all;                  // every tile was flagged before the workgroup started

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wn = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps tile offsets scalar
  const int l16 = lane & 15;
  const int lhi = lane >> 4;

  if (GEMM_A && a.select) {   // launched beside the 256-row kernel: run only if that one loses
    if (tid < 64) {
      const bool win = sq_gemm_a_wins(a.offsets, a.n_experts, a.max_tiles, a.sel, lane);
      if (lane == 0) s_sel = win ? 1 : 0;
    }
    __syncthreads();
    if (s_sel) return;
  }
  int ntiles = a.num_tiles[0];
  int order = a.unit_order;
  if (ntiles > a.max_tiles) {
    if (blockIdx.x == 0 && tid == 0) record_error(a.err, MOE_ERR_INVALID);
    ntiles = a.max_tiles;
    order = 1;
  }
  const int total = ntiles * a.n_units;
  const int slot = unit_slot(blockIdx.x, gridDim.x);
  const int nk = a.ksteps;  // even
  if (GEMM_A && a.cq != nullptr && blockIdx.x == 0 && tid == 0) *a.cq = 0u;
  // the coordinates and expert of the workgroup's units slot, slot + G, ... found once, one
  // per lane of wave 0 (each a search over the experts' offsets), so that a unit starts with
  // one LDS read instead of a chain of dependent loads while the matrix cores idle
  if (tid < 64) {
    const int uu = slot + lane * (int)gridDim.x;
    if (lane < kBigUnitSlots && uu < total) {
      int m, j;
      unit_coords(a, uu, order, m, j);
      s_uc[lane] = int4{m, j, a.tile_expert[m], 0};
    }
  }
  // ready flags: if the producer had raised every tile's before this workgroup started (it
  // ran before this launch, e.g. on the same stream), one acquire covers them all and no
  // unit polls; otherwise each unit waits on its tile's flag. Forward GEMM A reads
  // dispatch's count of raised flags (one thread, so the whole workgroup takes the same
  // branch); without a count (the backward's flags) the workgroup reads every tile's flag
  // once and takes the shortcut only if all of them carry this call's epoch.
  if (tid == 0)
    s_all = a.wait_ready && a.tiles_done != nullptr &&
            __hip_atomic_load(a.tiles_done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= (uint32_t)ntiles;
  __syncthreads();
  bool all_ready = s_all != 0;
  if (a.wait_ready && a.tiles_done == nullptr) {
    int mine = 1;
    for (int t = tid; t < ntiles; t += 64 * NW)
      mine &= __hip_atomic_load(&a.tile_ready[t], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == a.epoch;
    all_ready = __syncthreads_and(mine) != 0;
  }
  const bool poll_each = a.wait_ready && !all_ready;
  if (a.wait_ready && !poll_each) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");

  int it = 0;   // index of the unit among the workgroup's
  for (int u = slot; u < total; u += gridDim.x, ++it) {
    int m, j, e;
    if (it < kBigUnitSlots) {
      const int4 c = s_uc[it];
      m = __builtin_amdgcn_readfirstlane(c.x);
      j = __builtin_amdgcn_readfirstlane(c.y);
      e = __builtin_amdgcn_readfirstlane(c.z);
    } else {
      unit_coords(a, u, order, m, j);
      e = a.tile_expert[m];
    }
    const int m0 = m * BM;
    if (poll_each && !wait_tile_ready(a, m, &s_go)) continue;
    if (GEMM_A && a.ydone != nullptr && j == 0 && tid == 0) a.ydone[m] = 0u;  // for GEMM Y's combine

    // buffer resources: uniform bases, 32-bit lane offsets, uniform per-tile/step offsets
    const __amdgpu_buffer_rsrc_t ar = make_rsrc(a.A + (int64_t)m0 * a.lda, (uint32_t)(BM * a.lda));
    const __amdgpu_buffer_rsrc_t br = make_rsrc(a.B + (int64_t)e * a.b_expert, (uint32_t)a.b_expert);
    // this wave's weight rows: tiles 0..TN/2-1 from rbase0, TN/2..TN-1 from rbase1
    const int rbase0 = GEMM_A ? j * 256 + wn * HALF : j * 512 + wn * C::kWCols;
    const int rbase1 = GEMM_A ? a.up_row0 + j * 256 + wn * HALF : rbase0 + HALF;
    const uint32_t ldb = (uint32_t)a.ldb;
    const uint32_t lda = (uint32_t)a.lda;
    // lane's K bytes inside a step: bf16 16 at 16*lhi (+64 for the second MFMA), fp8 32 at 32*lhi
    const uint32_t lane_k = (uint32_t)lhi * (FP8 ? 32u : 16u);
    const uint32_t boff0 = (uint32_t)(rbase0 + l16) * ldb + lane_k;
    const uint32_t boff1 = (uint32_t)(rbase1 + l16) * ldb + lane_k;
    const uint32_t tstride = 16u * ldb;
    uint32_t aoff[C::kALoads];
#pragma unroll
    for (int i = 0; i < C::kALoads; ++i) {
      const int c = tid + i * C::kThreads;
      aoff[i] = (uint32_t)(c >> 3) * lda + (uint32_t)(c & 7) * 16u;
    }
    const float* bsx = nullptr;
    if constexpr (FP8 && !MX) bsx = a.B_s + (int64_t)e * a.bs_expert;
    const __amdgpu_buffer_rsrc_t bsr =
        MX ? make_rsrc(a.B_e8 + (int64_t)e * a.b_e8_expert, (uint32_t)a.b_e8_expert)
           : make_rsrc(bsx, FP8 ? (uint32_t)(a.bs_expert * 4) : 0u);
    // mxfp4 weight fragments [buffer][tile] (16 bytes: 32 e2m1 codes) and scale bytes
    u32x4 rbf[MX ? 2 : 1][MX ? TN : 1];
    uint32_t rsb[MX ? 2 : 1][MX ? TN : 1];
    uint32_t rax = 0;   // mxfp4: this thread's row's 4 A scale bytes of the step in flight
    // fp8 weight tile halves [buffer][tile][half] (16 bytes each: a 32-byte MFMA operand)
    u32x4 rbh[FP8 ? 2 : 1][FP8 ? TN : 1][2];

    // weight fragments [buffer][tile]: bf16 two 16-byte K halves, fp8 one 32-byte tuple
    u32x4 rb[2][TN][FP8 ? 1 : 2];
    i32x8_t rb8[2][FP8 ? TN : 1];
    // A (the pool tile: the stream that misses L2) is loaded two steps ahead into
    // one of two register sets, and written to LDS one step ahead
    u32x4 ra[2][C::kALoads];
    float ras[2] = {0.f, 0.f};
    float sbn[2][2];

    auto load_a = [&](auto SET, int ks) {
      constexpr int st = decltype(SET)::value;
      const uint32_t kofs = (uint32_t)ks * 128u;
#pragma unroll
      for (int i = 0; i < C::kALoads; ++i) {
        const int c = tid + i * C::kThreads;
        if (C::kAChunks % C::kThreads == 0 || c < C::kAChunks)
          ra[st][i] = __builtin_amdgcn_raw_buffer_load_b128(ar, aoff[i], kofs, 0);
      }
      if constexpr (FP8) {
        if (tid < BM) ras[st] = a.A_s[((int64_t)m * a.s_kblocks + ks) * BM + tid];
      }
    };
    auto store_a = [&](auto SET, int stage) {
      constexpr int st = decltype(SET)::value;
#pragma unroll
      for (int i = 0; i < C::kALoads; ++i) {
        const int c = tid + i * C::kThreads;
        if (C::kAChunks % C::kThreads == 0 || c < C::kAChunks)
          *reinterpret_cast<u32x4*>(&s_a[stage][0] + swz_a<false>(c >> 3, c & 7)) = ra[st][i];
      }
      if constexpr (FP8) {
        if (tid < BM) s_as[stage][tid] = ras[st];
      }
    };
    auto load_b = [&](auto BUF, int ks) {
      constexpr int bb = decltype(BUF)::value;
      const uint32_t kofs = (uint32_t)ks * 128u;
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        if constexpr (PACKED) {
          // tiled weights: the tile (row block, K tile) is 1 KiB contiguous, lane l at l*16
          const uint32_t rowblk = (uint32_t)((tn < TN / 2 ? rbase0 : rbase1) + (tn % (TN / 2)) * 16) >> 4;
          const uint32_t tbase = (rowblk * (uint32_t)a.ktiles + (uint32_t)ks * (FP8 ? 1u : 2u)) * (FP8 ? 2048u : 1024u);
          if constexpr (FP8) {
            const u32x4 lo = __builtin_amdgcn_raw_buffer_load_b128(br, (uint32_t)lane * 16u, tbase, 0);
            const u32x4 hi = __builtin_amdgcn_raw_buffer_load_b128(br, (uint32_t)lane * 16u, tbase + 1024u, 0);
            rb8[bb][tn] = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
          } else {
            rb[bb][tn][0] = __builtin_amdgcn_raw_buffer_load_b128(br, (uint32_t)lane * 16u, tbase, 0);
            rb[bb][tn][1] = __builtin_amdgcn_raw_buffer_load_b128(br, (uint32_t)lane * 16u, tbase + 1024u, 0);
          }
          continue;
        }
        const uint32_t vo = tn < TN / 2 ? boff0 : boff1;
        const uint32_t so = (uint32_t)(tn % (TN / 2)) * tstride + kofs;
        if constexpr (FP8) {
          const u32x4 lo = __builtin_amdgcn_raw_buffer_load_b128(br, vo, so, 0);
          const u32x4 hi = __builtin_amdgcn_raw_buffer_load_b128(br, vo, so + 16u, 0);
          rb8[bb][tn] = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        } else {
          rb[bb][tn][0] = __builtin_amdgcn_raw_buffer_load_b128(br, vo, so, 0);
          rb[bb][tn][1] = __builtin_amdgcn_raw_buffer_load_b128(br, vo, so + 64u, 0);
        }
      }
      if constexpr (FP8) {
        sbn[bb][0] = bsx[(rbase0 >> 7) * a.bs_ld + ks];
        sbn[bb][1] = bsx[(rbase1 >> 7) * a.bs_ld + ks];
      }
    };

    // one 16-byte weight fragment load (bf16): tile tn, K half kk of step ks into buffer BUF
    auto load_b1 = [&](auto BUF, int tn, int kk, int ks) {
      constexpr int bb = decltype(BUF)::value;
      if constexpr (PACKED) {
        const uint32_t rowblk = (uint32_t)((tn < TN / 2 ? rbase0 : rbase1) + (tn % (TN / 2)) * 16) >> 4;
        const uint32_t tbase = (rowblk * (uint32_t)a.ktiles + (uint32_t)ks * 2u + (uint32_t)kk) * 1024u;
        rb[bb][tn][kk] = __builtin_amdgcn_raw_buffer_load_b128(br, (uint32_t)lane * 16u, tbase, 0);
      } else {
        const uint32_t vo = tn < TN / 2 ? boff0 : boff1;
        const uint32_t so = (uint32_t)(tn % (TN / 2)) * tstride + (uint32_t)ks * 128u + (uint32_t)kk * 64u;
        rb[bb][tn][kk] = __builtin_amdgcn_raw_buffer_load_b128(br, vo, so, 0);
      }
    };

    auto load_b8h = [&](auto BUF, int tn, int hf, int ks) {
      constexpr int bb = decltype(BUF)::value;
      const uint32_t rowblk = (uint32_t)((tn < TN / 2 ? rbase0 : rbase1) + (tn % (TN / 2)) * 16) >> 4;
      const uint32_t tbase = (rowblk * (uint32_t)a.ktiles + (uint32_t)ks) * 2048u + (uint32_t)hf * 1024u;
      rbh[bb][tn][hf] = __builtin_amdgcn_raw_buffer_load_b128(br, (uint32_t)lane * 16u, tbase, 0);
    };
    // fp8: the A rows of step ks into LDS stage ST by LDS-DMA (row r at r*128, chunk c at
    // slot c ^ (r & 7) ^ ((r >> 3) & 1), as swz_a<true>: lane i of 1 KiB load q fetches row
    // 8q + i/8, chunk (i%8) ^ (i/8) ^ (q & 1)),
    // and the rows' activation scales into ras[0] (stored to LDS before the barrier)
    auto dma_rows = [&](auto STAGE, int ks) {
#pragma unroll
      for (int i = 0; i < C::kAStage / 1024 / NW; ++i) {
        const int q = wn * (C::kAStage / 1024 / NW) + i;
        const uint32_t off = (uint32_t)(q * 8 + (lane >> 3)) * (uint32_t)a.lda +
                             (uint32_t)((lane & 7) ^ (lane >> 3) ^ (q & 1)) * 16u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ar, (__attribute__((address_space(3))) void*)(ring(STAGE) + q * 1024), 16, off, (uint32_t)ks * 128u, 0, 0);
      }
    };
    // the rows' activation scales of step ks into ras[0] / rax (stored to LDS before the
    // barrier). Branch-free (a branch here would split the step into blocks, and the
    // compiler then hoists every LDS read of the step above its MFMAs): threads past the
    // tile's rows read, and later store, the last row's scale again
    auto load_ascale = [&](int ks) {
      if constexpr (MX)
        rax = reinterpret_cast<const uint32_t*>(a.A_e8)[((int64_t)m * a.s_kblocks + ks) * BM + min(tid, BM - 1)];
      else
        ras[0] = a.A_s[((int64_t)m * a.s_kblocks + ks) * BM + min(tid, BM - 1)];
    };
    auto dma_a = [&](auto STAGE, int ks) {
      dma_rows(STAGE, ks);
      load_ascale(ks);
    };
    // mxfp4: tile tn's fragment and scale byte of step ks into buffer BUF
    auto load_bmx = [&](auto BUF, int tn, int ks) {
      constexpr int bb = decltype(BUF)::value;
      const uint32_t rowblk = (uint32_t)((tn < TN / 2 ? rbase0 : rbase1) + (tn % (TN / 2)) * 16) >> 4;
      const uint32_t tix = rowblk * (uint32_t)a.ktiles + (uint32_t)ks;
      rbf[bb][tn] = __builtin_amdgcn_raw_buffer_load_b128(br, (uint32_t)lane * 16u, tix * 1024u, 0);
      rsb[bb][tn] = __builtin_amdgcn_raw_buffer_load_b8(bsr, (uint32_t)lane, tix * 64u, 0);
    };
    auto stage_mx = [&](auto STAGE) {
      constexpr int st = decltype(STAGE)::value;
      s_ax[st][min(tid, BM - 1)] = rax;
    };
    auto load_sb = [&](auto BUF, int ks) {
      constexpr int bb = decltype(BUF)::value;
      sbn[bb][0] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
          bsr, 0u, (uint32_t)((rbase0 >> 7) * a.bs_ld + ks) * 4u, 0));
      sbn[bb][1] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
          bsr, 0u, (uint32_t)((rbase1 >> 7) * a.bs_ld + ks) * 4u, 0));
    };
    float sbq[2] = {1.f, 1.f};  // fp8: the weight scales acc is expressed in
    // fp8: thread t stages row min(t, BM-1)'s activation scale of the next step, and
    // the ratio previous / next that the step multiplies acc by (threads past the
    // tile's rows write the same values for the last row again)
    float pa = 1.f;
    auto stage_scale = [&](auto STAGE) {
      constexpr int st = decltype(STAGE)::value;
      const float ns = ras[0];
      s_as[st][min(tid, BM - 1)] = ns;
      s_rt[st][min(tid, BM - 1)] = pa / ns;
      pa = ns;
    };
    f32x4_t acc[TM][TN];
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) acc[tm][tn] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float cur_s[FP8 ? TM : 1][2];  // fp8: scale that acc is currently expressed in
#pragma unroll
    for (int tm = 0; tm < (FP8 ? TM : 1); ++tm) cur_s[tm][0] = cur_s[tm][1] = 1.f;

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    // the pool rows of step ks into ring stage ST (the layout of dma_a)
    constexpr int kDma = C::kAStage / 1024 / NW;   // DMA instructions per wave per step
    auto dma_r = [&](auto ST, int ks) {
      uint8_t* base = ring(ST);
#pragma unroll
      for (int i = 0; i < kDma; ++i) {
        const int q = wn * kDma + i;
        const uint32_t off = (uint32_t)(q * 8 + (lane >> 3)) * (uint32_t)a.lda +
                             (uint32_t)((lane & 7) ^ (lane >> 3)) * 16u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ar, (__attribute__((address_space(3))) void*)(base + q * 1024), 16, off, (uint32_t)ks * 128u, 0, 0);
      }
    };
    if constexpr (RING && FP8) {
      // the ring's first three steps, then this step's scales and weights; one full wait
      using I2 = std::integral_constant<int, 2>;
      dma_rows(I0{}, 0);
      dma_rows(I1{}, nk > 1 ? 1 : 0);
      dma_rows(I2{}, nk > 2 ? 2 : nk - 1);
      load_ascale(0);
      if constexpr (MX) {
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) load_bmx(I0{}, tn, 0);
        wait_vm0();
        stage_mx(I0{});
      } else {
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          load_b8h(I0{}, tn, 0, 0);
          load_b8h(I0{}, tn, 1, 0);
        }
        load_sb(I0{}, 0);
        wait_vm0();
        pa = ras[0];
        stage_scale(I0{});
      }
    } else if constexpr (RING) {
      using I2 = std::integral_constant<int, 2>;
      dma_r(I0{}, 0);
      dma_r(I1{}, 1);
      dma_r(I2{}, 2);
      load_b(I0{}, 0);
      // the DMAs of steps 1 and 2 and the weight loads of step 0 may still be in flight
      __builtin_amdgcn_s_waitcnt(vmcnt_enc(2 * kDma + 2 * TN));
    } else if constexpr (MX) {
      dma_a(I0{}, 0);
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) load_bmx(I0{}, tn, 0);
      wait_vm0();
      stage_mx(I0{});
    } else if constexpr (FP8 && PACKED) {
      dma_a(I0{}, 0);
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        load_b8h(I0{}, tn, 0, 0);
        load_b8h(I0{}, tn, 1, 0);
      }
      load_sb(I0{}, 0);
      wait_vm0();
      pa = ras[0];        // ratio 1 at step 0 (acc is zero there anyway)
      stage_scale(I0{});
    } else {
      load_b(I0{}, 0);
      load_a(I0{}, 0);
      load_a(I1{}, nk > 1 ? 1 : 0);
      store_a(I0{}, 0);
    }
    if constexpr (RING) {
      // a __syncthreads would wait for every DMA in flight; the LDS writes above (fp8,
      // mxfp4 scales) are waited for here
      __builtin_amdgcn_s_waitcnt(kLgkm0);
      __builtin_amdgcn_s_barrier();
    } else {
      __syncthreads();
    }

    auto step = [&](auto BUF, int ks) {
      constexpr int bb = decltype(BUF)::value;
      // keep each step's instructions inside the step: hoisting the next step's loads
      // above these MFMAs would keep two copies of a B buffer alive
      __builtin_amdgcn_sched_barrier(0);
      // prefetch step ks+1 unconditionally (the last step reloads itself into the idle
      // buffer, which nobody reads): a branch here would make the compiler's load
      // counter waits cover the loads just issued and serialise the pipeline
      const int kn = ks + 1 < nk ? ks + 1 : ks;
      const int ka = ks + 2 < nk ? ks + 2 : nk - 1;
      load_a(std::integral_constant<int, bb>{}, ka);   // the set that held A(ks), already in LDS
      load_b(std::integral_constant<int, bb ^ 1>{}, kn);
      // issue the prefetch before this step's MFMAs (into the other buffer), not after them
      __builtin_amdgcn_sched_barrier(0);
      const uint8_t* sa = &s_a[bb][0];
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
        const int r = tm * 16 + l16;
        if constexpr (!FP8) {
#pragma unroll
          for (int kk = 0; kk < KS; ++kk) {
            const bf16x8_t fa = *reinterpret_cast<const bf16x8_t*>(sa + swz_a<false>(r, kk * 4 + lhi));
#pragma unroll
            for (int tn = 0; tn < TN; ++tn)
              acc[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  __builtin_bit_cast(bf16x8_t, rb[bb][tn][kk]), fa, acc[tm][tn], 0, 0, 0);
          }
        } else {
          const u32x4 lo = *reinterpret_cast<const u32x4*>(sa + swz_a<true>(r, 2 * lhi));
          const u32x4 hi = *reinterpret_cast<const u32x4*>(sa + swz_a<true>(r, 2 * lhi + 1));
          const i32x8_t fa = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
          // acc is kept in units of this K block's scale: rescale by old/new, then
          // accumulate the block's integer-grid product in place
          const float sar = s_as[bb][r];
          const float s0 = sar * sbn[bb][0], s1 = sar * sbn[bb][1];
          const float r0 = cur_s[tm][0] * __builtin_amdgcn_rcpf(s0);
          const float r1 = cur_s[tm][1] * __builtin_amdgcn_rcpf(s1);
          cur_s[tm][0] = s0;
          cur_s[tm][1] = s1;
#pragma unroll
          for (int tn = 0; tn < TN; ++tn) {
            const float rr = tn < TN / 2 ? r0 : r1;
            acc[tm][tn] *= rr;
            acc[tm][tn] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(rb8[bb][tn], fa, acc[tm][tn], 0, 0, 0,
                                                                           127, 0, 127);
          }
        }
      }
      store_a(std::integral_constant<int, bb ^ 1>{}, bb ^ 1);  // A(ks+1), loaded last step
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
    };

    // fp8 step: 8 groups (row tile tm) of TN 16x16x128 MFMAs, one K block per step.
    // The accumulator is held in units of the current block's scale a_s[row] *
    // b_s[column block]: each group first rescales its TN tiles by old/new (the old
    // activation scale kept per lane in ap[], the weight scales per wave), then
    // accumulates the block's code product in place. The next step's 8 weight loads
    // and 2 weight-scale loads go out over the first groups (all of them are needed
    // at the next step's first group); A for step ks+2 in group 0.
    // ST: the A stage this step reads (= BUF with two stages, ks % 4 in the ring)
    auto step_fp8 = [&](auto ST, auto BUF, int ks) {
      constexpr int bb = decltype(BUF)::value;
      using NB = std::integral_constant<int, bb ^ 1>;
      using SN = std::integral_constant<int, (decltype(ST)::value + 3) & 3>;
      const int kn = ks + 1 < nk ? ks + 1 : ks;
      const int kd = ks + 3 < nk ? ks + 3 : nk - 1;   // ring: past the end, reload the last step (unread)
      const uint8_t* sa = ring(ST);
      __builtin_amdgcn_sched_barrier(0);
      // weight part of old/new, uniform over the wave (acc is zero at step 0)
      const float sbc0 = sbn[bb][0], sbc1 = sbn[bb][1];
      const float wr0 = sbq[0] * __builtin_amdgcn_rcpf(sbc0);
      const float wr1 = sbq[1] * __builtin_amdgcn_rcpf(sbc1);
      auto rd_a = [&](int tm) {
        const int r = tm * 16 + l16;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(sa + swz_a<true>(r, 2 * lhi));
        const u32x4 hi = *reinterpret_cast<const u32x4*>(sa + swz_a<true>(r, 2 * lhi + 1));
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      };
      // fragments and row ratios are read one group ahead
      u32x8_t fa_cur = rd_a(0);
      float rt_cur = s_rt[bb][l16];
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
        u32x8_t fa_next = fa_cur;
        float rt_next = rt_cur;
        if (tm + 1 < TM) {
          fa_next = rd_a(tm + 1);
          rt_next = s_rt[bb][(tm + 1) * 16 + l16];
        }
        if (tm == 0) {
          if constexpr (RING) {
            load_ascale(kn);                        // first: the end-of-step wait counts from it
            __builtin_amdgcn_sched_barrier(0);
            dma_rows(SN{}, kd);
          } else {
            dma_a(NB{}, kn);
          }
          load_sb(NB{}, kn);
        }
        if (tm < TN) {
          load_b8h(NB{}, tm, 0, kn);
          load_b8h(NB{}, tm, 1, kn);
        }
        const float r0 = rt_cur * wr0, r1 = rt_cur * wr1;
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          acc[tm][tn] *= tn < TN / 2 ? r0 : r1;
          const u32x8_t fb = __builtin_shufflevector(rbh[bb][tn][0], rbh[bb][tn][1], 0, 1, 2, 3, 4, 5, 6, 7);
          acc[tm][tn] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              __builtin_bit_cast(i32x8_t, fb), __builtin_bit_cast(i32x8_t, fa_cur), acc[tm][tn], 0, 0, 0, 127, 0, 127);
        }
        __builtin_amdgcn_sched_barrier(0);
        fa_cur = fa_next;
        rt_cur = rt_next;
      }
      sbq[0] = sbc0;
      sbq[1] = sbc1;
      // the next step's A rows (LDS-DMA, which no register dependency waits for) are in,
      // issued in group 0; the weight loads of groups 1..TN-1 may stay in flight (their
      // registers are waited for where the next step uses them). Then the rows' scales go
      // to LDS and a bare barrier (a __syncthreads would add a workgroup release, which
      // waits for every load in flight) after this wave's LDS writes are done.
      // ring: this step's scale load is in (and with it step ks+1's rows, issued two
      // steps earlier); after it came its rows' DMA of step ks+3 and the step's 2 + 2 TN
      // weight and weight-scale loads, which may stay in flight
      __builtin_amdgcn_s_waitcnt(vmcnt_enc(RING ? C::kAStage / 1024 / NW + 2 + 2 * TN : 2 * (TN - 1)));
      stage_scale(NB{});
      __builtin_amdgcn_s_waitcnt(kLgkm0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
    };

    // mxfp4 step: 8 groups (row tile tm) of TN scaled MFMAs, no fp32 rescaling. The
    // next step's weight fragments and scale bytes go out over the first TN groups,
    // its A rows (LDS-DMA) and A scales in group 0; fragments and the lane's A scale
    // byte are read from LDS one group ahead.
    auto step_mx = [&](auto ST, auto BUF, int ks) {
      constexpr int bb = decltype(BUF)::value;
      using NB = std::integral_constant<int, bb ^ 1>;
      using SN = std::integral_constant<int, (decltype(ST)::value + 3) & 3>;
      const int kn = ks + 1 < nk ? ks + 1 : ks;
      const int kd = ks + 3 < nk ? ks + 3 : nk - 1;
      const uint8_t* sa = ring(ST);
      const uint8_t* sx = reinterpret_cast<const uint8_t*>(&s_ax[bb][0]);
      __builtin_amdgcn_sched_barrier(0);
      auto rd_a = [&](int tm) {
        const int r = tm * 16 + l16;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(sa + swz_a<true>(r, lhi));
        const u32x4 hi = *reinterpret_cast<const u32x4*>(sa + swz_a<true>(r, lhi + 4));
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      };
      u32x8_t fa_cur = rd_a(0);
      uint32_t xs_cur = sx[l16 * 4 + lhi];
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
        u32x8_t fa_next = fa_cur;
        uint32_t xs_next = xs_cur;
        if (tm + 1 < TM) {
          fa_next = rd_a(tm + 1);
          xs_next = sx[((tm + 1) * 16 + l16) * 4 + lhi];
        }
        if (tm == 0) {
          if constexpr (RING) {
            load_ascale(kn);
            __builtin_amdgcn_sched_barrier(0);
            dma_rows(SN{}, kd);
          } else {
            dma_a(NB{}, kn);
          }
        }
        if (tm < TN) load_bmx(NB{}, tm, kn);
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          const u32x8_t fb = __builtin_shufflevector(rbf[bb][tn], rbf[bb][tn], 0, 1, 2, 3, -1, -1, -1, -1);
          acc[tm][tn] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              __builtin_bit_cast(i32x8_t, fb), __builtin_bit_cast(i32x8_t, fa_cur), acc[tm][tn], 4, 0, 0,
              (int)rsb[bb][tn], 0, (int)xs_cur);
        }
        __builtin_amdgcn_sched_barrier(0);
        fa_cur = fa_next;
        xs_cur = xs_next;
      }
      // as in the fp8 step: the A rows (group 0) are in, the weight loads of groups
      // 1..TN-1 may stay in flight
      __builtin_amdgcn_s_waitcnt(vmcnt_enc(RING ? C::kAStage / 1024 / NW + 2 * TN : 2 * (TN - 1)));
      stage_mx(NB{});
      __builtin_amdgcn_s_waitcnt(kLgkm0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
    };

    // bf16 step: 16 groups (K half kk, row tile tm) of TN MFMAs. The next step's loads
    // are spread over the groups instead of issued as one burst (a wave issues in
    // order, and a burst of vector loads would hold it off its MFMAs until the
    // texture unit has taken them all): A for step ks+2 and the first K half of B for
    // step ks+1 early, the second K half mid-step, which is also the order in which
    // step ks+1 consumes them. LDS fragments are read one group ahead.
    auto step_bf16 = [&](auto BUF, int ks) {
      constexpr int bb = decltype(BUF)::value;
      using NB = std::integral_constant<int, bb ^ 1>;
      const int kn = ks + 1 < nk ? ks + 1 : ks;
      const int ka = ks + 2 < nk ? ks + 2 : nk - 1;
      const uint8_t* sa = &s_a[bb][0];
      __builtin_amdgcn_sched_barrier(0);
      bf16x8_t fa_cur = *reinterpret_cast<const bf16x8_t*>(sa + swz_a<false>(l16, lhi));
#pragma unroll
      for (int g = 0; g < 2 * TM; ++g) {
        const int kk = g / TM, tm = g % TM;
        bf16x8_t fa_next = fa_cur;
        if (g + 1 < 2 * TM) {
          const int kk1 = (g + 1) / TM, tm1 = (g + 1) % TM;
          fa_next = *reinterpret_cast<const bf16x8_t*>(sa + swz_a<false>(tm1 * 16 + l16, kk1 * 4 + lhi));
        }
        if (g == 0) load_a(std::integral_constant<int, bb>{}, ka);
        if (g >= 1 && g <= TN) load_b1(NB{}, g - 1, 0, kn);
        if (g >= TM && g < TM + TN) load_b1(NB{}, g - TM, 1, kn);
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
          acc[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8_t, rb[bb][tn][kk]), fa_cur, acc[tm][tn], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        fa_cur = fa_next;
      }
      store_a(std::integral_constant<int, bb ^ 1>{}, bb ^ 1);  // A(ks+1), loaded last step
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
    };

    // ring step: stage ST (= ks % 4), weights in buffer ks % 2; sends step ks+3 into the
    // stage step ks-1 read (every read of it is behind the last barrier)
    auto step_ring = [&](auto ST, auto BUF, int ks) {
      constexpr int st = decltype(ST)::value;
      constexpr int bb = decltype(BUF)::value;
      using NB = std::integral_constant<int, bb ^ 1>;
      using SN = std::integral_constant<int, (st + 3) & 3>;
      const int kn = ks + 1 < nk ? ks + 1 : ks;
      const int kd = ks + 3 < nk ? ks + 3 : nk - 1;   // past the end: reload the last step (unread)
      const uint8_t* sa = ring(ST);
      __builtin_amdgcn_sched_barrier(0);
      bf16x8_t fa_cur = *reinterpret_cast<const bf16x8_t*>(sa + swz_a<false>(l16, lhi));
#pragma unroll
      for (int g = 0; g < 2 * TM; ++g) {
        const int kk = g / TM, tm = g % TM;
        bf16x8_t fa_next = fa_cur;
        if (g + 1 < 2 * TM) {
          const int kk1 = (g + 1) / TM, tm1 = (g + 1) % TM;
          fa_next = *reinterpret_cast<const bf16x8_t*>(sa + swz_a<false>(tm1 * 16 + l16, kk1 * 4 + lhi));
        }
        if (g == 0) dma_r(SN{}, kd);
        if (g >= 1 && g <= TN) load_b1(NB{}, g - 1, 0, kn);
        if (g >= TM && g < TM + TN) load_b1(NB{}, g - TM, 1, kn);
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
          acc[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8_t, rb[bb][tn][kk]), fa_cur, acc[tm][tn], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        fa_cur = fa_next;
      }
      // in flight after step ks+1's DMAs (issued two steps ago), in order: weights of
      // ks-1, DMAs of ks+2, weights of ks, DMAs of ks+3, weights of ks+1
      __builtin_amdgcn_s_waitcnt(vmcnt_enc(2 * kDma + 3 * 2 * TN));
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
    };

    if constexpr (RING && FP8) {
      using I2 = std::integral_constant<int, 2>;
      using I3 = std::integral_constant<int, 3>;
      for (int ks = 0; ks < nk; ks += 4) {
        if constexpr (MX) {
          step_mx(I0{}, I0{}, ks);
          step_mx(I1{}, I1{}, ks + 1);
          step_mx(I2{}, I0{}, ks + 2);
          step_mx(I3{}, I1{}, ks + 3);
        } else {
          step_fp8(I0{}, I0{}, ks);
          step_fp8(I1{}, I1{}, ks + 1);
          step_fp8(I2{}, I0{}, ks + 2);
          step_fp8(I3{}, I1{}, ks + 3);
        }
      }
      wait_vm0();   // the reloads past the end land before the ring is refilled
    } else if constexpr (RING) {
      using I2 = std::integral_constant<int, 2>;
      using I3 = std::integral_constant<int, 3>;
      for (int ks = 0; ks < nk; ks += 4) {
        step_ring(I0{}, I0{}, ks);
        step_ring(I1{}, I1{}, ks + 1);
        step_ring(I2{}, I0{}, ks + 2);
        step_ring(I3{}, I1{}, ks + 3);
      }
      wait_vm0();   // the reloads past the end land before the ring is refilled
    }
    for (int ks = 0; ks < (RING ? 0 : nk); ks += 2) {
      if constexpr (RING) {
      } else if constexpr (MX) {
        step_mx(I0{}, I0{}, ks);
        step_mx(I1{}, I1{}, ks + 1);
      } else if constexpr (FP8 && PACKED) {
        step_fp8(I0{}, I0{}, ks);
        step_fp8(I1{}, I1{}, ks + 1);
      } else if constexpr (!FP8 && TM >= TN + 1) {
        step_bf16(std::integral_constant<int, 0>{}, ks);
        step_bf16(std::integral_constant<int, 1>{}, ks + 1);
      } else {
        step(std::integral_constant<int, 0>{}, ks);
        step(std::integral_constant<int, 1>{}, ks + 1);
      }
    }

    // ---------------- epilogue: lane holds row tm*16+l16, columns 4*lhi + (0..3) of each tile
    if constexpr (MX) {
      // block scales were applied by the MFMAs
    } else if constexpr (FP8 && PACKED) {
      // the last step's scales (its stage, and the reloaded copy in the other one)
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
        const float sl = s_as[(nk - 1) & 1][tm * 16 + l16];
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) acc[tm][tn] *= sl * sbq[tn < TN / 2 ? 0 : 1];
      }
    } else if constexpr (FP8) {
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) acc[tm][tn] *= cur_s[tm][tn < TN / 2 ? 0 : 1];
    }
    if constexpr (GEMM_A) {
      // h leaves through LDS: the block's BM x 256 tile is staged (16-byte chunks
      // swizzled by row), then stored as whole rows of the tile -- 512 bytes (bf16)
      // or 256 bytes (e4m3) each -- instead of 32- or 16-byte pieces of 16 rows.
      // One barrier; the stage is next written after the next unit's K loop.
      constexpr int HROW = FP8 ? 256 : 512;           // bytes of a tile row of h
      const int hb0 = (wn * HALF + 4 * lhi) * (FP8 ? 1 : 2);  // this lane's first byte in it
      auto hst = [&](int r, int b) {                   // staging address of row r, byte b
        return &s_hstage[r * HROW + ((((b >> 4) ^ (r & 7))) << 4) + (b & 15)];
      };
      auto hstore = [&]() {
        constexpr int LPR = HROW / 16;                 // lanes per row
#pragma unroll
        for (int q = 0; q < BM * HROW / 1024 / NW; ++q) {
          const int r = (wn * (BM * HROW / 1024 / NW) + q) * (64 / LPR) + lane / LPR;
          const int sl = lane % LPR;
          const u32x4 v = *reinterpret_cast<const u32x4*>(&s_hstage[r * HROW + sl * 16]);
          *reinterpret_cast<u32x4*>(a.out + (int64_t)(m0 + r) * a.ldo + j * HROW + ((sl ^ (r & 7)) << 4)) = v;
        }
      };
      if constexpr (!FP8) {
        if (a.g_save != nullptr) {
          // training: keep G (gate and up before the activation) for the backward pass.
          // It leaves through the same stage as h, gate columns then up columns, as whole
          // 512-byte rows of the unit's 256 columns of each. Bare barriers: the stage is
          // whole once every wave's LDS writes are done, and free again once every wave's
          // reads are (a __syncthreads would also wait for the G stores to complete).
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
            for (int tm = 0; tm < TM; ++tm) {
              const int r = tm * 16 + l16;
#pragma unroll
              for (int tn = 0; tn < TN / 2; ++tn) {
                u32x2 v;
                v.x = pack_bf16x2(acc[tm][tn + hf * (TN / 2)][0], acc[tm][tn + hf * (TN / 2)][1]);
                v.y = pack_bf16x2(acc[tm][tn + hf * (TN / 2)][2], acc[tm][tn + hf * (TN / 2)][3]);
                *reinterpret_cast<u32x2*>(hst(r, hb0 + tn * 32)) = v;
              }
            }
            __builtin_amdgcn_s_waitcnt(kLgkm0);
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            uint8_t* gcol = a.g_save + (int64_t)(hf * a.up_row0 + j * 256) * 2;
#pragma unroll
            for (int q = 0; q < BM * 512 / 1024 / NW; ++q) {
              const int r = (wn * (BM * 512 / 1024 / NW) + q) * 2 + lane / 32;
              const int sl = lane % 32;
              const u32x4 v = *reinterpret_cast<const u32x4*>(&s_hstage[r * 512 + sl * 16]);
              *reinterpret_cast<u32x4*>(gcol + (int64_t)(m0 + r) * a.g_ld + ((sl ^ (r & 7)) << 4)) = v;
            }
            __builtin_amdgcn_s_waitcnt(kLgkm0);
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
          }
        }
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
          const int r = tm * 16 + l16;
#pragma unroll
          for (int tn = 0; tn < TN / 2; ++tn) {
            u32x2 v;
            v.x = pack_bf16x2(silu_mul(acc[tm][tn][0], acc[tm][tn + TN / 2][0]),
                              silu_mul(acc[tm][tn][1], acc[tm][tn + TN / 2][1]));
            v.y = pack_bf16x2(silu_mul(acc[tm][tn][2], acc[tm][tn + TN / 2][2]),
                              silu_mul(acc[tm][tn][3], acc[tm][tn + TN / 2][3]));
            *reinterpret_cast<u32x2*>(hst(r, hb0 + tn * 32)) = v;
          }
        }
        __syncthreads();
        hstore();
      } else if constexpr (MX) {
        // MXFP8 h: a 1x32 block of a row = gate tiles 2b, 2b+1 of one wave, spread
        // over the row's 4 lanes (lhi): amax by two cross-lane steps, no LDS
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
          const int rl = tm * 16 + l16;
#pragma unroll
          for (int bi = 0; bi < HALF / 32; ++bi) {
            float am = 0.f;
#pragma unroll
            for (int tn = 2 * bi; tn < 2 * bi + 2; ++tn)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float h = silu_mul(acc[tm][tn][i], acc[tm][tn + TN / 2][i]);
                acc[tm][tn][i] = h;
                am = fmaxf(am, fabsf(h));
              }
            am = fmaxf(am, __shfl_xor(am, 16));
            am = fmaxf(am, __shfl_xor(am, 32));
            const int ex = mx_e4m3_shared_exp(am);
            const float inv = mx_inv_scale(ex);
#pragma unroll
            for (int tn = 2 * bi; tn < 2 * bi + 2; ++tn)
              *reinterpret_cast<uint32_t*>(hst(rl, hb0 + tn * 16)) =
                  pack_e4m3x4(acc[tm][tn][0] * inv, acc[tm][tn][1] * inv, acc[tm][tn][2] * inv, acc[tm][tn][3] * inv);
            const int blk = ((j * 256 + wn * HALF) >> 5) + bi;   // h's 32-column block
            if (lhi == 0)
              a.out_e8[(((int64_t)m * a.out_groups + (blk >> 2)) * BM + rl) * 4 + (blk & 3)] = (uint8_t)(ex + 127);
          }
        }
        __syncthreads();
        hstore();
      } else {
        // an h group of 128 columns = the HALF columns of 128/HALF consecutive waves
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
          float mx = 0.f;
#pragma unroll
          for (int tn = 0; tn < TN / 2; ++tn)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float h = silu_mul(acc[tm][tn][i], acc[tm][tn + TN / 2][i]);
              acc[tm][tn][i] = h;
              mx = fmaxf(mx, fabsf(h));
            }
          mx = fmaxf(mx, __shfl_xor(mx, 16));
          mx = fmaxf(mx, __shfl_xor(mx, 32));
          if (lhi == 0) s_red[wn][tm * 16 + l16] = mx;
        }
        __syncthreads();
        constexpr int GW = 128 / HALF;  // waves per h group
        const int w0 = wn / GW * GW;
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
          const int rl = tm * 16 + l16;
          float mx = s_red[w0][rl];
#pragma unroll
          for (int g = 1; g < GW; ++g) mx = fmaxf(mx, s_red[w0 + g][rl]);
          const float sc = mx > 0.f ? mx / 448.0f : 1.0f;
          const float inv = 1.0f / sc;  // h codes: h * (1/scale), one division per row
#pragma unroll
          for (int tn = 0; tn < TN / 2; ++tn)
            *reinterpret_cast<uint32_t*>(hst(rl, hb0 + tn * 16)) =
                pack_e4m3x4(acc[tm][tn][0] * inv, acc[tm][tn][1] * inv, acc[tm][tn][2] * inv, acc[tm][tn][3] * inv);
          if (wn % GW == 0 && lhi == 0)
            a.out_s[((int64_t)m * a.out_groups + ((j * 256 + wn * HALF) >> 7)) * BM + rl] = sc;
        }
        __syncthreads();  // (also: every s_red read is done before the next unit writes it)
        hstore();
      }
    } else if constexpr (EPI == 1) {
      // backward GEMM Y: acc = dh for row tm*16+l16, h columns c..c+3 of tile tn with
      // c = j*512 + wn*64 + tn*16 + 4*lhi. g and u come from G (columns c and I + c), the
      // results replace them: dg = dh u silu'(g), du = dh silu(g), s = 1 / (1 + e^-g),
      // silu'(g) = s (1 + g (1 - s)). G moves as whole 128-byte row segments (the wave's
      // 64 columns) through the wave's own LDS region, 32 rows at a time: row-contiguous
      // loads -> LDS -> fragment order -> results in place -> LDS -> row-contiguous stores.
      // The next 32 rows' loads are issued before this group's LDS work. A wave's LDS
      // accesses complete in order, and each staged value is read and rewritten by the
      // lane that owns it: no barrier.
      constexpr int SP = 32;                           // rows per group
      const int I2 = a.up_row0 * 2;                    // bytes from g to u in a G row
      uint8_t* st = &s_ystage[wn * 8192];              // g rows at 0, u rows at 4096
      const int colb = (j * 512 + wn * C::kWCols) * 2;
      const int lr = lane >> 3, sl = lane & 7;         // row-contiguous: row q*8 + lr, slot sl
      auto gsrc = [&](int sp, int q) {
        const int r = q * 8 + lr;
        return a.g_save + (int64_t)(m0 + sp * SP + r) * a.g_ld + colb + ((sl ^ (r & 7)) << 4);
      };
      auto sfrag = [&](int r, int b) { return st + r * 128 + ((((b >> 4) ^ (r & 7))) << 4) + (b & 15); };
      u32x4 gl[2][SP / 8], ul[2][SP / 8];
#pragma unroll
      for (int q = 0; q < SP / 8; ++q) {
        gl[0][q] = *reinterpret_cast<const u32x4*>(gsrc(0, q));
        ul[0][q] = *reinterpret_cast<const u32x4*>(gsrc(0, q) + I2);
      }
#pragma unroll
      for (int sp = 0; sp < BM / SP; ++sp) {
        const int cb = sp & 1;
        if (sp + 1 < BM / SP) {
#pragma unroll
          for (int q = 0; q < SP / 8; ++q) {
            gl[cb ^ 1][q] = *reinterpret_cast<const u32x4*>(gsrc(sp + 1, q));
            ul[cb ^ 1][q] = *reinterpret_cast<const u32x4*>(gsrc(sp + 1, q) + I2);
          }
        }
#pragma unroll
        for (int q = 0; q < SP / 8; ++q) {
          const int r = q * 8 + lr;
          *reinterpret_cast<u32x4*>(st + r * 128 + sl * 16) = gl[cb][q];
          *reinterpret_cast<u32x4*>(st + 4096 + r * 128 + sl * 16) = ul[cb][q];
        }
#pragma unroll
        for (int t = 0; t < SP / 16; ++t) {
          const int tm = sp * (SP / 16) + t;
          const int r = t * 16 + l16;
#pragma unroll
          for (int tn = 0; tn < TN; ++tn) {
            uint8_t* pg = sfrag(r, tn * 32 + 8 * lhi);
            const u32x2 gv = *reinterpret_cast<const u32x2*>(pg);
            const u32x2 uv = *reinterpret_cast<const u32x2*>(pg + 4096);
            const float g[4] = {bf16_lo(gv.x), bf16_hi(gv.x), bf16_lo(gv.y), bf16_hi(gv.y)};
            const float u[4] = {bf16_lo(uv.x), bf16_hi(uv.x), bf16_lo(uv.y), bf16_hi(uv.y)};
            float dg[4], du[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-g[i]));
              const float dh = acc[tm][tn][i];
              dg[i] = dh * u[i] * (sg * (1.0f + g[i] * (1.0f - sg)));
              du[i] = dh * (g[i] * sg);
            }
            u32x2 o;
            o.x = pack_bf16x2(dg[0], dg[1]);
            o.y = pack_bf16x2(dg[2], dg[3]);
            *reinterpret_cast<u32x2*>(pg) = o;
            o.x = pack_bf16x2(du[0], du[1]);
            o.y = pack_bf16x2(du[2], du[3]);
            *reinterpret_cast<u32x2*>(pg + 4096) = o;
          }
        }
#pragma unroll
        for (int q = 0; q < SP / 8; ++q) {
          const int r = q * 8 + lr;
          uint8_t* dst = const_cast<uint8_t*>(gsrc(sp, q));
          *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(st + r * 128 + sl * 16);
          *reinterpret_cast<u32x4*>(dst + I2) = *reinterpret_cast<const u32x4*>(st + 4096 + r * 128 + sl * 16);
        }
      }
    } else {
      // y rows go out in whole 128-byte segments: the wave's 64 columns of 64 rows at
      // a time are written to its own LDS region (16-byte chunks swizzled by row), then
      // read back row-contiguous, so each 1 KiB store covers 8 full rows' segments
      // instead of 32-byte pieces of 16 rows. The region is the wave's alone, and a
      // wave's LDS accesses complete in order: no barrier.
      uint8_t* st = &s_ystage[wn * 8192];
      const int colb = (j * 512 + wn * C::kWCols) * 2;
#pragma unroll
      for (int pass = 0; pass < BM / 64; ++pass) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int tm = pass * 4 + t;
          const int r = t * 16 + l16;
#pragma unroll
          for (int tn = 0; tn < TN; ++tn) {
            u32x2 v;
            v.x = pack_bf16x2(acc[tm][tn][0], acc[tm][tn][1]);
            v.y = pack_bf16x2(acc[tm][tn][2], acc[tm][tn][3]);
            const int b = tn * 32 + 8 * lhi;  // byte of the row's 128-byte segment
            *reinterpret_cast<u32x2*>(st + r * 128 + (((b >> 4) ^ (r & 7)) << 4) + (b & 15)) = v;
          }
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int r = q * 8 + (lane >> 3);
          const int sl = lane & 7;
          const u32x4 v = *reinterpret_cast<const u32x4*>(st + r * 128 + sl * 16);
          const int64_t row = m0 + pass * 64 + r;
          *reinterpret_cast<u32x4*>(a.out + row * a.ldo + colb + ((sl ^ (r & 7)) << 4)) = v;
        }
      }
      if (a.ydone != nullptr) {
        // publish the unit for combine: every wave's y stores are issued (barrier), then
        // one device-scope release and a count on the tile
        __syncthreads();
        if (tid == 0) {
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
          __hip_atomic_fetch_add(&a.ydone[m], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
  }
  if constexpr (!GEMM_A) {
    if (a.ydone != nullptr) combine_tail(a, &s_go);
  }
}

// ----------------------------------------------------------------------------
// Load-time weight permutation into MFMA fragment order (layout in moe355.h).
// One thread per 16-byte destination chunk: reads 16 source bytes, writes them
// to their tile slot, so a whole wave writes 1 KiB contiguously.
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(256) void pack_weights_kernel(const uint8_t* w, uint8_t* out, int64_t chunks,
                                                           int32_t row_bytes, int32_t fp8) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= chunks) return;
  // destination chunk c -> (tile, half, lane); a tile is 1 KiB (bf16) or 2 KiB (fp8)
  const int64_t tile = fp8 ? c >> 7 : c >> 6;
  const int half = fp8 ? (int)((c >> 6) & 1) : 0;
  const int lane = (int)(c & 63);
  const int ktiles = fp8 ? row_bytes / 128 : row_bytes / 64;   // K tiles per 16-row block
  const int64_t rb = tile / ktiles;            // global row block (experts stacked)
  const int kb = (int)(tile - rb * ktiles);
  const int64_t row = rb * 16 + (lane & 15);
  const int64_t col_byte = fp8 ? (int64_t)kb * 128 + 32 * (lane >> 4) + 16 * half
                               : (int64_t)kb * 64 + 16 * (lane >> 4);
  const u32x4 v = *reinterpret_cast<const u32x4*>(w + row * row_bytes + col_byte);
  *reinterpret_cast<u32x4*>(out + c * 16) = v;
}

int launch_pack_weights(const void* w, int32_t E, int32_t rows, int32_t K, int32_t dtype, void* out,
                        hipStream_t stream) {
  // an MXFP4 tile (16 rows x 64 bytes, lane l = row l%16, bytes 16*(l/16)..+16) has
  // the byte layout of a bf16 one
  const bool fp8 = dtype == MOE_FP8_E4M3_G128;
  const int32_t row_bytes = dtype == MOE_MXFP4 ? K / 2 : K * (fp8 ? 1 : 2);
  const int64_t chunks = (int64_t)E * rows * row_bytes / 16;
  const int64_t blocks = (chunks + 255) / 256;
  hipLaunchKernelGGL(pack_weights_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<const uint8_t*>(w), static_cast<uint8_t*>(out), chunks, row_bytes, (int)fp8);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// MXFP4 scale permutation (layout in moe355.h): one thread per destination byte.
__global__ __launch_bounds__(256) void pack_mx_scales_kernel(const uint8_t* s, uint8_t* out, int64_t n,
                                                             int32_t kblocks) {
  const int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (o >= n) return;
  const int l = (int)(o & 63);
  const int64_t tile = o >> 6;
  const int ktiles = kblocks / 4;
  const int64_t rb = tile / ktiles;            // global row block (experts stacked)
  const int kb = (int)(tile - rb * ktiles);
  out[o] = s[(rb * 16 + (l & 15)) * kblocks + kb * 4 + (l >> 4)];
}

int launch_pack_mx_scales(const void* s, int32_t E, int32_t rows, int32_t K, void* out, hipStream_t stream) {
  const int64_t n = (int64_t)E * rows * (K / 32);
  hipLaunchKernelGGL(pack_mx_scales_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     static_cast<const uint8_t*>(s), static_cast<uint8_t*>(out), n, K / 32);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// ----------------------------------------------------------------------------
// host side
// ----------------------------------------------------------------------------
// The big-tile kernel wants whole 256 (gate) + 256 (up) and 512-column units and an
// even number of 128-byte K steps; in fp8 it reads tiled weights only, at tile 128.
static bool big_a_ok(int32_t H, int32_t I, int32_t dtype, int32_t tile) {
  if (dtype == MOE_FP8_E4M3_G128 || dtype == MOE_MXFP4) return tile == 128 && I % 256 == 0 && H % 256 == 0;
  return dtype == MOE_BF16 && (tile == 64 || tile == 128) && I % 256 == 0 && H % 128 == 0;
}
static bool big_y_ok(int32_t H, int32_t I, int32_t dtype, int32_t tile) {
  if (dtype == MOE_FP8_E4M3_G128 || dtype == MOE_MXFP4) return tile == 128 && H % 512 == 0 && I % 256 == 0;
  return dtype == MOE_BF16 && (tile == 64 || tile == 128) && H % 512 == 0 && I % 128 == 0;
}

// training (G kept, backward available): bf16 on the big-tile kernel for both forward
// GEMMs and both backward data GEMMs (N = I and N = H in 512-column blocks)
bool ffn_train_ok(int32_t H, int32_t I, int32_t dtype, int32_t tile, int32_t block_n) {
  return dtype == MOE_BF16 && big_a_ok(H, I, dtype, tile) && big_y_ok(H, I, dtype, tile) && I % 512 == 0 &&
         H % 512 == 0 && (block_n == 0 || block_n == 512);
}

// 256 x 256 units (ffn_sq.hip): bf16 with tiled weights at tile 128; K stages of 32 in
// whole rounds of four (H, I % 128) and whole 256-column N blocks (2I, H % 256); 32-bit
// buffer offsets over a unit's rows and an expert's weights
bool ffn_sq_ok(int32_t H, int32_t I, int32_t dtype, int32_t tile, int32_t block_n, int32_t weight_layout,
               bool combine) {
  return dtype == MOE_BF16 && tile == 128 && weight_layout == MOE_WEIGHTS_MFMA_TILED && !combine &&
         (block_n == 0 || block_n == 512) && H % 256 == 0 && I % 128 == 0 &&
         (int64_t)2 * I * H * 2 < ((int64_t)1 << 32) && (int64_t)256 * std::max(H, I) * 2 < ((int64_t)1 << 31);
}

int ffn_supported(int32_t H, int32_t I, int32_t dtype, int32_t tile, int32_t block_n, int32_t weight_layout,
                  int32_t unit_rows, bool combine) {
  if (block_n != 0 && block_n != 128 && block_n != 256 && block_n != 512) return MOE_ERR_INVALID;
  if (unit_rows != 0 && unit_rows != 128 && unit_rows != 256) return MOE_ERR_INVALID;
  const bool sq = ffn_sq_ok(H, I, dtype, tile, block_n, weight_layout, combine);
  if (unit_rows == 256 && !sq) return MOE_ERR_UNSUPPORTED;
  // tiled bf16 weights on shapes only the 256 x 256 kernel takes
  if (sq && unit_rows != 128) return MOE_OK;
  const bool big_a = big_a_ok(H, I, dtype, tile);
  const bool big_y = big_y_ok(H, I, dtype, tile);
  // fp8 on the big-tile kernel needs tiled weights
  if (dtype == MOE_FP8_E4M3_G128 && block_n == 512 && weight_layout != MOE_WEIGHTS_MFMA_TILED)
    return MOE_ERR_UNSUPPORTED;
  if (block_n == 512 && !(big_a && big_y)) return MOE_ERR_UNSUPPORTED;
  // tiled weights are read by the big-tile kernel only, so both GEMMs must take it
  if (weight_layout == MOE_WEIGHTS_MFMA_TILED && (!(big_a && big_y) || (block_n != 0 && block_n != 512)))
    return MOE_ERR_UNSUPPORTED;
  if (dtype == MOE_BF16) {
    if (H % 128 != 0 || I % 64 != 0) return MOE_ERR_UNSUPPORTED;
    if (block_n == 256 && (tile < 64 || I % 128 != 0)) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
  }
  if (dtype == MOE_FP8_E4M3_G128) {
    if (H % 256 != 0 || I % 128 != 0 || tile < 64) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
  }
  if (dtype == MOE_MXFP4) {
    // the big-tile kernel with tiled weights is the only mxfp4 path
    if (weight_layout != MOE_WEIGHTS_MFMA_TILED || !(big_a && big_y) || (block_n != 0 && block_n != 512))
      return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
  }
  return MOE_ERR_INVALID;
}

// waves of a big-tile workgroup: each owns BM rows x 64 of the unit's 512 columns
constexpr int kBigWaves = 8;

template <int BM, int BN, int WM, int WN, bool FP8, bool GEMM_A>
static void launch_one(const FfnArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((ffn_gemm_kernel<BM, BN, WM, WN, FP8, GEMM_A>), dim3(grid), dim3(256), 0, s, a);
}

template <bool FP8, bool GEMM_A, bool PACKED>
static int launch_big(int tile, const FfnArgs& a, int grid, hipStream_t s) {
  constexpr int NW = kBigWaves;
  if (!FP8 && tile == 128 && a.ksteps % 4 == 0 && a.a_stages != 2)
    hipLaunchKernelGGL((ffn_big_kernel<128, NW, false, GEMM_A, PACKED, false, 0, true>), dim3(grid), dim3(64 * NW), 0,
                       s, a);
  else if (tile == 128) hipLaunchKernelGGL((ffn_big_kernel<128, NW, FP8, GEMM_A, PACKED>), dim3(grid), dim3(64 * NW), 0, s, a);
  else if (tile == 64) hipLaunchKernelGGL((ffn_big_kernel<64, NW, FP8, GEMM_A, PACKED>), dim3(grid), dim3(64 * NW), 0, s, a);
  else return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

template <bool GEMM_A>
static int launch_mx(int tile, int bn, bool packed, const FfnArgs& a, int grid, hipStream_t s) {
  if (bn != 512 || !packed || tile != 128) return MOE_ERR_UNSUPPORTED;
  if (a.ksteps % 4 == 0 && a.a_stages != 2)
    hipLaunchKernelGGL((ffn_big_kernel<128, kBigWaves, true, GEMM_A, true, true, 0, true>), dim3(grid),
                       dim3(64 * kBigWaves), 0, s, a);
  else
    hipLaunchKernelGGL((ffn_big_kernel<128, kBigWaves, true, GEMM_A, true, true>), dim3(grid), dim3(64 * kBigWaves),
                       0, s, a);
  return MOE_OK;
}

template <bool FP8, bool GEMM_A>
static int launch_shape(int tile, int bn, bool packed, const FfnArgs& a, int grid, hipStream_t s) {
  if (bn == 512) {
    if constexpr (FP8) {
      if (!packed || tile != 128) return MOE_ERR_UNSUPPORTED;  // fp8 big tiles read tiled weights
      // (the four-stage ring measured no faster for fp8, unlike bf16 and mxfp4: two stages)
      hipLaunchKernelGGL((ffn_big_kernel<128, kBigWaves, true, GEMM_A, true>), dim3(grid), dim3(64 * kBigWaves), 0, s, a);
      return MOE_OK;
    } else {
      return packed ? launch_big<FP8, GEMM_A, true>(tile, a, grid, s) : launch_big<FP8, GEMM_A, false>(tile, a, grid, s);
    }
  }
  if (packed) return MOE_ERR_UNSUPPORTED;
  if constexpr (FP8) {
    if (tile == 128) launch_one<128, 256, 2, 2, true, GEMM_A>(a, grid, s);
    else if (tile == 64) launch_one<64, 256, 1, 4, true, GEMM_A>(a, grid, s);
    else return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
  } else {
    switch (tile) {
      case 128:
        if (bn == 256) launch_one<128, 256, 2, 2, false, GEMM_A>(a, grid, s);
        else launch_one<128, 128, 2, 2, false, GEMM_A>(a, grid, s);
        return MOE_OK;
      case 64:
        if (bn == 256) launch_one<64, 256, 1, 4, false, GEMM_A>(a, grid, s);
        else launch_one<64, 128, 1, 4, false, GEMM_A>(a, grid, s);
        return MOE_OK;
      case 32: launch_one<32, 128, 1, 4, false, GEMM_A>(a, grid, s); return MOE_OK;
      case 16: launch_one<16, 128, 1, 4, false, GEMM_A>(a, grid, s); return MOE_OK;
    }
    return MOE_ERR_UNSUPPORTED;
  }
}

// N block of each GEMM: the big-tile kernel (512) where the shape allows it,
// else the largest the general kernel takes, unless overridden.
static void pick_block_n(const FfnLaunch& f, int tile, int& bn_a, int& bn_y) {
  if (f.dtype == MOE_MXFP4) {
    bn_a = bn_y = 512;
    return;
  }
  const bool fp8 = f.dtype == MOE_FP8_E4M3_G128;
  const bool tiled = f.weight_layout == MOE_WEIGHTS_MFMA_TILED;
  // fp8 reaches the big-tile kernel only with tiled weights
  const bool big_a = big_a_ok(f.H, f.I, f.dtype, tile) && (!fp8 || tiled);
  const bool big_y = big_y_ok(f.H, f.I, f.dtype, tile) && (!fp8 || tiled);
  if (f.block_n == 512) {
    bn_a = bn_y = 512;
    return;
  }
  if (f.block_n == 128 || f.block_n == 256) {
    bn_a = bn_y = fp8 ? 256 : f.block_n;
  } else {
    bn_a = big_a ? 512 : fp8 ? 256 : (tile >= 64 && f.I % 128 == 0) ? 256 : 128;
    bn_y = big_y ? 512 : fp8 ? 256 : (tile >= 64 && f.H % 256 == 0) ? 256 : 128;
  }
  if (!fp8 && bn_y == 256 && f.H % 256 != 0) bn_y = 128;
}

int launch_expert_ffn(const FfnLaunch& f, const WsLayout& L, char* ws, hipStream_t stream) {
  const moe_plan_t& p = *f.plan;
  const bool fp8 = f.dtype == MOE_FP8_E4M3_G128;
  const bool mx = f.dtype == MOE_MXFP4;
  const int H = f.H, I = f.I, tile = p.tile;
  const int eb = fp8 || mx ? 1 : 2;  // bytes per activation element
  int bn_a, bn_y;
  pick_block_n(f, tile, bn_a, bn_y);
  uint8_t* h = reinterpret_cast<uint8_t*>(ws + L.h);
  float* hs = fp8 ? reinterpret_cast<float*>(ws + L.hs) : nullptr;
  uint8_t* hs8 = mx ? reinterpret_cast<uint8_t*>(ws + L.hs) : nullptr;
  // combine on completion runs in the big-tile GEMM Y kernel; elsewhere the combine
  // kernel follows the FFN on the same stream
  const bool fuse = f.comb_out != nullptr && bn_y == 512;
  const int ntiles_cap = std::min(p.rows_cap, f.pool_rows) / tile;

  FfnArgs a{};
  a.tile_shift = __builtin_ctz((unsigned)tile);
  a.max_tiles = f.pool_rows / tile;
  a.n_experts = p.E_local;
  a.offsets = p.offsets;
  a.num_tiles = p.num_tiles;
  a.tile_expert = p.tile_expert;
  a.tile_ready = p.tile_ready;
  a.epoch = f.epoch;
  a.err = reinterpret_cast<uint32_t*>(ws + L.err);
  a.abort_epoch = reinterpret_cast<uint32_t*>(ws + L.abort);
  a.timeout = f.timeout_ticks;
  a.a_stages = f.a_stages;
  if (f.g_pool != nullptr) {
    a.g_save = static_cast<uint8_t*>(f.g_pool);
    a.g_ld = (int64_t)4 * I;
  }
  if (fuse) {
    a.ydone = reinterpret_cast<uint32_t*>(ws + L.ydone);
    a.cq = reinterpret_cast<uint32_t*>(ws + L.cq);
    a.pos = p.pos;
    a.topk_w = f.topk_w;
    a.comb_out = static_cast<uint8_t*>(f.comb_out);
    a.T = p.T;
    a.K = p.K;
    a.pool_rows = f.pool_rows;
  }

  // GEMM A: pool x w1^T -> SwiGLU -> h
  a.A = static_cast<const uint8_t*>(f.pool);
  a.A_s = fp8 ? static_cast<const float*>(f.pool_s) : nullptr;
  a.B = static_cast<const uint8_t*>(f.w1);
  a.B_s = fp8 ? static_cast<const float*>(f.w1_s) : nullptr;
  a.out = h;
  a.out_s = hs;
  a.A_e8 = mx ? static_cast<const uint8_t*>(f.pool_s) : nullptr;
  a.B_e8 = mx ? static_cast<const uint8_t*>(f.w1_s) : nullptr;
  a.out_e8 = hs8;
  a.b_e8_expert = (int64_t)2 * I * (H / 32);
  a.ksteps = H * eb / 128;
  a.lda = (int64_t)H * eb;
  a.b_expert = mx ? (int64_t)2 * I * (H / 2) : (int64_t)2 * I * H * eb;
  a.ldb = (int64_t)H * eb;
  a.up_row0 = I;
  a.ldo = (int64_t)I * eb;
  a.n_units = I / (bn_a / 2);
  a.s_kblocks = H / 128;
  a.bs_ld = H / 128;
  a.bs_expert = (int64_t)(2 * I / 128) * (H / 128);
  a.out_groups = I / 128;
  a.wait_ready = 1;
  a.tiles_done = reinterpret_cast<const uint32_t*>(ws + L.tiles_done);
  a.unit_order = bn_a == 512 ? (f.unit_order ? f.unit_order : mx ? 1 : 3) : 1;   // mxfp4: tiles then N blocks measured 1% faster
  const bool packed = f.weight_layout == MOE_WEIGHTS_MFMA_TILED;
  a.ktiles = H / (fp8 || mx ? 128 : 32);

  // 256-row units wherever they take the shape (unless 128 is asked for); the 128 x 512
  // units otherwise
  const bool sq = f.unit_rows != 128 && ffn_sq_ok(H, I, f.dtype, tile, f.block_n, f.weight_layout,
                                                  f.comb_out != nullptr);
  if (sq) {
    int grid = f.workgroups > 0 ? f.workgroups : device_cu_count();
    if (grid <= 0) return MOE_ERR_HIP;
    SqArgs q{};
    q.n_experts = p.E_local;
    q.max_tiles = f.pool_rows / 128;
    q.group = f.unit_order > 0 ? f.unit_order : 6;
    q.offsets = p.offsets;
    q.counts = p.counts;
    q.num_tiles = p.num_tiles;
    q.tile_ready = p.tile_ready;
    q.tiles_done = reinterpret_cast<const uint32_t*>(ws + L.tiles_done);
    q.epoch = f.epoch;
    q.err = reinterpret_cast<uint32_t*>(ws + L.err);
    q.abort_epoch = reinterpret_cast<uint32_t*>(ws + L.abort);
    q.timeout = f.timeout_ticks;
    // at most this many tile pairs (the tiles plus one odd tile per expert)
    const int64_t pairs_cap = (int64_t)ntiles_cap / 2 + p.E_local;
    // GEMM A: pool x w1^T -> SwiGLU -> h (and G when training)
    q.A = static_cast<const uint8_t*>(f.pool);
    q.lda = (int64_t)H * 2;
    q.B = static_cast<const uint8_t*>(f.w1);
    q.b_expert = (int64_t)2 * I * H * 2;
    q.ktiles = H / 32;
    q.out = h;
    q.ldo = (int64_t)I * 2;
    q.g_save = static_cast<uint8_t*>(f.g_pool);
    q.g_ld = (int64_t)4 * I;
    q.g_up = 2 * I;
    q.KS = H / 32;
    q.NB = 2 * I / 256;
    q.up_rb = I / 16;
    q.wait_ready = 1;
    int ga = std::max(1, (int)std::min<int64_t>(std::max(1, grid - f.dispatch_cus), pairs_cap * q.NB));
    // with the unit shape left to the library, GEMM A is launched on both kernels and the plan
    // decides on the device which one computes (sq_gemm_a_wins); the other returns at once
    const bool dual = f.unit_rows == 0 && bn_a == 512 && packed && big_a_ok(H, I, f.dtype, tile);
    const int ga_big = std::max(1, (int)std::min<int64_t>(std::max(1, grid - f.dispatch_cus),
                                                          (int64_t)ntiles_cap * a.n_units));
    const SqSelect sel{q.NB, ga, a.n_units, ga_big};
    q.select = dual ? 1 : 0;
    q.sel = sel;
    int rc = launch_ffn_sq(q, ga, true, f.g_pool != nullptr, stream);
    if (rc != MOE_OK) return rc;
    if (dual) {
      a.select = 1;
      a.sel = sel;
      rc = launch_shape<false, true>(tile, bn_a, packed, a, ga_big, stream);
      if (rc != MOE_OK) return rc;
      if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
      a.select = 0;
    }
    // GEMM Y: h x w2^T -> y_pool (same stream, so every h row is complete)
    q.A = h;
    q.lda = (int64_t)I * 2;
    q.B = static_cast<const uint8_t*>(f.w2);
    q.b_expert = (int64_t)H * I * 2;
    q.ktiles = I / 32;
    q.out = static_cast<uint8_t*>(f.y_pool);
    q.ldo = (int64_t)H * 2;
    q.g_save = nullptr;
    q.KS = I / 32;
    q.NB = H / 256;
    q.up_rb = 0;
    q.wait_ready = 0;
    q.select = 0;   // GEMM Y always runs on the 256-row units
    int gy = (int)std::min<int64_t>(grid, pairs_cap * q.NB);
    return launch_ffn_sq(q, std::max(1, gy), false, false, stream);
  }

  int grid = f.workgroups > 0 ? f.workgroups : device_cu_count();
  if (grid <= 0) return MOE_ERR_HIP;
  // GEMM A waits on flags that a concurrent dispatch raises: its persistent grid leaves
  // dispatch_cus CUs free (one workgroup fills a CU), so that dispatch can always run
  int ga = (int)std::min<int64_t>(std::max(1, grid - f.dispatch_cus), (int64_t)ntiles_cap * a.n_units);
  if (ga < 1) ga = 1;
  int rc = mx    ? launch_mx<true>(tile, bn_a, packed, a, ga, stream)
           : fp8 ? launch_shape<true, true>(tile, bn_a, packed, a, ga, stream)
                 : launch_shape<false, true>(tile, bn_a, packed, a, ga, stream);
  if (rc != MOE_OK) return rc;
  if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;

  // GEMM Y: h x w2^T -> y_pool (same stream, so every h row is complete)
  a.g_save = nullptr;
  a.A = h;
  a.A_s = hs;
  a.B = static_cast<const uint8_t*>(f.w2);
  a.B_s = fp8 ? static_cast<const float*>(f.w2_s) : nullptr;
  a.out = static_cast<uint8_t*>(f.y_pool);
  a.out_s = nullptr;
  a.A_e8 = hs8;
  a.B_e8 = mx ? static_cast<const uint8_t*>(f.w2_s) : nullptr;
  a.out_e8 = nullptr;
  a.b_e8_expert = (int64_t)H * (I / 32);
  a.ksteps = I * eb / 128;
  a.lda = (int64_t)I * eb;
  a.b_expert = mx ? (int64_t)H * (I / 2) : (int64_t)H * I * eb;
  a.ldb = (int64_t)I * eb;
  a.up_row0 = 0;
  a.ldo = (int64_t)H * 2;
  a.n_units = H / bn_y;
  a.s_kblocks = I / 128;
  a.bs_ld = I / 128;
  a.bs_expert = (int64_t)(H / 128) * (I / 128);
  a.wait_ready = 0;
  a.unit_order = bn_y == 512 ? (f.unit_order ? f.unit_order : mx ? 1 : 3) : 1;
  int gy = (int)std::min<int64_t>(grid, (int64_t)ntiles_cap * a.n_units);
  if (gy < 1) gy = 1;
  if (fuse) {
    // every workgroup must be able to be resident at once (its combine waits on the
    // units of the others), and the combine items want the whole device
    const int cus = std::max(1, device_cu_count());
    gy = std::min(grid, cus);
  }
  a.ktiles = I / (fp8 || mx ? 128 : 32);
  rc = mx    ? launch_mx<false>(tile, bn_y, packed, a, gy, stream)
       : fp8 ? launch_shape<true, false>(tile, bn_y, packed, a, gy, stream)
             : launch_shape<false, false>(tile, bn_y, packed, a, gy, stream);
  if (rc != MOE_OK) return rc;
  if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
  if (f.comb_out != nullptr && !fuse)
    return launch_combine(f.y_pool, f.pool_rows, f.topk_w, p, H, f.comb_out, stream);
  return MOE_OK;
}

// Backward data gradients on the big-tile kernel (bf16, tiled transposed weights):
// out[rows][N] = A[rows][K] . Bt[e]^T per pool tile, Bt[e] = w[e]^T in fragment order.
// epi 1 (backward GEMM Y): A = dy, Bt = W2^T [I][H], N = I; the epilogue turns dh into
// dG in place of G (g_pool [rows][2I]); its units wait for the ready flags that combine
// backward raises, as forward GEMM A's wait for dispatch's. epi 0 (backward GEMM A):
// A = dG, Bt = W1^T [H][2I], N = H, out = dx_pool.
int launch_ffn_dgrad(const moe_plan_t& p, int32_t pool_rows, const void* A, const void* Bt, int32_t N, int32_t K,
                     void* out, void* g_pool, int32_t I, int epi, int32_t workgroups, int32_t unit_order,
                     int32_t a_stages, uint32_t wait_epoch, uint64_t timeout_ticks, int32_t leave_cus,
                     const WsLayout& L, char* ws, hipStream_t stream) {
  const int tile = p.tile;
  FfnArgs a{};
  a.tile_shift = __builtin_ctz((unsigned)tile);
  a.max_tiles = pool_rows / tile;
  a.n_experts = p.E_local;
  a.offsets = p.offsets;
  a.num_tiles = p.num_tiles;
  a.tile_expert = p.tile_expert;
  a.tile_ready = p.tile_ready;
  a.err = reinterpret_cast<uint32_t*>(ws + L.err);
  a.abort_epoch = reinterpret_cast<uint32_t*>(ws + L.abort);
  a.A = static_cast<const uint8_t*>(A);
  a.B = static_cast<const uint8_t*>(Bt);
  a.out = static_cast<uint8_t*>(out);
  a.ksteps = K * 2 / 128;
  a.lda = (int64_t)K * 2;
  a.b_expert = (int64_t)N * K * 2;
  a.ldb = (int64_t)K * 2;
  a.up_row0 = epi == 1 ? I : 0;
  a.ldo = (int64_t)N * 2;
  a.n_units = N / 512;
  a.wait_ready = wait_epoch != 0 ? 1 : 0;
  a.epoch = wait_epoch;
  a.timeout = timeout_ticks;
  a.unit_order = unit_order ? unit_order : 3;
  a.ktiles = K / 32;
  a.g_save = static_cast<uint8_t*>(g_pool);
  a.g_ld = (int64_t)4 * I;
  int grid = workgroups > 0 ? workgroups : device_cu_count();
  if (grid <= 0) return MOE_ERR_HIP;
  grid = std::max(1, grid - leave_cus);
  const int ntiles_cap = std::min(p.rows_cap, pool_rows) / tile;
  grid = (int)std::max<int64_t>(1, std::min<int64_t>(grid, (int64_t)ntiles_cap * a.n_units));
  constexpr int NW = kBigWaves;
  const bool ring = a.ksteps % 4 == 0 && a_stages != 2;
  if (tile == 128 && ring) {
    if (epi == 1) hipLaunchKernelGGL((ffn_big_kernel<128, NW, false, false, true, false, 1, true>), dim3(grid), dim3(64 * NW), 0, stream, a);
    else hipLaunchKernelGGL((ffn_big_kernel<128, NW, false, false, true, false, 0, true>), dim3(grid), dim3(64 * NW), 0, stream, a);
  } else if (tile == 128) {
    if (epi == 1) hipLaunchKernelGGL((ffn_big_kernel<128, NW, false, false, true, false, 1>), dim3(grid), dim3(64 * NW), 0, stream, a);
    else hipLaunchKernelGGL((ffn_big_kernel<128, NW, false, false, true, false, 0>), dim3(grid), dim3(64 * NW), 0, stream, a);
  } else if (tile == 64) {
    if (epi == 1) hipLaunchKernelGGL((ffn_big_kernel<64, NW, false, false, true, false, 1>), dim3(grid), dim3(64 * NW), 0, stream, a);
    else hipLaunchKernelGGL((ffn_big_kernel<64, NW, false, false, true, false, 0>), dim3(grid), dim3(64 * NW), 0, stream, a);
  } else {
    return MOE_ERR_UNSUPPORTED;
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
