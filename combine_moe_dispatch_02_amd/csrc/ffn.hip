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
// Main loop per 128-byte K step (64 bf16 or 128 e4m3 per row):
//   global -> registers (16-byte lanes) for step k+1 while step k runs on MFMA
//   from LDS; registers -> the other LDS buffer; one barrier per step.
// LDS rows are 128 bytes, 16-byte chunks XOR-swizzled by (row & 7), so the 8
// lanes that read one chunk column from 8 consecutive rows hit 8 different
// bank groups.
// bf16: v_mfma_f32_16x16x32_bf16, A/B fragments = 8 consecutive K values of one
// row per lane (lane l: row l%16, K chunk l/16).
// fp8: v_mfma_scale_f32_16x16x128_f8f6f4 with unit scales (E8M0 127), one per
// 128-wide K block, then acc += partial * a_scale[row] * b_scale[block] in fp32.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

struct FfnArgs {
  const uint8_t* A;          // pool (GEMM A) or h (GEMM Y): [rows][Kdim] elements
  const float* A_s;          // fp8: activation group scales [rows][Kdim/128]
  const uint8_t* B;          // w1 or w2, expert-major
  const float* B_s;          // fp8: weight block scales, expert-major
  uint8_t* out;              // h (GEMM A) or y_pool (GEMM Y)
  float* out_s;              // fp8 GEMM A: h group scales [rows][I/128]
  int32_t ksteps;            // K steps of 128 bytes
  int64_t lda;               // bytes per A row
  int64_t b_expert;          // bytes per expert of B
  int64_t ldb;               // bytes per B row
  int32_t up_row0;           // GEMM A: first up row of w1 (= I)
  int64_t ldo;               // bytes per out row
  int32_t n_units;           // N blocks per tile
  int32_t s_kblocks;         // fp8: Kdim / 128
  int32_t bs_ld;             // fp8: B scale row stride (= Kdim / 128)
  int64_t bs_expert;         // fp8: B scale entries per expert
  int32_t out_groups;        // fp8 GEMM A: I / 128
  int32_t tile_shift;
  int32_t max_tiles;         // pool_rows / tile: tiles the buffers hold
  const int32_t* num_tiles;
  const int32_t* tile_expert;
  const uint32_t* tile_ready;
  uint32_t epoch;
  uint32_t* err;
  uint64_t timeout;
  int32_t wait_ready;
};

__device__ inline uint32_t swz(int row, int chunk) { return (uint32_t)(row * 128 + ((chunk ^ (row & 7)) << 4)); }

__device__ inline float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

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
  for (int u = blockIdx.x; u < total; u += gridDim.x) {
    const int m = u / a.n_units;
    const int j = u - m * a.n_units;
    const int m0 = m * BM;
    const int e = a.tile_expert[m];

    if (a.wait_ready) {
      if (tid == 0) {
        int go = 1;
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        while (__hip_atomic_load(&a.tile_ready[m], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != a.epoch) {
          if (load_error(a.err) != 0) { go = 0; break; }
          if (__builtin_amdgcn_s_memrealtime() - t0 > a.timeout) {
            record_error(a.err, MOE_ERR_TIMEOUT);
            go = 0;
            break;
          }
          __builtin_amdgcn_s_sleep(4);
        }
        s_go = go;
      }
      __syncthreads();
      const int go = s_go;
      __syncthreads();  // s_go is rewritten for the next unit only after everyone read it
      if (!go) continue;
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }

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
        if (tid < BM) ras = a.A_s[(int64_t)(m0 + tid) * a.s_kblocks + kt];
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
            const int row = m0 + rl;
#pragma unroll
            for (int tn = 0; tn < G::kTN / 2; ++tn) {
              const int col = hcol0 + tn * 16 + l16;
              a.out[(int64_t)row * a.ldo + col] = (uint8_t)e4m3_from_f32(hv[tm][tn][i] / sc);
            }
            if (wn == 0 && l16 == 0) a.out_s[(int64_t)row * a.out_groups + ((j * (BN / 2)) >> 7)] = sc;
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
// host side
// ----------------------------------------------------------------------------
int ffn_supported(int32_t H, int32_t I, int32_t dtype, int32_t tile, int32_t block_n) {
  if (block_n != 0 && block_n != 128 && block_n != 256) return MOE_ERR_INVALID;
  if (dtype == MOE_BF16) {
    if (H % 128 != 0 || I % 64 != 0) return MOE_ERR_UNSUPPORTED;
    if (block_n == 256 && (tile < 64 || I % 128 != 0)) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
  }
  if (dtype == MOE_FP8_E4M3_G128) {
    if (H % 256 != 0 || I % 128 != 0 || tile < 64) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
  }
  return MOE_ERR_INVALID;
}

template <int BM, int BN, int WM, int WN, bool FP8, bool GEMM_A>
static void launch_one(const FfnArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((ffn_gemm_kernel<BM, BN, WM, WN, FP8, GEMM_A>), dim3(grid), dim3(256), 0, s, a);
}

template <bool FP8, bool GEMM_A>
static int launch_shape(int tile, int bn, const FfnArgs& a, int grid, hipStream_t s) {
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

int launch_expert_ffn(const FfnLaunch& f, const WsLayout& L, char* ws, hipStream_t stream) {
  const moe_plan_t& p = *f.plan;
  const bool fp8 = f.dtype == MOE_FP8_E4M3_G128;
  const int H = f.H, I = f.I, tile = p.tile;
  const int eb = fp8 ? 1 : 2;  // bytes per element
  // N block per GEMM: the largest the shape allows, unless overridden
  int bn_a, bn_y;
  if (fp8) {
    bn_a = 256;
    bn_y = 256;
  } else if (f.block_n) {
    bn_a = bn_y = f.block_n;
  } else {
    bn_a = (tile >= 64 && I % 128 == 0) ? 256 : 128;
    bn_y = (tile >= 64 && H % 256 == 0) ? 256 : 128;
  }
  if (!fp8 && bn_y == 256 && H % 256 != 0) bn_y = 128;
  uint8_t* h = reinterpret_cast<uint8_t*>(ws + L.h);
  float* hs = fp8 ? reinterpret_cast<float*>(ws + L.hs) : nullptr;
  const int ntiles_cap = std::min(p.rows_cap, f.pool_rows) / tile;

  FfnArgs a{};
  a.tile_shift = __builtin_ctz((unsigned)tile);
  a.max_tiles = f.pool_rows / tile;
  a.num_tiles = p.num_tiles;
  a.tile_expert = p.tile_expert;
  a.tile_ready = p.tile_ready;
  a.epoch = f.epoch;
  a.err = reinterpret_cast<uint32_t*>(ws + L.err);
  a.timeout = f.timeout_ticks;

  // GEMM A: pool x w1^T -> SwiGLU -> h
  a.A = static_cast<const uint8_t*>(f.pool);
  a.A_s = f.pool_s;
  a.B = static_cast<const uint8_t*>(f.w1);
  a.B_s = f.w1_s;
  a.out = h;
  a.out_s = hs;
  a.ksteps = H * eb / 128;
  a.lda = (int64_t)H * eb;
  a.b_expert = (int64_t)2 * I * H * eb;
  a.ldb = (int64_t)H * eb;
  a.up_row0 = I;
  a.ldo = (int64_t)I * eb;
  a.n_units = I / (bn_a / 2);
  a.s_kblocks = H / 128;
  a.bs_ld = H / 128;
  a.bs_expert = (int64_t)(2 * I / 128) * (H / 128);
  a.out_groups = I / 128;
  a.wait_ready = 1;
  int grid = f.workgroups > 0 ? f.workgroups : device_cu_count();
  if (grid <= 0) return MOE_ERR_HIP;
  int ga = (int)std::min<int64_t>(grid, (int64_t)ntiles_cap * a.n_units);
  if (ga < 1) ga = 1;
  int rc = fp8 ? launch_shape<true, true>(tile, bn_a, a, ga, stream)
               : launch_shape<false, true>(tile, bn_a, a, ga, stream);
  if (rc != MOE_OK) return rc;
  if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;

  // GEMM Y: h x w2^T -> y_pool (same stream, so every h row is complete)
  a.A = h;
  a.A_s = hs;
  a.B = static_cast<const uint8_t*>(f.w2);
  a.B_s = f.w2_s;
  a.out = static_cast<uint8_t*>(f.y_pool);
  a.out_s = nullptr;
  a.ksteps = I * eb / 128;
  a.lda = (int64_t)I * eb;
  a.b_expert = (int64_t)H * I * eb;
  a.ldb = (int64_t)I * eb;
  a.up_row0 = 0;
  a.ldo = (int64_t)H * 2;
  a.n_units = H / bn_y;
  a.s_kblocks = I / 128;
  a.bs_ld = I / 128;
  a.bs_expert = (int64_t)(H / 128) * (I / 128);
  a.wait_ready = 0;
  int gy = (int)std::min<int64_t>(grid, (int64_t)ntiles_cap * a.n_units);
  if (gy < 1) gy = 1;
  rc = fp8 ? launch_shape<true, false>(tile, bn_y, a, gy, stream)
           : launch_shape<false, false>(tile, bn_y, a, gy, stream);
  if (rc != MOE_OK) return rc;
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
