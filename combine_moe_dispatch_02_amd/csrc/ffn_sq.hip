// A3 + A4 on 256 x 256 work units: the expert FFN's grouped GEMMs (bf16, MFMA-tiled
// weights, pool tile 128) with both operands brought into LDS by DMA.
//
// StreamEP README, "How it works": the forward grouped GEMMs "A" (w1, gate|up, then
// the activation) and "Y" (w2) read the expert-major, tile-padded pool as it stands
// and start on a pool tile once dispatch has marked it (per-tile streaming). The
// arithmetic is that of the 128 x 512 big-tile kernel (ffn.hip): one chain of
// v_mfma_f32_16x16x32_bf16 per output element over K in ascending order, the same
// SwiGLU epilogue, so h and y carry the same bits whichever kernel ran.
//
// Work unit = (expert e, two consecutive pool tiles m, m+1 of e, N block j of 256
// columns); an expert with an odd tile count ends with a one-tile unit, whose second
// row half (rows of the next segment, outside the DMA range) is computed from zeros and
// not stored. GEMM A's N block is 128 gate columns and
// the matching 128 up columns of w1, so SwiGLU stays in the lane that holds both.
// 8 waves: wave w computes rows 128 (w / 4) .. +128 and 64 of the 256 columns
// (w % 4), i.e. 8 x 4 MFMA tiles, 128 accumulators per lane.
//
// Operands. The pool (or h) rows move in K stages of 64 values, 128 bytes a row (one
// cache line): 256 rows, 32 KiB. They are stored row by row, their eight 16-byte chunks
// XOR-permuted by row % 8: the eight lanes of a DMA that fill one row fetch its whole
// line, and the eight lanes of a fragment read that share a chunk index (eight rows)
// land on eight distinct 16-byte slots of a 128-byte bank row. The weights move in K
// stages of 32 values: the tiled layout already holds MFMA fragments as contiguous 1 KiB
// blocks (lane l's 16 bytes = row l % 16, K values 8 (l / 16) .. +8 of a 32-wide K tile),
// 16 of them per stage (16 KiB), which the DMA copies as they are. Rows past the unit's
// real rows (a segment's padding) lie outside the DMA's buffer range: they are not
// fetched and land as zeros. Each wave issues its share by LDS-DMA (buffer_load ... lds),
// so no register holds a load in flight, and every request covers whole cache lines.
//
// Pipeline, in steps of 32 K values. Weights: a ring of four 16 KiB stages, three steps
// ahead. Pool rows: two 32 KiB stages of 64 K values, the next one loaded during the
// current one (issued at its first step, used two steps later). About 80 KiB per CU are
// in flight. Step s: wait for this wave's DMAs that step s reads (vmcnt), barrier (every
// wave's are in; the stages step s - 1 read are free), issue the DMAs of weight stage
// s + 3 and, on even steps, of pool-row stage s / 2 + 1, then the MFMAs of step s. The
// stages run on across units: the last steps of a unit load the next unit's first
// stages, so a unit's epilogue overlaps them. The last MFMA group of each step is
// issued after the next barrier, while the next step's first fragment reads are in
// flight. The stages are separate LDS objects used with constant indices (the K loop
// runs four steps per round), so the compiler can tell a step's reads from the DMA
// writes in flight to the other stages and adds no wait of its own.
//
// Output. Each wave stages one 16-row MFMA tile row at a time in its own 2 KiB of LDS
// (no barrier: a wave's LDS accesses complete in order) and stores whole row segments:
// 128 bytes (y, or G in training) or 64 bytes (h) per row.
//
// Ready flags. GEMM A starts on a tile once dispatch has marked it. If dispatch's
// count of marked tiles already equals the tile count when a wave starts (dispatch
// ran before, e.g. on the same stream), one acquire covers every tile; otherwise the
// wave waits on the flags of each unit's tiles before it loads them. A wait that
// outlasts the timeout records MOE_ERR_TIMEOUT and marks the call's epoch aborted,
// which ends the call's other waits; the unit is then computed from whatever the pool
// holds (the error says the results are invalid).
#include <type_traits>

#include "common.h"
#include "ffn_sq.h"
#include "kernels.h"

namespace moe {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kSqWaves = 8;
constexpr int kAStage = 32768;   // 256 pool rows x 128 bytes (64 K values)
constexpr int kBStage = 16384;   // 16 weight row blocks x 1 KiB (32 K values)

__device__ inline float sq_silu_mul(float g, float u) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u; }

// DMA sources of one unit for this wave: the unit's rows (A) and its expert's tiled
// weights (B), and the byte offsets of the wave's two B row blocks
struct SqSrc {
  __amdgpu_buffer_rsrc_t ar, br;
  uint32_t b0, b1;
};

template <bool GEMM_A>
__device__ __attribute__((always_inline)) inline SqSrc sq_src(const SqArgs& a, const SqUnit& U, int w) {
  SqSrc s;
  // the unit's real rows only: padding rows are not fetched
  const int real = __builtin_amdgcn_readfirstlane(min(U.two ? 256 : 128, a.offsets[U.e] + a.counts[U.e] - U.m * 128));
  s.ar = make_rsrc(a.A + (int64_t)U.m * 128 * a.lda, (uint32_t)(max(real, 0) * a.lda));
  s.br = make_rsrc(a.B + (int64_t)U.e * a.b_expert, (uint32_t)a.b_expert);
  // B blocks 2w, 2w + 1 of the unit's 16: GEMM A gate blocks 0..7, up blocks 8..15
  const int rb = GEMM_A ? (w < 4 ? U.j * 8 + 2 * w : a.up_rb + U.j * 8 + 2 * (w - 4)) : U.j * 16 + 2 * w;
  s.b0 = (uint32_t)rb * (uint32_t)a.ktiles * 1024u;
  s.b1 = s.b0 + (uint32_t)a.ktiles * 1024u;
  return s;
}

}  // namespace

template <bool GEMM_A, bool GSAVE>
__global__ __launch_bounds__(64 * kSqWaves, 1) void ffn_sq_kernel(SqArgs a) {
  static_assert(!GSAVE || GEMM_A, "G is kept by GEMM A");
  __shared__ __attribute__((aligned(16))) uint8_t s_a0[kAStage];
  __shared__ __attribute__((aligned(16))) uint8_t s_a1[kAStage];
  __shared__ __attribute__((aligned(16))) uint8_t s_b0[kBStage];
  __shared__ __attribute__((aligned(16))) uint8_t s_b1[kBStage];
  __shared__ __attribute__((aligned(16))) uint8_t s_b2[kBStage];
  __shared__ __attribute__((aligned(16))) uint8_t s_b3[kBStage];
  __shared__ __attribute__((aligned(16))) uint8_t s_out[kSqWaves * 2048];
  __shared__ int32_t s_ru[kMaxExpertsSq + 1];
  __shared__ int s_sel;
  auto aring = [&](auto ST) __attribute__((always_inline)) -> uint8_t* {
    if constexpr (decltype(ST)::value == 0) return s_a0;
    else return s_a1;
  };
  auto bring = [&](auto ST) __attribute__((always_inline)) -> uint8_t* {
    constexpr int k = decltype(ST)::value;
    if constexpr (k == 0) return s_b0;
    else if constexpr (k == 1) return s_b1;
    else if constexpr (k == 2) return s_b2;
    else return s_b3;
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg = w >> 2;   // row half of the unit
  const int cg = w & 3;    // column quarter of the unit

  int ntiles = a.num_tiles[0];
  if (ntiles > a.max_tiles) {
    if (blockIdx.x == 0 && tid == 0) record_error(a.err, MOE_ERR_INVALID);
    ntiles = a.max_tiles;
  }
  // row units per expert, prefix-summed; whether this launch is the call's GEMM A
  if (w == 0) {
    sq_row_units(a, s_ru, lane);
    if (a.select) {
      const bool win = sq_gemm_a_wins(a.offsets, a.n_experts, a.max_tiles, a.sel, lane);
      if (lane == 0) s_sel = win ? 1 : 0;
    }
  }
  __syncthreads();
  if (a.select && !s_sel) return;
  const int total = __builtin_amdgcn_readfirstlane(s_ru[a.n_experts] * a.NB);
  const int G = gridDim.x;
  int u = unit_slot(blockIdx.x, G);
  if (u >= total) return;

  // one acquire for every tile when dispatch has already marked them all
  bool poll_each = false;
  if (a.wait_ready) {
    const uint32_t done = __hip_atomic_load(a.tiles_done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    poll_each = done < (uint32_t)ntiles;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }

  const int KS = a.KS;
  // this wave's DMA lanes: pool rows 32w .. 32w + 31 of the unit, 8 rows per DMA; lane i fills
  // LDS bytes 16i .. 16i + 15 of a DMA's 1 KiB, i.e. row i / 8, chunk slot i % 8, which holds
  // the row's chunk (i % 8) ^ (row % 8)
  const uint32_t lda = (uint32_t)a.lda;
  const uint32_t a_vo = (uint32_t)(32 * w + (lane >> 3)) * lda + 16u * (uint32_t)((lane & 7) ^ ((lane >> 3) & 7));
  const uint32_t b_vo = 16u * (uint32_t)lane;
  // fragment read of pool rows: lane l takes row l % 16, chunk 4 kk + l / 16 of the stage
  const int a_frag0 = (lane & 15) * 128 + ((((lane >> 4)) ^ (lane & 7)) << 4);
  const int a_frag1 = (lane & 15) * 128 + (((4 + (lane >> 4)) ^ (lane & 7)) << 4);
  typedef __attribute__((address_space(3))) void* lds_t;
  // one DMA of pool-row stage kd (64 K values): rows 32w + 8q .. +8
  auto dma_a1 = [&](auto ST, const SqSrc& s, int kd, int q) __attribute__((always_inline)) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(s.ar, (lds_t)(aring(ST) + (4 * w + q) * 1024), 16, a_vo + 8u * q * lda,
                                             (uint32_t)kd * 128u, 0, 0);
  };
  // one DMA of weight stage kb (32 K values): this wave's row block 2w + q
  auto dma_b1 = [&](auto ST, const SqSrc& s, int kb, int q) __attribute__((always_inline)) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(s.br, (lds_t)(bring(ST) + (2 * w + q) * 1024), 16, b_vo,
                                             (q ? s.b1 : s.b0) + (uint32_t)kb * 1024u, 0, 0);
  };
  auto dma_a = [&](auto ST, const SqSrc& s, int kd) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 4; ++q) dma_a1(ST, s, kd, q);
  };
  auto dma_b = [&](auto ST, const SqSrc& s, int kb) __attribute__((always_inline)) {
    dma_b1(ST, s, kb, 0);
    dma_b1(ST, s, kb, 1);
  };
  // B row blocks of this wave's MFMA column tiles: GEMM A gate 2cg, 2cg + 1, up 8 + 2cg, 8 + 2cg + 1
  auto bblk = [&](int tn) __attribute__((always_inline)) { return GEMM_A ? (tn < 2 ? 2 * cg + tn : 8 + 2 * cg + (tn - 2)) : 4 * cg + tn; };

  SqUnit cur = sq_unit(a, s_ru, u);
  if (poll_each) sq_wait_tiles(a, cur);
  SqSrc cs = sq_src<GEMM_A>(a, cur, w);
  // the first unit's stages in the order the steady state issues them: weights 0, pool rows
  // 0 and weights 1 (as at step -2), weights 2 (step -1)
  dma_b(I0{}, cs, 0);
  dma_a(I0{}, cs, 0);
  dma_b(I1{}, cs, 1);
  dma_b(I2{}, cs, 2);

  f32x4_t acc[8][4];
  bf16x8_t fbp[4], fap;   // the previous stage's last MFMA group, issued after the next barrier

  for (;;) {
    const int un = u + G;
    const bool has_next = un < total;
    const SqUnit nx = has_next ? sq_unit(a, s_ru, un) : cur;
    const SqSrc ns = sq_src<GEMM_A>(a, nx, w);
    const bool store = rg == 0 || cur.two;   // a one-tile unit's second row half is not stored
#pragma unroll
    for (int tm = 0; tm < 8; ++tm)
#pragma unroll
      for (int tn = 0; tn < 4; ++tn) acc[tm][tn] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int tn = 0; tn < 4; ++tn) fbp[tn] = bf16x8_t{};
    fap = bf16x8_t{};   // zero operands: the first step's deferred group adds exactly 0

    // step ks (32 K values), ks % 4 = ST: weights from stage ST, pool rows from stage ST / 2,
    // K half ST % 2 of it
    auto step = [&](auto ST, int ks) __attribute__((always_inline)) {
      constexpr int st = decltype(ST)::value;
      using AS = std::integral_constant<int, st / 2>;          // pool-row stage read
      using AN = std::integral_constant<int, (st / 2) ^ 1>;    // pool-row stage loaded (even steps)
      using BN = std::integral_constant<int, (st + 3) & 3>;    // weight stage loaded
      constexpr bool EVEN = (st & 1) == 0;
      __builtin_amdgcn_sched_barrier(0);
      // this wave's DMAs that step ks reads are in (even steps: pool rows ks / 2 and weights
      // ks, with weights ks + 1, ks + 2 in flight behind them; odd steps: weights ks, with
      // weights ks + 1, pool rows ks / 2 + 1 and weights ks + 2 behind them); its reads of
      // step ks - 1 are done
      __builtin_amdgcn_s_waitcnt(vmcnt_enc(EVEN ? 4 : 8));
      __builtin_amdgcn_s_waitcnt(kLgkm0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      // even steps: pool-row stage ks / 2 + 1 (this unit's, the next unit's first, or a reload
      // nobody reads when there is no next unit); every step: weight stage ks + 3, likewise.
      // The DMAs go out one per MFMA group, pool rows first (the wait counts above rely on
      // that order), so that issuing them never holds the wave off its MFMAs for long.
      const int kd0 = (ks >> 1) + 1;
      const bool a_next = kd0 >= (KS >> 1);
      if constexpr (EVEN) {
        if (a_next && has_next && poll_each) sq_wait_tiles(a, nx);
      }
      const bool an = a_next && has_next;
      __amdgpu_buffer_rsrc_t d_ar = cs.ar;
      if (an) d_ar = ns.ar;
      const uint32_t d_ak = (uint32_t)(a_next ? (has_next ? 0 : (KS >> 1) - 1) : kd0) * 128u;
      const int kb0 = ks + 3;
      const bool b_next = kb0 >= KS;
      const bool bn = b_next && has_next;
      __amdgpu_buffer_rsrc_t d_br = cs.br;
      if (bn) d_br = ns.br;
      const uint32_t d_bk = (uint32_t)(b_next ? (has_next ? kb0 - KS : KS - 1) : kb0) * 1024u;
      const uint32_t d_b0 = (bn ? ns.b0 : cs.b0) + d_bk, d_b1 = (bn ? ns.b1 : cs.b1) + d_bk;
      // the DMA of group g (0 .. 5 on even steps, 0 .. 1 on odd ones)
      auto dma_g = [&](int g) __attribute__((always_inline)) {
        if (EVEN && g < 4) {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(d_ar, (lds_t)(aring(AN{}) + (4 * w + g) * 1024), 16,
                                                   a_vo + 8u * (uint32_t)g * lda, d_ak, 0, 0);
        } else {
          const int q = EVEN ? g - 4 : g;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(d_br, (lds_t)(bring(BN{}) + (2 * w + q) * 1024), 16, b_vo,
                                                   q ? d_b1 : d_b0, 0, 0);
        }
      };
      constexpr int NDMA = EVEN ? 6 : 2;
      __builtin_amdgcn_sched_barrier(0);
      {
        const uint8_t* sa = aring(AS{}) + (rg * 128) * 128 + (EVEN ? a_frag0 : a_frag1);
        const uint8_t* sb = bring(ST) + 16 * lane;
        bf16x8_t fb[4];
#pragma unroll
        for (int tn = 0; tn < 4; ++tn) fb[tn] = *reinterpret_cast<const bf16x8_t*>(sb + bblk(tn) * 1024);
        bf16x8_t fa = *reinterpret_cast<const bf16x8_t*>(sa);
        // the previous step's last group
#pragma unroll
        for (int tn = 0; tn < 4; ++tn)
          acc[7][tn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fbp[tn], fap, acc[7][tn], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma clang loop unroll(full)
        for (int tm = 0; tm < 7; ++tm) {
          if (tm < NDMA) dma_g(tm);
          const bf16x8_t fn = *reinterpret_cast<const bf16x8_t*>(sa + ((tm + 1) * 16) * 128);
#pragma unroll
          for (int tn = 0; tn < 4; ++tn)
            acc[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[tn], fa, acc[tm][tn], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
          fa = fn;
        }
        fap = fa;
#pragma unroll
        for (int tn = 0; tn < 4; ++tn) fbp[tn] = fb[tn];
      }
    };

    for (int ks = 0; ks < KS; ks += 4) {
      step(I0{}, ks);
      step(I1{}, ks + 1);
      step(I2{}, ks + 2);
      step(I3{}, ks + 3);
    }

#pragma unroll
    for (int tn = 0; tn < 4; ++tn)
      acc[7][tn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fbp[tn], fap, acc[7][tn], 0, 0, 0);
    if (store) {
      // ---- epilogue: lane holds row tm*16 + (lane & 15), columns 4 (lane >> 4) + (0..3) of each tile
      uint8_t* so = s_out + w * 2048;
      const int64_t row0 = (int64_t)cur.m * 128 + rg * 128;
      const int r = lane & 15;
      if constexpr (GEMM_A) {
#pragma unroll
        for (int tm = 0; tm < 8; ++tm) {
          if constexpr (GSAVE) {
            // G = [gate | up] before the activation: the wave's 32 gate and 32 up columns
            // as one 128-byte staging row, then 64-byte segments of the gate and up halves
#pragma unroll
            for (int tn = 0; tn < 4; ++tn) {
              u32x2 v;
              v.x = pack_bf16x2(acc[tm][tn][0], acc[tm][tn][1]);
              v.y = pack_bf16x2(acc[tm][tn][2], acc[tm][tn][3]);
              const int b = tn * 32 + 8 * (lane >> 4);
              *reinterpret_cast<u32x2*>(so + r * 128 + ((((b >> 4) ^ (r & 7))) << 4) + (b & 15)) = v;
            }
#pragma unroll
            for (int p = 0; p < 2; ++p) {
              const int rr = p * 8 + (lane >> 3), c = lane & 7;
              const u32x4 v = *reinterpret_cast<const u32x4*>(so + rr * 128 + ((c ^ (rr & 7)) << 4));
              const int64_t col = (c < 4 ? 0 : a.g_up) + (int64_t)(cur.j * 128 + cg * 32) * 2 + (c & 3) * 16;
              *reinterpret_cast<u32x4*>(a.g_save + (row0 + tm * 16 + rr) * a.g_ld + col) = v;
            }
          }
          // h = silu(gate) * up: 16 rows x 32 columns, staged as 64-byte rows
#pragma unroll
          for (int tn = 0; tn < 2; ++tn) {
            u32x2 v;
            v.x = pack_bf16x2(sq_silu_mul(acc[tm][tn][0], acc[tm][tn + 2][0]),
                              sq_silu_mul(acc[tm][tn][1], acc[tm][tn + 2][1]));
            v.y = pack_bf16x2(sq_silu_mul(acc[tm][tn][2], acc[tm][tn + 2][2]),
                              sq_silu_mul(acc[tm][tn][3], acc[tm][tn + 2][3]));
            const int b = tn * 32 + 8 * (lane >> 4);
            *reinterpret_cast<u32x2*>(so + r * 64 + ((((b >> 4) ^ ((r >> 2) & 3))) << 4) + (b & 15)) = v;
          }
          {
            const int rr = lane >> 2, c = lane & 3;
            const u32x4 v = *reinterpret_cast<const u32x4*>(so + rr * 64 + ((c ^ ((rr >> 2) & 3)) << 4));
            *reinterpret_cast<u32x4*>(a.out + (row0 + tm * 16 + rr) * a.ldo + (cur.j * 128 + cg * 32) * 2 + c * 16) = v;
          }
        }
      } else {
#pragma unroll
        for (int tm = 0; tm < 8; ++tm) {
#pragma unroll
          for (int tn = 0; tn < 4; ++tn) {
            u32x2 v;
            v.x = pack_bf16x2(acc[tm][tn][0], acc[tm][tn][1]);
            v.y = pack_bf16x2(acc[tm][tn][2], acc[tm][tn][3]);
            const int b = tn * 32 + 8 * (lane >> 4);
            *reinterpret_cast<u32x2*>(so + r * 128 + ((((b >> 4) ^ (r & 7))) << 4) + (b & 15)) = v;
          }
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            const int rr = p * 8 + (lane >> 3), c = lane & 7;
            const u32x4 v = *reinterpret_cast<const u32x4*>(so + rr * 128 + ((c ^ (rr & 7)) << 4));
            *reinterpret_cast<u32x4*>(a.out + (row0 + tm * 16 + rr) * a.ldo + (cur.j * 256 + cg * 64) * 2 + c * 16) = v;
          }
        }
      }
    }
    if (!has_next) break;
    u = un;
    cur = nx;
    cs = ns;
  }
  wait_vm0();   // the unread reloads of the last steps land before the workgroup ends
}

int launch_ffn_sq(const SqArgs& a, int grid, bool gemm_a, bool gsave, hipStream_t stream) {
  const dim3 g((unsigned)grid), b(64 * kSqWaves);
  if (gemm_a && gsave) hipLaunchKernelGGL((ffn_sq_kernel<true, true>), g, b, 0, stream, a);
  else if (gemm_a) hipLaunchKernelGGL((ffn_sq_kernel<true, false>), g, b, 0, stream, a);
  else hipLaunchKernelGGL((ffn_sq_kernel<false, false>), g, b, 0, stream, a);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
