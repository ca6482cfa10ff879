// A3 + A4 on 256 x 256 work units: the expert FFN's grouped GEMMs (bf16, MFMA-tiled weights,
// pool tile 128) with both operands brought into LDS by DMA, four waves, one per SIMD.
//
// StreamEP README, "How it works": the forward grouped GEMMs "A" (w1, gate|up, then the
// activation) and "Y" (w2) read the expert-major, tile-padded pool as it stands and start
// on a pool tile once dispatch has marked it (per-tile streaming). The arithmetic is that
// of the 128 x 512 big-tile kernel (ffn.hip): one chain of v_mfma_f32_16x16x32_bf16 per
// output element over K in ascending order, the same SwiGLU epilogue, so h and y carry the
// same bits whichever kernel ran.
//
// Work unit = (expert e, two consecutive pool tiles m, m+1 of e, N block j of 256
// columns); an expert with an odd tile count ends with a one-tile unit, whose second row
// half (rows of the next segment, outside the DMA range) is computed from zeros and not
// stored. GEMM A's N block is 128 gate columns and the matching 128 up columns of w1. Wave
// w computes rows 128 (w / 2) .. +128 and 128 of the 256 columns (w % 2; in GEMM A 64 gate
// and the matching 64 up columns, so SwiGLU stays in the lane that holds both): 8 x 8 MFMA
// tiles, 256 accumulators per lane, kept in the accumulation registers. Per 32-wide K step
// a wave reads 16 fragments from LDS for 64 MFMAs.
//
// Operands. The pool (or h) rows move in K stages of 64 values, 128 bytes a row (one cache
// line): 256 rows, 32 KiB, stored row by row with their eight 16-byte chunks XOR-permuted
// by row % 8, so that the eight lanes of a DMA that fill one row fetch its whole line and
// the lanes of a fragment read that share a chunk index land on distinct banks. The weights
// move in K stages of 32 values: the tiled layout already holds MFMA fragments as
// contiguous 1 KiB blocks, 16 of them per stage (16 KiB), which the DMA copies as they
// are. Rows past the unit's real rows lie outside the DMA's buffer range: they are not
// fetched and land as zeros. Every wave issues its share by LDS-DMA (buffer_load ... lds).
//
// Pipeline, in steps of 32 K values. Weights: four 16 KiB stages, stage s loaded during
// step s - 4 into the stage that step s - 1 read. Pool rows: two 32 KiB stages, stage d
// loaded during step 2d - 3. With one wave per SIMD no other wave covers a wait, so the
// fragments of step s + 1 are read during step s (two register sets). Step s: the first
// kPre MFMAs; wait for this wave's DMAs of the stages read during s; barrier (every wave's
// are in, and every wave has finished reading the stages of step s, which the DMAs of this
// step overwrite); then the remaining MFMAs with the step's memory operations between them
// (sq_op): the fragment reads of step s + 1 and the DMAs of weight stage s + 4 and, on odd
// steps, pool-row stage (s + 3) / 2. The stage count runs on across units: a unit's last
// steps load the next unit's first stages, and its first step's fragments are read again
// after the epilogue. The stages are separate LDS objects used with constant indices (the K
// loop runs four steps per round), so the compiler can tell a step's reads from the DMA
// writes in flight and adds no wait of its own.
//
// Output. Each wave stages one 16-row MFMA tile row at a time in its own 4 KiB of LDS (no
// barrier: a wave's LDS accesses complete in order) and stores whole row segments (256
// bytes of y or G a row, 128 bytes of h) through a buffer resource over the unit's rows.
//
// Ready flags. GEMM A starts on a tile once dispatch has marked it. If dispatch's count of
// marked tiles already equals the tile count when a workgroup starts (dispatch ran before,
// e.g. on the same stream), one acquire covers every tile; otherwise each wave waits on the
// flags of each unit's tiles before it loads them. A wait that outlasts the timeout records
// MOE_ERR_TIMEOUT and marks the call's epoch aborted, which ends the call's other waits; the
// unit is then computed from whatever the pool holds (the error says the results are
// invalid).
#include <type_traits>
#include <utility>

#include "common.h"
#include "ffn_sq.h"
#include "kernels.h"

namespace moe {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kSqWaves = 4;
constexpr int kPre = 2;            // MFMAs of a step issued before its barrier
constexpr int kAStage = 32768;   // 256 pool rows x 128 bytes (64 K values)
constexpr int kBStage = 16384;   // 16 weight row blocks x 1 KiB (32 K values)
constexpr int kUnitSlots = 64;   // units of a workgroup decoded up front (later ones one by one)

__device__ inline float sq_silu_mul(float g, float u) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u; }

// DMA sources of one unit for this wave: the unit's rows (base and bytes), its expert's
// tiled weights and the byte offset of the first of the wave's four weight row blocks (the
// next three follow at ktiles KiB each). Kept as plain pointers and sizes: the buffer
// resources are made where they are used.
struct SqSrc {
  const uint8_t* abase;
  const uint8_t* bbase;
  uint32_t abytes, b0;
};

template <bool GEMM_A>
__device__ __attribute__((always_inline)) inline SqSrc sq_src(const SqArgs& a, const SqUnit& U, const int32_t* s_end,
                                                           int w) {
  SqSrc s;
  const int real = __builtin_amdgcn_readfirstlane(min(U.two ? 256 : 128, s_end[U.e] - U.m * 128));
  s.abase = a.A + (int64_t)U.m * 128 * a.lda;
  s.abytes = (uint32_t)(max(real, 0) * a.lda);
  s.bbase = a.B + (int64_t)U.e * a.b_expert;
  // B blocks 4w .. 4w + 3 of the unit's 16: GEMM A gate blocks 0..7, up blocks 8..15
  const int rb = GEMM_A ? (w < 2 ? U.j * 8 + 4 * w : a.up_rb + U.j * 8 + 4 * (w - 2)) : U.j * 16 + 4 * w;
  s.b0 = (uint32_t)rb * (uint32_t)a.ktiles * 1024u;
  return s;
}

// c += a x b on the matrix core, with c kept in the accumulation registers and updated in
// place. (Left to the compiler, the 256 accumulators of a wave do not stay put: it moves some
// of them through the vector registers between steps.) The compiler does not see this as an
// MFMA, so the wait states around it are the caller's: the accumulators are read back only
// after 24 wait states (three s_nop 7) behind the last MFMA. The 64 MFMAs of a step update 64
// different accumulators, so no MFMA reads one that the one before wrote. A unit's first
// step uses mfma_first, which reads no accumulator.
__device__ __attribute__((always_inline)) inline void mfma_acc(f32x4_t& c, bf16x8_t a, bf16x8_t b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}

// c = a x b (the accumulator input is the constant 0): a unit's first K step, so that the
// accumulators need no zeroing writes between units. Same wait-state rules as mfma_acc.
__device__ __attribute__((always_inline)) inline void mfma_first(f32x4_t& c, bf16x8_t a, bf16x8_t b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=a"(c) : "v"(a), "v"(b));
}

// the four accumulators of c into vector registers, where the caller asks for them (left to
// itself, the compiler copies all 256 out at once when the K loop ends)
__device__ __attribute__((always_inline)) inline f32x4_t acc_read(const f32x4_t& c) {
  float x, y, z, w;
  asm volatile("v_accvgpr_read_b32 %0, %4\n\tv_accvgpr_read_b32 %1, %5\n\tv_accvgpr_read_b32 %2, %6\n\tv_accvgpr_read_b32 %3, %7"
               : "=v"(x), "=v"(y), "=v"(z), "=v"(w)
               : "a"(c[0]), "a"(c[1]), "a"(c[2]), "a"(c[3]));
  return f32x4_t{x, y, z, w};
}

// The memory operation issued after MFMA i of a step (i >= kPre; MFMA i is that of
// accumulator row i / 8, column tile i % 8), as kind << 4 | index: 1 pool-row fragment read,
// 2 weight fragment read, 3 pool-row DMA, 4 weight DMA, 0 none. In each of the first four
// rows (the first one's shifted past the kPre MFMAs issued before the barrier): two pairs of
// fragment reads, with a DMA after each pair on odd steps (pool rows) and after the first
// pair of every other row on even steps (weights); on odd steps the weight DMAs follow in
// rows 4 .. 7. Six operations back to back, then two MFMAs without one, measured faster
// than the operations spread evenly or issued one per MFMA from the barrier on.
static_assert(kPre <= 2, "the first row keeps six slots");
constexpr int sq_op(bool odd, int i) {
  const int g = i >> 3;
  const int tn = (i & 7) - (g == 0 ? kPre : 0);
  if (tn < 0) return 0;
  if (g < 4) {
    if (tn == 0 || tn == 3) return 1 << 4 | (2 * g + (tn == 3));
    if (tn == 1 || tn == 4) return 2 << 4 | (2 * g + (tn == 4));
    if (odd && (tn == 2 || tn == 5)) return 3 << 4 | (2 * g + (tn == 5));
    if (!odd && (g & 1) == 0 && tn == 2) return 4 << 4 | (g >> 1);
    return 0;
  }
  if (tn != 2) return 0;
  if (odd) return 4 << 4 | (g - 4);
  return (g & 1) == 0 ? (4 << 4 | (g >> 1)) : 0;
}

// c ? x : y on values: the next unit's or this unit's source. (A conditional on the two
// structs' members would select between their addresses, and the compiler then keeps every
// variable the K loop touches in memory.)
template <typename V>
__device__ __attribute__((always_inline)) inline V pick(bool c, V x, V y) {
  return c ? x : y;
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
  __shared__ __attribute__((aligned(16))) uint8_t s_out[kSqWaves * 4096];
  __shared__ int32_t s_ru[kMaxExpertsSq + 1];
  __shared__ int32_t s_t0[kMaxExpertsSq + 1];   // first pool tile of each expert (and the end)
  __shared__ int32_t s_end[kMaxExpertsSq];      // end of each expert's rows in the pool
  __shared__ int s_sel;
  __shared__ int4 s_units[kUnitSlots];        // this workgroup's first units, decoded
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
  const int rg = w >> 1;   // row half of the unit
  const int cg = w & 1;    // column half of the unit

  int ntiles = a.num_tiles[0];
  if (ntiles > a.max_tiles) {
    if (blockIdx.x == 0 && tid == 0) record_error(a.err, MOE_ERR_INVALID);
    ntiles = a.max_tiles;
  }
  for (int e = tid; e <= a.n_experts; e += 64 * kSqWaves) {
    const int o = a.offsets[e];
    s_t0[e] = min(o >> 7, a.max_tiles);
    if (e < a.n_experts) s_end[e] = o + a.counts[e];
  }
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
  // the workgroup's units u, u + G, ... decoded once, one per lane of wave 0 (each a search
  // over the experts' row-unit prefix), so that moving to the next unit reads one table
  // entry instead of searching between two units while the matrix core idles
  if (w == 0) {
    const int uu = u + lane * G;
    if (lane < kUnitSlots && uu < total) {
      const SqUnit U = sq_unit_lane(a, s_ru, s_t0, uu);
      s_units[lane] = int4{U.e, U.m, U.two, U.j};
    }
  }
  __syncthreads();
  int it = 0;   // index of the current unit among the workgroup's

  bool poll_each = false;
  if (a.wait_ready) {
    const uint32_t done = __hip_atomic_load(a.tiles_done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    poll_each = done < (uint32_t)ntiles;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }

  const int KS = a.KS;
  const int KH = KS >> 1;   // pool-row stages per unit
  // this wave's DMA lanes: pool rows 64w .. 64w + 63 of the unit, 8 rows per DMA; lane i
  // fills LDS bytes 16i .. 16i + 15 of a DMA's 1 KiB, i.e. row i / 8, chunk slot i % 8,
  // which holds the row's chunk (i % 8) ^ (row % 8)
  const uint32_t lda = (uint32_t)a.lda;
  const uint32_t a_vo = (uint32_t)(64 * w + (lane >> 3)) * lda + 16u * (uint32_t)((lane & 7) ^ ((lane >> 3) & 7));
  const uint32_t b_vo = 16u * (uint32_t)lane;
  const uint32_t bstr = (uint32_t)a.ktiles * 1024u;
  // fragment read of pool rows: lane l takes row l % 16, chunk 4 h + l / 16 of the stage
  // (h: the stage's K half)
  const int a_frag0 = (lane & 15) * 128 + ((((lane >> 4)) ^ (lane & 7)) << 4) + rg * 128 * 128;
  const int a_frag1 = (lane & 15) * 128 + (((4 + (lane >> 4)) ^ (lane & 7)) << 4) + rg * 128 * 128;
  typedef __attribute__((address_space(3))) void* lds_t;
  // B row blocks of this wave's MFMA column tiles: GEMM A gate 4cg .. +3, up 8 + 4cg .. +3
  auto bblk = [&](int tn) __attribute__((always_inline)) { return GEMM_A ? (tn < 4 ? 4 * cg + tn : 8 + 4 * cg + (tn - 4)) : 8 * cg + tn; };

  SqUnit cur = sq_unit(a, s_ru, s_t0, u);
  if (poll_each) sq_wait_tiles(a, cur);
  SqSrc cs = sq_src<GEMM_A>(a, cur, s_end, w);
  // the first unit's stages in the order the steady state issues them: weights 0 (step
  // -4), pool rows 0 and weights 1 (step -3), weights 2 (step -2), pool rows 1 and weights 3
  // (step -1)
  {
    const __amdgpu_buffer_rsrc_t car = make_rsrc(cs.abase, cs.abytes), cbr = make_rsrc(cs.bbase, (uint32_t)a.b_expert);
    // one pool-row stage (8 DMAs) and one weight stage (4 DMAs) of this wave
    auto pa = [&](uint8_t* dst, uint32_t koff) __attribute__((always_inline)) {
#pragma unroll
      for (int q = 0; q < 8; ++q)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(car, (lds_t)(dst + (8 * w + q) * 1024), 16, a_vo + 8u * q * lda,
                                                 koff, 0, 0);
    };
    auto pb = [&](uint8_t* dst, uint32_t boff) __attribute__((always_inline)) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(cbr, (lds_t)(dst + (4 * w + q) * 1024), 16, b_vo,
                                                 boff + (uint32_t)q * bstr, 0, 0);
    };
    pb(s_b0, cs.b0);
    pa(s_a0, 0u);
    pb(s_b1, cs.b0 + 1024u);
    pb(s_b2, cs.b0 + 2048u);
    pa(s_a1, 128u);
    pb(s_b3, cs.b0 + 3072u);
  }

  f32x4_t acc[8][8];
  bf16x8_t fa[2][8], fb[2][8];

  for (;;) {
    // this unit's stage 0 fragments. Its DMAs were issued at steps -4 and -3 of the unit (in
    // the previous unit's last steps, or above for the first unit), with 20 DMAs behind them
    // (and the previous unit's output stores, which the count does not rely on). (The last
    // step of the previous unit read them too; reading them again here keeps no fragment
    // register live across the epilogue.)
    __builtin_amdgcn_s_waitcnt(vmcnt_enc(20));
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      fa[0][t] = *reinterpret_cast<const bf16x8_t*>(s_a0 + a_frag0 + t * 16 * 128);
      fb[0][t] = *reinterpret_cast<const bf16x8_t*>(s_b0 + bblk(t) * 1024 + 16 * lane);
    }
    const int un = u + G;
    const bool has_next = un < total;
    SqUnit nx = cur;
    if (has_next) {
      if (it + 1 < kUnitSlots) {
        const int4 t = s_units[it + 1];
        nx.e = __builtin_amdgcn_readfirstlane(t.x);
        nx.m = __builtin_amdgcn_readfirstlane(t.y);
        nx.two = __builtin_amdgcn_readfirstlane(t.z);
        nx.j = __builtin_amdgcn_readfirstlane(t.w);
      } else {
        nx = sq_unit(a, s_ru, s_t0, un);
      }
    }
    const SqSrc ns = sq_src<GEMM_A>(a, nx, s_end, w);
    const bool store = rg == 0 || cur.two;   // a one-tile unit's second row half is not stored

    // step ks (32 K values), ks % 4 = ST: MFMAs on the fragments of register set ST % 2;
    // reads of step ks + 1 into the other set
    auto step = [&](auto ST, auto Z, int ks) __attribute__((always_inline)) {
      constexpr int st = decltype(ST)::value;
      constexpr bool FIRST = decltype(Z)::value;   // the unit's first K step: c = a x b
      auto mfma = [&](f32x4_t& c, bf16x8_t x, bf16x8_t y) __attribute__((always_inline)) {
        if constexpr (FIRST) mfma_first(c, x, y);
        else mfma_acc(c, x, y);
      };
      constexpr int P = st & 1, PN = P ^ 1;
      constexpr bool ODD = P == 1;
      using AR = std::integral_constant<int, ((st + 1) >> 1) & 1>;   // pool-row stage read (for step ks + 1)
      using BR = std::integral_constant<int, (st + 1) & 3>;          // weight stage read
      using AD = std::integral_constant<int, st == 1 ? 0 : 1>;       // pool-row stage loaded (odd steps)
      constexpr bool H1 = ((st + 1) & 1) != 0;                       // K half of the pool-row stage read
      __builtin_amdgcn_sched_barrier(0);
      // the sources of this step's DMAs (scalar work, issued while the previous step's last
      // MFMAs run): weight stage ks + 4 and, on odd steps, pool-row stage (ks + 3) / 2, this
      // unit's, the next unit's first ones, or a reload nobody reads when there is no next unit
      const int kb = ks + 4;
      const bool b_nx = kb >= KS;
      const bool bn = b_nx && has_next;
      const __amdgpu_buffer_rsrc_t d_br = make_rsrc(pick(bn, ns.bbase, cs.bbase), (uint32_t)a.b_expert);
      const uint32_t d_b = pick(bn, ns.b0, cs.b0) + (uint32_t)(b_nx ? (has_next ? kb - KS : KS - 1) : kb) * 1024u;
      __amdgpu_buffer_rsrc_t d_ar;
      uint32_t d_a = 0;
      if constexpr (ODD) {
        const int kd = (ks + 3) >> 1;
        const bool a_nx = kd >= KH;
        if constexpr (st == 1) {
          if (kd == KH && has_next && poll_each) sq_wait_tiles(a, nx);
        }
        const bool an = a_nx && has_next;
        d_ar = make_rsrc(pick(an, ns.abase, cs.abase), pick(an, ns.abytes, cs.abytes));
        d_a = (uint32_t)(a_nx ? (has_next ? kd - KH : KH - 1) : kd) * 128u;
      }
      __builtin_amdgcn_sched_barrier(0);
      // the step's first kPre MFMAs need nothing the barrier guards: they keep the matrix core
      // busy while the wave waits at it
#pragma unroll
      for (int i = 0; i < kPre; ++i) mfma(acc[i >> 3][i & 7], fb[P][i & 7], fa[P][i >> 3]);
      __builtin_amdgcn_sched_barrier(0);
      // this wave's DMAs of the stages read during this step are in (even steps: weights
      // ks + 1 and pool rows ks / 2, issued at step ks - 3, with 16 DMAs behind them; odd
      // steps: pool rows (ks + 1) / 2, issued first at step ks - 2, with 8 behind them); its
      // fragment reads of the previous step are done. (In a unit's first steps the previous
      // unit's output stores lie behind them too and count against the same budget: the
      // counter can retire stores before older loads, so only loads may be counted on.)
      __builtin_amdgcn_s_waitcnt(vmcnt_enc(ODD ? 8 : 16));
      __builtin_amdgcn_s_waitcnt(kLgkm0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      const uint8_t* ra = aring(AR{}) + (H1 ? a_frag1 : a_frag0);
      const uint8_t* rb = bring(BR{}) + 16 * lane;
      // the step's memory operations, spread over the MFMAs from the barrier on (a wave waits
      // while a memory instruction issues, and the MFMA just issued keeps the matrix core busy
      // meanwhile): the 16 fragment reads of step ks + 1 into the other register set, and the
      // DMAs, weight stage ks + 4 into the stage of ks (read during step ks - 1) and, on odd
      // steps, pool-row stage (ks + 3) / 2 before it (the wait counts above rely on that order)
      auto read_a = [&](int t) __attribute__((always_inline)) {
        fa[PN][t] = *reinterpret_cast<const bf16x8_t*>(ra + t * 16 * 128);
      };
      auto read_b = [&](int t) __attribute__((always_inline)) {
        fb[PN][t] = *reinterpret_cast<const bf16x8_t*>(rb + bblk(t) * 1024);
      };
      auto dma_a = [&](int q) __attribute__((always_inline)) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(d_ar, (lds_t)(aring(AD{}) + (8 * w + q) * 1024), 16,
                                                 a_vo + 8u * (uint32_t)q * lda, d_a, 0, 0);
      };
      auto dma_b = [&](int q) __attribute__((always_inline)) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(d_br, (lds_t)(bring(ST) + (4 * w + q) * 1024), 16, b_vo,
                                                 d_b + (uint32_t)q * bstr, 0, 0);
      };
      // MFMA i of the step (group i / 8, column tile i % 8), then its memory operation
      auto one = [&](auto II) __attribute__((always_inline)) {
        constexpr int i = decltype(II)::value;
        constexpr int g = i >> 3, tn = i & 7;
        mfma(acc[g][tn], fb[P][tn], fa[P][g]);
        constexpr int c = sq_op(ODD, i);
        if constexpr (c >> 4 == 1) read_a(c & 15);
        else if constexpr (c >> 4 == 2) read_b(c & 15);
        else if constexpr (c >> 4 == 3) dma_a(c & 15);
        else if constexpr (c >> 4 == 4) dma_b(c & 15);
        __builtin_amdgcn_sched_barrier(0);
      };
      [&]<int... Is>(std::integer_sequence<int, Is...>) __attribute__((always_inline)) {
        (one(std::integral_constant<int, Is + kPre>{}), ...);
      }(std::make_integer_sequence<int, 64 - kPre>{});
    };

    // K steps in rounds of four (KS is a multiple of four, at least four); the first step's
    // MFMAs start the accumulators from the constant 0
    using F = std::false_type;
    step(I0{}, std::true_type{}, 0);
    step(I1{}, F{}, 1);
    step(I2{}, F{}, 2);
    step(I3{}, F{}, 3);
    for (int ks = 4; ks < KS; ks += 4) {
      step(I0{}, F{}, ks);
      step(I1{}, F{}, ks + 1);
      step(I2{}, F{}, ks + 2);
      step(I3{}, F{}, ks + 3);
    }

    {
      // ---- epilogue: lane holds row tm*16 + (lane & 15), columns 4 (lane >> 4) + (0..3) of
      // each tile; the wave's 4 KiB of s_out stage 16 rows at a time. A wave whose rows are
      // not stored (the second half of a one-tile unit) stores into an empty range, which
      // drops them.
      // the lane index as a value computed here, so that the compiler derives the epilogue's
      // addresses from it inside the unit loop rather than keeping them live across the K loop
      int el;
      asm volatile("" : "=v"(el) : "0"(lane));
      // the last MFMAs' results are in before the first read of an accumulator
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
      __builtin_amdgcn_sched_barrier(0);
      uint8_t* so = s_out + w * 4096;
      const int64_t row0 = (int64_t)cur.m * 128 + rg * 128;
      const int r = el & 15;
      const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.out + row0 * a.ldo, store ? (uint32_t)(128 * a.ldo) : 0u);
      const uint32_t ldo = (uint32_t)a.ldo;
      // 256-byte staging rows, 16-byte chunks permuted by row
      auto st256 = [&](int row, int b) __attribute__((always_inline)) {
        return row * 256 + ((((b >> 4) ^ row) & 15) << 4) + (b & 15);
      };
      if constexpr (GSAVE) {
#pragma unroll
        for (int tm = 0; tm < 8; ++tm) {
          // one MFMA row at a time: its accumulators are read only here
          __builtin_amdgcn_sched_barrier(0);
          f32x4_t cv[8];
#pragma unroll
          for (int tn = 0; tn < 8; ++tn) cv[tn] = acc_read(acc[tm][tn]);
          if constexpr (GEMM_A) {
            if constexpr (GSAVE) {
              // G = [gate | up] before the activation: 64 gate and 64 up columns as one
              // 256-byte staging row, stored as 128-byte segments of the gate and up halves
#pragma unroll
              for (int tn = 0; tn < 8; ++tn) {
                u32x2 v;
                v.x = pack_bf16x2(cv[tn][0], cv[tn][1]);
                v.y = pack_bf16x2(cv[tn][2], cv[tn][3]);
                *reinterpret_cast<u32x2*>(so + st256(r, tn * 32 + 8 * (el >> 4))) = v;
              }
              const __amdgpu_buffer_rsrc_t rg_ = make_rsrc(a.g_save + row0 * a.g_ld, store ? (uint32_t)(128 * a.g_ld) : 0u);
#pragma unroll
              for (int p = 0; p < 4; ++p) {
                const int rr = p * 4 + (el >> 4), c = el & 15;
                const u32x4 v = *reinterpret_cast<const u32x4*>(so + st256(rr, c * 16));
                const uint32_t col = (uint32_t)((c < 8 ? 0 : a.g_up) + (cur.j * 128 + cg * 64) * 2 + (c & 7) * 16);
                buf_store16(v, rg_, (uint32_t)(tm * 16 + rr) * (uint32_t)a.g_ld + col);
              }
            }
            // h = silu(gate) * up: 16 rows x 64 columns, staged as 128-byte rows
#pragma unroll
            for (int tn = 0; tn < 4; ++tn) {
              u32x2 v;
              v.x = pack_bf16x2(sq_silu_mul(cv[tn][0], cv[tn + 4][0]), sq_silu_mul(cv[tn][1], cv[tn + 4][1]));
              v.y = pack_bf16x2(sq_silu_mul(cv[tn][2], cv[tn + 4][2]), sq_silu_mul(cv[tn][3], cv[tn + 4][3]));
              const int b = tn * 32 + 8 * (el >> 4);
              *reinterpret_cast<u32x2*>(so + 2048 + r * 128 + ((((b >> 4) ^ (r & 7))) << 4) + (b & 15)) = v;
            }
#pragma unroll
            for (int p = 0; p < 2; ++p) {
              const int rr = p * 8 + (el >> 3), c = el & 7;
              const u32x4 v = *reinterpret_cast<const u32x4*>(so + 2048 + rr * 128 + ((c ^ (rr & 7)) << 4));
              buf_store16(v, ro, (uint32_t)(tm * 16 + rr) * ldo + (uint32_t)((cur.j * 128 + cg * 64) * 2 + c * 16));
            }
          } else {
#pragma unroll
            for (int tn = 0; tn < 8; ++tn) {
              u32x2 v;
              v.x = pack_bf16x2(cv[tn][0], cv[tn][1]);
              v.y = pack_bf16x2(cv[tn][2], cv[tn][3]);
              *reinterpret_cast<u32x2*>(so + st256(r, tn * 32 + 8 * (el >> 4))) = v;
            }
#pragma unroll
            for (int p = 0; p < 4; ++p) {
              const int rr = p * 4 + (el >> 4), c = el & 15;
              const u32x4 v = *reinterpret_cast<const u32x4*>(so + st256(rr, c * 16));
              buf_store16(v, ro, (uint32_t)(tm * 16 + rr) * ldo + (uint32_t)((cur.j * 256 + cg * 128) * 2 + c * 16));
            }
          }
        }
      } else {
        // Software-pipelined over the eight MFMA rows: row tm's accumulators are read and
        // converted while the staging reads of row tm - 1 are in flight; then row tm - 1 is
        // stored and row tm staged. (A wave's LDS accesses execute in order, so row tm's
        // staging writes cannot overtake row tm - 1's reads of the same bytes.)
        // GEMM A: h = silu(gate) * up, 16 rows x 64 columns as 128-byte staging rows (4 x 8
        // bytes a lane, read back as 2 x 16); GEMM Y: 16 rows x 128 columns as 256-byte rows
        // (8 x 8 bytes a lane, read back as 4 x 16).
        constexpr int NP = GEMM_A ? 4 : 8;
        constexpr int NR = GEMM_A ? 2 : 4;
        auto prep = [&](int tm, u32x2(&pk)[NP]) __attribute__((always_inline)) {
          f32x4_t cv[8];
#pragma unroll
          for (int tn = 0; tn < 8; ++tn) cv[tn] = acc_read(acc[tm][tn]);
#pragma unroll
          for (int tn = 0; tn < NP; ++tn) {
            if constexpr (GEMM_A) {
              pk[tn].x = pack_bf16x2(sq_silu_mul(cv[tn][0], cv[tn + 4][0]), sq_silu_mul(cv[tn][1], cv[tn + 4][1]));
              pk[tn].y = pack_bf16x2(sq_silu_mul(cv[tn][2], cv[tn + 4][2]), sq_silu_mul(cv[tn][3], cv[tn + 4][3]));
            } else {
              pk[tn].x = pack_bf16x2(cv[tn][0], cv[tn][1]);
              pk[tn].y = pack_bf16x2(cv[tn][2], cv[tn][3]);
            }
          }
        };
        auto stage = [&](const u32x2(&pk)[NP]) __attribute__((always_inline)) {
#pragma unroll
          for (int tn = 0; tn < NP; ++tn) {
            const int b = tn * 32 + 8 * (el >> 4);
            if constexpr (GEMM_A)
              *reinterpret_cast<u32x2*>(so + 2048 + r * 128 + ((((b >> 4) ^ (r & 7))) << 4) + (b & 15)) = pk[tn];
            else
              *reinterpret_cast<u32x2*>(so + st256(r, b)) = pk[tn];
          }
        };
        auto fetch = [&](u32x4(&v)[NR]) __attribute__((always_inline)) {
#pragma unroll
          for (int p = 0; p < NR; ++p) {
            if constexpr (GEMM_A) {
              const int rr = p * 8 + (el >> 3), c = el & 7;
              v[p] = *reinterpret_cast<const u32x4*>(so + 2048 + rr * 128 + ((c ^ (rr & 7)) << 4));
            } else {
              const int rr = p * 4 + (el >> 4), c = el & 15;
              v[p] = *reinterpret_cast<const u32x4*>(so + st256(rr, c * 16));
            }
          }
        };
        auto put = [&](int tm, const u32x4(&v)[NR]) __attribute__((always_inline)) {
#pragma unroll
          for (int p = 0; p < NR; ++p) {
            if constexpr (GEMM_A) {
              const int rr = p * 8 + (el >> 3), c = el & 7;
              buf_store16(v[p], ro, (uint32_t)(tm * 16 + rr) * ldo + (uint32_t)((cur.j * 128 + cg * 64) * 2 + c * 16));
            } else {
              const int rr = p * 4 + (el >> 4), c = el & 15;
              buf_store16(v[p], ro, (uint32_t)(tm * 16 + rr) * ldo + (uint32_t)((cur.j * 256 + cg * 128) * 2 + c * 16));
            }
          }
        };
        u32x2 pk[NP];
        u32x4 v[NR];
        prep(0, pk);
        stage(pk);
        fetch(v);
#pragma unroll
        for (int tm = 1; tm < 8; ++tm) {
          __builtin_amdgcn_sched_barrier(0);
          prep(tm, pk);
          put(tm - 1, v);
          stage(pk);
          fetch(v);
        }
        put(7, v);
      }
    }
    if (!has_next) break;
    u = un;
    ++it;
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
