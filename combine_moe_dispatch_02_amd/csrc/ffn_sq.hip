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
// row half is neither computed nor stored. GEMM A's N block is 128 gate columns and
// the matching 128 up columns of w1, so SwiGLU stays in the lane that holds both.
// 8 waves: wave w computes rows 128 (w / 4) .. +128 and 64 of the 256 columns
// (w % 4), i.e. 8 x 4 MFMA tiles, 128 accumulators per lane.
//
// Operands. A K stage is 64 values (128 bytes, one cache line) of every row: 256 pool
// (or h) rows and 256 weight rows, 64 KiB of LDS. The pool rows are stored row by row,
// their eight 16-byte chunks XOR-permuted by row % 8: the eight lanes of a DMA that
// fill one row fetch its whole line, and the eight lanes of a fragment read that share
// a chunk index (eight rows) land on eight distinct 16-byte slots of a 128-byte bank
// row. The tiled weight layout already holds MFMA fragments as contiguous 1 KiB blocks
// (lane l's 16 bytes = row l % 16, K values 8 (l / 16) .. +8 of a 32-wide K tile), two
// per 16 rows and stage, which the DMA copies as they are. Each wave moves 8 of the
// stage's 64 KiB by LDS-DMA (buffer_load ... lds), so no register holds a load in
// flight, and every request covers whole cache lines.
//
// Pipeline. Two 64 KiB stages. Step ks: wait for this wave's DMAs of stage ks (vmcnt),
// barrier (every wave's are in; stage ks-1's slot is free), DMA stage ks+1 into that
// slot, then the MFMAs of stage ks. The stages run on across units: a unit's last step
// loads the next unit's first stage, so a unit's epilogue overlaps that load. The last
// MFMA group of each stage is issued after the next barrier, while the next stage's
// first fragment reads are in flight. The two stages are separate LDS objects used
// with constant indices (the K loop runs two steps per round), so the compiler can
// tell a step's reads from the DMA writes in flight to the other stage and adds no
// wait of its own.
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
#include "kernels.h"

namespace moe {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kSqWaves = 8;
constexpr int kStageBytes = 65536;   // 256 A rows x 128 bytes, then 16 B row blocks x 2 K tiles x 1 KiB
constexpr int kBHalf = 32768;        // B blocks start here
constexpr int kMaxExpertsSq = 1024;

__device__ inline float sq_silu_mul(float g, float u) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u; }

struct SqUnit {
  int e;     // local expert
  int m;     // first pool tile
  int two;   // 1: tiles m and m + 1; 0: tile m only
  int j;     // N block of 256 columns
};

// Unit u -> coordinates. s_ru[e] = row units (tile pairs, rounded up) of the experts
// before e. Within expert e, units go in groups of `group` row units; inside a group,
// N block by N block, the group's row units back to back: units that run together
// share weight panels and pool rows.
__device__ inline SqUnit sq_unit(const SqArgs& a, const int32_t* s_ru, int u) {
  int lo = 0, hi = a.n_experts - 1;
  while (lo < hi) {  // the last expert whose first unit is <= u (empty experts share a start)
    const int mid = (lo + hi + 1) >> 1;
    if (s_ru[mid] * a.NB <= u) lo = mid;
    else hi = mid - 1;
  }
  SqUnit r;
  r.e = lo;
  const int R = s_ru[lo + 1] - s_ru[lo];
  const int l = u - s_ru[lo] * a.NB;
  const int g = l / (a.group * a.NB);
  const int gsz = min(a.group, R - g * a.group);
  const int l2 = l - g * a.group * a.NB;
  r.j = l2 / gsz;
  const int ru = g * a.group + (l2 - r.j * gsz);
  const int t0 = min(a.offsets[lo] >> 7, a.max_tiles);
  const int t1 = min(a.offsets[lo + 1] >> 7, a.max_tiles);
  r.m = t0 + 2 * ru;
  r.two = r.m + 1 < t1;
  return r;
}

// DMA sources of one unit for this wave: the unit's rows (A) and its expert's tiled
// weights (B), and the byte offsets of the wave's two B row blocks
struct SqSrc {
  __amdgpu_buffer_rsrc_t ar, br;
  uint32_t b0, b1;
};

template <bool GEMM_A>
__device__ inline SqSrc sq_src(const SqArgs& a, const SqUnit& U, int w) {
  SqSrc s;
  s.ar = make_rsrc(a.A + (int64_t)U.m * 128 * a.lda, (uint32_t)((U.two ? 256 : 128) * a.lda));
  s.br = make_rsrc(a.B + (int64_t)U.e * a.b_expert, (uint32_t)a.b_expert);
  // B blocks 2w, 2w + 1 of the unit's 16: GEMM A gate blocks 0..7, up blocks 8..15
  const int rb = GEMM_A ? (w < 4 ? U.j * 8 + 2 * w : a.up_rb + U.j * 8 + 2 * (w - 4)) : U.j * 16 + 2 * w;
  s.b0 = (uint32_t)rb * (uint32_t)a.ktiles * 1024u;
  s.b1 = s.b0 + (uint32_t)a.ktiles * 1024u;
  return s;
}

// Wait until the unit's tiles carry this call's epoch (see the file comment).
__device__ inline void sq_wait_tiles(const SqArgs& a, const SqUnit& U) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (;;) {
    const bool r0 = __hip_atomic_load(&a.tile_ready[U.m], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == a.epoch;
    const bool r1 = !U.two ||
                    __hip_atomic_load(&a.tile_ready[U.m + 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == a.epoch;
    if (r0 && r1) break;
    if (__hip_atomic_load(a.abort_epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == a.epoch) break;
    if (__builtin_amdgcn_s_memrealtime() - t0 > a.timeout) {
      record_error(a.err, MOE_ERR_TIMEOUT);
      __hip_atomic_store(a.abort_epoch, a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    __builtin_amdgcn_s_sleep(4);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

}  // namespace

template <bool GEMM_A, bool GSAVE>
__global__ __launch_bounds__(64 * kSqWaves, 1) void ffn_sq_kernel(SqArgs a) {
  static_assert(!GSAVE || GEMM_A, "G is kept by GEMM A");
  __shared__ __attribute__((aligned(16))) uint8_t s_r0[kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_r1[kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_out[kSqWaves * 2048];
  __shared__ int32_t s_ru[kMaxExpertsSq + 1];
  auto ring = [&](auto ST) -> uint8_t* {
    if constexpr (decltype(ST)::value == 0) return s_r0;
    else return s_r1;
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;

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
  // row units per expert, prefix-summed: lane i of wave 0 sums a run of experts
  if (w == 0) {
    const int E = a.n_experts;
    const int per = (E + 63) >> 6;
    int sum = 0;
    for (int i = 0; i < per; ++i) {
      const int e = lane * per + i;
      if (e < E) {
        const int t0 = min(a.offsets[e] >> 7, a.max_tiles), t1 = min(a.offsets[e + 1] >> 7, a.max_tiles);
        sum += (t1 - t0 + 1) >> 1;
      }
    }
    const int incl = wave_inclusive_scan(sum);
    int run = incl - sum;
    for (int i = 0; i < per; ++i) {
      const int e = lane * per + i;
      if (e < E) {
        s_ru[e] = run;
        const int t0 = min(a.offsets[e] >> 7, a.max_tiles), t1 = min(a.offsets[e + 1] >> 7, a.max_tiles);
        run += (t1 - t0 + 1) >> 1;
      }
    }
    if (lane == 63) s_ru[E] = incl;
  }
  __syncthreads();
  const int total = s_ru[a.n_experts] * a.NB;
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
  auto dma = [&](auto ST, const SqSrc& s, int ks) {
    uint8_t* base = ring(ST);
    const uint32_t ka = (uint32_t)ks * 128u, kb = (uint32_t)ks * 2048u;
    typedef __attribute__((address_space(3))) void* lds_t;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(s.ar, (lds_t)(base + (4 * w + q) * 1024), 16, a_vo + 8u * q * lda, ka,
                                               0, 0);
    // B row blocks 2w, 2w + 1, K tiles 2ks, 2ks + 1 each
#pragma unroll
    for (int q = 0; q < 4; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(s.br, (lds_t)(base + kBHalf + (4 * w + q) * 1024), 16, b_vo,
                                               (q < 2 ? s.b0 : s.b1) + kb + (q & 1) * 1024u, 0, 0);
  };
  // B row blocks of this wave's MFMA column tiles: GEMM A gate 2cg, 2cg + 1, up 8 + 2cg, 8 + 2cg + 1
  auto bblk = [&](int tn) { return GEMM_A ? (tn < 2 ? 2 * cg + tn : 8 + 2 * cg + (tn - 2)) : 4 * cg + tn; };

  SqUnit cur = sq_unit(a, s_ru, u);
  if (poll_each) sq_wait_tiles(a, cur);
  SqSrc cs = sq_src<GEMM_A>(a, cur, w);
  dma(I0{}, cs, 0);

  f32x4_t acc[8][4];
  bf16x8_t fbp[4], fap;   // the previous stage's last MFMA group, issued after the next barrier

  for (;;) {
    const int un = u + G;
    const bool has_next = un < total;
    const SqUnit nx = has_next ? sq_unit(a, s_ru, un) : cur;
    const SqSrc ns = sq_src<GEMM_A>(a, nx, w);
    const bool compute = rg == 0 || cur.two;
#pragma unroll
    for (int tm = 0; tm < 8; ++tm)
#pragma unroll
      for (int tn = 0; tn < 4; ++tn) acc[tm][tn] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int tn = 0; tn < 4; ++tn) fbp[tn] = bf16x8_t{};
    fap = bf16x8_t{};   // zero operands: the first step's deferred group adds exactly 0

    auto step = [&](auto ST, int ks) {
      using SN = std::integral_constant<int, decltype(ST)::value ^ 1>;
      __builtin_amdgcn_sched_barrier(0);
      // this wave's DMAs of stage ks are in, and its reads of stage ks - 1 are done
      wait_vm0();
      __builtin_amdgcn_s_waitcnt(kLgkm0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      // stage ks + 1 into the slot of stage ks - 1: this unit's, the next unit's first, or
      // (last unit) a reload of this unit's last stage that nobody reads, so that every step
      // issues the same DMAs
      {
        SqSrc s = cs;
        int kk = ks + 1;
        if (kk >= KS) {
          if (has_next) {
            s = ns;
            kk = 0;
            if (poll_each) sq_wait_tiles(a, nx);
          } else {
            kk = KS - 1;
          }
        }
        dma(SN{}, s, kk);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (compute) {
        const uint8_t* sa = ring(ST) + (rg * 128) * 128;
        const uint8_t* sb = ring(ST) + kBHalf + 16 * lane;
        bf16x8_t fb[4];
#pragma unroll
        for (int tn = 0; tn < 4; ++tn) fb[tn] = *reinterpret_cast<const bf16x8_t*>(sb + (bblk(tn) * 2) * 1024);
        bf16x8_t fa = *reinterpret_cast<const bf16x8_t*>(sa + a_frag0);
        // the previous stage's last group
#pragma unroll
        for (int tn = 0; tn < 4; ++tn)
          acc[7][tn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fbp[tn], fap, acc[7][tn], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        // 16 groups: K half kk, row tile tm; A fragments read one group ahead, the second K
        // half's B fragments during the first half
        bf16x8_t fb1[4];
#pragma unroll
        for (int g = 0; g < 15; ++g) {
          const int kk = g >> 3, tm = g & 7;
          const int g1 = g + 1;
          const bf16x8_t fn =
              *reinterpret_cast<const bf16x8_t*>(sa + ((g1 & 7) * 16) * 128 + ((g1 >> 3) ? a_frag1 : a_frag0));
          if (g == 3) {
#pragma unroll
            for (int tn = 0; tn < 4; ++tn)
              fb1[tn] = *reinterpret_cast<const bf16x8_t*>(sb + (bblk(tn) * 2 + 1) * 1024);
          }
#pragma unroll
          for (int tn = 0; tn < 4; ++tn)
            acc[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kk ? fb1[tn] : fb[tn], fa, acc[tm][tn], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
          fa = fn;
        }
        fap = fa;
#pragma unroll
        for (int tn = 0; tn < 4; ++tn) fbp[tn] = fb1[tn];
      }
    };

    for (int ks = 0; ks < KS; ks += 2) {
      step(I0{}, ks);
      step(I1{}, ks + 1);
    }

    if (compute) {
#pragma unroll
      for (int tn = 0; tn < 4; ++tn)
        acc[7][tn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fbp[tn], fap, acc[7][tn], 0, 0, 0);
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
