// The backward pass around the expert GEMMs (StreamEP README, "How it works": the
// layer trains, the backward pass mirrors the forward's overlaps, and the backward
// grouped GEMMs A and Y are two of its four grouped GEMMs).
//
//   combine backward: dy_pool[pos[t,k]] = w[t,k] * dout[t] (bf16) and the gradient of
//                     the routing weights dw[t,k] = <dout[t], y_pool[pos[t,k]]> (fp32);
//                     the mirror of combine is a scatter into the pool, like dispatch.
//   weight gradients: C[e] = A_e^T B_e over the rows of expert e's pool segment
//                     (dW2[e] = dy_e^T h_e, dW1[e] = dG_e^T X_e), a grouped GEMM whose
//                     contraction runs over pool rows.
//   dispatch backward is the combine kernel with unit weights (combine.hip), and the
//   data gradients run on the forward's big-tile kernel (ffn.hip).
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {

// --------------------------------------------------------------------------------
// combine backward: one wave per token, 16-byte lanes. dout[t] is read once; for each
// local pair the y row is read for the dot product and the scaled dout row is stored.
// A block's four waves take a run of consecutive tokens, then publish them the way
// dispatch publishes its rows (the mirror of the forward's per-tile streaming): a
// barrier, one device-scope release by wave 0, then a relaxed count per stored pair on
// its tile's counter; the lane whose count completes the tile's real rows resets the
// counter (every store of this call to that tile is counted by then), acquires, and
// stores the epoch into tile_ready with release ordering.
// --------------------------------------------------------------------------------
struct CombineBwdArgs {
  const uint8_t* dout;
  const float* w;
  const uint8_t* y;
  const int32_t* pos;
  int32_t T, K, H;
  int32_t pool_rows;
  uint8_t* dy;
  float* dw;
  int32_t tile, tile_shift;
  int32_t tokens_per_block;   // a multiple of 4
  const int32_t* tile_expert;
  const int32_t* offsets;
  const int32_t* counts;
  uint32_t* tile_fill;
  uint32_t* tile_ready;
  uint32_t epoch;
};

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

template <int CPL>
__device__ inline void combine_bwd_token(const CombineBwdArgs& a, int t, int lane) {
  constexpr int KMAX = 16;
  const int64_t pair0 = (int64_t)t * a.K;
  int p = lane < a.K ? a.pos[pair0 + lane] : -1;
  if (p >= a.pool_rows) p = -1;
  const float wt = lane < a.K ? a.w[pair0 + lane] : 0.f;
  const uint64_t have = ballot(p >= 0);
  const uint32_t row_bytes = (uint32_t)a.H * 2u;
  const int nch = a.H >> 3;
  const __amdgpu_buffer_rsrc_t dr = make_rsrc(a.dout + (int64_t)t * row_bytes, row_bytes);
  float part[KMAX];
#pragma unroll
  for (int k = 0; k < KMAX; ++k) part[k] = 0.f;
  for (int c0 = 0; c0 < nch; c0 += kWave * CPL) {
    u32x4 d[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) d[i] = buf_load16(dr, (uint32_t)(c0 + i * kWave + lane) * 16u);
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
      if (k >= a.K || !((have >> k) & 1ull)) continue;
      const int pk = readlane(p, k);
      const float wk = __builtin_bit_cast(float, readlane(__builtin_bit_cast(int, wt), k));
      const __amdgpu_buffer_rsrc_t yr = make_rsrc(a.y + (int64_t)pk * row_bytes, row_bytes);
      const __amdgpu_buffer_rsrc_t or_ = make_rsrc(a.dy + (int64_t)pk * row_bytes, row_bytes);
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const uint32_t off = (uint32_t)(c0 + i * kWave + lane) * 16u;
        const u32x4 yv = buf_load16(yr, off);
        const uint32_t dd[4] = {d[i].x, d[i].y, d[i].z, d[i].w};
        const uint32_t yy[4] = {yv.x, yv.y, yv.z, yv.w};
        uint32_t o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float d0 = bf16_lo(dd[q]), d1 = bf16_hi(dd[q]);
          part[k] += d0 * bf16_lo(yy[q]);
          part[k] += d1 * bf16_hi(yy[q]);
          o[q] = pack_bf16x2(wk * d0, wk * d1);
        }
        buf_store16(u32x4{o[0], o[1], o[2], o[3]}, or_, off);
      }
    }
  }
  // every lane of the wave takes part in the reductions; lane k keeps pair k's sum
  float mine = 0.f;
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    if (k < a.K) {
      const float s = wave_sum(part[k]);
      if (lane == k) mine = ((have >> k) & 1ull) ? s : 0.f;
    }
  }
  if (lane < a.K) a.dw[pair0 + lane] = mine;
}

template <int CPL>
__global__ __launch_bounds__(256) void combine_backward_kernel(CombineBwdArgs a) {
  const int lane = lane_id();
  const int w = threadIdx.x >> 6;
  const int tb = blockIdx.x * a.tokens_per_block;        // the block's first token
  const int te = min(a.T, tb + a.tokens_per_block);
  for (int t = tb + w; t < te; t += 4) combine_bwd_token<CPL>(a, t, lane);

  __syncthreads();
  if (w != 0) return;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  const int npairs = (te - tb) * a.K;
  for (int q = lane; q < npairs; q += 64) {
    const int p = a.pos[(int64_t)tb * a.K + q];
    if (p < 0 || p >= a.pool_rows) continue;
    const int ti = p >> a.tile_shift;
    const uint32_t old = __hip_atomic_fetch_add(&a.tile_fill[ti], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int e = a.tile_expert[ti];
    const int real = min(a.tile, a.offsets[e] + a.counts[e] - (ti << a.tile_shift));
    if ((int)old + 1 == real) {
      __hip_atomic_store(&a.tile_fill[ti], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      __hip_atomic_store(&a.tile_ready[ti], a.epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

int launch_combine_backward(const void* dout, const float* topk_weights, const void* y_pool, int32_t pool_rows,
                            const moe_plan_t& p, int32_t H, void* dy_pool, float* d_topk_weights, uint32_t epoch,
                            const WsLayout& L, char* ws, hipStream_t stream) {
  CombineBwdArgs a;
  a.dout = static_cast<const uint8_t*>(dout);
  a.w = topk_weights;
  a.y = static_cast<const uint8_t*>(y_pool);
  a.pos = p.pos;
  a.T = p.T;
  a.K = p.K;
  a.H = H;
  a.pool_rows = pool_rows;
  a.dy = static_cast<uint8_t*>(dy_pool);
  a.dw = d_topk_weights;
  a.tile = p.tile;
  a.tile_shift = __builtin_ctz((unsigned)p.tile);
  a.tile_expert = p.tile_expert;
  a.offsets = p.offsets;
  a.counts = p.counts;
  a.tile_fill = reinterpret_cast<uint32_t*>(ws + L.bfill);
  a.tile_ready = p.tile_ready;
  a.epoch = epoch;
  // tokens per block: a multiple of the four waves, up to 64, leaving about two blocks per
  // CU (one device-scope release per block)
  const int cus = std::max(1, device_cu_count());
  a.tokens_per_block = std::max(4, std::min(64, p.T / (2 * cus)) & ~3);
  const int nch = H / 8;
  const dim3 grid((p.T + a.tokens_per_block - 1) / a.tokens_per_block);
  if (nch <= 64)
    hipLaunchKernelGGL(combine_backward_kernel<1>, grid, dim3(256), 0, stream, a);
  else if (nch <= 128)
    hipLaunchKernelGGL(combine_backward_kernel<2>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(combine_backward_kernel<4>, grid, dim3(256), 0, stream, a);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// --------------------------------------------------------------------------------
// Weight gradients: C[e] (N1 x N2, bf16) = sum over the real rows r of expert e's pool
// segment of A[r]^T B[r] (A [rows][N1], B [rows][N2], bf16), fp32 accumulation.
//
// Work unit = (expert, 256 x 256 output tile). Experts are ranked by row count, largest
// first, in every workgroup (a rank sort of the counts in LDS), and the units go out
// in that order, dealt boustrophedon over the grid's slots, so the long units start
// first. 8 waves, each 128 (N1) x 64 (N2) of the tile: the forward's 16x16x32 bf16
// MFMA layout with the B fragment first, so a lane holds one N1 row and four
// consecutive N2 columns.
//
// The contraction runs over pool rows, so both operands arrive K-major: a K step is 32
// pool rows of the 256 A columns and of the 256 B columns, copied as they are into LDS
// by LDS-DMA (512-byte rows, 16-byte chunks permuted per row by wg_swz; the DMA lands
// lane i at base + 16 i, so the permutation goes into the source addresses). The
// MFMA fragments (8 consecutive K of one column per lane) come out of the row-major
// tile through gfx950's transposing LDS read, ds_read_b64_tr_b16: within each group of
// 16 lanes, lane j reads 4 consecutive bf16 and lane i receives element i%4 of lanes
// i/4 + 4q, q = 0..3 -- so lane j of group g addresses row 8g + j/4 (+4 for the second
// half of the fragment), columns 4(j%4)..+4 of the 16-column block. Rows past the
// segment's real rows are read out of the buffer's range and land as zeros. A ring of
// four stages keeps three steps of DMA in flight (no registers held); one barrier per
// step, after a vmcnt wait that leaves the two newer steps outstanding. The stages are
// separate LDS objects used with constant indices, so the compiler can tell a step's
// reads from the DMA writes in flight (and adds no wait of its own).
//
// The K loop issues no vector ALU work: each lane's fragment and DMA offsets are fixed for
// the whole kernel (stage bases and the fragment's second half are immediate offsets), and
// the step's first row, the tile's first column and the segment's end go into the DMA's
// buffer resource (scalar work). At 16 cycles per MFMA and two waves per SIMD, per-step
// address arithmetic of about 90 vector instructions per wave had filled most of the issue
// slots the MFMAs leave. The last three steps of a unit already load the first three steps
// of the workgroup's next unit, whose output then goes out through a per-wave staging
// buffer while the ring keeps those steps.
// --------------------------------------------------------------------------------
struct WgradArgs {
  const uint8_t* A;
  const uint8_t* B;
  uint8_t* C;
  int32_t N1, N2;
  const int32_t* offsets;
  const int32_t* counts;
  int32_t E;
  int32_t tiles1, tiles2;      // N1 / 256, N2 / 256
};

constexpr int kWgTile = 256;
constexpr int kWgK = 32;                        // pool rows per K step
constexpr int kWgOpBytes = kWgK * kWgTile * 2;  // one operand's rows of a step: 16 KiB
constexpr int kWgMaxE = 1024;

typedef __bf16 wg_bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 wg_bf16x8 __attribute__((ext_vector_type(8)));
typedef float wg_f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) wg_bf16x4 wg_lds_bf16x4;

// byte of (row, byte b of the row) in a step's operand tile (512-byte rows)

// A transposing read touches 16 rows (8g + q and, for the second half, 8g + 4 + q; g, q
// = 0..3) at one 32-byte column segment; rows are 512 bytes apart, so the segment is moved
// by (q | g << 2) pairs of chunks: the 16 rows of a read land on 16 distinct 32-byte slots.
__device__ inline int wg_swz(int row) { return (((row & 3) | (((row >> 3) & 3) << 2)) << 1); }
__device__ inline uint32_t wg_at(int row, int b) {
  return (uint32_t)(row * 512 + ((((b >> 4) ^ wg_swz(row))) << 4) + (b & 15));
}

__global__ __launch_bounds__(512, 1) void wgrad_kernel(WgradArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t s_t0[2][kWgOpBytes];  // [A, B]
  __shared__ __attribute__((aligned(16))) uint8_t s_t1[2][kWgOpBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_t2[2][kWgOpBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_t3[2][kWgOpBytes];
  // experts in unit order with their segments: read from LDS when a unit starts (a global
  // load there would wait on every DMA and store the wave has in flight)
  __shared__ int s_order[kWgMaxE];
  __shared__ int s_r0[kWgMaxE];
  __shared__ int s_cnt[kWgMaxE];
  __shared__ __attribute__((aligned(16))) uint8_t s_out[8][2048];   // per-wave output staging
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2;          // N1 half
  const int wn = wave & 3;           // N2 quarter
  const int l16 = lane & 15;
  const int lhi = lane >> 4;

  // experts by descending row count (ties: lower index first)
  for (int e = tid; e < a.E; e += 512) {
    const int c = a.counts[e];
    int r = 0;
    for (int f = 0; f < a.E; ++f) {
      const int cf = a.counts[f];
      r += (cf > c) || (cf == c && f < e);
    }
    s_order[r] = e;
    s_r0[r] = a.offsets[e];
    s_cnt[r] = c;
  }
  __syncthreads();

  const int per_e = a.tiles1 * a.tiles2;
  const int total = a.E * per_e;
  const int G = gridDim.x;
  const int slot = (G & 7) == 0 ? (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3) : blockIdx.x;

  // DMA duty: wave w copies 1 KiB blocks 4w..4w+3 of a step (blocks 0..15: A, 16..31: B),
  // a block being two 512-byte rows; lane i lands at byte 16 i of its block
  const int blk0 = wave * 4;
  const bool dma_b = blk0 >= 16;
  const int lrow = (lane >> 5);      // row of the block this lane fills
  const int lchunk = lane & 31;      // LDS chunk slot it fills
  // fragment addressing: this lane's row in the 4-row group and its byte in the 16-column block
  const int frow = 8 * lhi + (l16 >> 2);
  const int fbyte = 8 * (l16 & 3);

  // a unit's sources: its expert, output tile and segment (wave-uniform), and its K steps
  // rounded up to whole rounds of four, at least one round (the steps past the segment add
  // zeros; a unit with no rows still runs one round, which carries the next unit's first
  // three steps)
  struct WgUnit {
    int e, t1, t2, r0, cnt, nr;
    bool ok;
  };
  auto unit_of = [&](int round) {
    WgUnit U;
    const int u = round * G + ((round & 1) ? G - 1 - slot : slot);
    U.ok = u < total;
    const int uu = U.ok ? u : 0;
    const int rk = uu / per_e;
    U.e = __builtin_amdgcn_readfirstlane(s_order[rk]);
    U.r0 = __builtin_amdgcn_readfirstlane(s_r0[rk]);
    U.cnt = __builtin_amdgcn_readfirstlane(s_cnt[rk]);
    const int tix = uu % per_e;
    U.t1 = tix / a.tiles2;
    U.t2 = tix % a.tiles2;
    const int nr = ((U.cnt + kWgK - 1) / kWgK + 3) & ~3;
    U.nr = nr > 4 ? nr : 4;
    return U;
  };

  const uint8_t* src = dma_b ? a.B : a.A;
  const uint32_t ld = (uint32_t)(dma_b ? a.N2 : a.N1) * 2u;
  // the lane's source offset within a step for each of its 4 blocks: row of the step times
  // the row pitch, plus its chunk moved by the row's permutation (the step's first row and
  // the tile's first column go into the buffer resource, so no per-step vector work)
  uint32_t voff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = 2 * ((blk0 + q) & 15) + lrow;
    voff[q] = (uint32_t)row * ld + (uint32_t)((lchunk ^ wg_swz(row)) << 4);
  }

  auto stage = [&](auto ST) -> uint8_t(*)[kWgOpBytes] {
    constexpr int k = decltype(ST)::value;
    if constexpr (k == 0) return s_t0;
    else if constexpr (k == 1) return s_t1;
    else if constexpr (k == 2) return s_t2;
    else return s_t3;
  };
  // the 4 DMAs of step s of a segment (r0, cnt) at byte column col0 into stage ST: the
  // resource starts at the step's first row and ends after the segment's last row, so the
  // rows past the segment read out of range (zeros, no traffic); cnt = 0 reads only zeros
  auto dma = [&](int r0, int cnt, uint32_t col0, int s, auto ST) {
    uint8_t* base = &stage(ST)[dma_b ? 1 : 0][0];
    const int left = cnt - s * kWgK;
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(src + (int64_t)(r0 + s * kWgK) * ld + col0, left > 0 ? (uint32_t)left * ld : 0u);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int blk = (blk0 + q) & 15;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(base + blk * 1024), 16, voff[q], 0, 0, 0);
    }
  };
  auto col_of = [&](const WgUnit& U) { return (uint32_t)((dma_b ? U.t2 : U.t1) * kWgTile) * 2u; };
  // the lane's fragment offsets within a step's operand tile: B fragments tn (N2 columns
  // wn*64 + tn*16 ..), A fragments tm (N1 columns wm*128 + tm*16 ..); the second half of a
  // fragment is 4 rows further (the row permutation ignores that row bit): +2048 bytes
  uint32_t fb_off[4], fa_off[8];
#pragma unroll
  for (int tn = 0; tn < 4; ++tn) fb_off[tn] = wg_at(frow, (wn * 64 + tn * 16) * 2 + fbyte);
#pragma unroll
  for (int tm = 0; tm < 8; ++tm) fa_off[tm] = wg_at(frow, (wm * 128 + tm * 16) * 2 + fbyte);
  auto frag = [&](const uint8_t* tile, uint32_t off) {
    const wg_bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((wg_lds_bf16x4*)(tile + off));
    const wg_bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((wg_lds_bf16x4*)(tile + off + 2048));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  using C2 = std::integral_constant<int, 2>;
  using C3 = std::integral_constant<int, 3>;

  int round = 0;
  WgUnit cur = unit_of(0);
  if (!cur.ok) return;
  // the first unit's steps 0..2 in flight, then wait for step 0. Every step issues its 4
  // DMAs (rows past the segment read zeros), so the counts below are exact. Later units'
  // first three steps go out during the last steps of the unit before (below).
  dma(cur.r0, cur.cnt, col_of(cur), 0, C0{});
  dma(cur.r0, cur.cnt, col_of(cur), 1, C1{});
  dma(cur.r0, cur.cnt, col_of(cur), 2, C2{});
  __builtin_amdgcn_s_waitcnt(0x0F78);  // vmcnt(8): step 0 has landed
  __syncthreads();

  wg_f32x4 acc[8][4];
  for (;;) {
    const WgUnit nxt = unit_of(round + 1);
    const uint32_t col_cur = col_of(cur), col_nxt = col_of(nxt);
    const int cnt_nxt = nxt.ok ? nxt.cnt : 0;
#pragma unroll
    for (int tm = 0; tm < 8; ++tm)
#pragma unroll
      for (int tn = 0; tn < 4; ++tn) acc[tm][tn] = wg_f32x4{0.f, 0.f, 0.f, 0.f};

    // step s computes from stage s % 4 and sends step s+3 into stage (s+3) % 4, the one
    // step s-1 read (all its reads are behind the last barrier). Past this unit's steps,
    // s+3 is the next unit's step s+3-nr (nr is a multiple of four, so the stages line up).
    auto step = [&](int s, auto ST, auto SN) {
      const uint8_t* ta = &stage(ST)[0][0];
      const uint8_t* tb = &stage(ST)[1][0];
      wg_bf16x8 fb[4];
#pragma unroll
      for (int tn = 0; tn < 4; ++tn) fb[tn] = frag(tb, fb_off[tn]);
      wg_bf16x8 fa_cur = frag(ta, fa_off[0]);
      // the step's first fragment reads go out before its DMAs, whose issue then overlaps
      // their latency (about 3% faster than the other way round)
      __builtin_amdgcn_sched_barrier(0);
      const bool here = s + 3 < cur.nr;
      dma(here ? cur.r0 : nxt.r0, here ? cur.cnt : cnt_nxt, here ? col_cur : col_nxt,
          here ? s + 3 : s + 3 - cur.nr, SN);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int tm = 0; tm < 8; ++tm) {
        wg_bf16x8 fa_next = fa_cur;
        if (tm + 1 < 8) fa_next = frag(ta, fa_off[tm + 1]);
#pragma unroll
        for (int tn = 0; tn < 4; ++tn)
          acc[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[tn], fa_cur, acc[tm][tn], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        fa_cur = fa_next;
      }
      // vmcnt(8): this wave's DMAs of step s+1 have landed (s+2, s+3 may not; loads land in
      // order, and a unit's output stores in between only make the wait longer); a bare
      // barrier then makes step s+1 whole for every wave. (A __syncthreads would add a
      // workgroup release, which waits for every DMA in flight.) The stage the next step
      // overwrites was read by this step, whose reads the MFMAs above have consumed.
      __builtin_amdgcn_s_waitcnt(0x0F78);
      __builtin_amdgcn_s_barrier();
    };
    // whole rounds of four steps (a branch between the steps would make the compiler
    // copy the accumulators at each exit)
    for (int s = 0; s < cur.nr; s += 4) {
      step(s, C0{}, C3{});
      step(s + 1, C1{}, C0{});
      step(s + 2, C2{}, C1{});
      step(s + 3, C3{}, C2{});
    }

    // Output through the wave's 2 KiB of staging: stored straight from the accumulators, a
    // lane's 8-byte pieces of 16 rows would make every store instruction touch 16 rows. Each
    // wave writes one 16-row tile row of its 128 x 64 bf16 block at a time (128-byte rows,
    // 16-byte chunks rotated by row), reads it back row-contiguous (a wave's LDS accesses
    // complete in order) and stores 2 x 8 whole 128-byte row segments. The ring is not
    // touched: it already holds the next unit's first steps.
    // Accumulator (tm, tn) of a lane: block row tm*16 + l16, block columns tn*16 + 4*lhi + (0..3).
    uint8_t* sw = &s_out[wave][0];
    // C[e][n1][n2]: block row r is n1 = t1*256 + wm*128 + r, block column c is n2 = t2*256 + wn*64 + c
    uint8_t* cbase = a.C + ((int64_t)cur.e * a.N1 + cur.t1 * kWgTile + wm * 128) * a.N2 * 2 +
                     (int64_t)(cur.t2 * kWgTile + wn * 64) * 2;
    // lane-dependent addresses formed here, from an opaque copy of the lane index: hoisted
    // above the K loop, they would hold registers there
    int el = lane;
    asm volatile("" : "+v"(el));
    const int e16 = el & 15, ehi = el >> 4, oc = el & 7, orow = el >> 3;
#pragma unroll
    for (int tm = 0; tm < 8; ++tm) {
#pragma unroll
      for (int tn = 0; tn < 4; ++tn) {
        u32x2 o;
        o.x = pack_bf16x2(acc[tm][tn][0], acc[tm][tn][1]);
        o.y = pack_bf16x2(acc[tm][tn][2], acc[tm][tn][3]);
        const int chunk = tn * 2 + (ehi >> 1);
        *reinterpret_cast<u32x2*>(sw + e16 * 128 + ((chunk ^ (e16 & 7)) << 4) + (ehi & 1) * 8) = o;
      }
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int row = p * 8 + orow;
        const u32x4 v = *reinterpret_cast<const u32x4*>(sw + row * 128 + ((oc ^ (row & 7)) << 4));
        *reinterpret_cast<u32x4*>(cbase + (int64_t)(tm * 16 + row) * a.N2 * 2 + oc * 16) = v;
      }
    }
    if (!nxt.ok) break;
    cur = nxt;
    ++round;
  }
  // the reloads of the last steps land before the workgroup ends
  wait_vm0();
}

int launch_wgrad(const moe_plan_t& p, int32_t pool_rows, const void* A, int32_t N1, const void* B, int32_t N2,
                 void* C, int32_t workgroups, hipStream_t stream) {
  WgradArgs a;
  a.A = static_cast<const uint8_t*>(A);
  a.B = static_cast<const uint8_t*>(B);
  a.C = static_cast<uint8_t*>(C);
  a.N1 = N1;
  a.N2 = N2;
  a.offsets = p.offsets;
  a.counts = p.counts;
  a.E = p.E_local;
  a.tiles1 = N1 / kWgTile;
  a.tiles2 = N2 / kWgTile;
  int grid = workgroups > 0 ? workgroups : device_cu_count();
  if (grid <= 0) return MOE_ERR_HIP;
  grid = std::min(grid, a.E * a.tiles1 * a.tiles2);
  hipLaunchKernelGGL(wgrad_kernel, dim3(grid), dim3(512), 0, stream, a);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// --------------------------------------------------------------------------------
// Load-time transposed weight permutation (bf16): out[e] is the fragment-ordered
// tiled layout (the bf16 one of moe_pack_weights) of w[e]^T, a [K][rows] matrix.
// One thread per 16-byte destination chunk, gathering its 8 values from 8 rows.
// --------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void pack_weights_t_kernel(const uint16_t* w, uint8_t* out, int64_t chunks,
                                                             int32_t rows, int32_t K) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= chunks) return;
  // transposed matrix per expert: n over K (its rows), k over rows (its K)
  const int64_t per_e = (int64_t)rows * K / 8;     // chunks per expert
  const int64_t e = c / per_e;
  const int64_t ce = c - e * per_e;
  const int64_t tile = ce >> 6;
  const int lane = (int)(ce & 63);
  const int ktiles = rows / 32;                     // K tiles per 16-row block of w^T
  const int64_t nb = tile / ktiles;
  const int kb = (int)(tile - nb * ktiles);
  const int64_t n = nb * 16 + (lane & 15);          // a column of w
  const int64_t k0 = (int64_t)kb * 32 + 8 * (lane >> 4);  // rows of w
  const uint16_t* src = w + e * (int64_t)rows * K;
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = (uint32_t)src[(k0 + 2 * i) * K + n] | ((uint32_t)src[(k0 + 2 * i + 1) * K + n] << 16);
  *reinterpret_cast<u32x4*>(out + c * 16) = u32x4{o[0], o[1], o[2], o[3]};
}

int launch_pack_weights_t(const void* w, int32_t E, int32_t rows, int32_t K, void* out, hipStream_t stream) {
  const int64_t chunks = (int64_t)E * rows * K / 8;
  hipLaunchKernelGGL(pack_weights_t_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(w), static_cast<uint8_t*>(out), chunks, rows, K);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
