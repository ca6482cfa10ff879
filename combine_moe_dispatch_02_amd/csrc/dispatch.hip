// A2 -- dispatch: copy every local (token, k) pair's activation row into its
// pool row and raise the per-tile ready flags.
//
// StreamEP README, "How it works": received pairs land directly in the
// expert-major, tile-padded pool (pool-layout dispatch), and dispatch signals
// each pool tile as it fills (per-tile streaming).
//
// Each token's row is read once (16-byte lanes) and stored to each of its
// local pairs' rows, so x is read T*H*2 bytes once and the pool written once per
// pair. In fp8 mode each 1x128 group (16 lanes x 8 values) is quantised on the
// way: scale = amax/448 in fp32 (1 for an all-zero group), code = e4m3(x /
// scale) with IEEE division, round to nearest even, saturating. In mxfp4 mode
// the activations become MXFP8 (OCP MX): each 1x32 block (4 lanes x 8 values)
// gets the E8M0 scale 2^e, e = floor(log2(amax)) - 8, and codes e4m3(x * 2^-e),
// exact scaling then the same rounding. Scales go to their tile-major words
// (scale_word: one K step of a pool tile reads them as consecutive words). A wave handles
// a run of 64/K tokens; a workgroup's runs are published with a single
// device-scope release (an L2 write-back on this chip, so it is paid per
// workgroup, not per row or per wave); each stored pair then bumps its tile's
// fill counter, and the lane that completes a tile's real rows stores the epoch
// into tile_ready with release ordering.
#include "common.h"
#include "kernels.h"

#include <algorithm>

namespace moe {

struct DispatchArgs {
  const uint16_t* x;
  int32_t T, K, H;
  int32_t tile, tile_shift;
  const int32_t* pos;
  const int32_t* tile_expert;
  const int32_t* offsets;
  const int32_t* counts;
  uint8_t* pool;
  void* pool_s;                // scale words, tile-major (scale_word): fp8 float, mxfp4 4 E8M0 bytes
  int32_t pool_rows;
  uint32_t* tile_fill;
  uint32_t* tile_ready;
  uint32_t* tiles_done;     // count of raised flags: equal to num_tiles once every tile is in
  uint32_t epoch;
  uint32_t* err;
  int32_t tokens_per_wave;  // tokens_per_wave * K <= 64
};

// max over the 4 lanes of a DPP quad (quad_perm [1,0,3,2] then [2,3,0,1])
__device__ inline float quad_max(float v) {
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xf, 0xf, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xf, 0xf, false)));
  return v;
}

// One token's row: read once, stored to each of its local pairs' rows.
// FMT: 0 bf16 copy, 1 fp8 1x128 groups, 2 MXFP8 1x32 blocks.
template <int CPL, int FMT>
__device__ inline void dispatch_token(const DispatchArgs& a, int t, int p, uint64_t dest, int lane) {
  constexpr bool FP8 = FMT != 0;
  const int H = a.H;
  const int nch = H >> 3;  // 16-byte chunks of 8 bf16 in a row
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x + (int64_t)t * H, (uint32_t)H * 2u);
  const int64_t out_row_bytes = FP8 ? H : (int64_t)H * 2;
  for (int c0 = 0; c0 < nch; c0 += kWave * CPL) {
    u32x4 v[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) v[i] = buf_load16_nt(xr, (uint32_t)(c0 + i * kWave + lane) * 16u);  // x is read once
    if constexpr (FMT == 0) {
      for (int k = 0; k < a.K; ++k) {
        if (!((dest >> k) & 1ull)) continue;
        const int pk = readlane(p, k);
        const __amdgpu_buffer_rsrc_t pr = make_rsrc(a.pool + (int64_t)pk * out_row_bytes, (uint32_t)out_row_bytes);
#pragma unroll
        for (int i = 0; i < CPL; ++i) buf_store16(v[i], pr, (uint32_t)(c0 + i * kWave + lane) * 16u);
      }
    } else if constexpr (FMT == 2) {
      u32x2 q[CPL];
      uint32_t sb[CPL];
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        float f[8];
        f[0] = bf16_lo(v[i].x); f[1] = bf16_hi(v[i].x);
        f[2] = bf16_lo(v[i].y); f[3] = bf16_hi(v[i].y);
        f[4] = bf16_lo(v[i].z); f[5] = bf16_hi(v[i].z);
        f[6] = bf16_lo(v[i].w); f[7] = bf16_hi(v[i].w);
        float m = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(f[j]));
        m = quad_max(m);                       // the 4 lanes of a DPP quad hold one block
        const int e = mx_e4m3_shared_exp(m);
        const float inv = mx_inv_scale(e);
        sb[i] = (uint32_t)(e + 127);
        q[i].x = pack_e4m3x4(f[0] * inv, f[1] * inv, f[2] * inv, f[3] * inv);
        q[i].y = pack_e4m3x4(f[4] * inv, f[5] * inv, f[6] * inv, f[7] * inv);
      }
      const int words = (H + 127) >> 7;
      for (int k = 0; k < a.K; ++k) {
        if (!((dest >> k) & 1ull)) continue;
        const int pk = readlane(p, k);
        const __amdgpu_buffer_rsrc_t pr = make_rsrc(a.pool + (int64_t)pk * out_row_bytes, (uint32_t)out_row_bytes);
        // byte (c >> 2) & 3 of the row's scale word for group c >> 4 (chunk c: 8 elements)
        uint8_t* srow = static_cast<uint8_t*>(a.pool_s) + scale_word(pk, 0, words, a.tile_shift) * 4;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
          const int c = c0 + i * kWave + lane;
          buf_store8(q[i], pr, (uint32_t)c * 8u);
          if ((lane & 3) == 0 && c < nch)
            srow[((int64_t)(c >> 4) << a.tile_shift) * 4 + ((c >> 2) & 3)] = (uint8_t)sb[i];
        }
      }
    } else {
      u32x2 q[CPL];
      float s[CPL];
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        float f[8];
        f[0] = bf16_lo(v[i].x); f[1] = bf16_hi(v[i].x);
        f[2] = bf16_lo(v[i].y); f[3] = bf16_hi(v[i].y);
        f[4] = bf16_lo(v[i].z); f[5] = bf16_hi(v[i].z);
        f[6] = bf16_lo(v[i].w); f[7] = bf16_hi(v[i].w);
        float m = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(f[j]));
        m = row16_max(m);                      // the 16 lanes of a DPP row hold one group
        const float sc = m > 0.f ? m / 448.0f : 1.0f;
        s[i] = sc;
        q[i].x = pack_e4m3x4(f[0] / sc, f[1] / sc, f[2] / sc, f[3] / sc);
        q[i].y = pack_e4m3x4(f[4] / sc, f[5] / sc, f[6] / sc, f[7] / sc);
      }
      const int groups = H >> 7;
      for (int k = 0; k < a.K; ++k) {
        if (!((dest >> k) & 1ull)) continue;
        const int pk = readlane(p, k);
        const __amdgpu_buffer_rsrc_t pr = make_rsrc(a.pool + (int64_t)pk * out_row_bytes, (uint32_t)out_row_bytes);
        float* srow = static_cast<float*>(a.pool_s) + scale_word(pk, 0, groups, a.tile_shift);
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
          const int c = c0 + i * kWave + lane;
          buf_store8(q[i], pr, (uint32_t)c * 8u);
          if ((lane & 15) == 0 && c < nch) srow[(int64_t)(c >> 4) << a.tile_shift] = s[i];
        }
      }
    }
  }
}

// A wave dispatches a run of `tpw` consecutive tokens (tpw * K <= 64). The block's
// WPB waves then publish together: a barrier (every store of the block has reached
// L2), one device-scope release by wave 0 (an L2 write-back on this chip, which is
// what makes the rows visible to the other XCDs -- paid once per block rather than
// once per wave: a write-back by every wave costs as much as before even when the
// L2 is mostly clean), then wave 0 bumps the fill count of every stored pair's tile
// (relaxed), and the lane whose count completes a tile acquires and stores the
// epoch into tile_ready (release). The host picks the largest WPB (up to 16) that
// still gives every CU a block.
template <int CPL, int FMT, int WPB>
__global__ __launch_bounds__(64 * WPB) void dispatch_kernel(DispatchArgs a) {
  const int lane = lane_id();
  const int w = threadIdx.x >> 6;
  const int tpw = a.tokens_per_wave;
  const int tb = blockIdx.x * WPB * tpw;  // the block's first token
  const int t0 = tb + w * tpw;
  const int ntok = t0 < a.T ? min(tpw, a.T - t0) : 0;
  for (int i = 0; i < ntok; ++i) {
    const int t = t0 + i;
    int p = lane < a.K ? a.pos[(int64_t)t * a.K + lane] : -1;
    if (p >= a.pool_rows) {
      record_error(a.err, MOE_ERR_INVALID);
      p = -1;
    }
    const uint64_t dest = ballot(p >= 0);
    if (dest != 0) dispatch_token<CPL, FMT>(a, t, p, dest, lane);
  }

  __syncthreads();
  if (w != 0) return;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  const int npairs = (min(a.T, tb + WPB * tpw) - tb) * a.K;
  for (int q = lane; q < npairs; q += 64) {
    int p = a.pos[(int64_t)tb * a.K + q];
    if (p >= a.pool_rows) p = -1;
    if (p >= 0) {
      const int ti = p >> a.tile_shift;
      const uint32_t old = __hip_atomic_fetch_add(&a.tile_fill[ti], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int e = a.tile_expert[ti];
      const int real = min(a.tile, a.offsets[e] + a.counts[e] - (ti << a.tile_shift));
      if ((int)old + 1 == real) {
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        __hip_atomic_store(&a.tile_ready[ti], a.epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_add(a.tiles_done, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

template <int FMT, int WPB>
static void launch_cpl(int cpl, dim3 grid, hipStream_t s, const DispatchArgs& a) {
  switch (cpl) {
    case 1: hipLaunchKernelGGL((dispatch_kernel<1, FMT, WPB>), grid, dim3(64 * WPB), 0, s, a); break;
    case 2: hipLaunchKernelGGL((dispatch_kernel<2, FMT, WPB>), grid, dim3(64 * WPB), 0, s, a); break;
    case 4: hipLaunchKernelGGL((dispatch_kernel<4, FMT, WPB>), grid, dim3(64 * WPB), 0, s, a); break;
    default: hipLaunchKernelGGL((dispatch_kernel<8, FMT, WPB>), grid, dim3(64 * WPB), 0, s, a); break;
  }
}

template <int FMT>
static void launch_wpb(int wpb, int cpl, int waves, hipStream_t s, const DispatchArgs& a) {
  const dim3 grid((waves + wpb - 1) / wpb);
  switch (wpb) {
    case 1: launch_cpl<FMT, 1>(cpl, grid, s, a); break;
    case 2: launch_cpl<FMT, 2>(cpl, grid, s, a); break;
    case 4: launch_cpl<FMT, 4>(cpl, grid, s, a); break;
    case 8: launch_cpl<FMT, 8>(cpl, grid, s, a); break;
    default: launch_cpl<FMT, 16>(cpl, grid, s, a); break;
  }
}

int launch_dispatch(const void* x, int32_t H, int32_t dtype, const moe_plan_t& p, int32_t pool_rows,
                    void* pool, void* pool_s, uint32_t epoch, const WsLayout& L, char* ws,
                    hipStream_t stream) {
  DispatchArgs a;
  a.x = static_cast<const uint16_t*>(x);
  a.T = p.T;
  a.K = p.K;
  a.H = H;
  a.tile = p.tile;
  a.tile_shift = __builtin_ctz((unsigned)p.tile);
  a.pos = p.pos;
  a.tile_expert = p.tile_expert;
  a.offsets = p.offsets;
  a.counts = p.counts;
  a.pool = static_cast<uint8_t*>(pool);
  a.pool_s = pool_s;
  a.pool_rows = pool_rows;
  a.tile_fill = reinterpret_cast<uint32_t*>(ws + L.fill);
  a.tile_ready = p.tile_ready;
  a.tiles_done = reinterpret_cast<uint32_t*>(ws + L.tiles_done);
  a.epoch = epoch;
  a.err = reinterpret_cast<uint32_t*>(ws + L.err);
  const int nch = H / 8;
  const int cpl = nch <= 64 ? 1 : nch <= 128 ? 2 : nch <= 256 ? 4 : 8;
  const int cus = std::max(1, device_cu_count());
  // tokens per wave: up to 64/K (one pos load per wave and token run), fewer when that
  // leaves under two waves per CU -- a wave walks its tokens one after another, so a
  // small batch wants one or two tokens per wave
  a.tokens_per_wave = std::max(1, std::min(64 / p.K, p.T / (2 * cus)));
  const int waves = (p.T + a.tokens_per_wave - 1) / a.tokens_per_wave;
  // waves per block: the largest power of two up to 16 that leaves a block per CU
  int wpb = 1;
  while (wpb < 16 && waves / (2 * wpb) >= cus) wpb *= 2;
  if (dtype == MOE_FP8_E4M3_G128)
    launch_wpb<1>(wpb, cpl, waves, stream, a);
  else if (dtype == MOE_MXFP4)
    launch_wpb<2>(wpb, cpl, waves, stream, a);
  else
    launch_wpb<0>(wpb, cpl, waves, stream, a);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
