// A5 -- combine: out[t] = sum over local k (ascending) of topk_weights[t,k] *
// y_pool[pos[t,k]], fp32 accumulation, one bf16 store per element.
//
// StreamEP README, "How it works": combine sends each token back once its
// expert outputs are computed; on one GPU that is a weighted gather-sum of the
// token's rows of the pool. A token with no local pair gets a zero row
// (its other pairs contribute 0), and weights are not renormalised.
//
// One wave per token, 16-byte lanes; each pair's row is read through a
// hardware-bounded buffer resource, and non-local pairs (pos = -1) are skipped
// on a wave-uniform mask.
#include "common.h"
#include "kernels.h"

namespace moe {

struct CombineArgs {
  const uint8_t* y;
  const float* w;
  const int32_t* pos;
  int32_t T, K, H;
  int32_t pool_rows;
  uint8_t* out;
};

template <int CPL>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const int lane = lane_id();
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  const int64_t pair0 = (int64_t)t * a.K;
  int p = lane < a.K ? a.pos[pair0 + lane] : -1;
  if (p >= a.pool_rows) p = -1;  // past the allocation: dispatch has reported it
  const float wt = lane < a.K ? a.w[pair0 + lane] : 0.f;
  const uint64_t have = ballot(p >= 0);
  const int H = a.H;
  const uint32_t row_bytes = (uint32_t)H * 2u;
  const int nch = H >> 3;
  const __amdgpu_buffer_rsrc_t orow = make_rsrc(a.out + (int64_t)t * row_bytes, row_bytes);

  for (int c0 = 0; c0 < nch; c0 += kWave * CPL) {
    float acc[CPL][8];
#pragma unroll
    for (int i = 0; i < CPL; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;
    for (int k = 0; k < a.K; ++k) {
      if (!((have >> k) & 1ull)) continue;
      const int pk = readlane(p, k);
      const float wk = __builtin_bit_cast(float, readlane(__builtin_bit_cast(int, wt), k));
      const __amdgpu_buffer_rsrc_t r = make_rsrc(a.y + (int64_t)pk * row_bytes, row_bytes);
      u32x4 v[CPL];
#pragma unroll
      for (int i = 0; i < CPL; ++i) v[i] = buf_load16(r, (uint32_t)(c0 + i * kWave + lane) * 16u);
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        acc[i][0] += wk * bf16_lo(v[i].x);
        acc[i][1] += wk * bf16_hi(v[i].x);
        acc[i][2] += wk * bf16_lo(v[i].y);
        acc[i][3] += wk * bf16_hi(v[i].y);
        acc[i][4] += wk * bf16_lo(v[i].z);
        acc[i][5] += wk * bf16_hi(v[i].z);
        acc[i][6] += wk * bf16_lo(v[i].w);
        acc[i][7] += wk * bf16_hi(v[i].w);
      }
    }
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      u32x4 o;
      o.x = pack_bf16x2(acc[i][0], acc[i][1]);
      o.y = pack_bf16x2(acc[i][2], acc[i][3]);
      o.z = pack_bf16x2(acc[i][4], acc[i][5]);
      o.w = pack_bf16x2(acc[i][6], acc[i][7]);
      buf_store16(o, orow, (uint32_t)(c0 + i * kWave + lane) * 16u);
    }
  }
}

int launch_combine(const void* y_pool, int32_t pool_rows, const float* topk_weights, const moe_plan_t& p,
                   int32_t H, void* out, hipStream_t stream) {
  CombineArgs a;
  a.y = static_cast<const uint8_t*>(y_pool);
  a.w = topk_weights;
  a.pos = p.pos;
  a.T = p.T;
  a.K = p.K;
  a.H = H;
  a.pool_rows = pool_rows;
  a.out = static_cast<uint8_t*>(out);
  const int nch = H / 8;
  const dim3 grid((p.T + 3) / 4);
  if (nch <= 64)
    hipLaunchKernelGGL(combine_kernel<1>, grid, dim3(256), 0, stream, a);
  else if (nch <= 128)
    hipLaunchKernelGGL(combine_kernel<2>, grid, dim3(256), 0, stream, a);
  else if (nch <= 256)
    hipLaunchKernelGGL(combine_kernel<4>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(combine_kernel<8>, grid, dim3(256), 0, stream, a);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
