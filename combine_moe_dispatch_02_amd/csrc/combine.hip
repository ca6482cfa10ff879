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
#include "combine.h"
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
  const float wt = lane < a.K ? (a.w != nullptr ? a.w[pair0 + lane] : 1.0f) : 0.f;
  const uint64_t have = ballot(p >= 0);
  combine_token<CPL>(a.y, p, wt, have, a.K, a.H, a.out + (int64_t)t * a.H * 2, lane);
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
