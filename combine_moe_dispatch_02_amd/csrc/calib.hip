// Measurement kernels: the rates the roofline fractions are read against, measured on
// the device the layer runs on (the spec peaks are printed beside them).
//
//  * mfma_loop_kernel: every wave issues back-to-back v_mfma_f32_16x16x32_bf16 on 16
//    independent accumulators (no operand loads, no dependent chains), so the matrix
//    cores run at the rate the clock under that load allows.
//  * stream_kernel: a grid-stride pass over a buffer with 16-byte accesses per lane:
//    read (summed into a per-thread word, so the loads are not dead), write (a fill), or
//    copy, the three access mixes of dispatch (reads once, writes K times) and combine
//    (reads K rows, writes one).
#include "common.h"
#include "kernels.h"

namespace moe {

typedef __bf16 cal_bf16x8 __attribute__((ext_vector_type(8)));
typedef float cal_f32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(512) void mfma_loop_kernel(int32_t iters, float* sink) {
  const int lane = threadIdx.x & 63;
  // operands that depend on the lane, so nothing folds
  cal_bf16x8 x, y;
  for (int i = 0; i < 8; ++i) {
    x[i] = (__bf16)(0.001f * (lane + i));
    y[i] = (__bf16)(0.002f * (lane - i));
  }
  cal_f32x4 acc[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) acc[k] = cal_f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 16; ++k) acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, acc[k], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 16; ++k) s += acc[k][0] + acc[k][1] + acc[k][2] + acc[k][3];
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// mode 0: read src, 1: write dst, 2: copy src -> dst; bytes % 16 == 0
__global__ __launch_bounds__(256) void stream_kernel(const u32x4* src, u32x4* dst, int64_t n16, int32_t mode,
                                                     uint32_t* sink) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (mode == 0) {
    uint32_t acc = 0;
    for (; i < n16; i += stride) {
      const u32x4 v = __builtin_nontemporal_load(src + i);
      acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
  } else if (mode == 1) {
    const u32x4 v = {(uint32_t)i, 1u, 2u, 3u};
    for (; i < n16; i += stride) dst[i] = v;
  } else {
    for (; i < n16; i += stride) dst[i] = src[i];
  }
}

int launch_calibrate_mfma(int32_t iters, float* sink, int32_t workgroups, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_loop_kernel, dim3((unsigned)workgroups), dim3(512), 0, stream, iters, sink);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int launch_calibrate_stream(const void* src, void* dst, int64_t bytes, int32_t mode, uint32_t* sink,
                            int32_t workgroups, hipStream_t stream) {
  hipLaunchKernelGGL(stream_kernel, dim3((unsigned)workgroups), dim3(256), 0, stream,
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), bytes / 16, mode, sink);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
