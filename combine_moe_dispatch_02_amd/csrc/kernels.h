// Host-side launchers of libmoe355's kernels (internal).
#pragma once

#include <hip/hip_runtime.h>

#include "common.h"

namespace moe {

int launch_plan(const int32_t* topk_idx, const moe_plan_t& p, const WsLayout& L, char* ws,
                hipStream_t stream);

int launch_dispatch(const void* x, int32_t H, int32_t dtype, const moe_plan_t& p, int32_t pool_rows,
                    void* pool, void* pool_s, uint32_t epoch, const WsLayout& L, char* ws,
                    hipStream_t stream);

struct FfnLaunch {
  const moe_plan_t* plan;
  int32_t pool_rows;
  const void* pool;
  const void* pool_s;   // fp8: float group scales; mxfp4: E8M0 bytes
  const void* w1;
  const void* w1_s;     // fp8: float block scales; mxfp4: packed E8M0 bytes
  const void* w2;
  const void* w2_s;
  int32_t H, I, dtype;
  uint32_t epoch;
  void* y_pool;
  int32_t block_n;
  int32_t workgroups;
  int32_t unit_order;
  int32_t weight_layout;
  int32_t a_stages;         // moe_tile_config.a_stages
  uint64_t timeout_ticks;   // s_memrealtime ticks (100 MHz)
  const float* topk_w;      // combine on completion: [T][K] weights (null = FFN only)
  void* comb_out;           // combine on completion: out [T][H] bf16 (null = FFN only)
  void* g_pool;             // training: G = [gate | up] bf16 [pool_rows][2I] (null = not kept)
};

int launch_expert_ffn(const FfnLaunch& f, const WsLayout& L, char* ws, hipStream_t stream);

// topk_weights null: unit weights (the dispatch's backward, a plain gather-sum)
int launch_combine(const void* y_pool, int32_t pool_rows, const float* topk_weights, const moe_plan_t& p,
                   int32_t H, void* out, hipStream_t stream);

// what the FFN supports (host-side check shared by validation and launch)
int ffn_supported(int32_t H, int32_t I, int32_t dtype, int32_t tile, int32_t block_n, int32_t weight_layout);
bool ffn_train_ok(int32_t H, int32_t I, int32_t dtype, int32_t tile, int32_t block_n);

int launch_pack_weights(const void* w, int32_t E, int32_t rows, int32_t K, int32_t dtype, void* out,
                        hipStream_t stream);

int launch_ffn_dgrad(const moe_plan_t& p, int32_t pool_rows, const void* A, const void* Bt, int32_t N, int32_t K,
                     void* out, void* g_pool, int32_t I, int epi, int32_t workgroups, int32_t unit_order,
                     int32_t a_stages, const WsLayout& L, char* ws, hipStream_t stream);

// backward.hip
int launch_combine_backward(const void* dout, const float* topk_weights, const void* y_pool, int32_t pool_rows,
                            const moe_plan_t& p, int32_t H, void* dy_pool, float* d_topk_weights,
                            hipStream_t stream);
int launch_wgrad(const moe_plan_t& p, int32_t pool_rows, const void* A, int32_t N1, const void* B, int32_t N2,
                 void* C, int32_t workgroups, hipStream_t stream);
int launch_pack_weights_t(const void* w, int32_t E, int32_t rows, int32_t K, void* out, hipStream_t stream);

int launch_pack_mx_scales(const void* s, int32_t E, int32_t rows, int32_t K, void* out, hipStream_t stream);

int device_cu_count();

}  // namespace moe
