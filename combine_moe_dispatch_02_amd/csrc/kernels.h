// Host-side launchers of libmoe355's kernels (internal).
#pragma once

#include <hip/hip_runtime.h>

#include "common.h"

namespace moe {

// shape and pointer checks of a moe_plan_t (abi.hip)
int check_plan(const moe_plan_t* p);

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
  int32_t dispatch_cus;     // moe_tile_config.dispatch_cus: CUs GEMM A leaves free
  int32_t unit_rows;        // moe_tile_config.unit_rows: 0 auto, 128, 256
  uint64_t timeout_ticks;   // s_memrealtime ticks (100 MHz)
  const float* topk_w;      // combine on completion: [T][K] weights (null = FFN only)
  void* comb_out;           // combine on completion: out [T][H] bf16 (null = FFN only)
  void* g_pool;             // training: G = [gate | up] bf16 [pool_rows][2I] (null = not kept)
};

int launch_expert_ffn(const FfnLaunch& f, const WsLayout& L, char* ws, hipStream_t stream);

// ffn_sq.hip: one grouped GEMM of the FFN on 256 x 256 units (bf16, tiled weights, tile 128)
// The two GEMM A unit shapes of a call launched back to back, each running only if the plan
// makes it the faster one (ffn_sq.h, sq_gemm_a_wins): units per tile pair and grid of the
// 256-row kernel, units per tile and grid of the 128-row kernel
struct SqSelect {
  int32_t nb_sq, grid_sq, nb_big, grid_big;
};

struct SqArgs {
  const uint8_t* A;          // pool (GEMM A) or h (GEMM Y), bf16 [rows][K]
  int64_t lda;               // bytes per A row
  const uint8_t* B;          // tiled weights, expert-major
  int64_t b_expert;          // bytes per expert of B
  int32_t ktiles;            // K / 32: tiles per 16-row block of B
  uint8_t* out;              // h (GEMM A) or y_pool (GEMM Y), bf16
  int64_t ldo;               // bytes per out row
  uint8_t* g_save;           // training GEMM A: G = [gate | up] bf16 [rows][2I]
  int64_t g_ld;              // bytes per G row
  int32_t g_up;              // bytes from a G row's gate columns to its up columns (2I / 2 * 2)
  int32_t KS;                // K / 32 steps (a multiple of 4)
  int32_t NB;                // N blocks of 256 columns
  int32_t up_rb;             // GEMM A: first 16-row block of w1's up rows (I / 16)
  int32_t n_experts;
  int32_t max_tiles;         // pool_rows / 128
  int32_t group;             // row units per walk group
  const int32_t* offsets;
  const int32_t* counts;
  const int32_t* num_tiles;
  const uint32_t* tile_ready;
  const uint32_t* tiles_done;
  uint32_t epoch;
  uint32_t* err;
  uint32_t* abort_epoch;
  uint64_t timeout;
  int32_t wait_ready;
  int32_t select;            // 1: return at once unless the 256-row units win (sel)
  SqSelect sel;
};
int launch_ffn_sq(const SqArgs& a, int grid, bool gemm_a, bool gsave, hipStream_t stream);

// topk_weights null: unit weights (the dispatch's backward, a plain gather-sum)
int launch_combine(const void* y_pool, int32_t pool_rows, const float* topk_weights, const moe_plan_t& p,
                   int32_t H, void* out, hipStream_t stream);

// what the FFN supports (host-side check shared by validation and launch)
int ffn_supported(int32_t H, int32_t I, int32_t dtype, int32_t tile, int32_t block_n, int32_t weight_layout,
                  int32_t unit_rows, bool combine);
bool ffn_train_ok(int32_t H, int32_t I, int32_t dtype, int32_t tile, int32_t block_n);
// shapes the 256 x 256 kernel takes (both GEMMs)
bool ffn_sq_ok(int32_t H, int32_t I, int32_t dtype, int32_t tile, int32_t block_n, int32_t weight_layout,
               bool combine);

int launch_pack_weights(const void* w, int32_t E, int32_t rows, int32_t K, int32_t dtype, void* out,
                        hipStream_t stream);

// wait_epoch != 0: each work unit first waits until its pool tile's ready flag equals
// wait_epoch (timeout_ticks bounds one wait), and the persistent grid leaves leave_cus CUs
int launch_ffn_dgrad(const moe_plan_t& p, int32_t pool_rows, const void* A, const void* Bt, int32_t N, int32_t K,
                     void* out, void* g_pool, int32_t I, int epi, int32_t workgroups, int32_t unit_order,
                     int32_t a_stages, uint32_t wait_epoch, uint64_t timeout_ticks, int32_t leave_cus,
                     const WsLayout& L, char* ws, hipStream_t stream);

// backward.hip
int launch_combine_backward(const void* dout, const float* topk_weights, const void* y_pool, int32_t pool_rows,
                            const moe_plan_t& p, int32_t H, void* dy_pool, float* d_topk_weights, uint32_t epoch,
                            const WsLayout& L, char* ws, hipStream_t stream);
int launch_wgrad(const moe_plan_t& p, int32_t pool_rows, const void* A, int32_t N1, const void* B, int32_t N2,
                 void* C, int32_t workgroups, hipStream_t stream);
int launch_pack_weights_t(const void* w, int32_t E, int32_t rows, int32_t K, void* out, hipStream_t stream);

int launch_pack_mx_scales(const void* s, int32_t E, int32_t rows, int32_t K, void* out, hipStream_t stream);

int device_cu_count();

// calib.hip
int launch_calibrate_mfma(int32_t iters, float* sink, int32_t workgroups, hipStream_t stream);
int launch_calibrate_stream(const void* src, void* dst, int64_t bytes, int32_t mode, uint32_t* sink,
                            int32_t workgroups, hipStream_t stream);

}  // namespace moe
