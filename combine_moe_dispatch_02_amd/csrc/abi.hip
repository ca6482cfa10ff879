// C ABI of libmoe355: argument validation, workspace layout, launches.
// The contract of each entry point is stated in include/moe355.h.
#include <hip/hip_runtime.h>
#include <rocprofiler-sdk-roctx/roctx.h>

#include <algorithm>
#include <cstring>

#include "common.h"
#include "kernels.h"

namespace moe {

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return n;
}

// a named roctx range around one entry point's launches (seen by rocprofv3 --marker-trace)
struct TraceRange {
  explicit TraceRange(const char* name) { roctxRangePushA(name); }
  ~TraceRange() { roctxRangePop(); }
};

static bool valid_tile(int32_t tile) { return tile == 16 || tile == 32 || tile == 64 || tile == 128; }

// shape checks common to every call that takes a plan
int check_plan(const moe_plan_t* p) {
  if (!p) return MOE_ERR_INVALID;
  if (p->T < 1 || p->K < 1 || p->K > 16 || p->E_local < 1 || p->E_local > 1024 || p->expert_begin < 0)
    return MOE_ERR_INVALID;
  if (!valid_tile(p->tile)) return MOE_ERR_INVALID;
  if ((int64_t)p->T * p->K > (int64_t)1 << 30) return MOE_ERR_UNSUPPORTED;
  const int64_t bound = pool_rows_bound(p->T, p->K, p->E_local, p->tile);
  if (bound > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  if (p->rows_cap < bound || p->rows_cap % p->tile != 0) return MOE_ERR_INVALID;
  if (!p->counts || !p->offsets || !p->pos || !p->src || !p->tile_expert || !p->num_tiles || !p->tile_ready)
    return MOE_ERR_INVALID;
  return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" {

MOE355_API size_t moe_pool_rows_upper_bound(int32_t T, int32_t K, int32_t E_local, int32_t tile) {
  if (T < 1 || K < 1 || K > 16 || E_local < 1 || E_local > 1024 || !valid_tile(tile)) return 0;
  return (size_t)pool_rows_bound(T, K, E_local, tile);
}

MOE355_API size_t moe_workspace_bytes(int32_t T, int32_t K, int32_t E_local, int32_t tile, int32_t pool_rows,
                                      int32_t I, int32_t dtype) {
  if (T < 1 || K < 1 || K > 16 || E_local < 1 || E_local > 1024 || !valid_tile(tile)) return 0;
  if (pool_rows < 0 || I < 0 || (dtype != MOE_BF16 && dtype != MOE_FP8_E4M3_G128 && dtype != MOE_MXFP4)) return 0;
  if (dtype == MOE_FP8_E4M3_G128 && I % 128 != 0) return 0;
  if (dtype == MOE_MXFP4 && I % 32 != 0) return 0;
  return ws_layout(T, K, E_local, tile, pool_rows, I, dtype).total;
}

MOE355_API int moe_plan(const int32_t* topk_idx, const moe_plan_t* plan, void* ws, size_t ws_bytes,
                        void* stream) {
  TraceRange trace("moe_plan");
  int rc = check_plan(plan);
  if (rc != MOE_OK) return rc;
  if (!topk_idx || !ws) return MOE_ERR_INVALID;
  const WsLayout L = ws_layout(plan->T, plan->K, plan->E_local, plan->tile, 0, 0, MOE_BF16);
  if (ws_bytes < L.plan_end) return MOE_ERR_INVALID;
  return launch_plan(topk_idx, *plan, L, static_cast<char*>(ws), static_cast<hipStream_t>(stream));
}

MOE355_API int moe_query_pool_rows(const moe_plan_t* plan, int32_t* host_P, void* stream) {
  int rc = check_plan(plan);
  if (rc != MOE_OK) return rc;
  if (!host_P) return MOE_ERR_INVALID;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(host_P, plan->offsets + plan->E_local, sizeof(int32_t), hipMemcpyDeviceToHost, s) !=
      hipSuccess)
    return MOE_ERR_HIP;
  return hipStreamSynchronize(s) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

MOE355_API int moe_dispatch(const void* x, int32_t H, int32_t act_dtype, const moe_plan_t* plan,
                            int32_t pool_rows, void* pool, void* pool_s, uint32_t epoch, void* ws,
                            size_t ws_bytes, void* stream) {
  TraceRange trace("moe_dispatch");
  int rc = check_plan(plan);
  if (rc != MOE_OK) return rc;
  if (!x || !pool || !ws || epoch == 0 || H < 8 || pool_rows < 0) return MOE_ERR_INVALID;
  if (act_dtype == MOE_BF16) {
    if (pool_s) return MOE_ERR_INVALID;
  } else if (act_dtype == MOE_FP8_E4M3_G128) {
    if (!pool_s) return MOE_ERR_INVALID;
    if (H % 128 != 0) return MOE_ERR_UNSUPPORTED;
  } else if (act_dtype == MOE_MXFP4) {
    if (!pool_s) return MOE_ERR_INVALID;
    if (H % 32 != 0) return MOE_ERR_UNSUPPORTED;
  } else {
    return MOE_ERR_INVALID;
  }
  // scale words are tile-major: a row of a partial last tile would address a word past
  // pool_rows * groups, so a scaled pool must hold whole tiles
  if (pool_s && pool_rows % plan->tile != 0) return MOE_ERR_INVALID;
  if (H % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)H * 2 > INT32_MAX / 2) return MOE_ERR_UNSUPPORTED;
  const WsLayout L = ws_layout(plan->T, plan->K, plan->E_local, plan->tile, 0, 0, MOE_BF16);
  if (ws_bytes < L.plan_end) return MOE_ERR_INVALID;
  return launch_dispatch(x, H, act_dtype, *plan, pool_rows, pool, pool_s, epoch, L, static_cast<char*>(ws),
                         static_cast<hipStream_t>(stream));
}

}  // extern "C"

// moe_expert_ffn and moe_expert_ffn_combine: the same validation and launch; the
// second also takes topk_weights and out (non-null) for combine on completion
static int expert_ffn(const moe_plan_t* plan, int32_t pool_rows, const void* pool, const void* pool_s,
                      const void* w1, const void* w1_s, const void* w2, const void* w2_s, int32_t H, int32_t I,
                      int32_t dtype, uint32_t epoch, void* ws, size_t ws_bytes, void* y_pool,
                      const float* topk_weights, void* out, void* g_pool, const moe_tile_config* cfg,
                      void* stream) {
  int rc = check_plan(plan);
  if (rc != MOE_OK) return rc;
  if (!pool || !w1 || !w2 || !ws || !y_pool || epoch == 0 || H < 1 || I < 1) return MOE_ERR_INVALID;
  if (pool_rows < 1 || pool_rows % plan->tile != 0) return MOE_ERR_INVALID;
  const bool scaled = dtype == MOE_FP8_E4M3_G128 || dtype == MOE_MXFP4;
  if (dtype != MOE_BF16 && !scaled) return MOE_ERR_INVALID;
  if (scaled && (!pool_s || !w1_s || !w2_s)) return MOE_ERR_INVALID;
  if (!scaled && (pool_s || w1_s || w2_s)) return MOE_ERR_INVALID;
  const int32_t block_n = cfg ? cfg->block_n : 0;
  const int32_t layout = cfg ? cfg->weight_layout : MOE_WEIGHTS_ROW_MAJOR;
  if (layout != MOE_WEIGHTS_ROW_MAJOR && layout != MOE_WEIGHTS_MFMA_TILED) return MOE_ERR_INVALID;
  const int32_t unit_rows = cfg ? cfg->unit_rows : 0;
  rc = ffn_supported(H, I, dtype, plan->tile, block_n, layout, unit_rows, out != nullptr);
  if (rc != MOE_OK) return rc;
  if ((int64_t)pool_rows * H * 2 > ((int64_t)1 << 40)) return MOE_ERR_UNSUPPORTED;
  const WsLayout L = ws_layout(plan->T, plan->K, plan->E_local, plan->tile, pool_rows, I, dtype);
  if (ws_bytes < L.total) return MOE_ERR_INVALID;
  if (cfg && cfg->gemm_workgroups < 0) return MOE_ERR_INVALID;
  if (g_pool != nullptr && !ffn_train_ok(H, I, dtype, plan->tile, block_n)) return MOE_ERR_UNSUPPORTED;
  FfnLaunch f{};
  f.g_pool = g_pool;
  f.topk_w = topk_weights;
  f.comb_out = out;
  f.plan = plan;
  f.pool_rows = pool_rows;
  f.pool = pool;
  f.pool_s = pool_s;
  f.w1 = w1;
  f.w1_s = w1_s;
  f.w2 = w2;
  f.w2_s = w2_s;
  f.H = H;
  f.I = I;
  f.dtype = dtype;
  f.epoch = epoch;
  f.y_pool = y_pool;
  f.block_n = block_n;
  f.workgroups = cfg ? cfg->gemm_workgroups : 0;
  f.unit_order = cfg ? cfg->unit_order : 0;
  f.weight_layout = layout;
  f.a_stages = cfg ? cfg->a_stages : 0;
  if (f.a_stages != 0 && f.a_stages != 2 && f.a_stages != 4) return MOE_ERR_INVALID;
  f.dispatch_cus = cfg ? cfg->dispatch_cus : 0;
  if (f.dispatch_cus < 0) return MOE_ERR_INVALID;
  f.unit_rows = unit_rows;
  if (f.unit_order < 0 || f.unit_order > 9) return MOE_ERR_INVALID;
  const uint64_t us = (cfg && cfg->spin_timeout_us) ? cfg->spin_timeout_us : 2000000u;
  f.timeout_ticks = us * 100u;  // s_memrealtime counts at 100 MHz
  return launch_expert_ffn(f, L, static_cast<char*>(ws), static_cast<hipStream_t>(stream));
}

extern "C" {

MOE355_API int moe_expert_ffn(const moe_plan_t* plan, int32_t pool_rows, const void* pool, const void* pool_s,
                              const void* w1, const void* w1_s, const void* w2, const void* w2_s, int32_t H,
                              int32_t I, int32_t dtype, uint32_t epoch, void* ws, size_t ws_bytes, void* y_pool,
                              const moe_tile_config* cfg, void* stream) {
  TraceRange trace("moe_expert_ffn");
  return expert_ffn(plan, pool_rows, pool, pool_s, w1, w1_s, w2, w2_s, H, I, dtype, epoch, ws, ws_bytes, y_pool,
                    nullptr, nullptr, nullptr, cfg, stream);
}

MOE355_API int moe_expert_ffn_combine(const moe_plan_t* plan, int32_t pool_rows, const void* pool,
                                      const void* pool_s, const void* w1, const void* w1_s, const void* w2,
                                      const void* w2_s, int32_t H, int32_t I, int32_t dtype, uint32_t epoch,
                                      void* ws, size_t ws_bytes, void* y_pool, const float* topk_weights, void* out,
                                      const moe_tile_config* cfg, void* stream) {
  TraceRange trace("moe_expert_ffn_combine");
  if (!topk_weights || !out) return MOE_ERR_INVALID;
  if (H % 8 != 0) return MOE_ERR_UNSUPPORTED;
  return expert_ffn(plan, pool_rows, pool, pool_s, w1, w1_s, w2, w2_s, H, I, dtype, epoch, ws, ws_bytes, y_pool,
                    topk_weights, out, nullptr, cfg, stream);
}

MOE355_API int moe_expert_ffn_train(const moe_plan_t* plan, int32_t pool_rows, const void* pool, const void* w1,
                                    const void* w2, int32_t H, int32_t I, uint32_t epoch, void* ws, size_t ws_bytes,
                                    void* y_pool, void* g_pool, const moe_tile_config* cfg, void* stream) {
  TraceRange trace("moe_expert_ffn_train");
  if (!g_pool) return MOE_ERR_INVALID;
  return expert_ffn(plan, pool_rows, pool, nullptr, w1, nullptr, w2, nullptr, H, I, MOE_BF16, epoch, ws, ws_bytes,
                    y_pool, nullptr, nullptr, g_pool, cfg, stream);
}

MOE355_API int moe_combine_backward(const void* dout, const float* topk_weights, const void* y_pool,
                                    int32_t pool_rows, const moe_plan_t* plan, int32_t H, void* dy_pool,
                                    float* d_topk_weights, uint32_t epoch, void* ws, size_t ws_bytes,
                                    void* stream) {
  TraceRange trace("moe_combine_backward");
  int rc = check_plan(plan);
  if (rc != MOE_OK) return rc;
  if (!dout || !topk_weights || !y_pool || !dy_pool || !d_topk_weights || !ws || H < 8 || pool_rows < 0 ||
      epoch == 0)
    return MOE_ERR_INVALID;
  if (H % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)H * 2 > INT32_MAX / 2) return MOE_ERR_UNSUPPORTED;
  const WsLayout L = ws_layout(plan->T, plan->K, plan->E_local, plan->tile, pool_rows, 0, MOE_BF16);
  if (ws_bytes < L.plan_end) return MOE_ERR_INVALID;
  return launch_combine_backward(dout, topk_weights, y_pool, pool_rows, *plan, H, dy_pool, d_topk_weights, epoch,
                                 L, static_cast<char*>(ws), static_cast<hipStream_t>(stream));
}

MOE355_API int moe_expert_ffn_backward(const moe_plan_t* plan, int32_t pool_rows, const void* pool,
                                       const void* dy_pool, void* g_pool, const void* w1t, const void* w2t, int32_t H,
                                       int32_t I, uint32_t epoch, void* ws, size_t ws_bytes, void* dx_pool, void* dw1,
                                       void* dw2, const moe_tile_config* cfg, void* stream) {
  TraceRange trace("moe_expert_ffn_backward");
  int rc = check_plan(plan);
  if (rc != MOE_OK) return rc;
  if (!pool || !dy_pool || !g_pool || !w1t || !w2t || !ws || !dx_pool || !dw1 || !dw2 || H < 1 || I < 1 ||
      epoch == 0)
    return MOE_ERR_INVALID;
  if (pool_rows < 1 || pool_rows % plan->tile != 0) return MOE_ERR_INVALID;
  const int32_t block_n = cfg ? cfg->block_n : 0;
  if (!ffn_train_ok(H, I, MOE_BF16, plan->tile, block_n)) return MOE_ERR_UNSUPPORTED;
  // 32-bit buffer offsets over the pool-sized operands
  if ((int64_t)pool_rows * std::max(2 * I, H) * 2 >= ((int64_t)1 << 32) - 16) return MOE_ERR_UNSUPPORTED;
  if (cfg && (cfg->gemm_workgroups < 0 || cfg->unit_order < 0 || cfg->unit_order > 9)) return MOE_ERR_INVALID;
  if (cfg && cfg->a_stages != 0 && cfg->a_stages != 2 && cfg->a_stages != 4) return MOE_ERR_INVALID;
  if (cfg && cfg->dispatch_cus < 0) return MOE_ERR_INVALID;
  const WsLayout L = ws_layout(plan->T, plan->K, plan->E_local, plan->tile, pool_rows, I, MOE_BF16);
  if (ws_bytes < L.total) return MOE_ERR_INVALID;
  char* w = static_cast<char*>(ws);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int32_t wgs = cfg ? cfg->gemm_workgroups : 0;
  const int32_t order = cfg ? cfg->unit_order : 0;
  const int32_t stages = cfg ? cfg->a_stages : 0;
  const int32_t leave = cfg ? cfg->dispatch_cus : 0;
  const uint64_t us = (cfg && cfg->spin_timeout_us) ? cfg->spin_timeout_us : 2000000u;
  const uint64_t ticks = us * 100u;  // s_memrealtime counts at 100 MHz
  // backward GEMM Y: dh = dy . W2 -> dG (over G), each unit after its dy tile's flag; then
  // dW2 = dy^T h
  rc = launch_ffn_dgrad(*plan, pool_rows, dy_pool, w2t, I, H, nullptr, g_pool, I, 1, wgs, order, stages, epoch,
                        ticks, leave, L, w, s);
  if (rc != MOE_OK) return rc;
  rc = launch_wgrad(*plan, pool_rows, dy_pool, H, w + L.h, I, dw2, wgs, s);
  if (rc != MOE_OK) return rc;
  // backward GEMM A: dx_pool = dG . W1, and dW1 = dG^T X
  rc = launch_ffn_dgrad(*plan, pool_rows, g_pool, w1t, H, 2 * I, dx_pool, nullptr, I, 0, wgs, order, stages, 0, 0,
                        0, L, w, s);
  if (rc != MOE_OK) return rc;
  return launch_wgrad(*plan, pool_rows, g_pool, 2 * I, pool, H, dw1, wgs, s);
}

MOE355_API int moe_dispatch_backward(const void* dx_pool, int32_t pool_rows, const moe_plan_t* plan, int32_t H,
                                     void* dx, void* stream) {
  TraceRange trace("moe_dispatch_backward");
  int rc = check_plan(plan);
  if (rc != MOE_OK) return rc;
  if (!dx_pool || !dx || H < 8 || pool_rows < 0) return MOE_ERR_INVALID;
  if (H % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)H * 2 > INT32_MAX / 2) return MOE_ERR_UNSUPPORTED;
  return launch_combine(dx_pool, pool_rows, nullptr, *plan, H, dx, static_cast<hipStream_t>(stream));
}

MOE355_API int moe_combine(const void* y_pool, int32_t pool_rows, const float* topk_weights,
                           const moe_plan_t* plan, int32_t H, void* out, void* stream) {
  TraceRange trace("moe_combine");
  int rc = check_plan(plan);
  if (rc != MOE_OK) return rc;
  if (!y_pool || !topk_weights || !out || H < 8 || pool_rows < 0) return MOE_ERR_INVALID;
  if (H % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)H * 2 > INT32_MAX / 2) return MOE_ERR_UNSUPPORTED;
  return launch_combine(y_pool, pool_rows, topk_weights, *plan, H, out, static_cast<hipStream_t>(stream));
}

MOE355_API int moe_pack_weights(const void* w, int32_t E, int32_t rows, int32_t K, int32_t dtype, void* out,
                                void* stream) {
  TraceRange trace("moe_pack_weights");
  if (!w || !out || E < 1 || rows < 1 || K < 1) return MOE_ERR_INVALID;
  if (dtype != MOE_BF16 && dtype != MOE_FP8_E4M3_G128 && dtype != MOE_MXFP4) return MOE_ERR_INVALID;
  if (rows % 16 != 0 || K % (dtype == MOE_BF16 ? 32 : 128) != 0) return MOE_ERR_UNSUPPORTED;
  const int64_t bytes = dtype == MOE_MXFP4 ? (int64_t)rows * K / 2 : (int64_t)rows * K * (dtype == MOE_BF16 ? 2 : 1);
  if (bytes > ((int64_t)1 << 32)) return MOE_ERR_UNSUPPORTED;
  const char* a = static_cast<const char*>(w);
  const char* b = static_cast<const char*>(out);
  if (a < b + bytes * E && b < a + bytes * E) return MOE_ERR_INVALID;  // overlap
  return launch_pack_weights(w, E, rows, K, dtype, out, static_cast<hipStream_t>(stream));
}

MOE355_API int moe_pack_weights_transposed(const void* w, int32_t E, int32_t rows, int32_t K, int32_t dtype,
                                           void* out, void* stream) {
  TraceRange trace("moe_pack_weights_transposed");
  if (!w || !out || E < 1 || rows < 1 || K < 1) return MOE_ERR_INVALID;
  if (dtype != MOE_BF16) return dtype == MOE_FP8_E4M3_G128 || dtype == MOE_MXFP4 ? MOE_ERR_UNSUPPORTED : MOE_ERR_INVALID;
  if (K % 16 != 0 || rows % 32 != 0) return MOE_ERR_UNSUPPORTED;
  const int64_t bytes = (int64_t)rows * K * 2;
  if (bytes > ((int64_t)1 << 32)) return MOE_ERR_UNSUPPORTED;
  const char* a = static_cast<const char*>(w);
  const char* b = static_cast<const char*>(out);
  if (a < b + bytes * E && b < a + bytes * E) return MOE_ERR_INVALID;  // overlap
  return launch_pack_weights_t(w, E, rows, K, out, static_cast<hipStream_t>(stream));
}

MOE355_API int moe_pack_mx_scales(const void* s, int32_t E, int32_t rows, int32_t K, void* out, void* stream) {
  TraceRange trace("moe_pack_mx_scales");
  if (!s || !out || E < 1 || rows < 1 || K < 1) return MOE_ERR_INVALID;
  if (rows % 16 != 0 || K % 128 != 0) return MOE_ERR_UNSUPPORTED;
  const int64_t bytes = (int64_t)rows * (K / 32);
  if (bytes * E > ((int64_t)1 << 40)) return MOE_ERR_UNSUPPORTED;
  const char* a = static_cast<const char*>(s);
  const char* b = static_cast<const char*>(out);
  if (a < b + bytes * E && b < a + bytes * E) return MOE_ERR_INVALID;  // overlap
  return launch_pack_mx_scales(s, E, rows, K, out, static_cast<hipStream_t>(stream));
}

MOE355_API int moe_calibrate_mfma(int32_t iters, float* sink, int32_t workgroups, void* stream) {
  if (!sink || iters < 1 || workgroups < 1 || workgroups > 65535) return MOE_ERR_INVALID;
  TraceRange trace("moe_calibrate_mfma");
  return launch_calibrate_mfma(iters, sink, workgroups, static_cast<hipStream_t>(stream));
}

MOE355_API int moe_calibrate_stream(const void* src, void* dst, int64_t bytes, int32_t mode, uint32_t* sink,
                                    int32_t workgroups, void* stream) {
  if (bytes < 16 || bytes % 16 != 0 || workgroups < 1 || workgroups > 65535) return MOE_ERR_INVALID;
  if (mode == 0 ? (!src || !sink) : mode == 1 ? !dst : mode == 2 ? (!src || !dst) : true) return MOE_ERR_INVALID;
  if (mode == 2) {
    const char* a = static_cast<const char*>(src);
    const char* b = static_cast<const char*>(dst);
    if (a < b + bytes && b < a + bytes) return MOE_ERR_INVALID;  // overlap
  }
  TraceRange trace("moe_calibrate_stream");
  return launch_calibrate_stream(src, dst, bytes, mode, sink, workgroups, static_cast<hipStream_t>(stream));
}

MOE355_API int moe_get_error(void* ws, size_t ws_bytes, void* stream) {
  if (!ws || ws_bytes < 256) return MOE_ERR_INVALID;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t code = 0;
  uint32_t* err = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + WsLayout{}.err);
  if (hipMemcpyAsync(&code, err, sizeof(code), hipMemcpyDeviceToHost, s) != hipSuccess) return MOE_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return MOE_ERR_HIP;
  if (code != 0) {
    if (hipMemsetAsync(err, 0, sizeof(uint32_t), s) != hipSuccess) return MOE_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return MOE_ERR_HIP;
  }
  return (int)code;
}

MOE355_API const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case MOE_ERR_HIP: return "HIP runtime error";
    case MOE_ERR_TIMEOUT: return "ready-flag wait timed out";
  }
  return "unknown status";
}

MOE355_API int moe_device_cu_count(void) { return device_cu_count(); }

}  // extern "C"
