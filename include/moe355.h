/*
 * moe355.h -- C ABI of the single-GPU MoE dispatch -> expert FFN -> combine path
 * on MI355X (gfx950).
 *
 * The layer is the streaming MoE layer of the StreamEP README ("How it works"):
 *   - pool-layout dispatch: every routed (token, k) pair is written straight
 *     into its expert's segment of one pool, segments padded to whole GEMM
 *     tiles, and that pool is what the grouped GEMM reads (no permute pass);
 *   - per-tile streaming: a flag per pool tile is raised once the tile's rows
 *     are written, and the GEMM's work units wait on those flags, so compute
 *     can start on full tiles while others are still being written;
 *   - caller-owned streams: the caller hands in the streams (one for compute,
 *     one for the data movement); at most one host synchronisation per layer,
 *     the optional read-back of the pool size;
 *   - the forward grouped GEMMs "A" (w1, gate|up, then SwiGLU) and "Y" (w2);
 *   - combine: each token's expert outputs are reduced with its topk_weights.
 *
 * Conventions for every entry point:
 *   - Pointers named as device pointers are caller-owned device memory of the
 *     current HIP device. The library never allocates or frees memory and never
 *     synchronises, except moe_query_pool_rows and moe_get_error, which say so.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). Work is
 *     enqueued asynchronously on it; the call returns before the GPU runs it.
 *   - Argument errors are returned synchronously, before anything is enqueued:
 *     MOE_ERR_INVALID (bad pointer, size or value), MOE_ERR_UNSUPPORTED (valid
 *     but not built: a shape or dtype outside the kernels' constraints).
 *     A failed launch returns MOE_ERR_HIP. Errors detected on the device (a
 *     ready-flag wait that timed out, a pool row past the allocation) are
 *     recorded in the workspace and returned by moe_get_error.
 *   - Layouts are row-major and dense: x[T][H], topk_idx[T][K], pool[rows][H],
 *     w1[E_local][2I][H] (rows 0..I-1 gate, I..2I-1 up), w2[E_local][H][I],
 *     y_pool[rows][H], out[T][H].
 *   - Types: bf16 is IEEE binary32's upper half; fp8 is OCP E4M3 ("fn": bias 7,
 *     max 448, no infinities). fp8 scales are fp32: activations one per 1x128
 *     group of the contraction dim (tile-major words for the pool, see
 *     moe_dispatch), weights one per
 *     128x128 block (w1_s[E_local][2I/128][H/128], w2_s[E_local][H/128][I/128]).
 */
#ifndef MOE355_H
#define MOE355_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE355_API __attribute__((visibility("default")))

/* Status codes. */
enum {
  MOE_OK = 0,
  MOE_ERR_INVALID = 1,     /* bad argument, or a device-side bound check failed */
  MOE_ERR_UNSUPPORTED = 2, /* valid request outside what the kernels implement */
  MOE_ERR_HIP = 3,         /* a HIP runtime call or kernel launch failed */
  MOE_ERR_TIMEOUT = 4      /* a ready-flag wait on the device ran out of time */
};

/* Weight layouts (moe_tile_config.weight_layout). */
enum {
  MOE_WEIGHTS_ROW_MAJOR = 0,  /* w[E][rows][K] as described above */
  MOE_WEIGHTS_MFMA_TILED = 1  /* the same values permuted by moe_pack_weights */
};

/* Storage types of activations and weights. */
enum {
  MOE_BF16 = 0,          /* bf16 activations and weights */
  MOE_FP8_E4M3_G128 = 1, /* e4m3 activations per 1x128 group, e4m3 weights per 128x128 block */
  MOE_MXFP4 = 2          /* MXFP8 activations (e4m3 + E8M0 scale per 1x32 block along K) and
                            MXFP4 weights (e2m1 codes, two per byte with the even K in the low
                            nibble, + E8M0 scale per 1x32 block along K); the OCP MX formats */
};

/*
 * Placement plan: an expert-major, tile-padded pool (StreamEP README, "How it
 * works", pool-layout dispatch). Shape fields are set by the caller; the arrays
 * are caller-allocated device memory written by moe_plan.
 *   counts[e]      pairs routed to local expert e                       [E_local]
 *   offsets[e]     first pool row of expert e; offsets[E_local] = P      [E_local+1]
 *   pos[q]         pool row of pair q = t*K+k, -1 if not local           [T*K]
 *   src[p]         pair id of pool row p; -1 for padding and rows >= P   [rows_cap]
 *   tile_expert[i] local expert of pool tile i; -1 for i >= num_tiles    [rows_cap/tile]
 *   num_tiles[0]   P / tile                                              [1]
 *   tile_ready[i]  epoch of the dispatch call that filled tile i         [rows_cap/tile]
 * A segment holds its expert's pairs in ascending q and is padded to whole
 * tiles; an expert with no pairs gets no rows. Ids outside
 * [expert_begin, expert_begin+E_local), including -1, are not local.
 */
typedef struct moe_plan_t {
  int32_t T, K, expert_begin, E_local, tile;
  int32_t rows_cap; /* length of src; must be >= moe_pool_rows_upper_bound(T,K,E_local,tile) */
  int32_t* counts;
  int32_t* offsets;
  int32_t* pos;
  int32_t* src;
  int32_t* tile_expert;
  int32_t* num_tiles;
  uint32_t* tile_ready;
} moe_plan_t;

/*
 * GEMM tiling and launch overrides ("TileConfig" of the README's usage note:
 * tiles and CU counts come from the weight shapes; the struct overrides them).
 * Pass NULL, or zero fields, for the built-in choice.
 */
typedef struct moe_tile_config {
  int32_t block_n;          /* N columns per work unit: 128, 256 or 512 (0 = auto) */
  int32_t gemm_workgroups;  /* persistent GEMM grid size (0 = one per CU) */
  uint32_t spin_timeout_us; /* bound on one ready-flag wait (0 = 2 000 000 us) */
  int32_t unit_order;       /* work-unit walk: 1 = pool tile major, 2 = expert, N block, tile,
                               k = 3..9: expert, group of k-1 N blocks, tile (0 = auto: 3 on
                               the big-tile kernel, 1 for mxfp4 and on the general kernel) */
  int32_t weight_layout;    /* MOE_WEIGHTS_ROW_MAJOR or MOE_WEIGHTS_MFMA_TILED (w1 and w2) */
  int32_t a_stages;         /* pool-row pipeline of the big-tile GEMMs: 4 = a ring of four LDS
                               stages three K steps ahead (bf16 and mxfp4, K steps % 4 == 0),
                               2 = two stages; 0 = auto (4 where available). Same results. */
  int32_t dispatch_cus;     /* CUs that GEMM A's persistent grid leaves free, so that a
                               moe_dispatch running at the same time on another stream always
                               has CUs to run on while GEMM A waits for its tiles (0 = none:
                               right when dispatch has finished before the FFN starts, e.g. on
                               the same stream). GEMM A's grid is then the grid size minus this
                               (at least 1); GEMM Y is not affected. Same results. */
  int32_t unit_rows;        /* rows of a GEMM work unit: 128 = one pool tile (128 x 512 units),
                               256 = two pool tiles of one expert (256 x 256 units, both operands
                               by LDS-DMA; bf16, tiled weights, tile 128, H % 256 == 0,
                               I % 128 == 0, not with combine on completion); 0 = auto: 256
                               where it applies, else 128, except that GEMM A, where both
                               shapes apply, is launched on both and each launch decides on
                               the device from the plan (tile pairs and tiles per expert,
                               rounds over the grid) whether it computes or returns at once.
                               With 256, unit_order k >= 1 walks each expert in groups of k
                               tile pairs (0 = auto: 6). Same results. */
} moe_tile_config;

/* Host-only size helpers (no device access). */

/* Pool rows any plan of this shape can need: the padded segments satisfy
 * ceil(c/tile)*tile <= c + tile - 1, so P <= T*K + E_local*(tile-1); the result
 * is that bound rounded down to whole tiles. Returns 0 for invalid sizes. */
MOE355_API size_t moe_pool_rows_upper_bound(int32_t T, int32_t K, int32_t E_local, int32_t tile);

/* Bytes of the device workspace that moe_plan, moe_dispatch, moe_expert_ffn and
 * moe_get_error share for one layer: plan scratch, per-tile fill counters, the
 * device error word, and the intermediate h (pool_rows x I: bf16, e4m3 + fp32
 * 1x128 group scales, or e4m3 + E8M0 1x32 block scales). pool_rows = 0 means
 * moe_pool_rows_upper_bound. Returns 0 for invalid sizes. The workspace must be
 * zero-filled once before its first use. */
MOE355_API size_t moe_workspace_bytes(int32_t T, int32_t K, int32_t E_local, int32_t tile,
                                      int32_t pool_rows, int32_t I, int32_t dtype);

/*
 * A1. Build the placement plan from topk_idx (device, int32 [T][K]): histogram
 * of local pairs, padded exclusive scan into offsets, and a stable rank of each
 * pair inside its expert (the plan's layout is described at moe_plan_t). Also
 * clears tile_ready and the workspace's fill counters for the dispatch that
 * follows. Deterministic: no result depends on scheduling.
 * Errors: MOE_ERR_INVALID for null pointers, T < 1, K not in [1,16],
 * E_local not in [1,1024], tile not in {16,32,64,128}, rows_cap too small,
 * expert_begin < 0, or a workspace smaller than moe_workspace_bytes(...,0,0,0).
 */
MOE355_API int moe_plan(const int32_t* topk_idx, const moe_plan_t* plan, void* ws, size_t ws_bytes,
                        void* stream);

/*
 * moe_plan without a workspace, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same plan arrays, with the same values, as moe_plan. Its scratch (the per-column
 * histogram and the blocks' completion counter) lives in a 4 MiB device array inside
 * the library, one per device, held until the process ends; it allocates nothing and
 * calls no allocating routine. The scratch needed is 256 + 4 * E_local * ceil(T*K / p)
 * bytes, p = 256 pairs per column when T*K <= 4096, else 1024 (e.g. T*K up to 1 048 576
 * pairs for E_local <= 1020). Every call on a device shares that device's array: calls
 * that overlap on one device (on different streams, or from different host threads)
 * race and must be ordered by the caller. Unlike moe_plan it prepares no workspace for
 * moe_dispatch (a layer workspace's fill counters are not cleared): a caller that
 * dispatches uses moe_plan with its workspace.
 * Errors: those of moe_plan (except the workspace size); MOE_ERR_UNSUPPORTED when the
 * scratch needed exceeds 4 MiB; MOE_ERR_HIP when the array's address cannot be found.
 */
MOE355_API int moe_plan_noalloc(const int32_t* topk_idx, const moe_plan_t* plan, void* stream);

/* The one host sync of the layer (README, "Caller-owned streams"): waits for
 * `stream`, then copies offsets[E_local] (= P, the pool rows in use) to *host_P. */
MOE355_API int moe_query_pool_rows(const moe_plan_t* plan, int32_t* host_P, void* stream);

/*
 * A2. Dispatch (StreamEP README, "How it works": pool-layout dispatch and per-tile
 * streaming): pool[pos[t,k]] = x[t] for every local pair (device x bf16 [T][H]).
 * bf16: pool is bf16 [pool_rows][H] and pool_s must be NULL.
 * fp8:  pool is e4m3 [pool_rows][H] and pool_s holds pool_rows * H/128 fp32
 *       scale words; each 1x128 group g of x[t] is stored as codes e4m3(x/s) with
 *       s = amax/448 (s = 1 for an all-zero group), rounded to nearest even and
 *       saturated.
 * mxfp4: pool is e4m3 [pool_rows][H] and pool_s holds pool_rows * ceil(H/128)
 *       4-byte words of E8M0 scales (MXFP8, OCP MX specification): per 1x32
 *       block, e = floor(log2(amax)) - 8 clamped to [-127, 127] (-127 for an
 *       all-zero block), scale byte e + 127, codes e4m3(x * 2^-e) rounded to
 *       nearest even and saturated. The scaling is exact, so the codes depend on
 *       x alone. Byte b of a row's word for group g is the scale of its block 4g+b.
 * Scale words are tile-major (tile = plan->tile): pool row p's word for its
 * 128-column group g is word ((p / tile) * groups + g) * tile + p % tile, with
 * groups = H/128 (fp8) or ceil(H/128) (mxfp4), so that one K step of a pool
 * tile reads tile consecutive words.
 * Padding rows are not written. After a tile's real rows are stored the tile's
 * tile_ready entry is set to `epoch` with release ordering (device scope).
 * epoch must be nonzero and should change from one layer call to the next.
 * A pair whose row is >= pool_rows is not written and records MOE_ERR_INVALID.
 * Errors: MOE_ERR_INVALID (null pointers, H < 8, epoch 0, bad dtype; fp8 and
 * mxfp4 with pool_rows % tile != 0, since a row of a partial tile has no scale word),
 * MOE_ERR_UNSUPPORTED (H % 8 != 0; fp8 with H % 128 != 0; mxfp4 with H % 32 != 0).
 */
MOE355_API int moe_dispatch(const void* x, int32_t H, int32_t act_dtype, const moe_plan_t* plan,
                            int32_t pool_rows, void* pool, void* pool_s, uint32_t epoch,
                            void* ws, size_t ws_bytes, void* stream);

/*
 * A3 + A4. Expert FFN over the pool (StreamEP README, "How it works": the forward
 * grouped GEMMs A and Y of the compute kernels, fed tile by tile under per-tile
 * streaming), as a persistent grouped GEMM on MFMA:
 *   GEMM A: g = pool_tile . w1[e]^T (fp32 accumulate), h = silu(g_gate) * g_up,
 *           silu(z) = z / (1 + exp(-z)); h is stored as bf16 (bf16 mode), as
 *           e4m3 + one fp32 scale per 1x128 group (fp8 mode), or as MXFP8 like
 *           the pool (mxfp4 mode) in the workspace;
 *   GEMM Y: y_pool_tile = h . w2[e]^T (fp32 accumulate), stored bf16.
 * fp8 mode applies activation and weight scales per 128-wide K block in fp32.
 * pool_s holds the scale words moe_dispatch writes (fp8 and mxfp4, tile-major).
 * mxfp4 mode: w1 / w2 are MXFP4 codes in the
 * tiled layout of moe_pack_weights and w1_s / w2_s their E8M0 scales in the
 * layout of moe_pack_mx_scales; the scales are applied per 32-wide K block by
 * the matrix cores (scaled MFMA), so no rescaling happens in fp32.
 * Each work unit waits until tile_ready of its tile equals `epoch` (acquire);
 * a wait longer than the timeout records MOE_ERR_TIMEOUT and skips the unit.
 * Rows of y_pool that are padding are computed from whatever the pool holds and
 * are never read by moe_combine. Only the first pool_rows/tile tiles are
 * computed; a plan that needs more records MOE_ERR_INVALID.
 * Errors: MOE_ERR_INVALID (null pointers, bad dtype, epoch 0, small workspace,
 * pool_rows not a multiple of tile, a moe_tile_config field out of its range),
 * MOE_ERR_UNSUPPORTED (bf16: H % 128 or
 * I % 64 nonzero; fp8: H % 256 or I % 128 nonzero, or tile < 64; tiled weights:
 * bf16 with tile 128, H % 256 == 0 and I % 128 == 0 (256-row units), or with tile
 * 64 or 128, H % 512 == 0 and I % 256 == 0 (one-tile units), only; mxfp4: tiled
 * weights, tile 128, H % 512 == 0 and I % 256 == 0 only; unit_rows 256 outside the
 * 256-row units' shapes).
 */
MOE355_API int moe_expert_ffn(const moe_plan_t* plan, int32_t pool_rows, const void* pool,
                              const void* pool_s, const void* w1, const void* w1_s, const void* w2,
                              const void* w2_s, int32_t H, int32_t I, int32_t dtype, uint32_t epoch,
                              void* ws, size_t ws_bytes, void* y_pool, const moe_tile_config* cfg,
                              void* stream);

/*
 * A3 + A4 + A5 with combine on completion (StreamEP README, "How it works": a
 * token's combine waits only for its own expert outputs, not the whole FFN). Does what moe_expert_ffn
 * followed by moe_combine(y_pool, pool_rows, topk_weights, plan, H, out) on the same
 * stream does, with the same bits in out and y_pool. When GEMM Y runs on the big-tile
 * kernel (block N 512), each of its work units publishes the tile's progress in the
 * workspace (device-scope release), and the kernel's workgroups, once out of GEMM
 * work, take the tokens one per wave, wait (acquire) until every tile holding one of
 * the token's pairs is finished, and write the token's row of out: there is no
 * FFN -> combine join. The GEMM Y grid is then at most the CU count. For other
 * shapes the combine kernel runs after the FFN. A wait that outlasts the timeout
 * records MOE_ERR_TIMEOUT and writes the token's row as zeros.
 * topk_weights: device fp32 [T][K]; out: device bf16 [T][H], every row written.
 * Errors: those of moe_expert_ffn; MOE_ERR_INVALID for null topk_weights or out.
 */
MOE355_API int moe_expert_ffn_combine(const moe_plan_t* plan, int32_t pool_rows, const void* pool,
                                      const void* pool_s, const void* w1, const void* w1_s, const void* w2,
                                      const void* w2_s, int32_t H, int32_t I, int32_t dtype, uint32_t epoch,
                                      void* ws, size_t ws_bytes, void* y_pool, const float* topk_weights, void* out,
                                      const moe_tile_config* cfg, void* stream);

/*
 * Training forward (bf16). moe_expert_ffn, plus G = [gate | up] = pool_tile . w1[e]^T
 * (before the activation) stored bf16 into g_pool [pool_rows][2I] for the backward
 * pass; h stays in the workspace, where moe_expert_ffn_backward reads it. Needs the
 * big-tile kernel for every GEMM of the pass: tile 64 or 128, H % 512 == 0,
 * I % 512 == 0 (block_n 0 or 512); weights as for moe_expert_ffn.
 * Errors: those of moe_expert_ffn; MOE_ERR_INVALID for a null g_pool;
 * MOE_ERR_UNSUPPORTED for other shapes.
 */
MOE355_API int moe_expert_ffn_train(const moe_plan_t* plan, int32_t pool_rows, const void* pool, const void* w1,
                                    const void* w2, int32_t H, int32_t I, uint32_t epoch, void* ws, size_t ws_bytes,
                                    void* y_pool, void* g_pool, const moe_tile_config* cfg, void* stream);

/*
 * Backward of A5 (StreamEP README, "How it works": the backward pass mirrors the
 * forward, so combine's backward is a scatter into the pool). For every local pair
 * (t, k) with row p = pos[t,k]: dy_pool[p] = topk_weights[t,k] * dout[t] (fp32 product,
 * bf16 RNE store) and d_topk_weights[t,k] = sum_h dout[t,h] * y_pool[p,h] (fp32);
 * d_topk_weights is 0 for non-local pairs. dout: device bf16 [T][H]; y_pool as
 * written by the forward; dy_pool: device bf16 [pool_rows][H] (padding rows are not
 * written; it may be y_pool itself, each row being read before the same lane overwrites
 * it); d_topk_weights: device fp32 [T][K].
 * Per-tile streaming, mirrored: once a pool tile's real dy rows are stored, its
 * tile_ready entry is set to `epoch` (release, device scope), as moe_dispatch does for
 * the pool, so that moe_expert_ffn_backward with the same epoch, on another stream, can
 * start on the tile while other tiles are still being written. epoch must be nonzero and
 * differ from the epoch of the forward's moe_dispatch (the flags are the plan's
 * tile_ready). ws is the layer workspace after moe_plan: its per-tile counters of this
 * call live there (each tile's counter is back at zero after the call, so the backward
 * may be run again for the same plan).
 * Errors: MOE_ERR_INVALID (null pointers, epoch 0, small workspace),
 * MOE_ERR_UNSUPPORTED (H % 8 != 0).
 */
MOE355_API int moe_combine_backward(const void* dout, const float* topk_weights, const void* y_pool,
                                    int32_t pool_rows, const moe_plan_t* plan, int32_t H, void* dy_pool,
                                    float* d_topk_weights, uint32_t epoch, void* ws, size_t ws_bytes,
                                    void* stream);

/*
 * Backward grouped GEMMs Y and A (StreamEP README, "How it works": the four grouped
 * GEMMs are forward A / Y and backward A / Y), bf16, after moe_expert_ffn_train with
 * the same plan, pool and workspace:
 *   backward Y: dh = dy_pool . W2[e]; dG = [dh * u * silu'(g) | dh * silu(g)] with
 *               g, u from G, written over G in g_pool; dW2[e] = sum over the expert's
 *               real rows of dy^T h (h from the workspace);
 *   backward A: dx_pool = dG . W1[e]; dW1[e] = sum over the real rows of dG^T x.
 * silu'(z) = s (1 + z (1 - s)), s = 1 / (1 + exp(-z)); fp32 accumulation, bf16 (RNE)
 * results. w1t / w2t: the weights transposed and tiled by moe_pack_weights_transposed
 * (w1 [E][2I][H] -> its [H][2I] transposes, w2 [E][H][I] -> [I][H]). Outputs: dx_pool
 * bf16 [pool_rows][H] (padding rows hold garbage, never read by moe_dispatch_backward),
 * dw1 bf16 [E_local][2I][H], dw2 bf16 [E_local][H][I] (zero for an expert with no
 * pair). Padding rows of dy_pool are excluded from the weight gradients.
 * Each backward-Y work unit waits until tile_ready of its pool tile equals `epoch`, the
 * epoch moe_combine_backward raised (acquire), so the two may run on different streams
 * (StreamEP README, "How it works": the backward mirrors the forward's overlaps); the
 * weight gradients and backward A follow in stream order. A wait longer than the
 * timeout records MOE_ERR_TIMEOUT and skips the unit. cfg->dispatch_cus CUs are left
 * out of backward Y's persistent grid, for a combine backward running beside it.
 * Errors: MOE_ERR_INVALID (null pointers, epoch 0, bad pool_rows, small workspace, bad
 * cfg), MOE_ERR_UNSUPPORTED (shapes outside moe_expert_ffn_train's, or a pool whose
 * pool_rows * max(2I, H) * 2 bytes reach 4 GiB).
 */
MOE355_API int moe_expert_ffn_backward(const moe_plan_t* plan, int32_t pool_rows, const void* pool,
                                       const void* dy_pool, void* g_pool, const void* w1t, const void* w2t, int32_t H,
                                       int32_t I, uint32_t epoch, void* ws, size_t ws_bytes, void* dx_pool,
                                       void* dw1, void* dw2, const moe_tile_config* cfg, void* stream);

/*
 * Backward of A2 (the mirror of dispatch: a gather-sum): dx[t] = sum over k with
 * pos[t,k] >= 0, in ascending k, of dx_pool[pos[t,k]], fp32, bf16 (RNE) store; a token
 * with no local pair gets zeros. dx_pool: device bf16 [pool_rows][H]; dx: device bf16
 * [T][H]. Errors: MOE_ERR_INVALID (null pointers), MOE_ERR_UNSUPPORTED (H % 8 != 0).
 */
MOE355_API int moe_dispatch_backward(const void* dx_pool, int32_t pool_rows, const moe_plan_t* plan, int32_t H,
                                     void* dx, void* stream);

/*
 * A5. Combine (StreamEP README, "How it works": combine, the reduction of each
 * token's expert outputs with its routing weights; the usage sample's topk_weights):
 * out[t] = sum over k with pos[t,k] >= 0, in ascending k, of
 * topk_weights[t,k] * y_pool[pos[t,k]], accumulated in fp32 and stored bf16
 * (round to nearest even). Every row of out (bf16 [T][H]) is written; a token
 * with no local pair gets zeros. Weights are not renormalised.
 * y_pool: device bf16 [pool_rows][H]; a pair whose row is >= pool_rows is
 * skipped (dispatch has already reported it). topk_weights: device fp32 [T][K].
 * The caller orders this after moe_expert_ffn (same stream, or an event).
 * Errors: MOE_ERR_INVALID (null pointers), MOE_ERR_UNSUPPORTED (H % 8 != 0).
 */
MOE355_API int moe_combine(const void* y_pool, int32_t pool_rows, const float* topk_weights,
                           const moe_plan_t* plan, int32_t H, void* out, void* stream);

/*
 * Load-time weight permutation for the expert GEMMs (callers that cannot keep a
 * second copy of the weights use row-major weights instead). Copies w (device,
 * [E][rows][K] row-major: bf16, e4m3, or packed e2m1 [E][rows][K/2] per dtype)
 * into out (device, same size, must not overlap w) in MFMA fragment order, so
 * that every weight-fragment load of the GEMM reads 1 KiB of contiguous memory:
 *   bf16: for each expert, 16-row x 32-column tiles (row block rb, K block kb) at
 *         byte ((rb * K/32) + kb) * 1024; lane l (0..63) of a tile holds the 8
 *         values w[rb*16 + l%16][kb*32 + 8*(l/16) ..+8] at byte l*16.
 *   fp8:  16 x 128 tiles at ((rb * K/128) + kb) * 2048; half h (0,1) of lane l at
 *         byte h*1024 + l*16 holds w[rb*16 + l%16][kb*128 + 32*(l/16) + 16h ..+16].
 *   mxfp4: 16 x 128 tiles at ((rb * K/128) + kb) * 1024; lane l at byte l*16 holds
 *         the 32 codes w[rb*16 + l%16][kb*128 + 32*(l/16) ..+32] (16 bytes as
 *         stored, low nibble first).
 * Values are moved, never changed. Use with moe_tile_config.weight_layout =
 * MOE_WEIGHTS_MFMA_TILED. Scales keep their layout (fp8) or are permuted by
 * moe_pack_mx_scales (mxfp4).
 * Errors: MOE_ERR_INVALID (null pointers, E/rows/K < 1, bad dtype),
 * MOE_ERR_UNSUPPORTED (rows % 16 != 0, K % 32 != 0 (bf16) or % 128 (fp8, mxfp4)).
 */
MOE355_API int moe_pack_weights(const void* w, int32_t E, int32_t rows, int32_t K, int32_t dtype, void* out,
                                void* stream);

/*
 * Load-time transposed re-layout for the backward data GEMMs (bf16 only): out[e] is
 * the bf16 tiled layout of moe_pack_weights applied to w[e]^T, the [K][rows] transpose
 * of w[e] ([rows][K] row-major): tile (nb, kb) of 16 x 32 at byte ((nb * rows/32) + kb)
 * * 1024, lane l holding w[e][kb*32 + 8*(l/16) + i][nb*16 + l%16], i = 0..7.
 * Errors: MOE_ERR_INVALID (null pointers, sizes < 1, unknown dtype, overlap),
 * MOE_ERR_UNSUPPORTED (fp8 / mxfp4, K % 16 != 0, rows % 32 != 0).
 */
MOE355_API int moe_pack_weights_transposed(const void* w, int32_t E, int32_t rows, int32_t K, int32_t dtype,
                                           void* out, void* stream);

/*
 * Load-time permutation of MXFP4 weight scales (E8M0 bytes, device, [E][rows][K/32]
 * row-major, one per 1x32 block along K) into the order the scaled MFMA takes them:
 * for each expert, the 16-row x 128-K tile (rb, kb) owns 64 bytes at
 * ((rb * K/128) + kb) * 64, and byte l holds s[rb*16 + l%16][kb*4 + l/16] (lane l's
 * operand scale). out has the size of s and must not overlap it.
 * Errors: MOE_ERR_INVALID (null pointers, E/rows/K < 1),
 * MOE_ERR_UNSUPPORTED (rows % 16 != 0 or K % 128 != 0).
 */
MOE355_API int moe_pack_mx_scales(const void* s, int32_t E, int32_t rows, int32_t K, void* out, void* stream);

/*
 * Measurement helpers (not part of a layer call): the rates the layer's roofline
 * fractions are read against, measured on the current device.
 * moe_calibrate_mfma: `workgroups` workgroups of 8 waves each issue `iters` x 16
 * back-to-back v_mfma_f32_16x16x32_bf16 (16 384 flops each) on register operands, i.e.
 * workgroups * 8 * iters * 16 * 16384 flops. sink: device float [workgroups * 512],
 * overwritten (it only keeps the result alive).
 * moe_calibrate_stream: one grid-stride pass of `workgroups` x 256 threads over `bytes`
 * (a multiple of 16) with 16-byte accesses: mode 0 reads src (sink: device uint32
 * [workgroups * 256]), 1 writes dst, 2 copies src to dst (non-overlapping).
 * Errors: MOE_ERR_INVALID (null pointers the mode needs, iters < 1, workgroups not in
 * [1, 65535], bytes < 16 or not a multiple of 16, unknown mode).
 */
MOE355_API int moe_calibrate_mfma(int32_t iters, float* sink, int32_t workgroups, void* stream);
MOE355_API int moe_calibrate_stream(const void* src, void* dst, int64_t bytes, int32_t mode, uint32_t* sink,
                                    int32_t workgroups, void* stream);

/* Waits for `stream`, returns the first error recorded on the device in the
 * workspace since the last call (MOE_OK if none) and clears it. */
MOE355_API int moe_get_error(void* ws, size_t ws_bytes, void* stream);

/* Static text for a status code. */
MOE355_API const char* moe_status_string(int status);

/* Number of compute units of the current device (0 if none is visible). */
MOE355_API int moe_device_cu_count(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE355_H */
