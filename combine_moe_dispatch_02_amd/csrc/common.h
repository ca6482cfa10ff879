// Internal device helpers of libmoe355 (gfx950, wave64). Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe355.h"

namespace moe {

constexpr int kWave = 64;

// --------------------------------------------------------------------------
// workspace layout (shared by every entry point; offsets depend only on shape)
// --------------------------------------------------------------------------
constexpr int kPlanWaves = 4;            // waves per plan block
constexpr int kPairsPerWave = 1024;      // pairs one plan wave ranks (at most)
// a batch that one plan block covers is split over all of its waves
inline int32_t plan_pairs_per_wave(int64_t pairs) {
  return pairs <= (int64_t)kPlanWaves * kPairsPerWave ? kPairsPerWave / 4 : kPairsPerWave;
}

struct WsLayout {
  size_t err = 0;        // uint32: first device error code (0 = none)
  size_t done = 64;      // uint32: plan blocks finished (reset by the last one)
  size_t abort = 128;    // uint32: epoch of the last FFN call whose ready-flag wait timed out
  size_t tiles_done = 192;  // uint32: tiles whose ready flag dispatch has raised (plan zeroes it)
  size_t hist = 256;     // int32 [ncols][E_local]: per-wave expert counts, then bases
  size_t fill = 0;       // uint32 [ntiles_cap]: rows stored per tile by dispatch
  size_t bfill = 0;      // uint32 [ntiles_cap], right after fill: dy rows stored per tile by
                         // combine backward (reset by the store that completes the tile)
  size_t ydone = 0;      // uint32 [ntiles_cap]: GEMM Y units finished per tile (combine on completion)
  size_t cq = 0;         // uint32: combine items claimed (combine on completion)
  size_t h = 0;          // h [pool_rows][I]: bf16, or e4m3 codes
  size_t hs = 0;         // h's scale words (pool_rows x ceil(I/128), tile-major as scale_word())
  size_t plan_end = 0;   // end of what plan/dispatch need
  size_t total = 0;
  int32_t ncols = 0;
  int32_t ppw = 0;       // pairs per plan column
  int32_t ntiles_cap = 0;
};

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Scales of quantised activations (the pool in fp8 and mxfp4 mode, and h) are kept
// tile-major, one 4-byte word per (pool row, 128-column K group): the fp32 group scale,
// or the group's four E8M0 block bytes in block order. Row p's word for group g is
// word ((p / tile) * groups + g) * tile + p % tile, so the words one K step of a tile
// needs are tile consecutive words (a row-major [rows][groups] array would make that
// step a gather of one word from each of tile rows).
__host__ __device__ inline int64_t scale_word(int64_t row, int32_t g, int32_t groups, int32_t tile_shift) {
  return (((row >> tile_shift) * groups + g) << tile_shift) + (row & ((1 << tile_shift) - 1));
}

inline int64_t pool_rows_bound(int64_t T, int64_t K, int64_t E, int64_t tile) {
  return (T * K + E * (tile - 1)) / tile * tile;
}

inline WsLayout ws_layout(int32_t T, int32_t K, int32_t E, int32_t tile, int64_t pool_rows,
                          int32_t I, int32_t dtype) {
  WsLayout L;
  const int64_t pairs = (int64_t)T * K;
  const int64_t cap = pool_rows_bound(T, K, E, tile);
  L.ppw = plan_pairs_per_wave(pairs);
  L.ncols = (int32_t)((pairs + L.ppw - 1) / L.ppw);
  L.ntiles_cap = (int32_t)(cap / tile);
  L.fill = align_up(L.hist + (size_t)L.ncols * E * 4, 256);
  L.bfill = L.fill + (size_t)L.ntiles_cap * 4;   // contiguous: plan clears both in one pass
  L.ydone = align_up(L.bfill + (size_t)L.ntiles_cap * 4, 256);
  L.cq = align_up(L.ydone + (size_t)L.ntiles_cap * 4, 256);
  L.plan_end = L.cq + 256;
  if (pool_rows <= 0) pool_rows = cap;
  size_t off = L.plan_end;
  if (I > 0) {
    const size_t elem = dtype == MOE_BF16 ? 2 : 1;
    L.h = off;
    off = align_up(off + (size_t)pool_rows * I * elem, 256);
    if (dtype == MOE_FP8_E4M3_G128 || dtype == MOE_MXFP4) {
      L.hs = off;
      off = align_up(off + (size_t)pool_rows * ((I + 127) / 128) * 4, 256);
    }
  }
  L.total = off;
  return L;
}

// --------------------------------------------------------------------------
// device error word: the first error recorded wins
// --------------------------------------------------------------------------
__device__ inline void record_error(uint32_t* err, uint32_t code) {
  uint32_t expected = 0;
  __hip_atomic_compare_exchange_strong(err, &expected, code, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline uint32_t load_error(const uint32_t* err) {
  return __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// --------------------------------------------------------------------------
// wave primitives
// --------------------------------------------------------------------------
__device__ inline int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0)); }

__device__ inline uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

// number of set bits of `mask` in lanes below this one
__device__ inline int mask_rank(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
}

// Lanes of the wave whose `key` is equal form one group; returns this lane's
// group as a lane mask. One ballot per key bit: a lane's peers are the valid
// lanes that agree with it on every bit. Must be called by the whole wave.
__device__ inline uint64_t match_key(uint32_t key, bool valid, int nbits) {
  uint64_t peers = ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (key >> b) & 1u;
    const uint64_t m = ballot(bit);
    peers &= bit ? m : ~m;
  }
  return peers;
}

template <int CTRL, int ROW_MASK>
__device__ inline int dpp_or_zero(int v) {
  // lanes without a valid source (outside the row, or rows masked off) read 0
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xf, false);
}

// Inclusive prefix sum over the 64 lanes from DPP moves: a Hillis-Steele scan
// inside each 16-lane row (row_shr 1, 2, 4, 8), then row 15 -> rows 1 and 3
// (row_bcast:15) and lane 31 -> rows 2 and 3 (row_bcast:31).
__device__ inline int wave_inclusive_scan(int v) {
  v += dpp_or_zero<0x111, 0xf>(v);
  v += dpp_or_zero<0x112, 0xf>(v);
  v += dpp_or_zero<0x114, 0xf>(v);
  v += dpp_or_zero<0x118, 0xf>(v);
  v += dpp_or_zero<0x142, 0xa>(v);
  v += dpp_or_zero<0x143, 0xc>(v);
  return v;
}

__device__ inline int readlane(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }

// max over the 16 lanes of a DPP row (rotations by 8, 4, 2, 1); every lane gets it
__device__ inline float row16_max(float v) {
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xf, 0xf, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124, 0xf, 0xf, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x122, 0xf, 0xf, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x121, 0xf, 0xf, false)));
  return v;
}

// --------------------------------------------------------------------------
// number formats
// --------------------------------------------------------------------------
__device__ inline float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// two floats -> packed bf16 pair (round to nearest even; the hardware convert)
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// OCP E4M3 ("fn") codes: round to nearest, ties to even; magnitudes >= 448
// saturate to 448; the sign is kept (also for zero). gfx950's v_cvt_pk_fp8_f32
// converts to this format; its codes equal the format definition's for every
// representable value, every tie between neighbours and the saturation point
// (the bit-exact fp8 dispatch tests hold it to the oracle's encoder). Inputs are
// clamped to +-448 first, so any finite value saturates. Four codes, little-endian.
__device__ inline uint32_t pack_e4m3x4(float a, float b, float c, float d) {
  a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
  b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
  c = __builtin_amdgcn_fmed3f(c, -448.0f, 448.0f);
  d = __builtin_amdgcn_fmed3f(d, -448.0f, 448.0f);
  int p = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  p = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, p, true);
  return (uint32_t)p;
}

// one code
__device__ inline uint32_t e4m3_from_f32(float v) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(v, -448.0f, 448.0f), 0.0f, 0, false) & 0xffu;
}

// MXFP8 block scale (OCP MX): shared exponent floor(log2(amax)) - 8 (8 = exponent
// of e4m3's largest normal), clamped to [-127, 127], -127 for amax = 0 (NaN-free
// input assumed). frexp's exponent is exact for subnormal amax too.
__device__ inline int mx_e4m3_shared_exp(float amax) {
  const int e = amax > 0.f ? __builtin_amdgcn_frexp_expf(amax) - 1 - 8 : -127;
  return max(-127, min(127, e));
}
// 2^-e for a shared exponent of mx_e4m3_shared_exp (-e <= 127, and e <= 119 keeps it
// normal): multiplying by it is exact, so the codes equal those of x / 2^e
__device__ inline float mx_inv_scale(int e) { return __builtin_amdgcn_ldexpf(1.0f, -e); }

// --------------------------------------------------------------------------
// persistent grids and wait counters
// --------------------------------------------------------------------------
// Workgroup g of a persistent grid of G runs on XCD g % 8 (the dispatcher deals
// workgroups to the XCDs round-robin); slot(g) gives each XCD a contiguous run of
// G/8 work units per round, so units that share operands share that XCD's L2.
__device__ inline int unit_slot(int g, int G) { return (G & 7) == 0 ? (g & 7) * (G >> 3) + (g >> 3) : g; }

// s_waitcnt vmcnt(0), the other counters left alone (LDS-DMA loads have no
// register result for the compiler to wait on)
__device__ inline void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// s_waitcnt vmcnt(n) (n < 64), the other counters left alone
constexpr int vmcnt_enc(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }
// s_waitcnt lgkmcnt(0), the other counters left alone
constexpr int kLgkm0 = 0xC07F;

// --------------------------------------------------------------------------
// buffer resources: hardware range checks (out-of-range loads read 0, stores drop)
// --------------------------------------------------------------------------
constexpr int kRsrcWord3 = 0x00020000;

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ inline u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
// the same load with the non-temporal cache policy (NT bit): for data read exactly once
__device__ inline u32x4 buf_load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);
}
__device__ inline void buf_store16(u32x4 v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
}
__device__ inline void buf_store8(u32x2 v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 0);
}

}  // namespace moe
