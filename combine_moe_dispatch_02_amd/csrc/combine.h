// The weighted gather-sum of one token (A5), shared by the combine kernel and the
// combine-on-completion tail of the GEMM Y kernel. Internal; not part of the C ABI.
#pragma once

#include "common.h"

namespace moe {

// One wave: out_row = sum over local k (ascending) of w_k * y[p_k], fp32 accumulation,
// one bf16 (RNE) store per element. Lane k < K holds the pair's pool row p (-1 when
// not local or past the pool) and weight wt; `have` is the ballot of p >= 0. Rows are
// read through hardware-bounded buffer resources, 16 bytes per lane, CPL chunks per
// lane at a time, with the non-temporal cache policy (each pool row is read once; at the
// skew workload this took the combine kernel from 240 to 211 us).
template <int CPL>
__device__ inline void combine_token(const uint8_t* y, int p, float wt, uint64_t have, int K, int H,
                                     uint8_t* out_row, int lane) {
  const uint32_t row_bytes = (uint32_t)H * 2u;
  const int nch = H >> 3;
  const __amdgpu_buffer_rsrc_t orow = make_rsrc(out_row, row_bytes);
  for (int c0 = 0; c0 < nch; c0 += kWave * CPL) {
    float acc[CPL][8];
#pragma unroll
    for (int i = 0; i < CPL; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;
    for (int k = 0; k < K; ++k) {
      if (!((have >> k) & 1ull)) continue;
      const int pk = readlane(p, k);
      const float wk = __builtin_bit_cast(float, readlane(__builtin_bit_cast(int, wt), k));
      const __amdgpu_buffer_rsrc_t r = make_rsrc(y + (int64_t)pk * row_bytes, row_bytes);
      u32x4 v[CPL];
#pragma unroll
      for (int i = 0; i < CPL; ++i) v[i] = buf_load16_nt(r, (uint32_t)(c0 + i * kWave + lane) * 16u);
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

// The same sum with every pair's loads issued before any is consumed: KMAX rows x CPL
// 16-byte chunks per lane in flight (for K <= KMAX). Rows of non-local k get an empty
// buffer resource (their loads return 0 and touch no memory) and are skipped in the
// sum, so the result has the bits of combine_token's.
template <int CPL, int KMAX>
__device__ inline void combine_token_wide(const uint8_t* y, int p, float wt, uint64_t have, int K, int H,
                                          uint8_t* out_row, int lane) {
  const uint32_t row_bytes = (uint32_t)H * 2u;
  const int nch = H >> 3;
  const __amdgpu_buffer_rsrc_t orow = make_rsrc(out_row, row_bytes);
  __amdgpu_buffer_rsrc_t r[KMAX];
  float wk[KMAX];
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    const bool on = k < K && ((have >> k) & 1ull);
    const int pk = readlane(p, k < K ? k : 0);
    r[k] = make_rsrc(y + (on ? (int64_t)pk * row_bytes : 0), on ? row_bytes : 0u);
    wk[k] = __builtin_bit_cast(float, readlane(__builtin_bit_cast(int, wt), k < K ? k : 0));
  }
  for (int c0 = 0; c0 < nch; c0 += kWave * CPL) {
    u32x4 v[KMAX][CPL];
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
#pragma unroll
      for (int i = 0; i < CPL; ++i) v[k][i] = buf_load16(r[k], (uint32_t)(c0 + i * kWave + lane) * 16u);
    float acc[CPL][8];
#pragma unroll
    for (int i = 0; i < CPL; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
      if (!(k < K && ((have >> k) & 1ull))) continue;
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        acc[i][0] += wk[k] * bf16_lo(v[k][i].x);
        acc[i][1] += wk[k] * bf16_hi(v[k][i].x);
        acc[i][2] += wk[k] * bf16_lo(v[k][i].y);
        acc[i][3] += wk[k] * bf16_hi(v[k][i].y);
        acc[i][4] += wk[k] * bf16_lo(v[k][i].z);
        acc[i][5] += wk[k] * bf16_hi(v[k][i].z);
        acc[i][6] += wk[k] * bf16_lo(v[k][i].w);
        acc[i][7] += wk[k] * bf16_hi(v[k][i].w);
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

}  // namespace moe
