// Work units of the 256-row GEMM kernel (ffn_sq.hip): a unit is two consecutive pool tiles
// of one expert (or its last, odd tile) and one N block of 256 columns: the unit walk, the
// per-expert prefix of row units and the ready-flag wait. Internal; not part of the C ABI.
#pragma once

#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kMaxExpertsSq = 1024;

struct SqUnit {
  int e;     // local expert
  int m;     // first pool tile
  int two;   // 1: tiles m and m + 1; 0: tile m only
  int j;     // N block of 256 columns
};

// Unit u -> coordinates (sq_unit_lane: u may differ between lanes). s_ru[e] = row units (tile pairs, rounded up) of the experts
// before e. Within expert e, units go in groups of `group` row units; inside a group,
// N block by N block, the group's row units back to back: units that run together
// share weight panels and pool rows.
// Each expert's first pool tile comes from a table (t0s[e] = min(offsets[e] / 128,
// max_tiles) for e <= E, in LDS), so that decoding a unit reads no global memory.
__device__ __attribute__((always_inline)) inline SqUnit sq_unit_lane(const SqArgs& a, const int32_t* s_ru,
                                                                         const int32_t* t0s, int u) {
  int lo = 0, hi = a.n_experts - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_ru[mid] * a.NB <= u) lo = mid;
    else hi = mid - 1;
  }
  SqUnit r;
  r.e = lo;
  const int R = s_ru[lo + 1] - s_ru[lo];
  const int l = u - s_ru[lo] * a.NB;
  const int g = l / (a.group * a.NB);
  const int gsz = min(a.group, R - g * a.group);
  const int l2 = l - g * a.group * a.NB;
  r.j = l2 / gsz;
  const int ru = g * a.group + (l2 - r.j * gsz);
  r.m = t0s[lo] + 2 * ru;
  r.two = r.m + 1 < t0s[lo + 1];
  return r;
}

// The same, for a unit index that is the same in every lane (the result in scalar registers).
__device__ __attribute__((always_inline)) inline SqUnit sq_unit(const SqArgs& a, const int32_t* s_ru,
                                                                    const int32_t* t0s, int u) {
  SqUnit r = sq_unit_lane(a, s_ru, t0s, u);
  r.e = __builtin_amdgcn_readfirstlane(r.e);
  r.m = __builtin_amdgcn_readfirstlane(r.m);
  r.two = __builtin_amdgcn_readfirstlane(r.two);
  r.j = __builtin_amdgcn_readfirstlane(r.j);
  return r;
}

// s_ru[e] for e <= E (row units of the experts before e; s_ru[E] = all of them): lane i
// of wave 0 sums a run of experts, then a wave scan. The caller syncs the workgroup.
__device__ __attribute__((always_inline)) inline void sq_row_units(const SqArgs& a, int32_t* s_ru, int lane) {
  const int E = a.n_experts;
  const int per = (E + 63) >> 6;
  int sum = 0;
  for (int i = 0; i < per; ++i) {
    const int e = lane * per + i;
    if (e < E) {
      const int t0 = min(a.offsets[e] >> 7, a.max_tiles), t1 = min(a.offsets[e + 1] >> 7, a.max_tiles);
      sum += (t1 - t0 + 1) >> 1;
    }
  }
  const int incl = wave_inclusive_scan(sum);
  int run = incl - sum;
  for (int i = 0; i < per; ++i) {
    const int e = lane * per + i;
    if (e < E) {
      s_ru[e] = run;
      const int t0 = min(a.offsets[e] >> 7, a.max_tiles), t1 = min(a.offsets[e + 1] >> 7, a.max_tiles);
      run += (t1 - t0 + 1) >> 1;
    }
  }
  if (lane == 63) s_ru[E] = incl;
}

// Which unit shape runs GEMM A when both kernels are launched for it (the 256-row one
// first, the 128-row one after it, each returning at once unless chosen). It is decided on
// the device from the plan, with the same answer in every workgroup of both launches: the
// 256-row units, unless the experts hold two tiles or more on average (with fewer the FFN
// streams weights, and a 256-row unit reads an expert's weight panel once per tile pair
// rather than once per tile) and 0.85 of their rounds over the grid exceeds the 128-row
// units' rounds (0.85: about what a 256-row unit costs against a 128-row unit of the same
// flops, measured at the skew and ep_share workloads). One wave evaluates it.
__device__ __attribute__((always_inline)) inline bool sq_gemm_a_wins(const int32_t* offsets, int E, int max_tiles,
                                                                     const SqSelect& s, int lane) {
  int pairs = 0, tiles = 0, nonempty = 0;
  for (int e = lane; e < E; e += 64) {
    const int t0 = min(offsets[e] >> 7, max_tiles), t1 = min(offsets[e + 1] >> 7, max_tiles);
    const int n = t1 - t0;
    pairs += (n + 1) >> 1;
    tiles += n;
    nonempty += n > 0 ? 1 : 0;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    pairs += __shfl_xor(pairs, o);
    tiles += __shfl_xor(tiles, o);
    nonempty += __shfl_xor(nonempty, o);
  }
  if (tiles < 2 * nonempty) return true;
  const int64_t r_sq = ((int64_t)pairs * s.nb_sq + s.grid_sq - 1) / s.grid_sq;
  const int64_t r_big = ((int64_t)tiles * s.nb_big + s.grid_big - 1) / s.grid_big;
  return 17 * r_sq <= 20 * r_big;
}

// Wait until the unit's tiles carry this call's epoch (see the file comment).
__device__ __attribute__((always_inline)) inline void sq_wait_tiles(const SqArgs& a, const SqUnit& U) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (;;) {
    const bool r0 = __hip_atomic_load(&a.tile_ready[U.m], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == a.epoch;
    const bool r1 = !U.two ||
                    __hip_atomic_load(&a.tile_ready[U.m + 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == a.epoch;
    if (r0 && r1) break;
    if (__hip_atomic_load(a.abort_epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == a.epoch) break;
    if (__builtin_amdgcn_s_memrealtime() - t0 > a.timeout) {
      record_error(a.err, MOE_ERR_TIMEOUT);
      __hip_atomic_store(a.abort_epoch, a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    __builtin_amdgcn_s_sleep(4);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

}  // namespace moe
