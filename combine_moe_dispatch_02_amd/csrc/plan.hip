// A1 -- placement plan: histogram of local (token, k) pairs, padded exclusive
// scan into expert offsets, stable rank of every pair inside its expert.
//
// StreamEP README, "How it works" (pool-layout dispatch): pairs land in an
// expert-major, tile-padded pool. Reading taken here: inside a segment pairs
// keep the order of q = t*K + k, a segment is ceil(count/tile)*tile rows, and
// ids outside [expert_begin, expert_begin + E_local) are not local.
//
// Scheme (no global atomics on counts, so every result is deterministic):
//   column c = one wave's run of ppw consecutive pairs (1024; 256 when one block
//           covers the batch, so that its four waves share it).
//   pass 1  each wave counts its column per expert: per 64 pairs, lanes with the
//           same expert are matched with one ballot per key bit, the lowest lane
//           of each group adds the group size to the wave's LDS counter row.
//           Counts go to hist[c][e]. The last block to finish (a device-scope
//           counter) reduces hist over columns into counts, scans the padded
//           counts into offsets (DPP wave scan), turns hist into per-column
//           bases, and writes tile_expert, num_tiles and the padding rows of src.
//   pass 2  each wave re-ranks its column the same way; a pair's row is
//           base[c][e] + (pairs of e earlier in the column), with the in-wave
//           part from mbcnt over the group mask. Writes pos and src.
// With a single block both passes run in one launch.
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kMaxExperts = 1024;

struct PlanArgs {
  const int32_t* topk_idx;
  int32_t pairs;          // T*K
  int32_t expert_begin;
  int32_t E;
  int32_t tile;
  int32_t tile_shift;     // log2(tile)
  int32_t key_bits;       // bits to tell local experts apart
  int32_t rows_cap;
  int32_t ntiles_cap;     // entries of tile_expert / tile_ready (rows_cap / tile)
  int32_t nfill;          // entries of the workspace's fill counters
  int32_t ncols;
  int32_t ppw;            // pairs per column
  int32_t* counts;
  int32_t* offsets;
  int32_t* pos;
  int32_t* src;
  int32_t* tile_expert;
  int32_t* num_tiles;
  uint32_t* tile_ready;
  uint32_t* tile_fill;
  int32_t* hist;
  uint32_t* done;
  uint32_t* tiles_done;   // dispatch's count of raised ready flags
};

// One wave's walk over its column. COUNT_ONLY: accumulate counts in run[];
// otherwise run[] holds the column's bases and rows are written.
template <bool COUNT_ONLY>
__device__ inline void rank_column(const PlanArgs& a, int col, int* run) {
  const int lane = lane_id();
  const int begin = col * a.ppw;
  const int end = min(begin + a.ppw, a.pairs);
  // the column's ids are loaded up front: one memory round trip instead of one per
  // 64 pairs (the walk below is serial through run[])
  constexpr int kIters = kPairsPerWave / kWave;
  int ids[kIters];
#pragma unroll
  for (int i = 0; i < kIters; ++i) {
    const int q = begin + i * kWave + lane;
    ids[i] = q < end ? a.topk_idx[q] : -1;
  }
#pragma unroll
  for (int i = 0; i < kIters; ++i) {
    const int base = begin + i * kWave;
    if (base >= end) break;
    const int q = base + lane;
    const bool in = q < end;
    const int id = ids[i];
    const int e = id - a.expert_begin;
    const bool local = in && id >= a.expert_begin && e < a.E;
    const uint64_t peers = match_key(local ? (uint32_t)e : 0u, local, a.key_bits);
    const int rank = mask_rank(peers);
    const int cnt = __popcll(peers);
    if (COUNT_ONLY) {
      if (local && rank == 0) run[e] += cnt;
    } else {
      int row = -1;
      if (local) {
        const int b = run[e];
        row = b + rank;
        if (rank == 0) run[e] = b + cnt;
      }
      if (in) a.pos[q] = row;
      if (local) a.src[row] = q;
    }
  }
}

// Block-wide exclusive scan of up to 4 ints per thread (256 threads); returns the
// total. scratch: 4 ints of LDS.
__device__ inline int block_exclusive_scan4(int v[4], int* scratch) {
  const int lane = lane_id();
  const int w = threadIdx.x >> 6;
  const int s = v[0] + v[1] + v[2] + v[3];
  const int incl = wave_inclusive_scan(s);
  if (lane == 63) scratch[w] = incl;
  __syncthreads();
  int wave_base = 0, total = 0;
  for (int i = 0; i < 4; ++i) {
    const int t = scratch[i];
    if (i < w) wave_base += t;
    total += t;
  }
  int run = wave_base + incl - s;
  for (int i = 0; i < 4; ++i) {
    const int x = v[i];
    v[i] = run;
    run += x;
  }
  __syncthreads();
  return total;
}

// The scan step, run by the last block of pass 1 (all 256 threads).
__device__ void plan_scan(const PlanArgs& a, int* s_cnt, int* s_off, int* s_half, int* scratch) {
  const int tid = threadIdx.x;
  const int E = a.E;
  // counts: reduce the columns. With E <= 128 two threads share an expert, each
  // summing half of the columns (s_half keeps the first half's sum for the bases
  // below); the loops are unrolled so that 16 column loads are in flight at a time
  // (one load per iteration would serialise their latency).
  const bool split = E <= 128;
  const int half = (a.ncols + 1) >> 1;
  for (int x = tid; x < (split ? 2 * E : E); x += 256) {
    const int e = split ? x >> 1 : x;
    const int c0 = split && (x & 1) ? half : 0;
    const int c1 = split && !(x & 1) ? half : a.ncols;
    int c = 0;
#pragma unroll 16
    for (int col = c0; col < c1; ++col) c += a.hist[col * E + e];
    if (split) {
      const int other = __shfl_xor(c, 1);
      if (!(x & 1)) s_half[e] = c;
      c += other;
    }
    if (!split || !(x & 1)) {
      s_cnt[e] = c;
      a.counts[e] = c;
    }
  }
  __syncthreads();
  // offsets: exclusive scan of the padded counts, 4 consecutive experts per thread
  int v[4];
  for (int i = 0; i < 4; ++i) {
    const int e = tid * 4 + i;
    v[i] = e < E ? ((s_cnt[e] + a.tile - 1) >> a.tile_shift) << a.tile_shift : 0;
  }
  const int P = block_exclusive_scan4(v, scratch);
  for (int i = 0; i < 4; ++i) {
    const int e = tid * 4 + i;
    if (e < E) {
      s_off[e] = v[i];
      a.offsets[e] = v[i];
    }
  }
  if (tid == 0) {
    s_off[E] = P;
    a.offsets[E] = P;
    a.num_tiles[0] = P >> a.tile_shift;
  }
  __syncthreads();
  const int ntiles = P >> a.tile_shift;
  // per-column bases, tile owners, padding rows
  for (int x = tid; x < (split ? 2 * E : E); x += 256) {
    const int e = split ? x >> 1 : x;
    const bool second = split && (x & 1);
    const int c0 = second ? half : 0;
    const int c1 = split && !second ? half : a.ncols;
    int run = s_off[e] + (second ? s_half[e] : 0);
#pragma unroll 16
    for (int col = c0; col < c1; ++col) {
      const int c = a.hist[col * E + e];
      a.hist[col * E + e] = run;
      run += c;
    }
    if (second) continue;
    const int seg_end = s_off[e + 1];
    for (int t = s_off[e] >> a.tile_shift; t < (seg_end >> a.tile_shift); ++t) a.tile_expert[t] = e;
    for (int r = s_off[e] + s_cnt[e]; r < seg_end; ++r) a.src[r] = -1;
  }
  for (int t = ntiles + tid; t < a.ntiles_cap; t += 256) a.tile_expert[t] = -1;
  for (int r = P + tid; r < a.rows_cap; r += 256) a.src[r] = -1;
  // a fresh start for the dispatch that follows
  for (int t = tid; t < a.ntiles_cap; t += 256) a.tile_ready[t] = 0u;
  for (int t = tid; t < a.nfill; t += 256) a.tile_fill[t] = 0u;
  if (tid == 0) *a.tiles_done = 0u;
}

__global__ __launch_bounds__(256) void plan_count_kernel(PlanArgs a) {
  __shared__ int s_run[kPlanWaves][kMaxExperts];
  __shared__ int s_off[kMaxExperts + 1];
  __shared__ int scratch[4];
  __shared__ int s_last;
  const int w = threadIdx.x >> 6;
  const int lane = lane_id();
  const int col = blockIdx.x * kPlanWaves + w;
  int* run = s_run[w];
  for (int e = lane; e < a.E; e += kWave) run[e] = 0;
  if (col < a.ncols) {
    rank_column<true>(a, col, run);
    for (int e = lane; e < a.E; e += kWave) a.hist[col * a.E + e] = run[e];
  }
  __syncthreads();
  if (gridDim.x > 1) {
    // the last block to finish scans; a single block needs no device-scope handshake
    if (threadIdx.x == 0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      const uint32_t prev = __hip_atomic_fetch_add(a.done, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      s_last = prev == gridDim.x - 1;
    }
    __syncthreads();
    if (!s_last) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  // s_run doubles as the counts array of the scan (the waves' rows are done)
  int* s_cnt = &s_run[0][0];
  int* s_half = &s_run[1][0];
  __syncthreads();
  plan_scan(a, s_cnt, s_off, s_half, scratch);
  if (threadIdx.x == 0) __hip_atomic_store(a.done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (gridDim.x != 1) return;
  // single block: place the pairs right away
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
  for (int e = lane; e < a.E; e += kWave) run[e] = col < a.ncols ? a.hist[col * a.E + e] : 0;
  if (col < a.ncols) rank_column<false>(a, col, run);
}

__global__ __launch_bounds__(256) void plan_place_kernel(PlanArgs a) {
  __shared__ int s_run[kPlanWaves][kMaxExperts];
  const int w = threadIdx.x >> 6;
  const int lane = lane_id();
  const int col = blockIdx.x * kPlanWaves + w;
  if (col >= a.ncols) return;
  int* run = s_run[w];
  for (int e = lane; e < a.E; e += kWave) run[e] = a.hist[col * a.E + e];
  rank_column<false>(a, col, run);
}

int launch_plan(const int32_t* topk_idx, const moe_plan_t& p, const WsLayout& L, char* ws,
                hipStream_t stream) {
  PlanArgs a;
  a.topk_idx = topk_idx;
  a.pairs = p.T * p.K;
  a.expert_begin = p.expert_begin;
  a.E = p.E_local;
  a.tile = p.tile;
  a.tile_shift = __builtin_ctz((unsigned)p.tile);
  int bits = 0;
  while ((1 << bits) < p.E_local) ++bits;
  a.key_bits = bits;
  a.rows_cap = p.rows_cap;
  a.ntiles_cap = p.rows_cap / p.tile;
  a.nfill = 2 * L.ntiles_cap;   // dispatch's and combine backward's counters (adjacent)
  a.ncols = L.ncols;
  a.ppw = L.ppw;
  a.counts = p.counts;
  a.offsets = p.offsets;
  a.pos = p.pos;
  a.src = p.src;
  a.tile_expert = p.tile_expert;
  a.num_tiles = p.num_tiles;
  a.tile_ready = p.tile_ready;
  a.tile_fill = reinterpret_cast<uint32_t*>(ws + L.fill);
  a.hist = reinterpret_cast<int32_t*>(ws + L.hist);
  a.done = reinterpret_cast<uint32_t*>(ws + L.done);
  a.tiles_done = reinterpret_cast<uint32_t*>(ws + L.tiles_done);
  const int blocks = (L.ncols + kPlanWaves - 1) / kPlanWaves;
  hipLaunchKernelGGL(plan_count_kernel, dim3(blocks), dim3(256), 0, stream, a);
  if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
  if (blocks > 1) {
    hipLaunchKernelGGL(plan_place_kernel, dim3(blocks), dim3(256), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
  }
  return MOE_OK;
}

// ----------------------------------------------------------------------------
// moe_plan_noalloc: moe_plan with its scratch (the per-column histogram and the blocks'
// completion counter) in a file-scope device array instead of a caller's workspace.
// Every call on a device shares that device's array.
// ----------------------------------------------------------------------------
constexpr size_t kPlanScratchBytes = (size_t)4 << 20;
static __device__ __align__(256) uint8_t scratch[kPlanScratchBytes];

// the array's device address, looked up once per device with that device current
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[1024];

static void* plan_scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 1024) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

// the completion counter starts at zero (a kernel, not a memset, so the call can be captured
// in a graph)
__global__ void zero_word_kernel(uint32_t* w) { *w = 0u; }

}  // namespace moe

extern "C" MOE355_API int moe_plan_noalloc(const int32_t* topk_idx, const moe_plan_t* plan, void* stream) {
  using namespace moe;
  int rc = check_plan(plan);
  if (rc != MOE_OK) return rc;
  if (!topk_idx) return MOE_ERR_INVALID;
  WsLayout L = ws_layout(plan->T, plan->K, plan->E_local, plan->tile, 0, 0, MOE_BF16);
  if (L.hist + (size_t)L.ncols * plan->E_local * 4 > kPlanScratchBytes) return MOE_ERR_UNSUPPORTED;
  char* base = static_cast<char*>(plan_scratch_ptr());
  if (base == nullptr) return MOE_ERR_HIP;
  // no layer workspace: nothing is prepared for moe_dispatch (no fill counters to clear)
  L.ntiles_cap = 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(zero_word_kernel, dim3(1), dim3(1), 0, s, reinterpret_cast<uint32_t*>(base + L.done));
  if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
  return launch_plan(topk_idx, *plan, L, base, s);
}
