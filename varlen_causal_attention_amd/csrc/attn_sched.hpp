// Work decomposition: turns the segment table into a list of (segment, tile)
// work items ordered heaviest first, so the long causal tiles of every
// segment start early and the short ones fill the tail.
//
// Causal tiles differ widely in cost: the last query tile of a long document
// walks all of its keys, the first one a single key tile (and the other way
// round for key blocks in the dK/dV pass). Dispatching in grid order leaves
// the heavy tiles of late segments for the end; longest-processing-time-first
// ordering bounds the makespan by the average load plus one tile.
#pragma once

#include "attn_common.hpp"

namespace vca {
namespace VCA_ELEM {

constexpr int kSchedBuckets = 2048;  // cost classes (costs clamp into the last one)

struct SchedArgs {
  const int32_t* cu_q;  // NULL: dense, every segment has Nq queries and Nk keys
  const int32_t* cu_k;
  int nseg, Nq, Nk, Tq, Tk;
  int by_keys;   // 0: tiles of `tile` query rows; 1: blocks of `tile` keys
  int tile;      // rows per work item
  int step;      // rows per inner step: keys per tile (by_keys = 0) or queries (1)
  int causal;
  int2* list;    // out: (segment, tile) in heavy-first order
  int* count;    // out: number of items
  int max_items; // capacity of list (a malformed table may ask for more)
  int seg_major; // 1: segments in table order, each one's items heaviest first
};

__device__ __forceinline__ int sched_cost(const SchedArgs& a, const SegGeom& g, int t) {
  const int shift = g.lk - g.lq;
  if (!a.by_keys) {
    int kv_end = g.lk;
    if (a.causal) kv_end = min(g.lk, (t + 1) * a.tile + shift);
    return kv_end > 0 ? (kv_end + a.step - 1) / a.step : 0;
  }
  int q_begin = 0;
  if (a.causal) q_begin = max(0, t * a.tile - shift);
  return g.lq > q_begin ? (g.lq - q_begin + a.step - 1) / a.step : 0;
}

// One workgroup of 16 waves: histogram of item costs, descending exclusive
// scan, scatter. Wave w takes segments w, w+16, ...; its lanes split the
// segment's tiles. Items of equal cost land in an arbitrary order; every item
// writes only its own outputs, so the order never changes a result.
__device__ __forceinline__ void schedule_list(const SchedArgs& a) {
  constexpr int NT = 1024, PER = kSchedBuckets / NT;  // buckets per thread
  __shared__ int hist[kSchedBuckets];
  __shared__ int wave_sum[NT / 64];
  __shared__ int total;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int i = tid; i < kSchedBuckets; i += NT) hist[i] = 0;
  if (tid == 0) total = 0;
  __syncthreads();
  int mine = 0;
  for (int s = w; s < a.nseg; s += NT / 64) {
    const SegGeom g = seg_geom(a.cu_q, a.cu_k, s, a.Nq, a.Nk, a.Tq, a.Tk);
    const int len = a.by_keys ? g.lk : g.lq;
    const int nt = (len + a.tile - 1) / a.tile;
    for (int t = lane; t < nt; t += 64) {
      atomicAdd(&hist[min(sched_cost(a, g, t), kSchedBuckets - 1)], 1);
      ++mine;
    }
  }
  atomicAdd(&total, mine);
  __syncthreads();
  // descending exclusive scan: bucket c starts after all buckets > c.
  // Thread i owns buckets kSchedBuckets-1-(i*PER .. i*PER+PER-1).
  int vals[PER], run = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    vals[j] = hist[kSchedBuckets - 1 - (tid * PER + j)];
    run += vals[j];
  }
  int incl = run;  // inclusive scan of per-thread sums within the wave
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int n = __shfl_up(incl, off, 64);
    if (lane >= off) incl += n;
  }
  if (lane == 63) wave_sum[w] = incl;
  __syncthreads();
  int base = incl - run;
  for (int i = 0; i < w; ++i) base += wave_sum[i];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    hist[kSchedBuckets - 1 - (tid * PER + j)] = base;
    base += vals[j];
  }
  if (tid == 0) *a.count = min(total, a.max_items);
  __syncthreads();
  for (int s = w; s < a.nseg; s += NT / 64) {
    const SegGeom g = seg_geom(a.cu_q, a.cu_k, s, a.Nq, a.Nk, a.Tq, a.Tk);
    const int len = a.by_keys ? g.lk : g.lq;
    const int nt = (len + a.tile - 1) / a.tile;
    for (int t = lane; t < nt; t += 64) {
      const int pos = atomicAdd(&hist[min(sched_cost(a, g, t), kSchedBuckets - 1)], 1);
      if (pos < a.max_items) a.list[pos] = make_int2(s, t);
    }
  }
}

// Segment-major order: the items of segment 0, heaviest first (query tiles:
// the last one; key blocks: the first one), then those of segment 1, ...
// The tiles of one segment and head then start close together and walk the
// same K/V tiles in step, so a tile read from HBM by one workgroup is still
// in L2 for the others; under a global heavy-first order they start far
// apart in time and, without a GQA group sharing the stream, miss L2. A
// segment's last tile walks all of its keys and is emitted first, so each
// segment's long tiles still start first.
// Segments are taken 1024 at a time: a block-wide scan of their item counts
// gives each one's first list position, then wave w writes segments w,
// w+16, ... of the chunk with its lanes splitting a segment's items.
__device__ __forceinline__ void schedule_seg_major(const SchedArgs& a) {
  constexpr int NT = 1024;
  __shared__ int wave_sum[NT / 64];
  __shared__ int seg_pos[NT], seg_n[NT];
  __shared__ int carry;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < a.nseg; base += NT) {
    const int s = base + tid;
    int n = 0;
    if (s < a.nseg) {
      const SegGeom g = seg_geom(a.cu_q, a.cu_k, s, a.Nq, a.Nk, a.Tq, a.Tk);
      n = ((a.by_keys ? g.lk : g.lq) + a.tile - 1) / a.tile;
    }
    int incl = n;  // inclusive scan over the block
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(incl, off, 64);
      if (lane >= off) incl += v;
    }
    if (lane == 63) wave_sum[w] = incl;
    __syncthreads();
    int pos = carry + incl - n;
    for (int i = 0; i < w; ++i) pos += wave_sum[i];
    seg_pos[tid] = pos;
    seg_n[tid] = n;
    __syncthreads();  // positions published; every thread has read carry
    if (tid == NT - 1) carry = pos + n;
    const int len = min(NT, a.nseg - base);
    for (int k = w; k < len; k += NT / 64) {
      const int p0 = seg_pos[k], nk = seg_n[k];
      for (int j = lane; j < nk; j += 64)
        if (p0 + j < a.max_items) a.list[p0 + j] = make_int2(base + k, a.by_keys ? j : nk - 1 - j);
    }
    __syncthreads();  // carry written; seg_pos / seg_n free for the next chunk
  }
  if (tid == 0) *a.count = min(carry, a.max_items);
}

[[maybe_unused]] static __global__ void __launch_bounds__(1024)
attn_schedule_kernel(const SchedArgs a) {
  if (a.seg_major) schedule_seg_major(a);
  else schedule_list(a);
}

// Two independent lists in one launch (workgroup i builds list i): the
// backward's query-tile and key-block lists.
struct SchedArgs2 {
  SchedArgs list[2];
};
[[maybe_unused]] static __global__ void __launch_bounds__(1024)
attn_schedule2_kernel(const SchedArgs2 a) {
  if (a.list[blockIdx.x].seg_major) schedule_seg_major(a.list[blockIdx.x]);
  else schedule_list(a.list[blockIdx.x]);
}

}  // namespace VCA_ELEM
}  // namespace vca
