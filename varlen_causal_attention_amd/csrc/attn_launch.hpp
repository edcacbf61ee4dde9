// Host-side launchers of the attention kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>

#include "attn_bwd.hpp"
#include "attn_fwd.hpp"
#include "attn_sched.hpp"

namespace vca {

// ---------------------------------------------------------------------------
// merge of two partial results ("gemma4_moe cp_attention" page, -inf-safe
// merge): one wave per (row, head); lanes cover the head dim.
// ---------------------------------------------------------------------------
struct MergeArgs {
  const void* out_a;
  const void* out_b;
  int a_f32, b_f32;
  const float* lse_a;
  const float* lse_b;
  float* out;
  float* lse;
  uint16_t* out_bf16;
  int rows, H, Dv;
};


// Head-dim pairs compiled into the library.
bool head_dims_supported(int dqk, int dv);

// Work lists: every pass orders its (segment, tile) items heaviest first.
// The list capacity is bounded with 32-row tiles, the smallest any pass uses.
constexpr int kListRows = 32;
inline size_t list_capacity(int64_t rows, int nseg) { return (size_t)((rows + kListRows - 1) / kListRows) + nseg; }
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
// forward workspace: [count][list]
inline size_t fwd_workspace_bytes(int64_t q_rows, int nseg) {
  return 256 + align256(sizeof(int2) * list_capacity(q_rows, nseg));
}
// backward workspace: [delta fp32, one per (q-head, query row)][counts][query list][key list]
inline size_t bwd_workspace_bytes(int64_t delta_elems, int64_t q_rows, int64_t k_rows, int nseg) {
  return align256(sizeof(float) * delta_elems) + 256 +
         align256(sizeof(int2) * list_capacity(q_rows, nseg)) +
         align256(sizeof(int2) * list_capacity(k_rows, nseg));
}

// Scheduler launch + forward kernel. ws: the forward workspace. q_rows: Tq
// (varlen) or B * Nq (dense), used for the list capacity.
hipError_t launch_fwd(FwdArgs a, int dqk, int dv, bool causal, int nseg, int Hq, int64_t q_rows,
                      void* ws, hipStream_t stream);

// delta pre-pass, dK/dV pass, dQ pass, in that order on one stream.
// ws: the backward workspace (delta first).
hipError_t launch_bwd(BwdArgs a, int dqk, int dv, bool causal, int nseg, int Hq, int Hkv,
                      int max_q, int64_t q_rows, int64_t k_rows, void* ws, hipStream_t stream);

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream);

}  // namespace vca
