// Host-side launchers of the attention kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>

#include "attn_bwd.hpp"
#include "attn_fwd.hpp"

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

// Grid: (q tiles of the longest segment, Hq, segments-or-batches).
hipError_t launch_fwd(const FwdArgs& a, int dqk, int dv, bool causal, int nseg, int Hq,
                      int max_q, hipStream_t stream);

// delta pre-pass, dK/dV pass, dQ pass, in that order on one stream.
hipError_t launch_bwd(const BwdArgs& a, int dqk, int dv, bool causal, int nseg, int Hq, int Hkv,
                      int max_q, int max_k, hipStream_t stream);

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream);

}  // namespace vca
