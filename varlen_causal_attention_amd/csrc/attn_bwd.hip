// Backward launcher: delta pre-pass, then the dK/dV and dQ passes, for every
// compiled head-dim pair. DS = number of waves that split one 32-row block by
// head-dim range (1 for Dqk <= 128, 2 up to 256, 4 for 512).
#include "attn_launch.hpp"

namespace vca {
namespace {

template <int DQK, int DV, int DS>
hipError_t bwd_dims(const BwdArgs& a, bool causal, int nseg, int Hq, int Hkv, int max_q,
                    int max_k, hipStream_t st) {
  constexpr int LPR = DV / 8 >= 64 ? 64 : DV / 8;
  constexpr int rows_per_block = 4 * (64 / LPR);
  if (max_q > 0) {
    const dim3 g((max_q + rows_per_block - 1) / rows_per_block, Hq, nseg);
    hipLaunchKernelGGL((attn_bwd_delta_kernel<DV>), g, dim3(256), 0, st, a);
  }
  constexpr int blk = 32 * (4 / DS);
  if (max_k > 0) {
    const dim3 g((max_k + blk - 1) / blk, Hkv, nseg);
    if (causal)
      hipLaunchKernelGGL((attn_bwd_dkdv_kernel<DQK, DV, DS, true>), g, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((attn_bwd_dkdv_kernel<DQK, DV, DS, false>), g, dim3(256), 0, st, a);
  }
  if (max_q > 0) {
    const dim3 g((max_q + blk - 1) / blk, Hq, nseg);
    if (causal)
      hipLaunchKernelGGL((attn_bwd_dq_kernel<DQK, DV, DS, true>), g, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((attn_bwd_dq_kernel<DQK, DV, DS, false>), g, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, int dqk, int dv, bool causal, int nseg, int Hq, int Hkv,
                      int max_q, int max_k, hipStream_t st) {
  if (nseg == 0 || Hq == 0) return hipSuccess;
  if (dqk == 64 && dv == 64) return bwd_dims<64, 64, 1>(a, causal, nseg, Hq, Hkv, max_q, max_k, st);
  if (dqk == 128 && dv == 128) return bwd_dims<128, 128, 1>(a, causal, nseg, Hq, Hkv, max_q, max_k, st);
  if (dqk == 192 && dv == 128) return bwd_dims<192, 128, 2>(a, causal, nseg, Hq, Hkv, max_q, max_k, st);
  if (dqk == 256 && dv == 256) return bwd_dims<256, 256, 2>(a, causal, nseg, Hq, Hkv, max_q, max_k, st);
  if (dqk == 512 && dv == 512) return bwd_dims<512, 512, 4>(a, causal, nseg, Hq, Hkv, max_q, max_k, st);
  return hipErrorInvalidValue;
}

}  // namespace vca
