// Backward launcher: delta pre-pass, then the dK/dV and dQ passes, for every
// compiled head-dim pair. DS = number of waves that split one 32-row block by
// head-dim range (1 for Dqk <= 128, 2 up to 256, 4 for 512).
#include "attn_launch.hpp"

namespace vca {
namespace {

// DS: waves splitting one 32-row block by head-dim range; NB/PF: LDS buffers
// and register prefetch of the dK/dV pass (KN, KP) and the dQ pass (QN, QP);
// BN keys per dQ tile; WPE waves per SIMD the dQ register budget targets.
template <int DQK, int DV, int DS, int KN, bool KP, int BN, int QN, bool QP, int WPE>
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
      hipLaunchKernelGGL((attn_bwd_dkdv_kernel<DQK, DV, DS, KN, KP, true>), g, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((attn_bwd_dkdv_kernel<DQK, DV, DS, KN, KP, false>), g, dim3(256), 0, st, a);
  }
  if (max_q > 0) {
    const dim3 g((max_q + blk - 1) / blk, Hq, nseg);
    if (causal)
      hipLaunchKernelGGL((attn_bwd_dq_kernel<DQK, DV, DS, BN, QN, QP, WPE, true>), g, dim3(256), 0,
                         st, a);
    else
      hipLaunchKernelGGL((attn_bwd_dq_kernel<DQK, DV, DS, BN, QN, QP, WPE, false>), g, dim3(256), 0,
                         st, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, int dqk, int dv, bool causal, int nseg, int Hq, int Hkv,
                      int max_q, int max_k, hipStream_t st) {
  if (nseg == 0 || Hq == 0) return hipSuccess;
#define VCA_BWD(DQK, DV, DS, KN, KP, BN, QN, QP, WPE) \
  bwd_dims<DQK, DV, DS, KN, KP, BN, QN, QP, WPE>(a, causal, nseg, Hq, Hkv, max_q, max_k, st)
  if (dqk == 64 && dv == 64) return VCA_BWD(64, 64, 1, 2, true, 32, 2, true, 2);
  if (dqk == 128 && dv == 128) return VCA_BWD(128, 128, 1, 2, true, 32, 2, true, 2);
  if (dqk == 192 && dv == 128) return VCA_BWD(192, 128, 2, 2, true, 32, 2, true, 1);
  if (dqk == 256 && dv == 256) return VCA_BWD(256, 256, 2, 2, true, 32, 2, true, 1);
  if (dqk == 512 && dv == 512) return VCA_BWD(512, 512, 4, 1, false, 32, 1, false, 1);
#undef VCA_BWD
  return hipErrorInvalidValue;
}

}  // namespace vca
