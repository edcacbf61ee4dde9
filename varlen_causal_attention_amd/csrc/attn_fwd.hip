// Forward launcher: instantiates the forward kernel for every compiled
// head-dim pair and both mask modes.
#include "attn_launch.hpp"

namespace vca {

bool head_dims_supported(int dqk, int dv) {
  return (dqk == 64 && dv == 64) || (dqk == 128 && dv == 128) || (dqk == 192 && dv == 128) ||
         (dqk == 256 && dv == 256) || (dqk == 512 && dv == 512);
}

namespace {
// BN = keys per tile, DS = waves sharing one 32-row query block, NBUF = LDS
// buffers for the K/V tiles, WPE = waves per SIMD the register budget targets.
template <int DQK, int DV, int BN, int DS, int NBUF, int WPE, bool PF>
hipError_t fwd_dims(const FwdArgs& a, bool causal, dim3 grid, hipStream_t st) {
  if (causal)
    hipLaunchKernelGGL((attn_fwd_kernel<DQK, DV, BN, DS, NBUF, WPE, PF, true>), grid, dim3(256 * DS),
                       0, st, a);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<DQK, DV, BN, DS, NBUF, WPE, PF, false>), grid,
                       dim3(256 * DS), 0, st, a);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_fwd(const FwdArgs& a, int dqk, int dv, bool causal, int nseg, int Hq,
                      int max_q, hipStream_t st) {
  const int tiles = (max_q + kFwdBM - 1) / kFwdBM;
  if (tiles == 0 || nseg == 0 || Hq == 0) return hipSuccess;
  const dim3 grid(tiles, Hq, nseg);
  if (dqk == 64 && dv == 64) return fwd_dims<64, 64, 64, 1, 2, 2, true>(a, causal, grid, st);
  if (dqk == 128 && dv == 128) return fwd_dims<128, 128, 64, 1, 2, 2, true>(a, causal, grid, st);
  if (dqk == 192 && dv == 128) return fwd_dims<192, 128, 64, 1, 2, 2, true>(a, causal, grid, st);
  if (dqk == 256 && dv == 256) return fwd_dims<256, 256, 64, 1, 2, 1, true>(a, causal, grid, st);
  if (dqk == 512 && dv == 512) return fwd_dims<512, 512, 32, 2, 1, 1, false>(a, causal, grid, st);
  return hipErrorInvalidValue;
}

}  // namespace vca
