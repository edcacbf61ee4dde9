// Launcher of the head-dim-128 dK/dV pass with split wave roles.
#include "attn_bwd_roles.hpp"
#include "attn_launch.hpp"

namespace vca {

hipError_t launch_dkdv_roles(const BwdArgs& a, bool causal, unsigned grid, hipStream_t st) {
  if (causal)
    hipLaunchKernelGGL(attn_bwd_dkdv_roles_kernel<true>, dim3(grid), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(attn_bwd_dkdv_roles_kernel<false>, dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace vca
