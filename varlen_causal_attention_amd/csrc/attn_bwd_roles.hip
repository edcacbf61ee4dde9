// Launcher of the head-dim-128 dK/dV pass with split wave roles.
#include "attn_bwd_roles.hpp"
#include "attn_launch.hpp"

namespace vca {
namespace VCA_ELEM {

// 32-key tiles per wave: 1 -> eight waves (two per SIMD), 2 -> four
constexpr int kRolesKT = 2;

hipError_t launch_dkdv_roles(const BwdArgs& a, bool causal, unsigned grid, hipStream_t st) {
  constexpr int NT = 512 / kRolesKT;
  if (causal)
    hipLaunchKernelGGL((attn_bwd_dkdv_roles_kernel<true, kRolesKT>), dim3(grid), dim3(NT), 0, st, a);
  else
    hipLaunchKernelGGL((attn_bwd_dkdv_roles_kernel<false, kRolesKT>), dim3(grid), dim3(NT), 0, st, a);
  return hipGetLastError();
}

}  // namespace VCA_ELEM
}  // namespace vca
