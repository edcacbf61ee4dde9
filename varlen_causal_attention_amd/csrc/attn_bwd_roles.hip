// Launchers of the dK/dV passes with split wave roles (head dim 128, and
// Dqk = 192 with Dv = 128).
#include "attn_bwd_roles.hpp"
#include "attn_bwd_roles192.hpp"
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

hipError_t launch_dkdv_roles192(const BwdArgs& a, bool causal, unsigned grid, hipStream_t st) {
  if (causal)
    hipLaunchKernelGGL((attn_bwd_dkdv_roles_qk192_kernel<true>), dim3(grid), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((attn_bwd_dkdv_roles_qk192_kernel<false>), dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace VCA_ELEM
}  // namespace vca
