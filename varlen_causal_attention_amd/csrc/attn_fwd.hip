// Forward launcher: instantiates the forward kernel for every compiled
// head-dim pair and both mask modes, plain and with the left window /
// softcap extension (a separate instantiation, so the plain kernels carry
// none of its registers or branches).
#include "attn_fwd.hpp"
#include "attn_fwd_wide.hpp"
#include "attn_launch.hpp"
#include "attn_sched.hpp"
#include "attn_timing.hpp"

namespace vca {
namespace VCA_ELEM {

namespace {
// BN = keys per tile, WPE = waves per SIMD the register budget targets,
// HPW = q-heads per workgroup (2: two heads of a GQA group share each K/V
// tile; the grid then has one workgroup per item and head pair).
template <int DQK, int DV, int BN, int WPE, int HPW = 1>
hipError_t fwd_dims(const FwdArgs& a, bool causal, dim3 grid, hipStream_t st) {
  TimedLaunch timer("attn_fwd", st);
  grid.x /= HPW;
  const dim3 block(256 * HPW);
  const bool ext = a.window > 0 || a.cap_in != 0.f;
  if (causal && ext)
    hipLaunchKernelGGL((attn_fwd_kernel<DQK, DV, BN, WPE, true, HPW, true>), grid, block, 0, st,
                       a);
  else if (causal)
    hipLaunchKernelGGL((attn_fwd_kernel<DQK, DV, BN, WPE, true, HPW>), grid, block, 0, st, a);
  else if (ext)
    hipLaunchKernelGGL((attn_fwd_kernel<DQK, DV, BN, WPE, false, HPW, true>), grid, block, 0, st,
                       a);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<DQK, DV, BN, WPE, false, HPW>), grid, block, 0, st, a);
  return hipGetLastError();
}
hipError_t fwd_wide(const FwdArgs& a, bool causal, dim3 grid, hipStream_t st) {
  TimedLaunch timer("attn_fwd", st);
  const bool ext = a.window > 0 || a.cap_in != 0.f;
  if (causal && ext)
    hipLaunchKernelGGL((attn_fwd_wide_kernel<true, true>), grid, dim3(256), 0, st, a);
  else if (causal)
    hipLaunchKernelGGL(attn_fwd_wide_kernel<true>, grid, dim3(256), 0, st, a);
  else if (ext)
    hipLaunchKernelGGL((attn_fwd_wide_kernel<false, true>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(attn_fwd_wide_kernel<false>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_fwd(FwdArgs a, int dqk, int dv, bool causal, int nseg, int Hq, int64_t q_rows,
                      void* ws, hipStream_t st) {
  if (nseg == 0 || Hq == 0 || q_rows == 0) return hipSuccess;
  if (!head_dims_supported(dqk, dv)) return hipErrorInvalidValue;
  char* w = static_cast<char*>(ws);
  SchedArgs sa{};
  sa.cu_q = a.cu_q;
  sa.cu_k = a.cu_k;
  sa.nseg = nseg;
  sa.Nq = a.Nq;
  sa.Nk = a.Nk;
  sa.Tq = a.Tq;
  sa.Tk = a.Tk;
  sa.by_keys = 0;
  sa.tile = kFwdBM;
  sa.step = 64;
  sa.causal = causal;
  sa.count = reinterpret_cast<int*>(w);
  sa.list = reinterpret_cast<int2*>(w + 256);
  sa.max_items = (int)list_capacity(q_rows, nseg);
  // segment-major: a segment's query tiles start together and share its K/V
  // tiles in L2 (192/128 varlen forward 2.90 -> 2.60 ms; about 2% at D=128)
  sa.seg_major = 1;
  {
    TimedLaunch timer("attn_schedule", st);
    hipLaunchKernelGGL(attn_schedule_kernel, dim3(1), dim3(1024), 0, st, sa);
  }
  a.items = sa.list;
  a.item_count = sa.count;
  a.H = Hq;
  // at most ceil(q_rows / 128) + nseg query tiles exist
  const int64_t items = (q_rows + kFwdBM - 1) / kFwdBM + nseg;
  const dim3 grid((unsigned)(items * Hq));
  if (dqk == 64 && dv == 64) return fwd_dims<64, 64, 64, 2>(a, causal, grid, st);
  if (dqk == 128 && dv == 128) {
    if (a.G % 2 == 0) return fwd_dims<128, 128, 128, 1, 2>(a, causal, grid, st);
    return fwd_dims<128, 128, 64, 2>(a, causal, grid, st);
  }
  if (dqk == 192 && dv == 128) return fwd_dims<192, 128, 64, 2>(a, causal, grid, st);
  if (dqk == 256 && dv == 256) return fwd_dims<256, 256, 64, 1>(a, causal, grid, st);
  return fwd_wide(a, causal, grid, st);
}

}  // namespace VCA_ELEM
}  // namespace vca
