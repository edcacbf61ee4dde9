// Merge launcher and kernel.
#include "attn_launch.hpp"
#include "attn_timing.hpp"

namespace vca {

__device__ __forceinline__ float load_elem(const void* p, int f32, int64_t i) {
  return f32 ? reinterpret_cast<const float*>(p)[i]
             : __uint_as_float(uint32_t(reinterpret_cast<const uint16_t*>(p)[i]) << 16);
}

__global__ void __launch_bounds__(256) attn_merge_kernel(const MergeArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t pair = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // row * H + h
  if (pair >= (int64_t)a.rows * a.H) return;
  const int row = int(pair / a.H), h = int(pair % a.H);
  const int64_t li = (int64_t)h * a.rows + row;
  const float la = a.lse_a[li], lb = a.lse_b[li];
  const float mx = fmaxf(la, lb);
  float wa = 0.f, wb = 0.f, l = kNegInf;
  if (mx != kNegInf) {
    const float ea = expf(la - mx), eb = expf(lb - mx);
    const float sum = ea + eb;
    wa = ea / sum;
    wb = eb / sum;
    l = mx + logf(sum);
  }
  const int64_t base = pair * a.Dv;
  for (int d = lane; d < a.Dv; d += 64) {
    const float v = wa * load_elem(a.out_a, a.a_f32, base + d) + wb * load_elem(a.out_b, a.b_f32, base + d);
    a.out[base + d] = v;
    if (a.out_bf16) {
      const __bf16 b = (__bf16)v;
      a.out_bf16[base + d] = __builtin_bit_cast(uint16_t, b);
    }
  }
  if (lane == 0) a.lse[li] = l;
}


hipError_t launch_merge(const MergeArgs& a, hipStream_t st) {
  const int64_t pairs = (int64_t)a.rows * a.H;
  if (pairs == 0) return hipSuccess;
  const dim3 grid((unsigned)((pairs + 3) / 4));
  TimedLaunch timer("attn_merge", st);
  hipLaunchKernelGGL(attn_merge_kernel, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace vca
