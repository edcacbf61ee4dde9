// Merge launcher and kernel.
#include "attn_common.hpp"
#include "attn_launch.hpp"
#include "attn_timing.hpp"

namespace vca {
using namespace VCA_ELEM;  // vector types and helpers (this unit is built once)

// Element types of the merge's inputs and copy (the ABI's dtype codes).
constexpr int kF32 = 1, kF16 = 2;  // else bf16 (0)

__device__ __forceinline__ float half_bits_to_f(uint32_t b, int type) {
  return type == kF16 ? (float)__builtin_bit_cast(_Float16, (uint16_t)(b & 0xffffu))
                      : __uint_as_float(b << 16);
}
__device__ __forceinline__ uint32_t f_to_half_bits(float v, int type) {
  return type == kF16 ? (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v)
                      : (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v);
}

__device__ __forceinline__ float load_elem(const void* p, int type, int64_t i) {
  return type == kF32 ? reinterpret_cast<const float*>(p)[i]
                      : half_bits_to_f(reinterpret_cast<const uint16_t*>(p)[i], type);
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
    const float v = wa * load_elem(a.out_a, a.a_type, base + d) +
                    wb * load_elem(a.out_b, a.b_type, base + d);
    a.out[base + d] = v;
    if (a.out_copy) a.out_copy[base + d] = (uint16_t)f_to_half_bits(v, a.copy_type);
  }
  if (lane == 0) a.lse[li] = l;
}


// Head dims that are a multiple of 8 with 16-byte aligned buffers: one thread
// per 8 consecutive elements of a (row, head), 16- and 32-byte loads and
// stores; each thread recomputes its row's weights from the two lse values.
__device__ __forceinline__ void load8(const void* p, int type, int64_t i, float (&v)[8]) {
  if (type == kF32) {
    const f32x4 x0 = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(p) + i);
    const f32x4 x1 = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(p) + i + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = x0[j];
      v[4 + j] = x1[j];
    }
  } else {
    const u32x4 x = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(p) + i);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = half_bits_to_f(x[j], type);
      v[2 * j + 1] = half_bits_to_f(x[j] >> 16, type);
    }
  }
}

__global__ void __launch_bounds__(256) attn_merge8_kernel(const MergeArgs a) {
  const int cpp = a.Dv >> 3;  // 8-element chunks per (row, head)
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= (int64_t)a.rows * a.H * cpp) return;
  const int64_t pair = c / cpp;  // row * H + h
  const int d0 = int(c - pair * cpp) * 8;
  const int row = int(pair / a.H), h = int(pair - (int64_t)row * a.H);
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
  const int64_t e = pair * a.Dv + d0;
  float va[8], vb[8], v[8];
  load8(a.out_a, a.a_type, e, va);
  load8(a.out_b, a.b_type, e, vb);
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = wa * va[j] + wb * vb[j];
  f32x4 o0, o1;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    o0[j] = v[j];
    o1[j] = v[4 + j];
  }
  *reinterpret_cast<f32x4*>(a.out + e) = o0;
  *reinterpret_cast<f32x4*>(a.out + e + 4) = o1;
  if (a.out_copy) {
    u32x4 b;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      b[j] = f_to_half_bits(v[2 * j], a.copy_type) | (f_to_half_bits(v[2 * j + 1], a.copy_type) << 16);
    *reinterpret_cast<u32x4*>(a.out_copy + e) = b;
  }
  if (d0 == 0) a.lse[li] = l;
}

// Zero the out rows (and set lse to -inf) of the (batch, position) rows a
// dense ring chunk must not produce. One workgroup per (row, batch), one
// wave per head in turn, lanes over the head dim.
__global__ void __launch_bounds__(256) attn_zero_rows_kernel(const ZeroRowsArgs a) {
  const int i = blockIdx.x, b = blockIdx.y;
  if (!a.rows[(int64_t)b * a.S + i]) return;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int h = w; h < a.H; h += 4) {
    const int64_t base = b * a.ob + h * a.oh + (int64_t)i * a.on;
    if (a.f32) {
      float* o = reinterpret_cast<float*>(a.out) + base;
      for (int d = lane; d < a.D; d += 64) o[d] = 0.f;
    } else {
      uint16_t* o = reinterpret_cast<uint16_t*>(a.out) + base;
      for (int d = lane; d < a.D; d += 64) o[d] = 0;
    }
    if (a.lse && lane == 0) a.lse[b * a.lse_sb + h * a.lse_sh + i] = kNegInf;
  }
}

hipError_t launch_zero_rows(const ZeroRowsArgs& a, hipStream_t st) {
  if (a.B == 0 || a.S == 0 || a.H == 0) return hipSuccess;
  TimedLaunch timer("attn_zero_rows", st);
  hipLaunchKernelGGL(attn_zero_rows_kernel, dim3((unsigned)a.S, (unsigned)a.B), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t st) {
  const int64_t pairs = (int64_t)a.rows * a.H;
  if (pairs == 0) return hipSuccess;
  auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  TimedLaunch timer("attn_merge", st);
  // The 8-wide kernel writes a row's lse from the thread of its first chunk
  // while the other chunks' threads read lse_a. When lse aliases lse_a that is
  // only ordered if all chunks of a (row, head) sit in one wave: 64 must be a
  // multiple of the chunk count Dv/8. Otherwise one wave per (row, head).
  const int cpp = a.Dv / 8;
  const bool one_wave = cpp >= 1 && cpp <= 64 && 64 % cpp == 0;
  if (a.Dv % 8 == 0 && al16(a.out_a) && al16(a.out_b) && al16(a.out) && al16(a.out_copy) &&
      (one_wave || a.lse != a.lse_a)) {
    const int64_t chunks = pairs * (a.Dv / 8);
    hipLaunchKernelGGL(attn_merge8_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)((pairs + 3) / 4)), dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace vca
