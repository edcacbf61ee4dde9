// Row movement of the packed ring layout ("gemma4_moe cp_attention" page:
// [B, H, S, D] -> packed [T, H, D] at flat indices b*S + pos and back, the
// packed lse [Hq, T] <-> dense [B, Hq, S] with -inf on rows no segment covers,
// the gradient scatter-add at the flat-index rows, and the in-place
// online-softmax merge of one chunk at its live rows only).
//
// One wave per (packed row t, head h): lanes cover the head dim with 16-byte
// accesses, so every row moves as contiguous bursts whatever the view's
// (b, h, s) strides. Element types are the ABI's dtype codes (16-bit rows move
// as raw bits, merges decode them to fp32).
#include "attn_common.hpp"
#include "attn_launch.hpp"
#include "attn_timing.hpp"

namespace vca {
using namespace VCA_ELEM;  // vector types and helpers (this unit is built once)

namespace {

constexpr int kF32 = 1, kF16 = 2;  // else bf16 (0)

__device__ __forceinline__ float bits_to_f(uint32_t b, int type) {
  return type == kF16 ? (float)__builtin_bit_cast(_Float16, (uint16_t)(b & 0xffffu))
                      : __uint_as_float(b << 16);
}

// dst[t, h, :] = src[b, h, s, :] (gather; mode 3 also rounds fp32 rows to a
// 16-bit dst_type) or dst view[b, h, s, :] (+)= src[t, h, :] (scatter), with
// index[t] = b*S + s; esz = element bytes of the dense side (2 or 4), D*esz a
// multiple of 16.
__global__ void __launch_bounds__(256) attn_rows_kernel(const RingRowsArgs a) {
  const int64_t pair = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // t * H + h
  if (pair >= (int64_t)a.T * a.H) return;
  const int lane = threadIdx.x & 63;
  const int t = (int)(pair / a.H), h = (int)(pair - (int64_t)t * a.H);
  const int64_t flat = a.index[t];
  const int64_t b = flat / a.S, s = flat - b * a.S;
  char* dense = static_cast<char*>(a.dense) + (b * a.sb + h * a.sh + s * a.sn) * a.esz;
  char* packed = static_cast<char*>(a.packed) + (pair * a.D) * a.esz;
  const int chunks = a.D * a.esz / 16;
  if (a.mode == 3) {
    // gather of fp32 rows into 16-bit ones (round to nearest even): eight
    // elements per lane and step
    const float* src = reinterpret_cast<const float*>(dense);
    uint16_t* dst = reinterpret_cast<uint16_t*>(static_cast<char*>(a.packed) + pair * a.D * 2);
    for (int c = lane; c < a.D / 8; c += 64) {
      const f32x4 x0 = reinterpret_cast<const f32x4*>(src)[2 * c];
      const f32x4 x1 = reinterpret_cast<const f32x4*>(src)[2 * c + 1];
      u32x4 r;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float lo = j < 2 ? x0[2 * j] : x1[2 * j - 4];
        const float hi = j < 2 ? x0[2 * j + 1] : x1[2 * j - 3];
        const uint32_t l16 = a.dst_type == kF16 ? __builtin_bit_cast(uint16_t, (_Float16)lo)
                                                : __builtin_bit_cast(uint16_t, (__bf16)lo);
        const uint32_t h16 = a.dst_type == kF16 ? __builtin_bit_cast(uint16_t, (_Float16)hi)
                                                : __builtin_bit_cast(uint16_t, (__bf16)hi);
        r[j] = l16 | (h16 << 16);
      }
      reinterpret_cast<u32x4*>(dst)[c] = r;
    }
    return;
  }
  for (int c = lane; c < chunks; c += 64) {
    u32x4* dp = reinterpret_cast<u32x4*>(dense) + c;
    u32x4* pp = reinterpret_cast<u32x4*>(packed) + c;
    if (a.mode == 0) {
      *pp = *dp;  // gather
    } else if (a.mode == 1) {
      *dp = *pp;  // scatter
    } else {
      // scatter-add, fp32 arithmetic, one rounding
      const u32x4 x = *pp, y = *dp;
      u32x4 r;
      if (a.type == kF32) {
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = __float_as_uint(__uint_as_float(x[j]) + __uint_as_float(y[j]));
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float lo = bits_to_f(x[j], a.type) + bits_to_f(y[j], a.type);
          const float hi = bits_to_f(x[j] >> 16, a.type) + bits_to_f(y[j] >> 16, a.type);
          const uint32_t l16 = a.type == kF16 ? __builtin_bit_cast(uint16_t, (_Float16)lo)
                                              : __builtin_bit_cast(uint16_t, (__bf16)lo);
          const uint32_t h16 = a.type == kF16 ? __builtin_bit_cast(uint16_t, (_Float16)hi)
                                              : __builtin_bit_cast(uint16_t, (__bf16)hi);
          r[j] = l16 | (h16 << 16);
        }
      }
      *dp = r;
    }
  }
}

// Every row (b, h, s) of a [B, H, S, D] view set to zero, and (when lse is
// set) lse[b, h, s] to -inf: the rows a scatter leaves untouched.
__global__ void __launch_bounds__(256) attn_fill_rows_kernel(const RingRowsArgs a) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // (b*H + h)*S + s
  if (row >= (int64_t)a.B * a.H * a.S) return;
  const int lane = threadIdx.x & 63;
  const int64_t s = row % a.S, bh = row / a.S;
  const int64_t h = bh % a.H, b = bh / a.H;
  u32x4* dp = reinterpret_cast<u32x4*>(static_cast<char*>(a.dense) +
                                        (b * a.sb + h * a.sh + s * a.sn) * a.esz);
  const int chunks = a.D * a.esz / 16;
  for (int c = lane; c < chunks; c += 64) dp[c] = zero_u32x4();
  if (a.lse_dense && lane == 0) a.lse_dense[row] = kNegInf;
}

// lse of the listed rows: packed [H, T] <-> dense [B, H, S] (contiguous)
__global__ void __launch_bounds__(256) attn_lse_rows_kernel(const RingRowsArgs a) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // h * T + t
  if (i >= (int64_t)a.T * a.H) return;
  const int h = (int)(i / a.T), t = (int)(i - (int64_t)h * a.T);
  const int64_t flat = a.index[t];
  const int64_t b = flat / a.S, s = flat - b * a.S;
  const int64_t d = (b * a.H + h) * a.S + s;
  if (a.mode == 0) a.lse_packed[i] = a.lse_dense[d];
  else a.lse_dense[d] = a.lse_packed[i];
}

// In-place -inf-safe online-softmax merge of a chunk's packed rows into the
// running fp32 accumulators at their flat-index rows: lse = logaddexp(lse_acc,
// lse_b), out = (e^lse_acc out_acc + e^lse_b out_b) / e^lse; both -inf leaves
// out 0, lse -inf. One wave per (t, h); lanes over the head dim.
__global__ void __launch_bounds__(256) attn_merge_rows_kernel(const RingRowsArgs a) {
  const int64_t pair = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // t * H + h
  if (pair >= (int64_t)a.T * a.H) return;
  const int lane = threadIdx.x & 63;
  const int t = (int)(pair / a.H), h = (int)(pair - (int64_t)t * a.H);
  const int64_t flat = a.index[t];
  const int64_t b = flat / a.S, s = flat - b * a.S;
  float* acc = static_cast<float*>(a.dense) + b * a.sb + h * a.sh + s * a.sn;
  float* la_p = a.lse_dense + (b * a.H + h) * a.S + s;
  const float la = *la_p, lb = a.lse_packed[(int64_t)h * a.T + t];
  const float mx = fmaxf(la, lb);
  float wa = 0.f, wb = 0.f, l = kNegInf;
  if (mx != kNegInf) {
    const float ea = expf(la - mx), eb = expf(lb - mx);
    const float sum = ea + eb;
    wa = ea / sum;
    wb = eb / sum;
    l = mx + logf(sum);
  }
  const char* pb = static_cast<const char*>(a.packed) + pair * a.D * a.esz;
  for (int d = lane; d < a.D; d += 64) {
    float vb;
    if (a.type == kF32) vb = reinterpret_cast<const float*>(pb)[d];
    else vb = bits_to_f(reinterpret_cast<const uint16_t*>(pb)[d], a.type);
    acc[d] = wa * acc[d] + wb * vb;
  }
  // every lane has read lse_acc above (same wave), so the write cannot race
  if (lane == 0) *la_p = l;
}

}  // namespace

hipError_t launch_ring_rows(const RingRowsArgs& a, int op, hipStream_t st) {
  const unsigned waves_grid = (unsigned)(((int64_t)a.T * a.H + 3) / 4);
  switch (op) {
    case kRingRows: {
      if ((int64_t)a.T * a.H == 0) return hipSuccess;
      TimedLaunch timer("attn_ring_rows", st);
      hipLaunchKernelGGL(attn_rows_kernel, dim3(waves_grid), dim3(256), 0, st, a);
      break;
    }
    case kRingFill: {
      const int64_t rows = (int64_t)a.B * a.H * a.S;
      if (rows == 0) return hipSuccess;
      TimedLaunch timer("attn_ring_fill", st);
      hipLaunchKernelGGL(attn_fill_rows_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st,
                         a);
      break;
    }
    case kRingLse: {
      const int64_t n = (int64_t)a.T * a.H;
      if (n == 0) return hipSuccess;
      TimedLaunch timer("attn_ring_lse", st);
      hipLaunchKernelGGL(attn_lse_rows_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                         a);
      break;
    }
    default: {
      if ((int64_t)a.T * a.H == 0) return hipSuccess;
      TimedLaunch timer("attn_merge_rows", st);
      hipLaunchKernelGGL(attn_merge_rows_kernel, dim3(waves_grid), dim3(256), 0, st, a);
      break;
    }
  }
  return hipGetLastError();
}

}  // namespace vca
