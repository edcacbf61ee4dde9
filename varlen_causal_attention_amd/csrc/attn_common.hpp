// Device-side building blocks shared by the attention kernels (gfx950 only).
//
// MFMA conventions used throughout (v_mfma_f32_32x32x16_bf16 / _f16, wave64):
//   A operand: lane l supplies row (l % 32), 8 contraction elements chosen by
//              the lane half (l / 32);
//   B operand: lane l supplies column (l % 32), 8 contraction elements chosen
//              by the lane half;
//   C/D:       lane l, register r holds row 8*(r/4) + 4*(l/32) + (r%4) and
//              column (l % 32).
// Which 8 contraction indices a lane half carries is free, as long as the A
// and B fragments of one product agree; the kernels use that freedom to feed
// a C tile back as a B operand without any lane exchange.
#pragma once

#include <hip/hip_runtime.h>
#include <limits.h>
#include <stdint.h>

#include "attn_args.hpp"

// Element type of q, k, v, out, dout, dq, dk, dv: every kernel translation
// unit is compiled once per type, bf16 into namespace vca::bf and (with
// VCA_ELEM_F16 defined) fp16 into vca::hf. Everything below depends on it only
// through elem_t, the 16-bit MFMA operand fragments and the 16-bit -> fp32
// decode helpers; accumulation is fp32 for both.
#ifdef VCA_ELEM_F16
#define VCA_ELEM hf
#define VCA_MFMA_32x32x16 "v_mfma_f32_32x32x16_f16"
#else
#define VCA_ELEM bf
#define VCA_MFMA_32x32x16 "v_mfma_f32_32x32x16_bf16"
#endif

namespace vca {
namespace VCA_ELEM {

#ifdef VCA_ELEM_F16
typedef _Float16 elem_t;
#else
typedef __bf16 elem_t;
#endif
typedef elem_t frag8 __attribute__((ext_vector_type(8)));
typedef elem_t elem4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16 mfma32(frag8 a, frag8 b, f32x16 c) {
#ifdef VCA_ELEM_F16
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
#else
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
#endif
}

// fp32 value of a 16-bit element held in the low bits of b (exact for both
// types)
__device__ __forceinline__ float elem_to_f(uint32_t b) {
#ifdef VCA_ELEM_F16
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(b & 0xffffu));
#else
  return __uint_as_float(b << 16);
#endif
}
// the low / high element of a 32-bit word of two packed elements
__device__ __forceinline__ float elem_lo_f(uint32_t w) { return elem_to_f(w & 0xffffu); }
__device__ __forceinline__ float elem_hi_f(uint32_t w) {
#ifdef VCA_ELEM_F16
  return elem_to_f(w >> 16);
#else
  return __uint_as_float(w & 0xffff0000u);
#endif
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}
__device__ __forceinline__ f32x16 splat16(float x) {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = x;
  return z;
}

__device__ __forceinline__ u32x4 ldg16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void sts16(uint16_t* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ void sts8(uint16_t* p, u32x2 v) { *reinterpret_cast<u32x2*>(p) = v; }
__device__ __forceinline__ frag8 lds_frag(const uint16_t* p) {
  return *reinterpret_cast<const frag8*>(p);
}
__device__ __forceinline__ frag8 as_frag(u32x4 v) { return __builtin_bit_cast(frag8, v); }

__device__ __forceinline__ u32x4 zero_u32x4() {
  u32x4 z = {0u, 0u, 0u, 0u};
  return z;
}

// Element e (0..7) of eight packed bf16 values.
__device__ __forceinline__ uint32_t elem_at(u32x4 v, int e) {
  return (v[e >> 1] >> ((e & 1) * 16)) & 0xffffu;
}

// Instruction-group masks for __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

// Ask the scheduler to run N MFMAs, each fed by one LDS read, with LEAD reads
// issued ahead of the first MFMA: reads, then (MFMA, read) pairs, then the
// last MFMAs. Keeps LEAD fragment reads in flight so the LDS latency hides
// behind the MFMA pipe instead of stalling every MFMA.
template <int N, int LEAD, int READS_PER_MFMA = 1>
__device__ __forceinline__ void pipeline_mfma_reads() {
  static_assert(LEAD <= N, "lead");
  __builtin_amdgcn_sched_group_barrier(kSchedDsRead, LEAD * READS_PER_MFMA, 0);
#pragma unroll
  for (int i = 0; i < N - LEAD; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, READS_PER_MFMA, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kSchedMfma, LEAD, 0);
}

// Partner lane across the two wave halves (l ^ 32).
// Hand-written MFMAs, for kernels whose operands or accumulators sit in the
// accumulation registers (AGPRs). The compiler does not see these
// as MFMAs, so they carry their own wait states: mfma_a's s_nop gives the 2 a
// VALU write of an A/B operand needs before the MFMA reads it (back-to-back
// MFMAs on one accumulator need none), and mfma_results_ready() waits out an
// MFMA before anything else reads or overwrites its result or C operand.
// S / dP: A from an LDS read, B from AGPRs (no VALU-written operand, so no
// wait states); C starts at zero (mfma_v0) or accumulates (mfma_v).
__device__ __forceinline__ void mfma_v0(f32x16& c, frag8 a, frag8 b_agpr) {
  asm(VCA_MFMA_32x32x16 " %0, %1, %2, 0" : "=&v"(c) : "v"(a), "a"(b_agpr));
}
__device__ __forceinline__ void mfma_v(f32x16& c, frag8 a, frag8 b_agpr) {
  asm(VCA_MFMA_32x32x16 " %0, %1, %2, %0" : "+v"(c) : "v"(a), "a"(b_agpr));
}
__device__ __forceinline__ void mfma_a(f32x16& acc, frag8 a, frag8 b) {
  asm("s_nop 1\n\t" VCA_MFMA_32x32x16 " %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// Orders the wait after the MFMAs that produced `x` (an asm with x as an
// in/out operand cannot move above them).
__device__ __forceinline__ void mfma_results_ready(f32x16& x0, f32x16& x1) {
  if (&x0 == &x1) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(x0));
  else asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(x0), "+v"(x1));
}
// Move a value into AGPRs at its definition, so the loop-carried value is
// allocated there (instead of living in VGPRs and being copied around every
// MFMA that takes it from an AGPR).
__device__ __forceinline__ f32x16 in_agprs(f32x16 x) {
  f32x16 r;
  asm volatile("; in agprs" : "=a"(r) : "0"(x));
  return r;
}
__device__ __forceinline__ frag8 in_agprs(frag8 x) {
  frag8 r;
  asm volatile("; in agprs" : "=a"(r) : "0"(x));
  return r;
}

// Through the gfx950 VALU half swap instead of an LDS permute: the swap
// exchanges the upper 32 lanes of its first operand with the lower 32 lanes
// of its second, so with both = x a lane of the lower half finds x[l + 32]
// in the second result and a lane of the upper half x[l - 32] in the first.
__device__ __forceinline__ float xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(__lane_id() < 32 ? r[1] : r[0]);
}

// Wait until every outstanding global load of this wave has landed
// (s_waitcnt vmcnt(0); expcnt and lgkmcnt left at "no wait"). Used once,
// after the loads of values that stay live across a loop, so the loop's
// own prefetches are never waited on before they are needed.
__device__ __forceinline__ void wait_global_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// s_waitcnt vmcnt(N): wait until at most N vector memory operations of this
// wave are outstanding (they complete in issue order); other counters free.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// gfx950 direct global -> LDS load (global_load_lds_dwordx4): lane l's 16
// bytes from g land at LDS byte address lds_base + 16*l; the data never
// passes through VGPRs. Issued as inline assembly on purpose: the compiler
// treats any outstanding LDS DMA as aliasing every later LDS read and every
// barrier and drains vmcnt in front of them, which would serialize a
// multi-stage pipeline. Callers therefore own the synchronization: a stage is
// read only after wait_vmcnt<> (own loads) and a barrier (everyone's). M0 is
// restored afterwards; the s_nops separate the M0 writes from the LDS DMA.
typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ lds_void* lds_ptr(const void* p) { return (lds_void*)p; }
// The LDS address reaches the asm as an integer taken from the array's
// address, so the array counts as escaped and the compiler keeps every later
// read of it (the "memory" clobber covers the write).
__device__ __forceinline__ void dma16(const uint16_t* g, lds_void* lds_base) {
  uint32_t saved;
  const uint32_t m0 = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_nop 0\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(g), "s"(m0)
      : "memory");
}
// The same load addressed as a wave-uniform base (SGPRs) plus a 32-bit
// per-lane byte offset: one VGPR per distinct offset instead of a 64-bit
// address per load.
__device__ __forceinline__ void dma16s(const uint16_t* sbase, uint32_t voff_bytes,
                                       lds_void* lds_base) {
  uint32_t saved;
  const uint32_t m0 = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_nop 0\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff_bytes), "s"(sbase), "s"(m0)
      : "memory");
}
// One row: lane l's 16 bytes from sbase + voff_bytes land at LDS byte
// address m0 + 16*l (m0 a wave-uniform LDS address as an integer).
__device__ __forceinline__ void dma16m(const uint16_t* sbase, uint32_t voff_bytes, uint32_t m0) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_nop 0\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff_bytes), "s"(sbase), "s"(m0)
      : "memory");
}
// Eight rows at once: row i's 16 bytes per lane come from p[i] + voff_bytes
// and land at LDS byte address m0[i] + 16*l (wave-uniform LDS addresses as
// integers). Counts as eight operations for vmcnt.
__device__ __forceinline__ void dma16_rows8(const uint16_t* const (&p)[8], uint32_t voff_bytes,
                                            const uint32_t (&m0)[8]) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %10\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %11\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %3\n\t"
      "s_mov_b32 m0, %12\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %4\n\t"
      "s_mov_b32 m0, %13\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %5\n\t"
      "s_mov_b32 m0, %14\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %6\n\t"
      "s_mov_b32 m0, %15\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %7\n\t"
      "s_mov_b32 m0, %16\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %8\n\t"
      "s_mov_b32 m0, %17\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %9\n\t"
      "s_nop 0\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff_bytes), "s"(p[0]), "s"(p[1]), "s"(p[2]), "s"(p[3]), "s"(p[4]), "s"(p[5]),
        "s"(p[6]), "s"(p[7]), "s"(m0[0]), "s"(m0[1]), "s"(m0[2]), "s"(m0[3]), "s"(m0[4]),
        "s"(m0[5]), "s"(m0[6]), "s"(m0[7])
      : "memory");
}
// Global stores whose vmcnt footprint is exactly one operation each (used
// where a wave counts its outstanding memory operations by hand). A store of
// more than 8 bytes reads its data VGPRs after issue: a VALU write to them in
// the next cycle would change what is stored. The compiler pads its own
// stores; these carry their own wait states.
__device__ __forceinline__ void stg16(uint16_t* p, u32x4 v) {
  asm volatile("global_store_dwordx4 %0, %1, off\n\ts_nop 1" ::"v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ void stg8(uint16_t* p, u32x2 v) {
  asm volatile("global_store_dwordx2 %0, %1, off\n\ts_nop 1" ::"v"(p), "v"(v) : "memory");
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// tanh(x) = 1 - 2 / (e^(2x) + 1): one exp2 and one reciprocal; saturates to
// +-1 without overflow (e^(2x) = inf gives 1, 0 gives -1)
__device__ __forceinline__ float fast_tanh(float x) {
  return 1.f - 2.f * __builtin_amdgcn_rcpf(fast_exp2(x * (2.f * 1.4426950408889634f)) + 1.f);
}
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Eight fp32 values -> eight elements (round to nearest even) as one MFMA fragment.
__device__ __forceinline__ frag8 to_frag(const float* x) {
  frag8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (elem_t)x[i];
  return r;
}

// Rows [row0, row0 + R) x D bf16 columns of a row-major global view, staged
// through registers (16-byte chunks; rows >= nrows read as zero) into a
// row-major LDS tile with row stride LS elements. load() may be issued a step
// ahead so the global latency overlaps other work; copy() goes straight
// through with few registers live.
template <int R, int D, int NT>
struct TileStage {
  static constexpr int CH = R * D / 8;
  static constexpr int PT = (CH + NT - 1) / NT;
  u32x4 r[PT];

  __device__ __forceinline__ void load(const uint16_t* base, int64_t sn, int row0, int nrows,
                                       int tid) {
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int c = tid + i * NT;
      const int row = c / (D / 8), cc = c % (D / 8);
      r[i] = (c < CH && row0 + row < nrows) ? ldg16(base + (int64_t)(row0 + row) * sn + cc * 8)
                                            : zero_u32x4();
    }
  }
  // Branch-free variant: rows past the end re-read row nrows - 1 (nrows >= 1),
  // which stays inside the segment; callers mask those rows out of every
  // result (their scores are hidden / their P is zero).
  // Head dims up to 128: a tile wholly inside the rows (every tile but a
  // segment's last) takes the scalar tile base plus a per-thread offset that
  // does not depend on the tile, so the compiler keeps it out of the loop.
  // (Wider tiles keep the plain form: the hoisted offsets cost registers
  // their kernels do not have.)
  __device__ __forceinline__ void load_clamped(const uint16_t* base, int64_t sn, int row0,
                                               int nrows, int tid) {
    if (D <= 128 && row0 + R <= nrows) {
      const uint16_t* b = base + (int64_t)row0 * sn;
#pragma unroll
      for (int i = 0; i < PT; ++i) {
        const int c = min(tid + i * NT, CH - 1);
        r[i] = ldg16(b + (int64_t)(c / (D / 8)) * sn + (c % (D / 8)) * 8);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int c = min(tid + i * NT, CH - 1);
      const int row = min(row0 + c / (D / 8), nrows - 1), cc = c % (D / 8);
      r[i] = ldg16(base + (int64_t)row * sn + cc * 8);
    }
  }
  template <int LS>
  __device__ __forceinline__ void store(uint16_t* dst, int tid) const {
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int c = tid + i * NT;
      if (c < CH) sts16(&dst[(c / (D / 8)) * LS + (c % (D / 8)) * 8], r[i]);
    }
  }
  template <int LS>
  __device__ __forceinline__ static void copy(uint16_t* dst, const uint16_t* base, int64_t sn,
                                              int row0, int nrows, int tid) {
    for (int c = tid; c < CH; c += NT) {
      const int row = c / (D / 8), cc = c % (D / 8);
      sts16(&dst[row * LS + cc * 8], row0 + row < nrows
                                         ? ldg16(base + (int64_t)(row0 + row) * sn + cc * 8)
                                         : zero_u32x4());
    }
  }
};

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// MFMA A-operand fragment read down the columns of a row-major LDS tile
// X[k][n] (row stride LS elements) with the gfx950 transposing LDS read
// (ds_read_b64_tr_b16). Within each 16-lane group, lane s points at row
// k0 + s/4 and columns 4*(s%4)..+3; the hardware hands lane i of the group
// column i of those four rows. Result: lane l gets column n0 + (l % 32) and
// rows {k0 + 4h + j, k0 + 8 + 4h + j : j < 4} (h = l / 32), the key/query
// order in which a 32x32 C tile holds its rows, so the fragment pairs with a
// C tile reused as the B operand.
__device__ __forceinline__ frag8 tr_frag(const uint16_t* X, int LS, int k0, int n0, int lane) {
  const int g = lane >> 4, s = lane & 15, h = lane >> 5;
  const int row = k0 + 4 * h + (s >> 2);
  const int c = n0 + 16 * (g & 1) + 4 * (s & 3);
  const uint16_t* p = X + row * LS + c;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)((__attribute__((address_space(3))) uint16_t*)p));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)((__attribute__((address_space(3))) uint16_t*)(p + 8 * LS)));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(frag8, v);
}

// ---- swizzled 128-wide tiles ---------------------------------------------
// Rows of kTileD = 128 bf16 elements (256 bytes), loaded straight into LDS
// by global_load_lds, four rows per 1 KB load (lane l: row 4j + l/16, stored
// piece l%16).
constexpr int kTileD = 128;
// Staged tiles are row-major with 256-byte rows; the 16-byte piece u of row r
// sits at position u ^ (4*(r%4) + (r/4)%4). A row read (ds_read_b128, 16
// consecutive rows per LDS cycle) then covers all 16 piece positions, and a
// transposing read (4 consecutive rows x 64 bytes per 32 lanes) covers all 16
// as well: both are free of bank conflicts.
__device__ __forceinline__ int rtile_off(int r, int u) {
  return r * kTileD + ((u ^ (((r & 3) << 2) | ((r >> 2) & 3))) << 3);
}
// A operand of S / dP: lane l gets row l%32 and the 8 head-dim elements of
// piece `piece` (= 2*ks + l/32).
__device__ __forceinline__ frag8 rtile_row(const uint16_t* X, int r, int piece) {
  return lds_frag(X + rtile_off(r, piece));
}
// A operand of dV^T / dK^T: lane l gets head-dim column n0 + l%32 and query
// rows {k0 + 4h + j, k0 + 8 + 4h + j : j < 4} (h = l/32) through the
// transposing read; the row order matches a 32x32 C tile reused as B.
__device__ __forceinline__ frag8 rtile_col(const uint16_t* X, int k0, int n0, int lane) {
  const int g = lane >> 4, s = lane & 15, h = lane >> 5;
  const int row = k0 + 4 * h + (s >> 2);
  const int c = n0 + 16 * (g & 1) + 4 * (s & 3);
  typedef __attribute__((address_space(3))) uint16_t lds_u16;
  const uint16_t* p0 = X + rtile_off(row, c >> 3) + (c & 7);
  const uint16_t* p1 = X + rtile_off(row + 8, c >> 3) + (c & 7);
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)((lds_u16*)p0));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)((lds_u16*)p1));
  return __builtin_bit_cast(frag8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// 64-column blocks (head-dim columns 128..191 of 192-wide rows) in 128-byte
// rows: piece u of row r sits at u ^ sw64(r), sw64(r) = 4*(x%2) + x/2 with
// x = (r/2) % 8. Two rows share one 256-byte bank line, so 16 consecutive
// rows reading one piece cover all 64 banks when sw64 permutes the 8
// positions within each row parity (it does); the transposing read (4 rows
// x 4 pieces per 32 lanes) puts rows r and r+2 in different 4-piece halves
// (sw64 differs in bit 2 between them), so it is free of conflicts as well.
__device__ __forceinline__ int sw64(int r) {
  const int x = (r >> 1) & 7;
  return ((x & 1) << 2) | (x >> 1);
}
__device__ __forceinline__ int r64_off(int r, int u) { return r * 64 + ((u ^ sw64(r)) << 3); }
__device__ __forceinline__ frag8 r64_row(const uint16_t* X, int r, int piece) {
  return lds_frag(X + r64_off(r, piece));
}
// rtile_col's operand (head-dim column n0 + l%32, rows k0 + 4h + j and
// k0 + 8 + 4h + j) from a 64-column block
__device__ __forceinline__ frag8 r64_col(const uint16_t* X, int k0, int n0, int lane) {
  const int g = lane >> 4, s = lane & 15, h = lane >> 5;
  const int row = k0 + 4 * h + (s >> 2);
  const int c = n0 + 16 * (g & 1) + 4 * (s & 3);
  typedef __attribute__((address_space(3))) uint16_t lds_u16;
  const uint16_t* p0 = X + r64_off(row, c >> 3) + (c & 7);
  const uint16_t* p1 = X + r64_off(row + 8, c >> 3) + (c & 7);
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)((lds_u16*)p0));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)((lds_u16*)p1));
  return __builtin_bit_cast(frag8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Workgroup -> (work item, q-head) for passes whose grid is items x H q-heads
// (GQA group size G). Consecutive workgroup ids are dispatched to the 8 XCDs
// in turn; when the kv heads divide evenly over the XCDs, XCD x gets every
// q-head of kv heads x, x+8, ..., so the workgroups that stream one kv head's
// K/V share that XCD's L2, items in list (heavy-first) order. Otherwise
// items outermost, heads innermost.
constexpr int kXcdCount = 8;
__device__ __forceinline__ void xcd_item_head(int bid, int H, int G, int& item, int& h) {
  if ((H / G) % kXcdCount == 0) {
    const int x = bid % kXcdCount, k = bid / kXcdCount;
    const int per = H / kXcdCount;  // q-heads per XCD
    item = k / per;
    const int j = k - item * per;
    h = (x + kXcdCount * (j / G)) * G + j % G;
  } else {
    item = bid / H;
    h = bid - item * H;
  }
}

// Segment geometry (SegGeom): cu arrays are clamped into [0, T] so a
// malformed table can never index outside the tensors.

__device__ __forceinline__ SegGeom seg_geom(const int32_t* cu_q, const int32_t* cu_k, int s,
                                            int Nq, int Nk, int Tq, int Tk) {
  SegGeom g;
  if (cu_q) {
    int qa = min(max(cu_q[s], 0), Tq);
    int qb = min(max(cu_q[s + 1], qa), Tq);
    int ka = min(max(cu_k[s], 0), Tk);
    int kb = min(max(cu_k[s + 1], ka), Tk);
    g.q_row0 = qa;
    g.lq = qb - qa;
    g.k_row0 = ka;
    g.lk = kb - ka;
  } else {
    g.q_row0 = 0;
    g.lq = Nq;
    g.k_row0 = 0;
    g.lk = Nk;
  }
  return g;
}

}  // namespace VCA_ELEM
}  // namespace vca
