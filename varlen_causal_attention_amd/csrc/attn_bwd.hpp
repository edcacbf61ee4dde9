// Backward kernels, recomputing from the caller's out/lse (NeMo-Automodel
// "ffpa_attention" page, dense and varlen backward entries: the ring feeds a
// globally merged out/lse, so the backward never uses a chunk-local one).
//
//   delta[i]  = sum_d dO[i,d] * O[i,d]         (dQ kernel prologue; delta kernel
//                                                for the two-phase head dims)
//   P[i,j]    = exp(scale * q_i.k_j - lse_i) on visible (i,j), 0 elsewhere and
//               on rows with lse = -inf
//   dV[j]    += sum_i P[i,j] dO[i]                            (dK/dV kernel)
//   dS[i,j]   = P[i,j] * (dO[i].v_j - delta[i])
//   dK[j]    += scale * sum_i dS[i,j] q_i                     (dK/dV kernel)
//   dQ[i]     = scale * sum_j dS[i,j] k_j                     (dQ kernel)
// dK/dV sum over the q-heads of each GQA group inside the dK/dV kernel.
//
// In the two generic kernels below each wave owns one 32-row block over the
// whole head dim (dK/dV: 32 keys; dQ: 32 queries). They serve the window /
// softcap variants and the head dims without a dedicated pass (dQ by
// recomputation at 64, and at 128 and 192/128 when the dS store is off);
// 256 and 512 take the two-phase backward.
#pragma once

#include <type_traits>

#include "attn_common.hpp"
#include "attn_fwd.hpp"

namespace vca {
namespace VCA_ELEM {


// Element offset of dS block (h, query tile starting at segment row q0, key
// tile starting at segment key k0), or -1 when the layout has no room for it
// (only with cu_seqlens that break their contract: a segment longer than
// max_k).
__device__ __forceinline__ int64_t ds_block(const BwdArgs& a, int s, const SegGeom& sg, int h,
                                            int q0, int k0) {
  const int qt_flat = a.cu_q ? (sg.q_row0 >> 5) + s + (q0 >> 5) : s * a.ds_qtb + (q0 >> 5);
  const int kt = k0 >> 5;
  if (kt >= a.ds_mkt || qt_flat >= a.ds_nqt) return -1;
  return (((int64_t)(h - a.ds_h0) * a.ds_nqt + qt_flat) * a.ds_mkt + kt) * 1024;
}

// Store one lane's share of a 32x32 dS block held as the two bf16 B
// fragments of dK^T += Q^T dS, in that fragment order.
__device__ __forceinline__ void ds_store(uint16_t* blk, int lane, frag8 f0, frag8 f1) {
  *reinterpret_cast<u32x4*>(blk + 8 * lane) = __builtin_bit_cast(u32x4, f0);
  *reinterpret_cast<u32x4*>(blk + 512 + 8 * lane) = __builtin_bit_cast(u32x4, f1);
}

// ---------------------------------------------------------------------------
// delta = rowsum(dO * O) in fp32. blockIdx = (row block, head, segment); a row
// is covered by DV/8 lanes (at most 64), each reading 16-byte chunks.
// ---------------------------------------------------------------------------
template <int DV>
__global__ void __launch_bounds__(256) attn_bwd_delta_kernel(const BwdArgs a) {
  constexpr int LPR = DV / 8 >= 64 ? 64 : DV / 8;  // lanes per row
  constexpr int RPW = 64 / LPR;                     // rows per wave
  constexpr int CPL = DV / 8 / LPR;                 // 16-byte chunks per lane
  const int s = blockIdx.z, h = blockIdx.y;
  const SegGeom sg = seg_geom(a.cu_q, a.cu_k, s, a.Nq, a.Nk, a.Tq, a.Tk);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int sub = lane / LPR, li = lane % LPR;
  const int row = (blockIdx.x * 4 + w) * RPW + sub;
  float acc = 0.f;
  const bool ok = row < sg.lq;
  if (ok) {
    const int64_t r = sg.q_row0 + row;
    const uint16_t* op = a.o.p + s * a.o.sb + r * a.o.sn + h * a.o.sh;
    const uint16_t* dp = a.dout.p + s * a.dout.sb + r * a.dout.sn + h * a.dout.sh;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int d0 = (c * LPR + li) * 8;
      const u32x4 ov = ldg16(op + d0), dv = ldg16(dp + d0);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        acc += elem_to_f(elem_at(ov, e)) * elem_to_f(elem_at(dv, e));
    }
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (ok && li == 0) {
    const int64_t idx = s * a.lse_sb + h * a.lse_sh + sg.q_row0 + row;
    a.delta[idx] = acc;
    // a row with lse = -inf attends nothing: +inf makes its P = exp2(s - lse2)
    // exactly zero on every key, masked or not (the dense cross chunk of a
    // ring sees its padding queries' keys)
    const float l = a.lse[idx];
    a.lse2[idx] = l == kNegInf ? __builtin_inff() : l * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// dK / dV: one workgroup = (segment, kv-head, block of 32*NW keys). The
// workgroup walks every (q-head of the group, 32-row query step) that can see
// its keys; each step's Q and dO rows are staged row-major in two LDS buffers
// (the next step's global loads issued a step ahead into registers), read
// row-wise as the A operand of S = Q K^T and dP = dO V^T, and column-wise
// (transposing LDS read) as the A operand of dK^T += Q^T dS and dV^T += dO^T P.
// ---------------------------------------------------------------------------
template <int DQK, int DV, int NW, bool CAUSAL, bool EXT = false>
__global__ void __launch_bounds__(64 * NW, NW / 4) attn_bwd_dkdv_kernel(const BwdArgs a) {
  constexpr int NT = 64 * NW;  // threads
  constexpr int KG = NW;       // 32-key groups per workgroup
  static_assert(DQK % 32 == 0 && DV % 32 == 0, "head dims");
  constexpr int NKS = DQK / 16, NVS = DV / 16;
  constexpr int NDB = DQK / 32, NVB = DV / 32;
  constexpr int BQ = 32;
  constexpr int QS = DQK + 16, OS = DV + 16;  // LDS row strides (elements)
  __shared__ __attribute__((aligned(16))) uint16_t sq[2][BQ * QS];
  __shared__ __attribute__((aligned(16))) uint16_t sdo[2][BQ * OS];
  __shared__ __attribute__((aligned(16))) float slse[2][BQ];
  __shared__ __attribute__((aligned(16))) float sdel[2][BQ];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int kg = w;  // this wave's 32-key group
  const int item = blockIdx.x / a.kvh_n, g = a.kvh0 + (blockIdx.x - item * a.kvh_n);
  if (item >= *a.count_k) return;
  const int2 st = a.items_k[item];
  const int s = st.x;
  const SegGeom sg = seg_geom(a.cu_q, a.cu_k, s, a.Nq, a.Nk, a.Tq, a.Tk);
  const int kb0 = st.y * (32 * KG);
  if (kb0 >= sg.lk) return;
  const int lq = sg.lq, lk = sg.lk, shift = lk - lq;
  const int gk0 = kb0 + kg * 32;        // first key of this wave's group
  const int key = gk0 + col;            // this lane's key (output column)

  const uint16_t* kbp = a.k.p + s * a.k.sb + (int64_t)sg.k_row0 * a.k.sn + g * a.k.sh;
  const uint16_t* vbp = a.v.p + s * a.v.sb + (int64_t)sg.k_row0 * a.v.sn + g * a.v.sh;

  // K and V fragments of this lane's key (B operands)
  frag8 kf[NKS], vf[NVS];
  {
    const bool ok = key < lk;
    const uint16_t* kp = kbp + (int64_t)(ok ? key : 0) * a.k.sn + half * 8;
    const uint16_t* vp = vbp + (int64_t)(ok ? key : 0) * a.v.sn + half * 8;
#pragma unroll
    for (int i = 0; i < NKS; ++i) kf[i] = as_frag(ok ? ldg16(kp + i * 16) : zero_u32x4());
#pragma unroll
    for (int i = 0; i < NVS; ++i) vf[i] = as_frag(ok ? ldg16(vp + i * 16) : zero_u32x4());
  }
  wait_global_loads();

  f32x16 dka[NDB], dva[NVB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) dka[i] = zero16();
#pragma unroll
  for (int i = 0; i < NVB; ++i) dva[i] = zero16();

  // query steps that can see any key of this block (with a left window, the
  // rows past the last one whose window still reaches the block's last key
  // see none of it)
  const int win = EXT && CAUSAL ? a.window : 0;
  const bool capped = EXT && a.cap_in != 0.f;
  int q_begin = 0;
  if (CAUSAL) q_begin = max(0, kb0 - shift);
  q_begin &= ~(BQ - 1);
  const int q_end = win > 0 ? max(0, min(lq, kb0 + 32 * KG - 1 - shift + win)) : lq;
  const int nq = q_end > q_begin ? (q_end - q_begin + BQ - 1) / BQ : 0;
  const int total = a.G * nq;

  using QStage = TileStage<BQ, DQK, NT>;
  using OStage = TileStage<BQ, DV, NT>;
  QStage qst;
  OStage ost;
  float lse_r = 0.f, del_r = 0.f;  // threads < BQ carry one row's lse / delta
  bool row_ok = false;

  // step it -> (q-head, first query): query steps from the segment's end
  // down, the group's q-heads innermost, so the key blocks of a segment read
  // each Q/dO tile at about the same time (shared in L2)
  auto step_ptrs = [&](int it, const uint16_t*& qp, const uint16_t*& dop, int64_t& lb, int& q0) {
    const int hh = it % a.G;
    q0 = q_begin + (nq - 1 - it / a.G) * BQ;
    const int h = g * a.G + hh;
    qp = a.q.p + s * a.q.sb + (int64_t)sg.q_row0 * a.q.sn + h * a.q.sh;
    dop = a.dout.p + s * a.dout.sb + (int64_t)sg.q_row0 * a.dout.sn + h * a.dout.sh;
    lb = s * a.lse_sb + h * a.lse_sh + sg.q_row0;
  };
  auto load_rows = [&](int it) {
    const uint16_t *qp, *dop;
    int64_t lb;
    int q0;
    step_ptrs(it, qp, dop, lb, q0);
    qst.load_clamped(qp, a.q.sn, q0, lq, tid);
    ost.load_clamped(dop, a.dout.sn, q0, lq, tid);
    // raw values only: using a loaded value here would make the wave wait for
    // every earlier load, the prefetched tiles included
    if (tid < BQ) {
      const int i = min(q0 + tid, lq - 1);
      lse_r = a.lse[lb + i];
      del_r = a.delta[lb + i];
      row_ok = q0 + tid < lq;
    }
  };
  auto store_rows = [&](int b) {
    qst.template store<QS>(sq[b], tid);
    ost.template store<OS>(sdo[b], tid);
    if (tid < BQ) {
      // base-2 lse; rows past the segment end or with lse = -inf get +inf (P = 0)
      slse[b][tid] = (row_ok && lse_r != kNegInf) ? lse_r * kLog2e : __builtin_inff();
      sdel[b][tid] = row_ok ? del_r : 0.f;
    }
  };

  if (total > 0) {
    load_rows(0);
    store_rows(0);
    if (total > 1) load_rows(1);
  }

  // dS block of the previous step, stored after this step's wait for its
  // prefetched rows and before the next prefetch: the compiler waits for
  // every outstanding memory operation when loads and stores are mixed, so
  // a store issued there is waited for only one step later
  int64_t pend_off = -1;
  frag8 pend0, pend1;
  auto flush_ds = [&]() {
    if (pend_off >= 0) ds_store(a.ds + pend_off, lane, pend0, pend1);
    pend_off = -1;
  };
  for (int it = 0; it < total; ++it) {
    const int buf = it & 1;
    const int q0 = q_begin + (nq - 1 - it / a.G) * BQ;
    __syncthreads();  // step `it` is in LDS; nobody still reads the other buffer
    if (it + 1 < total) {
      store_rows(buf ^ 1);
      flush_ds();
      if (it + 2 < total) load_rows(it + 2);
    } else {
      flush_ds();
    }
    // this 32-query step is hidden from every key of this wave's group?
    const bool live = gk0 < lk && !(CAUSAL && gk0 > q0 + BQ - 1 + shift) &&
                      !(win > 0 && gk0 + 31 <= q0 + shift - win);
    f32x16 sacc = zero16(), pacc = zero16();
    if (live) {
      // S[q][key] = Q K^T and dP[q][key] = dO V^T
#pragma unroll
      for (int i = 0; i < NKS; ++i)
        sacc = mfma32(lds_frag(&sq[buf][col * QS + half * 8 + i * 16]), kf[i], sacc);
#pragma unroll
      for (int i = 0; i < NVS; ++i)
        pacc = mfma32(lds_frag(&sdo[buf][col * OS + half * 8 + i * 16]), vf[i], pacc);
      pipeline_mfma_reads<NKS + NVS, 4>();
    }
    if (live) {
      // P and dS (rows q = q0 + 8*(r/4) + 4*half + r%4, column = key). Rows
      // past the segment end carry lse = +inf, so their P is 0 without a mask;
      // the key mask is only needed on steps that cross the causal diagonal
      // or hold keys past the segment end.
      const bool need_mask = gk0 + 31 >= lk || (CAUSAL && gk0 + 31 > q0 + shift) ||
                             (win > 0 && gk0 <= q0 + BQ - 1 + shift - win);
      float p[16], dsv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qr = (r >> 2) * 8 + half * 4 + (r & 3);
        // softcap: P = exp(cap * tanh(scale * s / cap) - lse), and the score
        // gradient takes the chain factor 1 - tanh^2
        float th = 0.f;
        if (EXT && capped) th = fast_tanh(a.cap_in * sacc[r]);
        float x = fast_exp2((EXT && capped ? a.cap_out * th : sacc[r] * a.scale_log2) -
                            slse[buf][qr]);
        if (need_mask) {
          bool vis = key < lk;
          if (CAUSAL) vis = vis && key <= q0 + qr + shift;
          if (EXT && win > 0) vis = vis && key > q0 + qr + shift - win;
          x = vis ? x : 0.f;
        }
        p[r] = x;
        dsv[r] = x * (pacc[r] - sdel[buf][qr]);
        if (EXT && capped) dsv[r] *= 1.f - th * th;
      }
      const frag8 p0 = to_frag(p), p1 = to_frag(p + 8);
      const frag8 s0 = to_frag(dsv), s1 = to_frag(dsv + 8);
      if (a.ds) {
        // this step is visible to the wave's key tile: its dS block for the
        // dQ pass, stored at the next step (see pend_off)
        pend_off = ds_block(a, s, sg, g * a.G + it % a.G, q0, gk0);
        pend0 = s0;
        pend1 = s1;
      }
      // dV^T[dv][key] += dO^T P ; dK^T[d][key] += Q^T dS
#pragma unroll
      for (int b = 0; b < NVB; ++b) {
        dva[b] = mfma32(tr_frag(sdo[buf], OS, 0, b * 32, lane), p0, dva[b]);
        dva[b] = mfma32(tr_frag(sdo[buf], OS, 16, b * 32, lane), p1, dva[b]);
      }
#pragma unroll
      for (int b = 0; b < NDB; ++b) {
        dka[b] = mfma32(tr_frag(sq[buf], QS, 0, b * 32, lane), s0, dka[b]);
        dka[b] = mfma32(tr_frag(sq[buf], QS, 16, b * 32, lane), s1, dka[b]);
      }
      pipeline_mfma_reads<2 * (NVB + NDB), 4, 2>();
    }
  }
  flush_ds();

  if (key < lk) {
    const int64_t r = sg.k_row0 + key;
    uint16_t* dkp = a.dk.p + s * a.dk.sb + r * a.dk.sn + g * a.dk.sh;
    uint16_t* dvp = a.dv.p + s * a.dv.sb + r * a.dv.sn + g * a.dv.sh;
#pragma unroll
    for (int b = 0; b < NDB; ++b)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        elem4 v4;
#pragma unroll
        for (int c = 0; c < 4; ++c) v4[c] = (elem_t)(dka[b][rr * 4 + c] * a.scale);
        *reinterpret_cast<elem4*>(dkp + b * 32 + rr * 8 + half * 4) = v4;
      }
#pragma unroll
    for (int b = 0; b < NVB; ++b)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        elem4 v4;
#pragma unroll
        for (int c = 0; c < 4; ++c) v4[c] = (elem_t)dva[b][rr * 4 + c];
        *reinterpret_cast<elem4*>(dvp + b * 32 + rr * 8 + half * 4) = v4;
      }
  }
}

// ---------------------------------------------------------------------------
// dK / dV for head dims that need no split (Dqk = Dv <= 128), software
// pipelined: one workgroup = (segment, kv-head, 128 keys), four waves of 32
// keys. The workgroup's K and V rows stay in LDS for its whole life, so the
// registers hold only the dK^T/dV^T accumulators and two generations of the
// score tiles. Each iteration issues the S/dP MFMAs of query step it+1 and
// computes P/dS of step it between them (the matrix pipe and the vector ALU
// run at the same time), then accumulates dV^T/dK^T of step it.
// The score accumulators start from -lse/scale and -delta instead of zero:
// P = exp2(scale*log2(e)*acc) and dS = P*acc then need no per-row operands,
// and rows past the segment end (lse = +inf there) come out as P = 0.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256, 1) attn_bwd_dkdv_pipe_kernel(const BwdArgs a) {
  constexpr int NKS = D / 16, NDB = D / 32;
  constexpr int BQ = 32, BK = 128;
  constexpr int KS = D + 8;   // K/V rows: row-wise reads only
  constexpr int QS = D + 16;  // Q/dO rows: row-wise and transposing reads
  __shared__ __attribute__((aligned(16))) uint16_t sk[BK * KS];
  __shared__ __attribute__((aligned(16))) uint16_t sv[BK * KS];
  __shared__ __attribute__((aligned(16))) uint16_t sq[2][BQ * QS];
  __shared__ __attribute__((aligned(16))) uint16_t sdo[2][BQ * QS];
  __shared__ __attribute__((aligned(16))) float slse[2][BQ];  // -lse * log2(e) / (scale*log2(e))
  __shared__ __attribute__((aligned(16))) float sdel[2][BQ];  // -delta

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches
  const int col = lane & 31, half = lane >> 5;
  const int item = blockIdx.x / a.kvh_n, g = a.kvh0 + (blockIdx.x - item * a.kvh_n);
  if (item >= *a.count_k) return;
  const int2 st = a.items_k[item];
  const int s = st.x;
  const SegGeom sg = seg_geom(a.cu_q, a.cu_k, s, a.Nq, a.Nk, a.Tq, a.Tk);
  const int kb0 = st.y * BK;
  if (kb0 >= sg.lk) return;
  const int lq = sg.lq, lk = sg.lk, shift = lk - lq;
  const int gk0 = kb0 + w * 32;
  const int key = gk0 + col;
  // first query row that sees this lane's key (keys past the segment: none)
  const int qmin = key < lk ? (CAUSAL ? key - shift : INT_MIN) : INT_MAX;

  const uint16_t* kbp = a.k.p + s * a.k.sb + (int64_t)sg.k_row0 * a.k.sn + g * a.k.sh;
  const uint16_t* vbp = a.v.p + s * a.v.sb + (int64_t)sg.k_row0 * a.v.sn + g * a.v.sh;
  TileStage<BK, D, 256>::template copy<KS>(sk, kbp, a.k.sn, kb0, lk, tid);
  TileStage<BK, D, 256>::template copy<KS>(sv, vbp, a.v.sn, kb0, lk, tid);
  wait_global_loads();

  int q_begin = 0;
  if (CAUSAL) q_begin = max(0, kb0 - shift);
  q_begin &= ~(BQ - 1);
  const int nq = lq > q_begin ? (lq - q_begin + BQ - 1) / BQ : 0;
  const int total = a.G * nq;
  const float inv_c = 1.f / a.scale_log2;

  using QStage = TileStage<BQ, D, 256>;
  QStage qst, ost;
  float lse_r = 0.f, del_r = 0.f;
  bool row_ok = false;
  auto load_rows = [&](int it) {
    const int hh = it / nq;
    const int q0 = q_begin + (it - hh * nq) * BQ;
    const int h = g * a.G + hh;
    const uint16_t* qp = a.q.p + s * a.q.sb + (int64_t)sg.q_row0 * a.q.sn + h * a.q.sh;
    const uint16_t* dop = a.dout.p + s * a.dout.sb + (int64_t)sg.q_row0 * a.dout.sn + h * a.dout.sh;
    qst.load_clamped(qp, a.q.sn, q0, lq, tid);
    ost.load_clamped(dop, a.dout.sn, q0, lq, tid);
    if (tid < BQ) {
      const int64_t lb = s * a.lse_sb + h * a.lse_sh + sg.q_row0;
      const int i = min(q0 + tid, lq - 1);
      lse_r = a.lse[lb + i];
      del_r = a.delta[lb + i];
      row_ok = q0 + tid < lq;
    }
  };
  auto store_rows = [&](int b) {
    qst.template store<QS>(sq[b], tid);
    ost.template store<QS>(sdo[b], tid);
    if (tid < BQ) {
      // rows past the segment end or with lse = -inf: a seed whose product
      // with c is -inf (-inf / c carries the sign of c), so P = 0
      slse[b][tid] = (row_ok && lse_r != kNegInf) ? -lse_r * kLog2e * inv_c : kNegInf * inv_c;
      sdel[b][tid] = row_ok ? -del_r : 0.f;
    }
  };
  // score tiles of step in buffer b: C starts at -lse/c (S) and -delta (dP)
  auto scores = [&](int b, f32x16& sacc, f32x16& pacc) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(&slse[b][r4 * 8 + half * 4]);
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(&sdel[b][r4 * 8 + half * 4]);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        sacc[r4 * 4 + c] = l4[c];
        pacc[r4 * 4 + c] = d4[c];
      }
    }
#pragma unroll
    for (int i = 0; i < NKS; ++i) {
      sacc = mfma32(lds_frag(&sq[b][col * QS + half * 8 + i * 16]),
                    lds_frag(&sk[(w * 32 + col) * KS + half * 8 + i * 16]), sacc);
      pacc = mfma32(lds_frag(&sdo[b][col * QS + half * 8 + i * 16]),
                    lds_frag(&sv[(w * 32 + col) * KS + half * 8 + i * 16]), pacc);
    }
  };

  f32x16 dka[NDB], dva[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) {
    dka[i] = zero16();
    dva[i] = zero16();
  }
  f32x16 sacc, pacc;
  if (total > 0) {
    load_rows(0);
    store_rows(0);
    if (total > 1) load_rows(1);
    __syncthreads();
    scores(0, sacc, pacc);
  }

  for (int it = 0; it < total; ++it) {
    const int buf = it & 1, nb = buf ^ 1;
    const int q0 = q_begin + (it % nq) * BQ;
    __syncthreads();  // every wave is done with step it-1 (its buffer is nb)
    if (it + 1 < total) {
      store_rows(nb);
      if (it + 2 < total) load_rows(it + 2);
    }
    __syncthreads();  // step it+1 is visible
    // scores of step it+1 (its buffer holds stale rows after the last step;
    // those results are never used)
    f32x16 sacc_n, pacc_n;
    scores(nb, sacc_n, pacc_n);
    // P and dS of step it: rows q = q0 + 8*(r/4) + 4*half + r%4
    float p[16], dsv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qi = q0 + (r >> 2) * 8 + half * 4 + (r & 3);
      float x = fast_exp2(sacc[r] * a.scale_log2);
      x = qi >= qmin ? x : 0.f;
      p[r] = x;
      dsv[r] = x * pacc[r];
    }
    const frag8 p0 = to_frag(p), p1 = to_frag(p + 8);
    const frag8 s0 = to_frag(dsv), s1 = to_frag(dsv + 8);
    // dV^T[dv][key] += dO^T P ; dK^T[d][key] += Q^T dS
#pragma unroll
    for (int b = 0; b < NDB; ++b) {
      dva[b] = mfma32(tr_frag(sdo[buf], QS, 0, b * 32, lane), p0, dva[b]);
      dva[b] = mfma32(tr_frag(sdo[buf], QS, 16, b * 32, lane), p1, dva[b]);
      dka[b] = mfma32(tr_frag(sq[buf], QS, 0, b * 32, lane), s0, dka[b]);
      dka[b] = mfma32(tr_frag(sq[buf], QS, 16, b * 32, lane), s1, dka[b]);
    }
    sacc = sacc_n;
    pacc = pacc_n;
  }

  if (key < lk) {
    const int64_t r = sg.k_row0 + key;
    uint16_t* dkp = a.dk.p + s * a.dk.sb + r * a.dk.sn + g * a.dk.sh;
    uint16_t* dvp = a.dv.p + s * a.dv.sb + r * a.dv.sn + g * a.dv.sh;
#pragma unroll
    for (int b = 0; b < NDB; ++b)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        elem4 k4, v4;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          k4[c] = (elem_t)(dka[b][rr * 4 + c] * a.scale);
          v4[c] = (elem_t)dva[b][rr * 4 + c];
        }
        *reinterpret_cast<elem4*>(dkp + b * 32 + rr * 8 + half * 4) = k4;
        *reinterpret_cast<elem4*>(dvp + b * 32 + rr * 8 + half * 4) = v4;
      }
  }
}

// ---------------------------------------------------------------------------
// dQ: one workgroup = (segment, q-head, block of 32*NW queries). Per BN-key
// tile, K and V are staged row-major in two LDS buffers (the next tile's
// global loads issued a tile ahead into registers, or loaded straight into
// LDS at head dim 128); S^T = K Q^T and dP^T = V dO^T read them row-wise,
// dQ^T += K^T dS^T column-wise.
// ---------------------------------------------------------------------------
template <int DQK, int DV, int BN, int WPE, int NW, bool CAUSAL, bool EXT = false>
__global__ void __launch_bounds__(64 * NW, WPE) attn_bwd_dq_kernel(const BwdArgs a) {
  constexpr int NT = 64 * NW;
  constexpr int QG = NW;  // 32-query groups per workgroup
  static_assert(DQK % 32 == 0 && DV % 32 == 0 && BN % 32 == 0, "head dims");
  constexpr int NKS = DQK / 16, NVS = DV / 16, NDB = DQK / 32, NKB = BN / 32;
  // K is read both row-wise and through the transposing read: a stride of
  // 32 bytes mod 256 is the compromise (2-way on the row reads, none on the
  // transposing reads); V is only read row-wise (16 bytes mod 256).
  constexpr int KS = DQK + 16, VS = DV + 8;
  // Head dim 128 (32-key tiles): K and V tiles go straight from global
  // memory into LDS (global_load_lds) in the swizzled layout of rtile_off,
  // one tile ahead, instead of through registers.
  constexpr bool DMA = DQK == kTileD && DV == kTileD && BN == 32 && NW == 4;
  __shared__ __attribute__((aligned(1024))) uint16_t sk[2][DMA ? BN * kTileD : BN * KS];
  __shared__ __attribute__((aligned(1024))) uint16_t sv[2][DMA ? BN * kTileD : BN * VS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches
  const int col = lane & 31, half = lane >> 5;
  const int qg = w;  // this wave's 32-query group
  int item, h;
  xcd_item_head(blockIdx.x, a.Hq, a.G, item, h);
  const int g = h / a.G;
  if (item >= *a.count_q) return;
  const int2 st = a.items_q[item];
  const int s = st.x;
  const SegGeom sg = seg_geom(a.cu_q, a.cu_k, s, a.Nq, a.Nk, a.Tq, a.Tk);
  const int m0 = st.y * (32 * QG);
  if (m0 >= sg.lq) return;
  const int lq = sg.lq, lk = sg.lk, shift = lk - lq;
  const int wq0 = m0 + qg * 32;
  const int qi = wq0 + col;  // this lane's query (output column)
  const bool qok = qi < lq;

  const uint16_t* qbp = a.q.p + s * a.q.sb + (int64_t)sg.q_row0 * a.q.sn + h * a.q.sh;
  const uint16_t* dobp = a.dout.p + s * a.dout.sb + (int64_t)sg.q_row0 * a.dout.sn + h * a.dout.sh;
  const uint16_t* kbp = a.k.p + s * a.k.sb + (int64_t)sg.k_row0 * a.k.sn + g * a.k.sh;
  const uint16_t* vbp = a.v.p + s * a.v.sb + (int64_t)sg.k_row0 * a.v.sn + g * a.v.sh;

  int kv_end = lk;
  if (CAUSAL) kv_end = min(lk, m0 + 32 * QG + shift);
  const int ntiles = kv_end > 0 ? (kv_end + BN - 1) / BN : 0;
  // left window: key tiles wholly below the first row's window are skipped
  const int win = EXT && CAUSAL ? a.window : 0;
  const int t0 = win > 0 ? min(ntiles, max(0, m0 + shift - win + 1) / BN) : 0;
  const bool capped = EXT && a.cap_in != 0.f;

  frag8 qf[NKS], df[NVS];
  {
    const uint16_t* qp = qbp + (int64_t)(qok ? qi : 0) * a.q.sn + half * 8;
    const uint16_t* dp = dobp + (int64_t)(qok ? qi : 0) * a.dout.sn + half * 8;
#pragma unroll
    for (int i = 0; i < NKS; ++i) qf[i] = as_frag(qok ? ldg16(qp + i * 16) : zero_u32x4());
#pragma unroll
    for (int i = 0; i < NVS; ++i) df[i] = as_frag(qok ? ldg16(dp + i * 16) : zero_u32x4());
  }
  const int64_t lidx = s * a.lse_sb + h * a.lse_sh + sg.q_row0 + (qok ? qi : 0);
  // This pass runs first and computes delta = rowsum(dO * O) of its own
  // queries: a lane holds the dO elements {16i + 8*half .. +7} of its query
  // row, sums their products with the same elements of O, and adds the
  // partner lane's half. The row's delta and lse*log2(e) (+inf for lse = -inf,
  // so P = 0 on every key) are stored for the dK/dV pass that follows.
  float l2 = __builtin_inff(), dl = 0.f;
  {
    const uint16_t* op = a.o.p + s * a.o.sb + (int64_t)(sg.q_row0 + (qok ? qi : 0)) * a.o.sn +
                         h * a.o.sh + half * 8;
    u32x4 ov[NVS];
#pragma unroll
    for (int i = 0; i < NVS; ++i) ov[i] = qok ? ldg16(op + i * 16) : zero_u32x4();
    float l = kNegInf;
    if (qok) l = a.lse[lidx];
#pragma unroll
    for (int i = 0; i < NVS; ++i) {
      const u32x4 dv4 = __builtin_bit_cast(u32x4, df[i]);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        dl += elem_to_f(elem_at(ov[i], e)) * elem_to_f(elem_at(dv4, e));
    }
    dl += xor32(dl);
    if (qok) l2 = l == kNegInf ? __builtin_inff() : l * kLog2e;
    if (qok && half == 0) {
      a.delta[lidx] = dl;
      a.lse2[lidx] = l2;
    }
  }
  wait_global_loads();

  // DMA: wave w loads K and V rows 8w..8w+7 of a tile (2 loads each): load
  // jj covers rows 8w + 4jj + l/16; stored piece l%16 of row r holds global
  // piece (l%16) ^ 4*(r%4) ^ (r/4)%4 = p0 ^ ((2w + jj) % 4).
  const int dl4 = lane >> 4, p0 = (lane & 15) ^ (dl4 << 2);
  auto issue_kv = [&](int tt) {
    const int b = tt & 1, kt0 = tt * BN;
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int rr = min(kt0 + 8 * w + 4 * jj + dl4, lk - 1);  // past the end: its last row
      const int pc = (p0 ^ ((2 * w + jj) & 3)) * 8;
      dma16(kbp + (int64_t)rr * a.k.sn + pc, lds_ptr(&sk[b][(2 * w + jj) * 512]));
      dma16(vbp + (int64_t)rr * a.v.sn + pc, lds_ptr(&sv[b][(2 * w + jj) * 512]));
    }
  };

  using KStage = TileStage<BN, DQK, NT>;
  using VStage = TileStage<BN, DV, NT>;
  KStage kst;
  VStage vst;
  if constexpr (DMA) {
    if (t0 < ntiles) issue_kv(t0);
  } else if (t0 < ntiles) {
    const int b0 = t0 & 1;
    kst.load_clamped(kbp, a.k.sn, t0 * BN, lk, tid);
    vst.load_clamped(vbp, a.v.sn, t0 * BN, lk, tid);
    kst.template store<KS>(sk[b0], tid);
    vst.template store<VS>(sv[b0], tid);
    if (t0 + 1 < ntiles) {
      kst.load_clamped(kbp, a.k.sn, (t0 + 1) * BN, lk, tid);
      vst.load_clamped(vbp, a.v.sn, (t0 + 1) * BN, lk, tid);
    }
  }


  f32x16 dqa[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) dqa[i] = zero16();

  for (int t = t0; t < ntiles; ++t) {
    const int k0 = t * BN;
    const int buf = t & 1;
    if constexpr (DMA) wait_vmcnt<0>();  // this wave's share of tile t has landed
    __syncthreads();
    if constexpr (DMA) {
      if (t + 1 < ntiles) issue_kv(t + 1);
    } else if (t + 1 < ntiles) {
      kst.template store<KS>(sk[buf ^ 1], tid);
      vst.template store<VS>(sv[buf ^ 1], tid);
      if (t + 2 < ntiles) {
        kst.load_clamped(kbp, a.k.sn, k0 + 2 * BN, lk, tid);
        vst.load_clamped(vbp, a.v.sn, k0 + 2 * BN, lk, tid);
      }
    }
    const bool live = wq0 < lq && !(CAUSAL && k0 > wq0 + 31 + shift) &&
                      !(win > 0 && k0 + BN - 1 <= wq0 + shift - win);
    f32x16 sacc[NKB], pacc[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      sacc[kb] = zero16();
      pacc[kb] = zero16();
    }
    if (live) {
      // partial S^T[key][q] = K Q^T and dP^T[key][q] = V dO^T over this wave's d ranges
#pragma unroll
      for (int i = 0; i < NKS; ++i)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          sacc[kb] = mfma32(DMA ? rtile_row(sk[buf], kb * 32 + col, 2 * i + half)
                                : lds_frag(&sk[buf][(kb * 32 + col) * KS + half * 8 +
                                                    i * 16]),
                            qf[i], sacc[kb]);
#pragma unroll
      for (int i = 0; i < NVS; ++i)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          pacc[kb] = mfma32(DMA ? rtile_row(sv[buf], kb * 32 + col, 2 * i + half)
                                : lds_frag(&sv[buf][(kb * 32 + col) * VS + half * 8 +
                                                    i * 16]),
                            df[i], pacc[kb]);
      pipeline_mfma_reads<(NKS + NVS) * NKB, 4>();
    }
    if (live) {
      // rows past the segment end carry l2 = +inf (P = 0); the key mask is only
      // needed on tiles that cross the diagonal or the segment end
      // (one uniform branch picks a masked or an unmasked copy of the loop, so
      // the mask costs no per-element branch on the other tiles)
      const bool need_mask = k0 + BN > lk || (CAUSAL && k0 + BN - 1 > wq0 + shift) ||
                             (win > 0 && k0 <= wq0 + 31 + shift - win);
      frag8 sf[2 * NKB];
      auto softmax_grad = [&](auto masked) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          float dsv[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            // softcap: P from the capped score, dS times 1 - tanh^2
            float th = 0.f;
            if (EXT && capped) th = fast_tanh(a.cap_in * sacc[kb][r]);
            float p = fast_exp2((EXT && capped ? a.cap_out * th : sacc[kb][r] * a.scale_log2) - l2);
            if constexpr (decltype(masked)::value) {
              const int kj = k0 + kb * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
              bool vis = kj < lk;
              if (CAUSAL) vis = vis && kj <= qi + shift;
              if (EXT && win > 0) vis = vis && kj > qi + shift - win;
              p = vis ? p : 0.f;
            }
            dsv[r] = p * (pacc[kb][r] - dl);
            if (EXT && capped) dsv[r] *= 1.f - th * th;
          }
          sf[2 * kb] = to_frag(dsv);
          sf[2 * kb + 1] = to_frag(dsv + 8);
        }
      };
      if (need_mask) softmax_grad(std::true_type{});
      else softmax_grad(std::false_type{});
      // dQ^T[d][q] += K^T dS^T (K^T read down the K tile's columns)
#pragma unroll
      for (int kk = 0; kk < 2 * NKB; ++kk)
#pragma unroll
        for (int b = 0; b < NDB; ++b)
          dqa[b] = mfma32(DMA ? rtile_col(sk[buf], kk * 16, b * 32, lane)
                              : tr_frag(sk[buf], KS, kk * 16, b * 32, lane),
                          sf[kk], dqa[b]);
      pipeline_mfma_reads<2 * NKB * NDB, 4, 2>();
    }
  }

  if (qok) {
    uint16_t* dqp = a.dq.p + s * a.dq.sb + (int64_t)(sg.q_row0 + qi) * a.dq.sn + h * a.dq.sh;
#pragma unroll
    for (int b = 0; b < NDB; ++b)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        uint16_t* dst = dqp + b * 32 + rr * 8 + half * 4;
        float add[4] = {0.f, 0.f, 0.f, 0.f};
        if (a.dq_accumulate) {
          const u32x2 old = *reinterpret_cast<const u32x2*>(dst);
          add[0] = elem_lo_f(old[0]);
          add[1] = elem_hi_f(old[0]);
          add[2] = elem_lo_f(old[1]);
          add[3] = elem_hi_f(old[1]);
        }
        elem4 v4;
#pragma unroll
        for (int c = 0; c < 4; ++c) v4[c] = (elem_t)(dqa[b][rr * 4 + c] * a.scale + add[c]);
        *reinterpret_cast<elem4*>(dst) = v4;
      }
  }
}

// ---------------------------------------------------------------------------
// dQ from the stored dS blocks: dQ[q] = scale * sum_j dS[q,j] k_j, a plain
// block GEMM (no recomputation of S or dP). One workgroup = (segment, q-head,
// 32*NW queries), wave w owns the query tile of rows 32w..32w+31 and walks
// the key tiles it can see. Per 32-key tile the workgroup stages the K rows
// (row-major, row stride KS) once for all its waves, and each wave its own
// 32x32 dS block (rearranged to keys x queries) in LDS; dQ^T[d][q] +=
// K^T dS^T takes both
// operands through the transposing LDS read, so the contraction order (keys
// 4h..4h+3, 8+4h.. of every 16) matches on both sides. The pass is bound by
// the dS bytes it reads from HBM.
// ---------------------------------------------------------------------------
// Staged dS block in LDS ([key][query position], 64-byte rows): piece p of
// row r at position p ^ ds_swz(r).
__device__ __forceinline__ int ds_swz(int r) { return (r >> 2) & 3; }
// tr_frag's operand (query column n0 + l%32 with n0 = 0, key rows k0 + 4h + j
// and k0 + 8 + 4h + j) from a staged dS block: the four rows one transposing
// read covers per 32 lanes share the swizzle, so they still cover all banks.
__device__ __forceinline__ frag8 ds_frag(const uint16_t* X, int k0, int lane) {
  const int g = lane >> 4, s = lane & 15, h = lane >> 5;
  const int row = k0 + 4 * h + (s >> 2);
  const int c = 16 * (g & 1) + 4 * (s & 3);
  typedef __attribute__((address_space(3))) uint16_t lds_u16;
  const uint16_t* p0 = X + row * 32 + (((c >> 3) ^ ds_swz(row)) << 3) + (c & 7);
  const uint16_t* p1 = X + (row + 8) * 32 + (((c >> 3) ^ ds_swz(row + 8)) << 3) + (c & 7);
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)((lds_u16*)p0));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)((lds_u16*)p1));
  return __builtin_bit_cast(frag8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

template <int DQK, int NW, bool CAUSAL>
__global__ void __launch_bounds__(64 * NW, 1) attn_bwd_dq_ds_kernel(const BwdArgs a) {
  constexpr int NT = 64 * NW;
  constexpr int NDB = DQK / 32;
  constexpr int BQ = 32 * NW;
  // K is only read through the transposing read (4 rows x 32 bytes per
  // 16-lane group): a row stride of 64 bytes mod 256 keeps those rows on
  // distinct banks
  constexpr int KS = DQK + (((32 - DQK) % 128) + 128) % 128;
  constexpr int KCH = 32 * DQK / 8;       // 16-byte chunks of a K tile
  constexpr int KPT = (KCH + NT - 1) / NT;  // per thread
  static_assert((KS * 2) % 256 == 64, "K row stride");
  __shared__ __attribute__((aligned(16))) uint16_t sk[2][32 * KS];
  __shared__ __attribute__((aligned(16))) uint16_t sds[2][NW][32 * 32];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  int item, hl;
  xcd_item_head(blockIdx.x, a.ds_nh, a.G, item, hl);
  const int h = a.ds_h0 + hl, g = h / a.G;
  if (item >= *a.count_q) return;
  const int2 st = a.items_q[item];
  const int s = st.x;
  const SegGeom sg = seg_geom(a.cu_q, a.cu_k, s, a.Nq, a.Nk, a.Tq, a.Tk);
  const int m0 = st.y * BQ;
  if (m0 >= sg.lq) return;
  const int lq = sg.lq, lk = sg.lk, shift = lk - lq;
  const int wq0 = m0 + 32 * w;
  // key tiles this wave's queries see (the blocks the dK/dV pass stored) and
  // the workgroup's (its last live wave's); with a left window the tiles
  // below the wave's first row's window hold no stored block, and the
  // workgroup starts at its first wave's first tile
  auto tiles_upto = [&](int rows_end) {
    int kv_end = lk;
    if (CAUSAL) kv_end = min(lk, rows_end + shift);
    return kv_end > 0 ? min((kv_end + 31) >> 5, a.ds_mkt) : 0;
  };
  const int win = CAUSAL ? a.window : 0;
  auto first_tile = [&](int row0) { return win > 0 ? max(0, row0 + shift - win + 1) >> 5 : 0; };
  const int nkt_w = wq0 < lq ? tiles_upto(wq0 + 32) : 0;
  const int kf_w = first_tile(wq0);
  const int ntiles = tiles_upto(min(m0 + BQ, ((lq + 31) >> 5) << 5));
  const int tb = min(ntiles, first_tile(m0));
  const int64_t blk0 = ds_block(a, s, sg, h, wq0 < lq ? wq0 : m0, 0);  // key tile t at +1024 t
  const uint16_t* kbp = a.k.p + s * a.k.sb + (int64_t)sg.k_row0 * a.k.sn + g * a.k.sh;

  u32x4 kr[KPT], dr[2];
  auto load = [&](int t) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      // rows past the segment end read as zero (their dS is zero as well)
      const int c = min(tid + NT * i, KCH - 1);
      const int row = 32 * t + c / (DQK / 8);
      kr[i] = row < lk ? ldg16(kbp + (int64_t)row * a.k.sn + (c % (DQK / 8)) * 8) : zero_u32x4();
    }
    if (t >= kf_w && t < nkt_w && blk0 >= 0) {
      const uint16_t* b = a.ds + blk0 + 1024 * t;
      dr[0] = ldg16(b + 8 * lane);
      dr[1] = ldg16(b + 512 + 8 * lane);
    }
  };
  auto store = [&](int b) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = tid + NT * i;
      if (c < KCH) sts16(&sk[b][(c / (DQK / 8)) * KS + (c % (DQK / 8)) * 8], kr[i]);
    }
    // to keys x queries, row-major: lane l's fragment j goes to key l % 32,
    // query positions 16j + 8h .. +7 (queries in the order 0-3, 8-11, 4-7,
    // 12-15 of every 16), its 16-byte piece p of the 64-byte row at position
    // p ^ ds_swz(row): 16 consecutive rows writing one piece then cover all
    // 64 banks (rows of 64 bytes put four rows in one bank line)
    const int r = lane & 31, sw = ds_swz(r);
    uint16_t* row = &sds[b][w][r * 32];
    sts16(row + (((lane >> 5) ^ sw) << 3), dr[0]);
    sts16(row + (((2 + (lane >> 5)) ^ sw) << 3), dr[1]);
  };

  f32x16 acc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) acc[i] = zero16();
  dr[0] = dr[1] = zero_u32x4();
  if (tb < ntiles) {
    load(tb);
    store(tb & 1);
    if (tb + 1 < ntiles) load(tb + 1);
  }
  for (int t = tb; t < ntiles; ++t) {
    const int buf = t & 1;
    __syncthreads();  // tile t is in LDS; nobody still reads the other buffer
    if (t + 1 < ntiles) {
      store(buf ^ 1);
      if (t + 2 < ntiles) load(t + 2);
    }
    if (t >= kf_w && t < nkt_w && blk0 >= 0) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const frag8 bfr = ds_frag(sds[buf][w], 16 * ks, lane);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          acc[db] = mfma32(tr_frag(sk[buf], KS, 16 * ks, 32 * db, lane), bfr, acc[db]);
      }
    }
  }

  // lane -> query: block column position col holds query perm(col) (the
  // middle two 4-query groups of every 16 are swapped)
  const int qi = wq0 + ((col & ~12) | ((col & 4) << 1) | ((col & 8) >> 1));
  if (qi < lq) {
    uint16_t* dqp = a.dq.p + s * a.dq.sb + (int64_t)(sg.q_row0 + qi) * a.dq.sn + h * a.dq.sh;
#pragma unroll
    for (int b = 0; b < NDB; ++b)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        uint16_t* dst = dqp + b * 32 + rr * 8 + half * 4;
        float add[4] = {0.f, 0.f, 0.f, 0.f};
        if (a.dq_accumulate) {
          const u32x2 old = *reinterpret_cast<const u32x2*>(dst);
          add[0] = elem_lo_f(old[0]);
          add[1] = elem_hi_f(old[0]);
          add[2] = elem_lo_f(old[1]);
          add[3] = elem_hi_f(old[1]);
        }
        elem4 v4;
#pragma unroll
        for (int c = 0; c < 4; ++c) v4[c] = (elem_t)(acc[b][rr * 4 + c] * a.scale + add[c]);
        *reinterpret_cast<elem4*>(dst) = v4;
      }
  }
}

}  // namespace VCA_ELEM
}  // namespace vca
