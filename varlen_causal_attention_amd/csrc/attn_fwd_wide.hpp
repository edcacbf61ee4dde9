// Forward kernel for head dim 512 (Dqk = Dv = 512): the same operation, work
// items, outputs and rounding points as attn_fwd_kernel (NeMo-Automodel
// "ffpa_attention" page, dense and varlen forward entries; "fa4" page for the
// bottom-right causal corner), organised around a 32 x 512 output block per
// wave.
//
// Four waves, one per SIMD, 128 query rows per workgroup. A wave owns 32
// query rows with all 512 head-dim columns: its Q fragments stay in VGPRs
// (128 registers) and its 32 x 512 O^T accumulator in the accumulation
// registers (256), so no partial scores are exchanged between waves. With no
// second wave on the SIMD to fill the matrix pipe while the softmax runs, a
// wave pipelines its own work: iteration t issues the scores S of key tile
// t+1 and the product O^T += V^T P^T of tile t-1, interleaved one MFMA each,
// while the VALU computes the softmax of tile t between them. A running-max
// change found in the softmax of tile t (lazy rescale, as in the other
// forward) is applied to O after the product of tile t-1 has landed.
//
// K tiles are loaded two tiles ahead of their scores, V tiles one tile ahead
// of their product, straight from global memory into LDS (global_load_lds),
// one barrier per tile. One 64-lane load moves one whole 1 KB row, so the
// tiles keep padded row strides: K rows 16 bytes apart mod 256 (row-wise
// 16-byte reads of 16 consecutive rows hit distinct banks), V rows 64 bytes
// apart (the transposing reads of two 16-lane groups hit distinct banks), and
// every fragment address is a fixed offset from one per-lane base.
#pragma once

#include "attn_fwd.hpp"

namespace vca {
namespace VCA_ELEM {

constexpr int kWideD = 512;
constexpr int kWideBN = 32;  // keys per tile

template <bool CAUSAL, bool EXT = false>
__global__ void __launch_bounds__(256, 1) attn_fwd_wide_kernel(const FwdArgs a) {
  constexpr int D = kWideD, BN = kWideBN;
  constexpr int NKS = D / 16;        // contraction steps of S
  constexpr int NDB = D / 32;        // 32-column blocks of O^T
  constexpr int KS = D + 8;           // K row stride (elements)
  constexpr int VS = D + 32;          // V row stride (elements)
  constexpr int NSLOT = 2 * NKS;     // MFMA slots of a pipelined iteration
  constexpr int LEAD = 4;            // LDS fragments read ahead of their MFMA
  static_assert(2 * NDB * 2 == NSLOT, "one product MFMA per score MFMA");
  __shared__ __attribute__((aligned(1024))) uint16_t sk[2][BN * KS];
  __shared__ __attribute__((aligned(1024))) uint16_t sv[2][BN * VS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  int item, h;
  xcd_item_head(blockIdx.x, a.H, a.G, item, h);
  const int kvh = h / a.G;
  if (item >= *a.item_count) return;
  const int2 st = a.items[item];
  const int s = st.x, tile = st.y;
  const SegGeom sg = seg_geom(a.cu_q, a.cu_k, s, a.Nq, a.Nk, a.Tq, a.Tk);
  const int m0 = tile * kFwdBM;
  if (m0 >= sg.lq) return;
  const int lq = sg.lq, lk = sg.lk;
  const int shift = lk - lq;

  const int wrow0 = m0 + 32 * w;  // first query row of this wave
  const int row = wrow0 + col;    // this lane's query row
  int kv_end = lk;
  if (CAUSAL) kv_end = min(lk, m0 + kFwdBM + shift);
  const int ntiles = kv_end > 0 ? (kv_end + BN - 1) / BN : 0;
  // left window: the key tiles below the workgroup's first window are
  // skipped; the loads start at key kofs, every key index below is absolute
  const int win = EXT && CAUSAL ? a.window : 0;
  const int tb = win > 0 ? min(ntiles, max(0, m0 + shift - win + 1) / BN) : 0;
  const int kofs = tb * BN, lke = lk - kofs;
  const int nt = ntiles - tb;  // tiles the workgroup loads
  const bool capped = EXT && a.cap_in != 0.f;
  const float cin = a.scale_log2 < 0.f ? -a.cap_in : a.cap_in;

  const uint16_t* qb = a.q.p + s * a.q.sb + (int64_t)sg.q_row0 * a.q.sn + h * a.q.sh;
  const uint16_t* kb = a.k.p + s * a.k.sb + (int64_t)(sg.k_row0 + kofs) * a.k.sn + kvh * a.k.sh;
  const uint16_t* vb = a.v.p + s * a.v.sb + (int64_t)(sg.k_row0 + kofs) * a.v.sn + kvh * a.v.sh;

  // Q fragments of this lane's row (rows past the segment's end read its
  // first row: their results are never stored)
  frag8 qf[NKS];
  {
    const uint16_t* src = qb + (int64_t)(row < lq ? row : 0) * a.q.sn + half * 8;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[ks] = as_frag(ldg16(src + ks * 16));
  }
  wait_global_loads();

  // Wave w loads rows 8w .. 8w+7 of a tile into buffer tile%2, one row per
  // load (lane l: bytes 16l .. 16l+15); rows past the segment's end re-read
  // its last row.
  const uint32_t loff = (uint32_t)lane * 16u;
  const uint32_t lds_k = (uint32_t)(uintptr_t)lds_ptr(&sk[0][0]);
  const uint32_t lds_v = (uint32_t)(uintptr_t)lds_ptr(&sv[0][0]);
  auto issue = [&](const uint16_t* base, int64_t sn, uint32_t lds, int LS, int tt) {
    const int r0 = tt * BN + 8 * w;
    const uint16_t* p[8];
    uint32_t m[8];
    if (r0 + 8 <= lke) {
      p[0] = base + (int64_t)r0 * sn;
#pragma unroll
      for (int i = 1; i < 8; ++i) p[i] = p[i - 1] + sn;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) p[i] = base + (int64_t)min(r0 + i, lke - 1) * sn;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) m[i] = lds + (uint32_t)(((tt & 1) * BN + 8 * w + i) * LS * 2);
    dma16_rows8(p, loff, m);
  };

  // MFMA operands read from LDS. Score step ks: K rows (keys) as A. Product
  // step j = 16 kk + db: V^T of keys 16kk.. and columns 32db.. as A.
  auto kfrag = [&](const uint16_t* K, int ks) { return lds_frag(K + col * KS + ks * 16 + half * 8); };
  auto vfrag = [&](const uint16_t* V, int j) { return tr_frag(V, VS, (j >> 4) * 16, (j & 15) * 32, lane); };

  f32x16 o[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) o[i] = in_agprs(zero16());
  float m_ref = kNegInf;  // base-2 running reference max of this row
  float lsum = 0.f;       // this lane half's share of the row sum
  float alpha = 1.f;      // rescale of O found by the latest softmax
  bool rescale = false;

  // softmax of the scores of tile tt, in place (scale, mask, lazy max, exp2,
  // row sum, bf16 P^T fragments), split into steps so the pipelined iteration can
  // place one between MFMAs: steps 0-15 scale (or softcap) and mask, 16 the
  // row max, 17-32 exp2, 33-34 pack.
  float mx = kNegInf, m_use = 0.f;
  auto sm_step = [&](int c, f32x16& sc, int tt, frag8* pf) {
    if (c < 16) {
      const int r = c;
      const int key = kofs + tt * BN + (r >> 2) * 8 + half * 4 + (r & 3);
      bool vis = key < lk && (!CAUSAL || key <= row + shift);
      if (EXT && win > 0) vis = vis && key > row + shift - win;
      const float x = EXT && capped ? a.cap_out * fast_tanh(cin * sc[r]) : sc[r] * a.scale_log2;
      sc[r] = vis ? x : kNegInf;
      mx = c == 0 ? sc[r] : fmaxf(mx, sc[r]);
    } else if (c == 16) {
      mx = fmaxf(mx, xor32(mx));
      const float m_new = fmaxf(m_ref, mx);
      const bool need = m_new > m_ref + kLazyRescale;
      const float m_set = need ? m_new : m_ref;
      alpha = need ? fast_exp2(m_ref - m_set) : 1.f;
      rescale = need;
      lsum *= alpha;
      m_ref = m_set;
      m_use = m_ref == kNegInf ? 0.f : m_ref;
    } else if (c < 33) {
      const int r = c - 17;
      sc[r] = fast_exp2(sc[r] - m_use);
      lsum += sc[r];
    } else if (c < 35) {
      float e[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) e[i] = sc[8 * (c - 33) + i];
      pf[c - 33] = to_frag(e);
    }
  };
  auto softmax = [&](f32x16& sc, int tt, frag8* pf) {
#pragma unroll
    for (int c = 0; c < 35; ++c) sm_step(c, sc, tt, pf);
  };
  auto scores = [&](const uint16_t* K) {
    f32x16 sc = zero16();
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) sc = mfma32(kfrag(K, ks), qf[ks], sc);
    return sc;
  };
  auto product = [&](const uint16_t* V, const frag8* pf) {
#pragma unroll
    for (int j = 0; j < 2 * NDB; ++j) mfma_a(o[j & 15], vfrag(V, j), pf[j >> 4]);
  };
  // O *= alpha once the products that were in flight have landed
  auto apply_rescale = [&]() {
    if (__any(rescale)) {
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                   : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]), "+a"(o[5]),
                     "+a"(o[6]), "+a"(o[7]));
      asm volatile("s_nop 0"
                   : "+a"(o[8]), "+a"(o[9]), "+a"(o[10]), "+a"(o[11]), "+a"(o[12]), "+a"(o[13]),
                     "+a"(o[14]), "+a"(o[15]));
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        f32x16 v = o[db];
#pragma unroll
        for (int r = 0; r < 16; ++r) v[r] *= alpha;
        o[db] = in_agprs(v);
      }
    }
    rescale = false;
  };

  // Every wave runs every tile the workgroup loads: a tile a row does not see
  // is fully masked, so its P is exactly zero and it changes neither O, the
  // row sum nor the running max. One code path keeps O in place in the
  // accumulation registers.
  f32x16 s_cur = zero16();
  frag8 pf_prev[2], pf_cur[2];
  if (nt > 0) {
    issue(kb, a.k.sn, lds_k, KS, 0);
    if (nt > 1) issue(kb, a.k.sn, lds_k, KS, 1);
    wait_vmcnt<0>();
    __syncthreads();
    s_cur = scores(&sk[0][0]);
    // t = 0: the softmax of tile 0 and the scores of tile 1 (no product yet;
    // O is still zero, so a max change needs no rescale of O)
    wait_vmcnt<0>();
    __syncthreads();
    if (nt > 2) issue(kb, a.k.sn, lds_k, KS, 2);
    issue(vb, a.v.sn, lds_v, VS, 0);
    softmax(s_cur, 0, pf_cur);
    if (nt > 1) s_cur = scores(&sk[1][0]);
    rescale = false;
    pf_prev[0] = pf_cur[0];
    pf_prev[1] = pf_cur[1];
  }
  for (int t = 1; t < nt; ++t) {
    wait_vmcnt<0>();  // this wave's share of K tile t+1 and V tile t-1 has landed
    __syncthreads();  // everyone's; nobody still reads K tile t or V tile t-2
    // loads of K tile t+2 and V tile t: one row after each of the first 16
    // products, so the memory pipe's queue never stalls the MFMA stream (past
    // the last tile the K loads re-read the segment's last row into the free
    // buffer)
    const int rk0 = (t + 2) * BN + 8 * w, rv0 = t * BN + 8 * w;
    const uint32_t mk0 = lds_k + (uint32_t)(((t & 1) * BN + 8 * w) * KS * 2);
    const uint32_t mv0 = lds_v + (uint32_t)(((t & 1) * BN + 8 * w) * VS * 2);
    // S of tile t+1 (even slots; on the last tile it reads a stale buffer and
    // is discarded) and O += V^T P^T of tile t-1 (odd slots), the softmax of
    // tile t between them
    const uint16_t* Kn = &sk[(t + 1) & 1][0];
    const uint16_t* Vp = &sv[(t + 1) & 1][0];
    f32x16 s_next = zero16();
    frag8 fr[NSLOT];
#pragma unroll
    for (int c = 0; c < LEAD; ++c) fr[c] = (c & 1) ? vfrag(Vp, c >> 1) : kfrag(Kn, c >> 1);
#pragma unroll
    for (int c = 0; c < NSLOT; ++c) {
      if (c + LEAD < NSLOT)
        fr[c + LEAD] = ((c + LEAD) & 1) ? vfrag(Vp, (c + LEAD) >> 1) : kfrag(Kn, (c + LEAD) >> 1);
      if (c & 1) {
        mfma_a(o[(c >> 1) & 15], fr[c], pf_prev[c >> 5]);
        const int j = c >> 1, i = j & 7;
        if (j < 8)
          dma16m(kb + (int64_t)min(rk0 + i, lke - 1) * a.k.sn, loff, mk0 + (uint32_t)(i * KS * 2));
        else if (j < 16)
          dma16m(vb + (int64_t)min(rv0 + i, lke - 1) * a.v.sn, loff, mv0 + (uint32_t)(i * VS * 2));
      } else {
        s_next = mfma32(fr[c], qf[c >> 1], s_next);
      }
      sm_step(c, s_cur, t, pf_cur);
      __builtin_amdgcn_sched_barrier(0);
    }
    s_cur = s_next;
    apply_rescale();
    pf_prev[0] = pf_cur[0];
    pf_prev[1] = pf_cur[1];
  }
  if (nt > 0) {
    wait_vmcnt<0>();
    __syncthreads();  // V tile nt-1 is in LDS
    product(&sv[(nt - 1) & 1][0], pf_prev);
  }

  // epilogue: O / l, lse = ln(sum exp(scaled scores))
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]), "+a"(o[5]),
                 "+a"(o[6]), "+a"(o[7]));
  asm volatile("s_nop 0"
               : "+a"(o[8]), "+a"(o[9]), "+a"(o[10]), "+a"(o[11]), "+a"(o[12]), "+a"(o[13]),
                 "+a"(o[14]), "+a"(o[15]));
  const float ltot = lsum + xor32(lsum);
  if (row < lq) {
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    uint16_t* ob = a.o.p + s * a.o.sb + (int64_t)(sg.q_row0 + row) * a.o.sn + h * a.o.sh;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        elem4 v4;
#pragma unroll
        for (int c = 0; c < 4; ++c) v4[c] = (elem_t)(o[db][rr * 4 + c] * inv);
        *reinterpret_cast<elem4*>(ob + db * 32 + rr * 8 + half * 4) = v4;
      }
    }
    if (half == 0) {
      const float l = ltot > 0.f ? (m_ref + log2f(ltot)) * kLn2 : kNegInf;
      a.lse[s * a.lse_sb + h * a.lse_sh + sg.q_row0 + row] = l;
    }
  }
}

}  // namespace VCA_ELEM
}  // namespace vca
