// Forward kernel: fused S = scale * Q K^T -> online softmax -> O = P V, with
// out (bf16) and the fp32 natural-log log-sum-exp per query row.
//
// Operation (NeMo-Automodel "ffpa_attention" page, dense and varlen forward
// entries; "fa4" page overview for the bottom-right causal corner): query i of
// a segment with lq queries and lk keys sees keys j < lk with, when causal,
// j <= i + (lk - lq). A row that sees nothing gets out 0 and lse -inf.
//
// Work item: one workgroup = one (segment or batch, q-head, 128-row q tile);
// four 32-row query blocks, one per wave (head dims 64 to 256; 512 has
// attn_fwd_wide.hpp).
// Per key tile:
//   * K tile [BN][Dqk] and V tile [BN][Dv] row-major in LDS;
//   * each wave computes S^T = K Q^T with Q held in registers, so a lane owns
//     one query (its column) and the row max / row sum are lane-local except
//     for one exchange with the partner lane of the other wave half;
//   * softmax in base 2 with scale*log2(e) folded in; the running max is only
//     moved when it grows by more than 2^8 (lazy rescale, exact either way);
//   * O^T += V^T P^T takes the S^T accumulators directly as the B operand; the
//     V^T fragments come from the row-major V tile through the transposing
//     LDS read, in the key order the S^T registers hold.
#pragma once

#include "attn_common.hpp"

namespace vca {
namespace VCA_ELEM {

constexpr float kLazyRescale = 8.0f;  // log2 units

template <int DQK, int DV, int BN, int WPE, bool CAUSAL, int HPW = 1, bool EXT = false>
__global__ void __launch_bounds__(256 * HPW, WPE) attn_fwd_kernel(const FwdArgs a) {
  // K/V tiles are double-buffered in LDS (one barrier per tile); outside the
  // direct-load modes below, the next tile's global loads are issued a tile
  // ahead into registers and stored to LDS after the barrier.
  // HPW = 2 runs two q-heads of one GQA group over the same query rows (four
  // waves each): every K/V tile brought into LDS feeds both, half the tile
  // loads per unit of work, with the same causal work per wave.
  // EXT adds the left window (tiles below every row's window are skipped,
  // the window's edge masked) and the logit softcap (scores become
  // cap * tanh(scale * s / cap) before the softmax).
  static_assert(DQK % 16 == 0 && DV % 32 == 0 && BN % 32 == 0, "tile shape");
  constexpr int NT = 256 * HPW;  // threads
  // LDS row strides (elements). K is only read row-wise (b128 per lane, 16
  // lanes per LDS cycle): a stride of 16 bytes mod 256 puts 16 consecutive
  // rows on distinct banks. V is only read through the transposing read (4
  // rows x 32 bytes per 16-lane group): 64 bytes mod 256 keeps the two
  // groups served together on distinct banks.
  constexpr int KS = DQK + 8;
  constexpr int VS = DV + 32;
  constexpr int NKB = BN / 32;
  constexpr int NDB = DV / 32;
  constexpr int NKS = DQK / 16;
  // DMA mode (Dqk = Dv a multiple of 128, two buffers): K and V tiles go
  // straight from global memory into LDS (global_load_lds), one tile ahead,
  // with no staging through registers and no LDS stores. A tile is stored as
  // CB column blocks [CB][BN][128], each block in the swizzled 256-byte-row
  // layout of rtile_off. The tile's BN/4 * CB groups of 4 rows x 256 bytes
  // are split evenly over the waves, NG (a multiple of 4) per wave.
  constexpr int CB = DQK / kTileD;
  constexpr int NG = DQK % kTileD == 0 ? BN * CB / (4 * 4 * HPW) : 0;
  constexpr bool DMA = DQK == DV && DQK % kTileD == 0 && NG >= 1 &&
                       (NG % 4 == 0 || 4 % NG == 0) && NG * 4 * 4 * HPW == BN * CB;
  // Split-K DMA mode (Dqk = 192, Dv = 128): the same direct loads, with K
  // stored as a block of columns 0..127 in 256-byte rows (rtile_off) followed
  // by a block of columns 128..191 in 128-byte rows (r64_off), and V as one
  // block of 256-byte rows. Per wave and tile: BN/16 groups of 4 rows x 256
  // bytes of K's first block and of V, BN/32 groups of 8 rows x 128 bytes of
  // K's second block.
  constexpr bool SPLITK =
      DQK == 192 && DV == kTileD && HPW == 1 && BN % 32 == 0;
  constexpr bool LDMA = DMA || SPLITK;  // tiles land in LDS by global_load_lds
  static_assert(LDMA || HPW == 1, "head pairs load their tiles with global_load_lds");
  constexpr int KBLK = BN * kTileD;  // elements per column block of a DMA tile
  __shared__ __attribute__((aligned(1024))) uint16_t sk[2][LDMA ? BN * DQK : BN * KS];
  __shared__ __attribute__((aligned(1024))) uint16_t sv[2][LDMA ? BN * DV : BN * VS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches
  const int qg = w % 4;  // query block of this wave within its q-head
  const int col = lane & 31, half = lane >> 5;
  int item, h;
  xcd_item_head(blockIdx.x, a.H / HPW, a.G / HPW, item, h);
  h = h * HPW + w / 4;
  const int kvh = h / a.G;
  if (item >= *a.item_count) return;
  const int2 st = a.items[item];
  const int s = st.x, tile = st.y;
  const SegGeom sg = seg_geom(a.cu_q, a.cu_k, s, a.Nq, a.Nk, a.Tq, a.Tk);
  const int m0 = tile * kFwdBM;
  if (m0 >= sg.lq) return;
  const int lq = sg.lq, lk = sg.lk;
  const int shift = lk - lq;

  const uint16_t* qb = a.q.p + s * a.q.sb + (int64_t)sg.q_row0 * a.q.sn + h * a.q.sh;
  const uint16_t* kb = a.k.p + s * a.k.sb + (int64_t)sg.k_row0 * a.k.sn + kvh * a.k.sh;
  const uint16_t* vb = a.v.p + s * a.v.sb + (int64_t)sg.k_row0 * a.v.sn + kvh * a.v.sh;

  const int wrow0 = m0 + 32 * qg;  // first query row of this wave
  const int row = wrow0 + col;     // this lane's query row
  int kv_end = lk;
  if (CAUSAL) kv_end = min(lk, m0 + kFwdBM + shift);
  const int ntiles = kv_end > 0 ? (kv_end + BN - 1) / BN : 0;
  // left window: key tiles wholly below the first row's window are skipped
  const int win = EXT && CAUSAL ? a.window : 0;
  const int t0 = win > 0 ? min(ntiles, max(0, m0 + shift - win + 1) / BN) : 0;
  const bool capped = EXT && a.cap_in != 0.f;

  // Scores are kept unscaled until the exponent: the row max is taken over
  // raw q.k and scaled once, and exp2(sl2 * s - m) is one fma per element. A
  // negative scale is folded into Q instead (negating bf16 is exact), so the
  // factor sl2 applied to the scores is always positive.
  const float sl2 = fabsf(a.scale_log2);
  const uint32_t qsign = a.scale_log2 < 0.f ? 0x80008000u : 0u;
  frag8 qf[NKS];
  {
    const bool ok = row < lq;
    const uint16_t* src = qb + (int64_t)(ok ? row : 0) * a.q.sn + half * 8;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[ks] = as_frag((ok ? ldg16(src + ks * 16) : zero_u32x4()) ^ qsign);
  }
  wait_global_loads();

  // DMA: group g = NG*w + jj of a tile is rows 4*(g % (BN/4)) + l/16 of
  // column block g / (BN/4), at LDS element offset 512*g; stored piece l%16
  // of row r holds block piece (l%16) ^ 4*(r%4) ^ (r/4)%4 = p0 ^ (g%4).
  // A full tile is addressed as a uniform base (its first row of the group,
  // column block) plus one of KO per-lane byte offsets (row l/16, piece):
  // g%4 runs through jj%4 when NG is a multiple of 4, else through
  // (NG*w + jj)%4 for the wave's NG groups.
  constexpr int KO = NG % 4 == 0 ? 4 : (NG > 0 ? NG : 1);
  const int dl = lane >> 4, p0 = (lane & 15) ^ (dl << 2);
  uint32_t koff[KO], voff[KO];
#pragma unroll
  for (int j = 0; j < KO; ++j) {
    const int pc = p0 ^ ((NG * w + j) & 3);
    koff[j] = (uint32_t)(dl * a.k.sn + pc * 8) * 2u;
    voff[j] = (uint32_t)(dl * a.v.sn + pc * 8) * 2u;
  }
  auto issue_kv = [&](int tt) {
    const int b = tt & 1, kt0 = tt * BN;
    if (kt0 + BN <= lk) {
#pragma unroll
      for (int jj = 0; jj < NG; ++jj) {
        const int g = NG * w + jj;
        const int c = g / (BN / 4), r0 = kt0 + 4 * (g % (BN / 4));
        dma16s(kb + (int64_t)r0 * a.k.sn + c * kTileD, koff[jj % KO], lds_ptr(&sk[b][g * 512]));
        dma16s(vb + (int64_t)r0 * a.v.sn + c * kTileD, voff[jj % KO], lds_ptr(&sv[b][g * 512]));
      }
    } else {
      // the segment's last tile: rows past its end re-read its last row
#pragma unroll
      for (int jj = 0; jj < NG; ++jj) {
        const int g = NG * w + jj;
        const int c = g / (BN / 4), rr = min(kt0 + 4 * (g % (BN / 4)) + dl, lk - 1);
        const int pc = c * kTileD + (p0 ^ ((NG * w + jj) & 3)) * 8;
        dma16(kb + (int64_t)rr * a.k.sn + pc, lds_ptr(&sk[b][g * 512]));
        dma16(vb + (int64_t)rr * a.v.sn + pc, lds_ptr(&sv[b][g * 512]));
      }
    }
  };

  // split-K mode: tile tt into buffer tt & 1; the segment's last tile
  // re-reads its last row for rows past the end (those keys are masked)
  auto issue_split = [&](int tt) {
    const int b = tt & 1, kt0 = tt * BN;
    const bool full = kt0 + BN <= lk;
#pragma unroll
    for (int jj = 0; jj < BN / 16; ++jj) {
      const int g = (BN / 16) * w + jj;  // rows 4g..4g+3 of K's first block and of V
      const int r = kt0 + 4 * g + dl;
      const int rr = full ? r : min(r, lk - 1);
      const int pc = (p0 ^ (g & 3)) * 8;
      dma16(kb + (int64_t)rr * a.k.sn + pc, lds_ptr(&sk[b][g * 512]));
      dma16(vb + (int64_t)rr * a.v.sn + pc, lds_ptr(&sv[b][g * 512]));
    }
#pragma unroll
    for (int jj = 0; jj < BN / 32; ++jj) {
      const int g = (BN / 32) * w + jj;  // rows 8g..8g+7 of K's second block
      const int rl = 8 * g + (lane >> 3);
      const int rr = full ? kt0 + rl : min(kt0 + rl, lk - 1);
      const int pc = kTileD + ((lane & 7) ^ sw64(rl)) * 8;
      dma16(kb + (int64_t)rr * a.k.sn + pc, lds_ptr(&sk[b][KBLK + g * 512]));
    }
  };

  using KStage = TileStage<BN, DQK, NT>;
  using VStage = TileStage<BN, DV, NT>;
  KStage kst;
  VStage vst;
  if constexpr (DMA) {
    if (t0 < ntiles) issue_kv(t0);
  } else if constexpr (SPLITK) {
    if (t0 < ntiles) issue_split(t0);
  } else if (t0 < ntiles) {
    const int b0 = t0 & 1;
    kst.load_clamped(kb, a.k.sn, t0 * BN, lk, tid);
    vst.load_clamped(vb, a.v.sn, t0 * BN, lk, tid);
    kst.template store<KS>(sk[b0], tid);
    vst.template store<VS>(sv[b0], tid);
    if (t0 + 1 < ntiles) {
      kst.load_clamped(kb, a.k.sn, (t0 + 1) * BN, lk, tid);
      vst.load_clamped(vb, a.v.sn, (t0 + 1) * BN, lk, tid);
    }
  }

  f32x16 o[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) o[i] = zero16();
  float m_ref = kNegInf;  // base-2 running reference max of this row
  float lsum = 0.f;       // this lane half's share of the row sum

  for (int t = t0; t < ntiles; ++t) {
    const int k0 = t * BN;
    const int buf = t & 1;
    if constexpr (LDMA) wait_vmcnt<0>();  // this wave's share of tile t has landed
    __syncthreads();  // tile t is in LDS; nobody still reads the other buffer
    if constexpr (DMA) {
      if (t + 1 < ntiles) issue_kv(t + 1);
    } else if constexpr (SPLITK) {
      if (t + 1 < ntiles) issue_split(t + 1);
    } else if (t + 1 < ntiles) {
      kst.template store<KS>(sk[buf ^ 1], tid);
      vst.template store<VS>(sv[buf ^ 1], tid);
      if (t + 2 < ntiles) {
        kst.load_clamped(kb, a.k.sn, k0 + 2 * BN, lk, tid);
        vst.load_clamped(vb, a.v.sn, k0 + 2 * BN, lk, tid);
      }
    }
    const bool live = wrow0 < lq && !(CAUSAL && k0 > wrow0 + 31 + shift) &&
                      !(win > 0 && k0 + BN - 1 < wrow0 + shift - win + 1);

    // S^T = K Q^T
    f32x16 sacc[NKB];
#pragma unroll
    for (int kbk = 0; kbk < NKB; ++kbk) sacc[kbk] = zero16();
    if (live) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int kbk = 0; kbk < NKB; ++kbk)
          sacc[kbk] = mfma32(
              SPLITK ? (ks < kTileD / 16
                            ? rtile_row(&sk[buf][0], kbk * 32 + col, 2 * ks + half)
                            : r64_row(&sk[buf][KBLK], kbk * 32 + col, 2 * (ks - kTileD / 16) + half))
              : DMA ? rtile_row(&sk[buf][((ks * 16) / kTileD) * KBLK], kbk * 32 + col,
                                ((ks * 16) % kTileD) / 8 + half)
                    : lds_frag(&sk[buf][(kbk * 32 + col) * KS + half * 8 + ks * 16]),
              qf[ks], sacc[kbk]);
      pipeline_mfma_reads<NKS * NKB, 4>();
    }
    if (live) {
      // softcap first (a masked score must stay -inf): scores then hold
      // cap * tanh(scale * s / cap) in base-2 units, and the factor below is 1.
      // Then the mask (diagonal, window-edge and tail tiles only) and the row
      // max of the raw scores, scaled once (mul > 0; a fully masked row keeps
      // -inf)
      if constexpr (EXT) {
        if (capped) {
#pragma unroll
          for (int kbk = 0; kbk < NKB; ++kbk)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              sacc[kbk][r] = a.cap_out * fast_tanh(a.cap_in * sacc[kbk][r]);
        }
      }
      const float mul = capped ? 1.f : sl2;
      const bool need_mask = (k0 + BN > lk) || (CAUSAL && k0 + BN - 1 > wrow0 + shift) ||
                             (win > 0 && k0 < wrow0 + 31 + shift - win + 1);
      if (need_mask) {
#pragma unroll
        for (int kbk = 0; kbk < NKB; ++kbk)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + kbk * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
            bool vis = key < lk && (!CAUSAL || key <= row + shift);
            if (EXT && win > 0) vis = vis && key > row + shift - win;
            sacc[kbk][r] = vis ? sacc[kbk][r] : kNegInf;
          }
      }
      float mx = kNegInf;
#pragma unroll
      for (int kbk = 0; kbk < NKB; ++kbk)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kbk][r]);
      mx = fmaxf(mx, xor32(mx)) * mul;

      // lazy rescale of the running reference
      const float m_new = fmaxf(m_ref, mx);
      const bool need = m_new > m_ref + kLazyRescale;
      if (__any(need)) {
        const float m_set = need ? m_new : m_ref;
        const float alpha = need ? fast_exp2(m_ref - m_set) : 1.f;
        lsum *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
        m_ref = m_set;
      }
      const float m_use = m_ref == kNegInf ? 0.f : m_ref;

      // P = exp2(x - m), row sum, pack to bf16 fragments
      frag8 pf[2 * NKB];
#pragma unroll
      for (int kbk = 0; kbk < NKB; ++kbk) {
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          p[r] = fast_exp2(fmaf(sacc[kbk][r], mul, -m_use));
          lsum += p[r];
        }
        pf[2 * kbk] = to_frag(p);
        pf[2 * kbk + 1] = to_frag(p + 8);
      }

      // O^T += V^T P^T over this wave's Dv range (V^T read down V's columns)
#pragma unroll
      for (int kk = 0; kk < 2 * NKB; ++kk)
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          o[db] = mfma32(LDMA ? rtile_col(&sv[buf][((db * 32) / kTileD) * KBLK], kk * 16,
                                         (db * 32) % kTileD, lane)
                             : tr_frag(sv[buf], VS, kk * 16, db * 32, lane),
                         pf[kk], o[db]);
      pipeline_mfma_reads<2 * NKB * NDB, 4, 2>();
    }
  }

  // epilogue: O / l, lse = ln(sum exp(scaled scores))
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
