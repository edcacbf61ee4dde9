// dK / dV pass for Dqk = 192, Dv = 128 with split wave roles (NeMo-Automodel
// "ffpa_attention" page, dense and varlen backward entries; same quantities
// as the other backward kernels). The design of attn_bwd_dkdv_roles_kernel,
// widened to 192-element Q rows:
//
//   one workgroup = (segment, kv-head, 128 keys) = two wave pairs of 64
//   keys, one wave per SIMD; in a pair, wave A computes S -> P -> dV and
//   wave B dP -> dS -> dK, A hands P to B through LDS; each wave keeps its
//   64 keys' K (A, 192 columns) or V (B, 128 columns) rows in AGPRs as MFMA
//   B operands and its 64 x 128 dV (A) or 64 x 192 dK (B) fp32 accumulators
//   in AGPRs; Q, dO, lse*log2(e) and delta come straight from global memory
//   into a six-stage LDS ring three steps ahead.
//
// Wave A issues 24 score MFMAs (S over 192) and 16 product MFMAs (dV over 128
// columns) per iteration, wave B 16 (dP over 128) and 24 (dK over 192): 40
// each, paired one score with one product while both kinds last, with one
// softmax element after each of the first 32.
//
// A staged Q tile (12 KB) is a 32 x 128 block of head-dim columns 0..127 in
// the 256-byte-row swizzle of rtile_off, followed by a 32 x 64 block of
// columns 128..191 in 128-byte rows: piece u of row r sits at u ^ sw64(r),
// sw64(r) = 4*(x%2) + x/2 with x = (r/2) % 8. Two rows share one 256-byte
// bank line, so 16 consecutive rows reading one piece cover all 64 banks
// when sw64 is a permutation over each row parity (it is); the transposing
// read (4 rows x 4 pieces per 32 lanes) puts rows r and r+2 in different
// 4-piece halves (sw64 differs in bit 2 between them), so it is free of
// conflicts as well.
#pragma once

#include "attn_bwd_roles.hpp"

namespace vca {
namespace VCA_ELEM {

constexpr int kR2Dq = 192;                        // Q/K head dim
constexpr int kR2Dv = 128;                        // V/dO head dim
constexpr int kR2TileA = kRBQ * kTileD;           // Q columns 0..127 of a step
constexpr int kR2TileB = kRBQ * 64;               // Q columns 128..191
constexpr int kR2TileQ = kR2TileA + kR2TileB;     // 6144 elements (12 KB)

__device__ __forceinline__ void agpr_results_ready(f32x16 (&acc)[6][2]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(acc[0][0]), "+a"(acc[0][1]), "+a"(acc[1][0]), "+a"(acc[1][1]),
                 "+a"(acc[2][0]), "+a"(acc[2][1]), "+a"(acc[3][0]), "+a"(acc[3][1]),
                 "+a"(acc[4][0]), "+a"(acc[4][1]), "+a"(acc[5][0]), "+a"(acc[5][1]));
}

template <bool CAUSAL>
__global__ void __launch_bounds__(256, 1) attn_bwd_dkdv_roles_qk192_kernel(const BwdArgs a) {
  constexpr int KT = 2;           // 32-key tiles per wave
  constexpr int NW = 4;           // waves
  constexpr int NT = 64 * NW;     // threads
  constexpr int NP = NW / 2;      // wave pairs
  constexpr int KP = 32 * KT;     // keys per pair
  constexpr int NS = kRStages;    // Q/dO/lse/delta stages in LDS
  // hand-issued loads per wave and step: two 4-row slices of Q columns
  // 0..127 and one 8-row slice of columns 128..191; role 0 also its pair's
  // four 4-row slices of dO and the step's 32 lse*log2(e) and 32 delta
  // values (one load: lanes 0-31 and 32-63). Role 1 also stores the dS
  // blocks: the loads are split so both roles reach the barrier together.
  constexpr int NDMA_R0 = 8, NDMA_R1 = 3;
  __shared__ __attribute__((aligned(1024))) uint16_t sq[NS][kR2TileQ];
  __shared__ __attribute__((aligned(1024))) uint16_t sdo[NS][kRTile];
  // per pair: lse*log2(e) of the step's query rows 0-31, then their delta
  __shared__ __attribute__((aligned(256))) float sld[NS][NP][64];
  __shared__ __attribute__((aligned(16))) u32x4 sp[2][NP][KT][2][64];  // [parity][pair][kt][j][lane]

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 31, h = lane >> 5;
  const int pair = w >> 1, role = w & 1;  // role 0: S, P, dV; role 1: dP, dS, dK
  const int item = blockIdx.x / a.kvh_n, g = a.kvh0 + (blockIdx.x - item * a.kvh_n);
  if (item >= *a.count_k) return;
  const int2 st = a.items_k[item];
  const int s = st.x;
  const SegGeom sg = seg_geom(a.cu_q, a.cu_k, s, a.Nq, a.Nk, a.Tq, a.Tk);
  const int kb0 = st.y * kRBK;
  if (kb0 >= sg.lk) return;
  const int lq = sg.lq, lk = sg.lk, shift = lk - lq;
  const int kp0 = kb0 + pair * KP;  // first key of this wave pair

  int q_begin = 0;
  if (CAUSAL) q_begin = max(0, kb0 - shift);
  q_begin &= ~(kRBQ - 1);
  const int nq = lq > q_begin ? (lq - q_begin + kRBQ - 1) / kRBQ : 0;
  const int total = a.G * nq;

  // step it -> (q-head, first query), from the segment's end down with the
  // group's q-heads innermost (as in the head-dim-128 kernel)
  auto step_head = [&](int it) { return g * a.G + it % a.G; };
  auto step_q0 = [&](int it) { return q_begin + (nq - 1 - it / a.G) * kRBQ; };
  auto stage = [](int it) { return (it + NS) % NS; };

  // Per-lane parts of the hand-issued loads. Q columns 0..127 and dO: slice
  // j = 2w + j2 holds rows 4j..4j+3, lane l row 4j + l/16 at stored piece
  // l%16 (global piece l%16 ^ swizzle). Q columns 128..191: slice w holds
  // rows 8w..8w+7, lane l row 8w + l/8 at stored piece l%8 (global piece
  // (l%8) ^ sw64(row)).
  // (computed at each issue from a lane id the compiler cannot see through:
  // held across the loop they would take registers this kernel does not
  // have, and a reload from scratch waits for every load in flight)
  auto issue = [&](int it, auto role_c) {
    constexpr int R = decltype(role_c)::value;
    const int b = stage(it);
    const int hh = step_head(it), q0 = step_q0(it);
    const uint16_t* qb = a.q.p + s * a.q.sb + (int64_t)sg.q_row0 * a.q.sn + hh * a.q.sh;
    const uint16_t* db = a.dout.p + s * a.dout.sb + (int64_t)sg.q_row0 * a.dout.sn + hh * a.dout.sh;
    // rows past the segment's end (its last step) re-read its last row
    const bool tail = q0 + kRBQ > lq;
    int ln = lane;
    asm volatile("; lane" : "+v"(ln));
    // a 4-row slice sl of Q columns 0..127 or of dO: lane row 4*sl + l/16,
    // stored piece l%16 = global piece (l%16) ^ swizzle
    auto slice = [&](const uint16_t* base, int64_t sn, uint16_t* dst, int sl) {
      const int r = 4 * sl + (ln >> 4);
      const int qi = tail ? min(q0 + r, lq - 1) : q0 + r;
      const int pc = ((ln & 15) ^ (((r & 3) << 2) | ((r >> 2) & 3))) * 8;
      dma16(base + (int64_t)qi * sn + pc, lds_ptr(&dst[sl * 512]));
    };
#pragma unroll
    for (int j2 = 0; j2 < 2; ++j2) slice(qb, a.q.sn, sq[b], 2 * w + j2);
    if constexpr (R == 0) {
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) slice(db, a.dout.sn, sdo[b], 4 * pair + j4);
    }
    {
      const int brow = 8 * w + (ln >> 3);
      const int bpiece = kTileD + ((ln & 7) ^ sw64(brow)) * 8;
      const int qi = tail ? min(q0 + brow, lq - 1) : q0 + brow;
      dma16(qb + (int64_t)qi * a.q.sn + bpiece, lds_ptr(&sq[b][kR2TileA + w * 512]));
    }
    if constexpr (R == 0) {
      const int r = ln & 31;
      const int qi = tail ? min(q0 + r, lq - 1) : q0 + r;
      const float* src = (ln < 32 ? a.lse2 : a.delta) + s * a.lse_sb + sg.q_row0 + hh * a.lse_sh;
      dma4(src + qi, lds_ptr(&sld[b][pair][0]));
    }
  };

  // One wave role: R = 0 (K rows, S, P, dV) or 1 (V rows, dP, dS, dK). Each
  // role has its own fragment and accumulator counts, so it runs its own
  // copy of the kernel body (the same barriers in the same order).
  auto role_main = [&](auto role_c) {
    constexpr int R = decltype(role_c)::value;
    constexpr int NDMA = R == 0 ? NDMA_R0 : NDMA_R1;        // this role's loads per step
    constexpr int NKS = R == 0 ? kR2Dq / 16 : kR2Dv / 16;  // contraction steps of S / dP
    constexpr int NPB = R == 0 ? kR2Dv / 32 : kR2Dq / 32;  // 32-column blocks of dV / dK
    constexpr int NSC = NKS * KT, NPR = 2 * NPB * KT;
    constexpr int NOP = NSC > NPR ? NSC : NPR;
    static_assert(2 * (NSC < NPR ? NSC : NPR) >= 16 * KT, "every softmax element gets a slot");

    // K (role 0) or V (role 1) rows of this pair's keys as B fragments
    frag8 kf[KT][NKS];
    {
      const uint16_t* base = R == 0 ? a.k.p + s * a.k.sb + (int64_t)sg.k_row0 * a.k.sn + g * a.k.sh
                                    : a.v.p + s * a.v.sb + (int64_t)sg.k_row0 * a.v.sn + g * a.v.sh;
      const int64_t sn = R == 0 ? a.k.sn : a.v.sn;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        const int key = min(kp0 + 32 * kt + col, lk - 1);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
          kf[kt][ks] = in_agprs(as_frag(ldg16(base + key * sn + 16 * ks + 8 * h)));
      }
    }
    // The lagging products of the first iterations read Q of "steps" -2 and
    // -1 (stages NS-2, NS-1), dO and delta of step -1 and P parity 1 before
    // any load reaches them: those must hold zeros, not stale bits.
    {
      const u32x4 z = zero_u32x4();
      u32x4* q4 = reinterpret_cast<u32x4*>(&sq[NS - 2][0]);
      for (int i = tid; i < 2 * kR2TileQ / 8; i += NT) q4[i] = z;
      u32x4* d4 = reinterpret_cast<u32x4*>(&sdo[NS - 1][0]);
      for (int i = tid; i < kRTile / 8; i += NT) d4[i] = z;
      for (int i = tid; i < NP * 64; i += NT) (&sld[NS - 1][0][0])[i] = 0.f;
      u32x4* p1 = &sp[1][0][0][0][0];
      for (int i = tid; i < NP * KT * 2 * 64; i += NT) p1[i] = z;
    }
    wait_global_loads();

    // MFMA A operands: score steps (row reads of Q or dO) and product blocks
    // (transposing reads of dO or Q; f = 2*block + query half)
    auto srow = [&](const uint16_t* X, int ks) {
      if (R == 0 && ks >= kTileD / 16) return r64_row(X + kR2TileA, col, 2 * (ks - kTileD / 16) + h);
      return rtile_row(X, col, 2 * ks + h);
    };
    auto pcol = [&](const uint16_t* X, int f) {
      const int blk = f >> 1;
      if (R == 1 && blk >= kTileD / 32) return r64_col(X + kR2TileA, 16 * (f & 1), 32 * (blk - kTileD / 32), lane);
      return rtile_col(X, 16 * (f & 1), 32 * blk, lane);
    };

    f32x16 acc[NPB][KT];  // dV^T (role 0) or dK^T (role 1): [head-dim block][key tile]
#pragma unroll
    for (int d = 0; d < NPB; ++d)
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) acc[d][kt] = in_agprs(zero16());
    frag8 tf0[KT][2], tf1[KT][2];  // P (role 0) or dS (role 1) of two consecutive steps
    f32x16 sc0[KT], sc1[KT];       // S (role 0) or dP (role 1) of two consecutive steps
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      sc0[kt] = zero16();
      sc1[kt] = zero16();
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        tf0[kt][j] = as_frag(zero_u32x4());
        tf1[kt][j] = as_frag(zero_u32x4());
      }
    }

    // One iteration's MFMAs: slot c issues score MFMA c (fragment step c/KT,
    // key tile c%KT) and product MFMA c (fragment f = c/KT) while each kind
    // lasts, each followed by a softmax element while those last; fragments
    // are read two fragment steps ahead.
    auto pipe = [&](const uint16_t* Xs, f32x16 (&out)[KT], const uint16_t* Xp,
                    const frag8 (&T)[KT][2], auto&& valu) {
      frag8 af[NKS];
      frag8 cf[2 * NPB];
      af[0] = srow(Xs, 0);
      af[1] = srow(Xs, 1);
      cf[0] = pcol(Xp, 0);
      cf[1] = pcol(Xp, 1);
#pragma unroll
      for (int c = 0; c < NOP; ++c) {
        if (c < NSC) {
          const int ks = c / KT, kt = c % KT;
          if (kt == 0 && ks + 2 < NKS) af[ks + 2] = srow(Xs, ks + 2);
          if (ks == 0) mfma_v0(out[kt], af[0], kf[kt][0]);
          else mfma_v(out[kt], af[ks], kf[kt][ks]);
        }
        if (2 * c < 16 * KT) valu(2 * c);
        __builtin_amdgcn_sched_barrier(0);
        if (c < NPR) {
          const int f = c / KT, kt = c % KT;
          if (kt == 0 && f + 2 < 2 * NPB) cf[f + 2] = pcol(Xp, f + 2);
          mfma_a(acc[f >> 1][kt], cf[f], T[kt][f & 1]);
        }
        if (2 * c + 1 < 16 * KT) valu(2 * c + 1);
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    // Role 0, iteration i: S of step i+1 (into nxt) and dV of step i-1
    // (Pold), with P of step i from cur (into Pnew, and to role 1 via LDS).
    auto step_a = [&](int i, f32x16 (&cur)[KT], f32x16 (&nxt)[KT], frag8 (&Pold)[KT][2],
                      frag8 (&Pnew)[KT][2]) {
      const int q0 = step_q0(i);
      float l2[16];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int qo = 8 * rr + 4 * h;
        const f32x4 v = *reinterpret_cast<const f32x4*>(&sld[stage(i)][pair][qo]);
#pragma unroll
        for (int c = 0; c < 4; ++c) l2[4 * rr + c] = v[c];
      }
      float p[KT][16];
      pipe(sq[stage(i + 1)], nxt, sdo[stage(i - 1)], Pold, [&](int e) {
        const int kt = e >> 4, r = e & 15;
        p[kt][r] = fast_exp2(cur[kt][r] * a.scale_log2 - l2[r]);
      });
      // diagonal blocks and segment tails: zero what the mask hides (a
      // select: hidden entries may be inf); keys past the segment end get
      // P = 0 too (their dS must be zero in the stored blocks)
      if (q0 + kRBQ > lq || kp0 + KP > lk || (CAUSAL && kp0 + KP - 1 > q0 + shift)) {
        const int qh = q0 + 4 * h;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          const int key = kp0 + 32 * kt + col;
          const int kmin = key - shift;  // first query that sees the key
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int qi = qh + 8 * (r >> 2) + (r & 3);
            bool vis = qi < lq && key < lk;
            if (CAUSAL) vis = vis && qi >= kmin;
            p[kt][r] = vis ? p[kt][r] : 0.f;
          }
        }
      }
      const int par = i & 1;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          Pnew[kt][j] = to_frag(&p[kt][8 * j]);
          sp[par][pair][kt][j][lane] = __builtin_bit_cast(u32x4, Pnew[kt][j]);
        }
    };
    // Role 1, iteration i: dP of step i (into nxt) and dK of step i-2
    // (Dold), with dS of step i-1 from cur and role 0's P (into Dnew).
    auto step_b = [&](int i, f32x16 (&cur)[KT], f32x16 (&nxt)[KT], frag8 (&Dold)[KT][2],
                      frag8 (&Dnew)[KT][2]) {
      float dl[16];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int qo = 8 * rr + 4 * h;
        const f32x4 v = *reinterpret_cast<const f32x4*>(&sld[stage(i - 1)][pair][32 + qo]);
#pragma unroll
        for (int c = 0; c < 4; ++c) dl[4 * rr + c] = v[c];
      }
      const int par = (i + 1) & 1;  // parity of step i-1
      u32x4 pv[KT][2];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int j = 0; j < 2; ++j) pv[kt][j] = sp[par][pair][kt][j][lane];
      float d[KT][16];
      pipe(sdo[stage(i)], nxt, sq[stage(i - 2)], Dold, [&](int e) {
        const int kt = e >> 4, r = e & 15;
        const uint32_t wv = pv[kt][r >> 3][(r & 7) >> 1];
        const float pe = (r & 1 ? elem_hi_f(wv) : elem_lo_f(wv));
        d[kt][r] = pe * (cur[kt][r] - dl[r]);
      });
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int j = 0; j < 2; ++j) Dnew[kt][j] = to_frag(&d[kt][8 * j]);
    };
    // Role 1 after the barrier of iteration i, before the loads of step i+3:
    // the dS blocks of step i-2 its queries can see, for the dQ pass (the
    // next iteration's wait for step i+2's loads covers them).
    auto store_ds = [&](int i, const frag8 (&D)[KT][2]) {
      if (!a.ds || i < 2 || i - 2 >= total) return;
      const int q0 = step_q0(i - 2), hh = step_head(i - 2);
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        const int k0 = kp0 + 32 * kt;
        if (k0 < lk && (!CAUSAL || k0 <= q0 + kRBQ - 1 + shift)) {
          const int64_t off = ds_block(a, s, sg, hh, q0, k0);
          if (off >= 0) ds_store(a.ds + off, lane, D[kt][0], D[kt][1]);
        }
      }
    };

    // Prologue: steps 0..2 in flight; role 0 computes S of step 0.
    if (total > 0) issue(0, role_c);
    if (total > 1) issue(1, role_c);
    if (total > 2) issue(2, role_c);
    if (total > 2) wait_vmcnt<2 * NDMA>();
    else if (total > 1) wait_vmcnt<NDMA>();
    else wait_vmcnt<0>();
    __syncthreads();
    if (R == 0 && total > 0) {
      frag8 af[NKS];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) af[ks] = srow(sq[0], ks);
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        mfma_v0(sc0[kt], af[0], kf[kt][0]);
#pragma unroll
        for (int ks = 1; ks < NKS; ++ks) mfma_v(sc0[kt], af[ks], kf[kt][ks]);
      }
      mfma_results_ready(sc0[0], sc0[KT - 1]);
    }
    // Iteration i (0..total+1): wait for step i+1's loads, one barrier,
    // issue step i+3's. Role 0 works for i <= total (its dV lags one step),
    // role 1 for every i (its dK lags two).
    auto iteration = [&](int i, f32x16 (&cur)[KT], f32x16 (&nxt)[KT], frag8 (&Told)[KT][2],
                         frag8 (&Tnew)[KT][2]) {
      if (i + 2 < total) wait_vmcnt<NDMA>();
      else wait_vmcnt<0>();
      __syncthreads();
      if (R == 1) store_ds(i, Told);  // Told: dS of step i-2
      if (i + 3 < total) issue(i + 3, role_c);
      if (R == 0) {
        if (i <= total) step_a(i, cur, nxt, Told, Tnew);
      } else {
        step_b(i, cur, nxt, Told, Tnew);
      }
    };
    for (int i = 0; i <= total + 1; i += 2) {
      iteration(i, sc0, sc1, tf0, tf1);
      if (i + 1 <= total + 1) iteration(i + 1, sc1, sc0, tf1, tf0);
    }

    // dV (role 0) or dK * scale (role 1) of keys kp0 + 32*kt + l%32
    agpr_results_ready(acc);
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      const int key = kp0 + 32 * kt + col;
      if (key >= lk) continue;
      const int64_t r = sg.k_row0 + key;
      const float mul = R == 0 ? 1.f : a.scale;
      uint16_t* out = R == 0 ? a.dv.p + s * a.dv.sb + r * a.dv.sn + g * a.dv.sh
                             : a.dk.p + s * a.dk.sb + r * a.dk.sn + g * a.dk.sh;
#pragma unroll
      for (int d = 0; d < NPB; ++d)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          elem4 v4;
#pragma unroll
          for (int c = 0; c < 4; ++c) v4[c] = (elem_t)(acc[d][kt][4 * rr + c] * mul);
          *reinterpret_cast<elem4*>(out + 32 * d + 8 * rr + 4 * h) = v4;
        }
    }
  };
  if (role == 0) role_main(std::integral_constant<int, 0>{});
  else role_main(std::integral_constant<int, 1>{});
}

}  // namespace VCA_ELEM
}  // namespace vca
