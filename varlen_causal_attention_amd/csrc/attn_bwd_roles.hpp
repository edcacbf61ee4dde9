// dK / dV pass for head dim 128 (Dqk = Dv = 128) with split wave roles
// (NeMo-Automodel "ffpa_attention" page, dense and varlen backward entries;
// same quantities as the other backward kernels):
//
//   P  = exp(scale * Q K^T - lse),  dV += P^T dO
//   dS = P * (dO V^T - delta),      dK += scale * dS^T Q
//
// One workgroup = (segment, kv-head, 128 keys): two wave pairs of 64 keys.
// In a pair, wave A computes S -> P -> dV and wave B computes dP -> dS -> dK;
// A hands P to B through LDS. Each wave keeps its 64 keys' K (A) or V (B)
// rows in registers as MFMA operands for the whole kernel, and its 64 x 128
// dV (A) or dK (B) accumulators in the accumulation registers. So a Q or dO
// fragment read from LDS feeds two MFMAs (one per 32-key half), half the LDS
// traffic per MFMA of one wave doing all four products for 32 keys.
//
// The workgroup walks every (q-head of the GQA group, 32-query step) that
// can see its keys. Q, dO, lse*log2(e) and delta of a step are loaded
// straight from global memory into LDS three steps ahead (six stages). Each
// iteration issues 32 MFMAs per wave, one VALU element of the softmax work
// after each: wave A runs S of step i+1 and dV of step i-1 while it computes
// P of step i (exp of S of step i); wave B runs dP of step i and dK of step
// i-2 while it computes dS of step i-1 (P of step i-1 arrives from A across
// the iteration's single barrier). The matrix pipe and the VALU stay busy
// together instead of taking turns.
#pragma once

#include "attn_bwd.hpp"

namespace vca {
namespace VCA_ELEM {

constexpr int kRD = kTileD;           // head dim
constexpr int kRBQ = 32;              // queries per step
constexpr int kRKP = 64;              // keys per wave pair
constexpr int kRBK = 2 * kRKP;        // keys per workgroup
constexpr int kRStages = 6;           // Q/dO/lse/delta stages in LDS
constexpr int kRTile = kRBQ * kRD;    // elements of one staged Q or dO tile (8 KB)

// gfx950 direct global -> LDS load of one dword per lane (lane l's 4 bytes
// land at lds_base + 4*l); same contract as dma16.
__device__ __forceinline__ void dma4(const float* g, lds_void* lds_base) {
  uint32_t saved;
  const uint32_t m0 = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %1, off\n\t"
      "s_nop 0\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(g), "s"(m0)
      : "memory");
}

// The S / dP products, the dV / dK accumulation and the AGPR helpers are the
// hand-written MFMAs of attn_common.hpp (mfma_v0, mfma_v, mfma_a, in_agprs):
// the K/V fragments (B operands of S / dP) and the 64x128 dV/dK
// accumulators live in the accumulation registers, leaving the VGPRs to the
// score tiles, staged fragments and softmax.
// The accumulators are in/out operands, so their reads stay below the wait.
__device__ __forceinline__ void agpr_results_ready(f32x16 (&acc)[4][2]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(acc[0][0]), "+a"(acc[0][1]), "+a"(acc[1][0]), "+a"(acc[1][1]),
                 "+a"(acc[2][0]), "+a"(acc[2][1]), "+a"(acc[3][0]), "+a"(acc[3][1]));
}
__device__ __forceinline__ void agpr_results_ready(f32x16 (&acc)[4][1]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(acc[0][0]), "+a"(acc[1][0]), "+a"(acc[2][0]), "+a"(acc[3][0]));
}
// KT: 32-key tiles per wave (2: four waves, one per SIMD; 1: eight waves,
// two per SIMD, whose softmax work then overlaps the other wave's MFMAs).
template <bool CAUSAL, int KT>
__global__ void __launch_bounds__(512 / KT, 1) attn_bwd_dkdv_roles_kernel(const BwdArgs a) {
  constexpr int NKS = kRD / 16;  // contraction steps of S / dP
  constexpr int NDB = kRD / 32;  // 32-wide head-dim blocks of dV / dK
  constexpr int NW = 8 / KT;     // waves
  constexpr int NT = 64 * NW;    // threads
  constexpr int NP = NW / 2;     // wave pairs
  constexpr int KP = 32 * KT;    // keys per pair
  constexpr int SPW = 8 / NW;    // Q (and dO) four-row slices per wave and step
  // hand-issued loads per wave and step: SPW slices of Q and of dO, and in
  // role 0 the step's 32 lse*log2(e) and 32 delta values (one load)
  constexpr int NDMA_R0 = 2 * SPW + 1, NDMA_R1 = 2 * SPW;
  constexpr int NS = kRStages;
  __shared__ __attribute__((aligned(1024))) uint16_t sq[NS][kRTile];
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

  // this wave's K (role 0) or V (role 1) rows as B fragments (kept in AGPRs):
  // kf[kt][ks] = row kp0 + 32*kt + l%32, head-dim elements 16*ks + 8*h ..+7
  frag8 kf[KT][NKS];
  {
    // field-wise selects (a runtime select of a whole View goes to scratch)
    const uint16_t* base = (role == 0 ? a.k.p : a.v.p) + s * (role == 0 ? a.k.sb : a.v.sb) +
                           (int64_t)sg.k_row0 * (role == 0 ? a.k.sn : a.v.sn) +
                           g * (role == 0 ? a.k.sh : a.v.sh);
    const int64_t sn = role == 0 ? a.k.sn : a.v.sn;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      const int key = min(kp0 + 32 * kt + col, lk - 1);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        kf[kt][ks] = in_agprs(as_frag(ldg16(base + key * sn + 16 * ks + 8 * h)));
    }
  }
  // The lagging products of the first iterations read Q of "steps" -2 and -1
  // (stages NS-2, NS-1), dO and delta of step -1 and P parity 1 before any
  // load reaches them: those must hold zeros, not stale bits (stage NS-2's
  // first load is issued after the first barrier).
  {
    const u32x4 z = zero_u32x4();
    u32x4* q4 = reinterpret_cast<u32x4*>(&sq[NS - 2][0]);
    for (int i = tid; i < 2 * kRTile / 8; i += NT) q4[i] = z;
    u32x4* d4 = reinterpret_cast<u32x4*>(&sdo[NS - 1][0]);
    for (int i = tid; i < kRTile / 8; i += NT) d4[i] = z;
    for (int i = tid; i < NP * 64; i += NT) (&sld[NS - 1][0][0])[i] = 0.f;
    u32x4* p1 = &sp[1][0][0][0][0];
    for (int i = tid; i < NP * KT * 2 * 64; i += NT) p1[i] = z;
  }
  wait_global_loads();

  // step it -> (q-head, first query); stage of step it (it >= -2). Query
  // steps run from the segment's end down, the group's q-heads innermost:
  // every key block of a segment starts on the same Q/dO tiles and walks
  // them in lockstep until it reaches its own first visible query, so the
  // workgroups sharing a tile read it from L2 at about the same time.
  auto step_head = [&](int it) { return g * a.G + it % a.G; };
  auto step_q0 = [&](int it) { return q_begin + (nq - 1 - it / a.G) * kRBQ; };
  auto stage = [](int it) { return (it + NS) % NS; };
  // Hand-issued loads of step it: SPW of the Q tile's 8 four-row slices and
  // SPW of dO's, and in role 0 the step's lse*log2(e) and delta values. Lane
  // l of slice j loads row 4j + l/16, stored piece l%16 (global piece l%16 ^
  // swizzle).
  int srow[SPW], spiece[SPW];
  int64_t qoff[SPW], doff[SPW];
#pragma unroll
  for (int j2 = 0; j2 < SPW; ++j2) {
    const int r = 4 * (SPW * w + j2) + (lane >> 4);
    srow[j2] = r;
    spiece[j2] = ((lane & 15) ^ (((r & 3) << 2) | ((r >> 2) & 3))) * 8;
    qoff[j2] = (int64_t)r * a.q.sn + spiece[j2];
    doff[j2] = (int64_t)r * a.dout.sn + spiece[j2];
  }
  auto issue = [&](int it, auto role_c) {
    constexpr int R = decltype(role_c)::value;
    const int b = stage(it);
    const int hh = step_head(it), q0 = step_q0(it);
    const uint16_t* qb = a.q.p + s * a.q.sb + (int64_t)sg.q_row0 * a.q.sn + hh * a.q.sh;
    const uint16_t* db = a.dout.p + s * a.dout.sb + (int64_t)sg.q_row0 * a.dout.sn + hh * a.dout.sh;
    if (q0 + kRBQ <= lq) {
      const uint16_t* qs = qb + (int64_t)q0 * a.q.sn;
      const uint16_t* ds = db + (int64_t)q0 * a.dout.sn;
#pragma unroll
      for (int j2 = 0; j2 < SPW; ++j2) {
        dma16(qs + qoff[j2], lds_ptr(&sq[b][(SPW * w + j2) * 512]));
        dma16(ds + doff[j2], lds_ptr(&sdo[b][(SPW * w + j2) * 512]));
      }
      if constexpr (R == 0)
        dma4((lane < 32 ? a.lse2 : a.delta) + s * a.lse_sb + sg.q_row0 + hh * a.lse_sh + q0 +
                 (lane & 31),
             lds_ptr(&sld[b][pair][0]));
    } else {
      // last step of the segment: rows past its end re-read its last row
#pragma unroll
      for (int j2 = 0; j2 < SPW; ++j2) {
        const int qi = min(q0 + srow[j2], lq - 1);
        dma16(qb + (int64_t)qi * a.q.sn + spiece[j2], lds_ptr(&sq[b][(SPW * w + j2) * 512]));
        dma16(db + (int64_t)qi * a.dout.sn + spiece[j2], lds_ptr(&sdo[b][(SPW * w + j2) * 512]));
      }
      if constexpr (R == 0)
        dma4((lane < 32 ? a.lse2 : a.delta) + s * a.lse_sb + sg.q_row0 + hh * a.lse_sh +
                 min(q0 + (lane & 31), lq - 1),
             lds_ptr(&sld[b][pair][0]));
    }
  };

  f32x16 acc[NDB][KT];  // dV^T (role 0) or dK^T (role 1): [head-dim block][key tile]
#pragma unroll
  for (int d = 0; d < NDB; ++d)
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) acc[d][kt] = in_agprs(zero16());
  // P (role 0) or dS (role 1) fragments [kt][j] of two consecutive steps
  frag8 tf0[KT][2], tf1[KT][2];
  // score tiles S (role 0) or dP (role 1) of two consecutive steps
  f32x16 sc0[KT], sc1[KT];
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

  // One iteration's 32 MFMAs: 16 of a score tile out = Xs K^T (8 head-dim
  // steps x 2 key halves) and 16 of the product acc += Xp^T T (4 head-dim
  // blocks x 2 query halves x 2 key halves), alternating, each followed by
  // one VALU element valu(e), e = 0..31. Fragments are read two MFMA pairs
  // ahead; sched_barrier pins the interleave.
  auto pipe = [&](const uint16_t* Xs, f32x16 (&out)[KT], const uint16_t* Xp,
                  const frag8 (&T)[KT][2], auto&& valu) {
    frag8 af[NKS];
    frag8 cf[2 * NDB];
    af[0] = rtile_row(Xs, col, h);
    af[1] = rtile_row(Xs, col, 2 + h);
    cf[0] = rtile_col(Xp, 0, 0, lane);
    cf[1] = rtile_col(Xp, 16, 0, lane);
#pragma unroll
    for (int c = 0; c < 8 * KT; ++c) {
      const int ks = c / KT, kt = c % KT, f = c / KT;  // f = 2*d + j
      if (kt == 0 && ks + 2 < NKS) af[ks + 2] = rtile_row(Xs, col, 2 * (ks + 2) + h);
      if (kt == 0 && f + 2 < 2 * NDB)
        cf[f + 2] = rtile_col(Xp, 16 * ((f + 2) & 1), 32 * ((f + 2) >> 1), lane);
      if (ks == 0) mfma_v0(out[kt], af[0], kf[kt][0]);
      else mfma_v(out[kt], af[ks], kf[kt][ks]);
      valu(2 * c);
      __builtin_amdgcn_sched_barrier(0);
      mfma_a(acc[f >> 1][kt], cf[f], T[kt][f & 1]);
      valu(2 * c + 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Role 0, iteration i: S of step i+1 (into nxt) and dV of step i-1 (Pold),
  // with P of step i from cur (into Pnew, and to role 1 through LDS).
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
    const uint16_t* Xs = sq[stage(i + 1)];  // stale past the last step: unused
    const uint16_t* Xp = sdo[stage(i - 1)];
    pipe(Xs, nxt, Xp, Pold, [&](int e) {
      const int kt = e >> 4, r = e & 15;
      p[kt][r] = fast_exp2(cur[kt][r] * a.scale_log2 - l2[r]);
    });
    // diagonal blocks and segment tails (a few steps per key block): zero
    // what the mask hides (a select: hidden entries may be inf, e.g. on rows
    // with lse = -inf). Keys past the segment end (their K rows repeat its
    // last key) get P = 0 too: their dS must be zero in the stored blocks.
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
  // Role 1, iteration i: dP of step i (into nxt) and dK of step i-2 (Dold),
  // with dS of step i-1 from cur and role 0's P (into Dnew).
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
  // Role 1 at the top of iteration i (after the barrier, before the loads of
  // step i+3): the dS blocks of step i-2 that its queries can see, for the dQ
  // pass. Issued ahead of those loads, the stores are covered by the next
  // iteration's wait for the loads of step i+2 (loads complete in order), a
  // full iteration later, so the hand-counted waits never stall on them.
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
  auto prologue = [&](auto role_c) {
    constexpr int N = decltype(role_c)::value == 0 ? NDMA_R0 : NDMA_R1;
    if (total > 0) issue(0, role_c);
    if (total > 1) issue(1, role_c);
    if (total > 2) issue(2, role_c);
    if (total > 2) wait_vmcnt<2 * N>();
    else if (total > 1) wait_vmcnt<N>();
    else wait_vmcnt<0>();
  };
  if (role == 0) prologue(std::integral_constant<int, 0>{});
  else prologue(std::integral_constant<int, 1>{});
  __syncthreads();
  if (role == 0 && total > 0) {
    frag8 af[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) af[ks] = rtile_row(sq[0], col, 2 * ks + h);
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      mfma_v0(sc0[kt], af[0], kf[kt][0]);
#pragma unroll
      for (int ks = 1; ks < NKS; ++ks) mfma_v(sc0[kt], af[ks], kf[kt][ks]);
    }
    mfma_results_ready(sc0[0], sc0[KT - 1]);
  }
  // Iteration i (0..total+1): wait for step i+1's loads, one barrier, issue
  // step i+3's. Role 0 works for i <= total (its dV lags one step), role 1
  // for every i (its dK lags two). Tiles and fragments of consecutive steps
  // alternate between the 0 and 1 copies. Each role runs its own copy of the
  // loop (same barriers), so values hoisted out of one role's loop do not
  // stay live in the other's.
  auto run = [&](auto role_c, auto&& body) {
    constexpr int R = decltype(role_c)::value;
    constexpr int N = R == 0 ? NDMA_R0 : NDMA_R1;
    auto iteration = [&](int i, f32x16 (&cur)[KT], f32x16 (&nxt)[KT], frag8 (&Told)[KT][2],
                         frag8 (&Tnew)[KT][2]) {
      if (i + 2 < total) wait_vmcnt<N>();
      else wait_vmcnt<0>();
      __syncthreads();
      if constexpr (R == 1) store_ds(i, Told);  // Told: dS of step i-2
      if (i + 3 < total) issue(i + 3, role_c);
      body(i, cur, nxt, Told, Tnew);
    };
    for (int i = 0; i <= total + 1; i += 2) {
      iteration(i, sc0, sc1, tf0, tf1);
      if (i + 1 <= total + 1) iteration(i + 1, sc1, sc0, tf1, tf0);
    }
  };
  if (role == 0)
    run(std::integral_constant<int, 0>{},
        [&](int i, f32x16 (&cur)[KT], f32x16 (&nxt)[KT], frag8 (&Told)[KT][2],
            frag8 (&Tnew)[KT][2]) {
          if (i <= total) step_a(i, cur, nxt, Told, Tnew);
        });
  else
    run(std::integral_constant<int, 1>{},
        [&](int i, f32x16 (&cur)[KT], f32x16 (&nxt)[KT], frag8 (&Told)[KT][2],
            frag8 (&Tnew)[KT][2]) { step_b(i, cur, nxt, Told, Tnew); });

  // dV (role 0) or dK * scale (role 1) of keys kp0 + 32*kt + l%32
  agpr_results_ready(acc);
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    const int key = kp0 + 32 * kt + col;
    if (key >= lk) continue;
    const int64_t r = sg.k_row0 + key;
    const float mul = role == 0 ? 1.f : a.scale;
    uint16_t* out = role == 0 ? a.dv.p + s * a.dv.sb + r * a.dv.sn + g * a.dv.sh
                              : a.dk.p + s * a.dk.sb + r * a.dk.sn + g * a.dk.sh;
#pragma unroll
    for (int d = 0; d < NDB; ++d)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        elem4 v4;
#pragma unroll
        for (int c = 0; c < 4; ++c) v4[c] = (elem_t)(acc[d][kt][4 * rr + c] * mul);
        *reinterpret_cast<elem4*>(out + 32 * d + 8 * rr + 4 * h) = v4;
      }
  }
}

}  // namespace VCA_ELEM
}  // namespace vca
