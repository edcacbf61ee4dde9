// Two-phase backward for large head dims (NeMo-Automodel "ffpa_attention"
// page, backward entries; same quantities as the fused kernels):
//
//   phase 1 (scores): per visible 128x128 (query tile, key tile) pair,
//       S = Q K^T and dP = dO V^T over the full head dims, then
//       P = exp(scale*S - lse) and dS = P * (dP - delta), stored as bf16 tiles;
//   phase 2 (products): three GEMM-shaped passes over the stored tiles,
//       dV = P^T dO and dK = scale * dS^T Q per (kv-head, key tile), summing
//       the q-heads of the GQA group, and dQ = scale * dS K per query tile.
//
// With a 512-wide head dim a workgroup cannot keep dK and dV of 64 keys in
// registers next to the score tiles, and splitting the score contraction
// across waves costs an fp32 exchange per tile. Writing P and dS once (2+2
// bytes per visible (query, key, head)) turns every matrix product into a
// plain tiled GEMM whose accumulators fit, at the price of that traffic.
//
// Tile store: a rectangle per row slot. Query tile qb of segment s owns row
// slot floor(q_row0/128) + s + qb (varlen; injective because each segment
// adds at most ceil(lq/128) <= floor(lq/128) + 1 slots) or s*nqb + qb
// (dense). A slot holds `tile_nkb` key tiles (max_k / 128 rounded up) per
// q-head; tile (slot, kb, h) starts at ((slot*tile_nkb + kb)*Hq + h)*128*128
// elements and is row-major [query][key]. Only visible tiles are written and
// read; key tiles at or past tile_nkb (a segment longer than max_k) are
// neither, so a wrong max_k gives wrong numbers, never an out-of-range access.
#pragma once

#include "attn_bwd.hpp"

namespace vca {

constexpr int kTile = 128;
constexpr int64_t kTileElems = (int64_t)kTile * kTile;

__device__ __forceinline__ int64_t tile_slot(const BwdArgs& a, const SegGeom& g, int s, int qb) {
  return a.tile_nqb_dense ? (int64_t)s * a.tile_nqb_dense + qb
                          : (int64_t)(g.q_row0 / kTile) + s + qb;
}
__device__ __forceinline__ int64_t tile_base(const BwdArgs& a, int64_t slot, int kb, int h) {
  return ((slot * a.tile_nkb + kb) * a.Hq + h) * kTileElems;
}
// key tiles a query tile's rows can see (capped by the tile store's width)
__device__ __forceinline__ int tile_row_extent(const BwdArgs& a, const SegGeom& g, int q0,
                                               bool causal) {
  int kv_end = g.lk;
  if (causal) kv_end = min(g.lk, q0 + kTile + (g.lk - g.lq));
  const int n = kv_end > 0 ? (kv_end + kTile - 1) / kTile : 0;
  return min(n, a.tile_nkb);
}
// first query tile that can see key tile kb
__device__ __forceinline__ int tile_col_start(const SegGeom& g, int kb, bool causal) {
  return causal ? max(0, kb * kTile - (g.lk - g.lq)) / kTile : 0;
}

// ---------------------------------------------------------------------------
// Phase 1. One workgroup of 8 waves = (segment, q-head, query tile); it walks
// the visible key tiles of its row. Waves 0-3 compute S^T = K Q^T, waves 4-7
// dP^T = V dO^T, each a 64x64 quarter (2x2 MFMA tiles: two A and two B
// fragments per four MFMAs). The head dims stream through LDS in chunks of
// KC columns, staged through registers a chunk ahead. At the end of a key
// tile the S waves write bf16 P into LDS, the dP waves turn it into dS, and
// the workgroup stores both tiles with 16-byte writes.
// ---------------------------------------------------------------------------
template <int DQK, int DV, bool CAUSAL>
__global__ void __launch_bounds__(512, 1) attn_bwd_scores_kernel(const BwdArgs a) {
  constexpr int NT = 512, KC = 64;
  static_assert(DQK % KC == 0 && DV % KC == 0, "head dims stream in 64-column chunks");
  constexpr int NCQ = DQK / KC, NCV = DV / KC, NC = NCQ > NCV ? NCQ : NCV;
  constexpr int LS = KC + 8;          // 144-byte rows: conflict-free row fragment reads
  constexpr int OS = kTile + 8;       // P / dS rows in the epilogue
  constexpr int STAGE = 4 * kTile * LS;
  static_assert(2 * kTile * OS <= STAGE, "epilogue tiles reuse one stage buffer");
  __shared__ __attribute__((aligned(16))) uint16_t smem[2][STAGE];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int role = w >> 2;               // 0: S (K, Q), 1: dP (V, dO)
  const int wk = (w >> 1) & 1, wq = w & 1;
  const int item = blockIdx.x / a.Hq, h = blockIdx.x - item * a.Hq, g = h / a.G;
  if (item >= *a.count_q) return;
  const int2 st = a.items_q[item];
  const int s = st.x;
  const SegGeom sg = seg_geom(a.cu_q, a.cu_k, s, a.Nq, a.Nk, a.Tq, a.Tk);
  const int q0 = st.y * kTile;
  if (q0 >= sg.lq) return;
  const int lq = sg.lq, lk = sg.lk, shift = lk - lq;
  const int nkt = tile_row_extent(a, sg, q0, CAUSAL);
  if (nkt == 0) return;
  const int64_t slot = tile_slot(a, sg, s, st.y);

  const uint16_t* qbp = a.q.p + s * a.q.sb + (int64_t)sg.q_row0 * a.q.sn + h * a.q.sh;
  const uint16_t* dobp = a.dout.p + s * a.dout.sb + (int64_t)sg.q_row0 * a.dout.sn + h * a.dout.sh;
  const uint16_t* kbp = a.k.p + s * a.k.sb + (int64_t)sg.k_row0 * a.k.sn + g * a.k.sh;
  const uint16_t* vbp = a.v.p + s * a.v.sb + (int64_t)sg.k_row0 * a.v.sn + g * a.v.sh;

  // per-lane row operand: lse*log2(e) (S waves) or delta (dP waves) of the
  // lane's two queries q0 + 64*wq + 32*u + col
  float rowv[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int qi = min(q0 + 64 * wq + 32 * u + col, lq - 1);
    const int64_t li = s * a.lse_sb + h * a.lse_sh + sg.q_row0 + qi;
    if (role == 0) {
      const float l = a.lse[li];
      rowv[u] = l == kNegInf ? __builtin_inff() : l * kLog2e;
    } else {
      rowv[u] = a.delta[li];
    }
  }
  wait_global_loads();

  // stage layout: [K | Q | V | dO] chunks, 128 rows x KC columns each
  using Chunk = TileStage<kTile, KC, NT>;
  Chunk ck, cq, cv, cd;
  auto load = [&](int it) {
    const int kt = it / NC, c = it - kt * NC;
    if (c < NCQ) {
      ck.load_clamped(kbp + c * KC, a.k.sn, kt * kTile, lk, tid);
      cq.load_clamped(qbp + c * KC, a.q.sn, q0, lq, tid);
    }
    if (c < NCV) {
      cv.load_clamped(vbp + c * KC, a.v.sn, kt * kTile, lk, tid);
      cd.load_clamped(dobp + c * KC, a.dout.sn, q0, lq, tid);
    }
  };
  auto store = [&](int it, uint16_t* buf) {
    const int c = it % NC;
    if (c < NCQ) {
      ck.template store<LS>(buf, tid);
      cq.template store<LS>(buf + kTile * LS, tid);
    }
    if (c < NCV) {
      cv.template store<LS>(buf + 2 * kTile * LS, tid);
      cd.template store<LS>(buf + 3 * kTile * LS, tid);
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int u = 0; u < 2; ++u) acc[t][u] = zero16();

  const int total = nkt * NC;
  load(0);
  store(0, smem[0]);
  if (total > 1) load(1);
  __syncthreads();

  const int my_nc = role == 0 ? NCQ : NCV;
  for (int it = 0; it < total; ++it) {
    const int kt = it / NC, c = it - kt * NC;
    uint16_t* buf = smem[it & 1];
    if (c < my_nc) {
      const uint16_t* A = buf + (2 * role) * kTile * LS;      // K or V rows (keys)
      const uint16_t* B = buf + (2 * role + 1) * kTile * LS;  // Q or dO rows (queries)
#pragma unroll
      for (int ks = 0; ks < KC / 16; ++ks) {
        const int d = ks * 16 + half * 8;
        const bf16x8 a0 = lds_frag(&A[(64 * wk + col) * LS + d]);
        const bf16x8 a1 = lds_frag(&A[(64 * wk + 32 + col) * LS + d]);
        const bf16x8 b0 = lds_frag(&B[(64 * wq + col) * LS + d]);
        const bf16x8 b1 = lds_frag(&B[(64 * wq + 32 + col) * LS + d]);
        acc[0][0] = mfma32(a0, b0, acc[0][0]);
        acc[0][1] = mfma32(a0, b1, acc[0][1]);
        acc[1][0] = mfma32(a1, b0, acc[1][0]);
        acc[1][1] = mfma32(a1, b1, acc[1][1]);
      }
    }
    if (it + 1 < total) store(it + 1, smem[(it + 1) & 1]);
    if (it + 2 < total) load(it + 2);
    __syncthreads();  // buf is free; chunk it+1 is visible
    if (c != NC - 1) continue;

    // ---- end of key tile kt: P and dS into buf, then out to the tile store
    uint16_t* sp = buf;
    uint16_t* sds = buf + kTile * OS;
    const int k0 = kt * kTile;
    if (role == 0) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int ql = 64 * wq + 32 * u + col, qi = q0 + ql;
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int kl = 64 * wk + 32 * t + rr * 8 + half * 4;
            bf16x4 p4;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int kj = k0 + kl + e;
              bool vis = qi < lq && kj < lk;
              if (CAUSAL) vis = vis && kj <= qi + shift;
              const float p = fast_exp2(acc[t][u][rr * 4 + e] * a.scale_log2 - rowv[u]);
              p4[e] = (__bf16)(vis ? p : 0.f);
            }
            *reinterpret_cast<bf16x4*>(&sp[ql * OS + kl]) = p4;
          }
        }
    }
    __syncthreads();
    if (role == 1) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int ql = 64 * wq + 32 * u + col;
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int kl = 64 * wk + 32 * t + rr * 8 + half * 4;
            const bf16x4 p4 = *reinterpret_cast<const bf16x4*>(&sp[ql * OS + kl]);
            bf16x4 d4;
#pragma unroll
            for (int e = 0; e < 4; ++e)
              d4[e] = (__bf16)((float)p4[e] * (acc[t][u][rr * 4 + e] - rowv[u]));
            *reinterpret_cast<bf16x4*>(&sds[ql * OS + kl]) = d4;
          }
        }
    }
    __syncthreads();
    {
      const int64_t base = tile_base(a, slot, kt, h);
      uint16_t* gp = a.tile_p + base;
      uint16_t* gd = a.tile_ds + base;
#pragma unroll
      for (int i = 0; i < kTile * kTile / 8 / NT; ++i) {
        const int chunk = tid + i * NT, row = chunk >> 4, cc = chunk & 15;
        *reinterpret_cast<u32x4*>(gp + row * kTile + cc * 8) =
            *reinterpret_cast<const u32x4*>(&sp[row * OS + cc * 8]);
        *reinterpret_cast<u32x4*>(gd + row * kTile + cc * 8) =
            *reinterpret_cast<const u32x4*>(&sds[row * OS + cc * 8]);
      }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int u = 0; u < 2; ++u) acc[t][u] = zero16();
    __syncthreads();  // buf is rewritten by the store of iteration it+1
  }
}

// ---------------------------------------------------------------------------
// Phase 2a. dV (IS_DK = false) or dK (true) of one (segment, kv-head, key
// tile): C^T[d][key] = sum over (q-head of the group, visible query tile,
// 32-query chunk) of X^T[d][q] T[q][key], X = dO or Q, T = P or dS. Both
// operands are read down their LDS columns (transposing read). 8 waves in a
// WR x (8/WR) grid over (keys, output columns).
// ---------------------------------------------------------------------------
template <int DOUT, int WR, bool CAUSAL, bool IS_DK>
__global__ void __launch_bounds__(512, 1) attn_bwd_dkdv_tiles_kernel(const BwdArgs a) {
  constexpr int NT = 512, QC = 32;
  constexpr int WC = 8 / WR, RK = kTile / WR, CD = DOUT / WC;
  static_assert(RK % 32 == 0 && CD % 32 == 0, "wave grid");
  constexpr int RT = RK / 32, CT = CD / 32;
  constexpr int AS = kTile + 32;   // tile rows: 320 bytes (transposing reads)
  constexpr int BS = DOUT + 32;    // X rows
  __shared__ __attribute__((aligned(16))) uint16_t sa[2][QC * AS];
  __shared__ __attribute__((aligned(16))) uint16_t sb[2][QC * BS];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int wk0 = (w % WR) * RK, wd0 = (w / WR) * CD;
  const int item = blockIdx.x / a.Hkv, hk = blockIdx.x - item * a.Hkv;
  if (item >= *a.count_k) return;
  const int2 st = a.items_k[item];
  const int s = st.x, kb = st.y;
  const SegGeom sg = seg_geom(a.cu_q, a.cu_k, s, a.Nq, a.Nk, a.Tq, a.Tk);
  const int k0 = kb * kTile;
  if (k0 >= sg.lk) return;
  const int lq = sg.lq;
  const int qb0 = tile_col_start(sg, kb, CAUSAL);
  const int nqb = (lq + kTile - 1) / kTile;
  const int per = kb < a.tile_nkb && nqb > qb0 ? (nqb - qb0) * (kTile / QC) : 0;
  const int total = a.G * per;

  const View X = IS_DK ? a.q : a.dout;
  const uint16_t* T = IS_DK ? a.tile_ds : a.tile_p;
  using XStage = TileStage<QC, DOUT, NT>;
  using TStage = TileStage<QC, kTile, NT>;
  XStage xs;
  TStage ts;
  auto load = [&](int it) {
    const int hh = it / per, rem = it - hh * per;
    const int qb = qb0 + rem / (kTile / QC), c = rem % (kTile / QC);
    const int h = hk * a.G + hh;
    const uint16_t* xp = X.p + s * X.sb + (int64_t)sg.q_row0 * X.sn + h * X.sh;
    xs.load_clamped(xp, X.sn, qb * kTile + c * QC, lq, tid);
    const uint16_t* tp = T + tile_base(a, tile_slot(a, sg, s, qb), kb, h) + c * QC * kTile;
    ts.load(tp, kTile, 0, QC, tid);
  };

  f32x16 acc[CT][RT];
#pragma unroll
  for (int u = 0; u < CT; ++u)
#pragma unroll
    for (int t = 0; t < RT; ++t) acc[u][t] = zero16();

  if (total > 0) {
    load(0);
    xs.template store<BS>(sb[0], tid);
    ts.template store<AS>(sa[0], tid);
    if (total > 1) load(1);
  }
  __syncthreads();
  for (int it = 0; it < total; ++it) {
    const int buf = it & 1;
#pragma unroll
    for (int ks = 0; ks < QC / 16; ++ks) {
      bf16x8 xf[CT], tf[RT];
#pragma unroll
      for (int u = 0; u < CT; ++u) xf[u] = tr_frag(sb[buf], BS, ks * 16, wd0 + 32 * u, lane);
#pragma unroll
      for (int t = 0; t < RT; ++t) tf[t] = tr_frag(sa[buf], AS, ks * 16, wk0 + 32 * t, lane);
#pragma unroll
      for (int u = 0; u < CT; ++u)
#pragma unroll
        for (int t = 0; t < RT; ++t) acc[u][t] = mfma32(xf[u], tf[t], acc[u][t]);
    }
    if (it + 1 < total) {
      xs.template store<BS>(sb[buf ^ 1], tid);
      ts.template store<AS>(sa[buf ^ 1], tid);
    }
    if (it + 2 < total) load(it + 2);
    __syncthreads();
  }

  const float mul = IS_DK ? a.scale : 1.f;
  const ViewW O = IS_DK ? a.dk : a.dv;
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int key = k0 + wk0 + 32 * t + col;
    if (key >= sg.lk) continue;
    uint16_t* op = O.p + s * O.sb + (int64_t)(sg.k_row0 + key) * O.sn + hk * O.sh + wd0;
#pragma unroll
    for (int u = 0; u < CT; ++u)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        bf16x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = (__bf16)(acc[u][t][rr * 4 + e] * mul);
        *reinterpret_cast<bf16x4*>(op + 32 * u + rr * 8 + half * 4) = v4;
      }
  }
}

// ---------------------------------------------------------------------------
// Phase 2b. dQ of one (segment, q-head, query tile): dQ^T[d][q] = sum over
// (visible key tile, 32-key chunk) of K^T[d][key] dS^T[key][q]. K is read
// down its LDS columns; dS rows supply 4+4 keys per lane in the order the
// transposing read delivers them. 8 waves in a WR x (8/WR) grid over
// (queries, head-dim columns).
// ---------------------------------------------------------------------------
template <int DQK, int WR, bool CAUSAL>
__global__ void __launch_bounds__(512, 1) attn_bwd_dq_tiles_kernel(const BwdArgs a) {
  constexpr int NT = 512, KC = 32;
  constexpr int WC = 8 / WR, RQ = kTile / WR, CD = DQK / WC;
  static_assert(RQ % 32 == 0 && CD % 32 == 0, "wave grid");
  constexpr int RT = RQ / 32, CT = CD / 32;
  constexpr int KS = DQK + 32;  // K rows (transposing reads)
  constexpr int SS = KC + 8;    // dS rows: 80 bytes
  __shared__ __attribute__((aligned(16))) uint16_t sk[2][KC * KS];
  __shared__ __attribute__((aligned(16))) uint16_t sds[2][kTile * SS];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int wq0 = (w % WR) * RQ, wd0 = (w / WR) * CD;
  const int item = blockIdx.x / a.Hq, h = blockIdx.x - item * a.Hq, g = h / a.G;
  if (item >= *a.count_q) return;
  const int2 st = a.items_q[item];
  const int s = st.x;
  const SegGeom sg = seg_geom(a.cu_q, a.cu_k, s, a.Nq, a.Nk, a.Tq, a.Tk);
  const int q0 = st.y * kTile;
  if (q0 >= sg.lq) return;
  const int lk = sg.lk;
  const int nkt = tile_row_extent(a, sg, q0, CAUSAL);
  const int total = nkt * (kTile / KC);
  const int64_t slot = tile_slot(a, sg, s, st.y);
  const uint16_t* kbp = a.k.p + s * a.k.sb + (int64_t)sg.k_row0 * a.k.sn + g * a.k.sh;

  using KStage = TileStage<KC, DQK, NT>;
  KStage ks_;
  u32x4 dsr;  // one 16-byte piece of the dS chunk per thread (128 rows x 64 bytes)
  const int drow = tid >> 2, dcc = tid & 3;
  auto load = [&](int it) {
    const int kt = it / (kTile / KC), c = it % (kTile / KC);
    ks_.load_clamped(kbp, a.k.sn, kt * kTile + c * KC, lk, tid);
    dsr = ldg16(a.tile_ds + tile_base(a, slot, kt, h) + drow * kTile + c * KC + dcc * 8);
  };
  auto store = [&](int b) {
    ks_.template store<KS>(sk[b], tid);
    sts16(&sds[b][drow * SS + dcc * 8], dsr);
  };

  f32x16 acc[CT][RT];
#pragma unroll
  for (int u = 0; u < CT; ++u)
#pragma unroll
    for (int t = 0; t < RT; ++t) acc[u][t] = zero16();

  if (total > 0) {
    load(0);
    store(0);
    if (total > 1) load(1);
  }
  __syncthreads();
  for (int it = 0; it < total; ++it) {
    const int buf = it & 1;
#pragma unroll
    for (int kk = 0; kk < KC / 16; ++kk) {
      bf16x8 kf[CT], sf[RT];
#pragma unroll
      for (int u = 0; u < CT; ++u) kf[u] = tr_frag(sk[buf], KS, kk * 16, wd0 + 32 * u, lane);
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const uint16_t* p = &sds[buf][(wq0 + 32 * t + col) * SS + kk * 16 + half * 4];
        const u32x2 lo = *reinterpret_cast<const u32x2*>(p);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(p + 8);
        const u32x4 v = {lo[0], lo[1], hi[0], hi[1]};
        sf[t] = as_frag(v);
      }
#pragma unroll
      for (int u = 0; u < CT; ++u)
#pragma unroll
        for (int t = 0; t < RT; ++t) acc[u][t] = mfma32(kf[u], sf[t], acc[u][t]);
    }
    if (it + 1 < total) store(buf ^ 1);
    if (it + 2 < total) load(it + 2);
    __syncthreads();
  }

#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int qi = q0 + wq0 + 32 * t + col;
    if (qi >= sg.lq) continue;
    uint16_t* dqp = a.dq.p + s * a.dq.sb + (int64_t)(sg.q_row0 + qi) * a.dq.sn + h * a.dq.sh + wd0;
#pragma unroll
    for (int u = 0; u < CT; ++u)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        uint16_t* dst = dqp + 32 * u + rr * 8 + half * 4;
        float add[4] = {0.f, 0.f, 0.f, 0.f};
        if (a.dq_accumulate) {
          const u32x2 old = *reinterpret_cast<const u32x2*>(dst);
          add[0] = __uint_as_float(old[0] << 16);
          add[1] = __uint_as_float(old[0] & 0xffff0000u);
          add[2] = __uint_as_float(old[1] << 16);
          add[3] = __uint_as_float(old[1] & 0xffff0000u);
        }
        bf16x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = (__bf16)(acc[u][t][rr * 4 + e] * a.scale + add[e]);
        *reinterpret_cast<bf16x4*>(dst) = v4;
      }
  }
}

}  // namespace vca
