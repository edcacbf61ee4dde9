// Two-phase backward for large head dims (NeMo-Automodel "ffpa_attention"
// page, backward entries; same quantities as the fused kernels):
//
//   phase 1 (scores): per visible 256x256 (query block, key block) pair,
//       S = Q K^T and dP = dO V^T over the full head dims, then
//       P = exp(scale*S - lse) and dS = P * (dP - delta), stored as bf16;
//   phase 2 (products): dV = P^T dO and dK = scale * dS^T Q per (kv-head,
//       key block, 256 output columns), summing the q-heads of the GQA group,
//       and dQ = scale * dS K per (q-head, query block, 256 output columns).
//
// With a 512-wide head dim a workgroup cannot keep dK and dV of 64 keys in
// registers next to the score tiles, and splitting the score contraction
// across waves costs an fp32 exchange per tile. Writing P and dS once (2+2
// bytes per visible (query, key, head)) turns every matrix product into a
// plain block GEMM whose accumulators fit, at the price of that traffic.
//
// Every pass is a block GEMM of 8 waves (scores: 256x256 C, each wave 64 rows
// x 128 columns; products: OB output columns, each wave 64 rows x OB/2 or
// OB/4 columns); the contraction streams through two LDS stages of 64
// elements per operand, loaded straight from global memory into LDS one
// stage ahead, with one barrier per stage.
//
// Block store: query block qb of segment s owns row slot
// floor(q_row0/256) + s + qb (varlen; injective because a segment adds at
// most ceil(lq/256) <= floor(lq/256) + 1 slots) or s*nqb + qb (dense). A slot
// holds tile_nkb key blocks (max_k/256 rounded up) per q-head; block
// (slot, kb, h) starts at ((slot*tile_nkb + kb)*Hq + h)*256*256 elements and
// is row-major [query][key], with the keys of each group of 16 stored in the
// order 0-3, 8-11, 4-7, 12-15 (key_perm): a 32x32 MFMA result tile then
// writes 16 contiguous bytes per lane, and the dQ pass reads the eight keys a
// lane feeds one MFMA as one 16-byte piece. Only blocks a query block can see
// are written (whole, masked entries as zeros) and read; key blocks at or past
// tile_nkb (a segment longer than max_k) are neither, so a wrong max_k gives
// wrong numbers, never an out-of-range access.
#pragma once

#include "attn_bwd.hpp"

namespace vca {
namespace VCA_ELEM {

constexpr int kBlk = 256;                            // block rows and columns
constexpr int kChunk = 64;                           // contraction elements per stage
constexpr int kOpElems = kBlk * kChunk;              // one staged operand (32 KB)
constexpr int64_t kBlkElems = (int64_t)kBlk * kBlk;  // one stored block
constexpr int kXcds = 8;
constexpr int kNT = 512;                             // threads per workgroup (8 waves)

__device__ __forceinline__ int64_t blk_slot(const BwdArgs& a, const SegGeom& g, int s, int qb) {
  return a.tile_nqb_dense ? (int64_t)s * a.tile_nqb_dense + qb
                          : (int64_t)(g.q_row0 / kBlk) + s + qb;
}
// the store holds the slots of one chunk, slot_lo .. slot_hi - 1
__device__ __forceinline__ int64_t blk_base(const BwdArgs& a, int64_t slot, int kb, int h) {
  return (((slot - a.slot_lo) * a.tile_nkb + kb) * a.Hq + h) * kBlkElems;
}
// key blocks the rows of the query block starting at q0 can see (capped by
// the store's width)
__device__ __forceinline__ int blk_row_extent(const BwdArgs& a, const SegGeom& g, int q0,
                                              bool causal) {
  int kv_end = g.lk;
  if (causal) kv_end = min(g.lk, q0 + kBlk + (g.lk - g.lq));
  const int n = kv_end > 0 ? (kv_end + kBlk - 1) / kBlk : 0;
  return min(n, a.tile_nkb);
}
// first query block that can see key block kb
__device__ __forceinline__ int blk_col_start(const SegGeom& g, int kb, bool causal) {
  return causal ? max(0, kb * kBlk - (g.lk - g.lq)) / kBlk : 0;
}
// Left window (win > 0, causal only): the first key block the rows of the
// query block starting at q0 can see (the one holding its first row's first
// visible key; every later block up to the extent is seen by some row)...
__device__ __forceinline__ int blk_row_first(const SegGeom& g, int q0, int win) {
  return win > 0 ? max(0, q0 + (g.lk - g.lq) - win + 1) / kBlk : 0;
}
// ...and one past the last query block that sees key block kb (its rows end
// where the window of a row no longer reaches the block's last key)
__device__ __forceinline__ int blk_col_end(const SegGeom& g, int kb, int win) {
  const int nqb = (g.lq + kBlk - 1) / kBlk;
  if (win <= 0) return nqb;
  const int q_end = min(g.lq, kb * kBlk + kBlk - 1 - (g.lk - g.lq) + win);
  return q_end > 0 ? min(nqb, (q_end + kBlk - 1) / kBlk) : 0;
}
// stored column of key k inside its block (swaps the middle two 4-key groups
// of every 16; its own inverse)
__device__ __forceinline__ int key_perm(int k) {
  return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

// Workgroups are dealt to the 8 XCDs round-robin by index. This map puts the
// PARTS workgroups of one (item, head) group on one XCD back to back, so they
// run together and share their common operand through that XCD's L2, while
// the groups keep their heavy-first order across the chip.
template <int PARTS>
__device__ __forceinline__ void xcd_work(int bid, int& group, int& part) {
  const int xcd = bid % kXcds, j = bid / kXcds;
  part = j % PARTS;
  group = (j / PARTS) * kXcds + xcd;
}
// Group -> (work item, head) for H heads in GQA groups of G (G = 1 for a
// kv-head pass). When the kv heads divide evenly over the XCDs, XCD x takes
// kv heads x, x+8, ... one after the other, and for each of them every item
// in list (heavy-first) order with the group's q-heads innermost: the groups
// that run together on an XCD are neighbouring items of one kv head and read
// the same K/V (and Q/dO) blocks through its L2. Otherwise items outermost.
__device__ __forceinline__ void xcd_item_head_major(int grp, int nitems, int H, int G, int& item,
                                                    int& h) {
  if ((H / G) % kXcds == 0) {
    const int x = grp % kXcds, k = grp / kXcds;
    const int per = nitems * G;  // groups per kv head on this XCD
    const int m = k / per, r = k - m * per;
    item = r / G;
    h = (x + kXcds * m) * G + (r - item * G);
  } else {
    item = grp / H;
    h = grp - item * H;
  }
}
template <int PARTS>
inline unsigned xcd_grid(unsigned groups) {
  return (groups + kXcds - 1) / kXcds * kXcds * PARTS;
}

// ---- staged operands -------------------------------------------------------
// Row mode: kBlk rows x kChunk contraction elements, 128-byte rows. The
// 16-byte piece p of row r sits at position p ^ ((r >> 1) & 7): the 16 rows
// one ds_read_b128 serves per LDS cycle land on distinct banks.
__device__ __forceinline__ frag8 row_frag(const uint16_t* X, int r, int piece) {
  return lds_frag(X + r * kChunk + ((piece ^ ((r >> 1) & 7)) << 3));
}
// Column mode: kChunk contraction rows x W columns (W = 128, 192 or 256).
// The 16-byte unit u of row r sits at position col_pos<W>(r, u), chosen so
// the four rows one transposing read covers per 32 lanes land in four
// different 64-byte bank groups: rows of 256 or 512 bytes all start on the
// same bank, so 64-byte windows are XORed with r & 3; rows of 384 bytes
// alternate between the two bank halves, so the window is XORed with bit 1
// of r. col_frag gives the same result as tr_frag: lane l gets column
// n0 + l%32 and rows {k0 + 4h + j, k0 + 8 + 4h + j} (h = l/32).
template <int W>
__device__ __forceinline__ int col_pos(int r, int u) {
  static_assert(W == 128 || W == 192 || W == 256, "column-mode widths");
  if constexpr (W == 192) return u ^ (((r >> 1) & 1) << 2);
  else return u ^ ((r & 3) << 2);
}
template <int W>
__device__ __forceinline__ frag8 col_frag(const uint16_t* X, int k0, int n0, int lane) {
  const int g = lane >> 4, s = lane & 15, h = lane >> 5;
  const int row = k0 + 4 * h + (s >> 2);
  const int c = n0 + 16 * (g & 1) + 4 * (s & 3);
  // rows row and row + 8 share the swizzle
  const uint16_t* p = X + row * W + (col_pos<W>(row, c >> 3) << 3) + (c & 7);
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)((__attribute__((address_space(3))) uint16_t*)p));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)((__attribute__((address_space(3))) uint16_t*)(p + 8 * W)));
  return __builtin_bit_cast(frag8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}
// Fill a row-mode operand: rp(r) points at the stage's first element of row
// r (r < 256). Wave w issues four 8-row loads.
template <class RowPtr>
__device__ __forceinline__ void fill_rows(const uint16_t* X, int w, int lane, RowPtr rp) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 32 * w + 8 * j + (lane >> 3);
    const int piece = (lane & 7) ^ ((r >> 1) & 7);
    dma16(rp(r) + piece * 8, lds_ptr(X + (32 * w + 8 * j) * kChunk));
  }
}
// Fill a column-mode operand of width W: rp(r) points at the first of the W
// columns of contraction row r (r < 64). The operand is W/8 contiguous 1 KB
// loads; wave w issues W/64 of them, each lane placing one 16-byte unit.
template <int W, class RowPtr>
__device__ __forceinline__ void fill_cols(const uint16_t* X, int w, int lane, RowPtr rp) {
  constexpr int NL = W / 64, RB = 2 * W;  // loads per wave, bytes per row
#pragma unroll
  for (int j = 0; j < NL; ++j) {
    const int blk = w * NL + j;                        // 1 KB block of the operand
    const int pos = blk * 1024 + 16 * lane;            // this lane's byte offset
    const int r = pos / RB, su = (pos % RB) / 16;      // row, stored unit
    dma16(rp(r) + col_pos<W>(r, su) * 8, lds_ptr(X + blk * 512));
  }
}

typedef const __attribute__((address_space(1))) float gfloat;

// ---------------------------------------------------------------------------
// Phase 1. One workgroup = (segment, q-head, query block, part); it takes key
// blocks part, part + kScoreSplit, ... of the row. Per key block it runs the
// S^T = K Q^T loop, writes P, then the dP^T = V dO^T loop (accumulators
// seeded with -delta) and writes dS = P * (dP - delta), re-reading its own P.
// Wave (wm, wn) owns keys 64*wm.. and queries 128*wn.. of the block. Masks
// are evaluated only for blocks that are not entirely visible.
// ---------------------------------------------------------------------------
constexpr int kScoreSplit = 4;

// EXT: 0 plain, 1 left window, 2 left window and softcap.
template <int DQK, int DV, bool CAUSAL, int EXT = 0>
__global__ void __launch_bounds__(kNT, 1) attn_bwd_scores_kernel(const BwdArgs a) {
  constexpr int NCQ = DQK / kChunk, NCV = DV / kChunk, NCT = NCQ + NCV;
  static_assert(DQK % kChunk == 0 && DV % kChunk == 0, "head dims stream in 64-element chunks");
  constexpr int NST = 16;  // hand-issued block stores per lane per epilogue
  __shared__ __attribute__((aligned(1024))) uint16_t stg[2][2 * kOpElems];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int wm = w >> 1, wn = w & 1;
  int grp, part;
  xcd_work<kScoreSplit>(blockIdx.x, grp, part);
  // kv-head-major: the q-heads of a GQA group run side by side on one XCD
  // and stream the same K/V blocks through its L2 (D=512 backward -1.8%)
  int item, h;
  xcd_item_head_major(grp, a.nq_items, a.Hq, a.G, item, h);
  const int g = h / a.G;
  if (item >= *a.count_q) return;
  const int2 st = a.items_q[item];
  const int s = st.x;
  const SegGeom sg = seg_geom(a.cu_q, a.cu_k, s, a.Nq, a.Nk, a.Tq, a.Tk);
  const int q0 = st.y * kBlk;
  if (q0 >= sg.lq) return;
  const int lq = sg.lq, lk = sg.lk, shift = lk - lq;
  const int ext = blk_row_extent(a, sg, q0, CAUSAL);
  // with a left window the block's key blocks start at kf (EXT only)
  const int win = EXT && CAUSAL ? a.window : 0;
  const bool capped = EXT == 2 && a.cap_in != 0.f;
  const int kf = EXT ? min(ext, blk_row_first(sg, q0, win)) : 0;
  const int nkt = ext - kf > part ? (ext - kf - part + kScoreSplit - 1) / kScoreSplit : 0;
  if (nkt == 0) return;
  const int64_t slot = blk_slot(a, sg, s, st.y);
  if (slot < a.slot_lo || slot >= a.slot_hi) return;  // another chunk's query block

  // lse*log2(e) and delta of the lane's four query columns
  float l2[4], dl[4];
  {
    gfloat* lp = (gfloat*)a.lse;
    gfloat* dp = (gfloat*)a.delta;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int qi = min(q0 + 128 * wn + 32 * u + col, lq - 1);
      const int64_t li = s * a.lse_sb + h * a.lse_sh + sg.q_row0 + qi;
      const float l = lp[li];
      l2[u] = l == kNegInf ? __builtin_inff() : l * kLog2e;
      dl[u] = dp[li];
    }
  }
  // consume the loads before any hand-issued memory operation: the compiler
  // then has nothing of its own outstanding when the loop counts by hand
  asm volatile("" ::"v"(l2[0]), "v"(l2[1]), "v"(l2[2]), "v"(l2[3]), "v"(dl[0]), "v"(dl[1]),
               "v"(dl[2]), "v"(dl[3]));

  const uint16_t* qbp = a.q.p + s * a.q.sb + (int64_t)sg.q_row0 * a.q.sn + h * a.q.sh;
  const uint16_t* dobp = a.dout.p + s * a.dout.sb + (int64_t)sg.q_row0 * a.dout.sn + h * a.dout.sh;
  const uint16_t* kbp = a.k.p + s * a.k.sb + (int64_t)sg.k_row0 * a.k.sn + g * a.k.sh;
  const uint16_t* vbp = a.v.p + s * a.v.sb + (int64_t)sg.k_row0 * a.v.sn + g * a.v.sh;
  auto issue = [&](int it, int stage) {
    const int kt = it / NCT, c = it - kt * NCT;
    const int k0 = (kf + part + kt * kScoreSplit) * kBlk;
    const bool sl = c < NCQ;
    const int c0 = (sl ? c : c - NCQ) * kChunk;
    const uint16_t* ab = (sl ? kbp : vbp) + c0;
    const int64_t asn = sl ? a.k.sn : a.v.sn;
    const uint16_t* bb = (sl ? qbp : dobp) + c0;
    const int64_t bsn = sl ? a.q.sn : a.dout.sn;
    fill_rows(stg[stage], w, lane, [&](int r) { return ab + (int64_t)min(k0 + r, lk - 1) * asn; });
    fill_rows(stg[stage] + kOpElems, w, lane,
              [&](int r) { return bb + (int64_t)min(q0 + r, lq - 1) * bsn; });
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[t][u] = zero16();

  const int total = nkt * NCT;
  issue(0, 0);
  // The loop's loads and stores are issued by hand, so a wave knows what it
  // has in flight when it waits for stage it: only the block stores of the
  // previous iteration's epilogue (if any) came after it. Operations retire
  // in issue order, so anything the compiler adds (register spills) only
  // makes such a wait stricter, never too weak.
  bool stored = false;
  for (int it = 0; it < total; ++it) {
    const int kt = it / NCT, c = it - kt * NCT, stage = it & 1;
    if (stored) wait_vmcnt<NST>();
    else wait_vmcnt<0>();
    stored = false;
    __syncthreads();  // stage it visible everywhere; stage it-1 is free
    if (it + 1 < total) issue(it + 1, stage ^ 1);
    {
      const uint16_t* A = stg[stage];
      const uint16_t* B = stg[stage] + kOpElems;
#pragma unroll
      for (int ks = 0; ks < kChunk / 16; ++ks) {
        frag8 af[2], bf[4];
#pragma unroll
        for (int t = 0; t < 2; ++t) af[t] = row_frag(A, 64 * wm + 32 * t + col, 2 * ks + half);
#pragma unroll
        for (int u = 0; u < 4; ++u) bf[u] = row_frag(B, 128 * wn + 32 * u + col, 2 * ks + half);
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int u = 0; u < 4; ++u) acc[t][u] = mfma32(af[t], bf[u], acc[t][u]);
      }
    }
    if (c != NCQ - 1 && c != NCT - 1) continue;

    // ---- epilogue: lane holds queries 128*wn + 32*u + col and, per 8 values
    // 8m..8m+7 of a result tile, the keys that are stored at columns
    // 64*wm + 32*t + 16*m + 8*half + 0..7 of the block
    const int kb = kf + part + kt * kScoreSplit, k0 = kb * kBlk;
    const int64_t base = blk_base(a, slot, kb, h);
    if (c == NCQ - 1) {
      uint16_t* pb = a.tile_p + base;
      // softcap: the chain factor 1 - tanh^2 of each element goes to the dS
      // block's place for the dS epilogue to pick up
      uint16_t* gb = a.tile_ds + base;
      auto pstore = [&](auto masked) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int qr = 128 * wn + 32 * u + col, qi = q0 + qr;
#pragma unroll
            for (int m = 0; m < 2; ++m) {
              frag8 p8, g8;
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                const int r = 8 * m + e;
                float th = 0.f;
                if (EXT == 2 && capped) th = fast_tanh(a.cap_in * acc[t][u][r]);
                float p = fast_exp2(
                    (EXT == 2 && capped ? a.cap_out * th : acc[t][u][r] * a.scale_log2) - l2[u]);
                if constexpr (decltype(masked)::value) {
                  const int kj = k0 + 64 * wm + 32 * t + 8 * (r >> 2) + 4 * half + (r & 3);
                  bool vis = qi < lq && kj < lk;
                  if (CAUSAL) vis = vis && kj <= qi + shift;
                  if (EXT && win > 0) vis = vis && kj > qi + shift - win;
                  p = vis ? p : 0.f;
                }
                p8[e] = (elem_t)p;
                if constexpr (EXT == 2) g8[e] = (elem_t)(1.f - th * th);
              }
              // (the offset is spelled out at each store: naming it once
              // makes the register allocator spill in the plain kernel)
              stg16(pb + qr * kBlk + 64 * wm + 32 * t + 16 * m + 8 * half,
                    __builtin_bit_cast(u32x4, p8));
              if (EXT == 2 && capped)
                stg16(gb + qr * kBlk + 64 * wm + 32 * t + 16 * m + 8 * half,
                      __builtin_bit_cast(u32x4, g8));
            }
          }
      };
      const bool full = q0 + kBlk <= lq && k0 + kBlk <= lk &&
                        (!CAUSAL || k0 + kBlk - 1 <= q0 + shift) &&
                        !(win > 0 && k0 <= q0 + kBlk - 1 + shift - win);
      if (full) pstore(std::false_type{});
      else pstore(std::true_type{});
    } else {
      const uint16_t* pb = a.tile_p + base;
      uint16_t* db = a.tile_ds + base;
      // this lane's own P, eight pieces in flight at a time
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        u32x4 pv[4][2];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int m = 0; m < 2; ++m)
            pv[u][m] = ldg16(pb + (128 * wn + 32 * u + col) * kBlk + 64 * wm + 32 * t + 16 * m +
                             8 * half);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int qr = 128 * wn + 32 * u + col;
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            const int off = qr * kBlk + 64 * wm + 32 * t + 16 * m + 8 * half;
            const frag8 p8 = as_frag(pv[u][m]);
            frag8 d8;
#pragma unroll
            for (int e = 0; e < 8; ++e)
              d8[e] = (elem_t)((float)p8[e] * acc[t][u][8 * m + e]);
            if (EXT == 2 && capped) {
              const frag8 g8 = as_frag(ldg16(db + off));
#pragma unroll
              for (int e = 0; e < 8; ++e) d8[e] = (elem_t)((float)d8[e] * (float)g8[e]);
            }
            stg16(db + off, __builtin_bit_cast(u32x4, d8));
          }
        }
      }
    }
    stored = true;
    // the dP loop starts from -delta (dS = P * dP then needs no row operand)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float x = c == NCQ - 1 ? -dl[u] : 0.f;
      asm volatile("" : "+v"(x));
#pragma unroll
      for (int t = 0; t < 2; ++t) acc[t][u] = splat16(x);
    }
  }
}

// Products run 8 waves over an (OB output columns) x (256 keys or queries)
// result: a WM x WN wave grid with RT x CT MFMA tiles per wave.
template <int OB>
struct ProdShape {
  static constexpr int WM = OB == 256 ? 4 : 2, WN = 8 / WM;
  static constexpr int RM = OB / WM, RN = kBlk / WN;  // rows / columns per wave
  static constexpr int RT = RM / 32, CT = RN / 32;
  static_assert(RM % 32 == 0 && RN % 32 == 0, "wave grid");
};
// output block width for a head dim: whole when it fits, else 256 at a time
constexpr int prod_block(int d) { return d > kBlk ? kBlk : d; }

// ---------------------------------------------------------------------------
// Phase 2a. dV (WHICH 0), dK (WHICH 1) or both (WHICH 2, part parity) of one
// (segment, kv-head, key block) and OB of its DOUT output columns:
//   C^T[d][key] = sum over (q-head of the group, visible query block, 64-row
//   chunk) of X^T[d][q] T[q][key],  X = dO or Q, T = P or dS.
// Both operands are staged in column mode and read down their columns. Query
// blocks run last to first, so the key blocks of one kv-head working side by
// side stream the same X rows at the same time.
// ---------------------------------------------------------------------------
template <int DOUT, int OB, bool CAUSAL, int WHICH>
__global__ void __launch_bounds__(kNT, 1) attn_bwd_dkdv_tiles_kernel(const BwdArgs a) {
  using S = ProdShape<OB>;
  constexpr int NDH = DOUT / OB, PARTS = (WHICH == 2 ? 2 : 1) * NDH, CPB = kBlk / kChunk;
  static_assert(DOUT % OB == 0, "output columns in whole blocks");
  __shared__ __attribute__((aligned(1024))) uint16_t stg[2][2 * kOpElems];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int wm = w / S::WN, wn = w % S::WN;
  int grp, part;
  xcd_work<PARTS>(blockIdx.x, grp, part);
  int item, hk;
  xcd_item_head_major(grp, a.nk_items, a.Hkv, 1, item, hk);
  if (item >= *a.count_k) return;
  const bool is_dk = WHICH == 2 ? (part & 1) != 0 : WHICH == 1;
  const int dh = WHICH == 2 ? part >> 1 : part;
  const int2 st = a.items_k[item];
  const int s = st.x, kb = st.y;
  const SegGeom sg = seg_geom(a.cu_q, a.cu_k, s, a.Nq, a.Nk, a.Tq, a.Tk);
  const int k0 = kb * kBlk;
  if (k0 >= sg.lk) return;
  const int lq = sg.lq;
  // query blocks qb0 .. nqb-1 see this key block (fewer with a left window);
  // this chunk holds those whose row slot lies in [slot_lo, slot_hi)
  const int64_t slot0 = blk_slot(a, sg, s, 0);
  const int qlo = (int)max((int64_t)blk_col_start(sg, kb, CAUSAL), a.slot_lo - slot0);
  const int nqb = (int)min((int64_t)blk_col_end(sg, kb, CAUSAL ? a.window : 0), a.slot_hi - slot0);
  const int per = kb < a.tile_nkb && nqb > qlo ? (nqb - qlo) * CPB : 0;
  const int total = a.G * per;

  // field-wise selects (a runtime choice between whole View structs sends
  // the kernel arguments through scratch memory)
  const uint16_t* xp = is_dk ? a.q.p : a.dout.p;
  const int64_t xsb = is_dk ? a.q.sb : a.dout.sb, xsh = is_dk ? a.q.sh : a.dout.sh;
  const int64_t xsn = is_dk ? a.q.sn : a.dout.sn;
  xp += s * xsb + (int64_t)sg.q_row0 * xsn + dh * OB;
  const uint16_t* T = is_dk ? a.tile_ds : a.tile_p;
  auto issue = [&](int it, int stage) {
    const int hh = it / per, rem = it - hh * per;
    const int qb = nqb - 1 - rem / CPB, c = rem % CPB;
    const int h = hk * a.G + hh;
    const int r0 = qb * kBlk + c * kChunk;
    const uint16_t* xh = xp + h * xsh;
    fill_cols<OB>(stg[stage], w, lane,
                  [&](int r) { return xh + (int64_t)min(r0 + r, lq - 1) * xsn; });
    const uint16_t* tb = T + blk_base(a, blk_slot(a, sg, s, qb), kb, h) + c * kChunk * kBlk;
    fill_cols<kBlk>(stg[stage] + kOpElems, w, lane, [&](int r) { return tb + r * kBlk; });
  };

  f32x16 acc[S::RT][S::CT];
#pragma unroll
  for (int t = 0; t < S::RT; ++t)
#pragma unroll
    for (int u = 0; u < S::CT; ++u) acc[t][u] = zero16();

  if (total > 0) issue(0, 0);
  for (int it = 0; it < total; ++it) {
    const int stage = it & 1;
    wait_vmcnt<0>();
    __syncthreads();
    if (it + 1 < total) issue(it + 1, stage ^ 1);
    const uint16_t* A = stg[stage];
    const uint16_t* B = stg[stage] + kOpElems;
#pragma unroll
    for (int ks = 0; ks < kChunk / 16; ++ks) {
      frag8 af[S::RT], bf[S::CT];
#pragma unroll
      for (int t = 0; t < S::RT; ++t) af[t] = col_frag<OB>(A, 16 * ks, S::RM * wm + 32 * t, lane);
#pragma unroll
      for (int u = 0; u < S::CT; ++u)
        bf[u] = col_frag<kBlk>(B, 16 * ks, S::RN * wn + 32 * u, lane);
#pragma unroll
      for (int t = 0; t < S::RT; ++t)
#pragma unroll
        for (int u = 0; u < S::CT; ++u) acc[t][u] = mfma32(af[t], bf[u], acc[t][u]);
    }
  }

  const float mul = is_dk ? a.scale : 1.f;
  uint16_t* op = is_dk ? a.dk.p : a.dv.p;
  const int64_t osb = is_dk ? a.dk.sb : a.dv.sb, osh = is_dk ? a.dk.sh : a.dv.sh;
  const int64_t osn = is_dk ? a.dk.sn : a.dv.sn;
  float* accp = is_dk ? a.acc_dk : a.acc_dv;
#pragma unroll
  for (int u = 0; u < S::CT; ++u) {
    const int key = k0 + key_perm(S::RN * wn + 32 * u + col);
    if (key >= sg.lk) continue;
    uint16_t* orow = op + s * osb + (int64_t)(sg.k_row0 + key) * osn + hk * osh + dh * OB;
    // fp32 accumulator row of this key when the backward runs in chunks
    float* arow = accp + (((int64_t)s * a.Nk + sg.k_row0 + key) * a.Hkv + hk) * DOUT + dh * OB;
#pragma unroll
    for (int t = 0; t < S::RT; ++t)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int c0 = S::RM * wm + 32 * t + rr * 8 + half * 4;
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[t][u][rr * 4 + e] * mul;
        if (a.acc_mode >= 2) v += *reinterpret_cast<const f32x4*>(arow + c0);
        if (a.acc_mode == 1 || a.acc_mode == 2) {
          *reinterpret_cast<f32x4*>(arow + c0) = v;
        } else {
          elem4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = (elem_t)v[e];
          *reinterpret_cast<elem4*>(orow + c0) = v4;
        }
      }
  }
}

// ---------------------------------------------------------------------------
// Phase 2b. dQ of one (segment, q-head, query block) and OB of its DQK output
// columns (part):  dQ^T[d][q] = sum over (visible key block, 64-key chunk) of
// K^T[d][key] dS^T[key][q]. K is staged in column mode and read down its
// columns; dS rows are staged in row mode, where the stored key order gives
// each lane its eight keys as one 16-byte piece.
// ---------------------------------------------------------------------------
template <int DQK, int OB, bool CAUSAL>
__global__ void __launch_bounds__(kNT, 1) attn_bwd_dq_tiles_kernel(const BwdArgs a) {
  using S = ProdShape<OB>;
  constexpr int NDH = DQK / OB, CPB = kBlk / kChunk;
  static_assert(DQK % OB == 0, "output columns in whole blocks");
  __shared__ __attribute__((aligned(1024))) uint16_t stg[2][2 * kOpElems];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int wm = w / S::WN, wn = w % S::WN;
  int grp, dh;
  xcd_work<NDH>(blockIdx.x, grp, dh);
  int item, h;
  xcd_item_head_major(grp, a.nq_items, a.Hq, a.G, item, h);
  const int g = h / a.G;
  if (item >= *a.count_q) return;
  const int2 st = a.items_q[item];
  const int s = st.x;
  const SegGeom sg = seg_geom(a.cu_q, a.cu_k, s, a.Nq, a.Nk, a.Tq, a.Tk);
  const int q0 = st.y * kBlk;
  if (q0 >= sg.lq) return;
  const int lk = sg.lk;
  // key blocks kf .. extent-1 (kf > 0 only with a left window)
  const int kext = blk_row_extent(a, sg, q0, CAUSAL);
  const int kf = min(kext, blk_row_first(sg, q0, CAUSAL ? a.window : 0));
  const int total = (kext - kf) * CPB;
  const int64_t slot = blk_slot(a, sg, s, st.y);
  if (slot < a.slot_lo || slot >= a.slot_hi) return;  // another chunk's query block
  const uint16_t* kbp =
      a.k.p + s * a.k.sb + (int64_t)sg.k_row0 * a.k.sn + g * a.k.sh + dh * OB;
  auto issue = [&](int it, int stage) {
    const int kb = kf + it / CPB, c = it % CPB;
    const int r0 = kb * kBlk + c * kChunk;
    fill_cols<OB>(stg[stage], w, lane,
                  [&](int r) { return kbp + (int64_t)min(r0 + r, lk - 1) * a.k.sn; });
    const uint16_t* db = a.tile_ds + blk_base(a, slot, kb, h) + c * kChunk;
    fill_rows(stg[stage] + kOpElems, w, lane, [&](int r) { return db + r * kBlk; });
  };

  f32x16 acc[S::RT][S::CT];
#pragma unroll
  for (int t = 0; t < S::RT; ++t)
#pragma unroll
    for (int u = 0; u < S::CT; ++u) acc[t][u] = zero16();

  if (total > 0) issue(0, 0);
  for (int it = 0; it < total; ++it) {
    const int stage = it & 1;
    wait_vmcnt<0>();
    __syncthreads();
    if (it + 1 < total) issue(it + 1, stage ^ 1);
    const uint16_t* A = stg[stage];
    const uint16_t* B = stg[stage] + kOpElems;
#pragma unroll
    for (int ks = 0; ks < kChunk / 16; ++ks) {
      frag8 af[S::RT], bf[S::CT];
#pragma unroll
      for (int t = 0; t < S::RT; ++t) af[t] = col_frag<OB>(A, 16 * ks, S::RM * wm + 32 * t, lane);
#pragma unroll
      for (int u = 0; u < S::CT; ++u)
        bf[u] = row_frag(B, S::RN * wn + 32 * u + col, 2 * ks + half);
#pragma unroll
      for (int t = 0; t < S::RT; ++t)
#pragma unroll
        for (int u = 0; u < S::CT; ++u) acc[t][u] = mfma32(af[t], bf[u], acc[t][u]);
    }
  }

#pragma unroll
  for (int u = 0; u < S::CT; ++u) {
    const int qi = q0 + S::RN * wn + 32 * u + col;
    if (qi >= sg.lq) continue;
    uint16_t* dqp = a.dq.p + s * a.dq.sb + (int64_t)(sg.q_row0 + qi) * a.dq.sn + h * a.dq.sh +
                    dh * OB;
#pragma unroll
    for (int t = 0; t < S::RT; ++t)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        uint16_t* dst = dqp + S::RM * wm + 32 * t + rr * 8 + half * 4;
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
        for (int e = 0; e < 4; ++e) v4[e] = (elem_t)(acc[t][u][rr * 4 + e] * a.scale + add[e]);
        *reinterpret_cast<elem4*>(dst) = v4;
      }
  }
}

}  // namespace VCA_ELEM
}  // namespace vca
