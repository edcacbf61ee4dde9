// Argument structures shared by the C ABI and the kernels of both element
// types (pointers to 16-bit elements are element-type agnostic).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vca {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// Tensor view: element (seg-or-batch b, row, head h, d) lives at
// base + b*sb + row*sn + h*sh + d. Varlen views have sb = 0 and rows offset by
// the segment's first row.
struct View {
  const uint16_t* p;
  int64_t sb, sh, sn;
};
struct ViewW {
  uint16_t* p;
  int64_t sb, sh, sn;
};

// Segment geometry: query rows [q_row0, q_row0 + lq) and key rows
// [k_row0, k_row0 + lk) of the packed tensors.
struct SegGeom {
  int q_row0, lq, k_row0, lk;
};

// forward: query rows per work item (four waves of 32)
constexpr int kFwdWaves = 4;
constexpr int kFwdBM = 32 * kFwdWaves;

struct FwdArgs {
  View q, k, v;
  ViewW o;
  float* lse;
  int64_t lse_sb, lse_sh;  // lse index = b*lse_sb + h*lse_sh + (q_row0 + i)
  const int32_t* cu_q;
  const int32_t* cu_k;
  int Nq, Nk, Tq, Tk;
  int G;            // Hq / Hkv
  int H;            // q-heads: blockIdx.x = item * H + head
  float scale_log2; // scale * log2(e)
  // Left window and logit softcap (FwdArgs and BwdArgs alike): window > 0
  // keeps only the keys j > i + (lk - lq) - window of a causal row; with
  // cap_in != 0 the scaled score x = scale * q.k becomes cap * tanh(x / cap),
  // computed as cap_out * tanh(cap_in * q.k) with cap_in = |scale| / cap (a
  // negative scale is folded into q) and cap_out = cap * log2(e).
  int window;
  float cap_in, cap_out;
  const int2* items;      // (segment, q tile) heavy first
  const int* item_count;
};

struct BwdArgs {
  View q, k, v, o, dout;
  ViewW dq, dk, dv;
  const float* lse;
  float* delta;            // workspace, same indexing as lse
  float* lse2;             // workspace: lse * log2(e) (+inf where lse = -inf), same indexing
  int64_t lse_sb, lse_sh;  // index = b*lse_sb + h*lse_sh + (q_row0 + i)
  const int32_t* cu_q;
  const int32_t* cu_k;
  int Nq, Nk, Tq, Tk;
  int G;
  float scale, scale_log2, inv_scale;  // inv_scale = 1 / scale (scale != 0)
  int window;             // as in FwdArgs
  float cap_in, cap_out;  // as in FwdArgs, with cap_in = scale / cap (signed)
  int dq_accumulate;
  int Hq, Hkv;
  const int2* items_q;    // (segment, query tile) for the dQ pass, heavy first
  const int* count_q;
  const int2* items_k;    // (segment, key block) for the dK/dV pass, heavy first
  const int* count_k;
  // two-phase backward only: bf16 P and dS tiles (workspace) and their layout
  uint16_t* tile_p;
  uint16_t* tile_ds;
  int tile_nkb;        // key tiles per row slot
  int tile_nqb_dense;  // dense: query tiles per batch; 0 for varlen
  int nq_items, nk_items;  // list capacities (grid sizes) of the two-phase passes
  // The store holds the row slots slot_lo .. slot_hi - 1 of one chunk (slot
  // s at (s - slot_lo)); the passes of a chunk touch only those query
  // blocks. acc_mode: 0 one chunk, dK/dV written directly; 1 first chunk,
  // 2 middle chunk, 3 last chunk: the dK/dV sums of the chunk go to
  // (1: =, 2: +=) the fp32 rows acc_dk / acc_dv ([key row][kv-head][D],
  // key row = batch * Nk + segment row), and the last chunk writes acc +
  // its sums to dk / dv.
  int slot_lo, slot_hi;
  int acc_mode;
  float* acc_dk;
  float* acc_dv;
  // kv-heads of this launch of a dK/dV pass: kvh0 .. kvh0 + kvh_n - 1
  int kvh0, kvh_n;
  // dS store (head dims 128 and 192/128): when ds is set, the dK/dV pass
  // writes every visible 32x32 block of dS (bf16) there and the dQ pass
  // reads them instead of recomputing S and dP. Block (q-head h, query tile
  // qt of a segment, key tile kt) sits at element
  //   (((h - ds_h0) * ds_nqt + qt_flat) * ds_mkt + kt) * 1024,
  // qt_flat = (first query row of the segment) / 32 + segment + qt (varlen)
  // or batch * ds_qtb + qt (dense, ds_qtb = ceil(Nq / 32)). A block is kept
  // in the order the dK/dV pass holds it: two MFMA B fragments of 64 lanes x
  // 8 bf16 (element 512 j + 8 l + e); lane l holds key l % 32, fragment j
  // the queries 16j + 4h + e (e < 4) and 16j + 8 + 4h + (e - 4) (e >= 4),
  // h = l / 32. Each store and load of a fragment moves 1 KB contiguously.
  uint16_t* ds;
  int ds_h0, ds_nh, ds_nqt, ds_mkt, ds_qtb;
};

}  // namespace vca
