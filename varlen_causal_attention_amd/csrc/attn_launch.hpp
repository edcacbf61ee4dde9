// Host-side launchers of the attention kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>

#include "attn_args.hpp"

namespace vca {

// ---------------------------------------------------------------------------
// merge of two partial results ("gemma4_moe cp_attention" page, -inf-safe
// merge): one wave per (row, head); lanes cover the head dim.
// ---------------------------------------------------------------------------
struct MergeArgs {
  const void* out_a;
  const void* out_b;
  int a_type, b_type;  // ATTN_BF16, ATTN_F32 or ATTN_F16
  const float* lse_a;
  const float* lse_b;
  float* out;
  float* lse;
  uint16_t* out_copy;  // optional 16-bit copy of out, of copy_type
  int copy_type;       // ATTN_BF16 or ATTN_F16
  int rows, H, Dv;
};


// Head-dim pairs compiled into the library.
bool head_dims_supported(int dqk, int dv);

// Work lists: every pass orders its (segment, tile) items heaviest first.
// The list capacity is bounded with 32-row tiles, the smallest any pass uses.
constexpr int kListRows = 32;
inline size_t list_capacity(int64_t rows, int nseg) { return (size_t)((rows + kListRows - 1) / kListRows) + nseg; }
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
// forward workspace: [count][list]
inline size_t fwd_workspace_bytes(int64_t q_rows, int nseg) {
  return 256 + align256(sizeof(int2) * list_capacity(q_rows, nseg));
}
// Backward workspace: [delta fp32, one per (q-head, query row)][counts]
// [query list][key list][lse*log2(e), like delta], then for the two-phase
// backward the P and dS block stores (bf16, 256x256 per (row slot, key block,
// q-head)).
constexpr int kBlockRows = 256;
struct TileGeom {
  int64_t slots;  // 256-query row slots
  int nkb;        // 256-key blocks per slot
  int nqb_dense;  // dense: query blocks per batch (slot = b*nqb + qb); 0: varlen
  // dS store (BwdArgs::ds): 32-row query tiles of the layout, 32-key tiles
  // per query tile, dense query tiles per batch (0: varlen)
  int64_t ds_nqt;
  int ds_mkt, ds_qtb;
};
inline TileGeom tile_geom_dense(int B, int Nq, int Nk) {
  const int nqb = (Nq + kBlockRows - 1) / kBlockRows;
  const int qtb = (Nq + 31) / 32;
  return TileGeom{(int64_t)B * nqb, (Nk + kBlockRows - 1) / kBlockRows, nqb, (int64_t)B * qtb,
                  (Nk + 31) / 32, qtb};
}
inline TileGeom tile_geom_varlen(int Tq, int nseg, int max_k) {
  // a segment's query tiles start at (first row) / 32 + segment index: the
  // tiles of consecutive segments never collide and stay below Tq/32 + nseg
  return TileGeom{(int64_t)Tq / kBlockRows + nseg + 1, (max_k + kBlockRows - 1) / kBlockRows, 0,
                  (int64_t)Tq / 32 + nseg, (max_k + 31) / 32, 0};
}
// Head-dim pairs whose backward runs in two phases through stored blocks.
inline bool bwd_uses_tiles(int dqk, int dv) {
  return dqk == dv && (dqk == 256 || dqk == 512);
}
// Head-dim pairs whose dQ pass can read dS blocks stored by the dK/dV pass
// instead of recomputing S and dP.
inline bool bwd_can_store_ds(int dqk, int dv) {
  return (dqk == 128 && dv == 128) || (dqk == 192 && dv == 128);
}
// Byte budget of the dS store: ATTN_BWD_DS_MIB (MiB; 0 turns the store off),
// default 8192. The store holds every visible 32x32 block of the q-heads of
// one launch; when even one GQA group's blocks exceed the budget the dQ pass
// recomputes S and dP instead.
size_t ds_budget_bytes();
// Byte budget of the two-phase P and dS block stores: ATTN_BWD_TILES_MIB
// (MiB), default 8192. The stores hold the blocks of as many 256-query row
// slots as fit (at least one); more slots run as consecutive chunks whose
// dK/dV sums meet in fp32 accumulators.
size_t tiles_budget_bytes();
struct BwdWorkspace {
  size_t list_q, list_k, lse2, tile_p, tile_ds, ds, total;
  int ds_kv_chunk;  // kv-heads per dK/dV + dQ launch pair of the dS path; 0: no dS store
  int64_t tile_chunk_slots;  // row slots per chunk of the two-phase backward
  size_t tile_acc_dk, tile_acc_dv;  // fp32 dK / dV accumulators (several chunks only)
};
inline BwdWorkspace bwd_workspace(int dqk, int dv, int Hq, int Hkv, int64_t q_rows, int64_t k_rows,
                                  int nseg, const TileGeom& tg) {
  BwdWorkspace w{};
  const size_t delta = align256(sizeof(float) * (size_t)Hq * (size_t)q_rows);
  w.list_q = delta + 256;
  w.list_k = w.list_q + align256(sizeof(int2) * list_capacity(q_rows, nseg));
  w.lse2 = w.list_k + align256(sizeof(int2) * list_capacity(k_rows, nseg));
  w.tile_p = w.lse2 + delta;
  w.tile_ds = w.tile_p;
  w.ds = w.tile_p;
  if (bwd_can_store_ds(dqk, dv) && Hkv > 0 && q_rows > 0 && k_rows > 0 && tg.ds_mkt > 0) {
    const size_t per_head = sizeof(uint16_t) * 1024 * (size_t)tg.ds_nqt * (size_t)tg.ds_mkt;
    const size_t group = per_head * (size_t)(Hq / Hkv);
    const size_t budget = ds_budget_bytes();
    if (group <= budget) {
      const size_t n = budget / group;
      w.ds_kv_chunk = (int)(n < (size_t)Hkv ? n : (size_t)Hkv);
      w.total = w.ds + align256(group * (size_t)w.ds_kv_chunk);
      return w;
    }
  }
  if (bwd_uses_tiles(dqk, dv)) {
    // one row slot's P (or dS) blocks over every key block and q-head
    const size_t per_slot =
        sizeof(uint16_t) * kBlockRows * kBlockRows * (size_t)tg.nkb * (size_t)Hq;
    int64_t chunk = tg.slots;
    if (per_slot > 0) {
      const int64_t fit = (int64_t)(tiles_budget_bytes() / (2 * per_slot));
      chunk = fit < 1 ? 1 : (fit < tg.slots ? fit : tg.slots);
    }
    w.tile_chunk_slots = chunk;
    const size_t blocks = per_slot * (size_t)chunk;
    w.tile_ds = w.tile_p + blocks;
    w.total = w.tile_ds + blocks;
    if (chunk < tg.slots) {
      w.tile_acc_dk = w.total;
      w.tile_acc_dv = w.tile_acc_dk + align256(sizeof(float) * (size_t)k_rows * Hkv * dqk);
      w.total = w.tile_acc_dv + align256(sizeof(float) * (size_t)k_rows * Hkv * dv);
    }
  } else {
    w.total = w.tile_p;
  }
  return w;
}

// Launchers of one element type, defined in the kernel translation units
// (compiled once per type: vca::bf for bf16, vca::hf for fp16); their
// arguments are the same for both.
namespace bf {
// Scheduler launch + forward kernel. ws: the forward workspace. q_rows: Tq
// (varlen) or B * Nq (dense), used for the list capacity.
hipError_t launch_fwd(FwdArgs a, int dqk, int dv, bool causal, int nseg, int Hq, int64_t q_rows,
                      void* ws, hipStream_t stream);

// delta pre-pass, then either the fused dK/dV and dQ passes or the two-phase
// scores + products passes, in that order on one stream. ws: the backward
// workspace laid out by bwd_workspace (delta first).
hipError_t launch_bwd(BwdArgs a, int dqk, int dv, bool causal, int nseg, int Hq, int Hkv,
                      int max_q, int64_t q_rows, int64_t k_rows, const TileGeom& tg, void* ws,
                      hipStream_t stream);

// Work lists of the backward (query tiles of q_tile rows costed in q_step
// keys, key blocks of k_tile keys costed in k_step queries) and the delta
// pre-pass; fills the list fields of a.
void bwd_prepare(BwdArgs& a, int dv, bool causal, int nseg, int Hq, int Hkv, int max_q,
                 int64_t q_rows, int64_t k_rows, const BwdWorkspace& wl, int q_tile, int q_step,
                 int k_tile, int k_step, void* ws, hipStream_t st);

// dK/dV pass of head dim 128 with split wave roles (attn_bwd_roles.hip);
// grid = (128-key blocks + segments) * Hkv.
hipError_t launch_dkdv_roles(const BwdArgs& a, bool causal, unsigned grid, hipStream_t st);
hipError_t launch_dkdv_roles192(const BwdArgs& a, bool causal, unsigned grid, hipStream_t st);

// Two-phase backward (the head-dim pairs bwd_uses_tiles names): lists,
// delta, scores, products.
hipError_t launch_bwd_tiles(BwdArgs a, int dqk, int dv, bool causal, int nseg, int Hq, int Hkv,
                            int max_q, int64_t q_rows, int64_t k_rows, const TileGeom& tg,
                            const BwdWorkspace& wl, void* ws, hipStream_t st);
}  // namespace bf
namespace hf {
// Scheduler launch + forward kernel. ws: the forward workspace. q_rows: Tq
// (varlen) or B * Nq (dense), used for the list capacity.
hipError_t launch_fwd(FwdArgs a, int dqk, int dv, bool causal, int nseg, int Hq, int64_t q_rows,
                      void* ws, hipStream_t stream);

// delta pre-pass, then either the fused dK/dV and dQ passes or the two-phase
// scores + products passes, in that order on one stream. ws: the backward
// workspace laid out by bwd_workspace (delta first).
hipError_t launch_bwd(BwdArgs a, int dqk, int dv, bool causal, int nseg, int Hq, int Hkv,
                      int max_q, int64_t q_rows, int64_t k_rows, const TileGeom& tg, void* ws,
                      hipStream_t stream);

// Work lists of the backward (query tiles of q_tile rows costed in q_step
// keys, key blocks of k_tile keys costed in k_step queries) and the delta
// pre-pass; fills the list fields of a.
void bwd_prepare(BwdArgs& a, int dv, bool causal, int nseg, int Hq, int Hkv, int max_q,
                 int64_t q_rows, int64_t k_rows, const BwdWorkspace& wl, int q_tile, int q_step,
                 int k_tile, int k_step, void* ws, hipStream_t st);

// dK/dV pass of head dim 128 with split wave roles (attn_bwd_roles.hip);
// grid = (128-key blocks + segments) * Hkv.
hipError_t launch_dkdv_roles(const BwdArgs& a, bool causal, unsigned grid, hipStream_t st);
hipError_t launch_dkdv_roles192(const BwdArgs& a, bool causal, unsigned grid, hipStream_t st);

// Two-phase backward (the head-dim pairs bwd_uses_tiles names): lists,
// delta, scores, products.
hipError_t launch_bwd_tiles(BwdArgs a, int dqk, int dv, bool causal, int nseg, int Hq, int Hkv,
                            int max_q, int64_t q_rows, int64_t k_rows, const TileGeom& tg,
                            const BwdWorkspace& wl, void* ws, hipStream_t st);
}  // namespace hf

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream);

// rows a dense ring chunk must not produce: out rows to 0, lse to -inf
struct ZeroRowsArgs {
  void* out;
  int f32;  // 0: 16-bit elements (bf16 or fp16), 1: fp32
  int64_t ob, oh, on;
  float* lse;
  int64_t lse_sb, lse_sh;
  const uint8_t* rows;  // [B, S]
  int B, H, S, D;
};
hipError_t launch_zero_rows(const ZeroRowsArgs& a, hipStream_t stream);

// Row movement and merges of the packed ring layout (attn_ring.hip).
struct RingRowsArgs {
  void* dense;           // [B, H, S, D] view, element strides sb, sh, sn (innermost 1)
  int64_t sb, sh, sn;
  void* packed;          // [T, H, D] contiguous
  const int32_t* index;  // [T] flat rows b*S + s
  float* lse_dense;      // [B, H, S] contiguous (or NULL)
  float* lse_packed;     // [H, T] contiguous
  int B, H, S, T, D;
  int type, esz;         // dtype code and its byte size
  int dst_type;          // mode 3: the 16-bit type fp32 rows are gathered into
  int mode;              // rows: 0 gather, 1 scatter, 2 scatter-add, 3 gather fp32 -> 16-bit;
                         // lse: 0 gather, 1 scatter
};
enum { kRingRows = 0, kRingFill = 1, kRingLse = 2, kRingMerge = 3 };
hipError_t launch_ring_rows(const RingRowsArgs& a, int op, hipStream_t stream);

}  // namespace vca
