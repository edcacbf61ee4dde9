// Launcher of the two-phase backward (scores, then dV/dK and dQ products).
#include "attn_bwd_tiles.hpp"
#include "attn_launch.hpp"
#include "attn_sched.hpp"
#include "attn_timing.hpp"

namespace vca {
namespace VCA_ELEM {
namespace {

template <int DQK, int DV, bool CAUSAL>
hipError_t bwd_tiles(BwdArgs a, int nseg, int Hq, int Hkv, int max_q, int64_t q_rows, int64_t k_rows,
                     const TileGeom& tg, const BwdWorkspace& wl, void* ws, hipStream_t st) {
  constexpr int OBQ = prod_block(DQK), OBV = prod_block(DV);
  bwd_prepare(a, DV, CAUSAL, nseg, Hq, Hkv, max_q, q_rows, k_rows, wl, kBlk, kBlk, kBlk, kBlk, ws,
              st);
  char* w = static_cast<char*>(ws);
  a.tile_p = reinterpret_cast<uint16_t*>(w + wl.tile_p);
  a.tile_ds = reinterpret_cast<uint16_t*>(w + wl.tile_ds);
  a.tile_nkb = tg.nkb;
  a.tile_nqb_dense = tg.nqb_dense;
  const unsigned q_items = (unsigned)((q_rows + kBlk - 1) / kBlk + nseg);
  const unsigned k_items = (unsigned)((k_rows + kBlk - 1) / kBlk + nseg);
  a.nq_items = (int)q_items;
  a.nk_items = (int)k_items;
  // The P/dS stores hold wl.tile_chunk_slots row slots: the three passes run
  // once per chunk of slots; with several chunks the dK/dV sums of each meet
  // in fp32 (first chunk stores, middle ones add, the last one writes dk/dv).
  const int64_t chunk = wl.tile_chunk_slots > 0 ? wl.tile_chunk_slots : tg.slots;
  const int64_t nchunks = tg.slots > 0 ? (tg.slots + chunk - 1) / chunk : 1;
  a.acc_dk = nchunks > 1 ? reinterpret_cast<float*>(w + wl.tile_acc_dk) : nullptr;
  a.acc_dv = nchunks > 1 ? reinterpret_cast<float*>(w + wl.tile_acc_dv) : nullptr;
  for (int64_t c = 0; c < nchunks; ++c) {
    a.slot_lo = (int)(c * chunk);
    a.slot_hi = (int)min(tg.slots, (c + 1) * chunk);
    a.acc_mode = nchunks == 1 ? 0 : (c == 0 ? 1 : (c + 1 < nchunks ? 2 : 3));
    if (q_rows > 0 && k_rows > 0) {
      TimedLaunch timer("attn_bwd_scores", st);
      // the left window and the softcap (ext) take their own scores kernel;
      // the product passes read the window's block ranges at run time
      const dim3 grid(xcd_grid<kScoreSplit>(q_items * Hq));
      if (a.cap_in != 0.f)
        hipLaunchKernelGGL((attn_bwd_scores_kernel<DQK, DV, CAUSAL, 2>), grid, dim3(kNT), 0, st, a);
      else if (a.window > 0)
        hipLaunchKernelGGL((attn_bwd_scores_kernel<DQK, DV, CAUSAL, 1>), grid, dim3(kNT), 0, st, a);
      else
        hipLaunchKernelGGL((attn_bwd_scores_kernel<DQK, DV, CAUSAL>), grid, dim3(kNT), 0, st, a);
    }
    if (k_rows > 0) {
      TimedLaunch timer("attn_bwd_dkdv_tiles", st);
      if constexpr (DQK == DV) {
        // dV and dK blocks of one launch, side by side
        hipLaunchKernelGGL((attn_bwd_dkdv_tiles_kernel<DV, OBV, CAUSAL, 2>),
                           dim3(xcd_grid<2 * (DV / OBV)>(k_items * Hkv)), dim3(kNT), 0, st, a);
      } else {
        hipLaunchKernelGGL((attn_bwd_dkdv_tiles_kernel<DV, OBV, CAUSAL, 0>),
                           dim3(xcd_grid<DV / OBV>(k_items * Hkv)), dim3(kNT), 0, st, a);
        hipLaunchKernelGGL((attn_bwd_dkdv_tiles_kernel<DQK, OBQ, CAUSAL, 1>),
                           dim3(xcd_grid<DQK / OBQ>(k_items * Hkv)), dim3(kNT), 0, st, a);
      }
    }
    if (q_rows > 0) {
      TimedLaunch timer("attn_bwd_dq_tiles", st);
      hipLaunchKernelGGL((attn_bwd_dq_tiles_kernel<DQK, OBQ, CAUSAL>),
                         dim3(xcd_grid<DQK / OBQ>(q_items * Hq)), dim3(kNT), 0, st, a);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipGetLastError();
}

template <int DQK, int DV>
hipError_t bwd_tiles_any(BwdArgs a, bool causal, int nseg, int Hq, int Hkv, int max_q,
                         int64_t q_rows, int64_t k_rows, const TileGeom& tg,
                         const BwdWorkspace& wl, void* ws, hipStream_t st) {
  return causal
             ? bwd_tiles<DQK, DV, true>(a, nseg, Hq, Hkv, max_q, q_rows, k_rows, tg, wl, ws, st)
             : bwd_tiles<DQK, DV, false>(a, nseg, Hq, Hkv, max_q, q_rows, k_rows, tg, wl, ws, st);
}

}  // namespace

hipError_t launch_bwd_tiles(BwdArgs a, int dqk, int dv, bool causal, int nseg, int Hq, int Hkv,
                            int max_q, int64_t q_rows, int64_t k_rows, const TileGeom& tg,
                            const BwdWorkspace& wl, void* ws, hipStream_t st) {
#define VCA_TILES(DQK, DV)                                                                       \
  if (dqk == DQK && dv == DV)                                                                    \
    return bwd_tiles_any<DQK, DV>(a, causal, nseg, Hq, Hkv, max_q, q_rows, k_rows, tg, wl, ws, st);
  VCA_TILES(256, 256)
  VCA_TILES(512, 512)
#undef VCA_TILES
  return hipErrorInvalidValue;
}

}  // namespace VCA_ELEM
}  // namespace vca
