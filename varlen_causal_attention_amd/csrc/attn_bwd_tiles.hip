// Launcher of the two-phase backward (scores, then dV/dK and dQ products).
#include "attn_bwd_tiles.hpp"
#include "attn_launch.hpp"
#include "attn_timing.hpp"

namespace vca {
namespace {

template <int D, bool CAUSAL>
hipError_t bwd_tiles(BwdArgs a, int nseg, int Hq, int Hkv, int max_q, int64_t q_rows, int64_t k_rows,
                     const TileGeom& tg, const BwdWorkspace& wl, void* ws, hipStream_t st) {
  bwd_prepare(a, D, CAUSAL, nseg, Hq, Hkv, max_q, q_rows, k_rows, wl, kBlk, kBlk, kBlk, kBlk, ws, st);
  char* w = static_cast<char*>(ws);
  a.tile_p = reinterpret_cast<uint16_t*>(w + wl.tile_p);
  a.tile_ds = reinterpret_cast<uint16_t*>(w + wl.tile_ds);
  a.tile_nkb = tg.nkb;
  a.tile_nqb_dense = tg.nqb_dense;
  const unsigned q_items = (unsigned)((q_rows + kBlk - 1) / kBlk + nseg);
  const unsigned k_items = (unsigned)((k_rows + kBlk - 1) / kBlk + nseg);
  if (q_rows > 0 && k_rows > 0) {
    TimedLaunch timer("attn_bwd_scores", st);
    hipLaunchKernelGGL((attn_bwd_scores_kernel<D, D, CAUSAL>),
                       dim3(xcd_grid<kScoreSplit>(q_items * Hq)), dim3(kNT), 0, st, a);
  }
  if (k_rows > 0) {
    TimedLaunch timer("attn_bwd_dkdv_tiles", st);
    hipLaunchKernelGGL((attn_bwd_dkdv_tiles_kernel<D, CAUSAL>),
                       dim3(xcd_grid<2 * (D / kBlk)>(k_items * Hkv)), dim3(kNT), 0, st, a);
  }
  if (q_rows > 0) {
    TimedLaunch timer("attn_bwd_dq_tiles", st);
    hipLaunchKernelGGL((attn_bwd_dq_tiles_kernel<D, CAUSAL>),
                       dim3(xcd_grid<D / kBlk>(q_items * Hq)), dim3(kNT), 0, st, a);
  }
  return hipGetLastError();
}

template <int D>
hipError_t bwd_tiles_any(BwdArgs a, bool causal, int nseg, int Hq, int Hkv, int max_q,
                         int64_t q_rows, int64_t k_rows, const TileGeom& tg,
                         const BwdWorkspace& wl, void* ws, hipStream_t st) {
  return causal ? bwd_tiles<D, true>(a, nseg, Hq, Hkv, max_q, q_rows, k_rows, tg, wl, ws, st)
                : bwd_tiles<D, false>(a, nseg, Hq, Hkv, max_q, q_rows, k_rows, tg, wl, ws, st);
}

}  // namespace

hipError_t launch_bwd_tiles(BwdArgs a, int d, bool causal, int nseg, int Hq, int Hkv, int max_q,
                            int64_t q_rows, int64_t k_rows, const TileGeom& tg,
                            const BwdWorkspace& wl, void* ws, hipStream_t st) {
  if (d == 256)
    return bwd_tiles_any<256>(a, causal, nseg, Hq, Hkv, max_q, q_rows, k_rows, tg, wl, ws, st);
  if (d == 512)
    return bwd_tiles_any<512>(a, causal, nseg, Hq, Hkv, max_q, q_rows, k_rows, tg, wl, ws, st);
  return hipErrorInvalidValue;
}

}  // namespace vca
