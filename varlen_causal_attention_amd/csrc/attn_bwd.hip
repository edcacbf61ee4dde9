// Backward launcher: delta pre-pass, then for every compiled head-dim pair
// either the fused dK/dV and dQ passes or the two-phase scores + products
// passes (their own translation unit, attn_bwd_tiles.hip).
#include "attn_bwd.hpp"
#include "attn_launch.hpp"
#include "attn_sched.hpp"
#include "attn_timing.hpp"

namespace vca {
namespace VCA_ELEM {
namespace {

// Work lists (query tiles of q_tile rows with key steps of q_step, key blocks
// of k_tile keys with query steps of k_step) and, when delta_pass, the delta
// pre-pass (the fused path's dQ pass computes delta itself). seg_major_lists puts
// both lists in segment-major order: the query tiles (key blocks) of one
// segment and head then read its K/V (Q/dO) in step and share them in L2,
// which pays where no GQA group of q-heads already shares each stream
// (192/128 backward -3.5%, D=512 -1%; with a group of four at D=128 the
// heavy-first order stays faster).
template <int DV>
void bwd_prologue(BwdArgs& a, bool causal, int nseg, int Hq, int Hkv, int max_q, int64_t q_rows,
                  int64_t k_rows, const BwdWorkspace& wl, int q_tile, int q_step, int k_tile,
                  int k_step, void* ws, hipStream_t st, bool delta_pass = true,
                  int seg_major_lists = 1) {
  char* w = static_cast<char*>(ws);
  const size_t delta_bytes = wl.list_q - 256;
  int* counts = reinterpret_cast<int*>(w + delta_bytes);
  int2* list_q = reinterpret_cast<int2*>(w + wl.list_q);
  int2* list_k = reinterpret_cast<int2*>(w + wl.list_k);
  SchedArgs sa{};
  sa.cu_q = a.cu_q;
  sa.cu_k = a.cu_k;
  sa.nseg = nseg;
  sa.Nq = a.Nq;
  sa.Nk = a.Nk;
  sa.Tq = a.Tq;
  sa.Tk = a.Tk;
  sa.causal = causal;
  // query tiles, cost = key steps walked
  sa.by_keys = 0;
  sa.tile = q_tile;
  sa.step = q_step;
  sa.list = list_q;
  sa.count = counts;
  sa.max_items = (int)list_capacity(q_rows, nseg);
  sa.seg_major = seg_major_lists;
  SchedArgs2 s2{};
  s2.list[0] = sa;
  // key blocks, cost = query steps walked
  sa.by_keys = 1;
  sa.tile = k_tile;
  sa.step = k_step;
  sa.list = list_k;
  sa.count = counts + 1;
  sa.max_items = (int)list_capacity(k_rows, nseg);
  s2.list[1] = sa;
  {
    TimedLaunch timer("attn_schedule", st);
    hipLaunchKernelGGL(attn_schedule2_kernel, dim3(2), dim3(1024), 0, st, s2);
  }
  a.lse2 = reinterpret_cast<float*>(w + wl.lse2);
  a.items_q = list_q;
  a.count_q = counts;
  a.items_k = list_k;
  a.count_k = counts + 1;
  a.Hq = Hq;
  a.Hkv = Hkv;

  constexpr int LPR = DV / 8 >= 64 ? 64 : DV / 8;
  constexpr int rows_per_block = 4 * (64 / LPR);
  if (delta_pass && max_q > 0) {
    TimedLaunch timer("attn_bwd_delta", st);
    const dim3 g((max_q + rows_per_block - 1) / rows_per_block, Hq, nseg);
    hipLaunchKernelGGL((attn_bwd_delta_kernel<DV>), g, dim3(256), 0, st, a);
  }
}

// NWK waves per dK/dV workgroup. The left window and the softcap (ext) take
// the generic dK/dV kernel at every head dim (same 128-key blocks).
template <int DQK, int DV, int NWK>
hipError_t launch_dkdv(const BwdArgs& a, bool causal, bool ext, unsigned grid, hipStream_t st) {
  constexpr bool kPipe = DQK == DV;  // software-pipelined dK/dV
  TimedLaunch timer("attn_bwd_dkdv", st);
  if (ext) {
    if (causal)
      hipLaunchKernelGGL((attn_bwd_dkdv_kernel<DQK, DV, NWK, true, true>), dim3(grid),
                         dim3(64 * NWK), 0, st, a);
    else
      hipLaunchKernelGGL((attn_bwd_dkdv_kernel<DQK, DV, NWK, false, true>),
                         dim3(grid), dim3(64 * NWK), 0, st, a);
  } else if constexpr (kPipe && DQK == 128) {
    const hipError_t e = launch_dkdv_roles(a, causal, grid, st);
    if (e != hipSuccess) return e;
  } else if constexpr (DQK == 192 && DV == 128 && NWK == 4) {
    const hipError_t e = launch_dkdv_roles192(a, causal, grid, st);
    if (e != hipSuccess) return e;
  } else if constexpr (kPipe) {
    if (causal)
      hipLaunchKernelGGL((attn_bwd_dkdv_pipe_kernel<DQK, true>), dim3(grid), dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((attn_bwd_dkdv_pipe_kernel<DQK, false>), dim3(grid), dim3(256), 0, st, a);
  } else {
    if (causal)
      hipLaunchKernelGGL((attn_bwd_dkdv_kernel<DQK, DV, NWK, true>), dim3(grid),
                         dim3(64 * NWK), 0, st, a);
    else
      hipLaunchKernelGGL((attn_bwd_dkdv_kernel<DQK, DV, NWK, false>), dim3(grid),
                         dim3(64 * NWK), 0, st, a);
  }
  return hipGetLastError();
}

// BN keys per dQ tile, WPE waves per SIMD the dQ register budget targets,
// NWK / NWQ waves per dK/dV / dQ workgroup.
template <int DQK, int DV, int BN, int WPE, int NWK, int NWQ>
hipError_t bwd_dims(BwdArgs a, bool causal, int nseg, int Hq, int Hkv, int max_q, int64_t q_rows,
                    int64_t k_rows, const TileGeom& tg, const BwdWorkspace& wl, void* ws,
                    hipStream_t st) {
  constexpr bool kPipe = DQK == DV;  // software-pipelined dK/dV
  constexpr int key_block = kPipe ? 128 : 32 * NWK;
  static_assert(key_block == 32 * NWK, "the generic dK/dV kernel takes the same blocks");
  constexpr int q_tile = 32 * NWQ;
  const bool ext = a.window > 0 || a.cap_in != 0.f;
  const int seg_major = (Hq / Hkv) % 2 == 0 ? 0 : 1;
  const int G = Hq / Hkv;
  a.kvh0 = 0;
  a.kvh_n = Hkv;
  a.ds = nullptr;
  if constexpr (DQK == 128 || DQK == 192) {
    if (wl.ds_kv_chunk > 0) {
      // dS store: the delta pre-pass, then per chunk of kv-heads the dK/dV
      // pass (which writes the chunk's dS blocks) and the dQ pass over them
      static_assert(key_block == 128, "dS blocks of 32 keys inside 128-key blocks");
      constexpr int dq_waves = 8;
      constexpr int dq_tile = 32 * dq_waves;
      bwd_prologue<DV>(a, causal, nseg, Hq, Hkv, max_q, q_rows, k_rows, wl, dq_tile, 32,
                       key_block, 32, ws, st, /*delta_pass=*/true, seg_major);
      a.ds = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + wl.ds);
      a.ds_nqt = (int)tg.ds_nqt;
      a.ds_mkt = tg.ds_mkt;
      a.ds_qtb = tg.ds_qtb;
      const unsigned kitems = (unsigned)((k_rows + key_block - 1) / key_block + nseg);
      const unsigned qitems = (unsigned)((q_rows + dq_tile - 1) / dq_tile + nseg);
      for (int g0 = 0; g0 < Hkv; g0 += wl.ds_kv_chunk) {
        const int n = min(wl.ds_kv_chunk, Hkv - g0);
        a.kvh0 = g0;
        a.kvh_n = n;
        a.ds_h0 = g0 * G;
        a.ds_nh = n * G;
        hipError_t e = launch_dkdv<DQK, DV, NWK>(a, causal, ext, kitems * n, st);
        if (e != hipSuccess) return e;
        TimedLaunch timer("attn_bwd_dq_ds", st);
        const dim3 g(qitems * (unsigned)(n * G));
        if (causal)
          hipLaunchKernelGGL((attn_bwd_dq_ds_kernel<DQK, dq_waves, true>), g, dim3(64 * dq_waves),
                             0, st, a);
        else
          hipLaunchKernelGGL((attn_bwd_dq_ds_kernel<DQK, dq_waves, false>), g, dim3(64 * dq_waves),
                             0, st, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
      }
      return hipSuccess;
    }
  }
  bwd_prologue<DV>(a, causal, nseg, Hq, Hkv, max_q, q_rows, k_rows, wl, q_tile, BN, key_block, 32,
                   ws, st,
                   /*delta_pass=*/false, seg_major);
  // the dQ pass first: it writes the delta and lse*log2(e) rows the dK/dV
  // pass reads
  if (q_rows > 0) {
    TimedLaunch timer("attn_bwd_dq", st);
    const dim3 g((unsigned)(((q_rows + q_tile - 1) / q_tile + nseg) * Hq));
    if (causal && ext)
      hipLaunchKernelGGL((attn_bwd_dq_kernel<DQK, DV, BN, WPE, NWQ, true, true>), g,
                         dim3(64 * NWQ), 0, st, a);
    else if (causal)
      hipLaunchKernelGGL((attn_bwd_dq_kernel<DQK, DV, BN, WPE, NWQ, true>), g,
                         dim3(64 * NWQ), 0, st, a);
    else if (ext)
      hipLaunchKernelGGL((attn_bwd_dq_kernel<DQK, DV, BN, WPE, NWQ, false, true>), g,
                         dim3(64 * NWQ), 0, st, a);
    else
      hipLaunchKernelGGL((attn_bwd_dq_kernel<DQK, DV, BN, WPE, NWQ, false>), g,
                         dim3(64 * NWQ), 0, st, a);
  }
  if (k_rows > 0) {
    const hipError_t e = launch_dkdv<DQK, DV, NWK>(
        a, causal, ext, (unsigned)(((k_rows + key_block - 1) / key_block + nseg) * Hkv), st);
    if (e != hipSuccess) return e;
  }
  return hipGetLastError();
}

}  // namespace


void bwd_prepare(BwdArgs& a, int dv, bool causal, int nseg, int Hq, int Hkv, int max_q,
                 int64_t q_rows, int64_t k_rows, const BwdWorkspace& wl, int q_tile, int q_step,
                 int k_tile, int k_step, void* ws, hipStream_t st) {
  switch (dv) {
    case 64:
      return bwd_prologue<64>(a, causal, nseg, Hq, Hkv, max_q, q_rows, k_rows, wl, q_tile, q_step,
                              k_tile, k_step, ws, st);
    case 128:
      return bwd_prologue<128>(a, causal, nseg, Hq, Hkv, max_q, q_rows, k_rows, wl, q_tile, q_step,
                               k_tile, k_step, ws, st);
    case 256:
      return bwd_prologue<256>(a, causal, nseg, Hq, Hkv, max_q, q_rows, k_rows, wl, q_tile, q_step,
                               k_tile, k_step, ws, st);
    default:
      return bwd_prologue<512>(a, causal, nseg, Hq, Hkv, max_q, q_rows, k_rows, wl, q_tile, q_step,
                               k_tile, k_step, ws, st);
  }
}

hipError_t launch_bwd(BwdArgs a, int dqk, int dv, bool causal, int nseg, int Hq, int Hkv, int max_q,
                      int64_t q_rows, int64_t k_rows, const TileGeom& tg, void* ws, hipStream_t st) {
  if (nseg == 0 || Hq == 0) return hipSuccess;
  const BwdWorkspace wl = bwd_workspace(dqk, dv, Hq, Hkv, q_rows, k_rows, nseg, tg);
  if (bwd_uses_tiles(dqk, dv))
    return launch_bwd_tiles(a, dqk, dv, causal, nseg, Hq, Hkv, max_q, q_rows, k_rows, tg, wl, ws,
                            st);
// arguments: DQK, DV, dQ key tile, dQ waves per SIMD, dK/dV waves per
// workgroup, dQ waves per workgroup
#define VCA_BWD(DQK, DV, BN, WPE, NWK, NWQ) \
  bwd_dims<DQK, DV, BN, WPE, NWK, NWQ>(a, causal, nseg, Hq, Hkv, max_q, q_rows, k_rows, tg, wl, ws, st)
  if (dqk == 64 && dv == 64) return VCA_BWD(64, 64, 32, 2, 4, 4);
  if (dqk == 128 && dv == 128) return VCA_BWD(128, 128, 32, 2, 4, 4);
  // 192/128: the fused passes at one wave per SIMD (dK/dV 360, dQ 285 registers) beat the
  // two-phase backward, whose P/dS stores and re-reads make it HBM-bound at these head dims
  // (14.0 -> 11.7 ms on the 32K-token varlen problem)
  if (dqk == 192 && dv == 128) return VCA_BWD(192, 128, 32, 1, 4, 4);
#undef VCA_BWD
  return hipErrorInvalidValue;
}

}  // namespace VCA_ELEM
}  // namespace vca
