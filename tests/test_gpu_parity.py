"""GPU parity: the HIP library through its C ABI against the fp64 oracle on the
same seeded bf16 inputs.

Tolerances (fixed for N(0,1) bf16 inputs): out max-abs <= 2e-2; lse max-abs
<= 5e-3 on finite entries with the -inf pattern matching exactly; dq, dk, dv
relative Frobenius error <= 5e-2. The oracle computes the backward from its
own forward (never from GPU outputs).
"""
import math

import numpy as np
import pytest
import torch

import workloads
from oracle import attention as orc

pytestmark = pytest.mark.gpu

OUT_TOL, LSE_TOL, GRAD_TOL = 2e-2, 5e-3, 5e-2


@pytest.fixture(scope="module")
def vca():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import varlen_causal_attention_amd as m

    m.load()
    return m


def dev(t):
    return t.to("cuda")


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_out(out, ref, tol=OUT_TOL):
    err = np.abs(host(out) - ref).max() if ref.size else 0.0
    assert err <= tol, f"out max-abs {err}"


def check_lse(lse, ref):
    got = host(lse)
    assert np.array_equal(np.isneginf(got), np.isneginf(ref)), "-inf rows differ"
    assert not np.isnan(got).any()
    fin = np.isfinite(ref)
    if fin.any():
        err = np.abs(got[fin] - ref[fin]).max()
        assert err <= LSE_TOL, f"lse max-abs {err}"


def check_grad(name, g, ref):
    g = host(g)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(g - ref)
    if den == 0:
        assert num == 0, f"{name}: expected zeros"
        return
    assert num / den <= GRAD_TOL, f"{name} rel-Frobenius {num / den}"


def rand(shape, g, dtype=torch.bfloat16):
    return workloads.randn_bf16(shape, g, dtype)


# ---------------------------------------------------------------- varlen
def run_varlen(vca, lens_q, lens_k, Hq, Hkv, Dqk, Dv, causal, seed, scale=None,
               dtype=torch.bfloat16):
    g = torch.Generator().manual_seed(seed)
    cu_q, cu_k = workloads.cumulative(lens_q), workloads.cumulative(lens_k)
    Tq, Tk = int(cu_q[-1]), int(cu_k[-1])
    q, k = rand((Tq, Hq, Dqk), g, dtype), rand((Tk, Hkv, Dqk), g, dtype)
    v, do = rand((Tk, Hkv, Dv), g, dtype), rand((Tq, Hq, Dv), g, dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(Dqk)
    ro, rl = orc.fwd_varlen(q, k, v, cu_q, cu_k, scale, causal)
    rdq, rdk, rdv = orc.bwd_varlen(do, q, k, v, ro, rl, cu_q, cu_k, scale, causal)
    cq, ck = dev(torch.from_numpy(cu_q)), dev(torch.from_numpy(cu_k))
    mq, mk = max(lens_q, default=0), max(lens_k, default=0)
    out, lse = vca.fwd_varlen(dev(q), dev(k), dev(v), cq, ck, mq, mk, scale, causal)
    dq, dk, dv = vca.bwd_varlen(dev(do), dev(q), dev(k), dev(v), out, lse, cq, ck, mq, mk, scale,
                                causal)
    torch.cuda.synchronize()
    check_out(out, ro)
    check_lse(lse, rl)
    check_grad("dq", dq, rdq)
    check_grad("dk", dk, rdk)
    check_grad("dv", dv, rdv)
    return out, lse, (dq, dk, dv), (ro, rl)


@pytest.mark.parametrize("dqk,dv", [(64, 64), (128, 128), (192, 128), (256, 256), (512, 512)])
@pytest.mark.parametrize("causal", [True, False])
def test_varlen_every_head_dim(vca, dqk, dv, causal):
    lens = [1, 37, 200, 129, 64, 300]
    run_varlen(vca, lens, lens, 4, 2, dqk, dv, causal, seed=11 + dqk + dv + causal)


@pytest.mark.parametrize("dqk,dv", [(64, 64), (128, 128), (192, 128), (256, 256), (512, 512)])
def test_varlen_negative_scale(vca, dqk, dv):
    # the caller's scale may be negative: the softmax is then over -|scale| q.k
    lens = [1, 100, 257, 64]
    run_varlen(vca, lens, lens, 4, 2, dqk, dv, True, seed=41 + dqk, scale=-0.7 / math.sqrt(dqk))


@pytest.mark.parametrize("dqk,dv", [(64, 64), (128, 128), (192, 128), (256, 256), (512, 512)])
@pytest.mark.parametrize("hq,hkv", [(8, 2), (4, 4)])
def test_varlen_ragged_unequal_segments(vca, dqk, dv, hq, hkv):
    # lq != lk per segment, zero-query and zero-key segments, lq > lk (empty
    # rows); an even GQA group and none (the two work-list orders)
    lens_q = [5, 0, 130, 70, 0, 3, 33]
    lens_k = [9, 40, 100, 70, 12, 0, 65]
    for causal in (True, False):
        run_varlen(vca, lens_q, lens_k, hq, hkv, dqk, dv, causal, seed=21 + causal + dqk + hkv)


@pytest.mark.parametrize("hq,hkv", [(2, 1), (1, 1)])
def test_varlen_long_segment_and_many_segments(vca, hq, hkv):
    # work lists with more than 64 items in one segment (a 9000-token
    # document: 71 query tiles, 71 key blocks) and with more than 1024
    # segments (1100 short documents), in both list orders (an even GQA group
    # keeps the backward lists heavy-first)
    run_varlen(vca, [9000], [9000], hq, hkv, 64, 64, True, seed=71 + hq)
    lens = [1 + (7 * i) % 5 for i in range(1100)]
    run_varlen(vca, lens, lens, hq, hkv, 128, 128, True, seed=73 + hq)


def test_varlen_gqa_group_sizes(vca):
    lens = [77, 300, 5]
    for hq, hkv in [(1, 1), (8, 1), (8, 8), (6, 2)]:
        run_varlen(vca, lens, lens, hq, hkv, 128, 128, True, seed=31 + hq + hkv)


def test_empty_rows_are_exact(vca):
    out, lse, grads, (ro, rl) = run_varlen(vca, [4, 6], [0, 3], 2, 1, 128, 128, True, seed=41)
    o, l = host(out), host(lse)
    assert np.all(o[:4] == 0.0) and np.all(np.isneginf(l[:, :4]))
    # second segment: lq=6 > lk=3, bottom-right leaves its first 3 rows empty
    assert np.all(o[4:7] == 0.0) and np.all(np.isneginf(l[:, 4:7]))
    assert np.all(host(grads[0])[:7] == 0.0)


# ---------------------------------------------------------------- dense
def run_dense(vca, B, Hq, Hkv, Nq, Nk, Dqk, Dv, causal, seed, layout="bhnd",
              dtype=torch.bfloat16):
    g = torch.Generator().manual_seed(seed)
    q, k = rand((B, Hq, Nq, Dqk), g, dtype), rand((B, Hkv, Nk, Dqk), g, dtype)
    v, do = rand((B, Hkv, Nk, Dv), g, dtype), rand((B, Hq, Nq, Dv), g, dtype)
    scale = 1.0 / math.sqrt(Dqk)
    ro, rl = orc.fwd_dense(q, k, v, scale, causal)
    rg = orc.bwd_dense(do, q, k, v, ro, rl, scale, causal)

    def put(t):
        if layout == "bshd":  # BSHD storage viewed as [B, H, S, D]
            return dev(t.transpose(1, 2).contiguous()).transpose(1, 2)
        return dev(t)

    out, lse = vca.fwd_dense(put(q), put(k), put(v), scale, causal)
    dq, dk, dv = vca.bwd_dense(put(do), put(q), put(k), put(v), out, lse, scale, causal)
    torch.cuda.synchronize()
    check_out(out, ro)
    check_lse(lse, rl)
    for name, a, b in zip(("dq", "dk", "dv"), (dq, dk, dv), rg):
        check_grad(name, a, b)
    return out, lse


def test_dense_small_causal_workload(vca):
    w = workloads.workload(1)
    t = w.tensors()
    ro, rl = orc.fwd_dense(t["q"], t["k"], t["v"], w.scale, True)
    rg = orc.bwd_dense(t["do"], t["q"], t["k"], t["v"], ro, rl, w.scale, True)
    out, lse = vca.fwd_dense(dev(t["q"]), dev(t["k"]), dev(t["v"]), w.scale, True)
    grads = vca.bwd_dense(dev(t["do"]), dev(t["q"]), dev(t["k"]), dev(t["v"]), out, lse, w.scale, True)
    torch.cuda.synchronize()
    check_out(out, ro)
    check_lse(lse, rl)
    for name, a, b in zip(("dq", "dk", "dv"), grads, rg):
        check_grad(name, a, b)


@pytest.mark.parametrize("Nq,Nk", [(130, 300), (300, 130), (257, 257)])
@pytest.mark.parametrize("dqk,dv", [(64, 64), (128, 128), (192, 128)])
def test_dense_bottom_right_alignment(vca, Nq, Nk, dqk, dv):
    run_dense(vca, 2, 4, 2, Nq, Nk, dqk, dv, True, seed=51 + Nq + dqk)


def test_dense_bshd_views_and_d512(vca):
    run_dense(vca, 1, 4, 2, 200, 200, 128, 128, True, seed=61, layout="bshd")
    run_dense(vca, 1, 2, 1, 160, 160, 512, 512, True, seed=62, layout="bshd")
    run_dense(vca, 1, 4, 4, 96, 96, 192, 128, False, seed=63)


# ---------------------------------------------------------------- full-size workloads
def nan_like(shape, dtype=torch.bfloat16):
    return torch.full(shape, float("nan"), dtype=dtype, device="cuda")


def assert_all_written(**tensors):
    """Outputs start NaN-filled, so an element no work item wrote (a dropped or
    misrouted tile) is still NaN."""
    for name, x in tensors.items():
        assert not torch.isnan(x).any().item(), f"{name}: elements left unwritten"


def run_full_varlen(vca, w, t):
    """The whole varlen workload on the GPU, into NaN-filled outputs."""
    cq = dev(torch.from_numpy(w.cu()))
    mx = max(w.lengths)
    T = w.T
    q, k, v, do = (dev(t[n]) for n in ("q", "k", "v", "do"))
    et = q.dtype
    out, lse = nan_like((T, w.Hq, w.Dv), et), nan_like((w.Hq, T), torch.float32)
    vca.fwd_varlen(q, k, v, cq, cq, mx, mx, w.scale, w.causal, out=out, lse=lse)
    dq, dk = nan_like((T, w.Hq, w.Dqk), et), nan_like((T, w.Hkv, w.Dqk), et)
    dv = nan_like((T, w.Hkv, w.Dv), et)
    vca.bwd_varlen(do, q, k, v, out, lse, cq, cq, mx, mx, w.scale, w.causal, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert_all_written(out=out, lse=lse, dq=dq, dk=dk, dv=dv)
    return out, lse, (dq, dk, dv)


class _Lookup:
    """Indexable stand-in for an oracle-side array of which only a few entries
    are known (the oracle's sampled rows): x[i, j] returns the stored entry."""

    def __init__(self, keys, values):
        self.d = {tuple(int(e) for e in k): v for k, v in zip(keys, values)}

    def __getitem__(self, idx):
        return self.d[tuple(int(e) for e in idx)]


def check_sampled(vca_out, t, cu, Hq, Hkv, scale, causal, seed, rows_per=2):
    """Every segment x q-head: `rows_per` seeded query rows (out, lse, dq);
    every non-empty segment x kv-head: one seeded key row (dk, dv), in the last
    eighth of the segment when causal (few queries see it, so the oracle's
    sub-problem stays small), plus per segment one key anywhere for one kv-head
    (rotating). The oracle side is computed from the inputs alone: sampled
    rows through its row samplers, key rows from the forward and backward of
    exactly the queries that see the key."""
    out, lse, (dq, dk, dv) = vca_out
    rng = np.random.default_rng(seed)
    G = Hq // Hkv
    # the row samplers slice k / v per row: upcast them once
    t = dict(t, k=orc.f64(t["k"]), v=orc.f64(t["v"]))
    toks, heads = [], []
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        if b == a:
            continue
        for h in range(Hq):
            pick = rng.integers(a, b, size=rows_per)
            pick[0] = a if h % 2 == 0 else b - 1  # segment edges on alternate heads
            toks += [int(x) for x in pick]
            heads += [h] * rows_per
    toks, heads = np.array(toks), np.array(heads)
    it, ih = torch.from_numpy(toks).to(out.device), torch.from_numpy(heads).to(out.device)
    ro, rl = orc.fwd_varlen_rows(t["q"], t["k"], t["v"], cu, cu, scale, causal, toks, heads)
    check_out(out[it, ih], ro)
    check_lse(lse[ih, it], rl)
    rdq = orc.bwd_varlen_rows(t["do"], t["q"], t["k"], t["v"],
                              _Lookup(zip(toks, heads), ro), _Lookup(zip(heads, toks), rl),
                              cu, cu, scale, causal, toks, heads)
    check_grad("dq rows", dq[it, ih], rdq)
    gk, gv, rk, rv = [], [], [], []
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        if b == a:
            continue
        L = b - a
        anywhere = s % Hkv
        for g in range(Hkv):
            lo = 0 if (not causal or g == anywhere) else (7 * L) // 8
            j = int(rng.integers(lo, L))
            i0 = j if causal else 0  # first query that sees key j (lq = lk)
            hs = list(range(g * G, (g + 1) * G))
            qq, dd = t["q"][a + i0:b][:, hs], t["do"][a + i0:b][:, hs]
            kk, vv = t["k"][a:b][:, [g]], t["v"][a:b][:, [g]]
            # bottom-right alignment keeps the visibility of the kept rows:
            # row i - i0 of L - i0 rows sees keys <= (i - i0) + L - (L - i0) = i
            cq1, ck1 = [0, L - i0], [0, L]
            so, sl = orc.fwd_varlen(qq, kk, vv, cq1, ck1, scale, causal)
            k1, v1 = orc.bwd_varlen_cols(dd, qq, kk, vv, so, sl, cq1, ck1, scale, causal,
                                         [j], [0])
            rk.append(k1[0])
            rv.append(v1[0])
            gk.append(dk[a + j, g])
            gv.append(dv[a + j, g])
    check_grad("dk rows", torch.stack(gk), np.array(rk))
    check_grad("dv rows", torch.stack(gv), np.array(rv))


def _segment_slice_check(vca, w, t, seg, kv_heads, res=None):
    """Run the whole workload on the GPU; check one segment x kv-head groups
    against the oracle, computed fully for that slice."""
    cu = w.cu()
    out, lse, (dq, dk, dv) = res if res is not None else run_full_varlen(vca, w, t)
    a, b = int(cu[seg]), int(cu[seg + 1])
    G = w.Hq // w.Hkv
    for g in kv_heads:
        hs = list(range(g * G, (g + 1) * G))
        sl = lambda x, heads: x[a:b][:, heads]  # noqa: E731
        qq, kk, vv, dd = sl(t["q"], hs), sl(t["k"], [g]), sl(t["v"], [g]), sl(t["do"], hs)
        cu1 = [0, b - a]
        ro, rl = orc.fwd_varlen(qq, kk, vv, cu1, cu1, w.scale, w.causal)
        rdq, rdk, rdv = orc.bwd_varlen(dd, qq, kk, vv, ro, rl, cu1, cu1, w.scale, w.causal)
        check_out(out[a:b][:, hs], ro)
        check_lse(lse[hs][:, a:b], rl)
        check_grad("dq", dq[a:b][:, hs], rdq)
        check_grad("dk", dk[a:b][:, [g]], rdk)
        check_grad("dv", dv[a:b][:, [g]], rdv)
    return out, lse, (dq, dk, dv)


def test_varlen_d128_workload_full_size(vca):
    w = workloads.workload(2)
    t = w.tensors()
    res = run_full_varlen(vca, w, t)
    out, lse, grads = _segment_slice_check(vca, w, t, seg=0, kv_heads=[0, 7], res=res)
    _segment_slice_check(vca, w, t, seg=7, kv_heads=[3], res=res)
    # properties at full size: finite everywhere, no empty row in causal self-attention
    assert torch.isfinite(lse).all() and torch.isfinite(out.float()).all()
    for gtn in grads:
        assert torch.isfinite(gtn.float()).all()
    check_sampled(res, t, w.cu(), w.Hq, w.Hkv, w.scale, True, seed=202)


def test_varlen_192_128_workload_full_size(vca):
    w = workloads.workload(4)
    t = w.tensors()
    res = run_full_varlen(vca, w, t)
    _segment_slice_check(vca, w, t, seg=4, kv_heads=[13], res=res)
    check_sampled(res, t, w.cu(), w.Hq, w.Hkv, w.scale, True, seed=204)


def test_dense_d512_workload_full_size(vca):
    w = workloads.workload(3)
    t = w.tensors()
    q, k, v, do = (dev(t[n]) for n in ("q", "k", "v", "do"))
    B, N = w.B, w.Nq
    out, lse = nan_like((B, w.Hq, N, w.Dv)), nan_like((B, w.Hq, N), torch.float32)
    vca.fwd_dense(q, k, v, w.scale, True, out=out, lse=lse)
    dq, dk, dv = (nan_like((B, w.Hq, N, w.Dqk)), nan_like((B, w.Hkv, N, w.Dqk)),
                  nan_like((B, w.Hkv, N, w.Dv)))
    vca.bwd_dense(do, q, k, v, out, lse, w.scale, True, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert_all_written(out=out, lse=lse, dq=dq, dk=dk, dv=dv)
    # every batch x head through the row samplers: the dense problem is the
    # varlen one with one segment per batch entry ([B, H, N, D] -> [B*N, H, D])
    thd = lambda x: x.transpose(1, 2).reshape(B * N, x.shape[1], x.shape[3])  # noqa: E731
    tt = {n: thd(t[n]) for n in ("q", "k", "v", "do")}
    res = (thd(out), lse.reshape(B, w.Hq, N).transpose(0, 1).reshape(w.Hq, B * N),
           (thd(dq), thd(dk), thd(dv)))
    check_sampled(res, tt, np.array([0, N, 2 * N]), w.Hq, w.Hkv, w.scale, True, seed=203)
    b, g = 1, 5
    G = w.Hq // w.Hkv
    hs = list(range(g * G, (g + 1) * G))
    qq, kk, vv, dd = t["q"][b:b + 1, hs], t["k"][b:b + 1, [g]], t["v"][b:b + 1, [g]], t["do"][b:b + 1, hs]
    ro, rl = orc.fwd_dense(qq, kk, vv, w.scale, True)
    rdq, rdk, rdv = orc.bwd_dense(dd, qq, kk, vv, ro, rl, w.scale, True)
    check_out(out[b:b + 1, hs], ro)
    check_lse(lse[b:b + 1, hs], rl)
    check_grad("dq", dq[b:b + 1, hs], rdq)
    check_grad("dk", dk[b:b + 1, [g]], rdk)
    check_grad("dv", dv[b:b + 1, [g]], rdv)
    assert torch.isfinite(lse).all()


def ring_share(vca, w, t):
    """One rank's ring share on the GPU: local causal chunk, earlier cross chunk,
    lse merge, then both chunk backwards from the merged out/lse (dq summed)."""
    ids = w.row_doc_ids()
    S = w.shard
    lq_cu, lk_cu, lmq, lmk = vca.doc_layout(ids, S, S, S, S, 0, "cuda")
    xq_cu, xk_cu, xmq, xmk = vca.doc_layout(ids, S, S, 0, S, 1, "cuda")
    q, do = dev(t["q"]), dev(t["do"])
    kl, vl, ke, ve = (dev(t[n]) for n in ("k_local", "v_local", "k_early", "v_early"))
    H, Hkv, et = w.Hq, w.Hkv, q.dtype
    o1, l1 = nan_like((S, H, w.Dv), et), nan_like((H, S), torch.float32)
    o2, l2 = nan_like((S, H, w.Dv), et), nan_like((H, S), torch.float32)
    vca.fwd_varlen(q, kl, vl, lq_cu, lk_cu, lmq, lmk, w.scale, True, out=o1, lse=l1)
    vca.fwd_varlen(q, ke, ve, xq_cu, xk_cu, xmq, xmk, w.scale, False, out=o2, lse=l2)
    mo, ml, mob = vca.merge(o1, l1, o2, l2, copy_dtype=et)
    dq, dkl = nan_like((S, H, w.Dqk), et), nan_like((S, Hkv, w.Dqk), et)
    dvl, dke = nan_like((S, Hkv, w.Dv), et), nan_like((S, Hkv, w.Dqk), et)
    dve = nan_like((S, Hkv, w.Dv), et)
    vca.bwd_varlen(do, q, kl, vl, mob, ml, lq_cu, lk_cu, lmq, lmk, w.scale, True, dq=dq, dk=dkl,
                   dv=dvl)
    vca.bwd_varlen(do, q, ke, ve, mob, ml, xq_cu, xk_cu, xmq, xmk, w.scale, False,
                   dq_accumulate=dq, dk=dke, dv=dve)
    torch.cuda.synchronize()
    assert_all_written(o1=o1, l1=l1, o2=o2, l2=l2, dq=dq, dkl=dkl, dvl=dvl, dke=dke, dve=dve)
    return (o1, l1), (o2, l2), (mo, ml), (dq, dkl, dvl, dke, dve)


def ring_share_dense(vca, w, t):
    """ring_share over the dense route ([1, H, S, D] views of the shard
    tensors, padding rows zeroed, merge in the flattened dense layout); the
    results come back in the packed [S, H, D] / [H, S] layout."""
    ids, S, H, D = w.row_doc_ids(), w.shard, w.Hq, w.Dv
    ok_l, pad = vca.dense_route(ids, S, S, S, S, 0)
    ok_x, _ = vca.dense_route(ids, S, S, 0, S, 1)
    assert ok_l and ok_x
    rows = dev(torch.from_numpy(pad))
    d = {k: dev(x).unsqueeze(0).transpose(1, 2) for k, x in t.items()}
    o1, l1 = vca.fwd_dense(d["q"], d["k_local"], d["v_local"], w.scale, True)
    vca.zero_rows(o1, l1, rows)
    o2, l2 = vca.fwd_dense(d["q"], d["k_early"], d["v_early"], w.scale, False)
    vca.zero_rows(o2, l2, rows)
    n = H * S
    mo, ml, mob = vca.merge(o1.view(n, 1, D), l1.view(1, n), o2.view(n, 1, D), l2.view(1, n),
                            bf16_copy=True)
    mob4, ml4 = mob.view(1, H, S, D), ml.view(1, H, S)
    dq, dkl, dvl = vca.bwd_dense(d["do"], d["q"], d["k_local"], d["v_local"], mob4, ml4, w.scale,
                                 True)
    _, dke, dve = vca.bwd_dense(d["do"], d["q"], d["k_early"], d["v_early"], mob4, ml4, w.scale,
                                False, dq_accumulate=dq)
    thd = lambda x: x[0].transpose(0, 1)  # noqa: E731  [1, H, S, D] -> [S, H, D]
    return ((thd(o1), l1[0]), (thd(o2), l2[0]), (mo.view(H, S, D).transpose(0, 1), ml.view(H, S)),
            tuple(thd(x) for x in (dq, dkl, dvl, dke, dve)))


@pytest.mark.parametrize("n", [5, 6])
def test_ring_share_workload(vca, n):
    # 5: packed documents (varlen route); 6: one document per row (dense route)
    check_ring_share(vca, n, torch.bfloat16)


def ring_share_gather(vca, w, t):
    """ring_share through the packed gather layout ("gemma4_moe cp_attention"
    page): each chunk's live tokens (documents shared by the query shard and
    the chunk) are gathered from [1, H, S, D] views of the shard tensors, run
    as varlen segments, merged in place at their rows into fp32 accumulators
    that start as "attends nothing" (out 0, lse -inf), and the backward
    gathers the merged out/lse, then scatters dq (added over the chunks),
    dk and dv back. Results come back in the packed [S, H, D] / [H, S] layout
    of ring_share."""
    ids, S, H, Hkv = w.row_doc_ids(), w.shard, w.Hq, w.Hkv
    d = {k: dev(x).unsqueeze(0).transpose(1, 2) for k, x in t.items()}  # [1, H, S, D] views
    et = d["q"].dtype
    loc = vca.ring_segments(ids[:, S:], ids[:, S:], device="cuda")
    crs = vca.ring_segments(ids[:, S:], ids[:, :S], device="cuda")
    acc = torch.empty((1, H, S, w.Dv), dtype=torch.float32, device="cuda")
    none = torch.empty(0, dtype=torch.int32, device="cuda")
    vca.scatter_rows(torch.empty((0, H, w.Dv), dtype=torch.float32, device="cuda"), none, acc,
                     mode=1)
    lacc = vca.scatter_lse(torch.empty((H, 0), dtype=torch.float32, device="cuda"), none, 1, S)
    partial = []
    chunks = ((loc, "k_local", "v_local", True), (crs, "k_early", "v_early", False))
    packed = []
    for seg, kn, vn, causal in chunks:
        qp = vca.gather_rows(d["q"], seg["q_index"])
        kp = vca.gather_rows(d[kn], seg["k_index"])
        vp = vca.gather_rows(d[vn], seg["k_index"])
        op, lp = vca.fwd_varlen(qp, kp, vp, seg["cu_q"], seg["cu_k"], seg["max_q"], seg["max_k"],
                                w.scale, causal)
        vca.merge_rows(acc, lacc, op, lp, seg["q_index"])
        # the chunk alone, scattered for the per-chunk checks (0 / -inf elsewhere)
        o_full = torch.empty((1, H, S, w.Dv), dtype=et, device="cuda")
        vca.scatter_rows(op, seg["q_index"], o_full, mode=1)
        l_full = vca.scatter_lse(lp, seg["q_index"], 1, S)
        partial.append((o_full[0].transpose(0, 1), l_full[0]))
        packed.append((seg, qp, kp, vp))
    dq = torch.empty((1, H, S, w.Dqk), dtype=et, device="cuda")
    grads = {}
    for i, ((seg, qp, kp, vp), (_, kn, vn, causal)) in enumerate(zip(packed, chunks)):
        mo_p = vca.gather_rows(acc, seg["q_index"], dtype=et)
        ml_p = vca.gather_lse(lacc, seg["q_index"])
        do_p = vca.gather_rows(d["do"], seg["q_index"])
        dqp, dkp, dvp = vca.bwd_varlen(do_p, qp, kp, vp, mo_p, ml_p, seg["cu_q"], seg["cu_k"],
                                       seg["max_q"], seg["max_k"], w.scale, causal)
        # dq: the first chunk assigns (zeroing rows it does not hold), later ones add
        vca.scatter_rows(dqp, seg["q_index"], dq, mode=1 if i == 0 else 2)
        dk = torch.empty((1, Hkv, S, w.Dqk), dtype=et, device="cuda")
        dv = torch.empty((1, Hkv, S, w.Dv), dtype=et, device="cuda")
        vca.scatter_rows(dkp, seg["k_index"], dk, mode=1)
        vca.scatter_rows(dvp, seg["k_index"], dv, mode=1)
        grads[kn] = (dk[0].transpose(0, 1), dv[0].transpose(0, 1))
    torch.cuda.synchronize()
    mo = acc[0].transpose(0, 1)
    return (partial[0], partial[1], (mo, lacc[0]),
            (dq[0].transpose(0, 1), *grads["k_local"], *grads["k_early"]))


def check_ring_share(vca, n, dtype, route="auto"):
    w = workloads.workload(n)
    t = w.tensors(dtype)
    share = ring_share_dense if w.single_doc else ring_share
    if route == "gather":
        share = ring_share_gather
    (o1, l1), (o2, l2), (mo, ml), (dq, dkl, dvl, dke, dve) = share(vca, w, t)
    torch.cuda.synchronize()
    ids = w.row_doc_ids()[0]
    S = w.shard
    q_pos, loc_pos, early_pos = np.arange(S, 2 * S), np.arange(S, 2 * S), np.arange(0, S)
    G = w.Hq // w.Hkv
    for g in (0, 6):
        hs = list(range(g * G, (g + 1) * G))
        q, do = t["q"][:, hs], t["do"][:, hs]
        kl, vl = t["k_local"][:, [g]], t["v_local"][:, [g]]
        ke, ve = t["k_early"][:, [g]], t["v_early"][:, [g]]
        k_all, v_all = torch.cat([ke, kl]), torch.cat([ve, vl])
        all_pos = np.arange(0, 2 * S)
        ro, rl = orc.fwd_doc_causal(q, k_all, v_all, ids[q_pos], q_pos, ids[all_pos], all_pos, w.scale)
        # per-chunk results and the merge
        r1 = orc.fwd_doc_causal(q, kl, vl, ids[q_pos], q_pos, ids[loc_pos], loc_pos, w.scale)
        r2 = orc.fwd_doc_causal(q, ke, ve, ids[q_pos], q_pos, ids[early_pos], early_pos, w.scale)
        check_out(o1[:, hs], r1[0])
        check_lse(l1[hs], r1[1])
        check_out(o2[:, hs], r2[0])
        check_lse(l2[hs], r2[1])
        check_out(mo[:, hs], ro)
        check_lse(ml[hs], rl)
        rdq, rdk, rdv = orc.bwd_doc_causal(do, q, k_all, v_all, ro, rl, ids[q_pos], q_pos,
                                           ids[all_pos], all_pos, w.scale)
        check_grad("dq", dq[:, hs], rdq)
        check_grad("dk_early", dke[:, [g]], rdk[:S])
        check_grad("dv_early", dve[:, [g]], rdv[:S])
        check_grad("dk_local", dkl[:, [g]], rdk[S:])
        check_grad("dv_local", dvl[:, [g]], rdv[S:])
    # every other kv-head group: seeded query rows (merged out, lse, dq) and
    # key rows of both chunks (dk, dv), the oracle computing each from the
    # inputs over exactly the rows involved
    rng = np.random.default_rng(205 + n)
    all_pos = np.arange(0, 2 * S)
    k_all_t = torch.cat([t["k_early"], t["k_local"]])
    v_all_t = torch.cat([t["v_early"], t["v_local"]])
    gq, rq, go, ro_s, gl, rl_s = [], [], [], [], [], []
    gk, rk, gv, rv = [], [], [], []
    for g in range(w.Hkv):
        if g in (0, 6):
            continue
        hs = list(range(g * G, (g + 1) * G))
        rows = rng.choice(S, size=12, replace=False)
        q, do = t["q"][rows][:, hs], t["do"][rows][:, hs]
        ka, va = k_all_t[:, [g]], v_all_t[:, [g]]
        o_r, l_r = orc.fwd_doc_causal(q, ka, va, ids[q_pos[rows]], q_pos[rows], ids, all_pos,
                                      w.scale)
        dq_r = orc.bwd_doc_causal(do, q, ka, va, o_r, l_r, ids[q_pos[rows]], q_pos[rows], ids,
                                  all_pos, w.scale)[0]
        ir = torch.from_numpy(rows).cuda()
        go.append(mo[ir][:, hs].float().cpu())
        ro_s.append(o_r)
        gl.append(ml[hs][:, ir].cpu())
        rl_s.append(l_r)
        gq.append(dq[ir][:, hs].float().cpu())
        rq.append(dq_r)
        for j in rng.choice(2 * S, size=4, replace=False):
            j = int(j)
            seen = np.nonzero((ids[q_pos] == ids[j]) & (ids[j] > 0) & (q_pos >= j))[0]
            got_k = (dke if j < S else dkl)[j % S, g].float().cpu()
            got_v = (dve if j < S else dvl)[j % S, g].float().cpu()
            if len(seen) == 0:
                exp_k, exp_v = np.zeros(w.Dqk), np.zeros(w.Dv)
            else:
                qs, ds = t["q"][seen][:, hs], t["do"][seen][:, hs]
                o_s, l_s = orc.fwd_doc_causal(qs, ka, va, ids[q_pos[seen]], q_pos[seen], ids,
                                              all_pos, w.scale)
                _, bk, bv = orc.bwd_doc_causal(ds, qs, ka[[j]], va[[j]], o_s, l_s,
                                               ids[q_pos[seen]], q_pos[seen], ids[[j]], [j],
                                               w.scale)
                exp_k, exp_v = bk[0, 0], bv[0, 0]
            gk.append(got_k)
            rk.append(exp_k)
            gv.append(got_v)
            rv.append(exp_v)
    check_out(torch.stack(go), np.stack(ro_s))
    check_lse(torch.stack(gl), np.stack(rl_s))
    check_grad("dq rows", torch.stack(gq), np.stack(rq))
    check_grad("dk rows", torch.stack(gk), np.stack(rk))
    check_grad("dv rows", torch.stack(gv), np.stack(rv))
    # padding queries: out 0, lse -inf, dq 0
    pad = np.nonzero(ids[q_pos] == 0)[0]
    assert len(pad) == w.pad_tail
    assert torch.all(mo[pad] == 0) and torch.all(torch.isneginf(ml[:, pad]))
    assert torch.all(dq[pad] == 0)


@pytest.mark.parametrize("d", [128, 512])
def test_ring_share_dense_route(vca, d):
    """Ring share whose rows are single documents (one with a pad tail): both
    chunks pass dense_route, run on the dense kernels over the raw
    [B, H, S, D] rows, get their padding queries zeroed (zero_rows), merge in
    the flattened dense layout, and run the dense backwards from the merged
    out/lse; every result matches the document-causal oracle."""
    g = torch.Generator().manual_seed(95 + d)
    B, S, Hq, Hkv = 2, 160, 4, 2
    ids = np.zeros((B, 2 * S), dtype=np.int32)
    ids[0, :] = 3
    ids[1, :2 * S - 60] = 4
    ok_l, pad = vca.dense_route(ids, S, S, S, S, 0)
    ok_x, pad_x = vca.dense_route(ids, S, S, 0, S, 1)
    assert ok_l and ok_x and np.array_equal(pad, pad_x) and pad.sum() == 60
    q, do = rand((B, Hq, S, d), g), rand((B, Hq, S, d), g)
    kl, vl, ke, ve = (rand((B, Hkv, S, d), g) for _ in range(4))
    scale = 1.0 / math.sqrt(d)
    rows = dev(torch.from_numpy(pad))
    o1, l1 = vca.fwd_dense(dev(q), dev(kl), dev(vl), scale, True)
    vca.zero_rows(o1, l1, rows)
    o2, l2 = vca.fwd_dense(dev(q), dev(ke), dev(ve), scale, False)
    vca.zero_rows(o2, l2, rows)
    n = B * Hq * S
    mo, ml, mob = vca.merge(o1.view(n, 1, d), l1.view(1, n), o2.view(n, 1, d), l2.view(1, n),
                            bf16_copy=True)
    mo4, ml4, mob4 = mo.view(B, Hq, S, d), ml.view(B, Hq, S), mob.view(B, Hq, S, d)
    dq, dkl, dvl = vca.bwd_dense(dev(do), dev(q), dev(kl), dev(vl), mob4, ml4, scale, True)
    _, dke, dve = vca.bwd_dense(dev(do), dev(q), dev(ke), dev(ve), mob4, ml4, scale, False,
                                dq_accumulate=dq)
    torch.cuda.synchronize()
    qpos, kpos = np.arange(S, 2 * S), np.arange(0, 2 * S)
    for b in range(B):
        qb, dob = q[b].transpose(0, 1), do[b].transpose(0, 1)
        k_all = torch.cat([ke[b], kl[b]], dim=1).transpose(0, 1)
        v_all = torch.cat([ve[b], vl[b]], dim=1).transpose(0, 1)
        r1 = orc.fwd_doc_causal(qb, kl[b].transpose(0, 1), vl[b].transpose(0, 1), ids[b, qpos],
                                qpos, ids[b, qpos], qpos, scale)
        check_out(o1[b].transpose(0, 1), r1[0])
        check_lse(l1[b], r1[1])
        ro, rl = orc.fwd_doc_causal(qb, k_all, v_all, ids[b, qpos], qpos, ids[b, kpos], kpos, scale)
        check_out(mo4[b].transpose(0, 1), ro)
        check_lse(ml4[b], rl)
        rdq, rdk, rdv = orc.bwd_doc_causal(dob, qb, k_all, v_all, ro, rl, ids[b, qpos], qpos,
                                           ids[b, kpos], kpos, scale)
        check_grad("dq", dq[b].transpose(0, 1), rdq)
        check_grad("dk_early", dke[b].transpose(0, 1), rdk[:S])
        check_grad("dv_early", dve[b].transpose(0, 1), rdv[:S])
        check_grad("dk_local", dkl[b].transpose(0, 1), rdk[S:])
        check_grad("dv_local", dvl[b].transpose(0, 1), rdv[S:])
    # padding queries: out 0, lse -inf, dq 0
    assert torch.all(mo4[1, :, S - 60:] == 0) and torch.all(torch.isneginf(ml4[1, :, S - 60:]))
    assert torch.all(dq[1, :, S - 60:] == 0)


def test_zero_rows_fp32_and_no_lse(vca):
    out = torch.ones((2, 3, 5, 7), device="cuda")
    rows = torch.zeros((2, 5), dtype=torch.bool, device="cuda")
    rows[1, 2] = True
    vca.zero_rows(out, None, rows)
    torch.cuda.synchronize()
    ref = torch.ones((2, 3, 5, 7))
    ref[1, :, 2] = 0
    assert torch.equal(out.cpu(), ref)


def test_merge_kernel_against_oracle(vca):
    g = torch.Generator().manual_seed(71)
    rows, H, Dv = 300, 4, 512
    oa, ob = rand((rows, H, Dv), g), rand((rows, H, Dv), g).float()
    la = torch.randn((H, rows), generator=g) * 3
    lb = torch.randn((H, rows), generator=g) * 3
    la[0, :50] = -math.inf
    lb[0, 25:75] = -math.inf
    lb[1, :10] = -math.inf
    ro, rl = orc.merge(oa, la, ob, lb)
    mo, ml, mob = vca.merge(dev(oa), dev(la), dev(ob), dev(lb), bf16_copy=True)
    torch.cuda.synchronize()
    assert np.abs(host(mo) - ro).max() < 1e-5
    check_lse(ml, rl)
    assert torch.equal(mob, mo.to(torch.bfloat16))
    # running-accumulator use: out aliases out_a, lse aliases lse_a
    acc, lacc = dev(oa.float()), dev(la.clone())
    vca.merge(acc, lacc, dev(ob), dev(lb), out=acc, lse=lacc)
    torch.cuda.synchronize()
    assert np.abs(host(acc) - ro).max() < 1e-5
    check_lse(lacc, rl)
    # a head dim that is not a multiple of 8 takes the element-wise kernel
    rows, H, Dv = 77, 3, 20
    oa, ob = rand((rows, H, Dv), g), rand((rows, H, Dv), g)
    la = torch.randn((H, rows), generator=g) * 3
    lb = torch.randn((H, rows), generator=g) * 3
    lb[2, :9] = -math.inf
    ro, rl = orc.merge(oa, la, ob, lb)
    mo, ml, mob = vca.merge(dev(oa), dev(la), dev(ob), dev(lb), bf16_copy=True)
    torch.cuda.synchronize()
    assert np.abs(host(mo) - ro).max() < 1e-5
    check_lse(ml, rl)
    assert torch.equal(mob, mo.to(torch.bfloat16))


# ---------------------------------------------------------------- robustness
def test_results_are_bitwise_deterministic(vca):
    w = workloads.small_varlen(81, [500, 33, 700], 8, 2, 128, 128)
    t = w.tensors()
    cq = dev(torch.from_numpy(w.cu()))
    q, k, v, do = (dev(t[n]) for n in ("q", "k", "v", "do"))
    res = []
    for _ in range(2):
        out, lse = vca.fwd_varlen(q, k, v, cq, cq, 700, 700, w.scale, True)
        grads = vca.bwd_varlen(do, q, k, v, out, lse, cq, cq, 700, 700, w.scale, True)
        res.append([x.clone() for x in (out, lse, *grads)])
    torch.cuda.synchronize()
    for a, b in zip(*res):
        assert torch.equal(a, b)


def test_outputs_stay_inside_their_views(vca):
    """Guard bands: outputs written through strided views of larger NaN-filled
    buffers leave every element outside the view untouched."""
    import ctypes as C
    from varlen_causal_attention_amd import _lib

    lib = _lib.load()
    g = torch.Generator().manual_seed(91)
    B, Hq, Hkv, N, D = 2, 4, 2, 150, 128
    q, k, v = (dev(rand(s, g)) for s in ((B, Hq, N, D), (B, Hkv, N, D), (B, Hkv, N, D)))
    big = torch.full((B, Hq + 1, N + 16, D + 64), float("nan"), dtype=torch.bfloat16, device="cuda")
    out = big[:, 1:, 8:8 + N, 32:32 + D]
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device="cuda")
    strides = _lib.i64_array(list(q.stride()[:3]) + list(k.stride()[:3]) + list(v.stride()[:3])
                             + list(out.stride()[:3]))
    args = (0, C.c_void_p(q.data_ptr()), C.c_void_p(k.data_ptr()), C.c_void_p(v.data_ptr()),
            C.c_void_p(out.data_ptr()), C.c_void_p(lse.data_ptr()), B, Hq, Hkv, N, N, D, D, strides,
            1 / math.sqrt(D), 1)
    stream = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    need = C.c_size_t(0)
    assert lib.attn_fwd_dense(*args, None, C.byref(need), stream) == 0
    ws = torch.empty(need.value, dtype=torch.uint8, device="cuda")
    have = C.c_size_t(need.value)
    st = lib.attn_fwd_dense(*args, C.c_void_p(ws.data_ptr()), C.byref(have), stream)
    assert st == 0, lib.attn_last_error()
    torch.cuda.synchronize()
    mask = torch.ones_like(big, dtype=torch.bool)
    mask[:, 1:, 8:8 + N, 32:32 + D] = False
    assert torch.isnan(big[mask].float()).all()
    assert torch.isfinite(out.float()).all()
    ref, _ = vca.fwd_dense(q, k, v, 1 / math.sqrt(D), True)
    assert torch.equal(ref, out)


def test_dq_accumulate_adds(vca):
    w = workloads.small_varlen(93, [90, 200], 4, 2, 128, 128)
    t = w.tensors()
    cq = dev(torch.from_numpy(w.cu()))
    q, k, v, do = (dev(t[n]) for n in ("q", "k", "v", "do"))
    out, lse = vca.fwd_varlen(q, k, v, cq, cq, 200, 200, w.scale, True)
    dq1, _, _ = vca.bwd_varlen(do, q, k, v, out, lse, cq, cq, 200, 200, w.scale, True)
    acc = dq1.clone()
    vca.bwd_varlen(do, q, k, v, out, lse, cq, cq, 200, 200, w.scale, True, dq_accumulate=acc)
    torch.cuda.synchronize()
    ref = dq1.float() * 2
    assert (acc.float() - ref).abs().max().item() <= 2 ** -7 * ref.abs().max().item() + 1e-6


def test_varlen_and_gradient_outputs_stay_inside_their_views(vca):
    """Guard bands for the varlen forward and both backward entries: out, dq,
    dk and dv written through strided views of larger NaN-filled buffers leave
    every element outside the view untouched and match plain outputs."""
    g = torch.Generator().manual_seed(92)
    lens = [70, 1, 200, 33]
    cu = workloads.cumulative(lens)
    T, Hq, Hkv = int(cu[-1]), 4, 2
    cq = dev(torch.from_numpy(cu))
    for dqk, dv_ in [(128, 128), (192, 128), (512, 512)]:
        q, do = dev(rand((T, Hq, dqk), g)), dev(rand((T, Hq, dv_), g))
        k, v = dev(rand((T, Hkv, dqk), g)), dev(rand((T, Hkv, dv_), g))
        scale = 1 / math.sqrt(dqk)

        def banded(h, d):
            big = nan_like((T + 9, h + 1, d + 48))
            return big, big[5:5 + T, 1:, 16:16 + d]

        bo, out = banded(Hq, dv_)
        vca.fwd_varlen(q, k, v, cq, cq, 200, 200, scale, True, out=out)
        bq, dq = banded(Hq, dqk)
        bk, dk = banded(Hkv, dqk)
        bv, dv = banded(Hkv, dv_)
        ref_o, lse = vca.fwd_varlen(q, k, v, cq, cq, 200, 200, scale, True)
        vca.bwd_varlen(do, q, k, v, ref_o, lse, cq, cq, 200, 200, scale, True, dq=dq, dk=dk, dv=dv)
        ref = vca.bwd_varlen(do, q, k, v, ref_o, lse, cq, cq, 200, 200, scale, True)
        torch.cuda.synchronize()
        for big, view, want in ((bo, out, ref_o), (bq, dq, ref[0]), (bk, dk, ref[1]),
                                (bv, dv, ref[2])):
            mask = torch.ones_like(big, dtype=torch.bool)
            mask[5:5 + T, 1:, 16:16 + view.shape[2]] = False
            assert torch.isnan(big[mask].float()).all(), f"write outside the view ({dqk})"
            assert torch.equal(view, want), f"view result differs ({dqk})"


def test_merge_in_place_with_head_dims_that_split_waves(vca):
    """In-place merge (lse aliasing lse_a) at head dims whose 8-element chunks
    do not tile a wave (Dv/8 not a divisor of 64, or above 64): every row's
    lse must still be combined from the original lse_a."""
    g = torch.Generator().manual_seed(72)
    for rows, H, Dv in ((97, 3, 96), (64, 2, 192), (40, 2, 1024)):
        oa, ob = rand((rows, H, Dv), g).float(), rand((rows, H, Dv), g)
        la = torch.randn((H, rows), generator=g) * 3
        lb = torch.randn((H, rows), generator=g) * 3
        la[0, :7] = -math.inf
        ro, rl = orc.merge(oa, la, ob, lb)
        acc, lacc = dev(oa.clone()), dev(la.clone())
        vca.merge(acc, lacc, dev(ob), dev(lb), out=acc, lse=lacc)
        torch.cuda.synchronize()
        assert np.abs(host(acc) - ro).max() < 1e-5, Dv
        check_lse(lacc, rl)


@pytest.mark.parametrize("dqk,dv", [(128, 128), (192, 128)])
def test_backward_ds_store_modes(vca, monkeypatch, dqk, dv):
    """Head dims 128 and 192/128 store dS in the dK/dV pass and compute dQ
    from it. The store's budget (ATTN_BWD_DS_MIB) picks how many kv-heads
    share one dK/dV + dQ launch pair; below one GQA group's blocks the dQ
    pass recomputes S and dP instead. Every mode matches the oracle, and the
    chunked store gives bitwise the same gradients as the single launch."""
    lens_q = [300, 0, 41, 130, 1]
    lens_k = [300, 20, 70, 130, 1]
    Hq, Hkv = 8, 4
    monkeypatch.delenv("ATTN_BWD_DS_MIB", raising=False)
    _, _, whole, _ = run_varlen(vca, lens_q, lens_k, Hq, Hkv, dqk, dv, True, seed=301 + dqk)
    # about 0.74 MiB of blocks per group of two q-heads: a 1 MiB budget runs
    # one kv-head per launch pair
    monkeypatch.setenv("ATTN_BWD_DS_MIB", "1")
    _, _, chunked, _ = run_varlen(vca, lens_q, lens_k, Hq, Hkv, dqk, dv, True, seed=301 + dqk)
    for a, b in zip(whole, chunked):
        assert torch.equal(a, b)
    monkeypatch.setenv("ATTN_BWD_DS_MIB", "0")
    run_varlen(vca, lens_q, lens_k, Hq, Hkv, dqk, dv, True, seed=301 + dqk)
    run_dense(vca, 2, 4, 2, 150, 150, dqk, dv, True, seed=303 + dqk)
    run_varlen(vca, lens_q, lens_k, Hq, Hkv, dqk, dv, False, seed=305 + dqk)



@pytest.mark.parametrize("dqk,dv", [(256, 256), (512, 512)])
def test_two_phase_backward_in_chunks(vca, monkeypatch, dqk, dv):
    """Head dims 256/512 under a small ATTN_BWD_TILES_MIB: the P/dS stores
    hold one (or two) 256-query row slots, the passes run once per chunk of
    slots and dK/dV meet in fp32 across the chunks. Gradients match the
    oracle, varlen and dense, causal and not."""
    lens = [1, 37, 200, 129, 64, 600]
    for mib in ("1", "8"):
        monkeypatch.setenv("ATTN_BWD_TILES_MIB", mib)
        run_varlen(vca, lens, lens, 4, 2, dqk, dv, True, seed=401 + dqk)
        run_varlen(vca, [5, 0, 130, 70, 0, 3, 33], [9, 40, 100, 70, 12, 0, 65], 4, 4, dqk, dv,
                   False, seed=403 + dqk)
        run_dense(vca, 2, 4, 2, 300, 520, dqk, dv, True, seed=405 + dqk)


def test_bench_ring_step_runs_chunks_side_by_side(vca):
    """bench.py's ring share step runs the local and the earlier chunk's
    forward and backward on two streams and adds the earlier chunk's dq in
    with the library's row scatter-add: the same out, lse, dk and dv
    (bitwise) as the two chunks run one after the other, and the same dq up
    to the one extra rounding of the earlier chunk's dq to bf16."""
    import bench

    p = bench.Problem(5)
    dq, dkl, dvl, dke, dve = p.step()
    out, lse = p.out.clone(), p.lse.clone()
    t, w = p.t, p.w
    cq, ck, mq, mk = p.local
    o1, l1 = vca.fwd_varlen(t["q"], t["k_local"], t["v_local"], cq, ck, mq, mk, w.scale, True)
    cq2, ck2, mq2, mk2 = p.cross
    o2, l2 = vca.fwd_varlen(t["q"], t["k_early"], t["v_early"], cq2, ck2, mq2, mk2, w.scale, False)
    _, rlse, rout = vca.merge(o1, l1, o2, l2, copy_dtype=torch.bfloat16)
    rdq, rdkl, rdvl = vca.bwd_varlen(t["do"], t["q"], t["k_local"], t["v_local"], rout, rlse, cq,
                                     ck, mq, mk, w.scale, True)
    _, rdke, rdve = vca.bwd_varlen(t["do"], t["q"], t["k_early"], t["v_early"], rout, rlse, cq2,
                                   ck2, mq2, mk2, w.scale, False, dq_accumulate=rdq)
    torch.cuda.synchronize()
    assert torch.equal(out, rout) and torch.equal(lse, rlse)
    for a, b in ((dkl, rdkl), (dvl, rdvl), (dke, rdke), (dve, rdve)):
        assert torch.equal(a, b)
    d = (dq.float() - rdq.float()).abs().max().item()
    assert d <= 2.0 ** -7 * rdq.float().abs().max().item(), f"dq differs by {d}"


# ---------------------------------------------------------------- fp16
@pytest.mark.parametrize("dqk,dv", [(64, 64), (128, 128), (192, 128), (256, 256), (512, 512)])
@pytest.mark.parametrize("causal", [True, False])
def test_fp16_every_head_dim(vca, dqk, dv, causal):
    """fp16 inputs ("ffpa_attention" page: bf16 and fp16 take the same path):
    ragged segments with zero-query and zero-key ones, GQA, every head dim."""
    lens_q = [1, 37, 0, 200, 129, 64, 3]
    lens_k = [1, 37, 12, 200, 129, 64, 0]
    run_varlen(vca, lens_q, lens_k, 8, 2, dqk, dv, causal, seed=401 + dqk + causal,
               dtype=torch.float16)
    run_dense(vca, 1, 4, 2, 130, 160, dqk, dv, causal, seed=403 + dqk, dtype=torch.float16)


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_fp16_workloads_full_size(vca, n):
    """Every workload at full size with fp16 inputs (the same draws rounded to
    float16): NaN-filled outputs all written, and the oracle on seeded rows
    and key rows of every segment (or batch entry) x head."""
    w = workloads.workload(n)
    if w.kind == "ring":
        check_ring_share(vca, n, torch.float16)
        return
    t = w.tensors(torch.float16)
    if w.kind == "varlen":
        res = run_full_varlen(vca, w, t)
        check_sampled(res, t, w.cu(), w.Hq, w.Hkv, w.scale, True, seed=500 + n)
        return
    q, k, v, do = (dev(t[x]) for x in ("q", "k", "v", "do"))
    B, N, et = w.B, w.Nq, q.dtype
    out, lse = nan_like((B, w.Hq, N, w.Dv), et), nan_like((B, w.Hq, N), torch.float32)
    vca.fwd_dense(q, k, v, w.scale, True, out=out, lse=lse)
    dq, dk, dv = (nan_like((B, w.Hq, N, w.Dqk), et), nan_like((B, w.Hkv, N, w.Dqk), et),
                  nan_like((B, w.Hkv, N, w.Dv), et))
    vca.bwd_dense(do, q, k, v, out, lse, w.scale, True, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert_all_written(out=out, lse=lse, dq=dq, dk=dk, dv=dv)
    if n == 1:  # small: the whole problem
        ro, rl = orc.fwd_dense(t["q"], t["k"], t["v"], w.scale, True)
        rg = orc.bwd_dense(t["do"], t["q"], t["k"], t["v"], ro, rl, w.scale, True)
        check_out(out, ro)
        check_lse(lse, rl)
        for name, a, b in zip(("dq", "dk", "dv"), (dq, dk, dv), rg):
            check_grad(name, a, b)
        return
    thd = lambda x: x.transpose(1, 2).reshape(B * N, x.shape[1], x.shape[3])  # noqa: E731
    tt = {x: thd(t[x]) for x in ("q", "k", "v", "do")}
    res = (thd(out), lse.reshape(B, w.Hq, N).transpose(0, 1).reshape(w.Hq, B * N),
           (thd(dq), thd(dk), thd(dv)))
    check_sampled(res, tt, np.array([0, N, 2 * N]), w.Hq, w.Hkv, w.scale, True, seed=500 + n)


def test_fp16_merge_copy_and_zero_rows(vca):
    g = torch.Generator().manual_seed(73)
    rows, H, Dv = 120, 2, 64
    oa, ob = rand((rows, H, Dv), g, torch.float16), rand((rows, H, Dv), g, torch.float16)
    la = torch.randn((H, rows), generator=g) * 3
    lb = torch.randn((H, rows), generator=g) * 3
    lb[1, :5] = -math.inf
    ro, rl = orc.merge(oa, la, ob, lb)
    mo, ml, mc = vca.merge(dev(oa), dev(la), dev(ob), dev(lb), copy_dtype=torch.float16)
    torch.cuda.synchronize()
    assert np.abs(host(mo) - ro).max() < 1e-5
    check_lse(ml, rl)
    assert mc.dtype == torch.float16 and torch.equal(mc, mo.to(torch.float16))
    out = torch.ones((1, 2, 4, 8), dtype=torch.float16, device="cuda")
    r = torch.zeros((1, 4), dtype=torch.bool, device="cuda")
    r[0, 1] = True
    vca.zero_rows(out, None, r)
    torch.cuda.synchronize()
    assert torch.all(out[0, :, 1] == 0) and torch.all(out[0, :, 0] == 1)



# ---------------------------------------------------------------- packed ring layout
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
def test_ring_row_moves_and_row_merge(vca, dtype):
    """gather_rows / scatter_rows (assign, assign with zeroed rest, add) /
    gather_lse / scatter_lse / merge_rows on BSHD-strided [B, H, S, D] views
    against the oracle's row moves and live-row merge."""
    g = torch.Generator().manual_seed(75)
    B, H, S, D = 2, 3, 37, 64
    store = rand((B, S, H, D), g, dtype)  # BSHD storage, viewed as [B, H, S, D]
    x = dev(store).transpose(1, 2)
    idx_np = np.array([5, 40, 0, 73, 36, 12, 50], dtype=np.int32)
    idx = dev(torch.from_numpy(idx_np))
    got = vca.gather_rows(x, idx)
    np.testing.assert_array_equal(host(got), orc.ring_gather(store.transpose(1, 2), idx_np))
    # assign into a view holding old values: named rows replaced, others kept
    old = rand((B, S, H, D), g, dtype)
    dst = dev(old).transpose(1, 2)
    vca.scatter_rows(got, idx, dst, mode=0)
    want = orc.f64(old.transpose(1, 2)).copy()
    named = orc.ring_scatter(orc.f64(got), idx_np, B, S, fill=np.nan)
    keep = np.isnan(named)
    np.testing.assert_array_equal(host(dst), np.where(keep, want, named))
    # assign with the rest zeroed = ring_scatter
    vca.scatter_rows(got, idx, dst, mode=1)
    np.testing.assert_array_equal(host(dst), orc.ring_scatter(orc.f64(got), idx_np, B, S))
    # add: named rows gain src (one rounding of the fp32 sum)
    base = dev(rand((B, S, H, D), g, dtype)).transpose(1, 2)
    ref = host(base) + orc.ring_scatter(orc.f64(got), idx_np, B, S)
    vca.scatter_rows(got, idx, base, mode=2)
    torch.cuda.synchronize()
    tol = 0 if dtype == torch.float32 else 2 ** -7 * np.abs(ref).max()
    assert np.abs(host(base) - ref).max() <= tol + 1e-6
    # lse moves
    lse = dev(torch.randn((B, H, S), generator=g))
    lp = vca.gather_lse(lse, idx)
    np.testing.assert_array_equal(host(lp), orc.ring_gather(host(lse)[..., None], idx_np)[..., 0].T)
    ld = vca.scatter_lse(lp, idx, B, S)
    np.testing.assert_array_equal(
        host(ld), orc.ring_scatter(host(lp).T[:, :, None], idx_np, B, S, fill=-np.inf)[..., 0])
    # live-row merge into fp32 accumulators (one live row starts at -inf)
    acc = dev(torch.randn((B, S, H, D), generator=g)).transpose(1, 2)
    lacc = dev(torch.randn((B, H, S), generator=g))
    lacc[0, 1, 5] = -math.inf
    ob = dev(rand((len(idx_np), H, D), g, dtype))
    lb = dev(torch.randn((H, len(idx_np)), generator=g))
    lb[2, 3] = -math.inf
    ro, rl = orc.ring_merge_rows(host(acc), host(lacc), host(ob), host(lb), idx_np)
    vca.merge_rows(acc, lacc, ob, lb, idx)
    torch.cuda.synchronize()
    assert np.abs(host(acc) - ro).max() < 1e-5
    check_lse(lacc, rl)
    # fp32 rows gathered into a 16-bit type round to nearest even
    if dtype != torch.float32:
        acc2 = dev(torch.randn((B, S, H, D), generator=g)).transpose(1, 2)
        r16 = vca.gather_rows(acc2, idx, dtype=dtype)
        assert torch.equal(r16, vca.gather_rows(acc2, idx).to(dtype))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_ring_share_gather_layout(vca, dtype):
    """The ring share at full size through the packed gather layout: partial
    chunk results, the in-place merge and both chunk backwards against the
    document-causal oracle (every kv-head group sampled)."""
    check_ring_share(vca, 5, dtype, route="gather")
