"""GPU parity of the left sliding window and the logit softcap (the _ex entry
points) against the fp64 oracle on the same seeded inputs.

The window follows the "attention utils" page's reading of a positive left
window (a query sees its W most recent keys, itself included); the softcap
turns every scaled score x into cap * tanh(x / cap) ("ffpa_attention" page,
softcap argument). Both apply per segment, with the bottom-right causal
alignment. Tolerances are those of the plain parity tests: out max-abs <=
2e-2, lse max-abs <= 5e-3 (with the -inf pattern exact), gradients relative
Frobenius <= 5e-2.
"""
import math

import numpy as np
import pytest
import torch

import workloads
from oracle import attention as orc

pytestmark = pytest.mark.gpu

OUT_TOL, LSE_TOL, GRAD_TOL = 2e-2, 5e-3, 5e-2
DIMS = [(64, 64), (128, 128), (192, 128), (256, 256), (512, 512)]


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


def check_out(out, ref):
    err = np.abs(host(out) - ref).max() if ref.size else 0.0
    assert err <= OUT_TOL, f"out max-abs {err}"


def check_lse(lse, ref):
    got = host(lse)
    assert np.array_equal(np.isneginf(got), np.isneginf(ref)), "-inf rows differ"
    fin = np.isfinite(ref)
    if fin.any():
        err = np.abs(got[fin] - ref[fin]).max()
        assert err <= LSE_TOL, f"lse max-abs {err}"


def check_grad(name, g, ref):
    g = host(g)
    den, num = np.linalg.norm(ref), np.linalg.norm(g - ref)
    if den == 0:
        # exact zeros in the oracle can come from a cancellation (a window of
        # one key: P = 1 and dP - delta = 0), which rounding leaves near zero
        err = np.abs(g).max() if g.size else 0.0
        assert err <= 1e-3, f"{name}: expected zeros, max-abs {err}"
        return
    assert num / den <= GRAD_TOL, f"{name} rel-Frobenius {num / den}"


def run_varlen(vca, lens_q, lens_k, Hq, Hkv, Dqk, Dv, causal, seed, window=0, softcap=0.0,
               dtype=torch.bfloat16, scale=None):
    g = torch.Generator().manual_seed(seed)
    cu_q, cu_k = workloads.cumulative(lens_q), workloads.cumulative(lens_k)
    Tq, Tk = int(cu_q[-1]), int(cu_k[-1])
    q = workloads.randn_bf16((Tq, Hq, Dqk), g, dtype)
    k = workloads.randn_bf16((Tk, Hkv, Dqk), g, dtype)
    v = workloads.randn_bf16((Tk, Hkv, Dv), g, dtype)
    do = workloads.randn_bf16((Tq, Hq, Dv), g, dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(Dqk)
    kw = dict(window=window or None, softcap=softcap or None)
    ro, rl = orc.fwd_varlen(q, k, v, cu_q, cu_k, scale, causal, **kw)
    rdq, rdk, rdv = orc.bwd_varlen(do, q, k, v, ro, rl, cu_q, cu_k, scale, causal, **kw)
    cq, ck = dev(torch.from_numpy(cu_q)), dev(torch.from_numpy(cu_k))
    mq, mk = max(lens_q, default=0), max(lens_k, default=0)
    out, lse = vca.fwd_varlen(dev(q), dev(k), dev(v), cq, ck, mq, mk, scale, causal,
                              window=window, softcap=softcap)
    grads = vca.bwd_varlen(dev(do), dev(q), dev(k), dev(v), out, lse, cq, ck, mq, mk, scale,
                           causal, window=window, softcap=softcap)
    torch.cuda.synchronize()
    check_out(out, ro)
    check_lse(lse, rl)
    for name, a, b in zip(("dq", "dk", "dv"), grads, (rdq, rdk, rdv)):
        check_grad(name, a, b)
    return out, lse, grads


@pytest.mark.parametrize("dqk,dv", DIMS)
@pytest.mark.parametrize("window", [1, 37, 300])
def test_window_every_head_dim(vca, dqk, dv, window):
    # windows of one key, inside one tile, and wider than most segments;
    # segments from 1 to 600 tokens span several tiles of every kernel
    lens = [1, 37, 200, 129, 64, 600]
    run_varlen(vca, lens, lens, 4, 2, dqk, dv, True, seed=1000 + dqk + window, window=window)


@pytest.mark.parametrize("dqk,dv", DIMS)
@pytest.mark.parametrize("causal", [True, False])
def test_softcap_every_head_dim(vca, dqk, dv, causal):
    # a small cap so tanh saturates on part of the scores; a larger scale
    # widens the score range
    lens = [1, 37, 200, 129, 300]
    run_varlen(vca, lens, lens, 4, 2, dqk, dv, causal, seed=1100 + dqk + causal, softcap=1.5,
               scale=2.0 / math.sqrt(dqk))


@pytest.mark.parametrize("dqk,dv", DIMS)
def test_window_and_softcap_ragged_segments(vca, dqk, dv):
    # lq != lk (bottom-right shift in both directions), zero-query and
    # zero-key segments, a negative scale, both options at once
    lens_q = [5, 0, 130, 70, 0, 3, 290]
    lens_k = [9, 40, 100, 70, 12, 0, 520]
    run_varlen(vca, lens_q, lens_k, 8, 2, dqk, dv, True, seed=1200 + dqk, window=45,
               softcap=3.0, scale=-1.0 / math.sqrt(dqk))


@pytest.mark.parametrize("dqk,dv", [(128, 128), (192, 128)])
def test_window_backward_store_modes(vca, monkeypatch, dqk, dv):
    """The dS store (dQ from the stored blocks, which a window leaves out
    below its edge) and the recompute dQ pass give the oracle's gradients."""
    lens = [700, 3, 260]
    for mib in ("8192", "0"):
        monkeypatch.setenv("ATTN_BWD_DS_MIB", mib)
        run_varlen(vca, lens, lens, 4, 1, dqk, dv, True, seed=1300 + dqk, window=100,
                   softcap=2.0)


@pytest.mark.parametrize("dqk,dv", [(256, 256), (512, 512)])
def test_window_two_phase_in_chunks(vca, monkeypatch, dqk, dv):
    """The two-phase backward run in chunks of 256-query row slots (a 1 MiB
    store budget): the window's block ranges meet the chunk ranges."""
    monkeypatch.setenv("ATTN_BWD_TILES_MIB", "1")
    lens = [3, 700, 260]
    run_varlen(vca, lens, lens, 4, 2, dqk, dv, True, seed=1350 + dqk, window=300, softcap=2.0)


def test_window_fp16(vca):
    lens = [3, 150, 333]
    for dqk, dv in DIMS:
        run_varlen(vca, lens, lens, 4, 2, dqk, dv, True, seed=1400 + dqk, window=64,
                   softcap=4.0, dtype=torch.float16)


def test_window_dense_gqa(vca):
    g = torch.Generator().manual_seed(1500)
    for (Nq, Nk, dqk, dv, W) in [(130, 300, 128, 128, 50), (300, 130, 64, 64, 7),
                                 (257, 257, 512, 512, 100), (200, 200, 256, 256, 199)]:
        B, Hq, Hkv = 2, 4, 2
        q = workloads.randn_bf16((B, Hq, Nq, dqk), g)
        k = workloads.randn_bf16((B, Hkv, Nk, dqk), g)
        v = workloads.randn_bf16((B, Hkv, Nk, dv), g)
        do = workloads.randn_bf16((B, Hq, Nq, dv), g)
        scale = 1.0 / math.sqrt(dqk)
        ro, rl = orc.fwd_dense(q, k, v, scale, True, window=W, softcap=2.5)
        rg = orc.bwd_dense(do, q, k, v, ro, rl, scale, True, window=W, softcap=2.5)
        out, lse = vca.fwd_dense(dev(q), dev(k), dev(v), scale, True, window=W, softcap=2.5)
        grads = vca.bwd_dense(dev(do), dev(q), dev(k), dev(v), out, lse, scale, True, window=W,
                              softcap=2.5)
        torch.cuda.synchronize()
        check_out(out, ro)
        check_lse(lse, rl)
        for name, a, b in zip(("dq", "dk", "dv"), grads, rg):
            check_grad(name, a, b)


class _Lookup:
    """The oracle's sampled rows as an indexable array: x[i, j] is the stored
    entry (only those indices are ever read by the row samplers)."""

    def __init__(self, keys, values):
        self.d = {tuple(int(e) for e in k): v for k, v in zip(keys, values)}

    def __getitem__(self, idx):
        return self.d[tuple(int(e) for e in idx)]


def test_window_long_segment_sampled(vca):
    """One 6000-token document at head dim 128 with a 1000-key window: the
    forward and dQ passes skip most key tiles and the dK/dV pass most query
    steps. Checked on sampled rows and key columns, each against the oracle
    on exactly the rows that see it."""
    L, Hq, Hkv, D, W = 6000, 2, 1, 128, 1000
    g = torch.Generator().manual_seed(1600)
    q = workloads.randn_bf16((L, Hq, D), g)
    k = workloads.randn_bf16((L, Hkv, D), g)
    v = workloads.randn_bf16((L, Hkv, D), g)
    do = workloads.randn_bf16((L, Hq, D), g)
    scale = 1.0 / math.sqrt(D)
    cu = np.array([0, L], dtype=np.int32)
    c = dev(torch.from_numpy(cu))
    out, lse = vca.fwd_varlen(dev(q), dev(k), dev(v), c, c, L, L, scale, True, window=W)
    dq, dk, dv = vca.bwd_varlen(dev(do), dev(q), dev(k), dev(v), out, lse, c, c, L, L, scale,
                                True, window=W)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 999, 1000, 1001, 2047, 4096, 5999] * Hq)
    heads = np.repeat(np.arange(Hq), 8)
    kf, vf = orc.f64(k), orc.f64(v)
    ro, rl = orc.fwd_varlen_rows(q, kf, vf, cu, cu, scale, True, rows, heads, window=W)
    it, ih = torch.from_numpy(rows).cuda(), torch.from_numpy(heads).cuda()
    check_out(out[it, ih], ro)
    check_lse(lse[ih, it], rl)
    rdq = orc.bwd_varlen_rows(do, q, kf, vf, _Lookup(zip(rows, heads), ro),
                              _Lookup(zip(heads, rows), rl), cu, cu, scale, True, rows, heads,
                              window=W)
    check_grad("dq rows", dq[it, ih], rdq)
    # key j is seen by rows j .. j + W - 1: the oracle runs on those rows only
    # (a shifted sub-problem with the same visibility)
    for j in (0, 1500, 5999):
        i1 = min(L, j + W)
        # rows j..i1-1 against keys 0..i1-1: the bottom-right shift i1 - (i1 - j)
        # = j keeps every kept row's visibility (keys in (row - W, row])
        qq, dd = q[j:i1], do[j:i1]
        kk, vv = k[:i1], v[:i1]
        cq1, ck1 = [0, i1 - j], [0, i1]
        so, sl = orc.fwd_varlen(qq, kk, vv, cq1, ck1, scale, True, window=W)
        k1, v1 = orc.bwd_varlen_cols(dd, qq, kk, vv, so, sl, cq1, ck1, scale, True, [j], [0],
                                     window=W)
        check_grad("dk col", dk[j, 0:1], k1[0][None])
        check_grad("dv col", dv[j, 0:1], v1[0][None])


def test_zero_options_are_the_plain_call(vca):
    """window = 0 and softcap = 0 through the _ex entry points give bitwise
    the plain call's results (ops passes NULL for them; the C side is called
    here with an explicit zero struct)."""
    import ctypes as C

    from varlen_causal_attention_amd import _lib

    lens = [100, 260]
    g = torch.Generator().manual_seed(1700)
    cu = workloads.cumulative(lens)
    T = int(cu[-1])
    q, k, v = (dev(workloads.randn_bf16((T, 2, 128), g)) for _ in range(3))
    c = dev(torch.from_numpy(cu))
    out0, lse0 = vca.fwd_varlen(q, k, v, c, c, 260, 260, 0.1, True)
    out1, lse1 = torch.empty_like(out0), torch.empty_like(lse0)
    lib = _lib.load()
    strides = _lib.i64_array([q.stride(0), q.stride(1)] * 4)
    ext = C.pointer(_lib.AttnExt(0, 0.0))
    need = C.c_size_t(0)
    args = (_lib.ATTN_BF16, C.c_void_p(q.data_ptr()), C.c_void_p(k.data_ptr()),
            C.c_void_p(v.data_ptr()), C.c_void_p(out1.data_ptr()), C.c_void_p(lse1.data_ptr()),
            C.c_void_p(c.data_ptr()), C.c_void_p(c.data_ptr()), 2, 260, 260, T, T, 2, 2, 128, 128,
            strides, 0.1, 1, ext)
    _lib.check(lib.attn_fwd_varlen_ex(*args, None, C.byref(need), None), "size")
    ws = torch.empty(need.value, dtype=torch.uint8, device="cuda")
    have = C.c_size_t(ws.numel())
    stream = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    _lib.check(lib.attn_fwd_varlen_ex(*args, C.c_void_p(ws.data_ptr()), C.byref(have), stream),
               "run")
    torch.cuda.synchronize()
    assert torch.equal(out0, out1) and torch.equal(lse0, lse1)
