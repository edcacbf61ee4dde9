"""Pins for the fp64 oracle, checked against what the pages and the mathematics
fix rather than against the oracle itself: hand-worked values, closed forms,
brute force on tiny inputs, finite differences, invariants and a library
routine (torch's fp64 SDPA with an explicit bottom-right mask)."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def _arr(x):
    return np.array([[float(e) for e in r] if isinstance(r, list) else float(r) for r in x])


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# ---------------------------------------------------------------- hand-worked
def test_golden_causal_forward_and_backward():
    g = json.load(open(GOLDEN))["causal_2x2"]
    q, k, v, do = (np.array(g[n])[:, None, :] for n in ("q", "k", "v", "do"))  # [T,1,D]
    cu = [0, 2]
    out, lse = orc.fwd_varlen(q, k, v, cu, cu, g["scale"], True)
    np.testing.assert_allclose(out[:, 0], g["out"], atol=1e-12)
    np.testing.assert_allclose(lse[0], g["lse"], atol=1e-12)
    dq, dk, dv = orc.bwd_varlen(do, q, k, v, out, lse, cu, cu, g["scale"], True)
    np.testing.assert_allclose(dq[:, 0], g["dq"], atol=1e-12)
    np.testing.assert_allclose(dk[:, 0], g["dk"], atol=1e-12)
    np.testing.assert_allclose(dv[:, 0], g["dv"], atol=1e-12)
    # the same numbers through the dense entry
    o2, l2 = orc.fwd_dense(q.transpose(1, 0, 2)[None], k.transpose(1, 0, 2)[None],
                           v.transpose(1, 0, 2)[None], g["scale"], True)
    np.testing.assert_allclose(o2[0, 0], g["out"], atol=1e-12)
    np.testing.assert_allclose(l2[0, 0], g["lse"], atol=1e-12)


def test_golden_noncausal_forward():
    g = json.load(open(GOLDEN))["noncausal_2x2"]
    q, k, v = (np.array(g[n])[:, None, :] for n in ("q", "k", "v"))
    out, lse = orc.fwd_varlen(q, k, v, [0, 2], [0, 2], g["scale"], False)
    np.testing.assert_allclose(out[:, 0], g["out"], atol=1e-12)
    np.testing.assert_allclose(lse[0], g["lse"], atol=1e-12)


def test_golden_merge():
    g = json.load(open(GOLDEN))["merge"]
    oa, ob = np.array(g["out_a"])[:, None, :], np.array(g["out_b"])[:, None, :]
    la, lb = _arr(g["lse_a"])[None], _arr(g["lse_b"])[None]
    out, lse = orc.merge(oa, la, ob, lb)
    np.testing.assert_allclose(out[:, 0], g["out"], atol=1e-12)
    np.testing.assert_array_equal(np.isinf(lse[0]), np.isinf(_arr(g["lse"])))
    fin = np.isfinite(_arr(g["lse"]))
    np.testing.assert_allclose(lse[0][fin], _arr(g["lse"])[fin], atol=1e-12)


# ---------------------------------------------------------------- closed forms
@pytest.mark.parametrize("lq,lk", [(5, 5), (3, 7), (7, 3), (1, 4), (4, 1), (6, 0), (1, 1)])
def test_uniform_scores_count_visible_keys(lq, lk):
    """q = 0 makes every score 0: lse_i = ln(#visible) and out_i = mean of the
    visible values. Bottom-right alignment fixes #visible = clip(i+lk-lq+1, 0, lk)."""
    rng = np.random.default_rng(0)
    q = np.zeros((lq, 1, 4))
    k = _rand(rng, lk, 1, 4)
    v = _rand(rng, lk, 1, 3)
    out, lse = orc.fwd_varlen(q, k, v, [0, lq], [0, lk], 0.7, True)
    for i in range(lq):
        n = min(max(i + lk - lq + 1, 0), lk)
        if n == 0:
            assert lse[0, i] == -np.inf
            np.testing.assert_array_equal(out[i, 0], 0.0)
        else:
            assert abs(lse[0, i] - math.log(n)) < 1e-12
            np.testing.assert_allclose(out[i, 0], v[:n, 0].mean(axis=0), atol=1e-12)


def test_identical_keys_give_mean_of_values():
    rng = np.random.default_rng(1)
    lq, lk, scale = 4, 6, 0.3
    q = _rand(rng, lq, 2, 5)
    krow = _rand(rng, 5)
    k = np.tile(krow, (lk, 1, 1))  # [lk, 1, 5]
    v = _rand(rng, lk, 1, 3)
    out, lse = orc.fwd_varlen(q, k, v, [0, lq], [0, lk], scale, False)
    for h in range(2):
        for i in range(lq):
            s = scale * q[i, h] @ krow
            assert abs(lse[h, i] - (s + math.log(lk))) < 1e-12
            np.testing.assert_allclose(out[i, h], v[:, 0].mean(axis=0), atol=1e-12)


def test_causal_query0_is_v0():
    rng = np.random.default_rng(2)
    q, k, v = _rand(rng, 8, 2, 4), _rand(rng, 8, 1, 4), _rand(rng, 8, 1, 6)
    out, lse = orc.fwd_varlen(q, k, v, [0, 8], [0, 8], 0.5, True)
    for h in range(2):
        np.testing.assert_allclose(out[0, h], v[0, 0], atol=1e-13)
        assert abs(lse[h, 0] - 0.5 * q[0, h] @ k[0, 0]) < 1e-12


def test_brute_force_single_rows():
    """Plain Python sums over the visible keys of every row, tiny sizes."""
    rng = np.random.default_rng(3)
    lq, lk, scale = 3, 5, 0.9
    q, k, v = _rand(rng, lq, 1, 2), _rand(rng, lk, 1, 2), _rand(rng, lk, 1, 2)
    out, lse = orc.fwd_varlen(q, k, v, [0, lq], [0, lk], scale, True)
    for i in range(lq):
        keys = [j for j in range(lk) if j <= i + lk - lq]
        w = [math.exp(scale * sum(q[i, 0, d] * k[j, 0, d] for d in range(2))) for j in keys]
        z = sum(w)
        assert abs(lse[0, i] - math.log(z)) < 1e-12
        for d in range(2):
            assert abs(out[i, 0, d] - sum(wj * v[j, 0, d] for wj, j in zip(w, keys)) / z) < 1e-12


# ---------------------------------------------------------------- library routine
def _sdpa_reference(q, k, v, vis, scale):
    """torch fp64 SDPA with an explicit boolean mask (True = attend)."""
    qt, kt, vt = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=torch.tensor(vis), scale=scale)
    return qt, kt, vt, out


@pytest.mark.parametrize("Nq,Nk,causal", [(9, 9, True), (5, 11, True), (7, 7, False), (6, 3, False)])
def test_matches_torch_sdpa_fp64(Nq, Nk, causal):
    rng = np.random.default_rng(4)
    B, Hq, Hkv, Dqk, Dv, scale = 2, 4, 2, 6, 5, 0.37
    q, k, v = _rand(rng, B, Hq, Nq, Dqk), _rand(rng, B, Hkv, Nk, Dqk), _rand(rng, B, Hkv, Nk, Dv)
    do = _rand(rng, B, Hq, Nq, Dv)
    out, lse = orc.fwd_dense(q, k, v, scale, causal)
    vis = orc.segment_visible(Nq, Nk, causal)
    # the library routine, fed K/V repeated per q-head (contiguous GQA groups)
    kr, vr = np.repeat(k, Hq // Hkv, axis=1), np.repeat(v, Hq // Hkv, axis=1)
    qt, kt, vt, ref = _sdpa_reference(q, kr, vr, vis, scale)
    np.testing.assert_allclose(out, ref.detach().numpy(), atol=1e-12)
    s = torch.tensor(scale * q @ kr.transpose(0, 1, 3, 2)).masked_fill(~torch.tensor(vis), -math.inf)
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), atol=1e-12)
    ref.backward(torch.tensor(do))
    dq, dk, dv = orc.bwd_dense(do, q, k, v, out, lse, scale, causal)
    np.testing.assert_allclose(dq, qt.grad.numpy(), atol=1e-11)
    G = Hq // Hkv
    dk_ref = kt.grad.numpy().reshape(B, Hkv, G, Nk, Dqk).sum(axis=2)
    dv_ref = vt.grad.numpy().reshape(B, Hkv, G, Nk, Dv).sum(axis=2)
    np.testing.assert_allclose(dk, dk_ref, atol=1e-11)
    np.testing.assert_allclose(dv, dv_ref, atol=1e-11)


# ---------------------------------------------------------------- gradients
def test_backward_matches_finite_differences():
    rng = np.random.default_rng(5)
    Tq, Hq, Hkv, Dqk, Dv, scale = 5, 2, 1, 3, 4, 0.8
    cu_q, cu_k = [0, 2, 5], [0, 3, 6]
    q, k, v = _rand(rng, Tq, Hq, Dqk), _rand(rng, 6, Hkv, Dqk), _rand(rng, 6, Hkv, Dv)
    do = _rand(rng, Tq, Hq, Dv)

    def loss(q_, k_, v_):
        o, _ = orc.fwd_varlen(q_, k_, v_, cu_q, cu_k, scale, True)
        return float((o * do).sum())

    out, lse = orc.fwd_varlen(q, k, v, cu_q, cu_k, scale, True)
    grads = orc.bwd_varlen(do, q, k, v, out, lse, cu_q, cu_k, scale, True)
    eps = 1e-6
    for which, x in enumerate((q, k, v)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which], args_m[which] = xp, xm
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        err = np.abs(num - grads[which]).max() / max(np.abs(num).max(), 1e-30)
        assert err < 1e-6, (which, err)


def test_lse_gradient_is_attention_over_keys():
    """d lse_i / d q_i = scale * sum_j P_ij k_j: the forward with v := k."""
    rng = np.random.default_rng(6)
    q, k = _rand(rng, 4, 1, 3), _rand(rng, 6, 1, 3)
    scale, eps = 0.6, 1e-6
    out_kk, lse = orc.fwd_varlen(q, k, k, [0, 4], [0, 6], scale, True)
    for i in range(4):
        for d in range(3):
            qp, qm = q.copy(), q.copy()
            qp[i, 0, d] += eps
            qm[i, 0, d] -= eps
            lp = orc.fwd_varlen(qp, k, k, [0, 4], [0, 6], scale, True)[1][0, i]
            lm = orc.fwd_varlen(qm, k, k, [0, 4], [0, 6], scale, True)[1][0, i]
            assert abs((lp - lm) / (2 * eps) - scale * out_kk[i, 0, d]) < 1e-7


# ---------------------------------------------------------------- invariants
def test_gqa_equals_mha_on_repeated_kv():
    rng = np.random.default_rng(7)
    T, Hq, Hkv, D = 12, 6, 2, 4
    cu = [0, 5, 12]
    q, k, v, do = _rand(rng, T, Hq, D), _rand(rng, T, Hkv, D), _rand(rng, T, Hkv, D), _rand(rng, T, Hq, D)
    kr, vr = np.repeat(k, Hq // Hkv, axis=1), np.repeat(v, Hq // Hkv, axis=1)
    o1, l1 = orc.fwd_varlen(q, k, v, cu, cu, 0.5, True)
    o2, l2 = orc.fwd_varlen(q, kr, vr, cu, cu, 0.5, True)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)
    g1 = orc.bwd_varlen(do, q, k, v, o1, l1, cu, cu, 0.5, True)
    g2 = orc.bwd_varlen(do, q, kr, vr, o2, l2, cu, cu, 0.5, True)
    np.testing.assert_allclose(g1[0], g2[0], atol=1e-13)
    np.testing.assert_allclose(g1[1], g2[1].reshape(T, Hkv, 3, D).sum(axis=2), atol=1e-12)
    np.testing.assert_allclose(g1[2], g2[2].reshape(T, Hkv, 3, D).sum(axis=2), atol=1e-12)


def test_varlen_is_concatenation_of_dense_documents():
    rng = np.random.default_rng(8)
    lens = [3, 7, 1, 5]
    T, H, D = sum(lens), 2, 4
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, do = (_rand(rng, T, H, D) for _ in range(4))
    o, l = orc.fwd_varlen(q, k, v, cu, cu, 0.4, True)
    g = orc.bwd_varlen(do, q, k, v, o, l, cu, cu, 0.4, True)
    for a, b in zip(cu[:-1], cu[1:]):
        bh = lambda x: x[a:b].transpose(1, 0, 2)[None]  # noqa: E731 - [1,H,n,D]
        od, ld = orc.fwd_dense(bh(q), bh(k), bh(v), 0.4, True)
        np.testing.assert_allclose(o[a:b], od[0].transpose(1, 0, 2), atol=1e-13)
        np.testing.assert_allclose(l[:, a:b], ld[0], atol=1e-13)
        gd = orc.bwd_dense(bh(do), bh(q), bh(k), bh(v), od, ld, 0.4, True)
        for x, y in zip(g, gd):
            np.testing.assert_allclose(x[a:b], y[0].transpose(1, 0, 2), atol=1e-12)
    # zero-query segments (keys nobody sees) change nothing for the queries and
    # give their keys zero gradients
    k2 = np.concatenate([k[:3], _rand(rng, 4, H, D), k[3:]])
    v2 = np.concatenate([v[:3], _rand(rng, 4, H, D), v[3:]])
    cu_q2 = [0, 3, 3, 10, 11, 16]
    cu_k2 = [0, 3, 7, 14, 15, 20]
    o2, l2 = orc.fwd_varlen(q, k2, v2, cu_q2, cu_k2, 0.4, True)
    np.testing.assert_allclose(o2, o, atol=1e-13)
    np.testing.assert_allclose(l2, l, atol=1e-13)
    g2 = orc.bwd_varlen(do, q, k2, v2, o2, l2, cu_q2, cu_k2, 0.4, True)
    np.testing.assert_array_equal(g2[1][3:7], 0.0)
    np.testing.assert_array_equal(g2[2][3:7], 0.0)
    np.testing.assert_allclose(np.delete(g2[1], range(3, 7), axis=0), g[1], atol=1e-12)


def test_zero_key_segment_rows_are_empty():
    rng = np.random.default_rng(9)
    q, k, v = _rand(rng, 4, 1, 3), _rand(rng, 2, 1, 3), _rand(rng, 2, 1, 3)
    for causal in (True, False):
        o, l = orc.fwd_varlen(q, k, v, [0, 3, 4], [0, 0, 2], 0.5, causal)
        np.testing.assert_array_equal(o[:3], 0.0)
        assert np.all(l[0, :3] == -np.inf) and np.isfinite(l[0, 3])
        g = orc.bwd_varlen(q, q, k, v, o, l, [0, 3, 4], [0, 0, 2], 0.5, causal)
        np.testing.assert_array_equal(g[0][:3], 0.0)


def test_merge_of_two_key_chunks_is_full_attention():
    rng = np.random.default_rng(10)
    Tq, Tk, H, D = 9, 14, 2, 4
    q, k, v, do = _rand(rng, Tq, H, D), _rand(rng, Tk, H, D), _rand(rng, Tk, H, D), _rand(rng, Tq, H, D)
    # global positions: keys 0..13, queries 5..13 (so early queries miss late keys)
    q_pos, k_pos = np.arange(5, 14), np.arange(14)
    q_doc = np.array([1, 1, 2, 2, 2, 0, 3, 3, 3])
    k_doc = np.array([1, 1, 1, 1, 2, 1, 1, 2, 2, 2, 0, 3, 3, 3])
    full_o, full_l = orc.fwd_doc_causal(q, k, v, q_doc, q_pos, k_doc, k_pos, 0.5)
    a, b = slice(0, 6), slice(6, 14)
    oa, la = orc.fwd_doc_causal(q, k[a], v[a], q_doc, q_pos, k_doc[a], k_pos[a], 0.5)
    ob, lb = orc.fwd_doc_causal(q, k[b], v[b], q_doc, q_pos, k_doc[b], k_pos[b], 0.5)
    mo, ml = orc.merge(oa, la, ob, lb)
    np.testing.assert_allclose(mo, full_o, atol=1e-13)
    np.testing.assert_array_equal(np.isinf(ml), np.isinf(full_l))
    np.testing.assert_allclose(ml[np.isfinite(ml)], full_l[np.isfinite(full_l)], atol=1e-13)
    # pad query (doc 0) is empty everywhere: out 0, lse -inf
    np.testing.assert_array_equal(mo[5], 0.0)
    assert np.all(ml[:, 5] == -np.inf)
    # backward per chunk with the merged out/lse: dq sums, dk/dv are slices
    gf = orc.bwd_doc_causal(do, q, k, v, full_o, full_l, q_doc, q_pos, k_doc, k_pos, 0.5)
    ga = orc.bwd_doc_causal(do, q, k[a], v[a], mo, ml, q_doc, q_pos, k_doc[a], k_pos[a], 0.5)
    gb = orc.bwd_doc_causal(do, q, k[b], v[b], mo, ml, q_doc, q_pos, k_doc[b], k_pos[b], 0.5)
    np.testing.assert_allclose(ga[0] + gb[0], gf[0], atol=1e-12)
    np.testing.assert_allclose(np.concatenate([ga[1], gb[1]]), gf[1], atol=1e-12)
    np.testing.assert_allclose(np.concatenate([ga[2], gb[2]]), gf[2], atol=1e-12)


def test_doc_causal_matches_brute_force():
    rng = np.random.default_rng(11)
    ids = np.array([1, 1, 1, 2, 2, 3, 3, 3, 3, 0, 0])
    S = len(ids)
    q_pos = np.arange(4, S)
    q, k, v = _rand(rng, len(q_pos), 1, 2), _rand(rng, S, 1, 2), _rand(rng, S, 1, 2)
    out, lse = orc.fwd_doc_causal(q, k, v, ids[q_pos], q_pos, ids, np.arange(S), 1.1)
    for r, p in enumerate(q_pos):
        keys = [j for j in range(S) if ids[j] == ids[p] and ids[p] > 0 and j <= p]
        if not keys:
            assert lse[0, r] == -np.inf and np.all(out[r] == 0)
            continue
        w = [math.exp(1.1 * (q[r, 0] @ k[j, 0])) for j in keys]
        assert abs(lse[0, r] - math.log(sum(w))) < 1e-12
        np.testing.assert_allclose(out[r, 0], sum(wj * v[j, 0] for wj, j in zip(w, keys)) / sum(w),
                                   atol=1e-12)


def test_sampled_rows_and_columns_match_full():
    rng = np.random.default_rng(12)
    cu_q = np.array([0, 0, 6, 9, 17])
    cu_k = np.array([0, 4, 10, 10, 21])
    Hq, Hkv, D = 4, 2, 3
    q, k, v, do = _rand(rng, 17, Hq, D), _rand(rng, 21, Hkv, D), _rand(rng, 21, Hkv, D), _rand(rng, 17, Hq, D)
    for causal in (True, False):
        o, l = orc.fwd_varlen(q, k, v, cu_q, cu_k, 0.6, causal)
        dq, dk, dv = orc.bwd_varlen(do, q, k, v, o, l, cu_q, cu_k, 0.6, causal)
        toks = np.array([0, 5, 6, 8, 9, 16])
        heads = np.array([0, 3, 1, 2, 0, 3])
        ro, rl = orc.fwd_varlen_rows(q, k, v, cu_q, cu_k, 0.6, causal, toks, heads)
        np.testing.assert_allclose(ro, o[toks, heads], atol=1e-13)
        np.testing.assert_allclose(rl, l[heads, toks], atol=1e-13)
        rq = orc.bwd_varlen_rows(do, q, k, v, o, l, cu_q, cu_k, 0.6, causal, toks, heads)
        np.testing.assert_allclose(rq, dq[toks, heads], atol=1e-12)
        kt = np.array([0, 3, 4, 10, 15, 20])
        kh = np.array([1, 0, 1, 0, 1, 0])
        rk, rv = orc.bwd_varlen_cols(do, q, k, v, o, l, cu_q, cu_k, 0.6, causal, kt, kh)
        np.testing.assert_allclose(rk, dk[kt, kh], atol=1e-12)
        np.testing.assert_allclose(rv, dv[kt, kh], atol=1e-12)


def test_doc_causal_gqa_equals_mha_on_repeated_kv():
    """GQA in the document-causal functions ("ffpa_attention" page: the forward
    handles GQA, the backward reduces dK/dV to the Hkv heads): with Hq = 4 and
    Hkv = 2, q-head h reads kv-head h // 2, so the result must equal the same
    call on K/V whose heads are repeated (Hkv = Hq, one q-head per kv-head),
    with dk/dv summed over each group of two. The equivalent hand-written
    segments through the varlen functions must give the same numbers."""
    rng = np.random.default_rng(13)
    Hq, Hkv, D, Dv = 4, 2, 3, 2
    # keys: positions 0..11; queries: the shard 5..11 (earlier keys are a
    # second chunk for the later queries of document 2)
    ids = np.array([1, 1, 2, 2, 2, 2, 2, 3, 3, 3, 0, 0])
    k_pos, q_pos = np.arange(12), np.arange(5, 12)
    q, do = _rand(rng, 7, Hq, D), _rand(rng, 7, Hq, Dv)
    k, v = _rand(rng, 12, Hkv, D), _rand(rng, 12, Hkv, Dv)
    kr, vr = np.repeat(k, Hq // Hkv, axis=1), np.repeat(v, Hq // Hkv, axis=1)
    args = (ids[q_pos], q_pos, ids, k_pos, 0.7)
    o, l = orc.fwd_doc_causal(q, k, v, *args)
    orr, lr = orc.fwd_doc_causal(q, kr, vr, *args)
    np.testing.assert_allclose(o, orr, atol=1e-13)
    np.testing.assert_array_equal(l, lr)
    # heads of one group read the same keys but differ through q: the two
    # q-heads of kv-head 0 must not coincide (guards against a collapsed map)
    assert np.abs(o[:, 0] - o[:, 1]).max() > 1e-3
    dq, dk, dv = orc.bwd_doc_causal(do, q, k, v, o, l, *args)
    dqr, dkr, dvr = orc.bwd_doc_causal(do, q, kr, vr, orr, lr, *args)
    np.testing.assert_allclose(dq, dqr, atol=1e-12)
    np.testing.assert_allclose(dk, dkr.reshape(12, Hkv, Hq // Hkv, D).sum(axis=2), atol=1e-12)
    np.testing.assert_allclose(dv, dvr.reshape(12, Hkv, Hq // Hkv, Dv).sum(axis=2), atol=1e-12)
    # the same problem as varlen segments, written out by hand: doc 2 has its
    # queries 5, 6 against keys 2..6 (bottom-right causal), doc 3 queries 7..9
    # against keys 7..9, the padding queries 10, 11 against nothing; doc 1 is
    # keys only. Query rows of the shard are 0..6, keys 0..11 in order.
    cu_q = [0, 0, 2, 5, 7, 7]
    cu_k = [0, 2, 7, 10, 10, 12]
    ov, lv = orc.fwd_varlen(q, k, v, cu_q, cu_k, 0.7, True)
    np.testing.assert_allclose(ov, o, atol=1e-13)
    np.testing.assert_array_equal(np.isinf(lv), np.isinf(l))
    np.testing.assert_allclose(lv[np.isfinite(lv)], l[np.isfinite(l)], atol=1e-13)
    gv = orc.bwd_varlen(do, q, k, v, o, l, cu_q, cu_k, 0.7, True)
    for a, b in zip(gv, (dq, dk, dv)):
        np.testing.assert_allclose(a, b, atol=1e-12)


def test_ring_gather_scatter_and_row_merge():
    """The packed ring layout's row moves and live-row merge ("gemma4_moe
    cp_attention" page): gather then scatter restores the named rows and
    fills the rest; merging one chunk at its rows equals the full merge of
    the dense accumulators with a chunk that is -inf (absent) elsewhere."""
    rng = np.random.default_rng(14)
    B, H, S, D = 2, 3, 5, 4
    x = rng.standard_normal((B, H, S, D))
    idx = np.array([7, 0, 3, 9, 5])  # b*S + s, in any order
    g = orc.ring_gather(x, idx)
    assert g.shape == (5, H, D)
    for t, f in enumerate(idx):
        np.testing.assert_array_equal(g[t], x[f // S, :, f % S])
    back = orc.ring_scatter(g, idx, B, S)
    for f in range(B * S):
        want = x[f // S, :, f % S] if f in idx else 0.0
        np.testing.assert_array_equal(back[f // S, :, f % S], want)
    acc = rng.standard_normal((B, H, S, D))
    lacc = rng.standard_normal((B, H, S))
    lacc[0, 1, 3] = -np.inf  # a live row nothing covered yet (flat 3)
    ob = rng.standard_normal((5, H, D))
    lb = rng.standard_normal((H, 5))
    lb[2, 1] = -np.inf
    mo, ml = orc.ring_merge_rows(acc, lacc, ob, lb, idx)
    dense_b = orc.ring_scatter(ob, idx, B, S)
    dense_lb = orc.ring_scatter(lb.T[:, :, None], idx, B, S, fill=-np.inf)[..., 0]
    flat = lambda a: a.transpose(0, 2, 1, 3).reshape(B * S, H, D)  # noqa: E731
    fo, fl = orc.merge(flat(acc), lacc.transpose(0, 2, 1).reshape(B * S, H).T, flat(dense_b),
                       dense_lb.transpose(0, 2, 1).reshape(B * S, H).T)
    np.testing.assert_allclose(flat(mo), fo, atol=1e-13)
    np.testing.assert_allclose(ml.transpose(0, 2, 1).reshape(B * S, H).T, fl, atol=1e-13)
    # rows no index names are untouched
    untouched = [f for f in range(B * S) if f not in idx]
    for f in untouched:
        np.testing.assert_array_equal(mo[f // S, :, f % S], acc[f // S, :, f % S])


# ---------------------------------------------------------------- window, softcap
@pytest.mark.parametrize("lq,lk,W", [(9, 9, 3), (5, 9, 4), (9, 5, 2), (7, 7, 1), (6, 6, 20)])
def test_left_window_counts_visible_keys(lq, lk, W):
    """A left window of W ("attention utils" page: a positive left window
    counts the visible keys, the current token included): with q = 0 every
    visible score is 0, so lse = ln(#visible) with #visible = the keys
    j <= i + lk - lq that are also among the last W of them, by brute force."""
    rng = np.random.default_rng(20 + W)
    k, v = _rand(rng, lk, 1, 3), _rand(rng, lk, 1, 2)
    q = np.zeros((lq, 1, 3))
    o, l = orc.fwd_varlen(q, k, v, [0, lq], [0, lk], 0.5, True, window=W)
    for i in range(lq):
        top = i + lk - lq  # last visible key
        seen = [j for j in range(lk) if j <= top and j >= top - W + 1]
        if not seen:
            assert l[0, i] == -np.inf and np.all(o[i] == 0)
            continue
        assert abs(l[0, i] - math.log(len(seen))) < 1e-12
        np.testing.assert_allclose(o[i, 0], v[seen, 0].mean(axis=0), atol=1e-12)


def test_window_of_one_sees_only_the_diagonal_key():
    rng = np.random.default_rng(21)
    q, k, v = _rand(rng, 6, 2, 4), _rand(rng, 6, 2, 4), _rand(rng, 6, 2, 3)
    o, l = orc.fwd_varlen(q, k, v, [0, 6], [0, 6], 0.7, True, window=1)
    np.testing.assert_allclose(o, v, atol=1e-12)
    np.testing.assert_allclose(l, 0.7 * np.einsum("thd,thd->ht", q, k), atol=1e-12)
    # a window covering the whole segment is plain causal attention
    o2, l2 = orc.fwd_varlen(q, k, v, [0, 6], [0, 6], 0.7, True, window=6)
    o3, l3 = orc.fwd_varlen(q, k, v, [0, 6], [0, 6], 0.7, True)
    np.testing.assert_allclose(o2, o3, atol=1e-13)
    np.testing.assert_allclose(l2, l3, atol=1e-13)
    with pytest.raises(ValueError):
        orc.fwd_varlen(q, k, v, [0, 6], [0, 6], 0.7, False, window=2)


def test_softcap_bounds_scores_and_matches_brute_force():
    """Soft-capped scores cap * tanh(s / cap): brute force on single rows,
    identical keys still give the mean of V, and a huge cap changes nothing."""
    rng = np.random.default_rng(22)
    q, k, v = 3 * _rand(rng, 5, 1, 4), 3 * _rand(rng, 7, 1, 4), _rand(rng, 7, 1, 2)
    cap = 2.5
    o, l = orc.fwd_varlen(q, k, v, [0, 5], [0, 7], 0.9, True, softcap=cap)
    for i in range(5):
        keys = [j for j in range(7) if j <= i + 2]
        sc = [cap * math.tanh(0.9 * float(q[i, 0] @ k[j, 0]) / cap) for j in keys]
        assert all(abs(x) <= cap for x in sc)
        w = [math.exp(x) for x in sc]
        assert abs(l[0, i] - math.log(sum(w))) < 1e-12
        np.testing.assert_allclose(o[i, 0], sum(wj * v[j, 0] for wj, j in zip(w, keys)) / sum(w),
                                   atol=1e-12)
    kk = np.repeat(k[:1], 7, axis=0)
    o, _ = orc.fwd_varlen(q, kk, v, [0, 5], [0, 7], 0.9, True, softcap=cap)
    for i in range(5):
        np.testing.assert_allclose(o[i, 0], v[: i + 3, 0].mean(axis=0), atol=1e-12)
    o1, l1 = orc.fwd_varlen(q, k, v, [0, 5], [0, 7], 0.9, True, softcap=1e9)
    o0, l0 = orc.fwd_varlen(q, k, v, [0, 5], [0, 7], 0.9, True)
    np.testing.assert_allclose(o1, o0, atol=1e-9)
    np.testing.assert_allclose(l1, l0, atol=1e-9)


@pytest.mark.parametrize("window,softcap", [(3, None), (None, 1.7), (4, 2.2)])
def test_window_softcap_backward_matches_finite_differences(window, softcap):
    """Gradients of sum(dO * out) with a left window and / or a softcap: the
    backward from the oracle's own out/lse against central differences."""
    rng = np.random.default_rng(23)
    T, H, D = 7, 1, 3
    q, k, v, do = (_rand(rng, T, H, D) for _ in range(4))
    cu = [0, 3, 7]
    kw = dict(window=window, softcap=softcap)
    o, l = orc.fwd_varlen(q, k, v, cu, cu, 0.8, True, **kw)
    dq, dk, dv = orc.bwd_varlen(do, q, k, v, o, l, cu, cu, 0.8, True, **kw)

    def f(qq, kk, vv):
        return float((do * orc.fwd_varlen(qq, kk, vv, cu, cu, 0.8, True, **kw)[0]).sum())

    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": q, "k": k, "v": v}
            args_m = {"q": q, "k": k, "v": v}
            args_p[name], args_m[name] = xp, xm
            num[idx] = (f(**{a[0] + a[0]: b for a, b in args_p.items()}) -
                        f(**{a[0] + a[0]: b for a, b in args_m.items()})) / (2 * eps)
        assert np.abs(num - g).max() <= 1e-6 * max(1.0, np.abs(g).max()), name
