"""fp64 CPU oracle for fused scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or run
this module; only the tests, the smoke check and the benchmark's CPU-baseline
leg do. It shares no code with the HIP library.

Every function is the plain definition written out in numpy float64. Inputs
are bf16 values upcast losslessly. Sources (NVIDIA NeMo-Automodel API pages):

* "ffpa_attention" page, API entries for the dense and varlen forward and
  backward wrappers: out has the query rows and the value head dim, lse is
  fp32 with shape [B, Hq, Nq] (dense) or [Hq, T] (varlen), GQA is handled
  inside the forward, the backward takes the caller's out/lse and returns
  dK/dV reduced to the Hkv heads.
* "fa4" page, module overview of document-causal attention: the causal mask
  sits at the bottom-right corner of every segment, i.e. a query at global
  position p sees the keys of its document up to p; zero-query segments tile
  the keys; padding queries return zero.
* "gemma4_moe cp_attention" page, the -inf-safe online-softmax merge entry:
  lse combines as logaddexp, out as the weighted mean of the two chunk outputs,
  and a row where both chunks are -inf keeps 0.

Readings where the pages are silent (each also listed with the design notes):
* lse is the natural log of the sum of exp over the *scaled* scores.
* a row with no visible key has out = 0 and lse = -inf; the backward treats
  lse = -inf as P = 0, so such a row has dq = 0 and adds nothing to dk/dv.
* GQA maps q-head h to kv-head h // (Hq / Hkv) (contiguous groups).
* causal alignment is bottom-right in every segment, dense inputs included.

Parity status: every public function here is pinned by tests/test_oracle.py
(closed forms, hand-worked fixtures, brute force, finite differences and a
library cross-check); none is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

NEG_INF = -np.inf
_ROW_BLOCK = 1024  # rows per score block, only to bound memory


def f64(x) -> np.ndarray:
    """Upcast a tensor or array (bf16 / fp32 / fp64) to a float64 numpy array."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        import torch  # local: only tensors need it

        x = x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------------------
# visibility
# ---------------------------------------------------------------------------
def causal_visible(lq: int, lk: int, rows=None, cols=None, window=None) -> np.ndarray:
    """Bottom-right causal visibility of one segment ("fa4" page, document-causal
    bullets): query i sees key j iff j <= i + (lk - lq). A left window W > 0
    ("attention utils" page, backend metadata: a positive left window counts
    the visible keys, the current token included) also requires
    j > i + (lk - lq) - W; None or W <= 0 means unbounded."""
    i = np.arange(lq) if rows is None else np.asarray(rows)
    j = np.arange(lk) if cols is None else np.asarray(cols)
    vis = j[None, :] <= i[:, None] + (lk - lq)
    if window is not None and window > 0:
        vis = vis & (j[None, :] > i[:, None] + (lk - lq) - window)
    return vis


def segment_visible(lq: int, lk: int, causal: bool, rows=None, cols=None,
                    window=None) -> np.ndarray:
    if causal:
        return causal_visible(lq, lk, rows, cols, window)
    if window is not None and window > 0:
        raise ValueError("a left window applies to causal attention only")
    m = lq if rows is None else len(rows)
    n = lk if cols is None else len(cols)
    return np.ones((m, n), dtype=bool)


def doc_causal_visible(q_doc, q_pos, k_doc, k_pos) -> np.ndarray:
    """Document-causal rule ("fa4" page overview): a query at global position p
    sees a key at j iff both carry the same document id > 0 and j <= p."""
    q_doc = np.asarray(q_doc)
    k_doc = np.asarray(k_doc)
    same = (q_doc[:, None] == k_doc[None, :]) & (q_doc[:, None] > 0)
    return same & (np.asarray(k_pos)[None, :] <= np.asarray(q_pos)[:, None])


# ---------------------------------------------------------------------------
# one head, one segment: the definitions
# ---------------------------------------------------------------------------
def capped(s, softcap):
    """Logit soft-capping of the scaled scores ("ffpa_attention" page: the
    softcap argument of the attention forward): cap * tanh(s / cap); None or
    0 leaves s unchanged."""
    if not softcap:
        return s
    return softcap * np.tanh(s / softcap)


def attend(q, k, v, vis, scale: float, softcap=None):
    """Softmax attention of rows q [m, Dqk] over keys k [n, Dqk] / values v [n, Dv]
    restricted to vis [m, n]. Returns (out [m, Dv], lse [m]).

    S = scale * q k^T (soft-capped when softcap is set); lse = log
    sum_{visible} exp(S); P = exp(S - lse) on visible entries; out = P v. Rows
    with nothing visible: out 0, lse -inf.
    """
    m = q.shape[0]
    out = np.zeros((m, v.shape[1]))
    lse = np.full(m, NEG_INF)
    for r0 in range(0, m, _ROW_BLOCK):
        r1 = min(m, r0 + _ROW_BLOCK)
        s = scale * (q[r0:r1] @ k.T)
        s = capped(s, softcap)
        s = np.where(vis[r0:r1], s, NEG_INF)
        live = vis[r0:r1].any(axis=1)
        mx = np.where(live, s.max(axis=1, initial=NEG_INF), 0.0)
        e = np.exp(s - mx[:, None])  # exp(-inf) = 0 on hidden entries
        tot = e.sum(axis=1)
        lse[r0:r1] = np.where(live, mx + np.log(np.where(live, tot, 1.0)), NEG_INF)
        p = e / np.where(live, tot, 1.0)[:, None]
        out[r0:r1] = p @ v
    return out, lse


def attend_backward(do, q, k, v, o, lse, vis, scale: float, softcap=None):
    """Gradients of sum(do * out) for one head and segment, recomputed from the
    caller-supplied o and lse ("ffpa_attention" page, backward entries).

    delta = rowsum(do * o); P = exp(S - lse) on visible entries (0 where lse is
    -inf); dV = P^T do; dP = do v^T; dS = P * (dP - delta);
    dQ = scale dS k; dK = scale dS^T q. With a softcap, S = cap tanh(X / cap)
    of the scaled scores X and dS carries the chain-rule factor
    dS/dX = 1 - tanh(X / cap)^2.

    With a subset of keys this still gives exact dK/dV for those keys (P uses
    the supplied lse, not a renormalised one); dQ is then the subset's part.
    """
    delta = (do * o).sum(axis=1)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros((k.shape[0], v.shape[1]))
    live = np.isfinite(lse)
    for r0 in range(0, q.shape[0], _ROW_BLOCK):
        r1 = min(q.shape[0], r0 + _ROW_BLOCK)
        x = scale * (q[r0:r1] @ k.T)
        s = capped(x, softcap)
        use = vis[r0:r1] & live[r0:r1, None]
        ref = np.where(live[r0:r1], lse[r0:r1], 0.0)
        p = np.exp(np.where(use, s - ref[:, None], NEG_INF))  # 0 where hidden or lse = -inf
        dv += p.T @ do[r0:r1]
        dp = do[r0:r1] @ v.T
        ds = p * (dp - delta[r0:r1, None])
        if softcap:
            ds = ds * (1.0 - np.tanh(x / softcap) ** 2)
        dq[r0:r1] = scale * (ds @ k)
        dk += scale * (ds.T @ q[r0:r1])
    return dq, dk, dv


# ---------------------------------------------------------------------------
# packed varlen THD: q [Tq, Hq, Dqk], k [Tk, Hkv, Dqk], v [Tk, Hkv, Dv]
# ---------------------------------------------------------------------------
def _segments(cu_q, cu_k):
    cu_q = np.asarray(cu_q, dtype=np.int64)
    cu_k = np.asarray(cu_k, dtype=np.int64)
    assert cu_q.shape == cu_k.shape
    return [(int(cu_q[s]), int(cu_q[s + 1]), int(cu_k[s]), int(cu_k[s + 1]))
            for s in range(len(cu_q) - 1)]


def fwd_varlen(q, k, v, cu_q, cu_k, scale: float, causal: bool, window=None, softcap=None):
    """Varlen forward ("ffpa_attention" page, varlen forward entry): returns
    out [Tq, Hq, Dv] and lse [Hq, Tq]; segment s pairs queries cu_q[s]:cu_q[s+1]
    with keys cu_k[s]:cu_k[s+1]."""
    q, k, v = f64(q), f64(k), f64(v)
    Tq, Hq, _ = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    out = np.zeros((Tq, Hq, v.shape[2]))
    lse = np.full((Hq, Tq), NEG_INF)
    for qa, qb, ka, kb in _segments(cu_q, cu_k):
        if qb == qa:
            continue
        vis = segment_visible(qb - qa, kb - ka, causal, window=window)
        for h in range(Hq):
            g = h // G
            o, l = attend(q[qa:qb, h], k[ka:kb, g], v[ka:kb, g], vis, scale, softcap)
            out[qa:qb, h] = o
            lse[h, qa:qb] = l
    return out, lse


def bwd_varlen(do, q, k, v, o, lse, cu_q, cu_k, scale: float, causal: bool, window=None,
               softcap=None):
    """Varlen backward from caller out/lse; dk/dv summed over each GQA group."""
    do, q, k, v, o, lse = f64(do), f64(q), f64(k), f64(v), f64(o), f64(lse)
    Hq = q.shape[1]
    Hkv = k.shape[1]
    G = Hq // Hkv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for qa, qb, ka, kb in _segments(cu_q, cu_k):
        if qb == qa or kb == ka:
            continue
        vis = segment_visible(qb - qa, kb - ka, causal, window=window)
        for h in range(Hq):
            g = h // G
            a, b, c = attend_backward(do[qa:qb, h], q[qa:qb, h], k[ka:kb, g], v[ka:kb, g],
                                      o[qa:qb, h], lse[h, qa:qb], vis, scale, softcap)
            dq[qa:qb, h] = a
            dk[ka:kb, g] += b
            dv[ka:kb, g] += c
    return dq, dk, dv


# ---------------------------------------------------------------------------
# dense SDPA layout: q [B, Hq, Nq, Dqk], k [B, Hkv, Nk, Dqk], v [B, Hkv, Nk, Dv]
# ---------------------------------------------------------------------------
def fwd_dense(q, k, v, scale: float, causal: bool, window=None, softcap=None):
    """Dense forward ("ffpa_attention" page, dense forward entry): returns
    out [B, Hq, Nq, Dv] and lse [B, Hq, Nq]."""
    q, k, v = f64(q), f64(k), f64(v)
    B, Hq, Nq, _ = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    out = np.zeros((B, Hq, Nq, v.shape[3]))
    lse = np.full((B, Hq, Nq), NEG_INF)
    vis = segment_visible(Nq, Nk, causal, window=window)
    for b in range(B):
        for h in range(Hq):
            o, l = attend(q[b, h], k[b, h // G], v[b, h // G], vis, scale, softcap)
            out[b, h] = o
            lse[b, h] = l
    return out, lse


def bwd_dense(do, q, k, v, o, lse, scale: float, causal: bool, window=None, softcap=None):
    """Dense backward ("ffpa_attention" page, dense backward entry): dq, dk, dv in
    [B, H, N, D] with dk/dv reduced to Hkv."""
    do, q, k, v, o, lse = f64(do), f64(q), f64(k), f64(v), f64(o), f64(lse)
    B, Hq, Nq, _ = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    vis = segment_visible(Nq, Nk, causal, window=window)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            a, c, d = attend_backward(do[b, h], q[b, h], k[b, g], v[b, g], o[b, h], lse[b, h],
                                      vis, scale, softcap)
            dq[b, h] = a
            dk[b, g] += c
            dv[b, g] += d
    return dq, dk, dv


# ---------------------------------------------------------------------------
# sampled rows / key columns (for sizes where full attention is too slow)
# ---------------------------------------------------------------------------
def _locate(cu, t):
    """Segment holding token t: the last s with cu[s] <= t. Empty segments that
    start at t come before the one that holds it, so they are never chosen."""
    return int(np.searchsorted(np.asarray(cu, dtype=np.int64), t, side="right")) - 1


def fwd_varlen_rows(q, k, v, cu_q, cu_k, scale, causal, tokens, heads, window=None,
                    softcap=None):
    """out [n, Dv] and lse [n] of the listed (token, q-head) rows of the varlen forward."""
    cu_q = np.asarray(cu_q, dtype=np.int64)
    cu_k = np.asarray(cu_k, dtype=np.int64)
    Hq, Hkv = q.shape[1], k.shape[1]
    G = Hq // Hkv
    outs, lses = [], []
    for t, h in zip(tokens, heads):
        t, h = int(t), int(h)
        s = _locate(cu_q, t)
        qa, qb, ka, kb = int(cu_q[s]), int(cu_q[s + 1]), int(cu_k[s]), int(cu_k[s + 1])
        vis = segment_visible(qb - qa, kb - ka, causal, rows=[t - qa], window=window)
        qq = f64(q[t, h])[None, :]
        o, l = attend(qq, f64(k[ka:kb, h // G]), f64(v[ka:kb, h // G]), vis, scale, softcap)
        outs.append(o[0])
        lses.append(l[0])
    return np.array(outs), np.array(lses)


def bwd_varlen_rows(do, q, k, v, o, lse, cu_q, cu_k, scale, causal, tokens, heads, window=None,
                    softcap=None):
    """dq [n, Dqk] of the listed (token, q-head) rows, from caller out/lse [Hq, Tq]."""
    cu_q = np.asarray(cu_q, dtype=np.int64)
    cu_k = np.asarray(cu_k, dtype=np.int64)
    Hq, Hkv = q.shape[1], k.shape[1]
    G = Hq // Hkv
    res = []
    for t, h in zip(tokens, heads):
        t, h = int(t), int(h)
        s = _locate(cu_q, t)
        qa, qb, ka, kb = int(cu_q[s]), int(cu_q[s + 1]), int(cu_k[s]), int(cu_k[s + 1])
        vis = segment_visible(qb - qa, kb - ka, causal, rows=[t - qa], window=window)
        g = h // G
        a, _, _ = attend_backward(f64(do[t, h])[None], f64(q[t, h])[None], f64(k[ka:kb, g]),
                                  f64(v[ka:kb, g]), f64(o[t, h])[None],
                                  np.array([float(lse[h, t])]), vis, scale, softcap)
        res.append(a[0])
    return np.array(res)


def bwd_varlen_cols(do, q, k, v, o, lse, cu_q, cu_k, scale, causal, tokens, kv_heads,
                    window=None, softcap=None):
    """dk [n, Dqk], dv [n, Dv] of the listed (key token, kv-head) rows, summed over
    the q-heads of the group and over every query that sees the key."""
    cu_q = np.asarray(cu_q, dtype=np.int64)
    cu_k = np.asarray(cu_k, dtype=np.int64)
    Hq, Hkv = q.shape[1], k.shape[1]
    G = Hq // Hkv
    dks, dvs = [], []
    for t, g in zip(tokens, kv_heads):
        t, g = int(t), int(g)
        s = _locate(cu_k, t)
        qa, qb, ka, kb = int(cu_q[s]), int(cu_q[s + 1]), int(cu_k[s]), int(cu_k[s + 1])
        dk = np.zeros(k.shape[2])
        dv = np.zeros(v.shape[2])
        if qb > qa:
            vis = segment_visible(qb - qa, kb - ka, causal, cols=[t - ka], window=window)
            kk = f64(k[t, g])[None]
            vv = f64(v[t, g])[None]
            for h in range(g * G, (g + 1) * G):
                _, b, c = attend_backward(f64(do[qa:qb, h]), f64(q[qa:qb, h]), kk, vv,
                                          f64(o[qa:qb, h]), f64(lse[h, qa:qb]), vis, scale, softcap)
                dk += b[0]
                dv += c[0]
        dks.append(dk)
        dvs.append(dv)
    return np.array(dks), np.array(dvs)


# ---------------------------------------------------------------------------
# document-causal attention on explicit document ids, and the chunk merge
# ---------------------------------------------------------------------------
def fwd_doc_causal(q, k, v, q_doc, q_pos, k_doc, k_pos, scale):
    """Attention of packed queries q [Tq, Hq, Dqk] over keys k [Tk, Hkv, Dqk] under
    the document-causal rule on explicit ids and global positions. Needs no
    segment list, so it checks any segment builder independently."""
    q, k, v = f64(q), f64(k), f64(v)
    Tq, Hq, _ = q.shape
    G = Hq // k.shape[1]
    vis = doc_causal_visible(q_doc, q_pos, k_doc, k_pos)
    out = np.zeros((Tq, Hq, v.shape[2]))
    lse = np.full((Hq, Tq), NEG_INF)
    for h in range(Hq):
        o, l = attend(q[:, h], k[:, h // G], v[:, h // G], vis, scale)
        out[:, h] = o
        lse[h] = l
    return out, lse


def bwd_doc_causal(do, q, k, v, o, lse, q_doc, q_pos, k_doc, k_pos, scale):
    """Backward of fwd_doc_causal from caller out [Tq, Hq, Dv] / lse [Hq, Tq]."""
    do, q, k, v, o, lse = f64(do), f64(q), f64(k), f64(v), f64(o), f64(lse)
    Hq = q.shape[1]
    G = Hq // k.shape[1]
    vis = doc_causal_visible(q_doc, q_pos, k_doc, k_pos)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for h in range(Hq):
        a, b, c = attend_backward(do[:, h], q[:, h], k[:, h // G], v[:, h // G], o[:, h],
                                  lse[h], vis, scale)
        dq[:, h] = a
        dk[:, h // G] += b
        dv[:, h // G] += c
    return dq, dk, dv


def merge(out_a, lse_a, out_b, lse_b):
    """Combine two chunk results of the same query rows ("gemma4_moe cp_attention"
    page, -inf-safe merge entry). out_* [rows, H, Dv], lse_* [H, rows].

    lse = log(e^lse_a + e^lse_b); out = (e^lse_a out_a + e^lse_b out_b) / e^lse.
    A row where both lse are -inf keeps out 0 and lse -inf.
    """
    out_a, lse_a, out_b, lse_b = f64(out_a), f64(lse_a), f64(out_b), f64(lse_b)
    lse = np.logaddexp(lse_a, lse_b)
    live = np.isfinite(lse)
    safe = np.where(live, lse, 0.0)
    wa = np.where(live, np.exp(lse_a - safe), 0.0)  # [H, rows]
    wb = np.where(live, np.exp(lse_b - safe), 0.0)
    out = wa.T[:, :, None] * out_a + wb.T[:, :, None] * out_b
    return out, np.where(live, lse, NEG_INF)


# ---------------------------------------------------------------------------
# packed ring layout ("gemma4_moe cp_attention" page: rows gathered at flat
# indices b*S + pos, scattered back, and one chunk merged in place at its live
# rows only)
# ---------------------------------------------------------------------------
def ring_gather(x, flat_index):
    """[B, H, S, D] -> [T, H, D]: row t is x[b, :, s] for flat_index[t] = b*S + s."""
    x = f64(x)
    B, H, S, D = x.shape
    idx = np.asarray(flat_index, dtype=np.int64)
    return x.transpose(0, 2, 1, 3).reshape(B * S, H, D)[idx]


def ring_scatter(xp, flat_index, B, S, fill=0.0):
    """[T, H, D] -> [B, H, S, D]: the inverse of ring_gather, `fill` on rows no
    index names."""
    xp = f64(xp)
    T, H, D = xp.shape
    out = np.full((B * S, H, D), fill)
    out[np.asarray(flat_index, dtype=np.int64)] = xp
    return out.reshape(B, S, H, D).transpose(0, 2, 1, 3)


def ring_merge_rows(out_acc, lse_acc, out_b, lse_b, flat_index):
    """Running accumulators out_acc [B, H, S, D] / lse_acc [B, H, S] after
    merging one chunk's packed rows (out_b [T, H, D], lse_b [H, T]) at its
    flat-index rows with the -inf-safe merge; other rows unchanged."""
    out_acc, lse_acc = f64(out_acc).copy(), f64(lse_acc).copy()
    B, H, S, D = out_acc.shape
    idx = np.asarray(flat_index, dtype=np.int64)
    flat_o = out_acc.transpose(0, 2, 1, 3).reshape(B * S, H, D)
    flat_l = lse_acc.transpose(0, 2, 1).reshape(B * S, H)
    mo, ml = merge(flat_o[idx], flat_l[idx].T, out_b, lse_b)
    flat_o[idx] = mo
    flat_l[idx] = ml.T
    return (flat_o.reshape(B, S, H, D).transpose(0, 2, 1, 3),
            flat_l.reshape(B, S, H).transpose(0, 2, 1))
