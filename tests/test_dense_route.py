"""Dense routing of ring chunks ("gemma4_moe cp_attention" page: the
dense-routing flags of the packed ring segments, the per-chunk dense
eligibility entry and the two single-document row predicates).

Host logic only (no GPU): the library's attn_dense_route against a plain
reading of the row predicates, and a semantic pin through the oracle: on
every chunk the library calls eligible, dense attention over the raw rows
(causal for the local chunk, non-causal for the cross chunk) with its padding
queries zeroed equals the document-causal rule on ids and positions.
"""
import zlib

import numpy as np
import pytest
import torch

from oracle import attention as orc

vca = pytest.importorskip("varlen_causal_attention_amd")


def single_doc_with_pad_suffix(row):
    """Row predicate of the "gemma4_moe cp_attention" page's single-document
    check with a pad tail: the ids > 0 form one run that starts at position 0
    and carries one id; any zeros come after that run. A row of zeros passes."""
    real = row[row > 0]
    if real.size == 0:
        return True
    n = real.size
    return bool(np.all(row[:n] == real[0]) and np.all(row[n:] == 0))


def exactly_one_doc(row):
    """Every position carries the same document id > 0 (no padding)."""
    return row.size > 0 and row[0] > 0 and bool(np.all(row == row[0]))


def reference_route(ids, q_start, q_len, k_start, k_len, mode):
    q_end, k_end = q_start + q_len, k_start + k_len
    ok = True
    if mode == 0:
        ok = k_end == q_end
        for row in ids:
            ok = ok and single_doc_with_pad_suffix(row[k_start:k_end])
    else:
        for row in ids:
            kr, qr = row[k_start:k_end], row[q_start:q_end]
            ok = ok and exactly_one_doc(kr) and single_doc_with_pad_suffix(qr)
            real = qr[qr > 0]
            ok = ok and (real.size == 0 or (kr.size > 0 and real[0] == kr[0]))
    return ok, ids[:, q_start:q_end] == 0


def random_rows(rng, B, S, kind):
    rows = np.zeros((B, S), dtype=np.int32)
    for b in range(B):
        if kind == "single":
            rows[b] = 1 + b
        elif kind == "pad_suffix":
            n = int(rng.integers(0, S + 1))
            rows[b, :n] = 3 + b
        elif kind == "two_docs":
            cut = int(rng.integers(1, S))
            rows[b, :cut] = 1
            rows[b, cut:] = 2
        elif kind == "pad_middle":
            rows[b] = 5
            a = int(rng.integers(1, S - 1))
            rows[b, a:a + 1] = 0
        else:  # random ids in few runs
            n_runs = int(rng.integers(1, 4))
            cuts = np.sort(rng.choice(np.arange(1, S), size=n_runs - 1, replace=False))
            vals = rng.integers(0, 3, size=n_runs)
            for v, a, e in zip(vals, np.r_[0, cuts], np.r_[cuts, S]):
                rows[b, a:e] = v
    return rows


CASES = [
    # (S, q_start, q_len, k_start, k_len, mode)
    (64, 32, 32, 32, 32, 0),   # ring local chunk: the rank's own shard
    (64, 32, 32, 0, 64, 0),    # keys start before the queries, end with them
    (64, 16, 16, 0, 48, 0),    # keys end past the queries: never dense
    (64, 32, 32, 0, 32, 1),    # ring cross chunk: an earlier shard
    (64, 40, 24, 8, 24, 1),
]


@pytest.mark.parametrize("kind", ["single", "pad_suffix", "two_docs", "pad_middle", "random"])
@pytest.mark.parametrize("case", CASES)
def test_route_matches_row_predicates(kind, case):
    S, qs, ql, ks, kl, mode = case
    rng = np.random.default_rng(zlib.crc32(repr((kind, case)).encode()))
    for _ in range(8):
        ids = random_rows(rng, 3, S, kind)
        if mode == 1 and kind == "pad_suffix":
            # a cross chunk's keys must be unpadded: pad only the query shard
            ids[:, :qs] = ids[:, qs:qs + 1].clip(min=1)
        ok, pad = vca.dense_route(ids, qs, ql, ks, kl, mode)
        rok, rpad = reference_route(ids, qs, ql, ks, kl, mode)
        assert ok == rok, (ids, case)
        assert np.array_equal(pad, rpad)


def test_route_examples():
    one = np.full((2, 64), 7, dtype=np.int32)
    assert vca.dense_route(one, 32, 32, 32, 32, 0)[0]
    assert vca.dense_route(one, 32, 32, 0, 32, 1)[0]
    padded = one.copy()
    padded[:, 50:] = 0
    ok, pad = vca.dense_route(padded, 32, 32, 32, 32, 0)
    assert ok and pad.sum() == 2 * 14 and pad[:, 18:].all()
    assert vca.dense_route(padded, 32, 32, 0, 32, 1)[0]      # queries padded, keys whole
    assert not vca.dense_route(padded, 16, 16, 0, 48, 0)[0]   # key range ends after the queries
    # a pad tail in the cross chunk's keys or a second document: not dense
    assert not vca.dense_route(padded, 56, 8, 32, 24, 1)[0]
    two = one.copy()
    two[1, 40:] = 8
    assert not vca.dense_route(two, 32, 32, 32, 32, 0)[0]
    assert not vca.dense_route(two, 32, 32, 0, 32, 1)[0]      # queries of doc 8 over keys of doc 7
    with pytest.raises(ValueError):
        vca.dense_route(one, 32, 32, 40, 24, 0)                # keys do not cover the queries
    with pytest.raises(ValueError):
        vca.dense_route(one, 16, 32, 0, 32, 1)                 # keys overlap the queries


@pytest.mark.parametrize("mode", [0, 1])
def test_dense_route_is_document_causal(mode):
    """Eligible chunks: dense attention over the raw rows (bottom-right
    causal for the local chunk, full for the cross chunk), padding queries
    zeroed, equals the document-causal rule on ids and positions."""
    rng = np.random.default_rng(90 + mode)
    B, S, H, D = 2, 48, 2, 16
    g = torch.Generator().manual_seed(91 + mode)
    qs, ql, ks, kl = (24, 24, 24, 24) if mode == 0 else (24, 24, 0, 24)
    checked = 0
    for trial in range(12):
        ids = np.zeros((B, S), dtype=np.int32)
        for b in range(B):
            doc = 1 + b + trial
            if mode == 0:
                n = int(rng.integers(0, S + 1))
                ids[b, :n] = doc
                # a different document earlier in the row stays outside the chunk
                ids[b, :ks] = np.where(ids[b, :ks] > 0, ids[b, :ks], doc + 50)
            else:
                ids[b, :qs] = doc
                n = int(rng.integers(0, ql + 1))
                ids[b, qs:qs + n] = doc
        ok, pad = vca.dense_route(ids, qs, ql, ks, kl, mode)
        if not ok:
            continue
        checked += 1
        q = torch.randn((B, H, ql, D), generator=g)
        k = torch.randn((B, H, kl, D), generator=g)
        v = torch.randn((B, H, kl, D), generator=g)
        out, lse = orc.fwd_dense(q, k, v, 0.25, causal=(mode == 0))
        out[np.repeat(pad[:, None, :], H, axis=1)] = 0.0
        lse[np.repeat(pad[:, None, :], H, axis=1)] = -np.inf
        for b in range(B):
            qpos, kpos = np.arange(qs, qs + ql), np.arange(ks, ks + kl)
            ro, rl = orc.fwd_doc_causal(q[b].transpose(0, 1), k[b].transpose(0, 1),
                                        v[b].transpose(0, 1), ids[b, qpos], qpos, ids[b, kpos],
                                        kpos, 0.25)
            assert np.allclose(out[b].transpose(1, 0, 2), ro, atol=1e-12)
            assert np.array_equal(np.isneginf(lse[b]), np.isneginf(rl))
            fin = np.isfinite(rl)
            assert np.allclose(lse[b][fin], rl[fin], atol=1e-12)
    assert checked >= 6
