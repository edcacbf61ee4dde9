"""Seeded synthetic inputs for the attention workloads.

This module only draws numbers and describes shapes: document-length splits,
document-id maps, bf16 tensors, and the visible-pair counts used to turn a
time into causal-adjusted FLOP/s. It holds none of the attention arithmetic,
so the fp64 oracle checks and the HIP path can both take their inputs from
here without sharing any computation.

Tensor recipe: ``g = torch.Generator().manual_seed(seed)``, then each tensor in
a fixed order is ``torch.randn(shape, generator=g, dtype=float32)`` rounded to
bfloat16 on the CPU (i.i.d. N(0,1) values, as the workloads state); the fp16
variants round the same draws to float16 instead.
Document lengths: ``rng = numpy.random.default_rng(seed)``; repeat
``L = min(rng.integers(lo, hi + 1), total - used)`` until ``total`` is covered,
so the last document is truncated to fit.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch


def doc_lengths(total: int, lo: int, hi: int, seed: int) -> list[int]:
    """Uniform document lengths in [lo, hi] covering ``total`` tokens."""
    rng = np.random.default_rng(seed)
    out: list[int] = []
    used = 0
    while used < total:
        n = min(int(rng.integers(lo, hi + 1)), total - used)
        out.append(n)
        used += n
    return out


def randn_bf16(shape, gen: torch.Generator, dtype=torch.bfloat16) -> torch.Tensor:
    """N(0,1) float32 draws rounded to bf16 (or to `dtype`, e.g. float16; CPU tensor)."""
    return torch.randn(shape, generator=gen, dtype=torch.float32).to(dtype)


def cumulative(lengths) -> np.ndarray:
    """int32 prefix offsets [0, l0, l0+l1, ...] (the cu_seqlens form)."""
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int32)


def causal_pairs(lq: int, lk: int) -> int:
    """Visible (query, key) pairs of a bottom-right aligned causal segment."""
    # query i sees keys 0 .. i + lk - lq, clipped to the lk keys that exist
    seen = np.arange(lq, dtype=np.int64) + (lk - lq + 1)
    return int(np.clip(seen, 0, lk).sum())


def segment_pairs(cu_q, cu_k, causal: bool) -> int:
    tot = 0
    for s in range(len(cu_q) - 1):
        lq = int(cu_q[s + 1] - cu_q[s])
        lk = int(cu_k[s + 1] - cu_k[s])
        tot += causal_pairs(lq, lk) if causal else lq * lk
    return tot


@dataclass
class Workload:
    """One attention problem: shapes, segment layout and seed."""

    name: str
    kind: str  # "dense" | "varlen" | "ring"
    seed: int
    Hq: int
    Hkv: int
    Dqk: int
    Dv: int
    causal: bool = True
    B: int = 1
    Nq: int = 0
    Nk: int = 0
    lengths: list = field(default_factory=list)  # varlen: document lengths (cu_q == cu_k)
    # ring (one rank of a two-rank ring): global row of 2*shard tokens
    shard: int = 0
    pad_tail: int = 0
    doc_lo: int = 0
    doc_hi: int = 0
    single_doc: bool = False  # ring: the row is one document (then the pad tail)
    route: str = "segments"   # ring: "segments" (cu_seqlens tiling the shard) or "gather"

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.Dqk)

    @property
    def T(self) -> int:
        return int(sum(self.lengths))

    def cu(self) -> np.ndarray:
        return cumulative(self.lengths)

    def pairs_per_head(self) -> int:
        if self.kind == "dense":
            per = causal_pairs(self.Nq, self.Nk) if self.causal else self.Nq * self.Nk
            return self.B * per
        if self.kind == "varlen":
            cu = self.cu()
            return segment_pairs(cu, cu, self.causal)
        ids = self.row_doc_ids()
        return ring_pairs(ids, self.shard)

    def pairs(self) -> int:
        return self.Hq * self.pairs_per_head()

    def fwd_flops(self) -> int:
        return 2 * self.pairs() * (self.Dqk + self.Dv)

    def bwd_flops(self) -> int:
        return 2 * self.pairs() * (3 * self.Dqk + 2 * self.Dv)

    # ---- ring workload: document ids of the global row -----------------
    def ring_docs(self) -> list[int]:
        if self.single_doc:
            return [2 * self.shard - self.pad_tail]
        return doc_lengths(2 * self.shard - self.pad_tail, self.doc_lo, self.doc_hi, self.seed)

    def row_doc_ids(self) -> np.ndarray:
        """[1, 2*shard] int32 document ids of the global row; 1-based, 0 = padding tail."""
        ids = np.zeros(2 * self.shard, dtype=np.int32)
        pos = 0
        for d, n in enumerate(self.ring_docs(), start=1):
            ids[pos:pos + n] = d
            pos += n
        return ids[None, :]

    # ---- tensors ---------------------------------------------------------
    def tensors(self, dtype=torch.bfloat16) -> dict:
        """CPU tensors (bf16, or `dtype`), drawn in a fixed order from the
        workload seed: the same float32 draws rounded to the element type."""
        g = torch.Generator().manual_seed(self.seed)

        def draw(shape, gen):
            return randn_bf16(shape, gen, dtype)

        if self.kind == "dense":
            q = draw((self.B, self.Hq, self.Nq, self.Dqk), g)
            k = draw((self.B, self.Hkv, self.Nk, self.Dqk), g)
            v = draw((self.B, self.Hkv, self.Nk, self.Dv), g)
            do = draw((self.B, self.Hq, self.Nq, self.Dv), g)
            return dict(q=q, k=k, v=v, do=do)
        if self.kind == "varlen":
            T = self.T
            q = draw((T, self.Hq, self.Dqk), g)
            k = draw((T, self.Hkv, self.Dqk), g)
            v = draw((T, self.Hkv, self.Dv), g)
            do = draw((T, self.Hq, self.Dv), g)
            return dict(q=q, k=k, v=v, do=do)
        S = self.shard
        q = draw((S, self.Hq, self.Dqk), g)
        k_local = draw((S, self.Hkv, self.Dqk), g)
        v_local = draw((S, self.Hkv, self.Dv), g)
        k_early = draw((S, self.Hkv, self.Dqk), g)
        v_early = draw((S, self.Hkv, self.Dv), g)
        do = draw((S, self.Hq, self.Dv), g)
        return dict(q=q, k_local=k_local, v_local=v_local, k_early=k_early,
                    v_early=v_early, do=do)


def ring_pairs(row_ids: np.ndarray, shard: int) -> int:
    """Visible pairs per head for the rank holding the second half of the row:
    query at p sees key j iff both share a document id > 0 and j <= p."""
    ids = row_ids[0]
    tot = 0
    q_ids = ids[shard:2 * shard]
    for d in np.unique(q_ids):
        if d == 0:
            continue
        key_pos = np.nonzero(ids == d)[0]
        q_pos = shard + np.nonzero(q_ids == d)[0]
        tot += int(np.searchsorted(key_pos, q_pos, side="right").sum())
    return tot


def workload(n: int) -> Workload:
    """The named workloads (1: small dense, 2: varlen D128, 3: dense D512,
    4: varlen 192/128, 5: one rank of a two-rank ring at D512, 6: the same
    rank when its row is a single document, the dense-routed ring chunks,
    7: workload 5 through the packed gather layout of live tokens)."""
    if n == 1:
        return Workload("dense_causal_b1_h4kv2_n256_d128", "dense", 1, Hq=4, Hkv=2, Dqk=128,
                        Dv=128, B=1, Nq=256, Nk=256)
    if n == 2:
        return Workload("varlen_doc_causal_t16384_h32kv8_d128", "varlen", 2, Hq=32, Hkv=8,
                        Dqk=128, Dv=128, lengths=doc_lengths(16384, 32, 4096, 2))
    if n == 3:
        return Workload("dense_causal_b2_h16kv8_n8192_d512", "dense", 3, Hq=16, Hkv=8, Dqk=512,
                        Dv=512, B=2, Nq=8192, Nk=8192)
    if n == 4:
        return Workload("varlen_doc_causal_t32768_h32_dqk192_dv128", "varlen", 4, Hq=32, Hkv=32,
                        Dqk=192, Dv=128, lengths=doc_lengths(32768, 512, 8192, 4))
    if n == 5:
        return Workload("ring_rank1_of2_q4096_h16kv8_d512", "ring", 5, Hq=16, Hkv=8, Dqk=512,
                        Dv=512, shard=4096, pad_tail=128, doc_lo=256, doc_hi=4096)
    if n == 6:
        return Workload("ring_rank1_of2_single_doc_q4096_h16kv8_d512", "ring", 6, Hq=16, Hkv=8,
                        Dqk=512, Dv=512, shard=4096, pad_tail=128, single_doc=True)
    if n == 7:
        return Workload("ring_rank1_of2_q4096_h16kv8_d512_gather", "ring", 5, Hq=16, Hkv=8,
                        Dqk=512, Dv=512, shard=4096, pad_tail=128, doc_lo=256, doc_hi=4096,
                        route="gather")
    raise ValueError(f"no workload {n}")


def small_varlen(seed: int, lengths, Hq: int, Hkv: int, Dqk: int, Dv: int,
                 causal: bool = True) -> Workload:
    """A reduced varlen problem for parity at sizes the oracle finishes in seconds."""
    return Workload(f"varlen_small_s{seed}", "varlen", seed, Hq=Hq, Hkv=Hkv, Dqk=Dqk, Dv=Dv,
                    causal=causal, lengths=list(lengths))
