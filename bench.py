"""Benchmark: one step = the whole attention hot path (forward, then backward
from the forward's out/lse) over one batch of seeded synthetic input, timed on
one MI355X. Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--workload N] [--all]

The headline (``value``) is the largest workload that fits one GPU: packed
varlen document-causal attention with unequal head dims (T=32768, H=32,
Dqk=192, Dv=128; 8.2 TFLOP per step). The same line carries, under
``configs``, forward/backward TFLOP/s, % of peak and a roofline entry for each
of the four large workloads (2 varlen D128, 3 dense D512, 4 varlen 192/128,
5 ring share D512). ``--workload`` moves the headline to another of the six
(1 small dense, 2, 3, 4, 5, 6 ring share of a single-document row, whose
chunks take the dense route); ``--all`` adds every workload's full record.
Throughput is causal-adjusted: FLOPs count only visible (query, key) pairs,
forward 2*pairs*(Dqk+Dv), backward 2*pairs*(3*Dqk+2*Dv).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

import workloads

PEAK_BF16_TFLOPS = 256 * 2.4e9 * 4096 / 1e12  # 256 CUs x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
PEAK_HBM_GBS = 8000.0
METRIC = "attention fwd/bwd TFLOP/s (causal-adjusted) and % of bf16 MFMA peak, 1 GPU"


def _dev(t):
    return t.to("cuda")


class Problem:
    """Device-resident inputs of one workload and closures for each stage."""

    def __init__(self, n: int, dtype=torch.bfloat16):
        import varlen_causal_attention_amd as vca

        self.vca = vca
        self.w = w = workloads.workload(n)
        self.dtype = dtype
        t = w.tensors(dtype)
        self.t = {k: _dev(v) for k, v in t.items()}
        if w.kind == "varlen":
            cu = torch.from_numpy(w.cu()).to("cuda")
            self.cu, self.mx = cu, max(w.lengths)
        elif w.kind == "ring":
            ids = w.row_doc_ids()
            S = w.shard
            # dense routing when both chunks qualify (single-document row):
            # the dense kernels run on [1, H, S, D] views of the shard tensors
            ok_l, pad = vca.dense_route(ids, S, S, S, S, 0)
            ok_x, _ = vca.dense_route(ids, S, S, 0, S, 1)
            self.dense = ok_l and ok_x and w.route != "gather"
            self.gather = w.route == "gather"
            if self.gather:
                # packed live tokens: gather indices of the documents each chunk shares
                self.d = {k: x.unsqueeze(0).transpose(1, 2) for k, x in self.t.items()}
                self.segs = (vca.ring_segments(ids[:, S:], ids[:, S:], device="cuda"),
                             vca.ring_segments(ids[:, S:], ids[:, :S], device="cuda"))
            elif self.dense:
                self.pad = torch.from_numpy(pad).to("cuda")
                self.d = {k: x.unsqueeze(0).transpose(1, 2) for k, x in self.t.items()}
            else:
                self.local = vca.doc_layout(ids, S, S, S, S, 0, "cuda")
                self.cross = vca.doc_layout(ids, S, S, 0, S, 1, "cuda")
        self.out = self.lse = None
        self.gather = getattr(self, "gather", False)

    def fwd_gather(self):
        """Ring share through the gather layout: per chunk gather its live
        tokens, varlen forward, merge in place at its rows into fp32
        accumulators that start as 'attends nothing'."""
        v, w, d, S, H = self.vca, self.w, self.d, self.w.shard, self.w.Hq
        none = torch.empty(0, dtype=torch.int32, device="cuda")
        acc = torch.empty((1, H, S, w.Dv), dtype=torch.float32, device="cuda")
        v.scatter_rows(torch.empty((0, H, w.Dv), dtype=torch.float32, device="cuda"), none, acc,
                       mode=1)
        lacc = v.scatter_lse(torch.empty((H, 0), dtype=torch.float32, device="cuda"), none, 1, S)
        self.packed = []
        for seg, kn, vn, causal in zip(self.segs, ("k_local", "k_early"), ("v_local", "v_early"),
                                       (True, False)):
            qp = v.gather_rows(d["q"], seg["q_index"])
            kp = v.gather_rows(d[kn], seg["k_index"])
            vp = v.gather_rows(d[vn], seg["k_index"])
            op, lp = v.fwd_varlen(qp, kp, vp, seg["cu_q"], seg["cu_k"], seg["max_q"],
                                  seg["max_k"], w.scale, causal)
            v.merge_rows(acc, lacc, op, lp, seg["q_index"])
            self.packed.append((seg, qp, kp, vp, causal))
        self.out, self.lse = acc, lacc

    def bwd_gather(self):
        """Per chunk: gather the merged out/lse and dO at its rows, varlen
        backward, scatter dq (assigned by the first chunk, added by the next)
        and the chunk's dk / dv back to [1, H, S, D]."""
        v, w, d, S = self.vca, self.w, self.d, self.w.shard
        dq = torch.empty((1, w.Hq, S, w.Dqk), dtype=self.dtype, device="cuda")
        res = [dq]
        for i, (seg, qp, kp, vp, causal) in enumerate(self.packed):
            mo = v.gather_rows(self.out, seg["q_index"], dtype=self.dtype)
            ml = v.gather_lse(self.lse, seg["q_index"])
            dop = v.gather_rows(d["do"], seg["q_index"])
            dqp, dkp, dvp = v.bwd_varlen(dop, qp, kp, vp, mo, ml, seg["cu_q"], seg["cu_k"],
                                         seg["max_q"], seg["max_k"], w.scale, causal)
            v.scatter_rows(dqp, seg["q_index"], dq, mode=1 if i == 0 else 2)
            for src, D in ((dkp, w.Dqk), (dvp, w.Dv)):
                g = torch.empty((1, w.Hkv, S, D), dtype=self.dtype, device="cuda")
                res.append(v.scatter_rows(src, seg["k_index"], g, mode=1))
        return tuple(res)

    def fwd(self):
        v, w, t = self.vca, self.w, self.t
        if w.kind == "ring" and self.gather:
            return self.fwd_gather()
        if w.kind == "dense":
            self.out, self.lse = v.fwd_dense(t["q"], t["k"], t["v"], w.scale, w.causal)
        elif w.kind == "varlen":
            self.out, self.lse = v.fwd_varlen(t["q"], t["k"], t["v"], self.cu, self.cu, self.mx,
                                              self.mx, w.scale, w.causal)
        elif self.dense:
            o1, l1, o2, l2 = self.partials()
            _, lse, out = v.merge(o1, l1, o2, l2, copy_dtype=self.dtype)
            self.out = out.view(1, w.Hq, w.shard, w.Dv)
            self.lse = lse.view(1, w.Hq, w.shard)
        else:
            o1, l1, o2, l2 = self.partials()
            _, self.lse, self.out = v.merge(o1, l1, o2, l2, copy_dtype=self.dtype)

    def partials(self):
        """Ring share: the two partial forward results the merge combines
        (dense route: [1, H, S, D] results with padding rows zeroed, flattened
        to the merge's [rows, 1, D] / [1, rows] layout)."""
        v, w, t = self.vca, self.w, self.t
        if self.dense:
            d, n = self.d, w.Hq * w.shard
            o1, l1 = v.fwd_dense(d["q"], d["k_local"], d["v_local"], w.scale, True)
            v.zero_rows(o1, l1, self.pad)
            o2, l2 = v.fwd_dense(d["q"], d["k_early"], d["v_early"], w.scale, False)
            v.zero_rows(o2, l2, self.pad)
            return o1.view(n, 1, w.Dv), l1.view(1, n), o2.view(n, 1, w.Dv), l2.view(1, n)
        # the two chunks' forwards are independent: the earlier chunk's runs on
        # a second stream (default priority) beside the local one, so the two
        # small grids share the CUs instead of running one after the other
        main = torch.cuda.current_stream()
        side = self.side_stream()
        rows, H = t["q"].shape[0], w.Hq
        o2 = torch.empty((rows, H, w.Dv), dtype=self.dtype, device="cuda")
        l2 = torch.empty((H, rows), dtype=torch.float32, device="cuda")
        side.wait_stream(main)
        with torch.cuda.stream(side):
            cq, ck, mq, mk = self.cross
            v.fwd_varlen(t["q"], t["k_early"], t["v_early"], cq, ck, mq, mk, w.scale, False,
                         out=o2, lse=l2)
        cq, ck, mq, mk = self.local
        o1, l1 = v.fwd_varlen(t["q"], t["k_local"], t["v_local"], cq, ck, mq, mk, w.scale, True)
        main.wait_stream(side)
        return o1, l1, o2, l2

    def side_stream(self):
        """Stream of the earlier chunk's passes: a second default-priority
        stream, or the current one while ``serial`` is set (each launch then
        has the chip to itself, which is how per-kernel durations are timed)."""
        if getattr(self, "serial", False):
            return torch.cuda.current_stream()
        if getattr(self, "_side", None) is None:
            self._side = torch.cuda.Stream()
        return self._side

    def bwd(self):
        v, w, t = self.vca, self.w, self.t
        if w.kind == "ring" and self.gather:
            return self.bwd_gather()
        if w.kind == "dense":
            return v.bwd_dense(t["do"], t["q"], t["k"], t["v"], self.out, self.lse, w.scale, w.causal)
        if w.kind == "varlen":
            return v.bwd_varlen(t["do"], t["q"], t["k"], t["v"], self.out, self.lse, self.cu,
                                self.cu, self.mx, self.mx, w.scale, w.causal)
        if self.dense:
            d = self.d
            dq, dkl, dvl = v.bwd_dense(d["do"], d["q"], d["k_local"], d["v_local"], self.out,
                                       self.lse, w.scale, True)
            _, dke, dve = v.bwd_dense(d["do"], d["q"], d["k_early"], d["v_early"], self.out,
                                      self.lse, w.scale, False, dq_accumulate=dq)
            return dq, dkl, dvl, dke, dve
        # the two chunks' backwards run side by side as well (each a small
        # grid); the earlier chunk's dq is then added into the local one's
        # in fp32 (the library's row scatter-add over every row)
        main = torch.cuda.current_stream()
        side = self.side_stream()
        rows = t["q"].shape[0]
        dq2 = torch.empty_like(t["q"])
        dke = torch.empty_like(t["k_early"])
        dve = torch.empty_like(t["v_early"])
        side.wait_stream(main)
        with torch.cuda.stream(side):
            cq, ck, mq, mk = self.cross
            v.bwd_varlen(t["do"], t["q"], t["k_early"], t["v_early"], self.out, self.lse, cq, ck,
                         mq, mk, w.scale, False, dq=dq2, dk=dke, dv=dve)
        cq, ck, mq, mk = self.local
        dq, dkl, dvl = v.bwd_varlen(t["do"], t["q"], t["k_local"], t["v_local"], self.out,
                                    self.lse, cq, ck, mq, mk, w.scale, True)
        main.wait_stream(side)
        if getattr(self, "_all_rows", None) is None:
            self._all_rows = torch.arange(rows, dtype=torch.int32, device="cuda")
        v.scatter_rows(dq2, self._all_rows, dq.unsqueeze(0).transpose(1, 2), mode=2)
        return dq, dkl, dvl, dke, dve

    def step(self):
        self.fwd()
        return self.bwd()


def time_stage(fn, iters: int) -> float:
    """Mean ms per call, HIP events on the current stream (the one the library
    launches on)."""
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(iters):
        fn()
    e1.record(s)
    e1.synchronize()
    return e0.elapsed_time(e1) / iters


def time_calls(fn, min_iters: int = 20, min_ms: float = 200.0, flush=None) -> dict:
    """Per-call HIP-event times (ms) of fn: at least min_iters calls and
    min_ms in total; flush (if given) runs between calls, outside the timed
    events (an L2/MALL flush for the HBM-bound cases)."""
    s = torch.cuda.current_stream()
    times = []
    total = 0.0
    while len(times) < min_iters or total < min_ms:
        if flush is not None:
            flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        fn()
        e1.record(s)
        e1.synchronize()
        t = e0.elapsed_time(e1)
        times.append(t)
        total += t
        if len(times) >= 10000:
            break
    times.sort()
    return {"median_ms": round(times[len(times) // 2], 4), "min_ms": round(times[0], 4),
            "iters": len(times)}


class L2Flush:
    """Writes a 512 MiB scratch buffer: evicts L2 and MALL between calls."""

    def __init__(self):
        self.buf = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")

    def __call__(self):
        self.buf.fill_(1)


def measure(n: int, steps: int, warmup: int, per_call: bool = True, flush=None,
            dtype=torch.bfloat16) -> dict:
    p = Problem(n, dtype)
    w = p.w
    for _ in range(warmup):
        p.step()
    torch.cuda.synchronize()
    # the timed region: exactly `steps` whole steps
    t0 = time.perf_counter()
    step_ms_ev = time_stage(p.step, steps)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    fwd_ms = time_stage(p.fwd, steps)
    bwd_ms = time_stage(p.bwd, steps)
    torch.cuda.synchronize()
    kernels = kernel_times(p, steps)
    ff, bf = w.fwd_flops(), w.bwd_flops()
    r = dict(workload=w.name, ms_per_step=step_ms_ev, wall_ms_per_step=wall,
             tflops_step=(ff + bf) / (step_ms_ev * 1e-3) / 1e12,
             fwd_ms=fwd_ms, bwd_ms=bwd_ms,
             fwd_tflops=ff / (fwd_ms * 1e-3) / 1e12, bwd_tflops=bf / (bwd_ms * 1e-3) / 1e12,
             fwd_flops=ff, bwd_flops=bf, pairs=w.pairs(), kernels=kernels)
    if per_call:
        # one forward call / one backward call: median and min over >= 20 calls
        # and >= 200 ms
        r["fwd_calls"] = time_calls(p.fwd)
        r["bwd_calls"] = time_calls(p.bwd)
        if w.kind == "ring" and not p.gather:
            # the lse merge alone (HBM-bound elementwise)
            parts = p.partials()
            r["merge_calls"] = time_calls(lambda: p.vca.merge(*parts, copy_dtype=p.dtype))
            if flush is not None:
                r["merge_calls_l2_flushed"] = time_calls(
                    lambda: p.vca.merge(*parts, copy_dtype=p.dtype), flush=flush)
        elif flush is not None:
            r["fwd_calls_l2_flushed"] = time_calls(p.fwd, flush=flush)
            r["bwd_calls_l2_flushed"] = time_calls(p.bwd, flush=flush)
    return r


def kernel_times(p: "Problem", steps: int) -> dict:
    """Per-kernel mean launch duration (ms) and launches per step, from HIP
    events the library records around each of its launches on their stream."""
    vca = p.vca
    vca.timing_read()  # drop anything recorded earlier
    # the ring share's two chunks overlap on two streams in a step; here they
    # run one after the other so that each launch's duration is that of the
    # kernel alone on the chip
    p.serial = True
    vca.timing_enable(True)
    try:
        for _ in range(steps):
            p.step()
        recs = vca.timing_read(1 << 16)
    finally:
        vca.timing_enable(False)
        p.serial = False
    agg: dict = {}
    for name, ms in recs:
        t, n = agg.get(name, (0.0, 0))
        agg[name] = (t + ms, n + 1)
    return {k: {"mean_ms": t / n, "per_step": n / steps} for k, (t, n) in agg.items()}


def kernel_work(w: "workloads.Workload", name: str):
    """(bound, algorithmic units per launch, unit) of one library kernel.
    Forward: 2*pairs*(Dqk+Dv) FLOPs. dK/dV pass: S, dP, dV, dK products,
    2*pairs*(2*Dqk+2*Dv). dQ pass: the dQ product only, 2*pairs*Dqk (its S/dP
    recomputation is not algorithmic work). Two-phase backward: scores S and
    dP, 2*pairs*(Dqk+Dv); products dV and dK, 2*pairs*(Dqk+Dv); dQ,
    2*pairs*Dqk. delta pass: bytes of O and dO read
    plus delta written. Merge: bytes of both inputs read and the output written."""
    pairs = w.pairs()
    rows = w.T if w.kind == "varlen" else (w.shard if w.kind == "ring" else w.B * w.Nq)
    chunks = 2 if w.kind == "ring" else 1
    if name == "attn_fwd":
        return "mfma", 2 * pairs * (w.Dqk + w.Dv) / chunks, "FLOP"
    if name == "attn_bwd_dkdv":
        return "mfma", 2 * pairs * (2 * w.Dqk + 2 * w.Dv) / chunks, "FLOP"
    if name in ("attn_bwd_dq", "attn_bwd_dq_ds"):
        return "mfma", 2 * pairs * w.Dqk / chunks, "FLOP"
    # two-phase backward (large head dims): scores S and dP, then products
    if name == "attn_bwd_scores":
        return "mfma", 2 * pairs * (w.Dqk + w.Dv) / chunks, "FLOP"
    if name == "attn_bwd_dkdv_tiles":
        return "mfma", 2 * pairs * (w.Dqk + w.Dv) / chunks, "FLOP"
    if name == "attn_bwd_dq_tiles":
        return "mfma", 2 * pairs * w.Dqk / chunks, "FLOP"
    if name == "attn_bwd_delta":
        return "hbm", rows * w.Hq * (2 * w.Dv * 2 + 4), "B"
    if name == "attn_merge":
        return "hbm", rows * w.Hq * (w.Dv * (2 + 2 + 4 + 2) + 4 * 3), "B"
    if name == "attn_zero_rows":
        return "hbm", w.pad_tail * w.Hq * (w.Dv * 2 + 4), "B"
    return None


def chunk_count(w: "workloads.Workload") -> int:
    """Calls of one pass per step in kernel_work's units (two ring chunks)."""
    return 2 if w.kind == "ring" else 1


def roofline(w: "workloads.Workload", kernels: dict) -> dict:
    """Roofline entry of the kernel that takes the most time per step."""
    ranked = sorted(kernels, key=lambda k: -kernels[k]["mean_ms"] * kernels[k]["per_step"])
    name = next(k for k in ranked if kernel_work(w, k) is not None)
    bound, units, unit = kernel_work(w, name)
    # a pass split over several launches (the dS-store backward runs one
    # dK/dV + dQ launch pair per chunk of kv-heads) does its step's work
    # over all of them: units per launch = step units / launches per step
    units = units * chunk_count(w) / kernels[name]["per_step"]
    sec = kernels[name]["mean_ms"] * 1e-3
    if bound == "mfma":
        achieved = units / sec / 1e12
        peak, u = PEAK_BF16_TFLOPS, "TFLOP/s"
    else:
        achieved = units / sec / 1e9
        peak, u = PEAK_HBM_GBS, "GB/s"
    return {"bound": bound, "kernel": name, "achieved": round(achieved, 2), "peak": round(peak, 1),
            "unit": u, "frac": round(achieved / peak, 4),
            "traffic": measured_traffic(name, w.name),
            "launch_ms": round(kernels[name]["mean_ms"], 4),
            "per_unit": PER_UNIT.get(name, unit),
            **({"launches": "ring chunks timed one after the other"} if w.kind == "ring" else {})}


PER_UNIT = {
    "attn_fwd": "2*pairs*(Dqk+Dv) FLOP",
    "attn_bwd_dkdv": "2*pairs*(2*Dqk+2*Dv) FLOP",
    "attn_bwd_dq": "2*pairs*Dqk FLOP",
    "attn_bwd_dq_ds": "2*pairs*Dqk FLOP",
    "attn_bwd_scores": "2*pairs*(Dqk+Dv) FLOP",
    "attn_bwd_dkdv_tiles": "2*pairs*(Dqk+Dv) FLOP",
    "attn_bwd_dq_tiles": "2*pairs*Dqk FLOP",
}


HERE = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(HERE, "profiles", "hbm_traffic.md")


def sources_digest() -> str:
    """sha256 over the library's kernel sources: counter figures taken from an
    older build stop applying as soon as any of them changes."""
    import hashlib
    csrc = os.path.join(HERE, "varlen_causal_attention_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".hpp", ".cpp")):
            h.update(f.encode())
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    counter summary (FETCH_SIZE + WRITE_SIZE, calibrated against a plain copy),
    or None when there is none for the current sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    want = sources_digest()
    with open(TRAFFIC_FILE) as fh:
        for line in fh:
            if not line.startswith("kernel="):
                continue
            kv = dict(x.split("=", 1) for x in line.split())
            if kv.get("kernel") == kernel and kv.get("workload") == workload \
                    and kv.get("sources") == want:
                return float(kv["bytes"])
    return None


def copy_calibration(gib: int = 1) -> None:
    """A plain elementwise copy of known size (reads and writes `gib` GiB),
    the reference the FETCH_SIZE / WRITE_SIZE counters are scaled by."""
    n = gib * (1 << 30) // 4
    src = torch.ones(n, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n * 4, "bytes_written": n * 4,
                      "dispatches": 3}), flush=True)


def gemm_reference() -> None:
    """The chip's practical bf16 matrix rate on plain square GEMMs through
    torch.matmul (hipBLASLt), timed like the bench steps: a reference for the
    attention kernels' rates beside the published peak, which assumes the
    2.4 GHz top clock that dense matrix work does not hold."""
    out = []
    for n, iters in ((8192, 20), (16384, 5)):
        a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
        b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
        for _ in range(3):
            torch.matmul(a, b)
        ms = time_stage(lambda: torch.matmul(a, b), iters)
        tf = 2.0 * n ** 3 / ms / 1e9
        out.append({"n": n, "ms": round(ms, 4), "tflops": round(tf, 1),
                    "pct_of_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2)})
        del a, b
    print(json.dumps({"gemm_reference": "torch.matmul bf16 n x n x n", "runs": out}), flush=True)


def cpu_baseline(n: int, budget_s: float = 12.0) -> dict:
    """The fp64 oracle on the host cores over a bounded sample of the workload:
    whole documents of one q-head group at a time (forward then backward),
    until the time budget is used; FLOPs counted the same causal-adjusted way."""
    from oracle import attention as orc

    w = workloads.workload(n)
    if w.kind != "varlen":
        w = workloads.workload(2)
    t = w.tensors()
    cu = w.cu()
    G = w.Hq // w.Hkv
    flops = 0
    ffl = bfl = 0
    tf = tb = 0.0
    done = []
    t0 = time.perf_counter()
    order = np.argsort(w.lengths)  # shortest documents first keeps the sample bounded
    for s in order:
        a, b = int(cu[s]), int(cu[s + 1])
        for g in range(w.Hkv):
            hs = list(range(g * G, (g + 1) * G))
            sl = lambda x, heads: x[a:b][:, heads]  # noqa: E731
            qq, kk, vv, dd = sl(t["q"], hs), sl(t["k"], [g]), sl(t["v"], [g]), sl(t["do"], hs)
            c1 = [0, b - a]
            t1 = time.perf_counter()
            ro, rl = orc.fwd_varlen(qq, kk, vv, c1, c1, w.scale, True)
            t2 = time.perf_counter()
            orc.bwd_varlen(dd, qq, kk, vv, ro, rl, c1, c1, w.scale, True)
            tf += t2 - t1
            tb += time.perf_counter() - t2
            pairs = len(hs) * workloads.causal_pairs(b - a, b - a)
            ffl += 2 * pairs * (w.Dqk + w.Dv)
            bfl += 2 * pairs * (3 * w.Dqk + 2 * w.Dv)
            flops = ffl + bfl
            done.append((b - a, g))
            if time.perf_counter() - t0 > budget_s:
                break
        if time.perf_counter() - t0 > budget_s:
            break
    el = time.perf_counter() - t0
    cores = len(os.sched_getaffinity(0))
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "fwd_gflops": round(ffl / tf / 1e9, 3) if tf else None,
            "bwd_gflops": round(bfl / tb / 1e9, 3) if tb else None,
            "fwd_s": round(tf, 3), "bwd_s": round(tb, 3), "blas": blas_name(),
            "sample": f"{w.name}: {len(done)} (document, kv-head group) slices, forward+backward in "
                      f"fp64 numpy, {el:.1f} s, BLAS threads = {cores}"}


def blas_name() -> str:
    """The BLAS numpy was built against (reported with the CPU baseline)."""
    try:
        cfg = np.show_config(mode="dicts")
        b = cfg["Build Dependencies"]["blas"]
        return f"{b.get('name')} {b.get('version', '')}".strip()
    except Exception:  # older numpy: no dict mode
        return "unknown"


LARGE_WORKLOADS = (2, 3, 4, 5)


def config_entry(w: "workloads.Workload", r: dict) -> dict:
    """Per-config summary: step, forward and backward throughput against the
    bf16 MFMA peak, per-call medians, and the dominant kernel's roofline."""
    pct = lambda x: round(100 * x / PEAK_BF16_TFLOPS, 2)  # noqa: E731
    e = {"ms_per_step": round(r["ms_per_step"], 4), "tflops_step": round(r["tflops_step"], 2),
         "pct_of_peak": pct(r["tflops_step"]),
         "fwd": {"ms": round(r["fwd_ms"], 4), "tflops": round(r["fwd_tflops"], 2),
                 "pct_of_peak": pct(r["fwd_tflops"])},
         "bwd": {"ms": round(r["bwd_ms"], 4), "tflops": round(r["bwd_tflops"], 2),
                 "pct_of_peak": pct(r["bwd_tflops"])},
         "pairs": r["pairs"], "roofline": roofline(w, r["kernels"]),
         "kernels_ms": {k: round(v["mean_ms"], 4) for k, v in r["kernels"].items()}}
    for k in ("fwd_calls", "bwd_calls", "merge_calls"):
        if k in r:
            e[k] = r[k]
    return e


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=4)
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-config entries of the other large workloads")
    ap.add_argument("--all", action="store_true", help="also report every workload")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB elementwise copy (counter calibration) and exit")
    ap.add_argument("--gemm-reference", action="store_true",
                    help="only time plain bf16 GEMMs (torch.matmul) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration()
        return
    if args.gemm_reference:
        gemm_reference()
        return
    m = measure(args.workload, args.steps, args.warmup)
    w = workloads.workload(args.workload)
    fwd_tf = m["fwd_tflops"]
    line = {
        "metric": METRIC,
        "value": round(m["tflops_step"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(m["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "kind": w.kind, "Hq": w.Hq, "Hkv": w.Hkv, "Dqk": w.Dqk,
                   "Dv": w.Dv, "tokens": w.T if w.kind == "varlen" else None,
                   "causal": w.causal, "pairs": m["pairs"]},
        "pct_of_peak": round(100 * m["tflops_step"] / PEAK_BF16_TFLOPS, 2),
        "fwd": {"ms": round(m["fwd_ms"], 4), "tflops": round(fwd_tf, 2),
                "pct_of_peak": round(100 * fwd_tf / PEAK_BF16_TFLOPS, 2), **m["fwd_calls"]},
        "bwd": {"ms": round(m["bwd_ms"], 4), "tflops": round(m["bwd_tflops"], 2),
                "pct_of_peak": round(100 * m["bwd_tflops"] / PEAK_BF16_TFLOPS, 2),
                **m["bwd_calls"]},
        "roofline": roofline(w, m["kernels"]),
        "kernels_ms": {k: round(v["mean_ms"], 4) for k, v in m["kernels"].items()},
        "wall_ms_per_step": round(m["wall_ms_per_step"], 4),
    }
    if not args.no_configs:
        # forward / backward throughput and the roofline of each large workload
        configs = {}
        for n in LARGE_WORKLOADS:
            r = m if n == args.workload else measure(n, max(5, args.steps // 2), 3)
            configs[r["workload"]] = config_entry(workloads.workload(n), r)
        line["configs"] = configs
        # workload 5 through the packed gather layout of live tokens
        r = measure(7, max(5, args.steps // 2), 3, per_call=False)
        line["ring_gather_layout"] = config_entry(workloads.workload(7), r)
        # the same workloads with fp16 inputs (same kernels, fp16 MFMA)
        line["configs_fp16"] = {}
        for n in LARGE_WORKLOADS:
            r = measure(n, max(5, args.steps // 2), 3, per_call=False, dtype=torch.float16)
            e = config_entry(workloads.workload(n), r)
            line["configs_fp16"][r["workload"]] = {k: e[k] for k in ("ms_per_step", "tflops_step",
                                                                    "pct_of_peak", "fwd", "bwd")}
    if args.all:
        per = {}
        flush = L2Flush()
        for n in range(1, 8):
            # the small workload and the ring share's merge are latency / HBM
            # bound: also timed with L2 and MALL flushed
            r = measure(n, max(3, args.steps // 2), 2, flush=flush if n in (1, 5, 6, 7) else None)
            per[r["workload"]] = {k: (round(v, 4) if isinstance(v, float) else v)
                                  for k, v in r.items() if k not in ("workload", "kernels")}
            per[r["workload"]]["kernels_ms"] = {k: round(v["mean_ms"], 4)
                                                for k, v in r["kernels"].items()}
        line["workloads"] = per
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(args.workload)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
