"""The no-allocation varlen forward (attn_fwd_varlen_noalloc) against the
workspace entry point it shares its kernels with: two calls in a row, the
second on a smaller input, through the C ABI; plus its size limit."""
import ctypes as C
import math

import numpy as np
import pytest
import torch

import workloads
from varlen_causal_attention_amd import _lib

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def vca():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import varlen_causal_attention_amd as m

    m.load()
    return m


def _case(seed, lens, Hq, Hkv, D, Dv):
    g = torch.Generator().manual_seed(seed)
    cu = workloads.cumulative(lens)
    T = int(cu[-1])
    q = workloads.randn_bf16((T, Hq, D), g).cuda()
    k = workloads.randn_bf16((T, Hkv, D), g).cuda()
    v = workloads.randn_bf16((T, Hkv, Dv), g).cuda()
    return q, k, v, torch.from_numpy(cu).cuda(), max(lens)


def _noalloc(lib, q, k, v, cu, mx, scale, causal, out, lse):
    Tq, Hq, D = q.shape
    Tk, Hkv, _ = k.shape
    Dv = v.shape[2]
    strides = _lib.i64_array(list(q.stride()[:2]) + list(k.stride()[:2]) + list(v.stride()[:2])
                             + list(out.stride()[:2]))
    P = lambda t: C.c_void_p(t.data_ptr())  # noqa: E731
    return lib.attn_fwd_varlen_noalloc(0, P(q), P(k), P(v), P(out), P(lse), P(cu), P(cu),
                                       cu.numel() - 1, mx, mx, Tq, Tk, Hq, Hkv, D, Dv, strides,
                                       scale, causal,
                                       C.c_void_p(torch.cuda.current_stream().cuda_stream))


@pytest.mark.parametrize("D,Dv", [(128, 128), (192, 128), (512, 512)])
def test_noalloc_matches_workspace_entry_twice(vca, D, Dv):
    lib = _lib.load()
    # a larger call, then a smaller one: the second must not see the first's list
    cases = [(201, [900, 1, 1500, 37, 640], 8, 2), (202, [150, 70], 4, 2)]
    for seed, lens, Hq, Hkv in cases:
        for causal in (1, 0):
            q, k, v, cu, mx = _case(seed + D, lens, Hq, Hkv, D, Dv)
            scale = 1 / math.sqrt(D)
            T = q.shape[0]
            out = torch.full((T, Hq, Dv), float("nan"), dtype=torch.bfloat16, device="cuda")
            lse = torch.full((Hq, T), float("nan"), dtype=torch.float32, device="cuda")
            st = _noalloc(lib, q, k, v, cu, mx, scale, causal, out, lse)
            assert st == 0, lib.attn_last_error()
            ref_o, ref_l = vca.fwd_varlen(q, k, v, cu, cu, mx, mx, scale, bool(causal))
            torch.cuda.synchronize()
            # the same kernels on the same inputs: bitwise equal
            assert torch.equal(out, ref_o), (seed, causal)
            assert torch.equal(lse, ref_l), (seed, causal)


def test_noalloc_python_binding(vca):
    q, k, v, cu, mx = _case(203, [300, 5, 77], 4, 4, 64, 64)
    out = torch.empty((q.shape[0], 4, 64), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((4, q.shape[0]), dtype=torch.float32, device="cuda")
    vca.fwd_varlen_noalloc(q, k, v, cu, cu, mx, mx, 0.125, True, out, lse)
    ref_o, ref_l = vca.fwd_varlen(q, k, v, cu, cu, mx, mx, 0.125, True)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)
