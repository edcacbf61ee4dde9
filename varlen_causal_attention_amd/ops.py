"""Torch-facing binding of the C ABI: shape checks, output allocation and
argument marshalling. Every step of the computation runs in the HIP library;
torch only provides device memory and the current stream.

Names and call shapes follow the dense / varlen forward and backward wrappers
of the NeMo-Automodel "ffpa_attention" page.
"""
from __future__ import annotations

import ctypes as C

import numpy as np
import torch

from ._lib import (ATTN_BF16, ATTN_DQ_ACCUMULATE, ATTN_F16, ATTN_F32, AttnExt, check, i64_array,
                   load)

# element types of q, k, v, out, dout and the gradients (one per call)
_DTYPES = {torch.bfloat16: ATTN_BF16, torch.float16: ATTN_F16}


def _stream(t: torch.Tensor) -> C.c_void_p:
    return C.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return C.c_void_p(t.data_ptr()) if t is not None and t.numel() > 0 else C.c_void_p(0)


def _need_gpu_half(**tensors):
    """(device, torch dtype) of GPU tensors that share one element type,
    bfloat16 or float16, each with a contiguous last dimension."""
    dev = dt = None
    for name, t in tensors.items():
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on the GPU")
        if t.dtype not in _DTYPES:
            raise ValueError(f"{name} must be bfloat16 or float16")
        if t.numel() > 0 and t.stride(-1) != 1:
            raise ValueError(f"{name} must have a contiguous last dimension")
        if dev is None:
            dev, dt = t.device, t.dtype
        elif t.device != dev:
            raise ValueError("all tensors must be on one device")
        elif t.dtype != dt:
            raise ValueError("q, k, v (and out, dout, gradients) must share one dtype")
    return dev, dt


def _dense_shapes(q, k, v):
    """(B, Hq, Hkv, Nq, Nk, Dqk, Dv) of dense [B, H, N, D] q/k/v, or ValueError."""
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("dense tensors are [B, H, N, D]")
    B, Hq, Nq, Dqk = q.shape
    Bk, Hkv, Nk, Dk = k.shape
    if Bk != B or Dk != Dqk or tuple(v.shape[:3]) != tuple(k.shape[:3]):
        raise ValueError("q/k/v shapes disagree")
    return B, Hq, Hkv, Nq, Nk, Dqk, v.shape[3]


def _varlen_shapes(q, k, v):
    """(Tq, Tk, Hq, Hkv, Dqk, Dv) of packed [T, H, D] q/k/v, or ValueError."""
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("varlen tensors are [T, H, D]")
    Tq, Hq, Dqk = q.shape
    Tk, Hkv, Dk = k.shape
    if Dk != Dqk or tuple(v.shape[:2]) != tuple(k.shape[:2]):
        raise ValueError("q/k/v shapes disagree")
    return Tq, Tk, Hq, Hkv, Dqk, v.shape[2]


def _output(t, shape, dtype, dev, name):
    """A caller-supplied output (any strides with a unit last one), checked, or
    a new tensor. The library writes every element of an output, so a caller
    may pass e.g. a view into a larger buffer."""
    if t is None:
        return torch.empty(shape, dtype=dtype, device=dev)
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or t.device != dev:
        raise ValueError(f"{name} must be a {dtype} tensor on {dev}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}")
    if t.numel() > 0 and t.stride(-1) != 1:
        raise ValueError(f"{name} must have a contiguous last dimension")
    return t


def _lse_output(t, shape, dev):
    if t is not None and not t.is_contiguous():
        raise ValueError("lse must be contiguous")
    return _output(t, shape, torch.float32, dev, "lse")


def _workspace(size: int, device) -> torch.Tensor:
    return torch.empty(max(size, 16), dtype=torch.uint8, device=device)


def is_supported(dqk: int, dv: int, dtype=torch.bfloat16) -> bool:
    return bool(load().attn_is_supported(_DTYPES.get(dtype, -1), dqk, dv))


def version() -> int:
    return int(load().attn_version())


# ---------------------------------------------------------------------------
# dense [B, H, N, D]
# ---------------------------------------------------------------------------
def _ext(window, softcap):
    """attn_ext pointer for the _ex entry points, or None for the plain call."""
    window, softcap = int(window), float(softcap)
    if window == 0 and softcap == 0.0:
        return None
    return C.pointer(AttnExt(window, softcap))


def _call(lib, name, ext, args, tail):
    """Call the plain entry point, or its _ex form with ext inserted after the
    arguments `args` (the causal flag is their last element)."""
    if ext is None:
        return getattr(lib, name)(*args, *tail)
    return getattr(lib, name + "_ex")(*args, ext, *tail)


def fwd_dense(q, k, v, scale: float, causal: bool, out=None, lse=None, window: int = 0,
              softcap: float = 0.0):
    """out [B, Hq, Nq, Dv] bf16 and lse [B, Hq, Nq] fp32 (natural log). out / lse
    may be given (out as any view with a unit last stride, lse contiguous).
    window > 0 (causal only): each query sees its `window` most recent keys;
    softcap > 0: scores become softcap * tanh(score / softcap)."""
    B, Hq, Hkv, Nq, Nk, Dqk, Dv = _dense_shapes(q, k, v)
    dev, dt = _need_gpu_half(q=q, k=k, v=v)
    out = _output(out, (B, Hq, Nq, Dv), dt, dev, "out")
    lse = _lse_output(lse, (B, Hq, Nq), dev)
    strides = i64_array(list(q.stride()[:3]) + list(k.stride()[:3]) + list(v.stride()[:3])
                        + list(out.stride()[:3]))
    lib = load()
    args = (_DTYPES[dt], _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, Nq, Nk, Dqk, Dv,
            strides, float(scale), int(bool(causal)))
    ext = _ext(window, softcap)
    need = C.c_size_t(0)
    check(_call(lib, "attn_fwd_dense", ext, args, (None, C.byref(need), _stream(q))),
          "attn_fwd_dense")
    ws = _workspace(need.value, dev)
    have = C.c_size_t(ws.numel())
    check(_call(lib, "attn_fwd_dense", ext, args, (_ptr(ws), C.byref(have), _stream(q))),
          "attn_fwd_dense")
    return out, lse


def bwd_dense(dout, q, k, v, out, lse, scale: float, causal: bool, dq_accumulate=None,
              dq=None, dk=None, dv=None, window: int = 0, softcap: float = 0.0):
    """(dq, dk, dv) from the caller's out/lse; dk/dv have Hkv heads.
    dq_accumulate: an existing dq tensor to add this call's dq into.
    dq / dk / dv: optional output views (unit last stride).
    window / softcap: as given to the forward that produced out/lse."""
    B, Hq, Hkv, Nq, Nk, Dqk, Dv = _dense_shapes(q, k, v)
    if tuple(out.shape) != (B, Hq, Nq, Dv) or tuple(dout.shape) != (B, Hq, Nq, Dv):
        raise ValueError("out/dout must be [B, Hq, Nq, Dv]")
    dev, dt = _need_gpu_half(dout=dout, q=q, k=k, v=v, out=out)
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, Nq) or not lse.is_contiguous():
        raise ValueError("lse must be contiguous fp32 [B, Hq, Nq]")
    if lse.device != dev:
        raise ValueError("lse must be on the GPU with the other tensors")
    flags = 0
    if dq_accumulate is not None:
        _need_gpu_half(dq=dq_accumulate, q=q)
        if tuple(dq_accumulate.shape) != tuple(q.shape):
            raise ValueError("dq_accumulate must have q's shape")
        if dq is not None:
            raise ValueError("give dq or dq_accumulate, not both")
        dq = dq_accumulate
        flags |= ATTN_DQ_ACCUMULATE
    else:
        dq = _output(dq, (B, Hq, Nq, Dqk), dt, dev, "dq")
    dk = _output(dk, (B, Hkv, Nk, Dqk), dt, dev, "dk")
    dv = _output(dv, (B, Hkv, Nk, Dv), dt, dev, "dv")
    strides = i64_array(sum((list(t.stride()[:3]) for t in (q, k, v, out, dout, dq, dk, dv)), []))
    lib = load()
    args = (_DTYPES[dt], _ptr(dout), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dq),
            _ptr(dk), _ptr(dv), B, Hq, Hkv, Nq, Nk, Dqk, Dv, strides, float(scale),
            int(bool(causal)))
    ext = _ext(window, softcap)
    need = C.c_size_t(0)
    check(_call(lib, "attn_bwd_dense", ext, args, (flags, None, C.byref(need), _stream(q))),
          "attn_bwd_dense")
    ws = _workspace(need.value, dev)
    have = C.c_size_t(ws.numel())
    check(_call(lib, "attn_bwd_dense", ext, args, (flags, _ptr(ws), C.byref(have), _stream(q))),
          "attn_bwd_dense")
    return dq, dk, dv


# ---------------------------------------------------------------------------
# packed varlen THD [T, H, D]
# ---------------------------------------------------------------------------
def _cu(cu, dev):
    if cu.dtype != torch.int32 or cu.device != dev or cu.dim() != 1 or not cu.is_contiguous():
        raise ValueError("cu_seqlens must be contiguous int32 [segments + 1] on the GPU")
    return C.c_void_p(cu.data_ptr())


def fwd_varlen(q, k, v, cu_q, cu_k, max_q: int, max_k: int, scale: float, causal: bool,
               out=None, lse=None, window: int = 0, softcap: float = 0.0):
    """out [Tq, Hq, Dv] bf16 and lse [Hq, Tq] fp32 (natural log). out / lse may
    be given (out as any view with a unit last stride, lse contiguous).
    window / softcap: as in fwd_dense, per segment."""
    Tq, Tk, Hq, Hkv, Dqk, Dv = _varlen_shapes(q, k, v)
    if cu_q.numel() != cu_k.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    dev, dt = _need_gpu_half(q=q, k=k, v=v)
    out = _output(out, (Tq, Hq, Dv), dt, dev, "out")
    lse = _lse_output(lse, (Hq, Tq), dev)
    strides = i64_array(list(q.stride()[:2]) + list(k.stride()[:2]) + list(v.stride()[:2])
                        + list(out.stride()[:2]))
    lib = load()
    args = (_DTYPES[dt], _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _cu(cu_q, dev),
            _cu(cu_k, dev), cu_q.numel() - 1, int(max_q), int(max_k), Tq, Tk, Hq, Hkv, Dqk, Dv,
            strides, float(scale), int(bool(causal)))
    ext = _ext(window, softcap)
    need = C.c_size_t(0)
    check(_call(lib, "attn_fwd_varlen", ext, args, (None, C.byref(need), _stream(q))),
          "attn_fwd_varlen")
    ws = _workspace(need.value, dev)
    have = C.c_size_t(ws.numel())
    check(_call(lib, "attn_fwd_varlen", ext, args, (_ptr(ws), C.byref(have), _stream(q))),
          "attn_fwd_varlen")
    return out, lse


def fwd_varlen_noalloc(q, k, v, cu_q, cu_k, max_q: int, max_k: int, scale: float, causal: bool,
                       out, lse):
    """attn_fwd_varlen_noalloc: the varlen forward into caller-given out
    [Tq, Hq, Dv] bf16 and lse [Hq, Tq] fp32 with no device allocation at all
    (its work list uses the library's static scratch). Calls that overlap on
    one GPU race."""
    Tq, Tk, Hq, Hkv, Dqk, Dv = _varlen_shapes(q, k, v)
    if cu_q.numel() != cu_k.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    if out is None or lse is None:
        raise ValueError("out and lse must be given")
    dev, dt = _need_gpu_half(q=q, k=k, v=v)
    out = _output(out, (Tq, Hq, Dv), dt, dev, "out")
    lse = _lse_output(lse, (Hq, Tq), dev)
    strides = i64_array(list(q.stride()[:2]) + list(k.stride()[:2]) + list(v.stride()[:2])
                        + list(out.stride()[:2]))
    st = load().attn_fwd_varlen_noalloc(
        _DTYPES[dt], _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _cu(cu_q, dev),
        _cu(cu_k, dev), cu_q.numel() - 1, int(max_q), int(max_k), Tq, Tk, Hq, Hkv, Dqk, Dv, strides, float(scale),
        int(bool(causal)), _stream(q))
    check(st, "attn_fwd_varlen_noalloc")
    return out, lse


def bwd_varlen(dout, q, k, v, out, lse, cu_q, cu_k, max_q: int, max_k: int, scale: float,
               causal: bool, dq_accumulate=None, dq=None, dk=None, dv=None, window: int = 0,
               softcap: float = 0.0):
    """(dq [Tq,Hq,Dqk], dk [Tk,Hkv,Dqk], dv [Tk,Hkv,Dv]) from the caller's out/lse.
    dq / dk / dv: optional output views (unit last stride).
    window / softcap: as given to the forward that produced out/lse."""
    Tq, Tk, Hq, Hkv, Dqk, Dv = _varlen_shapes(q, k, v)
    if tuple(out.shape) != (Tq, Hq, Dv) or tuple(dout.shape) != (Tq, Hq, Dv):
        raise ValueError("out/dout must be [Tq, Hq, Dv]")
    dev, dt = _need_gpu_half(dout=dout, q=q, k=k, v=v, out=out)
    if lse.dtype != torch.float32 or tuple(lse.shape) != (Hq, Tq) or not lse.is_contiguous():
        raise ValueError("lse must be contiguous fp32 [Hq, Tq]")
    if lse.device != dev:
        raise ValueError("lse must be on the GPU with the other tensors")
    if cu_q.numel() != cu_k.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    flags = 0
    if dq_accumulate is not None:
        _need_gpu_half(dq=dq_accumulate, q=q)
        if tuple(dq_accumulate.shape) != tuple(q.shape):
            raise ValueError("dq_accumulate must have q's shape")
        if dq is not None:
            raise ValueError("give dq or dq_accumulate, not both")
        dq = dq_accumulate
        flags |= ATTN_DQ_ACCUMULATE
    else:
        dq = _output(dq, (Tq, Hq, Dqk), dt, dev, "dq")
    dk = _output(dk, (Tk, Hkv, Dqk), dt, dev, "dk")
    dv = _output(dv, (Tk, Hkv, Dv), dt, dev, "dv")
    strides = i64_array(sum((list(t.stride()[:2]) for t in (q, k, v, out, dout, dq, dk, dv)), []))
    lib = load()
    args = (_DTYPES[dt], _ptr(dout), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dq),
            _ptr(dk), _ptr(dv), _cu(cu_q, dev), _cu(cu_k, dev), cu_q.numel() - 1, int(max_q),
            int(max_k), Tq, Tk, Hq, Hkv, Dqk, Dv, strides, float(scale), int(bool(causal)))
    ext = _ext(window, softcap)
    need = C.c_size_t(0)
    check(_call(lib, "attn_bwd_varlen", ext, args, (flags, None, C.byref(need), _stream(q))),
          "attn_bwd_varlen")
    ws = _workspace(need.value, dev)
    have = C.c_size_t(ws.numel())
    check(_call(lib, "attn_bwd_varlen", ext, args, (flags, _ptr(ws), C.byref(have), _stream(q))),
          "attn_bwd_varlen")
    return dq, dk, dv


# ---------------------------------------------------------------------------
# lse merge of two partial results of the same rows
# ---------------------------------------------------------------------------
def merge(out_a, lse_a, out_b, lse_b, out=None, lse=None, bf16_copy: bool = False,
          copy_dtype=None):
    """fp32 (out [rows, H, Dv], lse [H, rows]) of two partial results, plus a
    16-bit copy of out (to feed the backward) in copy_dtype (bfloat16 or
    float16; bf16_copy=True means bfloat16), else None. out/lse may be given
    (e.g. aliasing fp32 out_a / lse_a as running accumulators)."""
    rows, H, Dv = out_a.shape
    codes = {torch.bfloat16: ATTN_BF16, torch.float32: ATTN_F32, torch.float16: ATTN_F16}
    for name, t in (("out_a", out_a), ("out_b", out_b)):
        if t.device.type != "cuda" or t.dtype not in codes:
            raise ValueError(f"{name} must be a bf16, fp16 or fp32 GPU tensor")
        if tuple(t.shape) != (rows, H, Dv) or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous [rows, H, Dv]")
    for name, t in (("lse_a", lse_a), ("lse_b", lse_b)):
        if t.dtype != torch.float32 or tuple(t.shape) != (H, rows) or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous fp32 [H, rows]")
        if t.device != out_a.device:
            raise ValueError("all merge tensors must be on one device")
    dev = out_a.device
    if out is None:
        out = torch.empty((rows, H, Dv), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((H, rows), dtype=torch.float32, device=dev)
    if out.dtype != torch.float32 or tuple(out.shape) != (rows, H, Dv) or not out.is_contiguous():
        raise ValueError("out must be contiguous fp32 [rows, H, Dv]")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (H, rows) or not lse.is_contiguous():
        raise ValueError("lse must be contiguous fp32 [H, rows]")
    if copy_dtype is None and bf16_copy:
        copy_dtype = torch.bfloat16
    if copy_dtype is not None and copy_dtype not in _DTYPES:
        raise ValueError("copy_dtype must be bfloat16 or float16")
    ob = torch.empty((rows, H, Dv), dtype=copy_dtype, device=dev) if copy_dtype else None
    st = load().attn_merge(_ptr(out_a), codes[out_a.dtype], _ptr(lse_a), _ptr(out_b),
                           codes[out_b.dtype], _ptr(lse_b), _ptr(out), _ptr(lse), _ptr(ob),
                           _DTYPES[copy_dtype] if copy_dtype else ATTN_BF16, rows, H, Dv,
                           _stream(out_a))
    check(st, "attn_merge")
    return out, lse, ob


# ---------------------------------------------------------------------------
# document-causal segment layout (host)
# ---------------------------------------------------------------------------
def doc_segments(doc_ids, q_start: int, q_len: int, k_start: int, k_len: int, mode: int):
    """Per-segment (query lengths, key lengths) of the document-causal layout
    (mode 0: causal, keys cover the queries; mode 1: keys before queries)."""
    ids = np.ascontiguousarray(np.asarray(doc_ids, dtype=np.int32))
    if ids.ndim != 2:
        raise ValueError("doc_ids is [B, S]")
    B, S = ids.shape
    lib = load()
    n = C.c_int(0)
    cap = 2 * S * max(B, 1) + 2
    sq = (C.c_int32 * cap)()
    sk = (C.c_int32 * cap)()
    st = lib.attn_doc_segments(ids.ctypes.data_as(C.POINTER(C.c_int32)), B, S, q_start, q_len,
                               k_start, k_len, mode, sq, sk, cap, C.byref(n))
    check(st, "attn_doc_segments")
    return list(sq[:n.value]), list(sk[:n.value])


def doc_cu_seqlens(doc_ids, q_start: int, q_len: int, k_start: int, k_len: int, mode: int):
    """(cu_q, cu_k host int32 numpy arrays, max_q, max_k) of doc_segments'
    layout, as the library writes them."""
    ids = np.ascontiguousarray(np.asarray(doc_ids, dtype=np.int32))
    if ids.ndim != 2:
        raise ValueError("doc_ids is [B, S]")
    B, S = ids.shape
    cap = 2 * S * max(B, 1) + 2
    cu_q = np.zeros(cap + 1, dtype=np.int32)
    cu_k = np.zeros(cap + 1, dtype=np.int32)
    n, mq, mk = C.c_int(0), C.c_int(0), C.c_int(0)
    i32p = C.POINTER(C.c_int32)
    st = load().attn_doc_cu_seqlens(ids.ctypes.data_as(i32p), B, S, q_start, q_len, k_start, k_len,
                                    mode, cu_q.ctypes.data_as(i32p), cu_k.ctypes.data_as(i32p),
                                    cap, C.byref(n), C.byref(mq), C.byref(mk))
    check(st, "attn_doc_cu_seqlens")
    return cu_q[:n.value + 1].copy(), cu_k[:n.value + 1].copy(), mq.value, mk.value


def doc_layout(doc_ids, q_start: int, q_len: int, k_start: int, k_len: int, mode: int, device):
    """(cu_q, cu_k int32 on device, max_q, max_k) of doc_segments' layout."""
    cu_q, cu_k, mq, mk = doc_cu_seqlens(doc_ids, q_start, q_len, k_start, k_len, mode)
    return torch.from_numpy(cu_q).to(device), torch.from_numpy(cu_k).to(device), mq, mk


def dense_route(doc_ids, q_start: int, q_len: int, k_start: int, k_len: int, mode: int):
    """(eligible, pad_rows bool [B, q_len]) of one ring chunk: whether it can
    run on the dense kernels over the raw [B, H, S, D] rows (mode 0 causal
    local chunk, mode 1 non-causal cross chunk), and which of its queries are
    padding (to zero with zero_rows after the dense forward)."""
    ids = np.ascontiguousarray(np.asarray(doc_ids, dtype=np.int32))
    if ids.ndim != 2:
        raise ValueError("doc_ids is [B, S]")
    B, S = ids.shape
    pad = np.zeros((B, max(q_len, 0)), dtype=np.uint8)
    ok = C.c_int(0)
    check(load().attn_dense_route(ids.ctypes.data_as(C.POINTER(C.c_int32)), B, S, q_start, q_len,
                                  k_start, k_len, mode, pad.ctypes.data_as(C.c_void_p),
                                  C.byref(ok)), "attn_dense_route")
    return bool(ok.value), pad.astype(bool)


def zero_rows(out, lse, rows):
    """In place: out[b, :, i, :] = 0 and lse[b, :, i] = -inf where rows[b, i]
    (out a [B, H, S, D] bf16 or fp32 view, lse contiguous [B, H, S] fp32 or
    None, rows bool/uint8 [B, S] on the same GPU)."""
    if out.dim() != 4 or out.stride(3) != 1 or out.dtype not in (torch.bfloat16, torch.float16,
                                                                     torch.float32):
        raise ValueError("out must be a [B, H, S, D] bf16/fp16/fp32 view with unit last stride")
    B, H, S, D = out.shape
    if tuple(rows.shape) != (B, S) or rows.device != out.device:
        raise ValueError("rows must be [B, S] on the device of out")
    r = rows.to(torch.uint8).contiguous()
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, S)
                            or not lse.is_contiguous()):
        raise ValueError("lse must be contiguous fp32 [B, H, S]")
    dt = {torch.float32: ATTN_F32, torch.float16: ATTN_F16}.get(out.dtype, ATTN_BF16)
    ls = (H * S, S) if lse is not None else (0, 0)
    check(load().attn_zero_rows(_ptr(out), dt, out.stride(0), out.stride(1), out.stride(2),
                                _ptr(lse), ls[0], ls[1], _ptr(r), B, H, S, D, _stream(out)),
          "attn_zero_rows")
    return out, lse


# ---------------------------------------------------------------------------
# kernel timing (profiling aid)
# ---------------------------------------------------------------------------
def timing_enable(enable: bool = True) -> bool:
    """Record HIP events around every library kernel launched from this thread."""
    return bool(load().attn_timing_enable(int(bool(enable))))


def timing_read(max_records: int = 4096):
    """[(kernel label, ms)] of the launches recorded since the last read."""
    lib = load()
    name_len = 32
    names = C.create_string_buffer(max_records * name_len)
    ms = (C.c_float * max_records)()
    n = C.c_int(0)
    check(lib.attn_timing_read(max_records, names, name_len, ms, C.byref(n)), "attn_timing_read")
    raw = names.raw
    out = []
    for i in range(min(n.value, max_records)):
        label = raw[i * name_len:(i + 1) * name_len].split(b"\0", 1)[0].decode()
        out.append((label, float(ms[i])))
    return out


# ---------------------------------------------------------------------------
# packed ring layout: gather indices, row moves, live-row merge
# ---------------------------------------------------------------------------
_ROW_TYPES = {torch.bfloat16: ATTN_BF16, torch.float16: ATTN_F16, torch.float32: ATTN_F32}


def ring_segments(q_ids, k_ids, device=None):
    """The per-document segments a query shard ([B, Sq] ids) shares with one
    KV chunk ([B, Sk] ids), as gather indices into B*Sq / B*Sk plus
    cu_seqlens; None when no document is shared. With `device`, the index and
    cu arrays come back as int32 tensors there, else as numpy arrays."""
    qi = np.ascontiguousarray(np.asarray(q_ids, dtype=np.int32))
    ki = np.ascontiguousarray(np.asarray(k_ids, dtype=np.int32))
    if qi.ndim != 2 or ki.ndim != 2 or qi.shape[0] != ki.shape[0]:
        raise ValueError("q_ids [B, Sq] and k_ids [B, Sk] with the same B")
    B, Sq = qi.shape
    Sk = ki.shape[1]
    cap = B * min(Sq, Sk) + 1
    q_index = np.zeros(max(B * Sq, 1), dtype=np.int32)
    k_index = np.zeros(max(B * Sk, 1), dtype=np.int32)
    cu_q = np.zeros(cap + 1, dtype=np.int32)
    cu_k = np.zeros(cap + 1, dtype=np.int32)
    n, tq, tk, mq, mk = (C.c_int(0) for _ in range(5))
    p32 = lambda a: a.ctypes.data_as(C.POINTER(C.c_int32))  # noqa: E731
    check(load().attn_ring_segments(p32(qi), Sq, p32(ki), Sk, B, p32(q_index), p32(k_index),
                                    p32(cu_q), p32(cu_k), cap, C.byref(n), C.byref(tq),
                                    C.byref(tk), C.byref(mq), C.byref(mk)), "attn_ring_segments")
    if n.value == 0:
        return None
    seg = dict(q_index=q_index[:tq.value].copy(), k_index=k_index[:tk.value].copy(),
               cu_q=cu_q[:n.value + 1].copy(), cu_k=cu_k[:n.value + 1].copy(),
               max_q=mq.value, max_k=mk.value)
    if device is not None:
        for key in ("q_index", "k_index", "cu_q", "cu_k"):
            seg[key] = torch.from_numpy(seg[key]).to(device)
    return seg


def ring_inplace_preferred(live_rows: int, B: int, S: int, H: int, D: int,
                           dtype=torch.bfloat16) -> bool:
    """Whether merging a chunk's live rows in place beats scattering them."""
    return bool(load().attn_ring_inplace_preferred(int(live_rows), int(B), int(S), int(H), int(D),
                                                   _ROW_TYPES[dtype]))


def _index(index, dev):
    if index.dtype != torch.int32 or index.device != dev or index.dim() != 1 or \
            not index.is_contiguous():
        raise ValueError("index must be contiguous int32 [T] on the device")
    return C.c_void_p(index.data_ptr()) if index.numel() else C.c_void_p(0)


def _dense4(x, name):
    if x.dim() != 4 or x.dtype not in _ROW_TYPES or x.device.type != "cuda" or \
            (x.numel() and x.stride(3) != 1):
        raise ValueError(f"{name} must be a [B, H, S, D] GPU view with unit last stride")
    return x


def gather_rows(src, index, dtype=None):
    """[B, H, S, D] view -> packed [T, H, D] rows at flat indices b*S + s
    (dtype: the packed type; fp32 rows may be rounded to bf16 / fp16)."""
    _dense4(src, "src")
    B, H, S, D = src.shape
    dt = src.dtype if dtype is None else dtype
    out = torch.empty((index.numel(), H, D), dtype=dt, device=src.device)
    check(load().attn_gather_rows(_ROW_TYPES[src.dtype], _ptr(src), src.stride(0), src.stride(1),
                                  src.stride(2), _index(index, src.device), B, H, S, D,
                                  index.numel(), _ptr(out), _ROW_TYPES[dt], _stream(src)),
          "attn_gather_rows")
    return out


def scatter_rows(src, index, dst, mode=0):
    """In place: dst [B, H, S, D] rows at the flat indices receive the packed
    rows src [T, H, D] (mode 0), or every other row is zeroed too (mode 1), or
    src is added to them (mode 2, the gradient scatter-add)."""
    _dense4(dst, "dst")
    B, H, S, D = dst.shape
    if src.dtype != dst.dtype or tuple(src.shape) != (index.numel(), H, D) or \
            not src.is_contiguous() or src.device != dst.device:
        raise ValueError("src must be contiguous [T, H, D] of dst's dtype and device")
    check(load().attn_scatter_rows(_ROW_TYPES[dst.dtype], _ptr(src), _index(index, dst.device),
                                   index.numel(), H, D, _ptr(dst), dst.stride(0), dst.stride(1),
                                   dst.stride(2), B, S, int(mode), _stream(dst)),
          "attn_scatter_rows")
    return dst


def gather_lse(lse, index):
    """Dense [B, H, S] -> packed [H, T] at the flat indices."""
    if lse.dtype != torch.float32 or lse.dim() != 3 or not lse.is_contiguous():
        raise ValueError("lse must be contiguous fp32 [B, H, S]")
    B, H, S = lse.shape
    out = torch.empty((H, index.numel()), dtype=torch.float32, device=lse.device)
    check(load().attn_gather_lse(_ptr(lse), _index(index, lse.device), B, H, S, index.numel(),
                                 _ptr(out), _stream(lse)), "attn_gather_lse")
    return out


def scatter_lse(lse_pack, index, B: int, S: int, out=None):
    """Packed [H, T] -> dense [B, H, S], -inf on rows no index names (or, with
    out given, written into out in place with the other rows kept)."""
    H, T = lse_pack.shape
    if lse_pack.dtype != torch.float32 or not lse_pack.is_contiguous() or T != index.numel():
        raise ValueError("lse_pack must be contiguous fp32 [H, T]")
    fill = out is None
    if out is None:
        out = torch.empty((B, H, S), dtype=torch.float32, device=lse_pack.device)
    elif out.dtype != torch.float32 or tuple(out.shape) != (B, H, S) or not out.is_contiguous():
        raise ValueError("out must be contiguous fp32 [B, H, S]")
    check(load().attn_scatter_lse(_ptr(lse_pack), _index(index, lse_pack.device), T, H, _ptr(out),
                                  B, S, int(fill), _stream(lse_pack)), "attn_scatter_lse")
    return out


def merge_rows(out_acc, lse_acc, out_b, lse_b, index):
    """In place: merge one chunk's packed rows (out_b [T, H, D], lse_b [H, T])
    into the running fp32 accumulators out_acc [B, H, S, D] / lse_acc
    [B, H, S] at its flat-index rows only."""
    _dense4(out_acc, "out_acc")
    B, H, S, D = out_acc.shape
    if out_acc.dtype != torch.float32:
        raise ValueError("out_acc must be fp32")
    if lse_acc.dtype != torch.float32 or tuple(lse_acc.shape) != (B, H, S) or \
            not lse_acc.is_contiguous():
        raise ValueError("lse_acc must be contiguous fp32 [B, H, S]")
    T = index.numel()
    if tuple(out_b.shape) != (T, H, D) or not out_b.is_contiguous() or \
            out_b.dtype not in _ROW_TYPES:
        raise ValueError("out_b must be contiguous [T, H, D]")
    if lse_b.dtype != torch.float32 or tuple(lse_b.shape) != (H, T) or not lse_b.is_contiguous():
        raise ValueError("lse_b must be contiguous fp32 [H, T]")
    check(load().attn_merge_rows(_ptr(out_acc), out_acc.stride(0), out_acc.stride(1),
                                 out_acc.stride(2), _ptr(lse_acc), B, S, _ptr(out_b),
                                 _ROW_TYPES[out_b.dtype], _ptr(lse_b),
                                 _index(index, out_acc.device), T, H, D, _stream(out_acc)),
          "attn_merge_rows")
    return out_acc, lse_acc
