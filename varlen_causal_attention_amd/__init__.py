"""MI355X (gfx950) fused scaled-dot-product attention: forward and backward,
dense [B,H,N,D] and packed-THD varlen, GQA, bottom-right causal masks,
head dims up to 512 and unequal QK/V head dims, plus the online-softmax lse
merge of two partial results and the dense routing of ring chunks. All computation runs in the HIP library
libvca_attn.so (built in-tree by ``python -m varlen_causal_attention_amd.build``);
this package only marshals torch tensors into its C ABI.
"""
from ._lib import EXPORTED, LIB_PATH, AttnError, load
from .ops import (bwd_dense, bwd_varlen, dense_route, doc_cu_seqlens, doc_layout, doc_segments,
                  fwd_dense, fwd_varlen, fwd_varlen_noalloc, gather_lse, gather_rows,
                  is_supported, merge, merge_rows, ring_inplace_preferred, ring_segments,
                  scatter_lse, scatter_rows, timing_enable, timing_read, version, zero_rows)

__all__ = [
    "AttnError", "EXPORTED", "LIB_PATH", "load", "fwd_dense", "fwd_varlen", "fwd_varlen_noalloc",
    "bwd_dense", "bwd_varlen", "merge", "doc_segments", "doc_cu_seqlens", "doc_layout",
    "dense_route", "zero_rows", "ring_segments", "ring_inplace_preferred", "gather_rows",
    "scatter_rows", "gather_lse", "scatter_lse", "merge_rows",
    "is_supported", "version", "timing_enable", "timing_read",
]
