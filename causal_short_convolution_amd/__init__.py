"""Fused ShortConv K/V step for AMD Instinct MI355X (gfx950).

Causal depthwise convolution over tokens of the projected K and V, per-head RMSNorm, paged
KV-cache write and rolling conv-state update, in one HIP kernel per call; plus speculative
verification with per-token conv-state snapshots and the commit of an accepted prefix, and
variants that write MXFP8 (OCP microscaling) cache rows, and the backward of the step for
training (``shortconv_kv``: the step as a differentiable torch op). The compute lives in
``libshortconv.so`` (C ABI, ``include/shortconv.h``); this package only marshals torch tensors.
"""
from ._binding import (LIBRARY_PATH, ShortConvError, abi_version, last_error, load_library,
                       NOALLOC_SCRATCH_BYTES, shortconv_kv_backward,
                       shortconv_kv_backward_noalloc, shortconv_kv_backward_workspace_size,
                       shortconv_kv_decode, shortconv_kv_decode_mxfp8, shortconv_kv_prefill,
                       shortconv_kv_prefill_mxfp8, shortconv_kv_verify, shortconv_mxfp8_quantize,
                       shortconv_state_commit)
from .autograd import shortconv_kv

__all__ = [
    "LIBRARY_PATH",
    "ShortConvError",
    "shortconv_kv",
    "abi_version",
    "last_error",
    "load_library",
    "NOALLOC_SCRATCH_BYTES",
    "shortconv_kv_backward",
    "shortconv_kv_backward_noalloc",
    "shortconv_kv_backward_workspace_size",
    "shortconv_kv_decode",
    "shortconv_kv_decode_mxfp8",
    "shortconv_kv_prefill",
    "shortconv_kv_prefill_mxfp8",
    "shortconv_mxfp8_quantize",
    "shortconv_kv_verify",
    "shortconv_state_commit",
]
