"""ctypes binding of libshortconv.so (argument marshalling only: every step runs in the library).

Torch is used for device memory and streams: tensors are passed as raw device pointers and the
current torch stream of their device is passed as the hipStream_t. The library must be built
(``python -m causal_short_convolution_amd.build``); there is no fallback path of any kind.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY_PATH = os.path.join(_HERE, "libshortconv.so")

SC_DTYPE = {torch.float32: 0, torch.bfloat16: 1}
ERRORS = {-1: "SC_ERR_INVALID", -2: "SC_ERR_UNSUPPORTED", -3: "SC_ERR_HIP"}

_lib = None


class ShortConvError(RuntimeError):
    """A non-zero return of the C ABI (message from shortconv_last_error)."""

    def __init__(self, code: int, message: str):
        super().__init__(f"{ERRORS.get(code, code)}: {message}")
        self.code = code


def load_library(path: str = LIBRARY_PATH):
    """Load the built library (raises if it is missing: there is no other implementation)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is not built; run `python -m causal_short_convolution_amd.build` "
            "(the fused ShortConv K/V step has no implementation other than this HIP library)")
    lib = ctypes.CDLL(path)
    P, I32, I64, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    lib.shortconv_kv_prefill.restype = ctypes.c_int
    lib.shortconv_kv_prefill.argtypes = [P, P, I64, I64, P, I32, I64, P, P, P, P, F, P, P, I64, P,
                                         P, P, P, P, I64, I32, I32, I32, I32, P]
    lib.shortconv_kv_decode.restype = ctypes.c_int
    lib.shortconv_kv_decode.argtypes = [P, P, I64, I64, I32, P, P, P, P, F, P, P, I64, P, P, P, P,
                                        I64, I32, I32, I32, I32, P]
    lib.shortconv_kv_verify.restype = ctypes.c_int
    lib.shortconv_kv_verify.argtypes = [P, P, I64, I64, P, I32, I64, P, P, P, P, F, P, P, I64, P,
                                        P, P, I32, P, P, P, I64, I32, I32, I32, I32, P]
    lib.shortconv_state_commit.restype = ctypes.c_int
    lib.shortconv_state_commit.argtypes = [P, P, I32, P, I64, P, I32, P, P, I64, P, I32, I32, I32,
                                           I32, P]
    lib.shortconv_kv_prefill_mxfp8.restype = ctypes.c_int
    lib.shortconv_kv_prefill_mxfp8.argtypes = [P, P, I64, I64, P, I32, I64, P, P, P, P, F, P, P,
                                               I64, P, P, P, P, P, P, P, I64, I32, I32, I32, I32,
                                               P]
    lib.shortconv_kv_decode_mxfp8.restype = ctypes.c_int
    lib.shortconv_kv_decode_mxfp8.argtypes = [P, P, I64, I64, I32, P, P, P, P, F, P, P, I64, P, P,
                                              P, P, P, P, I64, I32, I32, I32, I32, P]
    lib.shortconv_mxfp8_quantize.restype = ctypes.c_int
    lib.shortconv_mxfp8_quantize.argtypes = [P, I64, I64, I32, I32, I32, P, P, P]
    lib.shortconv_kv_backward.restype = ctypes.c_int
    lib.shortconv_kv_backward.argtypes = [P, P, I64, I64, P, I32, I64, P, P, P, P, F, P, P, I64,
                                          P, P, P, P, P, P, P, P, P, P, P, P, P, P, P,
                                          ctypes.c_size_t, I32, I32, I32, I32, P]
    lib.shortconv_kv_backward_workspace_size.restype = ctypes.c_size_t
    lib.shortconv_kv_backward_workspace_size.argtypes = [I64, I32, I32, I32, I32, I32]
    lib.shortconv_last_error.restype = ctypes.c_char_p
    lib.shortconv_last_error.argtypes = []
    lib.shortconv_abi_version.restype = ctypes.c_int
    lib.shortconv_abi_version.argtypes = []
    _lib = lib
    return lib


def last_error() -> str:
    return load_library().shortconv_last_error().decode()


def abi_version() -> int:
    return int(load_library().shortconv_abi_version())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _rows(x: torch.Tensor, name: str):
    """[tokens, H, D] with contiguous (H, D); returns the token stride in elements."""
    if x.dim() != 3 or x.stride(2) != 1 or x.stride(1) != x.shape[2]:
        raise ValueError(f"{name} must be [tokens, heads, head_dim] with contiguous heads/head_dim")
    return x.stride(0) if x.shape[0] > 1 else x.shape[1] * x.shape[2]


def _stream_handle(device, stream):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _check(rc: int):
    if rc != 0:
        raise ShortConvError(rc, last_error())


def shortconv_kv_prefill(k, v, cu_seqlens, k_taps, v_taps, k_gamma, v_gamma, eps, k_state, v_state,
                         state_idx, has_initial_state, slot_mapping, k_cache, v_cache, *,
                         stream: Optional[torch.cuda.Stream] = None) -> None:
    """Fused ShortConv K/V prefill over packed sequences (see include/shortconv.h).

    k, v [T,H,D] (fp32 or bf16); cu_seqlens int32 [N+1]; taps fp32 [W,H,D]; gamma fp32 [D];
    k_state/v_state [S,W-1,H,D] or None (W == 1); state_idx int32 [N] or None;
    has_initial_state uint8/bool [N] or None; slot_mapping int64 [T]; caches [num_slots,H,D].
    """
    lib = load_library()
    W, H, D = k_taps.shape
    if has_initial_state is not None and has_initial_state.dtype == torch.bool:
        has_initial_state = has_initial_state.view(torch.uint8)
    S = k_state.shape[0] if k_state is not None else 0
    with torch.cuda.device(k.device):
        rc = lib.shortconv_kv_prefill(
            _ptr(k), _ptr(v), _rows(k, "k"), _rows(v, "v"), _ptr(cu_seqlens),
            cu_seqlens.shape[0] - 1, k.shape[0], _ptr(k_taps), _ptr(v_taps), _ptr(k_gamma),
            _ptr(v_gamma), float(eps), _ptr(k_state), _ptr(v_state), S, _ptr(state_idx),
            _ptr(has_initial_state), _ptr(slot_mapping), _ptr(k_cache), _ptr(v_cache),
            k_cache.shape[0], H, D, W, SC_DTYPE[k.dtype], _stream_handle(k.device, stream))
    _check(rc)


def shortconv_kv_decode(k_new, v_new, k_taps, v_taps, k_gamma, v_gamma, eps, k_state, v_state,
                        state_idx, slot_mapping, k_cache, v_cache, *,
                        stream: Optional[torch.cuda.Stream] = None) -> None:
    """Fused ShortConv K/V decode, one new token per sequence (see include/shortconv.h)."""
    lib = load_library()
    W, H, D = k_taps.shape
    S = k_state.shape[0] if k_state is not None else 0
    with torch.cuda.device(k_new.device):
        rc = lib.shortconv_kv_decode(
            _ptr(k_new), _ptr(v_new), _rows(k_new, "k_new"), _rows(v_new, "v_new"),
            k_new.shape[0], _ptr(k_taps), _ptr(v_taps), _ptr(k_gamma), _ptr(v_gamma), float(eps),
            _ptr(k_state), _ptr(v_state), S, _ptr(state_idx), _ptr(slot_mapping), _ptr(k_cache),
            _ptr(v_cache), k_cache.shape[0], H, D, W, SC_DTYPE[k_new.dtype],
            _stream_handle(k_new.device, stream))
    _check(rc)


def shortconv_kv_verify(k, v, cu_seqlens, k_taps, v_taps, k_gamma, v_gamma, eps, k_state, v_state,
                        state_idx, k_snap, v_snap, slot_mapping, k_cache, v_cache, *,
                        stream: Optional[torch.cuda.Stream] = None) -> None:
    """Speculative verification (see include/shortconv.h): outputs as a prefill that resumes
    every sequence from its stored state; pools read only; per-token states go to
    k_snap/v_snap [N, max_tokens, W-1, H, D] (None when W == 1)."""
    lib = load_library()
    W, H, D = k_taps.shape
    S = k_state.shape[0] if k_state is not None else 0
    max_tokens = k_snap.shape[1] if k_snap is not None else 1
    with torch.cuda.device(k.device):
        rc = lib.shortconv_kv_verify(
            _ptr(k), _ptr(v), _rows(k, "k"), _rows(v, "v"), _ptr(cu_seqlens),
            cu_seqlens.shape[0] - 1, k.shape[0], _ptr(k_taps), _ptr(v_taps), _ptr(k_gamma),
            _ptr(v_gamma), float(eps), _ptr(k_state), _ptr(v_state), S, _ptr(state_idx),
            _ptr(k_snap), _ptr(v_snap), max_tokens, _ptr(slot_mapping), _ptr(k_cache),
            _ptr(v_cache), k_cache.shape[0], H, D, W, SC_DTYPE[k.dtype],
            _stream_handle(k.device, stream))
    _check(rc)


def shortconv_state_commit(k_snap, v_snap, cu_seqlens, total_tokens, accepted, k_state, v_state,
                           state_idx, *, width, num_heads, head_dim,
                           stream: Optional[torch.cuda.Stream] = None) -> None:
    """Install the accepted prefix's snapshot in the state pools (see include/shortconv.h)."""
    lib = load_library()
    S = k_state.shape[0] if k_state is not None else 0
    max_tokens = k_snap.shape[1] if k_snap is not None else 1
    dev = k_state.device if k_state is not None else accepted.device
    dtype = k_state.dtype if k_state is not None else torch.bfloat16
    with torch.cuda.device(dev):
        rc = lib.shortconv_state_commit(
            _ptr(k_snap), _ptr(v_snap), max_tokens, _ptr(cu_seqlens), int(total_tokens),
            _ptr(accepted), cu_seqlens.shape[0] - 1, _ptr(k_state), _ptr(v_state), S,
            _ptr(state_idx), num_heads, head_dim, width, SC_DTYPE[dtype],
            _stream_handle(dev, stream))
    _check(rc)


def shortconv_kv_prefill_mxfp8(k, v, cu_seqlens, k_taps, v_taps, k_gamma, v_gamma, eps, k_state,
                               v_state, state_idx, has_initial_state, slot_mapping, k_codes,
                               v_codes, k_scales, v_scales, *,
                               stream: Optional[torch.cuda.Stream] = None) -> None:
    """Prefill writing MXFP8 cache rows: codes uint8 [num_slots,H,D], scales uint8
    [num_slots,H,D/32] (see include/shortconv.h)."""
    lib = load_library()
    W, H, D = k_taps.shape
    if has_initial_state is not None and has_initial_state.dtype == torch.bool:
        has_initial_state = has_initial_state.view(torch.uint8)
    S = k_state.shape[0] if k_state is not None else 0
    with torch.cuda.device(k.device):
        rc = lib.shortconv_kv_prefill_mxfp8(
            _ptr(k), _ptr(v), _rows(k, "k"), _rows(v, "v"), _ptr(cu_seqlens),
            cu_seqlens.shape[0] - 1, k.shape[0], _ptr(k_taps), _ptr(v_taps), _ptr(k_gamma),
            _ptr(v_gamma), float(eps), _ptr(k_state), _ptr(v_state), S, _ptr(state_idx),
            _ptr(has_initial_state), _ptr(slot_mapping), _ptr(k_codes), _ptr(v_codes),
            _ptr(k_scales), _ptr(v_scales), k_codes.shape[0], H, D, W, SC_DTYPE[k.dtype],
            _stream_handle(k.device, stream))
    _check(rc)


def shortconv_kv_decode_mxfp8(k_new, v_new, k_taps, v_taps, k_gamma, v_gamma, eps, k_state,
                              v_state, state_idx, slot_mapping, k_codes, v_codes, k_scales,
                              v_scales, *, stream: Optional[torch.cuda.Stream] = None) -> None:
    """Decode writing MXFP8 cache rows (see include/shortconv.h)."""
    lib = load_library()
    W, H, D = k_taps.shape
    S = k_state.shape[0] if k_state is not None else 0
    with torch.cuda.device(k_new.device):
        rc = lib.shortconv_kv_decode_mxfp8(
            _ptr(k_new), _ptr(v_new), _rows(k_new, "k_new"), _rows(v_new, "v_new"),
            k_new.shape[0], _ptr(k_taps), _ptr(v_taps), _ptr(k_gamma), _ptr(v_gamma), float(eps),
            _ptr(k_state), _ptr(v_state), S, _ptr(state_idx), _ptr(slot_mapping), _ptr(k_codes),
            _ptr(v_codes), _ptr(k_scales), _ptr(v_scales), k_codes.shape[0], H, D, W,
            SC_DTYPE[k_new.dtype], _stream_handle(k_new.device, stream))
    _check(rc)


def shortconv_mxfp8_quantize(x, codes, scales, *,
                             stream: Optional[torch.cuda.Stream] = None) -> None:
    """MXFP8-quantize rows x [rows,H,D] into codes [rows,H,D] and scales [rows,H,D/32] (uint8)."""
    lib = load_library()
    rows, H, D = x.shape
    with torch.cuda.device(x.device):
        rc = lib.shortconv_mxfp8_quantize(_ptr(x), _rows(x, "x"), rows, H, D, SC_DTYPE[x.dtype],
                                          _ptr(codes), _ptr(scales),
                                          _stream_handle(x.device, stream))
    _check(rc)


def shortconv_kv_backward_workspace_size(total_tokens, num_seqs, num_heads, head_dim, width,
                                         dtype) -> int:
    """Bytes of workspace ``shortconv_kv_backward`` needs (see include/shortconv.h)."""
    lib = load_library()
    code = SC_DTYPE[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    n = lib.shortconv_kv_backward_workspace_size(int(total_tokens), int(num_seqs), int(num_heads),
                                                 int(head_dim), int(width), code)
    if n == ctypes.c_size_t(-1).value:
        raise ShortConvError(-1, last_error())
    return int(n)


def shortconv_kv_backward(k, v, cu_seqlens, k_taps, v_taps, k_gamma, v_gamma, eps, k_state,
                          v_state, state_idx, has_initial_state, dy_k, dy_v, dk, dv, dk_taps,
                          dv_taps, dk_gamma, dv_gamma, *, dstate_out=(None, None),
                          dstate_in=(None, None), workspace: Optional[torch.Tensor] = None,
                          stream: Optional[torch.cuda.Stream] = None) -> None:
    """Gradients of the prefill step (see include/shortconv.h): from dy_k/dy_v (and optionally the
    new-state gradients ``dstate_out``) into dk/dv, the tap and gamma gradients and optionally the
    initial-window gradients ``dstate_in``. ``workspace`` (uint8 device tensor) is allocated here
    when not given."""
    lib = load_library()
    W, H, D = k_taps.shape
    N = cu_seqlens.shape[0] - 1
    T = k.shape[0]
    S = k_state.shape[0] if k_state is not None else 0
    need = shortconv_kv_backward_workspace_size(T, N, H, D, W, k.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=k.device)
    with torch.cuda.device(k.device):
        rc = lib.shortconv_kv_backward(
            _ptr(k), _ptr(v), _rows(k, "k"), _rows(v, "v"), _ptr(cu_seqlens), N, T, _ptr(k_taps),
            _ptr(v_taps), _ptr(k_gamma), _ptr(v_gamma), float(eps), _ptr(k_state), _ptr(v_state),
            S, _ptr(state_idx), _ptr(has_initial_state), _ptr(dy_k), _ptr(dy_v),
            _ptr(dstate_out[0]), _ptr(dstate_out[1]), _ptr(dk), _ptr(dv), _ptr(dk_taps),
            _ptr(dv_taps), _ptr(dk_gamma), _ptr(dv_gamma), _ptr(dstate_in[0]), _ptr(dstate_in[1]),
            _ptr(workspace), workspace.numel() * workspace.element_size(), H, D, W,
            SC_DTYPE[k.dtype], _stream_handle(k.device, stream))
    _check(rc)
