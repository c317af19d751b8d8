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
    lib.shortconv_kv_backward_noalloc.restype = ctypes.c_int
    lib.shortconv_kv_backward_noalloc.argtypes = [P, P, I64, I64, P, I32, I64, P, P, P, P, F, P, P,
                                                  I64, P, P, P, P, P, P, P, P, P, P, P, P, P, P,
                                                  I32, I32, I32, I32, P]
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


# ------------------------------------------------------------------------------------------------
# Argument checks. The library checks sizes, strides and alignment of what it is told, but it is
# told only pointers and sizes: a tensor of the wrong element type, shape or layout would be read
# or written past its end on the device. So every tensor is checked here, before the library is
# loaded or called, and a mismatch raises ValueError naming the argument.
# ------------------------------------------------------------------------------------------------
class _Args:
    """Collects the tensors of one call and checks each against what the C ABI expects."""

    def __init__(self, fn: str):
        self.fn = fn
        self.device = None

    def fail(self, msg: str):
        raise ValueError(f"{self.fn}: {msg}")

    def _device(self, t: torch.Tensor, name: str):
        if self.device is None:
            self.device = t.device
        elif t.device != self.device:
            self.fail(f"{name} is on {t.device}, other arguments on {self.device}")

    def tensor(self, t, name, dtypes, shape, *, optional=False, contiguous=True):
        """t must be a tensor with dtype in `dtypes` and the given shape (None = any extent),
        contiguous unless told otherwise, on the same device as the others."""
        if t is None:
            if optional:
                return None
            self.fail(f"{name} is required")
        if not isinstance(t, torch.Tensor):
            self.fail(f"{name} must be a torch.Tensor, got {type(t).__name__}")
        if t.dtype not in dtypes:
            want = " or ".join(str(d) for d in dtypes)
            self.fail(f"{name} must be {want}, got {t.dtype}")
        if t.dim() != len(shape) or any(s is not None and s != n for s, n in zip(shape, t.shape)):
            want = "[" + ", ".join("*" if s is None else str(s) for s in shape) + "]"
            self.fail(f"{name} must have shape {want}, got {list(t.shape)}")
        if contiguous and not t.is_contiguous():
            self.fail(f"{name} must be contiguous")
        self._device(t, name)
        return t

    def rows(self, t, name, H=None, D=None, dtypes=(torch.float32, torch.bfloat16)):
        """[tokens, H, D] rows with contiguous (H, D) and any token stride; returns the token
        stride in elements."""
        self.tensor(t, name, dtypes, (None, H, D), contiguous=False)
        if t.stride(2) != 1 or t.stride(1) != t.shape[2] or (t.shape[0] > 1 and t.stride(0) < 1):
            self.fail(f"{name} must be [tokens, heads, head_dim] with contiguous heads/head_dim")
        return t.stride(0) if t.shape[0] > 1 else t.shape[1] * t.shape[2]

    def on_gpu(self):
        if self.device is not None and self.device.type != "cuda":
            self.fail(f"tensors must be on a GPU, got {self.device}")


_I32, _I64, _U8, _F32 = (torch.int32,), (torch.int64,), (torch.uint8,), (torch.float32,)
_FLAGS = (torch.uint8, torch.bool)


def _step_common(a: _Args, k, v, k_taps, v_taps, k_gamma, v_gamma, k_state, v_state):
    """K/V rows, parameters and state pools shared by the prefill, decode and verify calls.
    Returns (W, H, D, k stride, v stride, number of state slots)."""
    ks = a.rows(k, "k")
    H, D = k.shape[1], k.shape[2]
    vs = a.rows(v, "v", H, D, (k.dtype,))
    if v.shape[0] != k.shape[0]:
        a.fail(f"k and v must have the same number of tokens, got {k.shape[0]} and {v.shape[0]}")
    a.tensor(k_taps, "k_taps", _F32, (None, H, D))
    W = k_taps.shape[0]
    a.tensor(v_taps, "v_taps", _F32, (W, H, D))
    a.tensor(k_gamma, "k_gamma", _F32, (D,))
    a.tensor(v_gamma, "v_gamma", _F32, (D,))
    S = _state_pools(a, k_state, v_state, W, H, D, k.dtype)
    return W, H, D, ks, vs, S


def _state_pools(a: _Args, k_state, v_state, W, H, D, dtype, names=("k_state", "v_state")):
    """Both state pools [S, W-1, H, D] of the row dtype, or both None; returns S (0 for None)."""
    if (k_state is None) != (v_state is None):
        a.fail(f"{names[0]} and {names[1]} must both be given or both be None")
    if k_state is None:
        return 0
    a.tensor(k_state, names[0], (dtype,), (None, W - 1, H, D))
    a.tensor(v_state, names[1], (dtype,), (k_state.shape[0], W - 1, H, D))
    return k_state.shape[0]


def _caches(a: _Args, k_cache, v_cache, H, D, dtype):
    a.tensor(k_cache, "k_cache", (dtype,), (None, H, D))
    a.tensor(v_cache, "v_cache", (dtype,), (k_cache.shape[0], H, D))
    return k_cache.shape[0]


def _mx_caches(a: _Args, k_codes, v_codes, k_scales, v_scales, H, D):
    a.tensor(k_codes, "k_codes", _U8, (None, H, D))
    n = k_codes.shape[0]
    a.tensor(v_codes, "v_codes", _U8, (n, H, D))
    a.tensor(k_scales, "k_scales", _U8, (n, H, D // 32))
    a.tensor(v_scales, "v_scales", _U8, (n, H, D // 32))
    return n


def _flags(t):
    return t.view(torch.uint8) if t is not None and t.dtype == torch.bool else t


def _stream_handle(device, stream):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _check(rc: int):
    if rc != 0:
        raise ShortConvError(rc, last_error())


def _prefill_args(fn, k, v, cu_seqlens, k_taps, v_taps, k_gamma, v_gamma, k_state, v_state,
                  state_idx, has_initial_state, slot_mapping):
    """Checks shared by the prefill entry points; returns (args, W, H, D, ks, vs, S, N)."""
    a = _Args(fn)
    W, H, D, ks, vs, S = _step_common(a, k, v, k_taps, v_taps, k_gamma, v_gamma, k_state, v_state)
    a.tensor(cu_seqlens, "cu_seqlens", _I32, (None,))
    N = cu_seqlens.shape[0] - 1
    if N < 0:
        a.fail("cu_seqlens must hold at least one entry (num_seqs + 1)")
    a.tensor(state_idx, "state_idx", _I32, (N,), optional=True)
    a.tensor(has_initial_state, "has_initial_state", _FLAGS, (N,), optional=True)
    a.tensor(slot_mapping, "slot_mapping", _I64, (k.shape[0],))
    return a, W, H, D, ks, vs, S, N


def shortconv_kv_prefill(k, v, cu_seqlens, k_taps, v_taps, k_gamma, v_gamma, eps, k_state, v_state,
                         state_idx, has_initial_state, slot_mapping, k_cache, v_cache, *,
                         stream: Optional[torch.cuda.Stream] = None) -> None:
    """Fused ShortConv K/V prefill over packed sequences (see include/shortconv.h).

    k, v [T,H,D] (fp32 or bf16, contiguous heads/head_dim, any token stride); cu_seqlens int32
    [N+1]; taps fp32 [W,H,D]; gamma fp32 [D]; k_state/v_state [S,W-1,H,D] of k's dtype, or both
    None (no state slots); state_idx int32 [N] or None; has_initial_state uint8/bool [N] or None;
    slot_mapping int64 [T]; caches [num_slots,H,D] of k's dtype. Every tensor on one GPU; a
    mismatch raises ValueError before anything is launched.
    """
    a, W, H, D, ks, vs, S, N = _prefill_args("shortconv_kv_prefill", k, v, cu_seqlens, k_taps,
                                             v_taps, k_gamma, v_gamma, k_state, v_state,
                                             state_idx, has_initial_state, slot_mapping)
    nslots = _caches(a, k_cache, v_cache, H, D, k.dtype)
    a.on_gpu()
    lib = load_library()
    with torch.cuda.device(k.device):
        rc = lib.shortconv_kv_prefill(
            _ptr(k), _ptr(v), ks, vs, _ptr(cu_seqlens), N, k.shape[0], _ptr(k_taps), _ptr(v_taps),
            _ptr(k_gamma), _ptr(v_gamma), float(eps), _ptr(k_state), _ptr(v_state), S,
            _ptr(state_idx), _ptr(_flags(has_initial_state)), _ptr(slot_mapping), _ptr(k_cache),
            _ptr(v_cache), nslots, H, D, W, SC_DTYPE[k.dtype], _stream_handle(k.device, stream))
    _check(rc)


def _decode_args(fn, k_new, v_new, k_taps, v_taps, k_gamma, v_gamma, k_state, v_state, state_idx,
                 slot_mapping):
    a = _Args(fn)
    W, H, D, ks, vs, S = _step_common(a, k_new, v_new, k_taps, v_taps, k_gamma, v_gamma, k_state,
                                      v_state)
    B = k_new.shape[0]
    a.tensor(state_idx, "state_idx", _I32, (B,), optional=True)
    a.tensor(slot_mapping, "slot_mapping", _I64, (B,))
    return a, W, H, D, ks, vs, S, B


def shortconv_kv_decode(k_new, v_new, k_taps, v_taps, k_gamma, v_gamma, eps, k_state, v_state,
                        state_idx, slot_mapping, k_cache, v_cache, *,
                        stream: Optional[torch.cuda.Stream] = None) -> None:
    """Fused ShortConv K/V decode, one new token per sequence (see include/shortconv.h).
    k_new, v_new [B,H,D]; state_idx int32 [B] or None; slot_mapping int64 [B]; the other
    arguments as for shortconv_kv_prefill."""
    a, W, H, D, ks, vs, S, B = _decode_args("shortconv_kv_decode", k_new, v_new, k_taps, v_taps,
                                            k_gamma, v_gamma, k_state, v_state, state_idx,
                                            slot_mapping)
    nslots = _caches(a, k_cache, v_cache, H, D, k_new.dtype)
    a.on_gpu()
    lib = load_library()
    with torch.cuda.device(k_new.device):
        rc = lib.shortconv_kv_decode(
            _ptr(k_new), _ptr(v_new), ks, vs, B, _ptr(k_taps), _ptr(v_taps), _ptr(k_gamma),
            _ptr(v_gamma), float(eps), _ptr(k_state), _ptr(v_state), S, _ptr(state_idx),
            _ptr(slot_mapping), _ptr(k_cache), _ptr(v_cache), nslots, H, D, W,
            SC_DTYPE[k_new.dtype], _stream_handle(k_new.device, stream))
    _check(rc)


def shortconv_kv_verify(k, v, cu_seqlens, k_taps, v_taps, k_gamma, v_gamma, eps, k_state, v_state,
                        state_idx, k_snap, v_snap, slot_mapping, k_cache, v_cache, *,
                        stream: Optional[torch.cuda.Stream] = None) -> None:
    """Speculative verification (see include/shortconv.h): outputs as a prefill that resumes
    every sequence from its stored state; pools read only; per-token states go to
    k_snap/v_snap [N, max_tokens, W-1, H, D] of k's dtype (None when W == 1)."""
    a, W, H, D, ks, vs, S, N = _prefill_args("shortconv_kv_verify", k, v, cu_seqlens, k_taps,
                                             v_taps, k_gamma, v_gamma, k_state, v_state,
                                             state_idx, None, slot_mapping)
    if W > 1 or k_snap is not None or v_snap is not None:
        a.tensor(k_snap, "k_snap", (k.dtype,), (N, None, W - 1, H, D))
        a.tensor(v_snap, "v_snap", (k.dtype,), (N, k_snap.shape[1], W - 1, H, D))
    max_tokens = k_snap.shape[1] if k_snap is not None else 1
    nslots = _caches(a, k_cache, v_cache, H, D, k.dtype)
    a.on_gpu()
    lib = load_library()
    with torch.cuda.device(k.device):
        rc = lib.shortconv_kv_verify(
            _ptr(k), _ptr(v), ks, vs, _ptr(cu_seqlens), N, k.shape[0], _ptr(k_taps), _ptr(v_taps),
            _ptr(k_gamma), _ptr(v_gamma), float(eps), _ptr(k_state), _ptr(v_state), S,
            _ptr(state_idx), _ptr(k_snap), _ptr(v_snap), max_tokens, _ptr(slot_mapping),
            _ptr(k_cache), _ptr(v_cache), nslots, H, D, W, SC_DTYPE[k.dtype],
            _stream_handle(k.device, stream))
    _check(rc)


def shortconv_state_commit(k_snap, v_snap, cu_seqlens, total_tokens, accepted, k_state, v_state,
                           state_idx, *, width, num_heads, head_dim,
                           stream: Optional[torch.cuda.Stream] = None) -> None:
    """Install the accepted prefix's snapshot in the state pools (see include/shortconv.h).
    k_snap/v_snap [N, max_tokens, W-1, H, D]; cu_seqlens int32 [N+1] as given to the verify call;
    accepted int32 [N]; k_state/v_state [S, W-1, H, D] of the snapshots' dtype; state_idx int32
    [N] or None. With width == 1 there is no state and nothing to install."""
    a = _Args("shortconv_state_commit")
    W, H, D = int(width), int(num_heads), int(head_dim)
    if W < 1:
        a.fail(f"width must be >= 1, got {W}")
    a.tensor(cu_seqlens, "cu_seqlens", _I32, (None,))
    N = cu_seqlens.shape[0] - 1
    if N < 0:
        a.fail("cu_seqlens must hold at least one entry (num_seqs + 1)")
    a.tensor(accepted, "accepted", _I32, (N,))
    a.tensor(state_idx, "state_idx", _I32, (N,), optional=True)
    dtype = torch.bfloat16
    max_tokens = 1
    if W > 1:
        a.tensor(k_snap, "k_snap", (torch.float32, torch.bfloat16), (N, None, W - 1, H, D))
        dtype = k_snap.dtype
        max_tokens = k_snap.shape[1]
        a.tensor(v_snap, "v_snap", (dtype,), (N, max_tokens, W - 1, H, D))
        if k_state is None or v_state is None:
            a.fail("k_state and v_state are required when width > 1")
    S = _state_pools(a, k_state, v_state, W, H, D, dtype) if W > 1 else 0
    a.on_gpu()
    lib = load_library()
    dev = a.device
    with torch.cuda.device(dev):
        rc = lib.shortconv_state_commit(
            _ptr(k_snap), _ptr(v_snap), max_tokens, _ptr(cu_seqlens), int(total_tokens),
            _ptr(accepted), N, _ptr(k_state), _ptr(v_state), S, _ptr(state_idx), H, D, W,
            SC_DTYPE[dtype], _stream_handle(dev, stream))
    _check(rc)


def shortconv_kv_prefill_mxfp8(k, v, cu_seqlens, k_taps, v_taps, k_gamma, v_gamma, eps, k_state,
                               v_state, state_idx, has_initial_state, slot_mapping, k_codes,
                               v_codes, k_scales, v_scales, *,
                               stream: Optional[torch.cuda.Stream] = None) -> None:
    """Prefill writing MXFP8 cache rows: codes uint8 [num_slots,H,D], scales uint8
    [num_slots,H,D/32] (see include/shortconv.h); other arguments as shortconv_kv_prefill."""
    a, W, H, D, ks, vs, S, N = _prefill_args("shortconv_kv_prefill_mxfp8", k, v, cu_seqlens,
                                             k_taps, v_taps, k_gamma, v_gamma, k_state, v_state,
                                             state_idx, has_initial_state, slot_mapping)
    nslots = _mx_caches(a, k_codes, v_codes, k_scales, v_scales, H, D)
    a.on_gpu()
    lib = load_library()
    with torch.cuda.device(k.device):
        rc = lib.shortconv_kv_prefill_mxfp8(
            _ptr(k), _ptr(v), ks, vs, _ptr(cu_seqlens), N, k.shape[0], _ptr(k_taps), _ptr(v_taps),
            _ptr(k_gamma), _ptr(v_gamma), float(eps), _ptr(k_state), _ptr(v_state), S,
            _ptr(state_idx), _ptr(_flags(has_initial_state)), _ptr(slot_mapping), _ptr(k_codes),
            _ptr(v_codes), _ptr(k_scales), _ptr(v_scales), nslots, H, D, W, SC_DTYPE[k.dtype],
            _stream_handle(k.device, stream))
    _check(rc)


def shortconv_kv_decode_mxfp8(k_new, v_new, k_taps, v_taps, k_gamma, v_gamma, eps, k_state,
                              v_state, state_idx, slot_mapping, k_codes, v_codes, k_scales,
                              v_scales, *, stream: Optional[torch.cuda.Stream] = None) -> None:
    """Decode writing MXFP8 cache rows (see include/shortconv.h)."""
    a, W, H, D, ks, vs, S, B = _decode_args("shortconv_kv_decode_mxfp8", k_new, v_new, k_taps,
                                            v_taps, k_gamma, v_gamma, k_state, v_state,
                                            state_idx, slot_mapping)
    nslots = _mx_caches(a, k_codes, v_codes, k_scales, v_scales, H, D)
    a.on_gpu()
    lib = load_library()
    with torch.cuda.device(k_new.device):
        rc = lib.shortconv_kv_decode_mxfp8(
            _ptr(k_new), _ptr(v_new), ks, vs, B, _ptr(k_taps), _ptr(v_taps), _ptr(k_gamma),
            _ptr(v_gamma), float(eps), _ptr(k_state), _ptr(v_state), S, _ptr(state_idx),
            _ptr(slot_mapping), _ptr(k_codes), _ptr(v_codes), _ptr(k_scales), _ptr(v_scales),
            nslots, H, D, W, SC_DTYPE[k_new.dtype], _stream_handle(k_new.device, stream))
    _check(rc)


def shortconv_mxfp8_quantize(x, codes, scales, *,
                             stream: Optional[torch.cuda.Stream] = None) -> None:
    """MXFP8-quantize rows x [rows,H,D] into codes [rows,H,D] and scales [rows,H,D/32] (uint8)."""
    a = _Args("shortconv_mxfp8_quantize")
    xs = a.rows(x, "x")
    rows, H, D = x.shape
    a.tensor(codes, "codes", _U8, (rows, H, D))
    a.tensor(scales, "scales", _U8, (rows, H, D // 32))
    a.on_gpu()
    lib = load_library()
    with torch.cuda.device(x.device):
        rc = lib.shortconv_mxfp8_quantize(_ptr(x), xs, rows, H, D, SC_DTYPE[x.dtype],
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


def _backward_args(fn, k, v, cu_seqlens, k_taps, v_taps, k_gamma, v_gamma, k_state, v_state,
                   state_idx, has_initial_state, dy_k, dy_v, dk, dv, dk_taps, dv_taps, dk_gamma,
                   dv_gamma, dstate_out, dstate_in):
    a = _Args(fn)
    W, H, D, ks, vs, S = _step_common(a, k, v, k_taps, v_taps, k_gamma, v_gamma, k_state, v_state)
    a.tensor(cu_seqlens, "cu_seqlens", _I32, (None,))
    N = cu_seqlens.shape[0] - 1
    if N < 0:
        a.fail("cu_seqlens must hold at least one entry (num_seqs + 1)")
    a.tensor(state_idx, "state_idx", _I32, (N,), optional=True)
    a.tensor(has_initial_state, "has_initial_state", _FLAGS, (N,), optional=True)
    T = k.shape[0]
    rows = ((k.dtype,), (T, H, D))
    for name, t in (("dy_k", dy_k), ("dy_v", dy_v), ("dk", dk), ("dv", dv)):
        a.tensor(t, name, *rows)
    for name, t in (("dk_taps", dk_taps), ("dv_taps", dv_taps)):
        a.tensor(t, name, _F32, (W, H, D))
    for name, t in (("dk_gamma", dk_gamma), ("dv_gamma", dv_gamma)):
        a.tensor(t, name, _F32, (D,))
    for pair, names in ((dstate_out, ("dstate_out[0]", "dstate_out[1]")),
                        (dstate_in, ("dstate_in[0]", "dstate_in[1]"))):
        if len(pair) != 2 or (pair[0] is None) != (pair[1] is None):
            a.fail(f"{names[0]} and {names[1]} must both be given or both be None")
        for name, t in zip(names, pair):
            a.tensor(t, name, (k.dtype,), (N, W - 1, H, D), optional=True)
    return a, W, H, D, ks, vs, S, N, T


def shortconv_kv_backward(k, v, cu_seqlens, k_taps, v_taps, k_gamma, v_gamma, eps, k_state,
                          v_state, state_idx, has_initial_state, dy_k, dy_v, dk, dv, dk_taps,
                          dv_taps, dk_gamma, dv_gamma, *, dstate_out=(None, None),
                          dstate_in=(None, None), workspace: Optional[torch.Tensor] = None,
                          stream: Optional[torch.cuda.Stream] = None) -> None:
    """Gradients of the prefill step (see include/shortconv.h): from dy_k/dy_v (and optionally the
    new-state gradients ``dstate_out``) into dk/dv, the tap and gamma gradients and optionally the
    initial-window gradients ``dstate_in``. dy/dk/dv [T,H,D] contiguous of k's dtype; tap and
    gamma gradients fp32 [W,H,D] / [D]; dstate pairs [N,W-1,H,D] of k's dtype or (None, None).
    ``workspace`` (a uint8 device tensor) is allocated here when not given."""
    a, W, H, D, ks, vs, S, N, T = _backward_args(
        "shortconv_kv_backward", k, v, cu_seqlens, k_taps, v_taps, k_gamma, v_gamma, k_state,
        v_state, state_idx, has_initial_state, dy_k, dy_v, dk, dv, dk_taps, dv_taps, dk_gamma,
        dv_gamma, dstate_out, dstate_in)
    a.tensor(workspace, "workspace", _U8, (None,), optional=True)
    a.on_gpu()
    need = shortconv_kv_backward_workspace_size(T, N, H, D, W, k.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=k.device)
    lib = load_library()
    with torch.cuda.device(k.device):
        rc = lib.shortconv_kv_backward(
            _ptr(k), _ptr(v), ks, vs, _ptr(cu_seqlens), N, T, _ptr(k_taps), _ptr(v_taps),
            _ptr(k_gamma), _ptr(v_gamma), float(eps), _ptr(k_state), _ptr(v_state), S,
            _ptr(state_idx), _ptr(_flags(has_initial_state)), _ptr(dy_k), _ptr(dy_v),
            _ptr(dstate_out[0]), _ptr(dstate_out[1]), _ptr(dk), _ptr(dv), _ptr(dk_taps),
            _ptr(dv_taps), _ptr(dk_gamma), _ptr(dv_gamma), _ptr(dstate_in[0]), _ptr(dstate_in[1]),
            _ptr(workspace), workspace.numel(), H, D, W, SC_DTYPE[k.dtype],
            _stream_handle(k.device, stream))
    _check(rc)


# The size of the static device scratch of shortconv_kv_backward_noalloc (SHORTCONV_NOALLOC_SCRATCH_BYTES
# in include/shortconv.h).
NOALLOC_SCRATCH_BYTES = 16 << 20


def shortconv_kv_backward_noalloc(k, v, cu_seqlens, k_taps, v_taps, k_gamma, v_gamma, eps,
                                  k_state, v_state, state_idx, has_initial_state, dy_k, dy_v, dk,
                                  dv, dk_taps, dv_taps, dk_gamma, dv_gamma, *,
                                  dstate_out=(None, None), dstate_in=(None, None),
                                  stream: Optional[torch.cuda.Stream] = None) -> None:
    """shortconv_kv_backward without a workspace argument and without any allocation: the library
    uses its static per-GPU scratch (see include/shortconv.h), so problems whose workspace exceeds
    NOALLOC_SCRATCH_BYTES are rejected, and calls that may overlap on one GPU must be ordered."""
    a, W, H, D, ks, vs, S, N, T = _backward_args(
        "shortconv_kv_backward_noalloc", k, v, cu_seqlens, k_taps, v_taps, k_gamma, v_gamma,
        k_state, v_state, state_idx, has_initial_state, dy_k, dy_v, dk, dv, dk_taps, dv_taps,
        dk_gamma, dv_gamma, dstate_out, dstate_in)
    a.on_gpu()
    lib = load_library()
    with torch.cuda.device(k.device):
        rc = lib.shortconv_kv_backward_noalloc(
            _ptr(k), _ptr(v), ks, vs, _ptr(cu_seqlens), N, T, _ptr(k_taps), _ptr(v_taps),
            _ptr(k_gamma), _ptr(v_gamma), float(eps), _ptr(k_state), _ptr(v_state), S,
            _ptr(state_idx), _ptr(_flags(has_initial_state)), _ptr(dy_k), _ptr(dy_v),
            _ptr(dstate_out[0]), _ptr(dstate_out[1]), _ptr(dk), _ptr(dv), _ptr(dk_taps),
            _ptr(dv_taps), _ptr(dk_gamma), _ptr(dv_gamma), _ptr(dstate_in[0]), _ptr(dstate_in[1]),
            H, D, W, SC_DTYPE[k.dtype], _stream_handle(k.device, stream))
    _check(rc)
