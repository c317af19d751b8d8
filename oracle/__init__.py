"""fp64 CPU oracle of the fused ShortConv K/V step -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the bench's CPU-baseline leg may import this package.
The HIP library never does, and this package imports nothing from it.

The step's arithmetic and its backward live in ``shortconv_oracle.c`` (fp64, one plain loop nest
per definition step; its header states the definition and the readings of the pages it follows).
This module marshals numpy arrays into it, writes out in numpy the parts that are bit copies or
encodings (the speculative-verification snapshots and commit, the MXFP8 encoding), holds the
acceptance metric, and applies the two scatters the step ends with:

* the cache write: row ``y[t]`` goes to ``cache[slot_mapping[t]]`` when ``0 <= slot < num_slots``
  (aib.vote English news item on SGLang/Miles day-0 Inkling support, paragraph 2: the fused
  kernel ends with the KV-cache write);
* the state-pool write: the new window of sequence ``s`` goes to ``pool[state_idx[s]]`` when the
  index is inside the pool (data-sketchers.com SGLang cookbook for Inkling-Small, section 2: the
  sconv state lives in a per-request pool).

Stored element types: ``"f32"`` arrays are ``numpy.float32``; ``"bf16"`` arrays are ``numpy.uint16``
holding the bf16 bit patterns. Every pin of this oracle is in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os
from contextlib import contextmanager
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

DTYPES = {"f32": (0, np.float32), "bf16": (1, np.uint16)}


def _bind(lib):
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.sc_oracle_prefill.restype = ctypes.c_int
    lib.sc_oracle_prefill.argtypes = [ctypes.c_int, I64, I64, I64, I64, P, P, I64, P, P,
                                      ctypes.c_float, P, I64, P, P, P, P, P, ctypes.c_int]
    lib.sc_oracle_decode.restype = ctypes.c_int
    lib.sc_oracle_decode.argtypes = [ctypes.c_int, I64, I64, I64, I64, P, I64, P, P,
                                     ctypes.c_float, P, I64, P, P, P, P, ctypes.c_int]
    lib.sc_oracle_backward.restype = ctypes.c_int
    lib.sc_oracle_backward.argtypes = [ctypes.c_int, I64, I64, I64, I64, P, P, I64, P, P,
                                       ctypes.c_float, P, I64, P, P, P, P, P, P, P, P, P, P, P,
                                       P, ctypes.c_int]
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _build
            _build.build()
        _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


@contextmanager
def library(path: str):
    """Run the oracle from another build of its source (used by the tests that plant mistakes in
    a copy of the oracle and check that the pins catch them)."""
    global _lib
    saved = _lib
    _lib = _bind(ctypes.CDLL(path))
    try:
        yield
    finally:
        _lib = saved


def _dtype_code(arr: np.ndarray) -> int:
    for code, npdt in DTYPES.values():
        if arr.dtype == npdt:
            return code
    raise TypeError(f"stored element type must be float32 or uint16 (bf16 bits), got {arr.dtype}")


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _token_rows(x: np.ndarray, H: int, D: int):
    """Return (array, token stride in elements) for a [T, H, D] array whose inner two dims are
    contiguous; the token dimension may be strided (e.g. a view into a wider projection)."""
    if x.ndim != 3 or x.shape[1:] != (H, D):
        raise ValueError(f"expected [T, {H}, {D}], got {x.shape}")
    item = x.itemsize
    if x.strides[2] != item or x.strides[1] != D * item or x.strides[0] % item:
        x = np.ascontiguousarray(x)
    stride = x.strides[0] // item if x.shape[0] > 0 else H * D
    return x, max(stride, H * D)


def prefill_one(x, cu_seqlens, taps, gamma, eps, state, state_idx, has_init, *, cond=False,
                nthreads=1):
    """One tensor (K or V) over packed sequences.

    Returns ``(y, new_state, cond)``: y fp64 [T,H,D]; new_state stored [N,W-1,H,D] (None if W==1);
    cond fp64 [T,H,D] or None. ``state_idx`` entries outside the pool mean "no state slot".
    """
    lib = _load()
    taps = np.ascontiguousarray(taps, dtype=np.float32)
    W, H, D = taps.shape
    gamma = np.ascontiguousarray(gamma, dtype=np.float32)
    assert gamma.shape == (D,)
    code = _dtype_code(x)
    x, xs = _token_rows(x, H, D)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    N = cu.shape[0] - 1
    T = x.shape[0]
    assert N >= 0 and cu[0] == 0 and cu[-1] <= T and np.all(np.diff(cu) >= 0)
    sidx = np.ascontiguousarray(state_idx if state_idx is not None else np.arange(N), dtype=np.int64)
    hinit = np.ascontiguousarray(has_init if has_init is not None else np.ones(N), dtype=np.uint8)
    if W > 1 and state is not None:
        state = np.ascontiguousarray(state)
        assert state.dtype == x.dtype and state.shape[1:] == (W - 1, H, D)
        n_state = state.shape[0]
    else:
        state, n_state = None, 0
    y = np.zeros((T, H, D), np.float64)
    cnd = np.zeros((T, H, D), np.float64) if cond else None
    new_state = np.zeros((N, W - 1, H, D), x.dtype) if W > 1 else None
    rc = lib.sc_oracle_prefill(code, H, D, W, N, _ptr(cu), _ptr(x), xs, _ptr(taps), _ptr(gamma),
                               float(eps), _ptr(state), n_state, _ptr(sidx), _ptr(hinit), _ptr(y),
                               _ptr(cnd), _ptr(new_state), int(nthreads))
    if rc != 0:
        raise ValueError("oracle prefill rejected its arguments")
    return y, new_state, cnd


def decode_one(x_new, taps, gamma, eps, state, state_idx, *, cond=False, nthreads=1):
    """One tensor (K or V), one new token per sequence. Returns ``(y, new_state, cond)`` as
    ``prefill_one`` does; rows of new_state for an out-of-pool index are left zero."""
    lib = _load()
    taps = np.ascontiguousarray(taps, dtype=np.float32)
    W, H, D = taps.shape
    gamma = np.ascontiguousarray(gamma, dtype=np.float32)
    code = _dtype_code(x_new)
    x_new, xs = _token_rows(x_new, H, D)
    B = x_new.shape[0]
    sidx = np.ascontiguousarray(state_idx if state_idx is not None else np.arange(B), dtype=np.int64)
    if W > 1 and state is not None:
        state = np.ascontiguousarray(state)
        assert state.dtype == x_new.dtype and state.shape[1:] == (W - 1, H, D)
        n_state = state.shape[0]
    else:
        state, n_state = None, 0
    y = np.zeros((B, H, D), np.float64)
    cnd = np.zeros((B, H, D), np.float64) if cond else None
    new_state = np.zeros((B, W - 1, H, D), x_new.dtype) if W > 1 else None
    rc = lib.sc_oracle_decode(code, H, D, W, B, _ptr(x_new), xs, _ptr(taps), _ptr(gamma),
                              float(eps), _ptr(state), n_state, _ptr(sidx), _ptr(y), _ptr(cnd),
                              _ptr(new_state), int(nthreads))
    if rc != 0:
        raise ValueError("oracle decode rejected its arguments")
    return y, new_state, cnd


@dataclass
class StepResult:
    """What one fused step produces, in the oracle's terms.

    y_k, y_v:     fp64 [T,H,D] normalized rows in token order.
    cond_k/v:     fp64 [T,H,D] rounding-error scale per element (or None).
    slots:        int64 [T]: the cache row token t lands in, or -1 when it is not written.
    k/v_state:    the whole state pool after the step (stored dtype), or None when W == 1.
    """
    y_k: np.ndarray
    y_v: np.ndarray
    cond_k: Optional[np.ndarray]
    cond_v: Optional[np.ndarray]
    slots: np.ndarray
    k_state: Optional[np.ndarray]
    v_state: Optional[np.ndarray]


def cache_slots(slot_mapping, num_slots):
    """Which cache row each token is written to; -1 where the slot is outside [0, num_slots)."""
    sm = np.asarray(slot_mapping, dtype=np.int64)
    return np.where((sm >= 0) & (sm < num_slots), sm, -1)


def _scatter_state(pool, new_rows, state_idx):
    if pool is None or new_rows is None:
        return None
    out = pool.copy()
    idx = np.asarray(state_idx, dtype=np.int64)
    ok = (idx >= 0) & (idx < pool.shape[0])
    out[idx[ok]] = new_rows[ok]
    return out


def fused_prefill(k, v, cu_seqlens, k_taps, v_taps, k_gamma, v_gamma, eps, k_state, v_state,
                  state_idx, has_initial_state, slot_mapping, num_slots, *, cond=True,
                  nthreads=1) -> StepResult:
    """The whole prefill step for K and V (same packing, state slots and cache slots)."""
    N = len(cu_seqlens) - 1
    sidx = np.arange(N) if state_idx is None else np.asarray(state_idx, np.int64)
    yk, nk, ck = prefill_one(k, cu_seqlens, k_taps, k_gamma, eps, k_state, sidx,
                             has_initial_state, cond=cond, nthreads=nthreads)
    yv, nv, cv = prefill_one(v, cu_seqlens, v_taps, v_gamma, eps, v_state, sidx,
                             has_initial_state, cond=cond, nthreads=nthreads)
    return StepResult(yk, yv, ck, cv, cache_slots(slot_mapping, num_slots),
                      _scatter_state(k_state, nk, sidx), _scatter_state(v_state, nv, sidx))


def fused_decode(k_new, v_new, k_taps, v_taps, k_gamma, v_gamma, eps, k_state, v_state,
                 state_idx, slot_mapping, num_slots, *, cond=True, nthreads=1) -> StepResult:
    """The whole decode step for K and V."""
    B = k_new.shape[0]
    sidx = np.arange(B) if state_idx is None else np.asarray(state_idx, np.int64)
    yk, nk, ck = decode_one(k_new, k_taps, k_gamma, eps, k_state, sidx, cond=cond,
                            nthreads=nthreads)
    yv, nv, cv = decode_one(v_new, v_taps, v_gamma, eps, v_state, sidx, cond=cond,
                            nthreads=nthreads)
    return StepResult(yk, yv, ck, cv, cache_slots(slot_mapping, num_slots),
                      _scatter_state(k_state, nk, sidx), _scatter_state(v_state, nv, sidx))


# ---------------------------------------------------------------------------------------------
# Speculative verification: k candidate tokens per sequence run from the stored conv state, and
# the state after every token is kept so that the state of any accepted prefix can be installed
# afterwards (speculative decoding with draft models or multi-token-prediction heads: aib.vote
# English news item on SGLang/Miles Inkling support, paragraph 3; data-sketchers.com SGLang
# cookbook for Inkling-Small, section 2 (MTP) and section 3.7 (DSpark)).
# ---------------------------------------------------------------------------------------------
def verify_snapshots(x, cu_seqlens, state, state_idx, width, max_tokens):
    """snapshots[s, i] = rows e[i+1 .. i+W-1] of e = [initial window, rows of sequence s], i.e. the
    conv state after its first i+1 tokens, as bit copies; written for i < min(L_s, max_tokens),
    zero elsewhere. The initial window is the stored state row (an index outside the pool means
    zeros). Returns None when W == 1."""
    R = width - 1
    if R == 0:
        return None
    cu = np.asarray(cu_seqlens, np.int64)
    N = len(cu) - 1
    H, D = x.shape[1], x.shape[2]
    snaps = np.zeros((N, max_tokens, R, H, D), x.dtype)
    for s in range(N):
        idx = int(state_idx[s])
        if state is not None and 0 <= idx < state.shape[0]:
            z = state[idx]
        else:
            z = np.zeros((R, H, D), x.dtype)
        e = np.concatenate([z, x[cu[s]:cu[s + 1]]], axis=0)
        for i in range(min(int(cu[s + 1] - cu[s]), max_tokens)):
            snaps[s, i] = e[i + 1:i + 1 + R]
    return snaps


def commit_state(pool, snapshots, accepted, cu_seqlens, state_idx, max_tokens):
    """pool[state_idx[s]] = snapshots[s, m-1] with m = min(accepted[s], L_s, max_tokens), for m >= 1
    and an index inside the pool; other rows keep their bits. Returns the new pool."""
    if pool is None:
        return None
    out = pool.copy()
    cu = np.asarray(cu_seqlens, np.int64)
    for s in range(len(cu) - 1):
        m = min(int(accepted[s]), int(cu[s + 1] - cu[s]), max_tokens)
        idx = int(state_idx[s])
        if m >= 1 and 0 <= idx < pool.shape[0]:
            out[idx] = snapshots[s, m - 1]
    return out


def fused_verify(k, v, cu_seqlens, k_taps, v_taps, k_gamma, v_gamma, eps, k_state, v_state,
                 state_idx, slot_mapping, num_slots, max_tokens, *, cond=True, nthreads=1):
    """Verification step for K and V: the outputs are those of a prefill that resumes every
    sequence from its stored state; the pools are not modified (the result's k_state/v_state are
    the input pools) and the per-token snapshots are returned as (k_snap, v_snap)."""
    N = len(cu_seqlens) - 1
    sidx = np.arange(N) if state_idx is None else np.asarray(state_idx, np.int64)
    ones = np.ones(N, np.uint8)
    yk, _, ck = prefill_one(k, cu_seqlens, k_taps, k_gamma, eps, k_state, sidx, ones, cond=cond,
                            nthreads=nthreads)
    yv, _, cv = prefill_one(v, cu_seqlens, v_taps, v_gamma, eps, v_state, sidx, ones, cond=cond,
                            nthreads=nthreads)
    W = np.asarray(k_taps).shape[0]
    ks = verify_snapshots(k, cu_seqlens, k_state, sidx, W, max_tokens)
    vs = verify_snapshots(v, cu_seqlens, v_state, sidx, W, max_tokens)
    res = StepResult(yk, yv, ck, cv, cache_slots(slot_mapping, num_slots), k_state, v_state)
    return res, ks, vs


# ---------------------------------------------------------------------------------------------
# MXFP8 cache rows. The cookbook's long-context recipe stores KV entries as block-scaled MXFP8
# instead of BF16, roughly doubling the tokens the pools hold (data-sketchers.com SGLang cookbook
# for Inkling-Small, section 3.6). Reading (the page names the format only): the OCP Microscaling
# (MX) v1.0 layout -- blocks of 32 consecutive elements along head_dim share one E8M0 scale
# X = 2^(floor(log2(max |v|)) - 8), clamped to [2^-127, 2^127] (an all-zero block gets 2^-127);
# each element is v / X rounded to OCP FP8 E4M3 (bias 7, no infinity, max normal 448) to nearest,
# ties to even, saturating at +-448. Scale byte = exponent + 127.
# ---------------------------------------------------------------------------------------------
MX_BLOCK = 32
E4M3_MAX = 448.0


def e4m3_decode(codes):
    """Value of each OCP E4M3 code (NaN for S.1111.111)."""
    c = np.asarray(codes, np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * 2.0 ** (e - 7))
    val = np.where((e == 0xF) & (m == 7), np.nan, val)
    return sign * val


def e4m3_encode(v):
    """Nearest OCP E4M3 code (ties to even), saturating at +-448; v finite (float64 array)."""
    v = np.asarray(v, np.float64)
    a = np.abs(v)
    sign = np.where(np.signbit(v), 0x80, 0).astype(np.int64)
    mant, ex = np.frexp(a)                    # a = mant * 2^ex, mant in [0.5, 1)
    e = ex - 1                                # floor(log2 a) for a > 0
    normal = a >= 2.0 ** -6
    # normal range: 3 fraction bits at exponent e
    m = np.rint((a / np.ldexp(1.0, e) - 1.0) * 8.0)   # exact scaling; rint rounds half to even
    up = m >= 8                               # rounding carried into the next binade
    e = np.where(up, e + 1, e)
    m = np.where(up, 0, m)
    code_n = ((e + 7) << 3) | m.astype(np.int64)
    # subnormal range: multiples of 2^-9 (a count of 8 is the smallest normal, code 0x08)
    code_s = np.rint(a * 2.0 ** 9).astype(np.int64)
    code = np.where(normal, code_n, code_s)
    code = np.where(a > E4M3_MAX, 0x7E, code)   # beyond the largest normal (incl. rounding up to 480)
    code = np.where(code > 0x7E, 0x7E, code)
    return (code | sign).astype(np.uint8)


def mx_scale_exponent(block_amax):
    """floor(log2(amax)) - 8, clamped to [-127, 127]; -127 for an all-zero block."""
    a = np.asarray(block_amax, np.float64)
    _, ex = np.frexp(a)
    e = np.where(a > 0, ex - 1 - 8, -127)
    return np.clip(e, -127, 127).astype(np.int64)


def mxfp8_quantize(y):
    """y float64 [..., D] (D a multiple of 32) -> (codes uint8 [..., D], scales uint8 [..., D/32])."""
    y = np.asarray(y, np.float64)
    D = y.shape[-1]
    assert D % MX_BLOCK == 0
    blocks = y.reshape(*y.shape[:-1], D // MX_BLOCK, MX_BLOCK)
    e = mx_scale_exponent(np.abs(blocks).max(axis=-1))
    scaled = blocks / np.ldexp(1.0, e)[..., None]
    codes = e4m3_encode(scaled).reshape(y.shape)
    return codes, (e + 127).astype(np.uint8)


def mxfp8_dequantize(codes, scales):
    c = np.asarray(codes)
    D = c.shape[-1]
    vals = e4m3_decode(c).reshape(*c.shape[:-1], D // MX_BLOCK, MX_BLOCK)
    x = np.ldexp(1.0, np.asarray(scales, np.int64) - 127)[..., None]
    return (vals * x).reshape(c.shape)


# ---------------------------------------------------------------------------------------------
# Backward: the gradients of the step for training (the English news item on SGLang/Miles
# Inkling support, paragraph 3: the RL trainer runs the model with train/infer-consistent
# kernels). The arithmetic -- the chain rule through the definition, step by step -- is
# sc_oracle_backward in shortconv_oracle.c, whose header states each step.
# ---------------------------------------------------------------------------------------------
@dataclass
class Grads:
    """Gradients of one tensor's step (all fp64): dx [T,H,D], dtaps [W,H,D], dgamma [D], and
    dstate [N,W-1,H,D] (None when W == 1), the gradient of each sequence's initial window rows
    (zero for a sequence that started from zeros)."""
    dx: np.ndarray
    dtaps: np.ndarray
    dgamma: np.ndarray
    dstate: Optional[np.ndarray]
    # error scales of an fp32 evaluation (see the C source), when asked for
    cond_dx: Optional[np.ndarray] = None
    cond_dtaps: Optional[np.ndarray] = None
    cond_dgamma: Optional[np.ndarray] = None
    cond_dstate: Optional[np.ndarray] = None


def backward_one(x, cu_seqlens, taps, gamma, eps, state, state_idx, has_init, g, gs=None, *,
                 cond=False, nthreads=1):
    """Backward of ``prefill_one`` for the loss whose gradient is ``g`` = dLoss/dy (fp64
    [T,H,D]) plus ``gs`` = dLoss/d(new state) (fp64 [N,W-1,H,D] or None). The chain rule through
    the definition; the C source states each step."""
    lib = _load()
    taps = np.ascontiguousarray(taps, dtype=np.float32)
    W, H, D = taps.shape
    gamma = np.ascontiguousarray(gamma, dtype=np.float32)
    code = _dtype_code(x)
    x, xs = _token_rows(x, H, D)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    N = cu.shape[0] - 1
    T = x.shape[0]
    assert N >= 0 and cu[0] == 0 and cu[-1] <= T and np.all(np.diff(cu) >= 0)
    sidx = np.ascontiguousarray(state_idx if state_idx is not None else np.arange(N), dtype=np.int64)
    hinit = np.ascontiguousarray(has_init if has_init is not None else np.ones(N), dtype=np.uint8)
    if W > 1 and state is not None:
        state = np.ascontiguousarray(state)
        assert state.dtype == x.dtype and state.shape[1:] == (W - 1, H, D)
        n_state = state.shape[0]
    else:
        state, n_state = None, 0
    g = np.ascontiguousarray(g, dtype=np.float64)
    assert g.shape == (T, H, D)
    if gs is not None and W > 1:
        gs = np.ascontiguousarray(gs, dtype=np.float64)
        assert gs.shape == (N, W - 1, H, D)
    else:
        gs = None
    dx = np.zeros((T, H, D), np.float64)
    dtaps = np.zeros((W, H, D), np.float64)
    dgamma = np.zeros(D, np.float64)
    dstate = np.zeros((N, W - 1, H, D), np.float64) if W > 1 else None
    if cond:
        cdx, cdt, cdg = np.zeros_like(dx), np.zeros_like(dtaps), np.zeros_like(dgamma)
        cds = np.zeros_like(dstate) if dstate is not None else None
    else:
        cdx = cdt = cdg = cds = None
    rc = lib.sc_oracle_backward(code, H, D, W, N, _ptr(cu), _ptr(x), xs, _ptr(taps), _ptr(gamma),
                                float(eps), _ptr(state), n_state, _ptr(sidx), _ptr(hinit), _ptr(g),
                                _ptr(gs), _ptr(dx), _ptr(dtaps), _ptr(dgamma), _ptr(dstate),
                                _ptr(cdx), _ptr(cdt), _ptr(cdg), _ptr(cds), int(nthreads))
    if rc != 0:
        raise ValueError("oracle backward rejected its arguments")
    return Grads(dx, dtaps, dgamma, dstate, cdx, cdt, cdg, cds)


def fused_backward(k, v, cu_seqlens, k_taps, v_taps, k_gamma, v_gamma, eps, k_state, v_state,
                   state_idx, has_init, gk, gv, gsk=None, gsv=None, *, cond=False, nthreads=1):
    """``backward_one`` for K and V: returns (Grads of K, Grads of V)."""
    a = backward_one(k, cu_seqlens, k_taps, k_gamma, eps, k_state, state_idx, has_init, gk, gsk,
                     cond=cond, nthreads=nthreads)
    b = backward_one(v, cu_seqlens, v_taps, v_gamma, eps, v_state, state_idx, has_init, gv, gsv,
                     cond=cond, nthreads=nthreads)
    return a, b


# ---------------------------------------------------------------------------------------------
# The acceptance metric for floating-point outputs (used by the parity tests).
#
# A correct kernel that accumulates in fp32 cannot meet a pure element-wise relative bound on
# elements whose taps cancel: the absolute error of a length-W dot product is a few units of
# fp32 roundoff times sum_k |w_k e_k|, not times |c| (Higham, Accuracy and Stability of Numerical
# Algorithms, 2nd ed., section 3.1). An element therefore passes when
#     |g - y| <= tol * |y| + FLOOR_ULPS * 2^-24 * cond
# with cond the oracle's error scale above, tol = 1e-5 for fp32 I/O and 3.9e-3 (one bf16 ulp in
# relative terms, >= the round-to-nearest bound 2^-8/(1+2^-8)) for bf16 I/O.
# ---------------------------------------------------------------------------------------------
TOL = {"f32": 1e-5, "bf16": 3.9e-3}
FLOOR_ULPS = 32.0


def widen(arr: np.ndarray) -> np.ndarray:
    """Exact widening of stored values (float32, or uint16 bf16 bits) to float64."""
    if arr.dtype == np.uint16:
        return (arr.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return arr.astype(np.float64)


def compare(got: np.ndarray, y: np.ndarray, cond: np.ndarray, dtype: str):
    """Element-wise acceptance test. ``got`` is stored values (float32 / uint16 bf16 bits).

    Returns a dict: ok, worst (max error / bound), max_rel_well_conditioned (plain max relative
    error over elements with cond <= 8|y|), n, and how far the plain relative criterion alone
    would be from passing: n_over_rel (elements whose error exceeds tol * |y|, which pass only
    through the rounding-error floor) and max_rel_over_rel (their largest err / |y|)."""
    g = widen(got)
    err = np.abs(g - y)
    bound = TOL[dtype] * np.abs(y) + FLOOR_ULPS * 2.0 ** -24 * cond
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, err / bound, np.where(err > 0, np.inf, 0.0))
        well = cond <= 8.0 * np.abs(y)
        rel = np.where(well & (y != 0), err / np.abs(y), 0.0)
        over = err > TOL[dtype] * np.abs(y)
        rel_over = np.where(over, np.where(y != 0, err / np.abs(y), np.inf), 0.0)
    finite = np.isfinite(g).all()
    return {
        "ok": bool(finite and (ratio <= 1.0).all()),
        "worst": float(ratio.max()) if ratio.size else 0.0,
        "max_rel_well_conditioned": float(rel.max()) if rel.size else 0.0,
        "n": int(y.size),
        "n_over_rel": int(over.sum()),
        "max_rel_over_rel": float(rel_over.max()) if rel_over.size else 0.0,
    }
