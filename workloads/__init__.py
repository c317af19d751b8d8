"""Seeded synthetic inputs for the fused ShortConv K/V step.

This package draws inputs and paging structure only; it holds none of the step's arithmetic and
imports neither the oracle nor the HIP library. Both sides (the oracle in tests, the HIP path in
tests and the bench) receive the same arrays from here.

Stored element types follow the oracle's convention: ``"f32"`` arrays are ``numpy.float32`` and
``"bf16"`` arrays are ``numpy.uint16`` holding bf16 bit patterns (fp32 draws rounded once, to
nearest-even).

Every random tensor comes from its own stream ``numpy.random.default_rng([seed, tag, stream])``
(PCG64 seeded through SeedSequence), so changing one tensor's recipe leaves the others unchanged.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

# stream ids (the third SeedSequence word)
_S_LENS, _S_K, _S_V, _S_KTAP, _S_VTAP, _S_KG, _S_VG, _S_KST, _S_VST = range(9)
_S_BLOCKS, _S_SIDX, _S_DEC_CTX, _S_START, _S_KOUT, _S_VOUT, _S_DK, _S_DV, _S_PAD = range(9, 18)
_S_ACCEPT = 18

# Finite bit patterns that untouched cache rows keep (checked bit for bit after a step).
SENTINEL = {"f32": np.uint32(0x5A5A5A5A), "bf16": np.uint16(0x5A5A)}
STORED = {"f32": np.float32, "bf16": np.uint16}


def rng(seed: int, tag: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(tag), int(stream)])


def to_bf16_bits(f: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(f, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normal_stored(g: np.random.Generator, shape, dtype: str, scale=1.0, outlier_p=0.0,
                   outlier_mul=1.0, g_out: Optional[np.random.Generator] = None):
    """N(0, scale^2) draws in fp32, optionally with a fraction of entries multiplied (outliers),
    then stored (bf16 rounding happens once, after the multiply). Drawn in chunks to bound memory."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=STORED[dtype])
    chunk = 1 << 24
    for a in range(0, n, chunk):
        b = min(n, a + chunk)
        f = g.standard_normal(b - a, dtype=np.float32)
        if scale != 1.0:
            f *= np.float32(scale)
        if outlier_p > 0.0:
            hit = g_out.random(b - a) < outlier_p
            f[hit] *= np.float32(outlier_mul)
        out[a:b] = f if dtype == "f32" else to_bf16_bits(f)
    return out.reshape(shape)


@dataclass
class Step:
    """Arguments of one library call (prefill or decode), host side."""
    kind: str                                  # "prefill" | "decode"
    k: np.ndarray                              # stored [T, H, D] (token dim may be strided)
    v: np.ndarray
    slot_mapping: np.ndarray                   # int64 [T]
    state_idx: np.ndarray                      # int32 [N] (prefill) or [B] (decode)
    cu_seqlens: Optional[np.ndarray] = None    # int32 [N+1] (prefill)
    has_init: Optional[np.ndarray] = None      # uint8 [N] (prefill)

    @property
    def tokens(self) -> int:
        return int(self.k.shape[0])

    @property
    def num_seqs(self) -> int:
        return int(len(self.cu_seqlens) - 1) if self.kind == "prefill" else int(self.k.shape[0])


@dataclass
class Workload:
    name: str
    dtype: str
    H: int
    D: int
    W: int
    eps: float
    k_taps: np.ndarray                         # float32 [W, H, D]
    v_taps: np.ndarray
    k_gamma: np.ndarray                        # float32 [D]
    v_gamma: np.ndarray
    num_slots: int                             # cache rows
    block_size: int
    k_state: Optional[np.ndarray]              # stored [S, W-1, H, D] initial pool (None if W==1)
    v_state: Optional[np.ndarray]
    steps: List[Step] = field(default_factory=list)
    recipe: str = ""

    @property
    def num_state_slots(self) -> int:
        return 0 if self.k_state is None else int(self.k_state.shape[0])

    @property
    def tokens(self) -> int:
        return sum(s.tokens for s in self.steps)


@dataclass
class Spec:
    """Recipe for a synthetic workload.

    prefill_lens[s] new tokens of prefill sequence s, starting at absolute position
    prefill_start[s] (0 = fresh sequence); has_init[s] says whether its window starts from a stored
    state. decode_ctx[b] is the context length of decode sequence b after its new token.
    """
    name: str = "custom"
    dtype: str = "bf16"
    H: int = 8
    D: int = 128
    W: int = 4
    eps: float = 1e-6
    seed: int = 0
    tag: int = 0
    prefill_lens: Sequence[int] = ()
    prefill_start: Optional[Sequence[int]] = None
    has_init: Optional[Sequence[int]] = None
    decode_ctx: Sequence[int] = ()
    block_size: int = 16
    contiguous_cache: bool = False             # slot = packed token index, no paging
    state_init: str = "normal"                 # "normal" | "zero"
    outlier_p: float = 0.0
    outlier_mul: float = 50.0
    token_pad: int = 0                         # extra elements after each token row (strided K/V)
    pad_slot_every: int = 0                    # every n-th token gets slot -1 (0 = never)
    spare_slots: int = 0                       # extra never-written cache rows at the pool end


def _paged_slots(g, ctx: np.ndarray, new: np.ndarray, bs: int):
    """Random permuted block tables. Sequence i holds ctx[i] tokens in ceil(ctx/bs) blocks drawn
    from one permutation of the pool; its last new[i] positions are the ones written now.
    Returns (slot_mapping of the new tokens in sequence order, number of cache rows)."""
    nblk = -(-ctx // bs)
    total = int(nblk.sum())
    perm = g.permutation(total).astype(np.int64)
    first = np.concatenate([[0], np.cumsum(nblk)[:-1]]).astype(np.int64)
    out = []
    for i in range(len(ctx)):
        pos = np.arange(ctx[i] - new[i], ctx[i], dtype=np.int64)
        table = perm[first[i]:first[i] + nblk[i]]
        out.append(table[pos // bs] * bs + pos % bs)
    sm = np.concatenate(out) if out else np.zeros(0, np.int64)
    return sm, total * bs


def _rows(g, T, H, D, dtype, pad, **kw):
    """[T, H, D] stored rows; with pad > 0 they are a view into [T, H*D + pad] storage."""
    if pad == 0:
        return _normal_stored(g, (T, H, D), dtype, **kw)
    base = np.zeros((T, H * D + pad), dtype=STORED[dtype])
    base[:, :H * D] = _normal_stored(g, (T, H * D), dtype, **kw)
    return base[:, :H * D].reshape(T, H, D)


def build(spec: Spec) -> Workload:
    s, t = spec.seed, spec.tag
    dt, H, D, W = spec.dtype, spec.H, spec.D, spec.W
    lens = np.asarray(spec.prefill_lens, dtype=np.int64)
    N = len(lens)
    starts = (np.zeros(N, np.int64) if spec.prefill_start is None
              else np.asarray(spec.prefill_start, dtype=np.int64))
    hinit = (np.zeros(N, np.uint8) if spec.has_init is None
             else np.asarray(spec.has_init, dtype=np.uint8))
    dctx = np.asarray(spec.decode_ctx, dtype=np.int64)
    B = len(dctx)

    k_taps = _normal_stored(rng(s, t, _S_KTAP), (W, H, D), "f32", scale=1.0 / np.sqrt(W))
    v_taps = _normal_stored(rng(s, t, _S_VTAP), (W, H, D), "f32", scale=1.0 / np.sqrt(W))
    k_gamma = (1.0 + 0.1 * rng(s, t, _S_KG).standard_normal(D, dtype=np.float32)).astype(np.float32)
    v_gamma = (1.0 + 0.1 * rng(s, t, _S_VG).standard_normal(D, dtype=np.float32)).astype(np.float32)

    S = N + B
    if W > 1:
        if spec.state_init == "zero":
            k_state = np.zeros((S, W - 1, H, D), STORED[dt])
            v_state = np.zeros((S, W - 1, H, D), STORED[dt])
        else:
            k_state = _normal_stored(rng(s, t, _S_KST), (S, W - 1, H, D), dt)
            v_state = _normal_stored(rng(s, t, _S_VST), (S, W - 1, H, D), dt)
    else:
        k_state = v_state = None
    sidx = rng(s, t, _S_SIDX).permutation(S).astype(np.int32)

    # cache placement: prefill sequences first, then decode sequences, one pool
    T = int(lens.sum())
    if spec.contiguous_cache:
        slots = np.arange(T + B, dtype=np.int64)
        num_slots = T + B
    else:
        ctx = np.concatenate([starts + lens, dctx]).astype(np.int64)
        new = np.concatenate([lens, np.ones(B, np.int64)])
        slots, num_slots = _paged_slots(rng(s, t, _S_BLOCKS), ctx, new, spec.block_size)
    if spec.pad_slot_every > 0:
        slots = slots.copy()
        slots[::spec.pad_slot_every] = -1
    num_slots += spec.spare_slots

    kw = dict(outlier_p=spec.outlier_p, outlier_mul=spec.outlier_mul)
    steps = []
    if N > 0 or B == 0:
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        k = _rows(rng(s, t, _S_K), T, H, D, dt, spec.token_pad, g_out=rng(s, t, _S_KOUT), **kw)
        v = _rows(rng(s, t, _S_V), T, H, D, dt, spec.token_pad, g_out=rng(s, t, _S_VOUT), **kw)
        steps.append(Step("prefill", k, v, slots[:T], sidx[:N].copy(), cu, hinit))
    if B > 0:
        k = _rows(rng(s, t, _S_DK), B, H, D, dt, spec.token_pad)
        v = _rows(rng(s, t, _S_DV), B, H, D, dt, spec.token_pad)
        steps.append(Step("decode", k, v, slots[T:T + B], sidx[N:N + B].copy()))

    return Workload(spec.name, dt, H, D, W, spec.eps, k_taps, v_taps, k_gamma, v_gamma,
                    int(num_slots), spec.block_size, k_state, v_state, steps)


# ---------------------------------------------------------------------------------------------
# The five measured workloads: a tiny fp32 reference, a packed variable-length prefill batch, a
# decode batch, one long prefill at width 8, and a mixed chunked-prefill + decode step. Every
# draw a workload leaves open is stated in its recipe string.
# ---------------------------------------------------------------------------------------------
# The five workloads, in order; each one's random streams are keyed by its tag (1..5).
CONFIG_NAMES = ("tiny_ref", "varlen_prefill", "decode", "long_prefill", "mixed")
_TAG = {name: i + 1 for i, name in enumerate(CONFIG_NAMES)}


def config_spec(name: str, seed: int = 0) -> Spec:
    """The recipe of one of the five workloads (CONFIG_NAMES), drawn with `seed`."""
    if name not in _TAG:
        raise ValueError(f"unknown workload {name!r}; one of {CONFIG_NAMES}")
    t = _TAG[name]
    if name == "tiny_ref":
        return Spec(name=name, dtype="f32", H=1, D=64, W=4, seed=seed, tag=t, prefill_lens=[64],
                    has_init=[1], state_init="zero", contiguous_cache=True)
    if name == "varlen_prefill":
        lens = rng(seed, t, _S_LENS).integers(512, 4096, size=8, endpoint=True)
        return Spec(name=name, dtype="bf16", H=8, D=128, W=4, seed=seed, tag=t,
                    prefill_lens=lens.tolist(), has_init=[0] * 8, block_size=16)
    if name == "decode":
        ctx = rng(seed, t, _S_DEC_CTX).integers(1, 32768, size=256, endpoint=True)
        return Spec(name=name, dtype="bf16", H=8, D=128, W=4, seed=seed, tag=t,
                    decode_ctx=ctx.tolist(), block_size=64)
    if name == "long_prefill":
        return Spec(name=name, dtype="bf16", H=8, D=128, W=8, seed=seed, tag=t,
                    prefill_lens=[131072], has_init=[0], block_size=64, outlier_p=0.01,
                    outlier_mul=50.0)
    g = rng(seed, t, _S_START)  # mixed
    starts = 2048 * g.integers(1, 15, size=64, endpoint=True)
    ctx = rng(seed, t, _S_DEC_CTX).integers(1, 32768, size=512, endpoint=True)
    return Spec(name=name, dtype="bf16", H=16, D=128, W=4, seed=seed, tag=t,
                prefill_lens=[2048] * 64, prefill_start=starts.tolist(), has_init=[1] * 64,
                decode_ctx=ctx.tolist(), block_size=16)


def config(name: str, seed: int = 0) -> Workload:
    """One of the five workloads (CONFIG_NAMES), built, with its recipe string."""
    w = build(config_spec(name, seed))
    w.recipe = RECIPES[name]
    return w


RECIPES = {
    "tiny_ref": "1 seq x 64 tokens, H=1, D=64, W=4, fp32; K,V~N(0,1); taps~N(0,1/W); "
                "gamma=1+0.1N(0,1); zero initial state; slot i = token i",
    "varlen_prefill": "8 seqs, lengths U{512..4096}, H=8, D=128, W=4, bf16; K,V~N(0,1); fresh "
                      "(zero) state; paged cache, block 16, one random permutation of the pool "
                      "as block tables",
    "decode": "256 decodes, H=8, D=128, W=4, bf16; state rows~N(0,1); state slots permuted; "
              "context U{1..32768}; paged cache, block 64, permuted block tables",
    "long_prefill": "1 seq x 131072 tokens, H=8, D=128, W=8, bf16; K,V~N(0,1) with each entry x50 "
                    "w.p. 0.01; fresh state; paged cache, block 64, permuted block table",
    "mixed": "64 chunks x 2048 tokens resuming at 2048*U{1..15} from state~N(0,1) + 512 decodes "
             "(context U{1..32768}), H=16, D=128, W=4, bf16; paged cache, block 16, permuted "
             "tables",
}


# ---------------------------------------------------------------------------------------------
# Speculative verification at the decode shape. The pages give no shapes for it; this takes the
# decode workload's sequences, each verifying a run of SPEC_TOKENS candidate tokens (the first
# being the token sampled last step), and draws how many of them the target model accepts.
# ---------------------------------------------------------------------------------------------
SPEC_TOKENS = 4
SPEC_RECIPE = ("256 sequences x 4 candidate tokens, H=8, D=128, W=4, bf16; every sequence resumes "
               "from its stored state (rows~N(0,1)); context U{5..32768} after the run; paged "
               "cache, block 64, permuted block tables; accepted count U{0..4} per sequence")


def spec_verify(seed: int = 0):
    """(workload, accepted): one verification call of SPEC_TOKENS tokens per sequence and the
    number of them accepted (int32 [256]), for the verify + state-commit pair."""
    ctx = rng(seed, 6, _S_DEC_CTX).integers(SPEC_TOKENS + 1, 32768, size=256, endpoint=True)
    spec = Spec(name="spec_verify", dtype="bf16", H=8, D=128, W=4, seed=seed, tag=6,
                prefill_lens=[SPEC_TOKENS] * 256, prefill_start=(ctx - SPEC_TOKENS).tolist(),
                has_init=[1] * 256, block_size=64)
    w = build(spec)
    w.recipe = SPEC_RECIPE
    accepted = rng(seed, 6, _S_ACCEPT).integers(0, SPEC_TOKENS, size=256,
                                                endpoint=True).astype(np.int32)
    return w, accepted
