"""Pins of the fp64 oracle against things other than itself.

The pages print no worked example, test vector or closed-form value for this step, so every pin
here is built from mathematics: exact rational brute force in a different formulation (a
lower-triangular Toeplitz matrix-vector product and a deque for the state), library routines
(PyTorch CPU fp64 depthwise conv1d and rms_norm) in the special cases that reduce to them, closed
forms, and invariants (causality, no leakage across packed sequences, decode == prefill,
chunked == one-shot, scale invariance, permutation).

Each ``pin_*`` function raises AssertionError on a mismatch. They are run by
``test_oracle_pins.py`` against the oracle as built, and by ``test_oracle_mutations.py`` against
copies of the oracle with planted mistakes, where at least one pin must fail per mistake.
"""
from collections import deque
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import torch
import torch.nn.functional as F

import oracle
import workloads

EPS32 = float(np.float32(1e-6))


def _stored(vals, dtype):
    """Store exactly representable values (asserts that storing loses nothing)."""
    f = np.asarray(vals, dtype=np.float32)
    if dtype == "f32":
        return f
    b = workloads.to_bf16_bits(f)
    assert np.array_equal(workloads.bf16_bits_to_f32(b), f), "value not exact in bf16"
    return b


def _rand_dyadic(g, shape, num_range, den):
    return g.integers(-num_range, num_range + 1, size=shape).astype(np.float64) / den


# ------------------------------------------------------------------------------------------------
# Exact rational brute force
# ------------------------------------------------------------------------------------------------
def _exact_prefill(xq, cu, tq, gq, eps, zq, has_init):
    """xq: [T][H][D] Fractions; tq: [W][H][D]; gq: [D]; zq: [N][W-1][H][D] or None.
    Returns (y as Decimal [T][H][D], new state [N][W-1][H][D] as Fractions).

    Convolution: per (sequence, head, channel), c = M e with M the L x (W-1+L) banded Toeplitz
    matrix M[p][p+k] = taps[k]. State: a deque of length W-1 that every token is pushed through.
    """
    getcontext().prec = 50
    W = len(tq)
    H = len(tq[0])
    D = len(tq[0][0])
    R = W - 1
    T = len(xq)
    N = len(cu) - 1
    y = [[[None] * D for _ in range(H)] for _ in range(T)]
    new_state = []
    for s in range(N):
        a, b = cu[s], cu[s + 1]
        L = b - a
        z = [[[(zq[s][i][h][d] if (zq is not None and has_init[s]) else Fraction(0))
               for d in range(D)] for h in range(H)] for i in range(R)]
        # state through a deque
        dq = deque(z, maxlen=R) if R > 0 else None
        for t in range(a, b):
            if R > 0:
                dq.append(xq[t])
        new_state.append([list(row) for row in dq] if R > 0 else [])
        for h in range(H):
            cols = []  # c[p][d]
            for d in range(D):
                e = [z[i][h][d] for i in range(R)] + [xq[t][h][d] for t in range(a, b)]
                M = [[Fraction(0)] * (R + L) for _ in range(L)]
                for p in range(L):
                    for k in range(W):
                        M[p][p + k] = tq[k][h][d]
                cols.append([sum(M[p][j] * e[j] for j in range(R + L)) for p in range(L)])
            for p in range(L):
                ss = sum(cols[d][p] * cols[d][p] for d in range(D))
                r2 = ss / D + Fraction(eps)
                r = (Decimal(r2.numerator) / Decimal(r2.denominator)).sqrt()
                for d in range(D):
                    num = cols[d][p] * gq[d]
                    y[a + p][h][d] = (Decimal(num.numerator) / Decimal(num.denominator)) / r
    return y, new_state


def pin_exact_rational():
    """Oracle == exact arithmetic on tiny dyadic inputs (both stored dtypes, W = 1..5, sequences
    shorter than W-1, zero-length sequences, mixed initial states)."""
    g = np.random.default_rng(1234)
    cases = [
        (1, 2, 1, [3], [0]),
        (2, 4, 3, [5, 0, 2], [1, 0, 1]),
        (2, 4, 4, [1, 6, 2], [1, 1, 0]),
        (1, 8, 4, [8], [1]),
        (2, 2, 5, [3, 4], [1, 0]),
        (1, 4, 2, [0, 4, 1], [0, 1, 1]),
    ]
    for dtype in ("f32", "bf16"):
        for H, D, W, lens, hin in cases:
            R = W - 1
            T = sum(lens)
            cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
            xv = _rand_dyadic(g, (T, H, D), 16, 4)
            tv = _rand_dyadic(g, (W, H, D), 8, 8)
            gv = (8 + g.integers(-2, 3, size=D)) / 8.0
            zv = _rand_dyadic(g, (len(lens), R, H, D), 12, 2) if R > 0 else None
            x = _stored(xv, dtype)
            st = _stored(zv, dtype) if R > 0 else None
            y, ns, cnd = oracle.prefill_one(x, cu, tv.astype(np.float32), gv.astype(np.float32),
                                            EPS32, st, np.arange(len(lens)), np.array(hin),
                                            cond=True)
            fr = np.vectorize(Fraction, otypes=[object])
            yq, nsq = _exact_prefill(fr(xv).tolist(), cu.tolist(), fr(tv).tolist(),
                                     fr(gv).tolist(), EPS32,
                                     fr(zv).tolist() if R > 0 else None, hin)
            ye = np.array([[[float(v) for v in row] for row in tok] for tok in yq]).reshape(y.shape)
            err = np.abs(y - ye)
            lim = 1e-14 * (np.abs(ye) + cnd) + 1e-300
            assert (err <= lim).all(), f"exact mismatch {dtype} H={H} D={D} W={W} lens={lens}"
            if R > 0:
                nse = np.array([[[[float(v) for v in row] for row in r] for r in s] for s in nsq])
                got = oracle.widen(ns)
                assert np.array_equal(got.reshape(nse.shape), nse), f"state mismatch W={W} {lens}"


# ------------------------------------------------------------------------------------------------
# Library routines: depthwise conv1d and rms_norm (PyTorch CPU, fp64)
# ------------------------------------------------------------------------------------------------
def _torch_prefill(x64, cu, taps, gamma, eps, z64, has_init):
    T, H, D = x64.shape
    W = taps.shape[0]
    R = W - 1
    C = H * D
    weight = torch.from_numpy(np.ascontiguousarray(taps.reshape(W, C).T)).double().unsqueeze(1)
    out = np.zeros_like(x64)
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        if b == a:
            continue
        z = z64[s] if (z64 is not None and has_init[s]) else np.zeros((R, H, D))
        e = np.concatenate([z, x64[a:b]], axis=0).reshape(R + b - a, C).T[None]
        c = F.conv1d(torch.from_numpy(np.ascontiguousarray(e)), weight, groups=C)  # [1, C, L]
        c = c[0].T.reshape(b - a, H, D)
        yt = F.rms_norm(c, (D,), weight=torch.from_numpy(gamma.astype(np.float64)), eps=eps)
        out[a:b] = yt.numpy()
    return out


def pin_torch_conv1d_rmsnorm():
    """Oracle == torch fp64 conv1d(groups=channels) followed by rms_norm on random inputs."""
    for name in ("tiny_ref", "varlen_prefill"):
        w = workloads.config(name)
        st = w.steps[0]
        if name == "varlen_prefill":  # keep it quick: three of its sequences
            cut = int(st.cu_seqlens[3])
            st = workloads.Step("prefill", st.k[:cut], st.v[:cut], st.slot_mapping[:cut],
                                st.state_idx[:3], st.cu_seqlens[:4], np.array([1, 0, 1], np.uint8))
        y, _, cnd = oracle.prefill_one(st.k, st.cu_seqlens, w.k_taps, w.k_gamma, w.eps, w.k_state,
                                       st.state_idx, st.has_init, cond=True)
        z = oracle.widen(w.k_state)[st.state_idx] if w.k_state is not None else None
        yt = _torch_prefill(oracle.widen(st.k), st.cu_seqlens, w.k_taps, w.k_gamma, EPS32, z,
                            st.has_init)
        assert (np.abs(y - yt) <= 1e-12 * (np.abs(yt) + cnd)).all(), f"torch mismatch {name}"
    # a random multi-sequence case with initial states, W = 3, fp32, token-strided input
    spec = workloads.Spec(dtype="f32", H=3, D=64, W=3, seed=7, prefill_lens=[1, 9, 0, 33],
                          has_init=[1, 0, 1, 1], token_pad=5)
    w = workloads.build(spec)
    st = w.steps[0]
    y, _, cnd = oracle.prefill_one(st.v, st.cu_seqlens, w.v_taps, w.v_gamma, w.eps, w.v_state,
                                   st.state_idx, st.has_init, cond=True)
    yt = _torch_prefill(oracle.widen(np.ascontiguousarray(st.v)), st.cu_seqlens, w.v_taps,
                        w.v_gamma, EPS32, oracle.widen(w.v_state)[st.state_idx], st.has_init)
    assert (np.abs(y - yt) <= 1e-12 * (np.abs(yt) + cnd)).all(), "torch mismatch strided case"


def pin_w1_is_rmsnorm():
    """W = 1 with unit taps: the step is RMSNorm alone (torch fp64 rms_norm)."""
    for dtype in ("f32", "bf16"):
        spec = workloads.Spec(dtype=dtype, H=2, D=128, W=1, seed=3, prefill_lens=[7, 1, 20])
        w = workloads.build(spec)
        st = w.steps[0]
        taps = np.ones((1, 2, 128), np.float32)
        y, ns, _ = oracle.prefill_one(st.k, st.cu_seqlens, taps, w.k_gamma, w.eps, None,
                                      st.state_idx, st.has_init)
        assert ns is None
        yt = F.rms_norm(torch.from_numpy(oracle.widen(st.k)), (128,),
                        weight=torch.from_numpy(w.k_gamma.astype(np.float64)), eps=EPS32).numpy()
        assert np.allclose(y, yt, rtol=1e-14, atol=0), "W=1 is not rms_norm"


# ------------------------------------------------------------------------------------------------
# Closed forms
# ------------------------------------------------------------------------------------------------
def pin_closed_forms():
    D = 8
    gamma = np.array([1.0, 0.5, 2.0, 1.25, 0.75, 1.5, 3.0, 0.25], np.float32)
    one = np.ones((1, 1, D), np.float32)
    cu = np.array([0, 1])
    # a row of +-a with eps = 0: r = a, so y = sign * gamma exactly
    row = np.array([3, -3, 3, 3, -3, -3, 3, -3], np.float32).reshape(1, 1, D)
    y, _, _ = oracle.prefill_one(row, cu, one, gamma, 0.0, None, [0], [0])
    assert np.array_equal(y[0, 0], np.sign(row[0, 0]) * gamma.astype(np.float64))
    # (2,-2,2,-2,...) -> (1,-1,1,-1,...) * gamma
    row = np.array([2, -2] * 4, np.float32).reshape(1, 1, D)
    y, _, _ = oracle.prefill_one(row, cu, one, gamma, 0.0, None, [0], [0])
    assert np.array_equal(y[0, 0], np.array([1, -1] * 4) * gamma.astype(np.float64))
    # D = 2, c = (3, 4): mean square 12.5, so y = (3, 4) * sqrt(2) / 5 * gamma
    g2 = np.array([1.0, 2.0], np.float32)
    row = np.array([3, 4], np.float32).reshape(1, 1, 2)
    y, _, _ = oracle.prefill_one(row, cu, np.ones((1, 1, 2), np.float32), g2, 0.0, None, [0], [0])
    expect = np.array([3.0, 8.0]) * np.sqrt(2.0) / 5.0
    assert np.allclose(y[0, 0], expect, rtol=4e-16, atol=0)
    # W = 2, taps (1, -1): c is the first difference; x0 = (1..8), x1 = x0 + 2 -> c = 2 everywhere
    x = np.stack([np.arange(1, 9), np.arange(3, 11)]).astype(np.float32).reshape(2, 1, D)
    taps = np.stack([-np.ones(D), np.ones(D)]).astype(np.float32).reshape(2, 1, D)
    y, ns, _ = oracle.prefill_one(x, np.array([0, 2]), taps, gamma, 0.0,
                                  np.zeros((1, 1, 1, D), np.float32), [0], [1])
    assert np.array_equal(y[1, 0], gamma.astype(np.float64))          # c = 2 -> r = 2 -> gamma
    # first token: window (0, x0) -> c = x0 = (1..8), whose mean square is 51/2
    assert np.allclose(y[0, 0], np.arange(1, 9) / np.sqrt(25.5) * gamma, rtol=1e-15, atol=0)
    assert np.array_equal(ns[0, 0], x[1])                              # state = last row
    # eps dominates: c = 0 everywhere -> y = 0 (no division by zero)
    y, _, _ = oracle.prefill_one(np.zeros((1, 1, D), np.float32), cu, one, gamma, EPS32, None,
                                 [0], [0])
    assert np.array_equal(y, np.zeros_like(y))
    # eps is inside the square root: c = (1,...,1), eps = 3 -> y = gamma / 2
    y, _, _ = oracle.prefill_one(np.ones((1, 1, D), np.float32), cu, one, gamma, 3.0, None, [0],
                                 [0])
    assert np.array_equal(y[0, 0], gamma.astype(np.float64) / 2.0)


def pin_delta_taps():
    """Taps = unit vector at k: every output is an exact shift of the W = 1 unit-tap output
    (state rows standing in for positions before the sequence)."""
    for dtype in ("f32", "bf16"):
        W, H, D = 4, 2, 64
        spec = workloads.Spec(dtype=dtype, H=H, D=D, W=W, seed=11, prefill_lens=[10, 2, 6],
                              has_init=[1, 1, 0])
        w = workloads.build(spec)
        st = w.steps[0]
        cu = st.cu_seqlens
        for k in range(W):
            taps = np.zeros((W, H, D), np.float32)
            taps[k] = 1.0
            y, _, _ = oracle.prefill_one(st.k, cu, taps, w.k_gamma, w.eps, w.k_state,
                                         st.state_idx, st.has_init)
            # reference: W = 1 unit tap applied to the extended sequence e = [z, x]
            for s in range(len(cu) - 1):
                a, b = int(cu[s]), int(cu[s + 1])
                z = (w.k_state[st.state_idx[s]] if st.has_init[s]
                     else np.zeros((W - 1, H, D), w.k_state.dtype))
                e = np.concatenate([z, st.k[a:b]], axis=0)
                y1, _, _ = oracle.prefill_one(e, np.array([0, len(e)]), np.ones((1, H, D),
                                              np.float32), w.k_gamma, w.eps, None, [0], [0])
                assert np.array_equal(y[a:b], y1[k:k + b - a]), f"delta tap {k} seq {s}"


# ------------------------------------------------------------------------------------------------
# Invariants
# ------------------------------------------------------------------------------------------------
def _small(dtype="bf16", W=4, lens=(40, 3, 0, 17), hin=(1, 0, 1, 1), seed=5, H=2, D=64):
    spec = workloads.Spec(dtype=dtype, H=H, D=D, W=W, seed=seed, prefill_lens=list(lens),
                          has_init=list(hin))
    return workloads.build(spec)


def _run(w, st, k=None, state=None, hin=None, cu=None, sidx=None):
    return oracle.prefill_one(st.k if k is None else k, st.cu_seqlens if cu is None else cu,
                              w.k_taps, w.k_gamma, w.eps, w.k_state if state is None else state,
                              st.state_idx if sidx is None else sidx,
                              st.has_init if hin is None else hin)


def pin_causality():
    w = _small()
    st = w.steps[0]
    y0, _, _ = _run(w, st)
    for p in (0, 5, 38):
        k2 = st.k.copy()
        k2[p + 1:40] ^= np.uint16(0x0040)  # perturb every later token of sequence 0
        y1, _, _ = _run(w, st, k=k2)
        assert np.array_equal(y1[:p + 1], y0[:p + 1]), f"output <= {p} saw the future"
        assert not np.array_equal(y1[p + 1:40], y0[p + 1:40]), "perturbation had no effect"


def pin_no_leakage():
    w = _small()
    st = w.steps[0]
    cu = st.cu_seqlens
    y0, n0, _ = _run(w, st)
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        if b == a:
            continue
        k2 = st.k.copy()
        k2[a:b] ^= np.uint16(0x0100)
        y1, n1, _ = _run(w, st, k=k2)
        others = np.ones(len(y0), bool)
        others[a:b] = False
        assert np.array_equal(y1[others], y0[others]), f"sequence {s} leaked into another"
        keep = np.arange(len(cu) - 1) != s
        assert np.array_equal(n1[keep], n0[keep]), f"sequence {s} leaked into another state"
    # perturbing sequence s's initial state changes only its first W-1 outputs (if it reads it)
    W = w.W
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        st2 = w.k_state.copy()
        st2[st.state_idx[s]] ^= np.uint16(0x0100)
        y1, n1, _ = _run(w, st, state=st2)
        mask = np.zeros(len(y0), bool)
        if st.has_init[s]:
            mask[a:min(b, a + W - 1)] = True
        assert np.array_equal(y1[~mask], y0[~mask]), f"state of {s} reached too far"
        if mask.any():
            assert not np.array_equal(y1[mask], y0[mask]), f"state of {s} had no effect"


def pin_permutation():
    w = _small(lens=(7, 12, 1, 30), hin=(1, 0, 1, 1))
    st = w.steps[0]
    cu = st.cu_seqlens
    y0, n0, _ = _run(w, st)
    perm = [2, 0, 3, 1]
    pieces = [st.k[cu[s]:cu[s + 1]] for s in perm]
    lens = [len(p) for p in pieces]
    cu2 = np.concatenate([[0], np.cumsum(lens)])
    y1, n1, _ = _run(w, st, k=np.concatenate(pieces), cu=cu2, hin=st.has_init[perm],
                     sidx=st.state_idx[perm])
    for j, s in enumerate(perm):
        assert np.array_equal(y1[cu2[j]:cu2[j + 1]], y0[cu[s]:cu[s + 1]])
        assert np.array_equal(n1[j], n0[s])


def pin_decode_equals_prefill():
    """Token-by-token decode from the initial state == one-shot prefill, outputs and state."""
    for dtype, W in (("bf16", 4), ("f32", 8), ("bf16", 2)):
        w = _small(dtype=dtype, W=W, lens=(13, 2, 5), hin=(1, 1, 1))
        st = w.steps[0]
        cu = st.cu_seqlens
        y0, n0, _ = _run(w, st)
        pool = w.k_state.copy()
        for s in range(len(cu) - 1):
            for t in range(int(cu[s]), int(cu[s + 1])):
                yd, nd, _ = oracle.decode_one(st.k[t:t + 1], w.k_taps, w.k_gamma, w.eps, pool,
                                              st.state_idx[s:s + 1])
                assert np.array_equal(yd[0], y0[t]), f"decode != prefill at token {t}"
                pool[st.state_idx[s]] = nd[0]
            assert np.array_equal(pool[st.state_idx[s]], n0[s]), "decode state != prefill state"


def pin_chunked_equals_oneshot():
    for W in (3, 4, 8):
        w = _small(W=W, lens=(50, 9), hin=(1, 0))
        st = w.steps[0]
        cu = st.cu_seqlens
        y0, n0, _ = _run(w, st)
        for s in range(2):
            a, b = int(cu[s]), int(cu[s + 1])
            pool = w.k_state.copy()
            hin = int(st.has_init[s])
            pos = a
            for chunk in (1, W - 2, 7, 2, 100):
                e = min(b, pos + chunk)
                y1, n1, _ = oracle.prefill_one(st.k[pos:e], np.array([0, e - pos]), w.k_taps,
                                               w.k_gamma, w.eps, pool, st.state_idx[s:s + 1],
                                               np.array([hin]))
                assert np.array_equal(y1, y0[pos:e]), f"chunk [{pos},{e}) W={W}"
                pool[st.state_idx[s]] = n1[0]
                hin = 1
                pos = e
                if pos == b:
                    break
            assert pos == b
            assert np.array_equal(pool[st.state_idx[s]], n0[s]), "chunked state"


def pin_short_sequence_state():
    """A sequence shorter than W-1 shifts its new rows in behind the surviving old rows."""
    W, H, D = 6, 1, 64
    w = _small(W=W, lens=(2, 0), hin=(1, 1), H=H, D=D)
    st = w.steps[0]
    _, n0, _ = _run(w, st)
    old0 = w.k_state[st.state_idx[0]]
    assert np.array_equal(n0[0], np.concatenate([old0[2:], st.k[0:2]]))
    old1 = w.k_state[st.state_idx[1]]
    assert np.array_equal(n0[1], old1)                       # zero-length: state passes through
    _, n1, _ = _run(w, st, hin=np.array([0, 0], np.uint8))
    assert np.array_equal(n1[0], np.concatenate([np.zeros_like(old0[:3]), st.k[0:2]]))
    assert not n1[1].any()                                   # fresh and empty: zeros


def pin_scale_invariance():
    """With eps = 0, scaling every input by 2^j leaves the output unchanged (bitwise)."""
    w = _small(dtype="f32", lens=(20, 5), hin=(1, 1))
    st = w.steps[0]
    y0, _, _ = oracle.prefill_one(st.k, st.cu_seqlens, w.k_taps, w.k_gamma, 0.0, w.k_state,
                                  st.state_idx, st.has_init)
    for j in (-7, 3, 20):
        s = np.float32(2.0 ** j)
        y1, _, _ = oracle.prefill_one(st.k * s, st.cu_seqlens, w.k_taps, w.k_gamma, 0.0,
                                      w.k_state * s, st.state_idx, st.has_init)
        assert np.array_equal(y0, y1), f"not scale invariant at 2^{j}"


def pin_placement_and_pools():
    """Cache rows: negative and out-of-range slots are not written; state rows go to
    pool[state_idx] and out-of-pool indices leave the pool as it was."""
    assert np.array_equal(oracle.cache_slots([3, -1, 9, 10, 0], 10), [3, -1, 9, -1, 0])
    w = _small(lens=(4, 4, 4), hin=(1, 1, 1))
    st = w.steps[0]
    sidx = st.state_idx.copy()
    sidx[1] = w.k_state.shape[0] + 3          # out of the pool
    r = oracle.fused_prefill(st.k, st.v, st.cu_seqlens, w.k_taps, w.v_taps, w.k_gamma, w.v_gamma,
                             w.eps, w.k_state, w.v_state, sidx, st.has_init, st.slot_mapping,
                             w.num_slots, cond=False)
    untouched = np.setdiff1d(np.arange(w.k_state.shape[0]), sidx[[0, 2]])
    assert np.array_equal(r.k_state[untouched], w.k_state[untouched])
    # the sequence without a slot starts from zeros
    z = w.k_state.copy()
    z[:] = 0
    y_zero, _, _ = oracle.prefill_one(st.k, st.cu_seqlens, w.k_taps, w.k_gamma, w.eps, z,
                                      st.state_idx, st.has_init)
    assert np.array_equal(r.y_k[4:8], y_zero[4:8])


def pin_cond_scale():
    """The error scale the acceptance metric uses: |gamma| * sum_k |w_k e_k| / r. With all terms
    of one sign there is no cancellation, so it equals |y|; with cancellation it exceeds |y|."""
    g = np.random.default_rng(99)
    H, D, W = 2, 64, 4
    x = np.abs(g.standard_normal((9, H, D))).astype(np.float32) + 0.1
    taps = np.abs(g.standard_normal((W, H, D))).astype(np.float32) + 0.1
    gamma = (1.0 + 0.5 * g.random(D)).astype(np.float32)
    z = np.abs(g.standard_normal((1, W - 1, H, D))).astype(np.float32)
    for dec in (False, True):
        if dec:
            y, _, c = oracle.decode_one(x[:1], taps, gamma, EPS32, z, [0], cond=True)
        else:
            y, _, c = oracle.prefill_one(x, [0, 9], taps, gamma, EPS32, z, [0], [1], cond=True)
        assert np.allclose(c, np.abs(y), rtol=1e-14, atol=0), "cond != |y| without cancellation"
        taps2 = taps.copy()
        taps2[0] *= -1
        if dec:
            y2, _, c2 = oracle.decode_one(x[:1], taps2, gamma, EPS32, z, [0], cond=True)
        else:
            y2, _, c2 = oracle.prefill_one(x, [0, 9], taps2, gamma, EPS32, z, [0], [1], cond=True)
        assert (c2 >= np.abs(y2) * (1 - 1e-14)).all() and (c2 > np.abs(y2) * 1.01).any()


def pin_verify_snapshots_and_commit():
    """Per-token snapshots equal the state a prefill of the first i+1 tokens leaves, and the state
    token-by-token decode reaches; commit installs the snapshot of the accepted prefix."""
    for dtype, W in (("bf16", 4), ("f32", 8), ("bf16", 2)):
        lens = [3, 0, 1, 8, 6]
        w = _small(dtype=dtype, W=W, lens=lens, hin=[1] * len(lens), H=2, D=64)
        st = w.steps[0]
        cu = st.cu_seqlens
        K = 7  # max_tokens below the longest sequence: its 8th token gets no snapshot
        r, ks, _ = oracle.fused_verify(st.k, st.v, cu, w.k_taps, w.v_taps, w.k_gamma, w.v_gamma,
                                       w.eps, w.k_state, w.v_state, st.state_idx, st.slot_mapping,
                                       w.num_slots, K, cond=False)
        assert np.array_equal(r.k_state, w.k_state), "verify must not touch the pool"
        for s in range(len(lens)):
            a = int(cu[s])
            pool = w.k_state.copy()
            for i in range(min(lens[s], K)):
                # prefill of the first i+1 tokens from the stored state
                _, ns, _ = oracle.prefill_one(st.k[a:a + i + 1], np.array([0, i + 1]), w.k_taps,
                                              w.k_gamma, w.eps, w.k_state,
                                              st.state_idx[s:s + 1], np.array([1]))
                assert np.array_equal(ks[s, i], ns[0]), f"snapshot {s},{i} != prefill state"
                # token-by-token decode
                yd, nd, _ = oracle.decode_one(st.k[a + i:a + i + 1], w.k_taps, w.k_gamma, w.eps,
                                              pool, st.state_idx[s:s + 1])
                pool[st.state_idx[s]] = nd[0]
                assert np.array_equal(ks[s, i], nd[0]), f"snapshot {s},{i} != decode state"
                assert np.array_equal(yd[0], r.y_k[a + i]), f"verify output {s},{i} != decode"
        acc = np.array([2, 5, 0, 9, 6])
        new = oracle.commit_state(w.k_state, ks, acc, cu, st.state_idx, K)
        for s in range(len(lens)):
            m = min(acc[s], lens[s], K)
            if m == 0:
                assert np.array_equal(new[st.state_idx[s]], w.k_state[st.state_idx[s]])
            else:
                _, ns, _ = oracle.prefill_one(st.k[cu[s]:cu[s] + m], np.array([0, m]), w.k_taps,
                                              w.k_gamma, w.eps, w.k_state,
                                              st.state_idx[s:s + 1], np.array([1]))
                assert np.array_equal(new[st.state_idx[s]], ns[0]), f"commit of {s}"


def pin_mxfp8_codes():
    """E4M3: every finite code decodes and re-encodes to itself; every midpoint between adjacent
    values rounds to the even code and a hair either side rounds to the nearer one; values beyond
    448 saturate; the smallest subnormal and normal sit where the format puts them."""
    codes = np.arange(0x00, 0x7F, dtype=np.uint8)            # +0 .. 448, NaN (0x7F) excluded
    vals = oracle.e4m3_decode(codes)
    assert vals[0x01] == 2.0 ** -9 and vals[0x08] == 2.0 ** -6 and vals[0x7E] == 448.0
    assert np.isnan(oracle.e4m3_decode(np.array([0x7F, 0xFF]))).all()
    assert np.array_equal(oracle.e4m3_encode(vals), codes)
    assert np.array_equal(oracle.e4m3_encode(-vals[1:]), codes[1:] | 0x80)
    mids = (vals[:-1] + vals[1:]) / 2.0
    even = np.where(codes[:-1] % 2 == 0, codes[:-1], codes[1:])
    assert np.array_equal(oracle.e4m3_encode(mids), even), "ties must go to the even code"
    gap = vals[1:] - vals[:-1]
    assert np.array_equal(oracle.e4m3_encode(mids - gap * 1e-6), codes[:-1])
    assert np.array_equal(oracle.e4m3_encode(mids + gap * 1e-6), codes[1:])
    big = np.array([448.0, 448.5, 463.99, 464.0, 480.0, 511.9, 1e6])
    assert (oracle.e4m3_encode(big) == 0x7E).all() and (oracle.e4m3_encode(-big) == 0xFE).all()


def pin_mxfp8_blocks():
    """Shared scale = 2^(floor(log2 amax) - 8) per 32-element block; an all-zero block gets the
    smallest scale; dequantized values sit within half a code step (relative 2^-4) of the input
    unless the element saturates at 448 * X."""
    y = np.zeros((4, 64))
    y[0, :32] = np.linspace(-1.0, 1.0, 32)               # amax = 1 -> exponent -8
    y[0, 32:] = 3.0 * 2.0 ** -20                          # amax in [2^-19, 2^-18) -> -27
    y[1, :32] = 0.0
    y[1, 32:] = 1.99                                      # scaled 509.4 -> saturates to 448
    y[2] = np.random.default_rng(5).standard_normal(64) * 40.0
    y[3, :32] = 2.0 ** -130 * np.arange(1, 33) / 32.0     # amax 2^-130 -> -138, clamped to -127
    y[3, 32:] = 2.0 ** 140                                # -> 132, clamped to 127 (scaled 2^13)
    codes, scales = oracle.mxfp8_quantize(y)
    assert scales[0, 0] == 127 - 8 and scales[0, 1] == 127 - 27
    assert scales[1, 0] == 0 and (codes[1, :32] == 0).all()
    assert (codes[1, 32:] == 0x7E).all() and scales[1, 1] == 127 - 8
    assert codes[0, 31] == 0x78 and codes[0, 0] == 0xF8  # +-1.0 -> +-256 = 2^8 -> exponent field 15
    assert scales[3, 0] == 0 and scales[3, 1] == 254 and (codes[3, 32:] == 0x7E).all()
    # 2^-130 * k/32 * 2^127 = k * 2^-8: subnormal codes 2k (k <= 3), then normals
    assert codes[3, 0] == 2 and codes[3, 2] == 6 and codes[3, 3] == 0x08
    deq = oracle.mxfp8_dequantize(codes, scales)
    blocks = y.reshape(4, 2, 32)
    x = np.ldexp(1.0, scales.astype(np.int64) - 127)[..., None]
    sat = (np.abs(blocks) > 448.0 * x).reshape(4, 64)
    sub = (np.abs(blocks) < 2.0 ** -6 * x).reshape(4, 64)
    err = np.abs(deq - y)
    ok = ~sat & ~sub
    assert (err[ok] <= 2.0 ** -4 * np.abs(y[ok]) * (1 + 1e-12)).all()
    assert np.allclose(deq[sat], np.sign(y[sat]) * 448.0 * np.repeat(x.reshape(4, 2), 32, 1)[sat])


# ------------------------------------------------------------------------------------------------
# Backward (the gradients of the step, for training)
# ------------------------------------------------------------------------------------------------
def _bwd_case(dtype="f32", W=4, H=2, D=8, lens=(6, 2, 0, 9), hin=(1, 0, 1, 1), seed=11, eps=None):
    spec = workloads.Spec(dtype=dtype, H=H, D=D, W=W, seed=seed, prefill_lens=list(lens),
                          has_init=list(hin))
    if eps is not None:
        spec.eps = eps
    w = workloads.build(spec)
    st = w.steps[0]
    g = np.random.default_rng(seed).standard_normal((st.tokens, H, D))
    gs = (np.random.default_rng(seed + 1).standard_normal((st.num_seqs, W - 1, H, D))
          if W > 1 else None)
    return w, st, g, gs


def _loss(w, st, g, gs, x=None, taps=None, gamma=None, state=None):
    """sum(g * y) + sum(gs * new state), through the forward oracle."""
    y, ns, _ = oracle.prefill_one(st.k if x is None else x, st.cu_seqlens,
                                  w.k_taps if taps is None else taps,
                                  w.k_gamma if gamma is None else gamma, w.eps,
                                  w.k_state if state is None else state, st.state_idx,
                                  st.has_init)
    total = float((g * y).sum())
    if gs is not None:
        total += float((gs * oracle.widen(ns)).sum())
    return total


def _central_differences(f, arr, h=2.0 ** -12):
    """d f / d arr by central differences; arr is fp32, and arr +- h is exact in fp32 for every
    |value| < 2^11, so the only errors are the O(h^2) truncation and fp64 roundoff."""
    out = np.zeros(arr.shape, np.float64)
    flat = arr.reshape(-1)
    for i in range(flat.size):
        keep = flat[i]
        flat[i] = keep + np.float32(h)
        up = f()
        flat[i] = keep - np.float32(h)
        down = f()
        flat[i] = keep
        out.reshape(-1)[i] = (up - down) / (2.0 * h)
    return out


def pin_backward_finite_differences():
    """Every gradient of the backward oracle equals the central difference of the forward
    oracle's loss sum(g*y) + sum(gs*new_state): input rows, taps, gamma and the state pool
    (through has_init, an empty sequence and one shorter than the window)."""
    for W in (4, 2):
        w, st, g, gs = _bwd_case(W=W)
        gr = oracle.backward_one(st.k, st.cu_seqlens, w.k_taps, w.k_gamma, w.eps, w.k_state,
                                 st.state_idx, st.has_init, g, gs)
        x = st.k.copy()
        taps = w.k_taps.copy()
        gamma = w.k_gamma.copy()
        pool = w.k_state.copy()
        fd_x = _central_differences(lambda: _loss(w, st, g, gs, x=x), x)
        fd_t = _central_differences(lambda: _loss(w, st, g, gs, taps=taps), taps)
        fd_g = _central_differences(lambda: _loss(w, st, g, gs, gamma=gamma), gamma)
        fd_s = _central_differences(lambda: _loss(w, st, g, gs, state=pool), pool)
        an_s = np.zeros_like(fd_s)
        for s in range(st.num_seqs):
            an_s[st.state_idx[s]] += gr.dstate[s]
        for name, fd, an in (("dx", fd_x, gr.dx), ("dtaps", fd_t, gr.dtaps),
                             ("dgamma", fd_g, gr.dgamma), ("dstate", fd_s, an_s)):
            assert np.allclose(an, fd, rtol=1e-6, atol=1e-6), \
                f"{name} != finite differences (W={W})"
    # bf16 storage changes nothing but the widening: same values stored as fp32 give the same
    # gradients, bit for bit
    w, st, g, gs = _bwd_case(dtype="bf16")
    a = oracle.backward_one(st.k, st.cu_seqlens, w.k_taps, w.k_gamma, w.eps, w.k_state,
                            st.state_idx, st.has_init, g, gs)
    b = oracle.backward_one(workloads.bf16_bits_to_f32(st.k), st.cu_seqlens, w.k_taps, w.k_gamma,
                            w.eps, workloads.bf16_bits_to_f32(w.k_state), st.state_idx,
                            st.has_init, g, gs)
    for f in ("dx", "dtaps", "dgamma", "dstate"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f"bf16 {f}"


def pin_backward_torch_autograd():
    """The backward oracle == PyTorch fp64 autograd through conv1d(groups=channels) and rms_norm,
    with the initial state prepended and a loss on the new state."""
    for W, dtype in ((4, "bf16"), (3, "f32")):
        w, st, g, gs = _bwd_case(dtype=dtype, W=W, H=3, D=64, lens=(20, 1, 0, 37), hin=(1, 1, 0, 1),
                                 seed=21)
        gr = oracle.backward_one(st.k, st.cu_seqlens, w.k_taps, w.k_gamma, w.eps, w.k_state,
                                 st.state_idx, st.has_init, g, gs)
        H, D, R, C = 3, 64, W - 1, 3 * 64
        x = torch.from_numpy(oracle.widen(st.k)).requires_grad_()
        taps = torch.from_numpy(w.k_taps.astype(np.float64)).requires_grad_()
        gamma = torch.from_numpy(w.k_gamma.astype(np.float64)).requires_grad_()
        z = torch.from_numpy(oracle.widen(w.k_state)[st.state_idx]).requires_grad_()
        weight = taps.reshape(W, C).T.unsqueeze(1)
        loss = torch.zeros((), dtype=torch.float64)
        cu = st.cu_seqlens
        for s in range(st.num_seqs):
            a, b = int(cu[s]), int(cu[s + 1])
            zs = z[s] if st.has_init[s] else torch.zeros((R, H, D), dtype=torch.float64)
            e = torch.cat([zs, x[a:b]], 0)
            if b > a:
                c = F.conv1d(e.reshape(R + b - a, C).T[None], weight, groups=C)[0].T
                y = F.rms_norm(c.reshape(b - a, H, D), (D,), weight=gamma, eps=EPS32)
                loss = loss + (torch.from_numpy(g[a:b]) * y).sum()
            loss = loss + (torch.from_numpy(gs[s]) * e[b - a:b - a + R]).sum()
        loss.backward()
        for name, ours, ref in (("dx", gr.dx, x.grad), ("dtaps", gr.dtaps, taps.grad),
                                ("dgamma", gr.dgamma, gamma.grad), ("dstate", gr.dstate, z.grad)):
            ref = ref.numpy()
            assert np.allclose(ours, ref, rtol=1e-10, atol=1e-10 * np.abs(ref).max()), \
                f"{name} != torch autograd (W={W}, {dtype})"


def pin_backward_invariants():
    """Euler's theorem on the loss sum(g*y) + sum(gs*new_state), exact in exact arithmetic:
    with eps = 0, y is invariant to scaling one head's taps, so sum_k,d dtaps*taps = 0 per head;
    y is invariant and the new state homogeneous of degree 1 in (x, initial window), so
    sum dx*x + sum dstate*z = sum gs*new_state; and y is linear in gamma, so
    sum dgamma*gamma = sum g*y (any eps)."""
    for W in (4, 8, 1):
        w, st, g, gs = _bwd_case(W=W, D=64, lens=(12, 2, 30), hin=(1, 1, 0), eps=0.0, seed=31)
        gr = oracle.backward_one(st.k, st.cu_seqlens, w.k_taps, w.k_gamma, w.eps, w.k_state,
                                 st.state_idx, st.has_init, g, gs)
        t64 = w.k_taps.astype(np.float64)
        per_head = (gr.dtaps * t64).sum(axis=(0, 2))
        scale = np.abs(gr.dtaps * t64).sum(axis=(0, 2))
        assert (np.abs(per_head) <= 1e-12 * scale).all(), f"taps scale invariance (W={W})"
        y, ns, _ = oracle.prefill_one(st.k, st.cu_seqlens, w.k_taps, w.k_gamma, w.eps, w.k_state,
                                      st.state_idx, st.has_init)
        x64 = oracle.widen(st.k)
        lhs_terms = [gr.dx * x64]
        rhs = 0.0
        if W > 1:
            z = oracle.widen(w.k_state)[st.state_idx] * st.has_init[:, None, None, None]
            lhs_terms.append(gr.dstate * z)
            rhs = float((gs * oracle.widen(ns)).sum())
        lhs = sum(float(t.sum()) for t in lhs_terms)
        mag = sum(float(np.abs(t).sum()) for t in lhs_terms) + abs(rhs)
        assert abs(lhs - rhs) <= 1e-12 * mag, f"input homogeneity (W={W})"
        gy = float((g * y).sum())
        dg = float((gr.dgamma * w.k_gamma.astype(np.float64)).sum())
        assert abs(dg - gy) <= 1e-12 * float(np.abs(g * y).sum()), f"gamma linearity (W={W})"


def pin_backward_locality():
    """The input gradient of token t depends on rows t-R .. t+R only: the full sequence's dx[t]
    equals the first row's gradient of the short sequence t .. t+R (cut at the sequence's end)
    that resumes from rows t-R .. t-1 as its stored state."""
    for W in (4, 2, 7):
        R = W - 1
        w, st, g, _ = _bwd_case(W=W, D=64, lens=(30, 5), hin=(1, 1), seed=41)
        full = oracle.backward_one(st.k, st.cu_seqlens, w.k_taps, w.k_gamma, w.eps, w.k_state,
                                   st.state_idx, st.has_init, g)
        x64 = st.k
        for s in range(2):
            a, b = int(st.cu_seqlens[s]), int(st.cu_seqlens[s + 1])
            z = w.k_state[st.state_idx[s]]
            e = np.concatenate([z, x64[a:b]], axis=0)  # stored rows, state first
            for p in range(b - a):
                rows = e[p + R: min(p + R + 1 + R, R + b - a)]
                st_rows = e[p:p + R][None]
                n = rows.shape[0]
                part = oracle.backward_one(np.ascontiguousarray(rows), np.array([0, n]), w.k_taps,
                                           w.k_gamma, w.eps, np.ascontiguousarray(st_rows),
                                           np.array([0]), np.array([1]), g[a + p:a + p + n])
                assert np.allclose(part.dx[0], full.dx[a + p], rtol=1e-12, atol=1e-12), \
                    f"locality of dx (W={W}, seq {s}, token {p})"


def pin_backward_chunked_equals_oneshot():
    """Chunked training: splitting sequences into two chunks (the second resuming from the
    first's new state) and feeding the second chunk's initial-window gradient to the first as
    its new-state gradient gives the one-shot input, tap and gamma gradients."""
    for W in (4, 2, 8):
        w, st, g, gs = _bwd_case(W=W, D=64, lens=(40, 11), hin=(1, 0), seed=51)
        one = oracle.backward_one(st.k, st.cu_seqlens, w.k_taps, w.k_gamma, w.eps, w.k_state,
                                  st.state_idx, st.has_init, g, gs)
        cut = (17, 5)  # split points inside each sequence
        cu = st.cu_seqlens
        idx1 = np.concatenate([np.arange(cu[s], cu[s] + cut[s]) for s in range(2)])
        idx2 = np.concatenate([np.arange(cu[s] + cut[s], cu[s + 1]) for s in range(2)])
        cu1 = np.array([0, cut[0], cut[0] + cut[1]])
        cu2 = np.array([0, 40 - cut[0], 40 - cut[0] + 11 - cut[1]])
        _, mid, _ = oracle.prefill_one(st.k[idx1], cu1, w.k_taps, w.k_gamma, w.eps, w.k_state,
                                       st.state_idx, st.has_init)
        second = oracle.backward_one(st.k[idx2], cu2, w.k_taps, w.k_gamma, w.eps, mid,
                                     np.arange(2), np.ones(2, np.uint8), g[idx2], gs)
        first = oracle.backward_one(st.k[idx1], cu1, w.k_taps, w.k_gamma, w.eps, w.k_state,
                                    st.state_idx, st.has_init, g[idx1], second.dstate)
        dx = np.zeros_like(one.dx)
        dx[idx1], dx[idx2] = first.dx, second.dx
        pairs = (("dx", dx, one.dx), ("dtaps", first.dtaps + second.dtaps, one.dtaps),
                 ("dgamma", first.dgamma + second.dgamma, one.dgamma),
                 ("dstate", first.dstate, one.dstate))
        for name, a, b in pairs:
            assert np.allclose(a, b, rtol=1e-11, atol=1e-11 * np.abs(b).max()), \
                f"chunked {name} (W={W})"


ALL_PINS = [
    pin_exact_rational,
    pin_torch_conv1d_rmsnorm,
    pin_w1_is_rmsnorm,
    pin_closed_forms,
    pin_delta_taps,
    pin_causality,
    pin_no_leakage,
    pin_permutation,
    pin_decode_equals_prefill,
    pin_chunked_equals_oneshot,
    pin_short_sequence_state,
    pin_scale_invariance,
    pin_placement_and_pools,
    pin_cond_scale,
    pin_verify_snapshots_and_commit,
    pin_mxfp8_codes,
    pin_mxfp8_blocks,
    pin_backward_finite_differences,
    pin_backward_torch_autograd,
    pin_backward_invariants,
    pin_backward_locality,
    pin_backward_chunked_equals_oneshot,
]
