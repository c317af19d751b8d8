"""A 2^20-token sequence (the pages' 1M-token context) through the prefill and its backward, checked
on sampled tokens against the oracle.

Each output of token t depends only on rows t-R .. t (prefill; R = W-1) or t-R .. t+R (input
gradient), so the oracle computes a sampled token exactly from a short sequence of those rows
whose initial state is the R rows before them. Inputs are drawn on the device from a seeded
generator (4 GB of K/V); only the rows the checks need come back to the host. The new state is
compared bit for bit, untouched cache rows keep their sentinel.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_harness import DEV, ORACLE_THREADS, to_dev, to_host
from causal_short_convolution_amd import shortconv_kv_backward, shortconv_kv_prefill

pytestmark = pytest.mark.gpu

H, D, W = 8, 128, 4
R = W - 1
LENS = [1 << 20, 37, 5]
HAS_INIT = [1, 0, 1]
BLOCK = 64


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.fixture(scope="module")
def case():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    spec = workloads.Spec(dtype="bf16", H=H, D=D, W=W, seed=77, prefill_lens=[1, 1, 1],
                          has_init=HAS_INIT)
    params = workloads.build(spec)  # taps, gamma, state pool and state slots (seeded)
    T = sum(LENS)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(20240520)
    k = torch.randn((T, H, D), generator=gen, device=DEV).to(torch.bfloat16)
    v = torch.randn((T, H, D), generator=gen, device=DEV).to(torch.bfloat16)
    # paged cache: one random permutation of the pool's 64-token blocks as block tables
    rng = np.random.default_rng(77)
    nblk = [(n + BLOCK - 1) // BLOCK for n in LENS]
    perm = rng.permutation(sum(nblk)).astype(np.int64)
    slots, first = [], 0
    for n, nb in zip(LENS, nblk):
        pos = np.arange(n, dtype=np.int64)
        slots.append(perm[first:first + nb][pos // BLOCK] * BLOCK + pos % BLOCK)
        first += nb
    slot = np.concatenate(slots)
    num_slots = sum(nblk) * BLOCK
    cu = np.concatenate([[0], np.cumsum(LENS)]).astype(np.int32)
    return dict(p=params, k=k, v=v, slot=slot, num_slots=num_slots, cu=cu, T=T)


def _samples(rng):
    """Sampled (sequence, position) pairs: random positions of the long sequence, its first
    rows, tile and span boundaries, its end, and every row of the short sequences."""
    L = LENS[0]
    pts = set(rng.integers(0, L, size=1500).tolist())
    pts |= {0, 1, 2, 3, 4, 7, 8, 9, 31, 32, 33, 63, 64, 65, L - 1, L - 2, L - 3, L - 4, L - 33}
    pts |= {j * 32 + d for j in rng.integers(1, L // 32, size=100).tolist() for d in (-1, 0, 1)}
    out = [(0, p) for p in sorted(pts) if 0 <= p < L]
    for s in (1, 2):
        out += [(s, p) for p in range(LENS[s])]
    return out


def _window_rows(x, c, params_state, sidx, s, p, before, after):
    """Rows e[p .. p+before] (the initial-state part from the pool or zeros) and x rows
    p+1 .. p+after of sequence s, as host bf16 bits [before + 1 + after, H, D]."""
    start, end = int(c["cu"][s]), int(c["cu"][s + 1])
    rows = []
    for q in range(p - before, p + 1 + after):
        if q < 0:
            if HAS_INIT[s]:
                rows.append(params_state[sidx[s]][R + q])
            else:
                rows.append(np.zeros((H, D), np.uint16))
        elif start + q < end:
            rows.append(None)
        else:
            break
    need = [start + q for q in range(p - before, p + 1 + after) if q >= 0 and start + q < end]
    got = _bits(x[torch.tensor(need, device=DEV)]) if need else np.zeros((0, H, D), np.uint16)
    it = iter(got)
    return np.stack([r if r is not None else next(it) for r in rows])


def test_million_token_prefill_sampled(case):
    c = case
    w = c["p"]
    kc = torch.empty((c["num_slots"], H, D), dtype=torch.bfloat16, device=DEV)
    vc = torch.empty_like(kc)
    kc.view(torch.int16).fill_(0x5A5A)
    vc.view(torch.int16).fill_(0x5A5A)
    ks, vs = to_dev(w.k_state), to_dev(w.v_state)
    sidx = w.steps[0].state_idx
    shortconv_kv_prefill(c["k"], c["v"], to_dev(c["cu"]), to_dev(w.k_taps), to_dev(w.v_taps),
                         to_dev(w.k_gamma), to_dev(w.v_gamma), w.eps, ks, vs,
                         to_dev(sidx.astype(np.int32)), to_dev(np.array(HAS_INIT, np.uint8)),
                         to_dev(c["slot"]), kc, vc)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    samples = _samples(rng)
    for name, x, cache, taps, gamma, pool in (("K", c["k"], kc, w.k_taps, w.k_gamma, w.k_state),
                                             ("V", c["v"], vc, w.v_taps, w.v_gamma, w.v_state)):
        # oracle: one-token sequences whose initial state is the R rows before the token
        win = np.stack([_window_rows(x, c, pool, sidx, s, p, R, 0) for s, p in samples])
        n = len(samples)
        y, _, cnd = oracle.prefill_one(np.ascontiguousarray(win[:, R]), np.arange(n + 1),
                                       taps, gamma, w.eps, np.ascontiguousarray(win[:, :R]),
                                       np.arange(n), np.ones(n, np.uint8), cond=True,
                                       nthreads=ORACLE_THREADS)
        toks = np.array([int(c["cu"][s]) + p for s, p in samples])
        got = _bits(cache[torch.from_numpy(c["slot"][toks]).to(DEV)])
        res = oracle.compare(got, y, cnd, "bf16")
        assert res["ok"], f"{name}: sampled cache rows differ from the oracle: {res}"
        # the new state of every sequence: its last R raw rows, bit for bit
        new = _bits(ks if name == "K" else vs)
        for s in range(3):
            L = LENS[s]
            exp = _window_rows(x, c, pool, sidx, s, L - 1, R - 1, 0)
            assert np.array_equal(new[sidx[s]], exp), f"{name}: state of sequence {s}"
    # a sample of rows no token maps to keep the sentinel
    used = np.zeros(c["num_slots"], bool)
    used[c["slot"]] = True
    free = np.flatnonzero(~used)
    pick = free[rng.integers(0, free.size, size=min(2048, free.size))]
    for cache in (kc, vc):
        assert (_bits(cache[torch.from_numpy(pick).to(DEV)]) == 0x5A5A).all()


def test_million_token_backward_sampled(case):
    c = case
    w = c["p"]
    T = c["T"]
    gen = torch.Generator(device=DEV)
    gen.manual_seed(99)
    dyk = torch.randn((T, H, D), generator=gen, device=DEV).to(torch.bfloat16)
    dyv = torch.randn((T, H, D), generator=gen, device=DEV).to(torch.bfloat16)
    dk, dv = torch.empty_like(dyk), torch.empty_like(dyv)
    grads = [torch.empty((W, H, D), device=DEV) for _ in range(2)] + \
            [torch.empty((D,), device=DEV) for _ in range(2)]
    sidx = w.steps[0].state_idx
    shortconv_kv_backward(c["k"], c["v"], to_dev(c["cu"]), to_dev(w.k_taps), to_dev(w.v_taps),
                          to_dev(w.k_gamma), to_dev(w.v_gamma), w.eps, to_dev(w.k_state),
                          to_dev(w.v_state), to_dev(sidx.astype(np.int32)),
                          to_dev(np.array(HAS_INIT, np.uint8)), dyk, dyv, dk, dv, *grads)
    torch.cuda.synchronize()
    assert all(torch.isfinite(t).all() for t in grads)
    rng = np.random.default_rng(6)
    samples = _samples(rng)[::2]
    for name, x, dy, dx, taps, gamma, pool in (
            ("K", c["k"], dyk, dk, w.k_taps, w.k_gamma, w.k_state),
            ("V", c["v"], dyv, dv, w.v_taps, w.v_gamma, w.v_state)):
        # the input gradient of token t: a short sequence of rows t .. t+R whose initial state is
        # the R rows before t; its first row's gradient is dx[t]
        xs, ss, gs, cu = [], [], [], [0]
        for s, p in samples:
            rows = _window_rows(x, c, pool, sidx, s, p, R, R)
            n_after = rows.shape[0] - (R + 1)
            start = int(c["cu"][s])
            ss.append(rows[:R])
            xs.append(rows[R:])
            idx = torch.arange(start + p, start + p + 1 + n_after, device=DEV)
            gs.append(oracle.widen(_bits(dy[idx])))
            cu.append(cu[-1] + 1 + n_after)
        x_cat = np.concatenate(xs)
        g_cat = np.concatenate(gs)
        n = len(samples)
        ref = oracle.backward_one(x_cat, np.array(cu), taps, gamma, w.eps, np.stack(ss),
                                  np.arange(n), np.ones(n, np.uint8), g_cat, cond=True,
                                  nthreads=ORACLE_THREADS)
        first = np.array(cu[:-1])
        toks = np.array([int(c["cu"][s]) + p for s, p in samples])
        got = oracle.widen(_bits(dx[torch.from_numpy(toks).to(DEV)]))
        exact, cond = ref.dx[first], ref.cond_dx[first]
        bound = 3.9e-3 * np.abs(exact) + 64 * 2.0 ** -24 * cond
        assert (np.abs(got - exact) <= bound).all(), f"{name}: sampled input gradients differ"
