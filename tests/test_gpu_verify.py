"""GPU parity of speculative verification (per-token conv-state snapshots) and of the commit of
an accepted prefix, against the oracle; plus the bit-exact relations to prefill."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_harness import (BITS_DT, DEV, TORCH_DT, DeviceWorkload, judge, rows_to_dev, to_dev,
                         to_host)
from causal_short_convolution_amd import (shortconv_kv_prefill, shortconv_kv_verify,
                                          shortconv_state_commit)

pytestmark = pytest.mark.gpu

SNAP_SENTINEL = {"f32": 0x3C3C3C3C, "bf16": 0x3C3C}


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _verify_workload(dtype, H, D, W, lens, seed):
    spec = workloads.Spec(dtype=dtype, H=H, D=D, W=W, seed=seed, prefill_lens=lens,
                          has_init=[1] * len(lens), block_size=16, pad_slot_every=11)
    return workloads.build(spec)


def _snap_buffer(w, n, max_tokens):
    if w.W == 1:
        return None, None
    shape = (n, max_tokens, w.W - 1, w.H, w.D)
    bufs = []
    for _ in range(2):
        t = torch.empty(shape, dtype=TORCH_DT[w.dtype], device=DEV)
        t.view(BITS_DT[w.dtype]).fill_(SNAP_SENTINEL[w.dtype])
        bufs.append(t)
    return bufs


def _run_verify(w, max_tokens):
    dw = DeviceWorkload(w)
    d = dw.steps[0]
    ks, vs = _snap_buffer(w, w.steps[0].num_seqs, max_tokens)
    shortconv_kv_verify(d["k"], d["v"], d["cu"], dw.k_taps, dw.v_taps, dw.k_gamma, dw.v_gamma,
                        w.eps, dw.k_state, dw.v_state, d["sidx"], ks, vs, d["slot"], dw.k_cache,
                        dw.v_cache)
    torch.cuda.synchronize()
    return dw, ks, vs


def _check_snaps(w, got, exp, lens, max_tokens):
    g = to_host(got, w.dtype)
    for s, L in enumerate(lens):
        n = min(L, max_tokens)
        assert np.array_equal(g[s, :n], exp[s, :n]), f"snapshots of sequence {s}"
        rest = g[s, n:].view(np.uint32 if w.dtype == "f32" else np.uint16)
        assert (rest == SNAP_SENTINEL[w.dtype]).all(), f"snapshot past the run of sequence {s}"


CASES = [("bf16", 8, 128, 4), ("f32", 2, 64, 8), ("bf16", 3, 256, 2), ("bf16", 4, 128, 1),
         ("f32", 1, 128, 5)]


@pytest.mark.parametrize("dtype,H,D,W", CASES, ids=[f"{a}-H{b}-D{c}-W{d}" for a, b, c, d in CASES])
def test_verify_matches_oracle(dtype, H, D, W):
    lens = [1, 4, 0, 8, 3, 17, 40, 2]
    max_tokens = 20  # below the longest run: its last tokens get no snapshot
    w = _verify_workload(dtype, H, D, W, lens, seed=200 + W)
    st = w.steps[0]
    dw, ks, vs = _run_verify(w, max_tokens)
    r, eks, evs = oracle.fused_verify(st.k, st.v, st.cu_seqlens, w.k_taps, w.v_taps, w.k_gamma,
                                      w.v_gamma, w.eps, w.k_state, w.v_state, st.state_idx,
                                      st.slot_mapping, w.num_slots, max_tokens)
    judge(dw, results=[r])  # cache rows, sentinel rows, and the pools left untouched
    if W > 1:
        _check_snaps(w, ks, eks, lens, max_tokens)
        _check_snaps(w, vs, evs, lens, max_tokens)


def test_verify_equals_prefill_bitwise():
    lens = [5, 1, 16, 9]
    w = _verify_workload("bf16", 8, 128, 4, lens, seed=7)
    dw, ks, _ = _run_verify(w, 16)
    pre = DeviceWorkload(w)
    pre.run()
    for a, b in ((dw.k_cache, pre.k_cache), (dw.v_cache, pre.v_cache)):
        assert np.array_equal(to_host(a, "bf16"), to_host(b, "bf16"))
    # the last snapshot of each run is the state prefill leaves
    st = w.steps[0]
    snaps = to_host(ks, "bf16")
    pool = to_host(pre.k_state, "bf16")
    for s, L in enumerate(lens):
        assert np.array_equal(snaps[s, L - 1], pool[st.state_idx[s]])


def test_commit_matches_oracle():
    lens = [3, 0, 6, 1, 8]
    max_tokens = 8
    w = _verify_workload("bf16", 8, 128, 4, lens, seed=9)
    st = w.steps[0]
    dw, ks, vs = _run_verify(w, max_tokens)
    accepted = np.array([2, 3, 0, 1, 8], np.int32)
    shortconv_state_commit(ks, vs, dw.steps[0]["cu"], st.tokens, to_dev(accepted), dw.k_state,
                           dw.v_state, dw.steps[0]["sidx"], width=w.W, num_heads=w.H,
                           head_dim=w.D)
    torch.cuda.synchronize()
    _, eks, evs = oracle.fused_verify(st.k, st.v, st.cu_seqlens, w.k_taps, w.v_taps, w.k_gamma,
                                      w.v_gamma, w.eps, w.k_state, w.v_state, st.state_idx,
                                      st.slot_mapping, w.num_slots, max_tokens, cond=False)
    for dev, pool, snaps in ((dw.k_state, w.k_state, eks), (dw.v_state, w.v_state, evs)):
        exp = oracle.commit_state(pool, snaps, accepted, st.cu_seqlens, st.state_idx, max_tokens)
        assert np.array_equal(to_host(dev, "bf16"), exp)


def test_speculative_rounds_match_prefill_of_accepted_tokens():
    """Three rounds of verify + commit with random acceptance leave every state exactly where a
    prefill of only the accepted tokens leaves it."""
    H, D, W, N, K = 8, 128, 4, 6, 5
    g = np.random.default_rng(11)
    base = workloads.build(workloads.Spec(dtype="bf16", H=H, D=D, W=W, seed=12,
                                          prefill_lens=[1] * N, has_init=[1] * N))
    taps = to_dev(base.k_taps)
    gam = to_dev(base.k_gamma)
    pool = to_dev(base.k_state)
    sidx = to_dev(base.steps[0].state_idx)
    accepted_rows = [[] for _ in range(N)]
    for rnd in range(3):
        x = workloads._normal_stored(workloads.rng(13, rnd, 0), (N * K, H, D), "bf16")
        cu = np.arange(0, N * K + 1, K, dtype=np.int32)
        xd = rows_to_dev(x)
        snaps = torch.empty((N, K, W - 1, H, D), dtype=torch.bfloat16, device=DEV)
        cache = torch.zeros((N * K, H, D), dtype=torch.bfloat16, device=DEV)
        slots = torch.arange(N * K, dtype=torch.int64, device=DEV)
        shortconv_kv_verify(xd, xd, to_dev(cu), taps, taps, gam, gam, base.eps, pool, pool.clone(),
                            sidx, snaps, snaps.clone(), slots, cache, cache.clone())
        acc = g.integers(0, K + 1, size=N).astype(np.int32)
        shortconv_state_commit(snaps, snaps.clone(), to_dev(cu), N * K, to_dev(acc), pool,
                               pool.clone(), sidx, width=W, num_heads=H, head_dim=D)
        for s in range(N):
            accepted_rows[s].extend(x[s * K:s * K + acc[s]])
    torch.cuda.synchronize()
    got = to_host(pool, "bf16")
    for s in range(N):
        rows = (np.stack(accepted_rows[s]) if accepted_rows[s]
                else np.zeros((0, H, D), np.uint16))
        _, ns, _ = oracle.prefill_one(rows, np.array([0, len(rows)]), base.k_taps, base.k_gamma,
                                      base.eps, base.k_state, base.steps[0].state_idx[s:s + 1],
                                      np.array([1]))
        assert np.array_equal(got[base.steps[0].state_idx[s]], ns[0]), f"sequence {s}"


def test_verify_commit_graph_replay_matches_eager():
    """Verify + commit captured in a HIP graph: every replay, with the pools, caches and
    snapshots restored or cleared eagerly in between, gives the eager run's bits."""
    lens = [4, 1, 0, 4, 3]
    max_tokens = 4
    w = _verify_workload("bf16", 8, 128, 4, lens, seed=21)
    st = w.steps[0]
    accepted = to_dev(np.array([3, 1, 0, 4, 2], np.int32))
    dw = DeviceWorkload(w)
    d = dw.steps[0]
    ks, vs = _snap_buffer(w, st.num_seqs, max_tokens)
    k0, v0 = dw.k_state.clone(), dw.v_state.clone()

    def step():
        shortconv_kv_verify(d["k"], d["v"], d["cu"], dw.k_taps, dw.v_taps, dw.k_gamma,
                            dw.v_gamma, w.eps, dw.k_state, dw.v_state, d["sidx"], ks, vs,
                            d["slot"], dw.k_cache, dw.v_cache)
        shortconv_state_commit(ks, vs, d["cu"], st.tokens, accepted, dw.k_state, dw.v_state,
                               d["sidx"], width=w.W, num_heads=w.H, head_dim=w.D)

    def outputs():
        return [to_host(t, "bf16") for t in (dw.k_cache, dw.v_cache, dw.k_state, dw.v_state,
                                             ks, vs)]

    step()
    torch.cuda.synchronize()
    eager = outputs()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(3):
        dw.k_state.copy_(k0)
        dw.v_state.copy_(v0)
        for t in (dw.k_cache, dw.v_cache, ks, vs):
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = outputs()
        rows = st.slot_mapping[st.slot_mapping >= 0]
        for a, b in zip(got[:2], eager[:2]):
            assert np.array_equal(a[rows], b[rows])
        for name, a, b in zip(("k_state", "v_state"), got[2:4], eager[2:4]):
            assert np.array_equal(a, b), name
        for s, L in enumerate(lens):  # snapshots that exist (the rest were zeroed)
            n = min(L, max_tokens)
            for a, b in zip(got[4:], eager[4:]):
                assert np.array_equal(a[s, :n], b[s, :n]), f"snapshots of sequence {s}"


def test_spec_verify_workload_at_full_size():
    """The bench's speculative step (workloads.spec_verify: 256 sequences x 4 candidate tokens,
    decode-sized paged pool) at full size: cache rows against the oracle, every snapshot and the
    committed pools bit for bit."""
    w, accepted = workloads.spec_verify(0)
    st = w.steps[0]
    mt = workloads.SPEC_TOKENS
    dw, ks, vs = _run_verify(w, mt)
    r, eks, evs = oracle.fused_verify(st.k, st.v, st.cu_seqlens, w.k_taps, w.v_taps, w.k_gamma,
                                      w.v_gamma, w.eps, w.k_state, w.v_state, st.state_idx,
                                      st.slot_mapping, w.num_slots, mt)
    judge(dw, [r])
    lens = np.diff(st.cu_seqlens).tolist()
    _check_snaps(w, ks, eks, lens, mt)
    _check_snaps(w, vs, evs, lens, mt)
    d = dw.steps[0]
    shortconv_state_commit(ks, vs, d["cu"], st.tokens, to_dev(accepted), dw.k_state, dw.v_state,
                           d["sidx"], width=w.W, num_heads=w.H, head_dim=w.D)
    torch.cuda.synchronize()
    for dev, pool, snaps in ((dw.k_state, w.k_state, eks), (dw.v_state, w.v_state, evs)):
        exp = oracle.commit_state(pool, snaps, accepted, st.cu_seqlens, st.state_idx, mt)
        assert np.array_equal(to_host(dev, "bf16"), exp)
