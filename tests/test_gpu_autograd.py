"""The differentiable op (causal_short_convolution_amd.shortconv_kv) in a training pattern: two
chunks of the same sequences, the second resuming from the first's new state without detaching
it, under one loss. The gradients autograd accumulates (through both chunks and the state hand-
over) must equal the oracle's one-shot gradients of the whole sequences."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_harness import DEV, to_dev
from causal_short_convolution_amd import shortconv_kv

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _bound_ok(got, exact, cond, tol, K):
    return (np.abs(got - exact) <= tol * np.abs(exact) + K * 2.0 ** -24 * cond).all()


@pytest.mark.parametrize("W", [4, 8, 1])
def test_two_chunk_training_step_matches_oneshot_gradients(W):
    H, D = 4, 128
    lens = [70, 23]
    cut = [40, 9]
    spec = workloads.Spec(dtype="f32", H=H, D=D, W=W, seed=90 + W, prefill_lens=lens,
                          has_init=[0, 0])
    w = workloads.build(spec)
    st = w.steps[0]
    cu = st.cu_seqlens
    idx1 = np.concatenate([np.arange(cu[s], cu[s] + cut[s]) for s in range(2)])
    idx2 = np.concatenate([np.arange(cu[s] + cut[s], cu[s + 1]) for s in range(2)])
    cu1 = np.array([0, cut[0], cut[0] + cut[1]], np.int32)
    cu2 = np.array([0, lens[0] - cut[0], lens[0] - cut[0] + lens[1] - cut[1]], np.int32)
    g = np.random.default_rng(W).standard_normal((st.tokens, H, D)).astype(np.float32)

    def leaf(a):
        return to_dev(np.ascontiguousarray(a)).requires_grad_()

    k, v = leaf(st.k), leaf(st.v)
    kt, vt, kg, vg = leaf(w.k_taps), leaf(w.v_taps), leaf(w.k_gamma), leaf(w.v_gamma)
    gk, gv = to_dev(g), to_dev(g * 0.5)
    i1, i2 = torch.from_numpy(idx1).to(DEV), torch.from_numpy(idx2).to(DEV)
    y1k, y1v, s1k, s1v = shortconv_kv(k[i1], v[i1], to_dev(cu1), kt, vt, kg, vg, w.eps)
    y2k, y2v, _, _ = shortconv_kv(k[i2], v[i2], to_dev(cu2), kt, vt, kg, vg, w.eps, s1k, s1v)
    loss = ((y1k * gk[i1]).sum() + (y1v * gv[i1]).sum() + (y2k * gk[i2]).sum() +
            (y2v * gv[i2]).sum())
    loss.backward()
    torch.cuda.synchronize()
    for name, x, taps, gamma, gg, dx, dt, dg in (
            ("K", st.k, w.k_taps, w.k_gamma, g, k.grad, kt.grad, kg.grad),
            ("V", st.v, w.v_taps, w.v_gamma, g * 0.5, v.grad, vt.grad, vg.grad)):
        ref = oracle.backward_one(x, cu, taps, gamma, w.eps, None, np.arange(2),
                                  np.zeros(2, np.uint8), gg.astype(np.float64), cond=True)
        assert _bound_ok(dx.cpu().numpy(), ref.dx, ref.cond_dx, 1e-5, 64), f"{name}: dx"
        assert _bound_ok(dt.cpu().numpy(), ref.dtaps, ref.cond_dtaps, 1e-5, 96), f"{name}: taps"
        assert _bound_ok(dg.cpu().numpy(), ref.dgamma, ref.cond_dgamma, 1e-5, 96), f"{name}: gamma"


def test_bf16_outputs_match_forward_and_state():
    """bf16: the op's outputs equal the oracle's rows (tolerance) and its new states are the
    sequences' last raw rows, bit for bit."""
    spec = workloads.Spec(dtype="bf16", H=8, D=128, W=4, seed=5, prefill_lens=[60, 2, 31],
                          has_init=[1, 1, 1])
    w = workloads.build(spec)
    st = w.steps[0]
    init_k = w.k_state[st.state_idx]
    init_v = w.v_state[st.state_idx]
    yk, yv, sk, sv = shortconv_kv(to_dev(st.k), to_dev(st.v), to_dev(st.cu_seqlens),
                                  to_dev(w.k_taps), to_dev(w.v_taps), to_dev(w.k_gamma),
                                  to_dev(w.v_gamma), w.eps, to_dev(init_k), to_dev(init_v))
    torch.cuda.synchronize()
    r = oracle.fused_prefill(st.k, st.v, st.cu_seqlens, w.k_taps, w.v_taps, w.k_gamma, w.v_gamma,
                             w.eps, init_k, init_v, np.arange(3), np.ones(3, np.uint8),
                             np.arange(st.tokens), st.tokens)

    def bits(t):
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    for got, y, c in ((yk, r.y_k, r.cond_k), (yv, r.y_v, r.cond_v)):
        assert oracle.compare(bits(got), y, c, "bf16")["ok"]
    assert np.array_equal(bits(sk), r.k_state) and np.array_equal(bits(sv), r.v_state)
