"""The backward's acceptance rule itself (CPU only).

The GPU backward is judged by |got - exact| <= tol*|exact| + K * 2^-24 * cond, with the oracle's
first-order error scale cond (K = 64 for row gradients, 96 for the tap and gamma gradients;
tests/test_gpu_backward.py). Here a numpy model of an fp32 evaluation -- every product and sum
rounded to fp32, no fused multiply-adds, and the tap and gamma gradients summed sequentially over
all tokens, all of which is worse than the kernel -- must pass that rule, and results with a
planted mistake (five times the fp32 tolerance, two bf16 ulps, a wrong row) must fail it. The model is test
scaffolding for the rule, not a second oracle.
"""
import numpy as np

import oracle
import workloads

K_ROWS, K_PARAMS = 64.0, 96.0
TOL = {"f32": 1e-5, "bf16": 3.9e-3}
f = np.float32


def _fp32_model(w, st, g, gs):
    """fp32 evaluation of the backward of tensor K; returns (dx, dtaps, dgamma, dstate)."""
    taps, gamma = w.k_taps.astype(f), w.k_gamma.astype(f)
    W, H, D = taps.shape
    R = W - 1
    x = oracle.widen(st.k).astype(f)
    pool = oracle.widen(w.k_state).astype(f) if w.k_state is not None else None
    dx = np.zeros(x.shape, f)
    dtaps = np.zeros(taps.shape, f)
    dgamma = np.zeros(D, f)
    dstate = np.zeros((st.num_seqs, R, H, D), f)
    cu = st.cu_seqlens
    for s in range(st.num_seqs):
        a, b = int(cu[s]), int(cu[s + 1])
        L = b - a
        idx = st.state_idx[s]
        from_state = R > 0 and st.has_init[s] and 0 <= idx < (0 if pool is None else len(pool))
        z = pool[idx] if from_state else np.zeros((R, H, D), f)
        e = np.concatenate([z, x[a:b]], axis=0)
        dc = np.zeros((L, H, D), f)
        for p in range(L):
            c = (taps[0] * e[p]).astype(f)
            for k in range(1, W):
                c = (c + (taps[k] * e[p + k]).astype(f)).astype(f)
            ss = np.zeros(H, f)
            for d in range(D):
                ss = (ss + (c[:, d] * c[:, d]).astype(f)).astype(f)
            inv = (f(1.0) / np.sqrt((ss * f(1.0 / D) + f(w.eps)).astype(f))).astype(f)
            chat = (c * inv[:, None]).astype(f)
            gp = g[a + p].astype(f)
            dchat = (gp * gamma).astype(f)
            pj = np.zeros(H, f)
            for d in range(D):
                pj = (pj + (dchat[:, d] * chat[:, d]).astype(f)).astype(f)
            pj = (pj * f(1.0 / D)).astype(f)
            dc[p] = ((dchat - (chat * pj[:, None]).astype(f)).astype(f) * inv[:, None]).astype(f)
            dgamma = (dgamma + (gp * chat).astype(f).sum(axis=0, dtype=f)).astype(f)
            for k in range(W):
                dtaps[k] = (dtaps[k] + (dc[p] * e[p + k]).astype(f)).astype(f)
        for i in range(R + L):
            acc = np.zeros((H, D), f)
            for k in range(W):
                p = i - k
                if 0 <= p < L:
                    acc = (acc + (taps[k] * dc[p]).astype(f)).astype(f)
            if gs is not None and i >= L:
                acc = (acc + gs[s, i - L].astype(f)).astype(f)
            if i >= R:
                dx[a + i - R] = acc
            elif from_state:
                dstate[s, i] = acc
    return dx, dtaps, dgamma, dstate


def _store(a, dtype):
    return workloads.to_bf16_bits(a) if dtype == "bf16" else a


def _worst(got, exact, cond, tol, K):
    gw = oracle.widen(got) if got.dtype in (np.uint16, np.float32) else got
    err = np.abs(gw - exact)
    bound = tol * np.abs(exact) + K * 2.0 ** -24 * cond
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, err / bound, np.where(err > 0, np.inf, 0.0))
    return float(ratio.max()) if ratio.size else 0.0


def _case(dtype, W, seed=5, outliers=0.0):
    spec = workloads.Spec(dtype=dtype, H=2, D=64, W=W, seed=seed, prefill_lens=[40, 2, 0, 23],
                          has_init=[1, 1, 0, 1], outlier_p=outliers)
    w = workloads.build(spec)
    st = w.steps[0]
    rng = np.random.default_rng(seed)
    g = oracle.widen(_store(rng.standard_normal((st.tokens, 2, 64)).astype(f), dtype))
    gs = (oracle.widen(_store(rng.standard_normal((st.num_seqs, W - 1, 2, 64)).astype(f), dtype))
          if W > 1 else None)
    ref = oracle.backward_one(st.k, st.cu_seqlens, w.k_taps, w.k_gamma, w.eps, w.k_state,
                              st.state_idx, st.has_init, g, gs, cond=True)
    return w, st, g, gs, ref


def _judge_all(dtype, model, ref, W):
    dx, dtaps, dgamma, dstate = model
    tol = TOL[dtype]
    worst = [_worst(_store(dx, dtype), ref.dx, ref.cond_dx, tol, K_ROWS),
             _worst(dtaps, ref.dtaps, ref.cond_dtaps, 1e-5, K_PARAMS),
             _worst(dgamma, ref.dgamma, ref.cond_dgamma, 1e-5, K_PARAMS)]
    if W > 1:
        worst.append(_worst(_store(dstate, dtype), ref.dstate, ref.cond_dstate, tol, K_ROWS))
    return worst


def test_fp32_evaluation_passes():
    for dtype in ("f32", "bf16"):
        for W in (1, 4, 8):
            for outliers in (0.0, 0.02):
                w, st, g, gs, ref = _case(dtype, W, outliers=outliers)
                worst = _judge_all(dtype, _fp32_model(w, st, g, gs), ref, W)
                assert max(worst) <= 1.0, (dtype, W, outliers, worst)


def test_planted_mistakes_fail():
    for dtype in ("f32", "bf16"):
        w, st, g, gs, ref = _case(dtype, 4)
        model = _fp32_model(w, st, g, gs)
        # 5x the fp32 tolerance, or two bf16 units in the last place
        rel = 2.0 * 2.0 ** -8 if dtype == "bf16" else 5e-5
        plants = {
            "dx scaled by 5 fp32 tolerances / 2 bf16 ulps": (model[0] * f(1 + rel), *model[1:]),
            "dtaps scaled by 2e-4": (model[0], model[1] * f(1 + 2e-4), *model[2:]),
            "dgamma scaled by 2e-4": (*model[:2], model[2] * f(1 + 2e-4), model[3]),
            "dstate rows swapped": (*model[:3], model[3][:, ::-1].copy()),
            "dx one token off": (np.roll(model[0], 1, axis=0), *model[1:]),
        }
        for name, planted in plants.items():
            worst = _judge_all(dtype, planted, ref, 4)
            assert max(worst) > 1.0, f"{dtype}: planted mistake passed: {name} ({worst})"
