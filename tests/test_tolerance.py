"""The acceptance metric itself (CPU only).

A numpy model of an fp32-accumulating kernel (products and sums rounded to fp32, one final
rounding to the stored type) must pass the metric on realistic inputs, including heavy outliers,
and results with a planted mistake must fail it. The model is test scaffolding for the metric,
not a second oracle.
"""
import numpy as np

import oracle
import workloads


def _fp32_model(x, cu, taps, gamma, eps, z, has_init, dtype):
    f = np.float32
    xw = oracle.widen(x).astype(f)
    zw = oracle.widen(z).astype(f) if z is not None else None
    W, H, D = taps.shape
    R = W - 1
    out = np.zeros(x.shape, f)
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        zz = zw[s] if (zw is not None and has_init[s]) else np.zeros((R, H, D), f)
        e = np.concatenate([zz, xw[a:b]], axis=0)
        c = taps[0] * e[0:b - a]
        for k in range(1, W):
            c = (c + taps[k] * e[k:k + b - a]).astype(f)
        ss = np.zeros(c.shape[:2], f)
        for d in range(D):
            ss = (ss + c[:, :, d] * c[:, :, d]).astype(f)
        r = np.sqrt((ss * f(1.0 / D) + f(eps)).astype(f)).astype(f)
        inv = (f(1.0) / r).astype(f)
        out[a:b] = (c * inv[:, :, None]).astype(f) * gamma
    if dtype == "bf16":
        return workloads.to_bf16_bits(out)
    return out


def _check(w, st, plant=None):
    z = w.k_state[st.state_idx] if w.k_state is not None else None
    g = _fp32_model(st.k, st.cu_seqlens, w.k_taps, w.k_gamma, w.eps, z, st.has_init, w.dtype)
    if plant:
        g = plant(g)
    y, _, c = oracle.prefill_one(st.k, st.cu_seqlens, w.k_taps, w.k_gamma, w.eps, w.k_state,
                                 st.state_idx, st.has_init, cond=True)
    return oracle.compare(g, y, c, w.dtype)


def test_fp32_model_passes_config1():
    w = workloads.config("tiny_ref")
    r = _check(w, w.steps[0])
    assert r["ok"], r
    assert r["max_rel_well_conditioned"] <= oracle.TOL["f32"]


def test_fp32_model_passes_bf16_with_outliers():
    spec = workloads.Spec(dtype="bf16", H=8, D=128, W=8, seed=4, prefill_lens=[3000, 17],
                          has_init=[0, 1], outlier_p=0.01, outlier_mul=50.0)
    w = workloads.build(spec)
    r = _check(w, w.steps[0])
    assert r["ok"], r
    assert r["max_rel_well_conditioned"] <= oracle.TOL["bf16"]


def test_planted_errors_fail():
    w = workloads.config("tiny_ref")
    st = w.steps[0]

    def bump(g):
        g = g.copy()
        g[10, 0, 3] *= np.float32(1 + 5e-5)
        return g

    def swap(g):
        g = g.copy()
        g[[5, 6]] = g[[6, 5]]
        return g

    for plant in (bump, swap):
        assert not _check(w, st, plant)["ok"], plant.__name__

    spec = workloads.Spec(dtype="bf16", H=2, D=128, W=4, seed=8, prefill_lens=[200],
                          has_init=[0])
    wb = workloads.build(spec)

    def two_ulps(g):
        g = g.copy()
        g[77, 1, 5] += np.uint16(2)
        return g

    assert _check(wb, wb.steps[0])["ok"]
    assert not _check(wb, wb.steps[0], two_ulps)["ok"]


def test_nonfinite_fails():
    w = workloads.config("tiny_ref")

    def nan(g):
        g = g.copy()
        g[0, 0, 0] = np.nan
        return g

    assert not _check(w, w.steps[0], nan)["ok"]


def test_compare_reports_elements_that_pass_only_through_the_floor():
    # fp32: an exact element, one off by 5e-6 relative (inside tol * |y|), and a cancelled one
    # (|y| = 1e-6 with a conditioning scale of 4: its error of 1e-7 is far above tol * |y| but
    # inside the floor 32 * 2^-24 * 4 = 7.6e-6); only the last needs the floor
    y = np.array([1.0, 2.0, 1e-6])
    cond = np.array([1.0, 2.0, 4.0])
    got = np.array([1.0, 2.0 * (1 + 5e-6), 1e-6 + 1e-7], dtype=np.float32)
    r = oracle.compare(got, y, cond, "f32")
    assert r["ok"] and r["n"] == 3 and r["n_over_rel"] == 1
    expect = abs(float(np.float32(1e-6 + 1e-7)) - 1e-6) / 1e-6
    assert abs(r["max_rel_over_rel"] - expect) < 1e-9
    # without the cancelled element nothing relies on the floor
    r2 = oracle.compare(got[:2], y[:2], cond[:2], "f32")
    assert r2["ok"] and r2["n_over_rel"] == 0 and r2["max_rel_over_rel"] == 0.0
