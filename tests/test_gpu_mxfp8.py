"""GPU parity of the MXFP8 cache-row variants and of the standalone MXFP8 quantizer.

Where floating point decides a code, both sides decide from the same value: the standalone
quantizer is fed exactly representable inputs, and the fused path is checked against the oracle's
quantizer applied to the fused kernel's own fp32 output (fp32 I/O, where that output is what the
plain entry point stores). For bf16 I/O, where the fp32 output is not observable, a byte may differ
from the oracle's only where the fp64 value lies within the fp32 error bound of the decision that
sets it (an E4M3 midpoint or zero for a code, a power of two for a block's scale), and then by one
step.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_harness import DEV, DeviceWorkload, rows_to_dev, to_dev, to_host
from causal_short_convolution_amd import (shortconv_kv_decode_mxfp8, shortconv_kv_prefill_mxfp8,
                                          shortconv_mxfp8_quantize)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _stored(vals, dtype):
    f = np.asarray(vals, np.float32)
    if dtype == "f32":
        return f
    b = workloads.to_bf16_bits(f)
    assert np.array_equal(workloads.bf16_bits_to_f32(b), f)
    return b


def _quantize_on_gpu(x):
    rows, H, D = x.shape
    xd = rows_to_dev(x)
    codes = torch.full((rows, H, D), 0xA5, dtype=torch.uint8, device=DEV)
    scales = torch.full((rows, H, D // 32), 0xA5, dtype=torch.uint8, device=DEV)
    shortconv_mxfp8_quantize(xd, codes, scales)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()


def _adversarial_rows(D):
    """Blocks that sit on every decision the quantizer makes: E4M3 ties (all code midpoints),
    the saturation boundary 448/464/480, subnormal ties, zeros of both signs, an all-zero
    block, and block maxima just below the next power of two (elements that saturate)."""
    vals = oracle.e4m3_decode(np.arange(0x00, 0x7F))
    mids = (vals[:-1] + vals[1:]) / 2.0
    pool = np.concatenate([mids, vals, [460.0, 464.0, 470.0, 480.0, 500.0, 0.0, -0.0]])
    rows = []
    g = np.random.default_rng(3)
    for e in (-8, -3, 0, 5, 20):
        for _ in range(4):
            r = g.choice(pool, size=D) * g.choice([-1.0, 1.0], size=D)
            r[::32] = 256.0  # every block's maximum sets the scale to 2^0 before rescaling
            rows.append(r * 2.0 ** e)
    r = np.zeros(D)
    r[32:] = 1.9921875 * 2.0 ** g.integers(-30, 30, size=D - 32)   # maxima just under 2^(k+1)
    rows.append(r)
    return np.array(rows)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_quantizer_is_exact(dtype, D):
    H = 2
    adv = _adversarial_rows(D)
    g = np.random.default_rng(D)
    rnd = g.standard_normal((40, D)) * np.exp2(g.integers(-12, 12, size=(40, 1)))
    rnd[5, :40] = 0.0
    vals = np.concatenate([adv, rnd]).astype(np.float32)
    vals = vals[: len(vals) // H * H]          # whole (row, head) groups
    if dtype == "bf16":
        vals = workloads.bf16_bits_to_f32(workloads.to_bf16_bits(vals))
    x = _stored(vals.reshape(-1, H, D), dtype)
    codes, scales = _quantize_on_gpu(x)
    ec, es = oracle.mxfp8_quantize(oracle.widen(x))
    assert np.array_equal(scales, es), "scale bytes differ"
    assert np.array_equal(codes, ec), f"codes differ at {np.argwhere(codes != ec)[:5].tolist()}"


def test_quantizer_extreme_exponents():
    """Block maxima far outside E4M3's own range: the scale exponent clamps at -127/+127."""
    D = 64
    rows = np.zeros((4, D), np.float32)
    rows[0, :32] = np.float32(2.0 ** -130) * np.arange(1, 33)   # subnormal inputs, clamp at -127
    rows[1, :32] = np.float32(2.0 ** 126) * np.linspace(-1, 1, 32)  # scale 2^118
    rows[2, 32:] = np.float32(2.0 ** -100)
    rows[3] = np.float32(3.0e38)
    x = rows.reshape(4, 1, D)
    codes, scales = _quantize_on_gpu(x)
    ec, es = oracle.mxfp8_quantize(oracle.widen(x))
    assert np.array_equal(scales, es) and np.array_equal(codes, ec)


def _fused_pair(w):
    """Run the plain and the MXFP8 prefill+decode on identical copies; return both device runs."""
    plain = DeviceWorkload(w)
    plain.run()
    mx = DeviceWorkload(w, caches=False)
    H, D = w.H, w.D
    mx.k_codes = torch.full((w.num_slots, H, D), 0xA5, dtype=torch.uint8, device=DEV)
    mx.v_codes = torch.full_like(mx.k_codes, 0xA5)
    mx.k_scales = torch.full((w.num_slots, H, D // 32), 0xA5, dtype=torch.uint8, device=DEV)
    mx.v_scales = torch.full_like(mx.k_scales, 0xA5)
    for d in mx.steps:
        if d["kind"] == "prefill":
            shortconv_kv_prefill_mxfp8(d["k"], d["v"], d["cu"], mx.k_taps, mx.v_taps, mx.k_gamma,
                                       mx.v_gamma, w.eps, mx.k_state, mx.v_state, d["sidx"],
                                       d["hinit"], d["slot"], mx.k_codes, mx.v_codes,
                                       mx.k_scales, mx.v_scales)
        else:
            shortconv_kv_decode_mxfp8(d["k"], d["v"], mx.k_taps, mx.v_taps, mx.k_gamma,
                                      mx.v_gamma, w.eps, mx.k_state, mx.v_state, d["sidx"],
                                      d["slot"], mx.k_codes, mx.v_codes, mx.k_scales,
                                      mx.v_scales)
    torch.cuda.synchronize()
    return plain, mx


def _written_slots(w):
    s = np.concatenate([st.slot_mapping for st in w.steps])
    return s[(s >= 0) & (s < w.num_slots)]


@pytest.mark.parametrize("H,D,W", [(2, 64, 4), (3, 128, 8), (1, 256, 2), (12, 256, 3)])
def test_fused_mx_equals_quantized_fp32_output(H, D, W):
    spec = workloads.Spec(dtype="f32", H=H, D=D, W=W, seed=40 + W, prefill_lens=[37, 0, 5, 100],
                          has_init=[1, 0, 1, 0], decode_ctx=[3, 50], pad_slot_every=13,
                          outlier_p=0.02)
    w = workloads.build(spec)
    plain, mx = _fused_pair(w)
    rows = _written_slots(w)
    for cache, codes, scales in ((plain.k_cache, mx.k_codes, mx.k_scales),
                                 (plain.v_cache, mx.v_codes, mx.v_scales)):
        y32 = to_host(cache, "f32")[rows].astype(np.float64)
        ec, es = oracle.mxfp8_quantize(y32)
        assert np.array_equal(scales.cpu().numpy()[rows], es)
        assert np.array_equal(codes.cpu().numpy()[rows], ec)
        untouched = np.setdiff1d(np.arange(w.num_slots), rows)
        assert (codes.cpu().numpy()[untouched] == 0xA5).all()
        assert (scales.cpu().numpy()[untouched] == 0xA5).all()
    for a, b in ((plain.k_state, mx.k_state), (plain.v_state, mx.v_state)):
        assert np.array_equal(to_host(a, "f32"), to_host(b, "f32")), "conv state must not change"


def _fp32_bound(y, cond):
    """Error bound of an fp32 evaluation of the step (the fp32 parity rule of the oracle)."""
    return oracle.TOL["f32"] * np.abs(y) + oracle.FLOOR_ULPS * 2.0 ** -24 * cond


def test_fused_mx_bf16_differs_only_at_decisions_within_fp32_error():
    """bf16 I/O: the MXFP8 kernel quantizes its fp32 rows, which lie within the fp32 error bound B
    of the oracle's fp64 rows y. So its bytes equal the oracle quantizer's on y, except where y is
    within B of a decision: a block whose maximum is within B of a power of two (scale one step
    apart), or an element whose scaled value is within B of an E4M3 midpoint or of zero (codes one
    step apart, or the two zeros). Codes are judged under the kernel's own scale."""
    spec = workloads.Spec(dtype="bf16", H=8, D=128, W=4, seed=51, prefill_lens=[300, 17, 1000],
                          has_init=[0, 1, 1], decode_ctx=[9, 70, 2], outlier_p=0.01)
    w = workloads.build(spec)
    plain, mx = _fused_pair(w)
    from gpu_harness import oracle_steps
    res = oracle_steps(w)
    vals = oracle.e4m3_decode(np.arange(0x00, 0x7F))
    mids = (vals[:-1] + vals[1:]) / 2.0
    n_scale = n_code = n_el = 0
    for name, codes_d, scales_d in (("K", mx.k_codes, mx.k_scales), ("V", mx.v_codes, mx.v_scales)):
        codes = codes_d.cpu().numpy()
        scales = scales_d.cpu().numpy()
        for r in res:
            ok = r.slots >= 0
            if not ok.any():
                continue
            y = (r.y_k if name == "K" else r.y_v)[ok]
            b = _fp32_bound(y, (r.cond_k if name == "K" else r.cond_v)[ok])
            gc, gs = codes[r.slots[ok]], scales[r.slots[ok]]
            ec, es = oracle.mxfp8_quantize(y)
            # scales: equal, or one apart with a power of two within B of the block maximum
            amax = np.abs(y).reshape(*gs.shape, 32).max(-1)
            bmax = b.reshape(*gs.shape, 32).max(-1)
            k = np.round(np.log2(np.maximum(amax, 1e-300)))
            near = np.abs(amax - np.exp2(k)) <= bmax
            ds = np.abs(gs.astype(int) - es.astype(int))
            assert ((ds == 0) | ((ds == 1) & near)).all(), f"{name}: scale off a 2^k decision"
            n_scale += int((ds != 0).sum())
            # codes under the kernel's scale
            e = np.repeat(gs.astype(np.int64) - 127, 32, axis=-1)
            scaled = y * np.exp2(-e.astype(np.float64))
            bs = b * np.exp2(-e.astype(np.float64))
            exp_c = oracle.e4m3_encode(scaled)
            diff = gc != exp_c
            a = np.abs(scaled)
            j = np.clip(np.searchsorted(mids, a), 1, len(mids) - 1)
            dist = np.minimum(np.abs(a - mids[j - 1]), np.abs(a - mids[j]))
            at_mid = dist <= bs
            at_zero = a <= bs
            assert (~diff | at_mid | at_zero).all(), \
                f"{name}: code differs off a decision at {np.argwhere(diff & ~at_mid & ~at_zero)[:3]}"
            gv, ev = oracle.e4m3_decode(gc), oracle.e4m3_decode(exp_c)
            step = np.maximum(np.abs(ev) * 2.0 ** -3, 2.0 ** -9)
            assert (np.abs(gv - ev)[diff] <= step[diff] * (1 + 1e-12)).all(), f"{name}: > 1 step"
            n_code += int(diff.sum())
            n_el += int(y.size)
    print(f"bytes off the oracle's at fp32-error decisions: {n_scale} scales, {n_code} codes "
          f"of {n_el}")
    for a, b in ((plain.k_state, mx.k_state), (plain.v_state, mx.v_state)):
        assert np.array_equal(to_host(a, "bf16"), to_host(b, "bf16")), "conv state must not change"


def test_mx_rejects_missing_scales():
    # the binding refuses the call before the library sees it (the library's own null-scale
    # check is exercised from the host in test_abi_cpu.py)
    w = workloads.build(workloads.Spec(dtype="bf16", H=8, D=128, W=4, seed=2, prefill_lens=[4],
                                       has_init=[0]))
    dw = DeviceWorkload(w, caches=False)
    d = dw.steps[0]
    codes = torch.zeros((w.num_slots, 8, 128), dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError, match="k_scales is required"):
        shortconv_kv_prefill_mxfp8(d["k"], d["v"], d["cu"], dw.k_taps, dw.v_taps, dw.k_gamma,
                                   dw.v_gamma, w.eps, dw.k_state, dw.v_state, d["sidx"],
                                   d["hinit"], d["slot"], codes, codes.clone(), None, None)


def test_fused_mx_bf16_equals_quantized_plain_rows_but_double_rounding():
    """bf16 I/O: the plain and the MXFP8 prefill compute the same fp32 rows (same lane layout,
    same arithmetic); the plain one rounds them to bf16. Quantizing those bf16 rows with the
    oracle gives the MXFP8 kernel's codes and scales exactly, except where rounding to bf16 first
    can flip a decision: a scaled element exactly on an E4M3 midpoint (one step apart), or a
    block whose bf16 maximum is exactly a power of two (its scale one below)."""
    spec = workloads.Spec(dtype="bf16", H=8, D=128, W=4, seed=61, prefill_lens=[700, 33, 1500],
                          has_init=[1, 0, 1], decode_ctx=[12, 90], outlier_p=0.01)
    w = workloads.build(spec)
    plain, mx = _fused_pair(w)
    rows = _written_slots(w)
    mids = oracle.e4m3_decode(np.arange(0, 0x7E))
    mids = (mids + oracle.e4m3_decode(np.arange(1, 0x7F))) / 2.0
    flips = 0
    for cache, codes_d, scales_d in ((plain.k_cache, mx.k_codes, mx.k_scales),
                                     (plain.v_cache, mx.v_codes, mx.v_scales)):
        yb = oracle.widen(to_host(cache, "bf16")[rows])
        ec, es = oracle.mxfp8_quantize(yb)
        gc, gs = codes_d.cpu().numpy()[rows], scales_d.cpu().numpy()[rows]
        blocks = np.abs(yb).reshape(*yb.shape[:-1], -1, 32).max(-1)
        pow2 = (blocks > 0) & (np.frexp(blocks)[0] == 0.5)
        bad_scale = gs != es
        assert (pow2 | ~bad_scale).all(), "a scale differs off a power-of-two block maximum"
        assert ((es.astype(int) - gs.astype(int))[bad_scale] == 1).all()
        same = np.repeat(gs == es, 32, axis=-1)
        e = np.repeat(es.astype(np.int64) - 127, 32, axis=-1)
        scaled = np.abs(yb) * np.exp2(-e.astype(np.float64))
        tie = np.isin(scaled, mids)
        diff = (gc != ec) & same
        assert (tie | ~diff).all(), "a code differs off an E4M3 midpoint"
        step = np.abs(oracle.e4m3_decode(gc) - oracle.e4m3_decode(ec))
        gap = np.maximum(np.abs(oracle.e4m3_decode(ec)) * 2.0 ** -3, 2.0 ** -9)
        assert (step[diff] <= gap[diff] * (1 + 1e-12)).all(), "a flipped code is more than a step"
        flips += int(diff.sum()) + int(bad_scale.sum())
    print(f"double-rounding flips: {flips}")


def test_mx_graph_replay_matches_eager():
    """MXFP8 prefill + decode captured in a HIP graph: every replay (state restored eagerly in
    between) writes the eager run's code and scale bytes."""
    spec = workloads.Spec(dtype="bf16", H=8, D=128, W=4, seed=71, prefill_lens=[90, 5, 33],
                          has_init=[1, 0, 1], decode_ctx=[12, 40])
    w = workloads.build(spec)
    plain, mx = _fused_pair(w)  # mx holds the eager MXFP8 results
    eager = [t.cpu().numpy() for t in (mx.k_codes, mx.v_codes, mx.k_scales, mx.v_scales)]
    mx2 = DeviceWorkload(w, caches=False)
    for name in ("k_codes", "v_codes", "k_scales", "v_scales"):
        setattr(mx2, name, torch.zeros_like(getattr(mx, name)))
    k0, v0 = mx2.k_state.clone(), mx2.v_state.clone()

    def step():
        for d in mx2.steps:
            if d["kind"] == "prefill":
                shortconv_kv_prefill_mxfp8(d["k"], d["v"], d["cu"], mx2.k_taps, mx2.v_taps,
                                           mx2.k_gamma, mx2.v_gamma, w.eps, mx2.k_state,
                                           mx2.v_state, d["sidx"], d["hinit"], d["slot"],
                                           mx2.k_codes, mx2.v_codes, mx2.k_scales, mx2.v_scales)
            else:
                shortconv_kv_decode_mxfp8(d["k"], d["v"], mx2.k_taps, mx2.v_taps, mx2.k_gamma,
                                          mx2.v_gamma, w.eps, mx2.k_state, mx2.v_state,
                                          d["sidx"], d["slot"], mx2.k_codes, mx2.v_codes,
                                          mx2.k_scales, mx2.v_scales)

    step()  # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    rows = _written_slots(w)
    for _ in range(3):
        mx2.k_state.copy_(k0)
        mx2.v_state.copy_(v0)
        for name in ("k_codes", "v_codes", "k_scales", "v_scales"):
            getattr(mx2, name).zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [t.cpu().numpy() for t in (mx2.k_codes, mx2.v_codes, mx2.k_scales, mx2.v_scales)]
        for a, b in zip(got, eager):
            assert np.array_equal(a[rows], b[rows])


def test_varlen_workload_mx_rows_at_full_size():
    """The bench's MXFP8 measurement (the varlen prefill workload with MXFP8 rows) at full size:
    codes and scales equal the oracle's quantization of the plain kernel's bf16 rows except at
    the identified double-rounding ties; the conv state equals the plain run's."""
    w = workloads.config("varlen_prefill")
    plain, mx = _fused_pair(w)
    rows = _written_slots(w)
    mids = oracle.e4m3_decode(np.arange(0, 0x7E))
    mids = (mids + oracle.e4m3_decode(np.arange(1, 0x7F))) / 2.0
    for cache, codes_d, scales_d in ((plain.k_cache, mx.k_codes, mx.k_scales),
                                     (plain.v_cache, mx.v_codes, mx.v_scales)):
        for a in range(0, rows.size, 4096):
            sel = rows[a:a + 4096]
            idx = torch.from_numpy(sel).to(DEV)
            yb = oracle.widen(to_host(cache.index_select(0, idx), "bf16"))
            ec, es = oracle.mxfp8_quantize(yb)
            gc = codes_d.index_select(0, idx).cpu().numpy()
            gs = scales_d.index_select(0, idx).cpu().numpy()
            blocks = np.abs(yb).reshape(*yb.shape[:-1], -1, 32).max(-1)
            pow2 = (blocks > 0) & (np.frexp(blocks)[0] == 0.5)
            assert (pow2 | (gs == es)).all(), "a scale differs off a power-of-two block maximum"
            same = np.repeat(gs == es, 32, axis=-1)
            e = np.repeat(es.astype(np.int64) - 127, 32, axis=-1)
            tie = np.isin(np.abs(yb) * np.exp2(-e.astype(np.float64)), mids)
            assert (tie | ~((gc != ec) & same)).all(), "a code differs off an E4M3 midpoint"
    for a, b in ((plain.k_state, mx.k_state), (plain.v_state, mx.v_state)):
        assert np.array_equal(to_host(a, "bf16"), to_host(b, "bf16"))


def _check_mx_against_plain_bf16(w, plain, mx, every=4096):
    """MXFP8 bytes of a bf16 workload against the oracle's quantization of the plain kernel's
    bf16 rows: equal except at double-rounding ties (an E4M3 midpoint, a power-of-two block
    maximum). Checked on the blocks of 4 096 written rows that start every `every` rows (every
    row by default); the conv state in full."""
    rows = _written_slots(w)
    mids = oracle.e4m3_decode(np.arange(0, 0x7E))
    mids = (mids + oracle.e4m3_decode(np.arange(1, 0x7F))) / 2.0
    for cache, codes_d, scales_d in ((plain.k_cache, mx.k_codes, mx.k_scales),
                                     (plain.v_cache, mx.v_codes, mx.v_scales)):
        for a in range(0, rows.size, every):
            sel = rows[a:a + 4096]
            idx = torch.from_numpy(sel).to(DEV)
            yb = oracle.widen(to_host(cache.index_select(0, idx), "bf16"))
            ec, es = oracle.mxfp8_quantize(yb)
            gc = codes_d.index_select(0, idx).cpu().numpy()
            gs = scales_d.index_select(0, idx).cpu().numpy()
            blocks = np.abs(yb).reshape(*yb.shape[:-1], -1, 32).max(-1)
            pow2 = (blocks > 0) & (np.frexp(blocks)[0] == 0.5)
            assert (pow2 | (gs == es)).all(), "a scale differs off a power-of-two block maximum"
            same = np.repeat(gs == es, 32, axis=-1)
            e = np.repeat(es.astype(np.int64) - 127, 32, axis=-1)
            tie = np.isin(np.abs(yb) * np.exp2(-e.astype(np.float64)), mids)
            assert (tie | ~((gc != ec) & same)).all(), "a code differs off an E4M3 midpoint"
    for a, b in ((plain.k_state, mx.k_state), (plain.v_state, mx.v_state)):
        assert np.array_equal(to_host(a, "bf16"), to_host(b, "bf16"))


def test_mixed_workload_mx_rows_at_full_size():
    """The mixed workload (64 resumed chunks of 2 048 tokens, 16 KV heads x 128, then 512
    decodes) with MXFP8 rows at full size. Its prefill grid is large enough (131 072 tokens / 16
    x 8 column slices = 65 536 waves) for the library to run MXFP8 rows in 16-token runs per
    wave, so this checks that kernel against the plain kernel's rows and the oracle quantizer (on
    a quarter of the rows: a block of 4 096 in every 16 384, spread over the whole step)."""
    w = workloads.config("mixed")
    plain, mx = _fused_pair(w)
    _check_mx_against_plain_bf16(w, plain, mx, every=16384)


@pytest.mark.parametrize("W", [1, 3])
def test_fused_mx_runs_equal_quantized_fp32_output(W):
    """fp32 I/O, 16 KV heads x 256: 32 column slices, so 17 000 packed tokens (ragged sequences,
    some resuming from a stored state, a few dropped slots) make a grid of 33 984 waves, enough
    for the 16-token runs per wave. Codes and scales are the oracle quantizer's on the plain
    kernel's fp32 rows, bit for bit; the conv state is the plain run's."""
    spec = workloads.Spec(dtype="f32", H=16, D=256, W=W, seed=90 + W,
                          prefill_lens=[5000, 1, 17, 0, 3333, 6000, 2649],
                          has_init=[1, 0, 1, 1, 0, 1, 0], pad_slot_every=977, outlier_p=0.01)
    w = workloads.build(spec)
    assert sum(spec.prefill_lens) // 16 * 32 >= 32768
    plain, mx = _fused_pair(w)
    rows = _written_slots(w)
    for cache, codes, scales in ((plain.k_cache, mx.k_codes, mx.k_scales),
                                 (plain.v_cache, mx.v_codes, mx.v_scales)):
        for a in range(0, rows.size, 2048):
            sel = rows[a:a + 2048]
            idx = torch.from_numpy(sel).to(DEV)
            y32 = to_host(cache.index_select(0, idx), "f32").astype(np.float64)
            ec, es = oracle.mxfp8_quantize(y32)
            assert np.array_equal(scales.index_select(0, idx).cpu().numpy(), es)
            assert np.array_equal(codes.index_select(0, idx).cpu().numpy(), ec)
        untouched = np.setdiff1d(np.arange(w.num_slots), rows)
        assert (codes.cpu().numpy()[untouched] == 0xA5).all()
        assert (scales.cpu().numpy()[untouched] == 0xA5).all()
    for a, b in ((plain.k_state, mx.k_state), (plain.v_state, mx.v_state)):
        if a is not None:  # (W = 1 keeps no state)
            assert np.array_equal(to_host(a, "f32"), to_host(b, "f32")), "state must not change"


def test_fused_mx_runs_bf16_narrow_heads():
    """bf16 rows, 32 KV heads x 64 (8 lanes per head), W = 2: 8 column slices, so 70 000 packed
    tokens make a grid of 35 000 waves and the library runs MXFP8 rows in 16-token runs. Bytes
    against the oracle quantizer of the plain kernel's rows (double-rounding ties aside), on a
    quarter of the rows; the conv state in full."""
    spec = workloads.Spec(dtype="bf16", H=32, D=64, W=2, seed=77,
                          prefill_lens=[30000, 7, 0, 19993, 20000], has_init=[1, 0, 1, 0, 1],
                          pad_slot_every=1009, outlier_p=0.01)
    w = workloads.build(spec)
    assert sum(spec.prefill_lens) // 16 * 8 >= 32768
    plain, mx = _fused_pair(w)
    _check_mx_against_plain_bf16(w, plain, mx, every=16384)
