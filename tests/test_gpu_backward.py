"""GPU parity of the backward (shortconv_kv_backward) against the fp64 oracle's backward.

Judging rule: an element passes when |got - exact| <= tol*|exact| + K * 2^-24 * cond, with cond
the oracle's first-order error scale of an fp32 evaluation (oracle/shortconv_oracle.c, backward),
tol = 1e-5 for fp32 outputs and 3.9e-3 (one bf16 ulp) for bf16 outputs, K = 64 for the row
gradients (dx, initial-window gradient) and 96 for the parameter gradients: each product carries
dc's row-level error (64 units of M) and the kernel adds each lane's products over at most 64
tokens in fp32, then 4 waves, then the workgroup partials in fp64, so at most 68 roundings of
sum(|terms|) on top -- 68 * 2^-24 * sum((M + |dc|) |e|), with margin. Rows that the call must not
write keep their sentinel; the tap and gamma gradients are bit-identical across runs.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_harness import DEV, ORACLE_THREADS, TORCH_DT, rows_to_dev, to_dev, to_host
from causal_short_convolution_amd import (ShortConvError, shortconv_kv_backward,
                                          shortconv_kv_backward_workspace_size)

pytestmark = pytest.mark.gpu

K_ROWS = 64.0
K_PARAMS = 96.0
TOL = {"f32": 1e-5, "bf16": 3.9e-3}


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _stored_normal(g, shape, dtype):
    f = g.standard_normal(shape, dtype=np.float32)
    return f if dtype == "f32" else workloads.to_bf16_bits(f)


def _judge(name, got, exact, cond, tol, K):
    g = oracle.widen(got) if got.dtype in (np.uint16, np.float32) else got.astype(np.float64)
    err = np.abs(g - exact)
    bound = tol * np.abs(exact) + K * 2.0 ** -24 * cond
    assert np.isfinite(g).all(), f"{name}: non-finite values"
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, err / bound, np.where(err > 0, np.inf, 0.0))
    worst = float(ratio.max()) if ratio.size else 0.0
    at = np.unravel_index(np.argmax(ratio), ratio.shape)
    assert worst <= 1.0, f"{name}: worst error / bound = {worst:.3g} at {at}"
    return worst


class BwdCase:
    def __init__(self, dtype, H, D, W, lens, hin, seed, gs=True, dstate=True, eps=None,
                 token_pad=0, spec=None):
        if spec is None:
            spec = workloads.Spec(dtype=dtype, H=H, D=D, W=W, seed=seed, prefill_lens=list(lens),
                                  has_init=list(hin), token_pad=token_pad)
            if eps is not None:
                spec.eps = eps
        self.w = w = workloads.build(spec)
        self.st = st = w.steps[0]
        self.dtype, self.H, self.D, self.W = w.dtype, w.H, w.D, w.W
        R = w.W - 1
        N, T = st.num_seqs, st.tokens
        g = np.random.default_rng(1000 + spec.seed)
        self.dyk = _stored_normal(g, (T, w.H, w.D), w.dtype)
        self.dyv = _stored_normal(g, (T, w.H, w.D), w.dtype)
        self.gsk = _stored_normal(g, (N, R, w.H, w.D), w.dtype) if (gs and R > 0) else None
        self.gsv = _stored_normal(g, (N, R, w.H, w.D), w.dtype) if (gs and R > 0) else None
        self.want_dstate = dstate and R > 0

    def prepare(self):
        """Device inputs and sentinel-filled outputs of one backward call."""
        w, st = self.w, self.st
        R, N, T = self.W - 1, st.num_seqs, st.tokens
        dt = TORCH_DT[self.dtype]
        bits = torch.int32 if self.dtype == "f32" else torch.int16
        sentinel = 0x5A5A5A5A if self.dtype == "f32" else 0x5A5A

        def filled(shape):
            t = torch.empty(shape, dtype=dt, device=DEV)
            t.view(bits).fill_(sentinel)
            return t

        b = dict(k=rows_to_dev(st.k), v=rows_to_dev(st.v),
                 cu=to_dev(st.cu_seqlens.astype(np.int32)), kt=to_dev(w.k_taps),
                 vt=to_dev(w.v_taps), kg=to_dev(w.k_gamma), vg=to_dev(w.v_gamma),
                 ks=to_dev(w.k_state), vs=to_dev(w.v_state),
                 sidx=to_dev(st.state_idx.astype(np.int32)),
                 hinit=to_dev(st.has_init.astype(np.uint8)), dyk=to_dev(self.dyk),
                 dyv=to_dev(self.dyv), gsk=to_dev(self.gsk), gsv=to_dev(self.gsv),
                 dk=filled((T, self.H, self.D)), dv=filled((T, self.H, self.D)),
                 dks=filled((N, R, self.H, self.D)) if self.want_dstate else None,
                 dvs=filled((N, R, self.H, self.D)) if self.want_dstate else None,
                 dkt=torch.full((self.W, self.H, self.D), float("nan"), device=DEV),
                 dvt=torch.full((self.W, self.H, self.D), float("nan"), device=DEV),
                 dkg=torch.full((self.D,), float("nan"), device=DEV),
                 dvg=torch.full((self.D,), float("nan"), device=DEV))
        return b

    def launch(self, b, workspace=None):
        shortconv_kv_backward(b["k"], b["v"], b["cu"], b["kt"], b["vt"], b["kg"], b["vg"],
                              self.w.eps, b["ks"], b["vs"], b["sidx"], b["hinit"], b["dyk"],
                              b["dyv"], b["dk"], b["dv"], b["dkt"], b["dvt"], b["dkg"], b["dvg"],
                              dstate_out=(b["gsk"], b["gsv"]), dstate_in=(b["dks"], b["dvs"]),
                              workspace=workspace)

    def collect(self, b):
        out = dict(dk=to_host(b["dk"], self.dtype), dv=to_host(b["dv"], self.dtype),
                   dkt=b["dkt"].cpu().numpy(), dvt=b["dvt"].cpu().numpy(),
                   dkg=b["dkg"].cpu().numpy(), dvg=b["dvg"].cpu().numpy())
        if self.want_dstate:
            out["dks"] = to_host(b["dks"], self.dtype)
            out["dvs"] = to_host(b["dvs"], self.dtype)
        return out

    def run_gpu(self):
        b = self.prepare()
        self.launch(b)
        torch.cuda.synchronize()
        return self.collect(b)

    def oracle(self):
        w, st = self.w, self.st
        wid = oracle.widen
        return oracle.fused_backward(
            st.k, st.v, st.cu_seqlens, w.k_taps, w.v_taps, w.k_gamma, w.v_gamma, w.eps, w.k_state,
            w.v_state, st.state_idx, st.has_init, wid(self.dyk), wid(self.dyv),
            None if self.gsk is None else wid(self.gsk),
            None if self.gsv is None else wid(self.gsv), cond=True, nthreads=ORACLE_THREADS)

    def check(self, got=None):
        got = self.run_gpu() if got is None else got
        gk, gv = self.oracle()
        tol = TOL[self.dtype]
        worst = {}
        for t, gr in (("k", gk), ("v", gv)):
            worst["d" + t] = _judge(f"d{t}", got["d" + t], gr.dx, gr.cond_dx, tol, K_ROWS)
            worst["d" + t + "_taps"] = _judge(f"d{t}_taps", got["d" + t + "t"], gr.dtaps,
                                              gr.cond_dtaps, 1e-5, K_PARAMS)
            worst["d" + t + "_gamma"] = _judge(f"d{t}_gamma", got["d" + t + "g"], gr.dgamma,
                                               gr.cond_dgamma, 1e-5, K_PARAMS)
            if self.want_dstate:
                worst["d" + t + "_state"] = _judge(f"d{t}_state", got["d" + t + "s"], gr.dstate,
                                                   gr.cond_dstate, tol, K_ROWS)
        return worst


SHAPES = [
    # dtype, H, D, W, lens, has_init
    ("bf16", 8, 128, 4, [100, 1, 0, 17, 64, 3], [1, 0, 1, 1, 0, 1]),
    ("bf16", 2, 64, 8, [40, 5, 0, 130, 7], [1, 1, 0, 1, 1]),
    ("bf16", 1, 256, 2, [9, 33, 1], [0, 1, 1]),
    ("bf16", 3, 128, 1, [20, 0, 7], [1, 1, 0]),
    ("f32", 1, 64, 4, [64, 2, 19], [0, 1, 1]),
    ("f32", 4, 128, 8, [30, 6, 71], [1, 0, 1]),
    ("f32", 2, 256, 3, [2, 50, 0, 13], [1, 1, 1, 0]),
    ("bf16", 16, 128, 6, [200, 3], [1, 1]),
    ("bf16", 40, 256, 4, [30, 2, 0, 9], [1, 0, 1, 1]),  # 80 column slices of K|V
]


@pytest.mark.parametrize("dtype,H,D,W,lens,hin", SHAPES,
                         ids=[f"{s[0]}-H{s[1]}-D{s[2]}-W{s[3]}" for s in SHAPES])
def test_backward_matches_oracle(dtype, H, D, W, lens, hin):
    case = BwdCase(dtype, H, D, W, lens, hin, seed=7 + W + H)
    case.check()


@pytest.mark.parametrize("gs,dstate", [(False, True), (True, False), (False, False)])
def test_backward_optional_state_gradients(gs, dstate):
    case = BwdCase("bf16", 4, 128, 4, [15, 2, 0, 40], [1, 1, 1, 0], seed=3, gs=gs, dstate=dstate)
    case.check()


def test_backward_token_strided_inputs_and_eps_zero():
    case = BwdCase("f32", 2, 64, 4, [33, 1, 12], [1, 0, 1], seed=9, token_pad=12, eps=0.0)
    case.check()


def test_backward_is_deterministic():
    case = BwdCase("bf16", 8, 128, 4, [500, 37, 260], [1, 0, 1], seed=11)
    a = case.run_gpu()
    b = case.run_gpu()
    for key in a:
        assert np.array_equal(a[key].view(np.uint8), b[key].view(np.uint8)), key
    case.check(a)


@pytest.mark.parametrize("name", ["varlen_prefill", "long_prefill"])
def test_backward_reference_workload_shapes(name):
    """The varlen prefill and long prefill workloads, at full size."""
    spec = workloads.config_spec(name)
    case = BwdCase(None, None, None, None, None, None, seed=None, spec=spec)
    worst = case.check()
    print(f"{name} backward worst error/bound: {worst}")


# Shapes large enough that each workgroup walks several consecutive tiles (tiles x column slices
# at least 2 x 2048), so a tile's last input-gradient rows are finished by the next tile of the
# same workgroup where the sequence continues into it, and recomputed where it does not (a
# sequence boundary, the group's last tile, or rows that carry the new-state loss). Sequence
# lengths put boundaries inside walked groups; every case has new-state losses.
WALK = [
    # dtype, H, D, W, lens: bf16 over one-tensor slices (W = 8: no early loads; W = 6: 16-token
    # spans with early loads; W = 5: early loads; W = 4), bf16 and fp32 over slices mixing K and V
    # lanes, fp32 over one-tensor slices
    ("bf16", 8, 128, 8, [9000, 37, 6001, 0, 8100, 1, 913]),
    ("bf16", 4, 128, 6, [20000, 7, 15001, 3000]),
    ("bf16", 8, 128, 5, [20000, 3, 9001, 4100]),
    ("bf16", 8, 128, 4, [12000, 9, 8001, 6200, 2]),
    ("bf16", 3, 64, 7, [40000, 17, 30001, 15000]),
    ("f32", 4, 64, 7, [33000, 5, 30001, 5000]),
    ("f32", 3, 64, 6, [36000, 30001, 3]),
]


@pytest.mark.parametrize("dtype,H,D,W,lens", WALK,
                         ids=[f"{s[0]}-H{s[1]}-D{s[2]}-W{s[3]}" for s in WALK])
def test_backward_walking_several_tiles(dtype, H, D, W, lens):
    from causal_short_convolution_amd import shortconv_kv_backward_workspace_size
    hin = [1 if i % 2 == 0 else 0 for i in range(len(lens))]
    case = BwdCase(dtype, H, D, W, lens, hin, seed=50 + W)
    T, N = sum(lens), len(lens)
    # the workspace holds one partial per (group, slice): fewer groups than tiles means the
    # workgroups walk several tiles
    lpt = H * D // 4
    slices = (2 * lpt + 63) // 64
    pure = lpt % 64 == 0
    bt = (12 if pure and W <= 4 else 16 if W <= 5 or pure else 10) if dtype == "bf16" else \
        (16 if W <= 1 else 8)
    tiles = T // (4 * bt) + N
    partial = slices * (W + 1) * 256 * 4
    size = shortconv_kv_backward_workspace_size(T, N, H, D, W, TORCH_DT[dtype])
    assert size < 0.75 * tiles * partial, "the workgroups walk one tile each"
    case.check()


@pytest.mark.parametrize("seed", range(8))
def test_backward_walking_several_tiles_random(seed):
    """Seeded random shapes (dtype, heads, head_dim, width, packing, resumed sequences, new-state
    losses) sized so that each workgroup walks at least two tiles."""
    from causal_short_convolution_amd import shortconv_kv_backward_workspace_size
    rng = np.random.default_rng(300 + seed)
    dtype = ("bf16", "f32")[int(rng.integers(2))]
    H, D = [(8, 128), (4, 64), (3, 64), (2, 128), (6, 64), (16, 64), (1, 256)][rng.integers(7)]
    W = int(rng.integers(2, 9))
    lpt = H * D // 4
    slices = (2 * lpt + 63) // 64
    pure = lpt % 64 == 0
    bt = (12 if pure and W <= 4 else 16 if W <= 5 or pure else 10) if dtype == "bf16" else 8
    T = (2 * 1024 // slices + 1) * 4 * bt + int(rng.integers(0, 4 * bt * 40))
    cuts = np.sort(rng.integers(0, T, size=int(rng.integers(0, 8))))
    lens = np.diff(np.concatenate([[0], cuts, [T]])).tolist()
    if rng.random() < 0.3:
        lens.insert(int(rng.integers(len(lens))), 0)
    hin = [int(x) for x in rng.integers(0, 2, size=len(lens))]
    tiles = sum(lens) // (4 * bt) + len(lens)
    size = shortconv_kv_backward_workspace_size(sum(lens), len(lens), H, D, W, TORCH_DT[dtype])
    assert size < 0.75 * tiles * slices * (W + 1) * 1024, "the workgroups walk one tile each"
    case = BwdCase(dtype, H, D, W, lens, hin, seed=int(rng.integers(1 << 30)),
                   gs=bool(rng.random() < 0.7))
    case.check()


def test_backward_without_sequences_zeroes_parameter_gradients():
    H, D, W = 2, 64, 4
    dkt = torch.full((W, H, D), float("nan"), device=DEV)
    dvt = torch.full_like(dkt, 1.0)
    dkg, dvg = torch.full((D,), 2.0, device=DEV), torch.full((D,), 3.0, device=DEV)
    taps = torch.zeros((W, H, D), device=DEV)
    gam = torch.ones(D, device=DEV)
    empty = torch.zeros((0, H, D), dtype=torch.bfloat16, device=DEV)
    shortconv_kv_backward(empty, empty, torch.zeros(1, dtype=torch.int32, device=DEV), taps, taps,
                          gam, gam, 1e-6, None, None, None, None, empty, empty, empty, empty,
                          dkt, dvt, dkg, dvg)
    torch.cuda.synchronize()
    for t in (dkt, dvt, dkg, dvg):
        assert (t == 0).all()


def test_backward_rejects_short_workspace():
    case = BwdCase("bf16", 8, 128, 4, [50, 3], [1, 1], seed=2)
    w, st = case.w, case.st
    need = shortconv_kv_backward_workspace_size(st.tokens, st.num_seqs, 8, 128, 4, torch.bfloat16)
    assert need > 0
    ws = torch.empty(need - 16, dtype=torch.uint8, device=DEV)
    dk = torch.empty((st.tokens, 8, 128), dtype=torch.bfloat16, device=DEV)
    g = torch.empty((4, 8, 128), device=DEV)
    gm = torch.empty(128, device=DEV)
    with pytest.raises(ShortConvError, match="workspace"):
        shortconv_kv_backward(rows_to_dev(st.k), rows_to_dev(st.v),
                              to_dev(st.cu_seqlens.astype(np.int32)), to_dev(w.k_taps),
                              to_dev(w.v_taps), to_dev(w.k_gamma), to_dev(w.v_gamma), w.eps,
                              to_dev(w.k_state), to_dev(w.v_state),
                              to_dev(st.state_idx.astype(np.int32)),
                              to_dev(st.has_init.astype(np.uint8)), dk, dk, dk.clone(), dk.clone(),
                              g, g.clone(), gm, gm.clone(), workspace=ws)


def test_backward_graph_replay_matches_eager():
    """The backward's launches captured in a HIP graph: every replay, with the outputs cleared
    eagerly in between, gives the eager run's bits (the sums' workspace included in the graph)."""
    case = BwdCase("bf16", 8, 128, 4, [300, 3, 0, 40], [1, 0, 1, 1], seed=12)
    eager = case.run_gpu()
    b = case.prepare()
    st = case.st
    need = shortconv_kv_backward_workspace_size(st.tokens, st.num_seqs, case.H, case.D, case.W,
                                                torch.bfloat16)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    case.launch(b, ws)  # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        case.launch(b, ws)
    for _ in range(3):
        for key in ("dk", "dv", "dks", "dvs", "dkt", "dvt", "dkg", "dvg"):
            b[key].zero_()
        ws.fill_(0xFF)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = case.collect(b)
        for key in eager:
            assert np.array_equal(np.ascontiguousarray(got[key]).view(np.uint8),
                                  np.ascontiguousarray(eager[key]).view(np.uint8)), key


@pytest.mark.parametrize("W", [4, 8])
def test_chunked_backward_composes_to_oneshot(W):
    """Chunked training on the GPU: the second chunk resumes from the first's new state; its
    initial-window gradient is the first chunk's new-state gradient. The composed input, tap and
    gamma gradients equal the oracle's one-shot ones within the one-shot error bound (fp32 I/O,
    so the handed-over gradient is rounded at fp32 precision)."""
    case = BwdCase("f32", 4, 128, W, [90, 37], [1, 0], seed=81 + W)
    w, st = case.w, case.st
    cu = st.cu_seqlens
    cut = (50, 9)
    idx1 = np.concatenate([np.arange(cu[s], cu[s] + cut[s]) for s in range(2)])
    idx2 = np.concatenate([np.arange(cu[s] + cut[s], cu[s + 1]) for s in range(2)])
    cu1 = np.array([0, cut[0], cut[0] + cut[1]], np.int32)
    cu2 = np.array([0, 90 - cut[0], 90 - cut[0] + 37 - cut[1]], np.int32)
    _, mid, _ = oracle.prefill_one(st.k[idx1], cu1, w.k_taps, w.k_gamma, w.eps, w.k_state,
                                   st.state_idx, st.has_init)
    H, D, R = case.H, case.D, W - 1

    def run(x, cuv, pool, sidx, hinit, dy, gs):
        n = len(cuv) - 1
        T = x.shape[0]
        xd = to_dev(np.ascontiguousarray(x))
        dx = torch.empty((T, H, D), device=DEV)
        dst = torch.empty((n, R, H, D), device=DEV)
        dt, dtv = torch.empty((W, H, D), device=DEV), torch.empty((W, H, D), device=DEV)
        dg, dgv = torch.empty(D, device=DEV), torch.empty(D, device=DEV)
        dv_dummy = torch.empty_like(dx)
        dst_v = torch.empty_like(dst)
        gsd = to_dev(np.ascontiguousarray(gs, np.float32)) if gs is not None else None
        shortconv_kv_backward(xd, xd, to_dev(cuv), to_dev(w.k_taps), to_dev(w.k_taps),
                              to_dev(w.k_gamma), to_dev(w.k_gamma), w.eps, to_dev(pool),
                              to_dev(pool), to_dev(sidx.astype(np.int32)),
                              to_dev(hinit.astype(np.uint8)), to_dev(dy), to_dev(dy), dx,
                              dv_dummy, dt, dtv, dg, dgv, dstate_out=(gsd, gsd),
                              dstate_in=(dst, dst_v))
        torch.cuda.synchronize()
        return dx.cpu().numpy(), dt.cpu().numpy(), dg.cpu().numpy(), dst.cpu().numpy()

    dyk = case.dyk
    gs = oracle.widen(case.gsk)
    dx2, dt2, dg2, ds2 = run(st.k[idx2], cu2, mid, np.arange(2), np.ones(2), dyk[idx2], gs)
    dx1, dt1, dg1, ds1 = run(st.k[idx1], cu1, w.k_state, st.state_idx, st.has_init, dyk[idx1],
                             ds2)
    one = oracle.backward_one(st.k, cu, w.k_taps, w.k_gamma, w.eps, w.k_state, st.state_idx,
                              st.has_init, oracle.widen(dyk), gs, cond=True)
    dx = np.zeros_like(one.dx)
    dx[idx1], dx[idx2] = dx1, dx2
    _judge("dx", dx, one.dx, one.cond_dx, 1e-5, K_ROWS)
    _judge("dtaps", dt1 + dt2, one.dtaps, one.cond_dtaps, 1e-5, K_PARAMS)
    _judge("dgamma", dg1 + dg2, one.dgamma, one.cond_dgamma, 1e-5, K_PARAMS)
    _judge("dstate", ds1, one.dstate, one.cond_dstate, 1e-5, K_ROWS)


def test_backward_five_thousand_sequences():
    """The backward over 5 000 short packed sequences (a three-round tile search)."""
    g = np.random.default_rng(19)
    n = 5000
    lens = g.integers(0, 5, size=n).tolist()
    hin = (g.random(n) < 0.5).astype(int).tolist()
    case = BwdCase("bf16", 2, 64, 4, lens, hin, seed=20)
    case.check()
