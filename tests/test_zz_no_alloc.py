"""The backward entry point that allocates nothing (shortconv_kv_backward_noalloc), through the C
ABI, against shortconv_kv_backward with a caller-provided workspace.

Both run the same kernels; the no-alloc one keeps its parameter-gradient partials in the library's
static per-GPU scratch. The two calls in a row below (the second smaller than the first) check
that nothing the first call leaves in the scratch reaches the second: every output must equal the
workspace entry point's bit for bit. A problem larger than the scratch is rejected on the host,
before any launch, with its outputs left as they were.
"""
import numpy as np
import pytest
import torch

import workloads
from gpu_harness import DEV, TORCH_DT, rows_to_dev, to_dev, to_host
from causal_short_convolution_amd import (NOALLOC_SCRATCH_BYTES, ShortConvError,
                                          shortconv_kv_backward, shortconv_kv_backward_noalloc,
                                          shortconv_kv_backward_workspace_size)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _normal(g, shape, dtype):
    f = g.standard_normal(shape, dtype=np.float32)
    return f if dtype == "f32" else workloads.to_bf16_bits(f)


class Problem:
    """Device inputs of one backward call (fresh and resumed sequences, a new-state loss)."""

    def __init__(self, dtype, H, D, W, lens, hinit, seed):
        w = workloads.build(workloads.Spec(dtype=dtype, H=H, D=D, W=W, seed=seed,
                                           prefill_lens=list(lens), has_init=list(hinit)))
        st = w.steps[0]
        self.w, self.dtype, self.H, self.D, self.W = w, dtype, H, D, W
        self.N, self.T, R = st.num_seqs, st.tokens, W - 1
        g = np.random.default_rng(seed + 77)
        self.args = dict(
            k=rows_to_dev(st.k), v=rows_to_dev(st.v), cu=to_dev(st.cu_seqlens.astype(np.int32)),
            kt=to_dev(w.k_taps), vt=to_dev(w.v_taps), kg=to_dev(w.k_gamma), vg=to_dev(w.v_gamma),
            ks=to_dev(w.k_state), vs=to_dev(w.v_state),
            sidx=to_dev(st.state_idx.astype(np.int32)), hinit=to_dev(st.has_init.astype(np.uint8)),
            dyk=to_dev(_normal(g, (self.T, H, D), dtype)),
            dyv=to_dev(_normal(g, (self.T, H, D), dtype)),
            gsk=to_dev(_normal(g, (self.N, R, H, D), dtype)) if R > 0 else None,
            gsv=to_dev(_normal(g, (self.N, R, H, D), dtype)) if R > 0 else None)

    def outputs(self):
        """Output tensors filled with NaN, so that anything left unwritten shows."""
        dt, H, D, W, R = TORCH_DT[self.dtype], self.H, self.D, self.W, self.W - 1
        out = dict(dk=torch.full((self.T, H, D), float("nan"), dtype=dt, device=DEV),
                   dv=torch.full((self.T, H, D), float("nan"), dtype=dt, device=DEV),
                   dkt=torch.full((W, H, D), float("nan"), device=DEV),
                   dvt=torch.full((W, H, D), float("nan"), device=DEV),
                   dkg=torch.full((D,), float("nan"), device=DEV),
                   dvg=torch.full((D,), float("nan"), device=DEV))
        if R > 0:
            out["dks"] = torch.full((self.N, R, H, D), float("nan"), dtype=dt, device=DEV)
            out["dvs"] = torch.full((self.N, R, H, D), float("nan"), dtype=dt, device=DEV)
        return out

    def call(self, fn, out, **kw):
        a = self.args
        fn(a["k"], a["v"], a["cu"], a["kt"], a["vt"], a["kg"], a["vg"], self.w.eps, a["ks"],
           a["vs"], a["sidx"], a["hinit"], a["dyk"], a["dyv"], out["dk"], out["dv"], out["dkt"],
           out["dvt"], out["dkg"], out["dvg"], dstate_out=(a["gsk"], a["gsv"]),
           dstate_in=(out.get("dks"), out.get("dvs")), **kw)

    def host(self, out):
        return {k: (to_host(t, self.dtype) if t.dtype != torch.float32 else t.cpu().numpy())
                for k, t in out.items()}


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint8)


def _as_float(a):
    """Stored values as float32 (uint16 arrays hold bf16 bit patterns)."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32)
    return a


@pytest.mark.parametrize("dtype,H,D,W", [("bf16", 8, 128, 4), ("f32", 2, 64, 8),
                                         ("bf16", 4, 256, 1)])
def test_noalloc_equals_workspace_backward_on_two_calls(dtype, H, D, W):
    big = Problem(dtype, H, D, W, lens=(700, 33, 1200, 5, 0, 260), hinit=(1, 0, 1, 1, 1, 0),
                  seed=31)
    small = Problem(dtype, H, D, W, lens=(90, 17), hinit=(0, 1), seed=32)
    for p in (big, small):
        assert shortconv_kv_backward_workspace_size(p.T, p.N, H, D, W, TORCH_DT[dtype]) <= \
            NOALLOC_SCRATCH_BYTES
    # the reference: the workspace entry point, a fresh workspace per call
    refs = []
    for p in (big, small):
        out = p.outputs()
        p.call(shortconv_kv_backward, out)
        torch.cuda.synchronize()
        refs.append(p.host(out))
    # the no-alloc entry point twice in a row, big then small: the second call finds the first
    # call's partials in the scratch
    for p, ref in zip((big, small), refs):
        out = p.outputs()
        p.call(shortconv_kv_backward_noalloc, out)
        torch.cuda.synchronize()
        got = p.host(out)
        assert set(got) == set(ref)
        for name in ref:
            assert np.isfinite(_as_float(got[name])).all(), f"{name} left unwritten"
            assert np.array_equal(_bits(got[name]), _bits(ref[name])), \
                f"{name} differs from shortconv_kv_backward (T={p.T})"


def test_noalloc_rejects_a_problem_beyond_the_scratch():
    H, D, W, T = 8, 128, 8, 131072
    need = shortconv_kv_backward_workspace_size(T, 1, H, D, W, torch.bfloat16)
    if need <= NOALLOC_SCRATCH_BYTES:
        pytest.skip("this problem fits the scratch")
    dt = torch.bfloat16
    rows = [torch.empty((T, H, D), dtype=dt, device=DEV) for _ in range(4)]
    dk = torch.full((T, H, D), 7.0, dtype=dt, device=DEV)
    taps = torch.zeros((W, H, D), device=DEV)
    gam = torch.ones(D, device=DEV)
    dkt = torch.full((W, H, D), 3.0, device=DEV)
    dkg = torch.full((D,), 3.0, device=DEV)
    with pytest.raises(ShortConvError, match="SC_ERR_UNSUPPORTED.*static scratch"):
        shortconv_kv_backward_noalloc(
            rows[0], rows[1], torch.tensor([0, T], dtype=torch.int32, device=DEV), taps, taps,
            gam, gam, 1e-6, None, None, None, None, rows[2], rows[3], dk, dk.clone(), dkt,
            dkt.clone(), dkg, dkg.clone())
    torch.cuda.synchronize()
    assert bool((dk == 7.0).all()) and bool((dkt == 3.0).all()) and bool((dkg == 3.0).all())
