"""Seeded random sweep of shapes and structure (deterministic: case i draws from seed i): dtype,
heads, head_dim, width, sequence lengths (including empty ones and ones shorter than the window),
initial states, padding slots and token strides; each case runs prefill + decode and the backward
through the C ABI and is judged against the oracle like the fixed cases."""
import numpy as np
import pytest
import torch

import workloads
from gpu_harness import DeviceWorkload, judge
from test_gpu_backward import BwdCase

pytestmark = pytest.mark.gpu

N_CASES = 24


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _case(i):
    g = np.random.default_rng(1000 + i)
    dtype = ("f32", "bf16")[int(g.integers(2))]
    D = int(g.choice([64, 128, 256]))
    H = int(g.choice([1, 2, 3, 5, 8, 12]))
    W = int(g.integers(1, 9))
    n = int(g.integers(1, 7))
    lens = [int(x) for x in g.choice([0, 1, 2, 3, 5, 8, 17, 33, 64, 65, 100, 257], size=n)]
    hin = [int(x) for x in g.integers(0, 2, size=n)]
    dec = [int(x) for x in g.integers(1, 300, size=int(g.integers(0, 5)))]
    spec = workloads.Spec(dtype=dtype, H=H, D=D, W=W, seed=2000 + i, prefill_lens=lens,
                          has_init=hin, decode_ctx=dec, block_size=int(g.choice([1, 16, 64])),
                          pad_slot_every=int(g.choice([0, 0, 7])),
                          token_pad=int(g.choice([0, 8 if dtype == "bf16" else 4])))
    return spec


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_forward(i):
    spec = _case(i)
    w = workloads.build(spec)
    dw = DeviceWorkload(w)
    dw.run()
    judge(dw)


@pytest.mark.parametrize("i", range(0, N_CASES, 2))
def test_random_backward(i):
    s = _case(i)
    if sum(s.prefill_lens) == 0:
        pytest.skip("no tokens")
    case = BwdCase(s.dtype, s.H, s.D, s.W, list(s.prefill_lens), list(s.has_init), seed=3000 + i,
                   token_pad=s.token_pad)
    case.check()
