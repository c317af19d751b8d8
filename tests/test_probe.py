"""The measurement probe that the bench times beside the fused step (csrc/copy_probe.hip): its
ceilings are only meaningful if every form moves exactly the bytes it claims to move.

CPU: the library loads, exports its entry points, and rejects bad arguments before launching.
GPU: every plain copy form reproduces its source byte for byte; every scatter form puts row t of
K and V at cache row slot[t] (strided sources, a ragged token count, dropped slots) and touches
nothing else."""
import ctypes
import os

import numpy as np
import pytest

from causal_short_convolution_amd import build as hip_build

P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int


def _lib():
    if not os.path.exists(hip_build.PROBE_LIB):
        pytest.skip("probe library not built")
    lib = ctypes.CDLL(hip_build.PROBE_LIB)
    lib.sc_probe_copy_variant.restype = I
    lib.sc_probe_copy_variant.argtypes = [P, P, I64, I, I, P]
    lib.sc_probe_scatter_rows.restype = I
    lib.sc_probe_scatter_rows.argtypes = [P, P, I64, I64, P, P, I64, P, I64, I64, I, I, P]
    return lib


def test_probe_exports_and_rejects_bad_arguments():
    lib = _lib()
    fake = P(4096)  # never dereferenced: every call below returns before any launch
    assert lib.sc_probe_copy_variant(fake, fake, 15, 0, 1, None) == -1      # not a multiple of 16
    assert lib.sc_probe_copy_variant(fake, fake, 32, 6, 1, None) == -1      # no such form
    assert lib.sc_probe_copy_variant(fake, fake, 32, 3, 0, None) == -1      # no workgroups
    assert lib.sc_probe_copy_variant(None, fake, 32, 0, 1, None) == -1
    assert lib.sc_probe_copy_variant(fake, fake, 0, 0, 1, None) == 0        # nothing to copy
    args = dict(k=fake, v=fake, ks=256, vs=256, kc=fake, vc=fake, rb=256, slot=fake, t=4, ns=8)

    def call(variant=0, bpc=1, **kw):
        a = {**args, **kw}
        return lib.sc_probe_scatter_rows(a["k"], a["v"], a["ks"], a["vs"], a["kc"], a["vc"],
                                         a["rb"], a["slot"], a["t"], a["ns"], variant, bpc, None)
    assert call(rb=24) == -1            # row not a multiple of 16
    assert call(ks=128) == -1           # stride shorter than a row
    assert call(vs=264) == -1           # stride not 16-byte aligned
    assert call(variant=7) == -1
    assert call(variant=5) == -1        # the fused-prefill forms need rows of whole KiB
    assert call(slot=None) == -1
    assert call(t=-1) == -1
    assert call(t=0, slot=None) == 0    # no tokens: nothing to do, nothing checked


@pytest.mark.gpu
@pytest.mark.parametrize("variant,bpc", [(0, 1), (1, 1), (2, 1), (3, 2), (3, 4), (4, 2), (5, 1)])
def test_copy_forms_are_exact(variant, bpc):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib = _lib()
    n = 16 * (3 * 256 * 8 * 5 + 77)  # several chunks of every form and a ragged tail
    g = torch.Generator(device="cpu").manual_seed(variant)
    src = torch.randint(0, 256, (n,), dtype=torch.uint8, generator=g).to("cuda:0")
    dst = torch.full((n + 64,), 0xA5, dtype=torch.uint8, device="cuda:0")
    stream = P(torch.cuda.current_stream().cuda_stream)
    assert lib.sc_probe_copy_variant(P(src.data_ptr()), P(dst.data_ptr()), n, variant, bpc,
                                     stream) == 0
    torch.cuda.synchronize()
    assert torch.equal(dst[:n], src)
    assert bool((dst[n:] == 0xA5).all()), "the copy wrote past its end"


@pytest.mark.gpu
@pytest.mark.parametrize("variant,bpc", [(0, 1), (1, 1), (2, 1), (3, 1), (4, 2), (4, 4), (5, 1),
                                         (6, 1)])
@pytest.mark.parametrize("row_bytes,tokens", [(2048, 1037), (4096, 301), (1024, 1), (512, 77)])
def test_scatter_forms_move_rows_to_slots(variant, bpc, row_bytes, tokens):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib = _lib()
    rng = np.random.default_rng(row_bytes + tokens + variant)
    num_slots = tokens + 40
    slot = rng.permutation(num_slots)[:tokens].astype(np.int64)
    slot[rng.random(tokens) < 0.05] = -1          # padded tokens: dropped
    slot[min(3, tokens - 1)] = num_slots + 7      # outside the pool: dropped
    pad = 48                                      # source rows strided (a fused projection)
    kv = [torch.from_numpy(rng.integers(0, 256, (tokens, row_bytes + pad), dtype=np.uint8))
          .to("cuda:0") for _ in range(2)]
    caches = [torch.full((num_slots, row_bytes), 0xA5, dtype=torch.uint8, device="cuda:0")
              for _ in range(2)]
    sd = torch.from_numpy(slot).to("cuda:0")
    stream = P(torch.cuda.current_stream().cuda_stream)
    if variant >= 5 and row_bytes % 1024:
        assert lib.sc_probe_scatter_rows(P(kv[0].data_ptr()), P(kv[1].data_ptr()), row_bytes + pad,
                                         row_bytes + pad, P(caches[0].data_ptr()),
                                         P(caches[1].data_ptr()), row_bytes, P(sd.data_ptr()),
                                         tokens, num_slots, variant, bpc, stream) == -1
        return
    rc = lib.sc_probe_scatter_rows(P(kv[0].data_ptr()), P(kv[1].data_ptr()), row_bytes + pad,
                                   row_bytes + pad, P(caches[0].data_ptr()),
                                   P(caches[1].data_ptr()), row_bytes, P(sd.data_ptr()), tokens,
                                   num_slots, variant, bpc, stream)
    assert rc == 0
    torch.cuda.synchronize()
    ok = (slot >= 0) & (slot < num_slots)
    for src, cache in zip(kv, caches):
        got = cache.cpu().numpy()
        exp = np.full((num_slots, row_bytes), 0xA5, np.uint8)
        exp[slot[ok]] = src.cpu().numpy()[ok, :row_bytes]
        assert np.array_equal(got, exp)
