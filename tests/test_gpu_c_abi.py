"""The C ABI used from plain C: tests/abi_c/from_c.c (C99, only include/shortconv.h and the HIP
runtime) allocates its own device buffers, runs one prefill and writes the results back; they
must match the oracle as the binding's results do (placement and state bit for bit, rows within
the tolerance, untouched rows keeping their sentinel)."""
import ctypes
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "abi_c", "libfrom_c.so")


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("dtype,W", [("bf16", 4), ("f32", 3)])
def test_prefill_from_c(tmp_path, dtype, W):
    if not os.path.exists(LIB):
        from abi_c import build
        build.build()
    lib = ctypes.CDLL(LIB)
    lib.sc_c_prefill.restype = ctypes.c_int
    lib.sc_c_prefill.argtypes = [ctypes.c_char_p]
    H, D = 4, 128
    spec = workloads.Spec(dtype=dtype, H=H, D=D, W=W, seed=8, prefill_lens=[50, 0, 7, 130],
                          has_init=[1, 1, 0, 1], block_size=16, pad_slot_every=11, spare_slots=9)
    w = workloads.build(spec)
    st = w.steps[0]
    N, T, S = st.num_seqs, st.tokens, w.num_state_slots
    stored = np.float32 if dtype == "f32" else np.uint16
    sentinel = workloads.SENTINEL[dtype]
    cache = np.full((w.num_slots, H, D), sentinel, dtype=stored)
    files = {
        "k.bin": np.ascontiguousarray(st.k), "v.bin": np.ascontiguousarray(st.v),
        "kt.bin": w.k_taps, "vt.bin": w.v_taps, "kg.bin": w.k_gamma, "vg.bin": w.v_gamma,
        "cu.bin": st.cu_seqlens.astype(np.int32), "sidx.bin": st.state_idx.astype(np.int32),
        "hinit.bin": st.has_init.astype(np.uint8), "slot.bin": st.slot_mapping.astype(np.int64),
        "ks.bin": w.k_state, "vs.bin": w.v_state, "kc.bin": cache, "vc.bin": cache,
    }
    for name, arr in files.items():
        np.ascontiguousarray(arr).tofile(tmp_path / name)
    code = 0 if dtype == "f32" else 1
    (tmp_path / "meta.txt").write_text(
        f"{T} {N} {H} {D} {W} {S} {w.num_slots} {code} {repr(float(w.eps))}\n")
    assert lib.sc_c_prefill(str(tmp_path).encode()) == 0

    def out(name, shape):
        return np.fromfile(tmp_path / name, dtype=stored).reshape(shape)

    r = oracle.fused_prefill(st.k, st.v, st.cu_seqlens, w.k_taps, w.v_taps, w.k_gamma, w.v_gamma,
                             w.eps, w.k_state, w.v_state, st.state_idx, st.has_init,
                             st.slot_mapping, w.num_slots)
    for name, y, cond, new_state, got_state in (
            ("K", r.y_k, r.cond_k, r.k_state, "ks_out.bin"),
            ("V", r.y_v, r.cond_v, r.v_state, "vs_out.bin")):
        got = out(("kc_out.bin" if name == "K" else "vc_out.bin"), (w.num_slots, H, D))
        ok = r.slots >= 0
        res = oracle.compare(got[r.slots[ok]], y[ok], cond[ok], dtype)
        assert res["ok"], f"{name}: cache rows from C differ from the oracle: {res}"
        untouched = np.setdiff1d(np.arange(w.num_slots), r.slots[ok])
        assert (got[untouched].view(np.uint8) == cache[untouched].view(np.uint8)).all()
        assert np.array_equal(out(got_state, new_state.shape), new_state), f"{name}: state"
