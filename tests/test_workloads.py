"""The seeded input generator (CPU): same seed, same inputs; another seed, other inputs; each
tensor from its own stream, so a change to one recipe leaves the other tensors unchanged; the
five configurations have the shapes and structure their recipes state."""
import hashlib

import numpy as np

import workloads


def _digest(w):
    h = hashlib.sha256()
    for a in (w.k_taps, w.v_taps, w.k_gamma, w.v_gamma, w.k_state, w.v_state):
        if a is not None:
            h.update(np.ascontiguousarray(a).tobytes())
    for st in w.steps:
        for a in (st.k, st.v, st.slot_mapping, st.state_idx, st.cu_seqlens, st.has_init):
            if a is not None:
                h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def test_same_seed_same_inputs_other_seed_other_inputs():
    for name in ("tiny_ref", "varlen_prefill", "decode"):
        a, b = workloads.config(name, seed=0), workloads.config(name, seed=1)
        assert _digest(a) == _digest(workloads.config(name, seed=0)) and _digest(a) != _digest(b)


def test_streams_are_independent():
    base = workloads.Spec(dtype="bf16", H=2, D=64, W=4, seed=3, prefill_lens=[20, 7],
                          has_init=[1, 0])
    a = workloads.build(base)
    base.outlier_p = 0.05  # changes only the K/V draws
    b = workloads.build(base)
    assert not np.array_equal(a.steps[0].k, b.steps[0].k)
    for name in ("k_taps", "v_taps", "k_gamma", "v_gamma", "k_state", "v_state"):
        assert np.array_equal(getattr(a, name), getattr(b, name)), name
    assert np.array_equal(a.steps[0].slot_mapping, b.steps[0].slot_mapping)


def test_config_shapes_and_structure():
    w2 = workloads.config("varlen_prefill")
    st = w2.steps[0]
    lens = np.diff(st.cu_seqlens)
    assert st.num_seqs == 8 and ((lens >= 512) & (lens <= 4096)).all() and w2.tokens == 17060
    assert (st.has_init == 0).all() and w2.W == 4 and (w2.H, w2.D, w2.dtype) == (8, 128, "bf16")
    # paged: distinct slots inside the pool, 16-token blocks contiguous within a block
    assert len(np.unique(st.slot_mapping)) == st.tokens and st.slot_mapping.max() < w2.num_slots
    first = st.slot_mapping[:16]
    assert (np.diff(first) == 1).all() and first[0] % 16 == 0
    w3 = workloads.config("decode")
    d = w3.steps[0]
    assert d.kind == "decode" and d.tokens == 256 and len(np.unique(d.state_idx)) == 256
    # the large ones by their recipes (building them draws ~10^9 numbers)
    s4 = workloads.config_spec("long_prefill")
    assert s4.W == 8 and list(s4.prefill_lens) == [131072] and s4.outlier_p == 0.01
    s5 = workloads.config_spec("mixed")
    assert s5.H == 16 and list(s5.prefill_lens) == [2048] * 64 and len(s5.decode_ctx) == 512
    assert all(s5.has_init) and all(p % 2048 == 0 and 2048 <= p <= 2048 * 15
                                    for p in s5.prefill_start)
