"""Write tests/golden/tiny_ref_oracle.json from the oracle (and the seeded generator) only.

The pages print no worked example, table of values or test vector for the fused ShortConv K/V
step (the English aib.vote news item on SGLang/Miles Inkling support gives only a speed ratio),
so no stored value here comes from them. This fixture is a regression snapshot of the oracle on
the 64-token fp32 reference workload, seed 0: it fails if the oracle's arithmetic or the input
generator drifts. Its correctness rests on the pins in tests/oracle_pins.py, not on itself.

Run from the repository root:  python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import workloads  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_ref_oracle.json")
TOKENS = [0, 1, 2, 3, 31, 62, 63]
CHANNELS = [0, 1, 7, 31, 63]


def sha(*arrays):
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def snapshot():
    w = workloads.config("tiny_ref")
    st = w.steps[0]
    r = oracle.fused_prefill(st.k, st.v, st.cu_seqlens, w.k_taps, w.v_taps, w.k_gamma, w.v_gamma,
                             w.eps, w.k_state, w.v_state, st.state_idx, st.has_init,
                             st.slot_mapping, w.num_slots, cond=False)
    return {
        "workload": w.recipe,
        "seed": 0,
        "input_sha256": sha(st.k, st.v, w.k_taps, w.v_taps, w.k_gamma, w.v_gamma, w.k_state),
        "tokens": TOKENS,
        "channels": CHANNELS,
        "y_k_hex": [[float(r.y_k[t, 0, d]).hex() for d in CHANNELS] for t in TOKENS],
        "y_v_hex": [[float(r.y_v[t, 0, d]).hex() for d in CHANNELS] for t in TOKENS],
        "k_state_sha256": sha(r.k_state),
        "v_state_sha256": sha(r.v_state),
    }


if __name__ == "__main__":
    with open(OUT, "w") as f:
        json.dump(snapshot(), f, indent=1)
        f.write("\n")
    print(OUT)
