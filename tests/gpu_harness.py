"""GPU-side test plumbing: move a synthetic workload to the device, run it through the C ABI (via
the Python binding), and judge the result against the oracle.

Judging rules (the bar):
  * cache placement: every row the oracle writes is compared element by element (oracle.compare:
    tolerance 1e-5 relative for fp32 I/O, one bf16 ulp (3.9e-3) for bf16 I/O, plus the rounding
    floor for cancelling taps); every other cache row must still hold the sentinel, bit for bit;
  * conv state: the whole pool must equal the oracle's, bit for bit.
"""
import os

import numpy as np
import torch

import oracle
import workloads
from causal_short_convolution_amd import shortconv_kv_decode, shortconv_kv_prefill

DEV = "cuda:0"
TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}
BITS_DT = {"f32": torch.int32, "bf16": torch.int16}
ORACLE_THREADS = max(1, min(16, os.cpu_count() or 1))
CHUNK = 8192  # cache rows compared per batch


def to_dev(a: np.ndarray, dtype: str = None):
    """numpy stored array -> device tensor (uint16 bf16 bits become torch.bfloat16)."""
    if a is None:
        return None
    if a.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(DEV)


def rows_to_dev(x: np.ndarray):
    """[T,H,D] host rows (possibly a strided view) -> device rows with the same token stride."""
    T, H, D = x.shape
    item = x.itemsize
    stride = x.strides[0] // item if T > 1 else H * D
    if stride == H * D:
        return to_dev(np.ascontiguousarray(x))
    base = np.zeros((T, stride), dtype=x.dtype)
    base[:, :H * D] = x.reshape(T, H * D)
    return to_dev(base)[:, :H * D].view(T, H, D)


def to_host(t: torch.Tensor, dtype: str) -> np.ndarray:
    t = t.detach()
    if dtype == "bf16":
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.contiguous().cpu().numpy()


def sentinel_cache(num_slots, H, D, dtype):
    c = torch.empty((num_slots, H, D), dtype=TORCH_DT[dtype], device=DEV)
    c.view(BITS_DT[dtype]).fill_(int(workloads.SENTINEL[dtype]))  # both patterns are positive
    return c


class DeviceWorkload:
    """Device copies of a workload's inputs, pools and per-step arguments."""

    def __init__(self, w: workloads.Workload, caches=True):
        self.w = w
        self.k_taps = to_dev(w.k_taps)
        self.v_taps = to_dev(w.v_taps)
        self.k_gamma = to_dev(w.k_gamma)
        self.v_gamma = to_dev(w.v_gamma)
        self.k_state = to_dev(w.k_state)
        self.v_state = to_dev(w.v_state)
        self.k_cache = sentinel_cache(w.num_slots, w.H, w.D, w.dtype) if caches else None
        self.v_cache = sentinel_cache(w.num_slots, w.H, w.D, w.dtype) if caches else None
        self.steps = []
        for st in w.steps:
            d = dict(kind=st.kind, k=rows_to_dev(st.k), v=rows_to_dev(st.v),
                     slot=to_dev(st.slot_mapping.astype(np.int64)),
                     sidx=to_dev(st.state_idx.astype(np.int32)))
            if st.kind == "prefill":
                d["cu"] = to_dev(st.cu_seqlens.astype(np.int32))
                d["hinit"] = to_dev(st.has_init.astype(np.uint8))
            self.steps.append(d)

    def launch(self, i, stream=None):
        w, d = self.w, self.steps[i]
        if d["kind"] == "prefill":
            shortconv_kv_prefill(d["k"], d["v"], d["cu"], self.k_taps, self.v_taps, self.k_gamma,
                                 self.v_gamma, w.eps, self.k_state, self.v_state, d["sidx"],
                                 d["hinit"], d["slot"], self.k_cache, self.v_cache, stream=stream)
        else:
            shortconv_kv_decode(d["k"], d["v"], self.k_taps, self.v_taps, self.k_gamma,
                                self.v_gamma, w.eps, self.k_state, self.v_state, d["sidx"],
                                d["slot"], self.k_cache, self.v_cache, stream=stream)

    def run(self, stream=None):
        for i in range(len(self.steps)):
            self.launch(i, stream)
        torch.cuda.synchronize()


def oracle_steps(w: workloads.Workload):
    """Oracle results for each step in order, the state pools carried from step to step."""
    ks, vs = w.k_state, w.v_state
    out = []
    for st in w.steps:
        if st.kind == "prefill":
            r = oracle.fused_prefill(st.k, st.v, st.cu_seqlens, w.k_taps, w.v_taps, w.k_gamma,
                                     w.v_gamma, w.eps, ks, vs, st.state_idx, st.has_init,
                                     st.slot_mapping, w.num_slots, nthreads=ORACLE_THREADS)
        else:
            r = oracle.fused_decode(st.k, st.v, w.k_taps, w.v_taps, w.k_gamma, w.v_gamma, w.eps,
                                    ks, vs, st.state_idx, st.slot_mapping, w.num_slots,
                                    nthreads=ORACLE_THREADS)
        ks, vs = r.k_state, r.v_state
        out.append(r)
    return out


def judge(dw: DeviceWorkload, results=None):
    """Compare a finished device run with the oracle. Returns a report dict; raises
    AssertionError on any violation."""
    w = dw.w
    results = results or oracle_steps(w)
    report = {"worst": 0.0, "max_rel_well_conditioned": 0.0, "rows": 0, "elements": 0,
              "n_over_rel": 0, "max_rel_over_rel": 0.0}
    written = []
    for r in results:
        ok = r.slots >= 0
        slots = r.slots[ok]
        written.append(slots)
        if slots.size == 0:
            continue
        rows = np.flatnonzero(ok)
        for a in range(0, rows.size, CHUNK):
            sel = rows[a:a + CHUNK]
            idx = torch.from_numpy(r.slots[sel]).to(DEV)
            for name, y, cnd, cache in (("K", r.y_k, r.cond_k, dw.k_cache),
                                        ("V", r.y_v, r.cond_v, dw.v_cache)):
                got = to_host(cache.index_select(0, idx), w.dtype)
                c = oracle.compare(got, y[sel], cnd[sel], w.dtype)
                assert c["ok"], f"{name} cache rows {sel[0]}.. outside tolerance: {c}"
                report["worst"] = max(report["worst"], c["worst"])
                report["max_rel_well_conditioned"] = max(report["max_rel_well_conditioned"],
                                                         c["max_rel_well_conditioned"])
                report["elements"] += c["n"]
                report["n_over_rel"] += c["n_over_rel"]
                report["max_rel_over_rel"] = max(report["max_rel_over_rel"],
                                                 c["max_rel_over_rel"])
        report["rows"] += int(slots.size)
    # every other row keeps the sentinel bits
    all_written = np.concatenate(written) if written else np.zeros(0, np.int64)
    sent = workloads.SENTINEL[w.dtype]
    sent_i = int(np.asarray(sent).view(np.int32 if w.dtype == "f32" else np.int16))
    for cache in (dw.k_cache, dw.v_cache):
        bits = cache.view(BITS_DT[w.dtype])
        if all_written.size:
            bits.index_fill_(0, torch.from_numpy(all_written).to(DEV), sent_i)
        assert not bool((bits != sent_i).any()), "a cache row that no token maps to was written"
    # conv-state pools, bit for bit
    final = results[-1] if results else None
    if w.k_state is not None and final is not None:
        for name, exp, dev in (("K", final.k_state, dw.k_state), ("V", final.v_state, dw.v_state)):
            got = to_host(dev, w.dtype)
            if not np.array_equal(got.view(np.uint8), exp.view(np.uint8)):
                bad = np.argwhere(got != exp)
                raise AssertionError(f"{name} conv state differs at {len(bad)} elements, "
                                     f"first {bad[:3].tolist()}")
    return report
