#!/usr/bin/env python3
"""Benchmark of the fused ShortConv K/V step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload varlen_prefill] [--no-cpu-baseline]
                    [--no-decode] [--no-extras] [--only main|decode|mxfp8|verify|backward|copy]

A step is one call of the fused step over one batch of the workload (for the default workload:
8 packed sequences of U{512..4096} tokens, 8 KV heads x 128, W = 4, bf16 rows with fp32
arithmetic, paged cache with 16-token blocks). Inputs are resident in HBM before timing starts.
The batch is replicated into enough distinct device buffers that consecutive steps never find
their data in the 256 MB Infinity Cache; step i uses replica i mod R.

The K timed launches are captured once into a HIP graph and replayed (host launch cost would
otherwise pace short kernels); --eager launches them from Python instead.

Prints ONE JSON line: tokens/s over the timed steps (wall clock between two device
synchronizations), the average duration of one step (device time between HIP events recorded on
the launch stream before the first and after the last launch, divided by K), algorithmic HBM
bytes / that duration against the 8 TB/s peak (`roofline`, with the counter-measured `traffic`
while profiles/ holds counters for these kernel sources), a same-bytes copy (`copy_ceiling`), and
the fp64 CPU oracle timed on the host's cores and on one core (`cpu_baseline`). Beside the
headline workload the line carries the same measurement for each of the other four workloads
(`tiny_ref`, `decode`, `long_prefill`, `mixed`: time, algorithmic bytes, fraction of 8 TB/s,
same-bytes copy ceiling, the oracle on the host), for the two large ones also with MXFP8 cache
rows and the backward of their prefill call, and for the headline workload the MXFP8 rows, a
speculative verify + commit step and the backward. --no-extras keeps the headline only.
--only NAME runs one measurement and prints a line of text instead (for profiling and sweeps);
--workload picks another of the five workloads as the headline.

Profiling helpers (run under rocprofv3, then summarize):
    --calibrate-copy         also run a plain device copy of known size (counter calibration)
    --summarize-profile DIR  turn rocprofv3 CSV output in DIR into a summary for profiles/
"""
import argparse
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused ShortConv K/V tokens/s + achieved HBM GB/s (% of 8 TB/s), prefill & decode"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, AMD published peak
MALL_BYTES = 256 << 20          # MI355X Infinity Cache
COLD_FLUSH_BYTES = 2 * MALL_BYTES  # scratch written before every cold launch
COLD_LAUNCHES = 60
KERNEL_SRC = [os.path.join(ROOT, "causal_short_convolution_amd", "csrc", f)
              for f in ("kernels.hip", "device_common.h")]
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "fused_kernels_traffic.md")
COPY_BYTES = 512 << 20          # calibration copy: 512 MiB read + 512 MiB written
KERNELS = ("prefill_kernel", "prefill_slice_kernel", "prefill_run_kernel", "decode_kernel",
           "verify_kernel", "commit_kernel", "mx_quantize_kernel", "backward_kernel",
           "backward_chunk_kernel", "backward_final_kernel")
# DRAM-side request sizes on gfx950, as the calibration copy shows (512 MiB read in 4 Mi
# TCC_EA0_RDREQ_DRAM requests, 512 MiB written in 8 Mi TCC_EA0_WRREQ_DRAM requests)
DRAM_RD_BYTES, DRAM_WR_BYTES = 128, 64


def kernel_source_sha():
    """sha256 of the prefill kernel's sources (kernels.hip, then device_common.h)."""
    h = hashlib.sha256()
    for path in KERNEL_SRC:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


# ------------------------------------------------------------------------------------------------
# Algorithmic bytes: what the step must move, with no halo re-reads and no metadata caching.
# R = H * D * element bytes (one token row of K or V); C = one cache row: R, or for MXFP8 rows
# H * D code bytes + H * D / 32 scale bytes.
#   prefill: per token read K and V rows, write K and V cache rows, read the int64 slot (2R + 2C
#            + 8); per sequence read cu_seqlens, state_idx, has_init (9 B) and write 2 (W-1) state
#            rows, plus 2 (W-1) state rows read when it resumes from a stored state; taps and
#            gamma once.
#   decode:  per token 2R new rows + 2 (W-1) R state read + 2 (W-1) R state written + 2C cache
#            rows + 8 B slot + 4 B state index; taps and gamma once.
#   verify:  as prefill resuming every sequence from its state, but instead of the state write,
#            2 (W-1) R snapshot bytes per token; commit: per sequence cu_seqlens, accepted and
#            state_idx (12 B) and, where it accepts a token, 2 (W-1) R snapshot read + 2 (W-1) R
#            state written.
# ------------------------------------------------------------------------------------------------
def cache_row_bytes(w, cache):
    E = 4 if w.dtype == "f32" else 2
    return w.H * w.D * E if cache == "io" else w.H * w.D + w.H * w.D // 32


def algorithmic_bytes(w, step, cache="io"):
    E = 4 if w.dtype == "f32" else 2
    R = w.H * w.D * E
    C = cache_row_bytes(w, cache)
    params = 2 * (w.W * w.H * w.D * 4 + w.D * 4)
    if step.kind == "prefill":
        T, N = step.tokens, step.num_seqs
        n_init = int(step.has_init.sum()) if w.W > 1 else 0
        state = 2 * (w.W - 1) * R * (N + n_init) if w.W > 1 else 0
        return T * (2 * R + 2 * C + 8) + N * 9 + 4 + state + params
    B = step.tokens
    return B * (2 * R + 2 * C + 4 * (w.W - 1) * R + 12) + params


def verify_bytes(w, accepted, max_tokens):
    """(verify bytes, commit bytes) of one speculative step of workload w."""
    import numpy as np
    st = w.steps[0]
    E = 4 if w.dtype == "f32" else 2
    R = w.H * w.D * E
    rows = 2 * (w.W - 1) * R
    lens = np.diff(st.cu_seqlens.astype(np.int64))
    N, T = st.num_seqs, st.tokens
    params = 2 * (w.W * w.H * w.D * 4 + w.D * 4)
    verify = (T * (4 * R + 8) + N * 8 + 4 + rows * N + rows * int(np.minimum(lens, max_tokens)
                                                                  .sum()) + params)
    m = np.minimum(np.minimum(accepted, lens), max_tokens)
    commit = N * 12 + 4 + 2 * rows * int((m >= 1).sum())
    return verify, commit


def input_digest(w):
    """sha256 (first 16 hex digits) of every input array of workload w, in a fixed order: the
    bench's numbers are tied to exactly these inputs."""
    import numpy as np
    h = hashlib.sha256()
    for a in (w.k_taps, w.v_taps, w.k_gamma, w.v_gamma, w.k_state, w.v_state):
        if a is not None:
            h.update(np.ascontiguousarray(a).tobytes())
    for st in w.steps:
        for a in (st.k, st.v, st.slot_mapping, st.state_idx, st.cu_seqlens, st.has_init):
            if a is not None:
                h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="varlen_prefill",
                    choices=["tiny_ref", "varlen_prefill", "decode", "long_prefill", "mixed"])
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-decode", action="store_true", help="skip the decode measurement")
    ap.add_argument("--no-extras", action="store_true",
                    help="measure the headline workload only (no other workloads, MXFP8 rows, "
                         "speculative verify or backward)")
    ap.add_argument("--only", default=None,
                    choices=["main", "decode", "mxfp8", "verify", "backward", "copy", "pattern",
                             "cold"],
                    help="run one measurement only (for profiling); prints no JSON line")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="CPU time budget of the oracle baseline sample")
    ap.add_argument("--eager", action="store_true", help="launch from Python instead of a graph")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-launch legs (e.g. under a kernel trace of the warm steps)")
    ap.add_argument("--cold-flush", default="write", choices=["write", "read"],
                    help="how --only cold evicts the caches before each launch")
    ap.add_argument("--summarize-profile", default=None, nargs="+", metavar="DIR")
    return ap.parse_args()


# ------------------------------------------------------------------------------------------------
# Device side
# ------------------------------------------------------------------------------------------------
def device_replicas(w, torch, n_rep, reseed=None, cache="io"):
    """n_rep device copies of workload w (fresh buffers each). With reseed, replica r > 0 is
    drawn again with another seed (reseed(r)), so its slots differ and writes never revisit a
    row, and all replicas share one cache pool (decode-style pools are tens of GB). cache="io"
    allocates I/O-dtype cache rows, "mxfp8" code and scale rows, None no cache at all."""
    import numpy as np
    from causal_short_convolution_amd import _binding  # noqa: F401  (fails loudly if not built)

    dev = "cuda:0"
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def t(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(dt).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    shared = dict(k_taps=t(w.k_taps), v_taps=t(w.v_taps), k_gamma=t(w.k_gamma),
                  v_gamma=t(w.v_gamma), eps=w.eps)
    reps = []
    for r in range(n_rep):
        wr = reseed(r) if (reseed is not None and r > 0) else w
        steps = []
        for st in wr.steps:
            d = dict(shared, kind=st.kind)
            d["k"], d["v"] = t(st.k), t(st.v)
            d["slot"] = t(st.slot_mapping.astype(np.int64))
            d["sidx"] = t(st.state_idx.astype(np.int32))
            if st.kind == "prefill":
                d["cu"] = t(st.cu_seqlens.astype(np.int32))
                d["hinit"] = t(st.has_init.astype(np.uint8))
            steps.append(d)
        rep = {"steps": steps, "num_slots": wr.num_slots,
               "k_state": t(wr.k_state), "v_state": t(wr.v_state)}
        reps.append(rep)
    def pool(ns):
        if cache == "io":
            return {"k_cache": torch.empty((ns, w.H, w.D), dtype=dt, device=dev),
                    "v_cache": torch.empty((ns, w.H, w.D), dtype=dt, device=dev)}
        u8 = torch.uint8
        return {"k_cache": torch.empty((ns, w.H, w.D), dtype=u8, device=dev),
                "v_cache": torch.empty((ns, w.H, w.D), dtype=u8, device=dev),
                "k_scales": torch.empty((ns, w.H, w.D // 32), dtype=u8, device=dev),
                "v_scales": torch.empty((ns, w.H, w.D // 32), dtype=u8, device=dev)}

    if cache is None:
        pass
    elif reseed is not None:  # one pool large enough for every replica's slots
        shared_pool = pool(max(r["num_slots"] for r in reps))
        for r in reps:
            r.update(shared_pool)
    else:
        for r in reps:
            r.update(pool(r["num_slots"]))
    return reps


def launcher(w, rep, cache="io"):
    """One bench step: every call of the workload, in order, on the current stream."""
    import causal_short_convolution_amd as sc
    calls = []
    mx = cache == "mxfp8"
    for d in rep["steps"]:
        sc_args = (d["k_taps"], d["v_taps"], d["k_gamma"], d["v_gamma"], d["eps"],
                   rep["k_state"], rep["v_state"], d["sidx"])
        out = (rep["k_cache"], rep["v_cache"]) + ((rep["k_scales"], rep["v_scales"]) if mx else ())
        if d["kind"] == "prefill":
            fn = sc.shortconv_kv_prefill_mxfp8 if mx else sc.shortconv_kv_prefill
            calls.append(lambda d=d, fn=fn, a=sc_args, o=out: fn(
                d["k"], d["v"], d["cu"], *a, d["hinit"], d["slot"], *o))
        else:
            fn = sc.shortconv_kv_decode_mxfp8 if mx else sc.shortconv_kv_decode
            calls.append(lambda d=d, fn=fn, a=sc_args, o=out: fn(d["k"], d["v"], *a, d["slot"],
                                                                 *o))

    def step():
        for c in calls:
            c()
    return step


def verify_launcher(w, rep, accepted, max_tokens, torch):
    """One speculative step: verify the candidate runs (cache rows + per-token snapshots), then
    commit the accepted prefix of each sequence into the state pools."""
    import causal_short_convolution_amd as sc
    d = rep["steps"][0]
    shape = (w.steps[0].num_seqs, max_tokens, w.W - 1, w.H, w.D)
    k_snap = torch.empty(shape, dtype=d["k"].dtype, device=d["k"].device)
    v_snap = torch.empty_like(k_snap)
    acc = torch.from_numpy(accepted).to(d["k"].device)
    T = d["k"].shape[0]

    def step():
        sc.shortconv_kv_verify(d["k"], d["v"], d["cu"], d["k_taps"], d["v_taps"], d["k_gamma"],
                               d["v_gamma"], d["eps"], rep["k_state"], rep["v_state"], d["sidx"],
                               k_snap, v_snap, d["slot"], rep["k_cache"], rep["v_cache"])
        sc.shortconv_state_commit(k_snap, v_snap, d["cu"], T, acc, rep["k_state"],
                                  rep["v_state"], d["sidx"], width=w.W, num_heads=w.H,
                                  head_dim=w.D)
    return step


def time_steps(torch, fns, steps, warmup, graph=True):
    """Warm up, then time exactly `steps` launches (step i runs replica i mod R).

    graph=True: the `steps` launches are captured once into a HIP graph (torch.cuda.CUDAGraph)
    and the timed region is one replay, so host-side launch cost does not pace the device;
    graph=False: plain launches from Python. Returns (wall seconds between two device
    synchronizations, device milliseconds between events recorded on the launch stream
    before the first and after the last launch)."""
    for i in range(warmup):
        fns[i % len(fns)]()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(steps):
                fns[i % len(fns)]()
        g.replay()  # untimed: first replay uploads the graph
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record()
        g.replay()
        end.record()
        torch.cuda.synchronize()
    else:
        t0 = time.perf_counter()
        start.record()
        for i in range(steps):
            fns[i % len(fns)]()
        end.record()
        torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, start.elapsed_time(end)


def replica_count(step_bytes):
    """Distinct input copies so that a step never finds its data in the Infinity Cache: enough
    that 2x its capacity passes between two uses of a copy; one when a step alone moves 4x it."""
    if step_bytes >= 4 * MALL_BYTES:
        return 1
    return max(2, math.ceil(2 * MALL_BYTES / step_bytes) + 1)


def measure(torch, w, steps, warmup, reseed=None, graph=True, cache="io"):
    alg = sum(algorithmic_bytes(w, st, cache) for st in w.steps)
    tokens = w.tokens
    n_rep = replica_count(alg)
    reps = device_replicas(w, torch, n_rep, reseed, cache)
    fns = [launcher(w, r, cache) for r in reps]
    wall, dev_ms = time_steps(torch, fns, steps, warmup, graph)
    del reps, fns
    per_step_ms = dev_ms / steps
    return {
        "cache": cache,
        "tokens_per_step": tokens,
        "launches_per_step": len(w.steps),
        "replicas": n_rep,
        "launch": "hip graph replay" if graph else "eager",
        "wall_s": wall,
        "ms_per_step": 1e3 * wall / steps,
        "tokens_per_s": tokens * steps / wall,
        "kernel_us_mean": 1e3 * per_step_ms,
        "algorithmic_bytes": alg,
        "achieved_GBps": alg / (per_step_ms * 1e-3) / 1e9,
    }


def measure_verify(torch, steps, warmup, seed, graph=True):
    """Speculative verify + commit at the decode shape (workloads.spec_verify)."""
    import workloads
    w, accepted = workloads.spec_verify(seed)
    mt = workloads.SPEC_TOKENS
    vb, cb = verify_bytes(w, accepted, mt)
    n_rep = replica_count(vb + cb)
    draws = {0: (w, accepted)}

    def reseed(r):
        draws[r] = workloads.spec_verify(seed + 1000 * r)
        return draws[r][0]

    reps = device_replicas(w, torch, n_rep, reseed)
    fns = [verify_launcher(draws[i][0], r, draws[i][1], mt, torch) for i, r in enumerate(reps)]
    wall, dev_ms = time_steps(torch, fns, steps, warmup, graph)
    del reps, fns
    per_ms = dev_ms / steps
    return {"workload": w.name, "recipe": w.recipe, "tokens_per_step": w.tokens,
            "launches_per_step": 2, "replicas": n_rep, "ms_per_step": 1e3 * wall / steps,
            "tokens_per_s": w.tokens * steps / wall, "kernel_us_mean": 1e3 * per_ms,
            "algorithmic_bytes": vb + cb, "verify_bytes": vb, "commit_bytes": cb,
            "achieved_GBps": (vb + cb) / (per_ms * 1e-3) / 1e9}


def backward_bytes(w):
    """Algorithmic bytes of one backward call over workload w's prefill: per token read the K
    and V rows and their output gradients and write the two input-gradient rows (6R); per
    sequence that resumes from a stored state read its 2 (W-1) R state rows; taps and gamma read,
    their gradients written. The fp32 partials the kernel passes through its workspace are not
    counted (they are the implementation's, not the method's)."""
    st = w.steps[0]
    E = 4 if w.dtype == "f32" else 2
    R = w.H * w.D * E
    n_init = int(st.has_init.sum()) if w.W > 1 else 0
    params = 2 * 2 * (w.W * w.H * w.D * 4 + w.D * 4)
    return st.tokens * 6 * R + n_init * 2 * (w.W - 1) * R + st.num_seqs * 9 + 4 + params


def measure_backward(torch, w, steps, warmup, graph=True):
    """One backward call (shortconv_kv_backward) over the prefill call of workload w (its first
    call), with random output gradients; no new-state loss, no initial-state gradient."""
    import numpy as np
    import causal_short_convolution_amd as sc
    st = w.steps[0]
    dev = "cuda:0"
    alg = backward_bytes(w)
    n_rep = replica_count(alg)
    reps = device_replicas(w, torch, n_rep, cache=None)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    T, H, D, W = st.tokens, w.H, w.D, w.W
    ws = torch.empty(max(16, sc.shortconv_kv_backward_workspace_size(T, st.num_seqs, H, D, W, dt)),
                     dtype=torch.uint8, device=dev)
    grads = [torch.empty((W, H, D), device=dev) for _ in range(2)] + \
            [torch.empty((D,), device=dev) for _ in range(2)]
    hinit = torch.from_numpy(st.has_init.astype(np.uint8)).to(dev)
    fns = []
    for r in reps:
        d = r["steps"][0]
        dyk = torch.randn((T, H, D), device=dev).to(dt)
        dyv = torch.randn((T, H, D), device=dev).to(dt)
        dk, dv = torch.empty_like(dyk), torch.empty_like(dyv)

        def go(d=d, r=r, dyk=dyk, dyv=dyv, dk=dk, dv=dv):
            sc.shortconv_kv_backward(d["k"], d["v"], d["cu"], d["k_taps"], d["v_taps"],
                                     d["k_gamma"], d["v_gamma"], d["eps"], r["k_state"],
                                     r["v_state"], d["sidx"], hinit, dyk, dyv, dk, dv, *grads,
                                     workspace=ws)
        fns.append(go)
    wall, dev_ms = time_steps(torch, fns, steps, warmup, graph)
    del reps, fns
    per_ms = dev_ms / steps
    return {"workload": w.name, "tokens_per_step": T, "launches_per_step": 3, "replicas": n_rep,
            "ms_per_step": 1e3 * wall / steps, "tokens_per_s": T * steps / wall,
            "kernel_us_mean": 1e3 * per_ms, "algorithmic_bytes": alg,
            "workspace_bytes": ws.numel(), "achieved_GBps": alg / (per_ms * 1e-3) / 1e9}


# Copy forms of the probe library (see csrc/copy_probe.hip) tried for the same-bytes ceiling:
# (variant, workgroups per compute unit for the persistent forms, label).
COPY_FORMS = [(0, 1, "one-shot 4x16B/lane nt"), (1, 1, "one-shot 8x16B/lane nt"),
              (2, 1, "one-shot 2x16B/lane nt"), (5, 1, "one-shot 4x16B/lane cached"),
              (3, 2, "persistent 2 WG/CU, 4x16B chunks, pipelined"),
              (3, 4, "persistent 4 WG/CU, 4x16B chunks, pipelined"),
              (3, 8, "persistent 8 WG/CU, 4x16B chunks, pipelined"),
              (4, 2, "persistent 2 WG/CU, 8x16B chunks, pipelined"),
              (4, 4, "persistent 4 WG/CU, 8x16B chunks, pipelined")]


def copy_ceiling(torch, bytes_moved, steps, warmup, forms=None):
    """Same-bytes ceiling: plain copies that read bytes_moved/2 and write bytes_moved/2, in the
    same rotating-replica regime and graph replay as the fused kernel, in several forms (one-shot
    grids with 2-8 loads of 16 B per lane, persistent pipelined grids); the fastest is the
    ceiling, and every form's rate is returned in `forms`."""
    import ctypes
    from causal_short_convolution_amd import build as hip_build
    lib = ctypes.CDLL(hip_build.PROBE_LIB)
    lib.sc_probe_copy_variant.restype = ctypes.c_int
    lib.sc_probe_copy_variant.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    half = (bytes_moved // 2) // 16 * 16
    n_rep = replica_count(2 * half)
    bufs = [(torch.empty(half, dtype=torch.uint8, device="cuda:0"),
             torch.empty(half, dtype=torch.uint8, device="cuda:0")) for _ in range(n_rep)]

    def fn(src, dst, variant, bpc):
        def go():
            rc = lib.sc_probe_copy_variant(ctypes.c_void_p(src.data_ptr()),
                                           ctypes.c_void_p(dst.data_ptr()), half, variant, bpc,
                                           ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
            if rc != 0:
                raise RuntimeError(f"sc_probe_copy_variant failed: {rc}")
        return go

    table = []
    for variant, bpc, label in (forms or COPY_FORMS):
        _, dev_ms = time_steps(torch, [fn(a, b, variant, bpc) for a, b in bufs], steps, warmup,
                               graph=True)
        per_ms = dev_ms / steps
        table.append({"form": label, "kernel_us_mean": round(1e3 * per_ms, 3),
                      "GBps": round(2 * half / (per_ms * 1e-3) / 1e9, 1)})
    best = max(table, key=lambda r: r["GBps"])
    del bufs
    return {"bytes_moved": 2 * half, "kernel_us_mean": best["kernel_us_mean"],
            "GBps": best["GBps"], "form": best["form"], "forms": table}


# Forms of the probe's scatter (see csrc/copy_probe.hip) tried for the same-pattern ceiling.
SCATTER_FORMS = [(0, 1, "one-shot, 1 token per lane"), (1, 1, "one-shot, 2 tokens per lane"),
                 (2, 1, "one-shot, 4 tokens per lane"), (3, 1, "one-shot, 8 tokens per lane"),
                 (4, 2, "persistent 2 WG/CU, 4 tokens per unit, pipelined"),
                 (4, 4, "persistent 4 WG/CU, 4 tokens per unit, pipelined"),
                 (5, 1, "fused prefill's memory side, 8 tokens per wave"),
                 (6, 1, "fused prefill's memory side, 4 tokens per wave")]


def pattern_ceiling(torch, w, steps, warmup, forms=None):
    """Same-pattern ceiling of a workload made of prefill calls: the probe moves each call's K and
    V rows to their cache rows (row t to row slot[t]) and does nothing else -- no state rows, no
    halo, no arithmetic -- with the same inputs, replica rotation and graph replay as the fused
    step. Bytes moved: every row read plus every row written. The fastest form is the ceiling."""
    import ctypes
    import numpy as np
    from causal_short_convolution_amd import build as hip_build
    assert all(st.kind == "prefill" for st in w.steps)
    lib = ctypes.CDLL(hip_build.PROBE_LIB)
    lib.sc_probe_scatter_rows.restype = ctypes.c_int
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.sc_probe_scatter_rows.argtypes = [P, P, I64, I64, P, P, I64, P, I64, I64, I, I, P]
    item = 2 if w.dtype == "bf16" else 4
    row_bytes = w.H * w.D * item
    forms = [f for f in (forms or SCATTER_FORMS) if f[0] < 5 or row_bytes % 1024 == 0]
    moved = 0
    for st in w.steps:
        ok = (st.slot_mapping >= 0) & (st.slot_mapping < w.num_slots)
        moved += 2 * row_bytes * (len(st.slot_mapping) + int(np.count_nonzero(ok)))
    n_rep = replica_count(moved)
    reps = device_replicas(w, torch, n_rep, None, "io")

    def fn(rep, variant, bpc):
        calls = []
        for d in rep["steps"]:
            k, v = d["k"], d["v"]
            calls.append((P(k.data_ptr()), P(v.data_ptr()), k.stride(0) * item,
                          v.stride(0) * item, P(rep["k_cache"].data_ptr()),
                          P(rep["v_cache"].data_ptr()), row_bytes, P(d["slot"].data_ptr()),
                          k.shape[0], rep["k_cache"].shape[0]))

        def go():
            stream = P(torch.cuda.current_stream().cuda_stream)
            for c in calls:
                rc = lib.sc_probe_scatter_rows(*c, variant, bpc, stream)
                if rc != 0:
                    raise RuntimeError(f"sc_probe_scatter_rows failed: {rc}")
        return go

    table = []
    for variant, bpc, label in forms:
        _, dev_ms = time_steps(torch, [fn(r, variant, bpc) for r in reps], steps, warmup,
                               graph=True)
        per_ms = dev_ms / steps
        table.append({"form": label, "kernel_us_mean": round(1e3 * per_ms, 3),
                      "GBps": round(moved / (per_ms * 1e-3) / 1e9, 1)})
    best = max(table, key=lambda r: r["GBps"])
    del reps
    return {"bytes_moved": moved, "kernel_us_mean": best["kernel_us_mean"], "GBps": best["GBps"],
            "form": best["form"], "forms": table}


def pattern_entry(p, kernel_us):
    return {"what": "the fastest of several gather/scatter copies of the step's K/V rows to "
                    "their cache rows alone (no state rows, halo or arithmetic)",
            "bytes_moved": p["bytes_moved"], "kernel_us_mean": p["kernel_us_mean"],
            "GBps": p["GBps"], "frac_of_peak": p["GBps"] / HBM_PEAK_GBPS, "form": p["form"],
            "fused_time_over_pattern_time": kernel_us / p["kernel_us_mean"],
            "forms": p["forms"]}


def calibration_copy(torch):
    n = COPY_BYTES // 2
    src = torch.empty(n, dtype=torch.bfloat16, device="cuda:0").normal_()
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()


# ------------------------------------------------------------------------------------------------
# CPU baseline: the fp64 oracle, as it stands, on the same workload
# ------------------------------------------------------------------------------------------------
def host_cores():
    """(threads the oracle runs on, CPUs this process may use). The first is the host's CPU share
    for this GPU: OMP_NUM_THREADS when the environment sets it (shared GPU hosts give each GPU a
    fixed share of their cores), else every CPU in this process's affinity set."""
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:  # not Linux
        avail = os.cpu_count() or 1
    share = os.environ.get("OMP_NUM_THREADS", "")
    threads = min(avail, int(share)) if share.isdigit() and int(share) > 0 else avail
    return max(1, threads), avail


def _timed(fn, budget_s):
    """Run fn repeatedly for about budget_s seconds of CPU time; (repetitions, wall, cpu)."""
    reps = 0
    c0, t0 = time.process_time(), time.perf_counter()
    while True:
        fn()
        reps += 1
        if time.process_time() - c0 >= budget_s:
            break
    return reps, time.perf_counter() - t0, time.process_time() - c0


def oracle_step_fn(w, threads):
    """The oracle on every call of workload w, the state pools carried from call to call."""
    import oracle

    def run():
        ks, vs = w.k_state, w.v_state
        for st in w.steps:
            if st.kind == "prefill":
                r = oracle.fused_prefill(st.k, st.v, st.cu_seqlens, w.k_taps, w.v_taps, w.k_gamma,
                                         w.v_gamma, w.eps, ks, vs, st.state_idx, st.has_init,
                                         st.slot_mapping, w.num_slots, cond=False,
                                         nthreads=threads)
            else:
                r = oracle.fused_decode(st.k, st.v, w.k_taps, w.v_taps, w.k_gamma, w.v_gamma,
                                        w.eps, ks, vs, st.state_idx, st.slot_mapping,
                                        w.num_slots, cond=False, nthreads=threads)
            ks, vs = r.k_state, r.v_state
    return run


def cpu_baseline(w, budget_s, one_core_s):
    """The oracle on the whole workload w (every call, fp64), repeated for about budget_s seconds
    of CPU time on the host's cores, and for about one_core_s seconds on one thread."""
    threads, avail = host_cores()
    n, wall, cpu = _timed(oracle_step_fn(w, threads), budget_s)
    out = {"value": w.tokens * n / wall, "unit": "tokens/s", "cores": threads,
           "kind": "oracle",
           "sample": f"the whole {w.name} workload ({w.tokens} tokens, K and V, fp64) "
                     f"repeated {n}x: {wall:.1f} s wall, {cpu:.1f} s CPU on {threads} threads",
           "nproc": avail}
    if one_core_s > 0:
        n1, wall1, cpu1 = _timed(oracle_step_fn(w, 1), one_core_s)
        out["one_core"] = {"value": w.tokens * n1 / wall1, "unit": "tokens/s", "cores": 1,
                           "sample": f"the same workload repeated {n1}x on one thread: "
                                     f"{wall1:.1f} s wall"}
    return out


def cpu_baseline_extras(w, budget_s):
    """The oracle beside the extra measurements of workload w (a prefill workload), each on the
    same workload as its GPU figure and about budget_s seconds of CPU on the host's cores: the
    MXFP8 rows of w's prefill (the step plus the quantizer), the speculative verify + commit step
    and the backward of w's prefill."""
    import numpy as np
    import oracle
    import workloads
    threads, _ = host_cores()
    out = {}
    st = w.steps[0]

    def mx():
        r = oracle.fused_prefill(st.k, st.v, st.cu_seqlens, w.k_taps, w.v_taps, w.k_gamma,
                                 w.v_gamma, w.eps, w.k_state, w.v_state, st.state_idx,
                                 st.has_init, st.slot_mapping, w.num_slots, cond=False,
                                 nthreads=threads)
        oracle.mxfp8_quantize(r.y_k)
        oracle.mxfp8_quantize(r.y_v)
    n, wall, cpu = _timed(mx, budget_s)
    out["mxfp8_cache"] = {"value": st.tokens * n / wall, "unit": "tokens/s", "cores": threads,
                          "sample": f"{w.name} prefill + MXFP8 encoding x{n}: {wall:.1f} s wall, "
                                    f"{cpu:.1f} s CPU"}
    wv, acc = workloads.spec_verify(0)
    sv = wv.steps[0]

    def verify():
        _, ks, vs = oracle.fused_verify(sv.k, sv.v, sv.cu_seqlens, wv.k_taps, wv.v_taps,
                                        wv.k_gamma, wv.v_gamma, wv.eps, wv.k_state, wv.v_state,
                                        sv.state_idx, sv.slot_mapping, wv.num_slots,
                                        workloads.SPEC_TOKENS, cond=False, nthreads=threads)
        oracle.commit_state(wv.k_state, ks, acc, sv.cu_seqlens, sv.state_idx,
                            workloads.SPEC_TOKENS)
        oracle.commit_state(wv.v_state, vs, acc, sv.cu_seqlens, sv.state_idx,
                            workloads.SPEC_TOKENS)
    n, wall, cpu = _timed(verify, budget_s)
    out["spec_verify"] = {"value": sv.tokens * n / wall, "unit": "tokens/s", "cores": threads,
                          "sample": f"spec_verify (verify + commit) x{n}: {wall:.1f} s wall, "
                                    f"{cpu:.1f} s CPU"}
    out["backward"] = cpu_baseline_backward(w, budget_s)
    return out


def cpu_baseline_backward(w, budget_s):
    """The oracle's backward of workload w's prefill call, about budget_s seconds of CPU."""
    import numpy as np
    import oracle
    threads, _ = host_cores()
    st = w.steps[0]
    g = np.random.default_rng(0).standard_normal((st.tokens, w.H, w.D))

    def bwd():
        oracle.fused_backward(st.k, st.v, st.cu_seqlens, w.k_taps, w.v_taps, w.k_gamma,
                              w.v_gamma, w.eps, w.k_state, w.v_state, st.state_idx,
                              st.has_init, g, g, nthreads=threads)
    n, wall, cpu = _timed(bwd, budget_s)
    return {"value": st.tokens * n / wall, "unit": "tokens/s", "cores": threads,
            "sample": f"{w.name} backward x{n}: {wall:.1f} s wall, {cpu:.1f} s CPU"}


# ------------------------------------------------------------------------------------------------
# Profile summaries (rocprofv3 CSV output -> a short text summary for profiles/)
# ------------------------------------------------------------------------------------------------
def summarize_profile(dirs):
    """Summarize rocprofv3 CSV output: kernel-trace statistics, and per-dispatch HBM traffic of
    the fused kernels from FETCH_SIZE / WRITE_SIZE passes, each scaled by what the same counter
    reads for the calibration copy (--calibrate-copy: COPY_BYTES read and COPY_BYTES written)."""
    import csv

    def short(name):
        return name.replace("sc::(anonymous namespace)::", "").replace(
            "(anonymous namespace)::", "").replace("void ", "").replace("sc::", "")
    out = []
    per = {}  # (kernel, counter) -> values per dispatch
    for d in dirs:
        for path in sorted(glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)):
            out.append(f"kernel stats ({os.path.relpath(path, ROOT)}):")
            with open(path) as f:
                for row in csv.DictReader(f):
                    out.append(f"  {short(row['Name'])[:60]:60s} calls={row['Calls']:>5s} "
                               f"avg_ns={float(row['AverageNs']):10.1f} "
                               f"min_ns={row['MinNs']:>8s} max_ns={row['MaxNs']:>8s}")
        for path in sorted(glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)):
            # one line per (kernel, grid): a kernel that serves several workloads (of different
            # shapes) gets one line for each
            durs, res = {}, {}
            with open(path) as f:
                for row in csv.DictReader(f):
                    ns = int(row["End_Timestamp"]) - int(row["Start_Timestamp"])
                    name = short(row["Kernel_Name"]).split("(")[0]
                    grid = "x".join(row[c] for c in ("Grid_Size_X", "Grid_Size_Y") if c in row)
                    durs.setdefault((name, grid), []).append(ns)
                    res[name] = (row.get("VGPR_Count"), row.get("LDS_Block_Size"),
                                 row.get("Scratch_Size"))
            out.append(f"per-dispatch durations by kernel and grid ({os.path.relpath(path, ROOT)}):")
            for (name, grid), v in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
                v = sorted(v)

                def q(f, v=v):
                    return v[min(len(v) - 1, int(f * len(v)))]
                out.append(f"  {name[:56]:56s} grid={grid:>11s} n={len(v):>5d} "
                           f"mean_ns={sum(v) / len(v):10.1f} p10_ns={q(0.1):>8d} "
                           f"median_ns={q(0.5):>8d} p90_ns={q(0.9):>8d}")
            out.append("kernel resources as the tracer reports them (VGPR_Count in its own units, not "
                       "the register allocation, which the compiler's resource report gives; LDS and "
                       "scratch bytes):")
            for name, (vg, lds, scr) in sorted(res.items()):
                if any(k in name for k in KERNELS):
                    out.append(f"  {name[:56]:56s} vgpr={vg} lds={lds} scratch={scr}")
        for path in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"),
                                     recursive=True)):
            with open(path) as f:
                for row in csv.DictReader(f):
                    name = short(row["Kernel_Name"])
                    kind = ("copy" if "copyBuffer" in name else name.split("(")[0]
                            if any(k in name for k in KERNELS) else None)
                    if kind:
                        per.setdefault((kind, row["Counter_Name"]), []).append(
                            float(row["Counter_Value"]))
    known_kib = COPY_BYTES / 1024.0
    factors = {}
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        copies = sorted(per.get(("copy", ctr), []))[-5:]  # the calibration copies are the largest
        if copies:
            factors[ctr] = known_kib / (sum(copies) / len(copies))
            out.append(f"calibration copy {ctr}: {sum(copies) / len(copies):.1f} KiB per dispatch "
                       f"for {known_kib:.0f} KiB moved -> factor {factors[ctr]:.4f}")
    for ctr, size in (("TCC_EA0_RDREQ_DRAM_sum", DRAM_RD_BYTES),
                      ("TCC_EA0_WRREQ_DRAM_sum", DRAM_WR_BYTES)):
        copies = sorted(per.get(("copy", ctr), []))[-5:]
        if copies:
            mean = sum(copies) / len(copies)
            out.append(f"calibration copy {ctr}: {mean:.0f} requests per dispatch x {size} B = "
                       f"{mean * size / COPY_BYTES:.4f} x the {COPY_BYTES} bytes moved")

    def mean(kind, ctr):
        v = per.get((kind, ctr))
        return sum(v) / len(v) if v else None
    for kind in sorted({k for k, _ in per if k != "copy"}):
        f_kib, w_kib = mean(kind, "FETCH_SIZE"), mean(kind, "WRITE_SIZE")
        if f_kib is not None and w_kib is not None and len(factors) == 2:
            tr = 1024.0 * (f_kib * factors["FETCH_SIZE"] + w_kib * factors["WRITE_SIZE"])
            out.append(f"{kind}: FETCH_SIZE {f_kib:.1f} KiB, WRITE_SIZE {w_kib:.1f} KiB per "
                       f"dispatch -> {tr:.0f} HBM bytes per launch (calibrated)")
        rd, wr = mean(kind, "TCC_EA0_RDREQ_DRAM_sum"), mean(kind, "TCC_EA0_WRREQ_DRAM_sum")
        if rd is not None and wr is not None:
            out.append(f"{kind}: DRAM requests {rd:.0f} read x {DRAM_RD_BYTES} B + {wr:.0f} write x "
                       f"{DRAM_WR_BYTES} B = {rd * DRAM_RD_BYTES + wr * DRAM_WR_BYTES:.0f} bytes per "
                       f"dispatch ({rd * DRAM_RD_BYTES:.0f} read, {wr * DRAM_WR_BYTES:.0f} written)")
        waves, valu = mean(kind, "SQ_WAVES"), mean(kind, "SQ_INSTS_VALU")
        if waves and valu is not None:
            out.append(f"{kind}: {valu / waves:.1f} VALU instructions per wave")
        others = sorted({c for k, c in per if k == kind})
        out.append(f"{kind}: counters (mean per dispatch): " + ", ".join(
            f"{c} {mean(kind, c):.1f}" for c in others))
    print("\n".join(out))


# ------------------------------------------------------------------------------------------------
def measure_cold(torch, w, launches=COLD_LAUNCHES, warmup=3, flush="write"):
    """The cold protocol: before every timed step a 512 MiB scratch write (twice the Infinity
    Cache) evicts the step's data from every cache; each step is then timed alone, eagerly, by HIP
    events on its stream (the interval includes the launch's own dispatch latency, which a graph
    replay hides), and the median over the launches is reported with p10 and p90. A kernel trace
    of `--only cold` gives the same launches' kernel durations. flush="read" reads the scratch
    instead, which evicts as much but leaves no dirty lines for the step to write back."""
    alg = sum(algorithmic_bytes(w, st) for st in w.steps)
    reps = device_replicas(w, torch, 1)
    step = launcher(w, reps[0])
    scratch = torch.empty(COLD_FLUSH_BYTES, dtype=torch.uint8, device="cuda:0")
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(launches)]
    words = scratch.view(torch.int32)
    for i in range(warmup + launches):
        if flush == "read":
            torch.amax(words)
        else:
            scratch.fill_(i & 0xFF)
        if i >= warmup:
            evs[i - warmup][0].record()
        step()
        if i >= warmup:
            evs[i - warmup][1].record()
    torch.cuda.synchronize()
    us = sorted(1e3 * a.elapsed_time(b) for a, b in evs)
    del reps, scratch

    def q(f):
        return us[min(len(us) - 1, int(f * len(us)))]
    med = q(0.5)
    return {"launches": launches, "flush": flush, "flush_bytes": COLD_FLUSH_BYTES, "median_us": med,
            "p10_us": q(0.1), "p90_us": q(0.9), "achieved_GBps": alg / (med * 1e-6) / 1e9,
            "frac_of_hbm_peak": alg / (med * 1e-6) / 1e9 / HBM_PEAK_GBPS,
            "timing": "eager launch between HIP events, after a cache-evicting scratch " +
                      ("read" if flush == "read" else "write")}


def cold_pair(torch, w):
    """The cold protocol with both flushes: the scratch written (as the protocol states) and read
    (the same eviction, with no dirty lines left in the caches)."""
    return {f"{fl}_flush": _round(measure_cold(torch, w, flush=fl)) for fl in ("write", "read")}


def config_measure(torch, name, args, graph, cache="io"):
    """The fused step on workload `name` (every call of one step, in order), with the same-bytes
    copy ceiling. Returns (workload, entry)."""
    import workloads
    w = workloads.config(name, seed=args.seed)
    has_decode = any(st.kind == "decode" for st in w.steps)
    reseed = ((lambda r: workloads.config(name, seed=args.seed + 1000 * r))
              if has_decode else None)
    m = measure(torch, w, args.steps, args.warmup, reseed, graph, cache)
    entry = {"workload": w.name, "recipe": w.recipe, **_round(m),
             "kernels": "+".join(f"{x.kind}_kernel" for x in w.steps),
             "frac_of_hbm_peak": m["achieved_GBps"] / HBM_PEAK_GBPS}
    if cache == "io":
        c = copy_ceiling(torch, m["algorithmic_bytes"], args.steps, args.warmup)
        entry["copy_ceiling_GBps"] = c["GBps"]
        entry["kernel_over_copy"] = m["achieved_GBps"] / c["GBps"]
        if all(st.kind == "prefill" for st in w.steps):
            p = pattern_ceiling(torch, w, args.steps, args.warmup)
            entry["pattern_ceiling"] = pattern_entry(p, m["kernel_us_mean"])
    return w, entry


def free_device(torch):
    import gc
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def main():
    args = parse()
    if args.summarize_profile:
        summarize_profile(args.summarize_profile)
        return 0
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only; --gpus {args.gpus} is not supported (the step "
              "shards with no communication across heads or sequences, so a multi-GPU run would "
              "be this run per GPU)", file=sys.stderr)
        return 2
    from causal_short_convolution_amd import _binding
    if not os.path.exists(_binding.LIBRARY_PATH):
        from causal_short_convolution_amd import build
        build.build()
    import torch
    import workloads
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1

    n = args.workload
    w = workloads.config(n, seed=args.seed)
    has_decode = any(st.kind == "decode" for st in w.steps)
    reseed_main = ((lambda r: workloads.config(n, seed=args.seed + 1000 * r))
                   if has_decode else None)
    graph = not args.eager
    if args.only:
        print(f"bench.py: measuring {args.only} only", flush=True)
        if args.only == "main":
            m = measure(torch, w, args.steps, args.warmup, reseed_main, graph)
        elif args.only == "mxfp8":
            m = measure(torch, w, args.steps, args.warmup, reseed_main, graph, cache="mxfp8")
        elif args.only == "decode":
            m = measure(torch, workloads.config("decode", seed=args.seed), args.steps, args.warmup,
                        lambda r: workloads.config("decode", seed=args.seed + 1000 * r), graph)
        elif args.only == "backward":
            m = measure_backward(torch, w, args.steps, args.warmup, graph)
        elif args.only == "copy":
            m = measure(torch, w, 1, 0, reseed_main, graph)
            m = copy_ceiling(torch, m["algorithmic_bytes"], args.steps, args.warmup)
            m["achieved_GBps"] = m["GBps"]
        elif args.only == "pattern":
            m = pattern_ceiling(torch, w, args.steps, args.warmup)
            m["achieved_GBps"] = m["GBps"]
            print(json.dumps(m["forms"]), flush=True)
        elif args.only == "cold":
            m = measure_cold(torch, w, flush=args.cold_flush)
            m["kernel_us_mean"] = m["median_us"]  # (the median, for the line below)
        else:
            m = measure_verify(torch, args.steps, args.warmup, args.seed, graph)
        print(f"bench.py: {args.only}: {m['kernel_us_mean']:.2f} us per step, "
              f"{m['achieved_GBps']:.0f} GB/s", flush=True)
        if args.calibrate_copy:
            calibration_copy(torch)
        return 0

    def progress(what):
        print(f"bench.py: {what}", file=sys.stderr, flush=True)

    progress(f"{n}: fused step")
    main_m = measure(torch, w, args.steps, args.warmup, reseed_main, graph)
    cold = None
    if not args.no_cold:
        progress(f"{n}: cold launches")
        cold = cold_pair(torch, w)
        free_device(torch)
    extra = {}
    others = [] if args.no_extras else [c for c in workloads.CONFIG_NAMES if c != n]
    if args.no_decode and "decode" in others:
        others.remove("decode")
    big = ("long_prefill", "mixed")
    for name in others:
        progress(f"{name}: fused step")
        wc, entry = config_measure(torch, name, args, graph)
        free_device(torch)
        if not args.no_cold:
            progress(f"{name}: cold launches")
            entry["cold_protocol"] = cold_pair(torch, wc)
            free_device(torch)
        if name in big:
            progress(f"{name}: MXFP8 cache rows")
            _, mx = config_measure(torch, name, args, graph, cache="mxfp8")
            free_device(torch)
            entry["mxfp8_cache"] = {k: mx[k] for k in ("kernel_us_mean", "algorithmic_bytes",
                                                       "achieved_GBps", "frac_of_hbm_peak",
                                                       "tokens_per_s")}
            progress(f"{name}: backward of the prefill call")
            bm = measure_backward(torch, wc, args.steps, args.warmup, graph)
            free_device(torch)
            entry["backward"] = {**_round(bm),
                                 "frac_of_hbm_peak": bm["achieved_GBps"] / HBM_PEAK_GBPS}
        if not args.no_cpu_baseline:
            progress(f"{name}: oracle on the host")
            cb = cpu_baseline(wc, args.cpu_seconds / 3, 0)
            cb.pop("nproc")
            entry["cpu_baseline"] = cb
            if name in big:
                entry["cpu_baseline"]["backward"] = cpu_baseline_backward(wc, args.cpu_seconds / 3)
        extra[name] = entry
        del wc
    if not args.no_extras:
        progress(f"{n}: MXFP8 cache rows")
        mm = measure(torch, w, args.steps, args.warmup, reseed_main, graph, cache="mxfp8")
        extra["mxfp8_cache"] = {"workload": w.name, **_round(mm),
                                "frac_of_hbm_peak": mm["achieved_GBps"] / HBM_PEAK_GBPS,
                                "vs_io_cache_time": mm["kernel_us_mean"] /
                                main_m["kernel_us_mean"]}
        progress("spec_verify: verify + commit")
        vm = measure_verify(torch, args.steps, args.warmup, args.seed, graph)
        extra["spec_verify"] = {**_round(vm),
                                "frac_of_hbm_peak": vm["achieved_GBps"] / HBM_PEAK_GBPS}
        progress(f"{n}: backward")
        bm = measure_backward(torch, w, args.steps, args.warmup, graph)
        extra["backward"] = {**_round(bm),
                             "frac_of_hbm_peak": bm["achieved_GBps"] / HBM_PEAK_GBPS}
        free_device(torch)
    if args.calibrate_copy:
        calibration_copy(torch)
    progress(f"{n}: same-bytes copy")
    ceil = copy_ceiling(torch, main_m["algorithmic_bytes"], args.steps, args.warmup)
    pattern = None
    if all(st.kind == "prefill" for st in w.steps):
        progress(f"{n}: same-pattern copy")
        pattern = pattern_entry(pattern_ceiling(torch, w, args.steps, args.warmup),
                                main_m["kernel_us_mean"])

    traffic = traffic_dram = None
    if os.path.exists(TRAFFIC_SUMMARY) and args.workload == "varlen_prefill":
        txt = open(TRAFFIC_SUMMARY).read()
        kv = dict(line.split(":", 1) for line in txt.splitlines() if line.startswith("- ")
                  and ":" in line)
        kv = {k[2:].strip(): v.strip() for k, v in kv.items()}
        if kv.get("kernel_source_sha256") == kernel_source_sha():
            traffic = float(kv["hbm_bytes_per_launch"])
            traffic_dram = float(kv["dram_side_bytes_per_launch"])

    line = {
        "metric": METRIC,
        "value": main_m["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_m["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # the arithmetic type of the step (rows are stored as config.io and widened exactly)
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "recipe": w.recipe, "seed": args.seed,
                   "tokens_per_step": w.tokens, "launches_per_step": len(w.steps),
                   "seqs": sum(x.num_seqs for x in w.steps), "heads": w.H,
                   "head_dim": w.D, "width": w.W, "io": w.dtype, "arithmetic": "f32",
                   "block_size": w.block_size, "replicas": main_m["replicas"],
                   "input_sha256": input_digest(w), "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": main_m["achieved_GBps"], "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": main_m["achieved_GBps"] / HBM_PEAK_GBPS,
                     "traffic": traffic,
                     # the same launch's bytes from the DRAM-side request counters
                     "traffic_dram_side": traffic_dram,
                     "kernel": "+".join(f"{x.kind}_kernel" for x in w.steps),
                     "algorithmic_bytes_per_launch": main_m["algorithmic_bytes"],
                     "kernel_us_mean": main_m["kernel_us_mean"],
                     "launch": main_m["launch"]},
        "copy_ceiling": {"what": "the fastest of several plain copies of the same bytes (one-shot "
                                 "and persistent grids, 16 B per lane), same replica rotation and "
                                 "graph replay",
                         "bytes_moved": ceil["bytes_moved"], "GBps": ceil["GBps"],
                         "form": ceil["form"], "kernel_us_mean": ceil["kernel_us_mean"],
                         "frac_of_peak": ceil["GBps"] / HBM_PEAK_GBPS,
                         "kernel_over_copy": main_m["achieved_GBps"] / ceil["GBps"],
                         "forms": ceil["forms"]},
        **({"pattern_ceiling": pattern} if pattern else {}),
        **({"cold_protocol": cold} if cold else {}),
        **extra,
    }
    if not args.no_cpu_baseline:
        progress(f"{n}: oracle on the host")
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, args.cpu_seconds / 3)
        if not args.no_extras:
            line["cpu_baseline"]["extras"] = cpu_baseline_extras(w, args.cpu_seconds / 3)
    print(json.dumps(line), flush=True)
    return 0


def _round(m):
    return {k: (round(v, 4) if isinstance(v, float) else v) for k, v in m.items()}


if __name__ == "__main__":
    sys.exit(main())
