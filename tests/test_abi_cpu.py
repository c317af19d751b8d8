"""The C-ABI library on the host (no GPU): it loads, exports every symbol include/shortconv.h
declares, and rejects bad arguments before anything reaches the HIP runtime.

Pointer arguments here are fake integers; every call either fails validation or returns SC_OK
without launching, so none is ever dereferenced.
"""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "shortconv.h")


@pytest.fixture(scope="module")
def lib():
    from causal_short_convolution_amd import _binding
    if not os.path.exists(_binding.LIBRARY_PATH):
        from causal_short_convolution_amd import build
        build.build()
    return _binding.load_library()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(shortconv_\w+)\s*\(", text, re.M)))


def test_header_declares_the_boundary():
    assert declared_functions() == ["shortconv_abi_version", "shortconv_kv_backward",
                                    "shortconv_kv_backward_noalloc",
                                    "shortconv_kv_backward_workspace_size", "shortconv_kv_decode",
                                    "shortconv_kv_decode_mxfp8", "shortconv_kv_prefill",
                                    "shortconv_kv_prefill_mxfp8", "shortconv_kv_verify",
                                    "shortconv_last_error", "shortconv_mxfp8_quantize",
                                    "shortconv_state_commit"]


def test_library_exports_every_declared_symbol(lib):
    from causal_short_convolution_amd import _binding
    out = subprocess.run(["nm", "-D", "--defined-only", _binding.LIBRARY_PATH], check=True,
                         capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)
    # nothing else with code is exported: the boundary is the header
    assert exported == set(declared_functions())


def test_abi_version(lib):
    text = open(HEADER).read()
    v = int(re.search(r"#define SHORTCONV_ABI_VERSION (\d+)", text).group(1))
    assert lib.shortconv_abi_version() == v


FAKE = 0x100000  # 16-byte aligned, never dereferenced


def prefill_args(**over):
    a = dict(k=FAKE, v=FAKE, ks=1024, vs=1024, cu=FAKE, n=2, T=10, kt=FAKE, vt=FAKE, kg=FAKE,
             vg=FAKE, eps=1e-6, kst=FAKE, vst=FAKE, S=2, sidx=FAKE, hinit=FAKE, slot=FAKE,
             kc=FAKE, vc=FAKE, slots=100, H=8, D=128, W=4, dtype=1, stream=None)
    a.update(over)
    return [a[k] for k in ("k", "v", "ks", "vs", "cu", "n", "T", "kt", "vt", "kg", "vg", "eps",
                           "kst", "vst", "S", "sidx", "hinit", "slot", "kc", "vc", "slots", "H",
                           "D", "W", "dtype", "stream")]


def decode_args(**over):
    a = dict(k=FAKE, v=FAKE, ks=1024, vs=1024, B=3, kt=FAKE, vt=FAKE, kg=FAKE, vg=FAKE, eps=1e-6,
             kst=FAKE, vst=FAKE, S=3, sidx=FAKE, slot=FAKE, kc=FAKE, vc=FAKE, slots=100, H=8,
             D=128, W=4, dtype=1, stream=None)
    a.update(over)
    return [a[k] for k in ("k", "v", "ks", "vs", "B", "kt", "vt", "kg", "vg", "eps", "kst", "vst",
                           "S", "sidx", "slot", "kc", "vc", "slots", "H", "D", "W", "dtype",
                           "stream")]


INVALID, UNSUPPORTED = -1, -2

PREFILL_CASES = [
    (dict(dtype=7), UNSUPPORTED, "dtype"),
    (dict(D=96), UNSUPPORTED, "head_dim"),
    (dict(W=0), UNSUPPORTED, "width"),
    (dict(W=9), UNSUPPORTED, "width"),
    (dict(H=0), INVALID, "num_heads"),
    (dict(k=None), INVALID, "null K"),
    (dict(vt=None), INVALID, "taps"),
    (dict(slot=None), INVALID, "slot_mapping"),
    (dict(kc=None), INVALID, "cache"),
    (dict(kst=None), INVALID, "conv state"),
    (dict(n=-1), INVALID, "num_seqs"),
    (dict(T=-5), INVALID, "total_tokens"),
    (dict(T=1 << 31), INVALID, "total_tokens"),
    (dict(cu=None), INVALID, "cu_seqlens"),
    (dict(ks=1000), INVALID, "stride"),
    (dict(vs=1028, dtype=1), INVALID, "16 bytes"),
    (dict(k=FAKE + 8), INVALID, "aligned"),
    (dict(eps=-1.0), INVALID, "eps"),
    (dict(eps=float("nan")), INVALID, "eps"),
    (dict(slots=-1), INVALID, "num_slots"),
    (dict(S=-1), INVALID, "num_state_slots"),
]


@pytest.mark.parametrize("over,code,msg", PREFILL_CASES, ids=[c[2] + str(i) for i, c in
                                                               enumerate(PREFILL_CASES)])
def test_prefill_rejects(lib, over, code, msg):
    rc = lib.shortconv_kv_prefill(*prefill_args(**over))
    assert rc == code
    err = lib.shortconv_last_error().decode()
    assert err.startswith("shortconv_kv_prefill") and msg in err, err


DECODE_CASES = [
    (dict(dtype=2), UNSUPPORTED, "dtype"),
    (dict(D=32), UNSUPPORTED, "head_dim"),
    (dict(B=-1), INVALID, "batch"),
    (dict(kc=None), INVALID, "cache"),
    (dict(vst=None), INVALID, "conv state"),
    (dict(ks=64, D=128, H=1, dtype=0), INVALID, "stride"),
]


@pytest.mark.parametrize("over,code,msg", DECODE_CASES, ids=[c[2] + str(i) for i, c in
                                                             enumerate(DECODE_CASES)])
def test_decode_rejects(lib, over, code, msg):
    rc = lib.shortconv_kv_decode(*decode_args(**over))
    assert rc == code
    assert msg in lib.shortconv_last_error().decode()


def test_empty_work_returns_ok_without_launch(lib):
    # no sequences; no decodes; width 1 with no tokens: nothing to launch, no HIP call made
    assert lib.shortconv_kv_prefill(*prefill_args(n=0, T=0, k=None, v=None, slot=None,
                                                  cu=None)) == 0
    assert lib.shortconv_kv_decode(*decode_args(B=0, k=None, v=None, slot=None)) == 0
    assert lib.shortconv_kv_prefill(*prefill_args(W=1, T=0, kst=None, vst=None)) == 0
    assert lib.shortconv_last_error().decode() == ""


def test_state_may_be_null_for_width_one_or_empty_pool(lib):
    # validation only: these fail later on something else (unsupported head_dim) rather than on
    # the missing state, proving the state check accepts them
    rc = lib.shortconv_kv_prefill(*prefill_args(W=1, kst=None, vst=None, D=48))
    assert rc == UNSUPPORTED
    rc = lib.shortconv_kv_prefill(*prefill_args(S=0, kst=None, vst=None, eps=-1.0))
    assert rc == INVALID and "eps" in lib.shortconv_last_error().decode()


def test_python_binding_fails_loudly_without_library(tmp_path):
    from causal_short_convolution_amd import _binding
    saved = _binding._lib
    _binding._lib = None
    try:
        with pytest.raises(ImportError, match="not built"):
            _binding.load_library(str(tmp_path / "missing.so"))
    finally:
        _binding._lib = saved


def backward_args(**over):
    a = dict(k=FAKE, v=FAKE, ks=1024, vs=1024, cu=FAKE, n=2, T=10, kt=FAKE, vt=FAKE, kg=FAKE,
             vg=FAKE, eps=1e-6, kst=FAKE, vst=FAKE, S=2, sidx=FAKE, hinit=FAKE, dyk=FAKE,
             dyv=FAKE, gsk=None, gsv=None, dk=FAKE, dv=FAKE, dkt=FAKE, dvt=FAKE, dkg=FAKE,
             dvg=FAKE, dsk=None, dsv=None, ws=FAKE, wsb=1 << 40, H=8, D=128, W=4, dtype=1,
             stream=None)
    a.update(over)
    return [a[k] for k in ("k", "v", "ks", "vs", "cu", "n", "T", "kt", "vt", "kg", "vg", "eps",
                           "kst", "vst", "S", "sidx", "hinit", "dyk", "dyv", "gsk", "gsv", "dk",
                           "dv", "dkt", "dvt", "dkg", "dvg", "dsk", "dsv", "ws", "wsb", "H", "D",
                           "W", "dtype", "stream")]


BACKWARD_CASES = [
    (dict(dtype=3), UNSUPPORTED, "dtype"),
    (dict(D=32), UNSUPPORTED, "head_dim"),
    (dict(W=9), UNSUPPORTED, "width"),
    (dict(H=0), INVALID, "num_heads"),
    (dict(n=-1), INVALID, "num_seqs"),
    (dict(T=1 << 31), INVALID, "total_tokens"),
    (dict(kt=None), INVALID, "taps or gamma"),
    (dict(dvg=None), INVALID, "gradient"),
    (dict(dyk=None), INVALID, "output gradient"),
    (dict(dv=None), INVALID, "input gradient"),
    (dict(cu=None), INVALID, "cu_seqlens"),
    (dict(vst=None), INVALID, "conv state"),
    (dict(gsk=FAKE), INVALID, "new-state gradient"),
    (dict(dsv=FAKE), INVALID, "initial-state gradient"),
    (dict(eps=float("inf")), INVALID, "eps"),
    (dict(ks=100), INVALID, "stride"),
    (dict(dk=FAKE + 4), INVALID, "aligned"),
    (dict(ws=None), INVALID, "workspace"),
    (dict(wsb=16), INVALID, "workspace"),
]


@pytest.mark.parametrize("over,code,msg", BACKWARD_CASES, ids=[c[2] + str(i) for i, c in
                                                               enumerate(BACKWARD_CASES)])
def test_backward_rejects(lib, over, code, msg):
    from causal_short_convolution_amd import _binding
    _binding.load_library()
    rc = lib.shortconv_kv_backward(*backward_args(**over))
    assert rc == code
    err = lib.shortconv_last_error().decode()
    assert err.startswith("shortconv_kv_backward") and msg in err, err


def test_backward_workspace_size(lib):
    from causal_short_convolution_amd import _binding
    _binding.load_library()  # sets the ctypes signatures
    size = lib.shortconv_kv_backward_workspace_size
    # bf16, H=8, D=128, W=4: 256 lanes per tensor -> 8 slices of 64, each holding one tensor, so
    # tiles of 4 waves x 12 tokens: 17060 // 48 + 8 = 363 tiles; 363 * 8 slices // 1024 = 2
    # tiles per group, 182 groups; an fp32 partial of (W + 1) * 64 lanes * 4 channels per slice
    # and group, then fp64 sums of chunks of 64 groups (3 chunks)
    assert size(17060, 8, 8, 128, 4, 1) == 182 * 8 * 5 * 256 * 4 + 3 * 8 * 5 * 256 * 8
    # the long prefill (W=8 over one-tensor slices -> 16-token spans): 131072 // 64 + 1 = 2049
    # tiles, 4 per group (64 tokens per lane), 513 groups, 9 chunks
    assert size(131072, 1, 8, 128, 8, 1) == 513 * 8 * 9 * 256 * 4 + 9 * 8 * 9 * 256 * 8
    assert size(0, 0, 8, 128, 4, 1) == 0
    assert size(10, 2, 8, 96, 4, 1) == 2 ** 64 - 1  # unsupported head_dim -> SIZE_MAX
    assert "head_dim" in lib.shortconv_last_error().decode()


def noalloc_args(**over):
    """shortconv_kv_backward_noalloc's arguments: the backward's without the workspace pair."""
    a = backward_args(**over)
    return a[:29] + a[31:]


@pytest.mark.parametrize("over,code,msg", [
    (dict(W=9), UNSUPPORTED, "width"),
    (dict(n=-1), INVALID, "num_seqs"),
    # 131072 tokens at width 8 need ~62 MB of partials: beyond the 16 MiB static scratch
    (dict(T=131072, n=1, W=8), UNSUPPORTED, "static scratch"),
], ids=["width", "num_seqs", "too_large"])
def test_noalloc_backward_rejects_before_any_device_call(lib, over, code, msg):
    from causal_short_convolution_amd import _binding
    _binding.load_library()
    rc = lib.shortconv_kv_backward_noalloc(*noalloc_args(**over))
    assert rc == code
    err = lib.shortconv_last_error().decode()
    assert err.startswith("shortconv_kv_backward_noalloc") and msg in err, err


def test_mxfp8_entry_points_reject_null_scales(lib):
    from causal_short_convolution_amd import _binding
    _binding.load_library()
    a = prefill_args()
    # shortconv_kv_prefill_mxfp8: the prefill's arguments with the scale pair after the codes
    mx = a[:20] + [FAKE, None] + a[20:]
    assert lib.shortconv_kv_prefill_mxfp8(*mx) == INVALID
    assert "scale" in lib.shortconv_last_error().decode()
    d = decode_args()
    mxd = d[:17] + [None, FAKE] + d[17:]
    assert lib.shortconv_kv_decode_mxfp8(*mxd) == INVALID
    assert "scale" in lib.shortconv_last_error().decode()
