"""The torch binding rejects malformed tensor arguments before the library is loaded or called.

The C ABI receives raw pointers and sizes; a tensor of the wrong element type, shape or layout
would be read or written past its end on the device. Every call of the binding therefore checks
each tensor first. These tests run on host tensors: a well-formed argument set gets through every
check and stops only at "tensors must be on a GPU"; each malformed variant stops at the argument
it breaks. The library loader is replaced by one that fails the test, so a check that let a bad
argument through to the library would show.
"""
import pytest
import torch

from causal_short_convolution_amd import _binding

T, N, H, D, W, S, SLOTS, M = 40, 3, 2, 64, 4, 5, 64, 4
BF, F32, I32, I64, U8 = torch.bfloat16, torch.float32, torch.int32, torch.int64, torch.uint8


@pytest.fixture(autouse=True)
def no_library(monkeypatch):
    def refuse(*_a, **_k):
        raise AssertionError("the binding reached the library with arguments it should reject")
    monkeypatch.setattr(_binding, "load_library", refuse)


def z(shape, dtype):
    return torch.zeros(shape, dtype=dtype)


def prefill_args():
    return dict(k=z((T, H, D), BF), v=z((T, H, D), BF),
                cu_seqlens=torch.tensor([0, 10, 25, T], dtype=I32),
                k_taps=z((W, H, D), F32), v_taps=z((W, H, D), F32),
                k_gamma=z((D,), F32), v_gamma=z((D,), F32), eps=1e-6,
                k_state=z((S, W - 1, H, D), BF), v_state=z((S, W - 1, H, D), BF),
                state_idx=z((N,), I32), has_initial_state=z((N,), U8),
                slot_mapping=z((T,), I64), k_cache=z((SLOTS, H, D), BF),
                v_cache=z((SLOTS, H, D), BF))


def decode_args():
    return dict(k_new=z((N, H, D), BF), v_new=z((N, H, D), BF),
                k_taps=z((W, H, D), F32), v_taps=z((W, H, D), F32),
                k_gamma=z((D,), F32), v_gamma=z((D,), F32), eps=1e-6,
                k_state=z((S, W - 1, H, D), BF), v_state=z((S, W - 1, H, D), BF),
                state_idx=z((N,), I32), slot_mapping=z((N,), I64),
                k_cache=z((SLOTS, H, D), BF), v_cache=z((SLOTS, H, D), BF))


def mx_prefill_args():
    a = prefill_args()
    del a["k_cache"], a["v_cache"]
    a.update(k_codes=z((SLOTS, H, D), U8), v_codes=z((SLOTS, H, D), U8),
             k_scales=z((SLOTS, H, D // 32), U8), v_scales=z((SLOTS, H, D // 32), U8))
    return a


def mx_decode_args():
    a = decode_args()
    del a["k_cache"], a["v_cache"]
    a.update(k_codes=z((SLOTS, H, D), U8), v_codes=z((SLOTS, H, D), U8),
             k_scales=z((SLOTS, H, D // 32), U8), v_scales=z((SLOTS, H, D // 32), U8))
    return a


def verify_args():
    a = prefill_args()
    out = {}
    for key, val in a.items():
        if key == "has_initial_state":
            continue
        if key == "slot_mapping":  # the snapshots come before the slots in the signature
            out.update(k_snap=z((N, M, W - 1, H, D), BF), v_snap=z((N, M, W - 1, H, D), BF))
        out[key] = val
    return out


def commit_args():
    return dict(k_snap=z((N, M, W - 1, H, D), BF), v_snap=z((N, M, W - 1, H, D), BF),
                cu_seqlens=torch.tensor([0, 10, 25, T], dtype=I32), total_tokens=T,
                accepted=z((N,), I32), k_state=z((S, W - 1, H, D), BF),
                v_state=z((S, W - 1, H, D), BF), state_idx=z((N,), I32),
                width=W, num_heads=H, head_dim=D)


def backward_args():
    a = prefill_args()
    del a["slot_mapping"], a["k_cache"], a["v_cache"]
    a.update(dy_k=z((T, H, D), BF), dy_v=z((T, H, D), BF), dk=z((T, H, D), BF),
             dv=z((T, H, D), BF), dk_taps=z((W, H, D), F32), dv_taps=z((W, H, D), F32),
             dk_gamma=z((D,), F32), dv_gamma=z((D,), F32),
             dstate_out=(z((N, W - 1, H, D), BF), z((N, W - 1, H, D), BF)),
             dstate_in=(z((N, W - 1, H, D), BF), z((N, W - 1, H, D), BF)),
             workspace=z((1024,), U8))
    return a


def quantize_args():
    return dict(x=z((T, H, D), BF), codes=z((T, H, D), U8), scales=z((T, H, D // 32), U8))


ENTRY = {
    "prefill": (_binding.shortconv_kv_prefill, prefill_args),
    "decode": (_binding.shortconv_kv_decode, decode_args),
    "prefill_mxfp8": (_binding.shortconv_kv_prefill_mxfp8, mx_prefill_args),
    "decode_mxfp8": (_binding.shortconv_kv_decode_mxfp8, mx_decode_args),
    "verify": (_binding.shortconv_kv_verify, verify_args),
    "commit": (_binding.shortconv_state_commit, commit_args),
    "backward": (_binding.shortconv_kv_backward, backward_args),
    "quantize": (_binding.shortconv_mxfp8_quantize, quantize_args),
}


def call(entry, args):
    fn, _ = ENTRY[entry]
    kw = {k: v for k, v in args.items()
          if k in ("dstate_out", "dstate_in", "workspace", "width", "num_heads", "head_dim")}
    pos = [v for k, v in args.items() if k not in kw]
    return fn(*pos, **kw)


@pytest.mark.parametrize("entry", sorted(ENTRY))
def test_well_formed_arguments_reach_the_device_check(entry):
    with pytest.raises(ValueError, match="must be on a GPU"):
        call(entry, ENTRY[entry][1]())


def _noncontig(t):
    """Same shape and dtype, every other element of a larger buffer (not contiguous)."""
    return torch.zeros(t.shape[:-1] + (2 * t.shape[-1],), dtype=t.dtype)[..., ::2]


# (entry, argument, replacement builder, message fragment)
BAD = [
    # index arrays: element type and length
    ("prefill", "cu_seqlens", lambda a: a["cu_seqlens"].to(I64), "cu_seqlens must be torch.int32"),
    ("prefill", "state_idx", lambda a: a["state_idx"].to(I64), "state_idx must be torch.int32"),
    ("prefill", "state_idx", lambda a: z((N + 1,), I32), "state_idx must have shape"),
    ("prefill", "slot_mapping", lambda a: a["slot_mapping"].to(I32),
     "slot_mapping must be torch.int64"),
    ("prefill", "slot_mapping", lambda a: z((T - 1,), I64), "slot_mapping must have shape"),
    ("prefill", "has_initial_state", lambda a: z((N,), I32), "has_initial_state must be"),
    ("prefill", "has_initial_state", lambda a: z((N + 2,), U8), "has_initial_state must have"),
    ("decode", "state_idx", lambda a: a["state_idx"].to(I64), "state_idx must be torch.int32"),
    ("decode", "slot_mapping", lambda a: a["slot_mapping"].to(I32),
     "slot_mapping must be torch.int64"),
    ("commit", "accepted", lambda a: a["accepted"].to(I64), "accepted must be torch.int32"),
    ("commit", "cu_seqlens", lambda a: a["cu_seqlens"].to(I64), "cu_seqlens must be torch.int32"),
    # parameters
    ("prefill", "k_taps", lambda a: a["k_taps"].to(BF), "k_taps must be torch.float32"),
    ("prefill", "v_taps", lambda a: z((W - 1, H, D), F32), "v_taps must have shape"),
    ("prefill", "k_taps", lambda a: z((W, H + 1, D), F32), "k_taps must have shape"),
    ("prefill", "k_taps", lambda a: _noncontig(a["k_taps"]), "k_taps must be contiguous"),
    ("prefill", "k_gamma", lambda a: z((D // 2,), F32), "k_gamma must have shape"),
    ("prefill", "v_gamma", lambda a: a["v_gamma"].to(torch.float64),
     "v_gamma must be torch.float32"),
    # rows
    ("prefill", "v", lambda a: a["v"].to(F32), "v must be torch.bfloat16"),
    ("prefill", "v", lambda a: z((T, H, D // 2), BF), "v must have shape"),
    ("prefill", "v", lambda a: z((T - 1, H, D), BF), "same number of tokens"),
    ("prefill", "k", lambda a: z((T, D, H), BF).transpose(1, 2), "contiguous heads/head_dim"),
    ("prefill", "k", lambda a: z((T, H, D), torch.float16), "k must be torch.float32 or"),
    # caches
    ("prefill", "k_cache", lambda a: z((SLOTS, H, D), F32), "k_cache must be torch.bfloat16"),
    ("prefill", "v_cache", lambda a: z((SLOTS - 1, H, D), BF), "v_cache must have shape"),
    ("prefill", "k_cache", lambda a: z((SLOTS, H, 2 * D), BF), "k_cache must have shape"),
    ("prefill", "k_cache", lambda a: _noncontig(a["k_cache"]), "k_cache must be contiguous"),
    ("decode", "v_cache", lambda a: z((SLOTS, H, D), F32), "v_cache must be torch.bfloat16"),
    ("prefill_mxfp8", "k_codes", lambda a: z((SLOTS, H, D), BF), "k_codes must be torch.uint8"),
    ("prefill_mxfp8", "v_scales", lambda a: z((SLOTS, H, D), U8), "v_scales must have shape"),
    ("decode_mxfp8", "k_scales", lambda a: z((SLOTS, H, D // 32), I32),
     "k_scales must be torch.uint8"),
    # state pools
    ("prefill", "k_state", lambda a: z((S, W - 1, H, D), F32), "k_state must be torch.bfloat16"),
    ("prefill", "v_state", lambda a: z((S, W, H, D), BF), "v_state must have shape"),
    ("prefill", "v_state", lambda a: z((S + 1, W - 1, H, D), BF), "v_state must have shape"),
    ("prefill", "v_state", lambda a: None, "both be given or both be None"),
    ("decode", "k_state", lambda a: _noncontig(a["k_state"]), "k_state must be contiguous"),
    ("commit", "k_state", lambda a: z((S, W - 1, H, D), F32), "k_state must be torch.bfloat16"),
    # speculative snapshots
    ("verify", "k_snap", lambda a: z((N, M, W, H, D), BF), "k_snap must have shape"),
    ("verify", "v_snap", lambda a: z((N, M + 1, W - 1, H, D), BF), "v_snap must have shape"),
    ("verify", "k_snap", lambda a: z((N, M, W - 1, H, D), F32), "k_snap must be torch.bfloat16"),
    ("commit", "v_snap", lambda a: z((N + 1, M, W - 1, H, D), BF), "v_snap must have shape"),
    # backward
    ("backward", "dy_k", lambda a: z((T, H, D), F32), "dy_k must be torch.bfloat16"),
    ("backward", "dy_v", lambda a: _noncontig(a["dy_v"]), "dy_v must be contiguous"),
    ("backward", "dk", lambda a: z((T, H, D), F32), "dk must be torch.bfloat16"),
    ("backward", "dv", lambda a: z((T + 1, H, D), BF), "dv must have shape"),
    ("backward", "dk_taps", lambda a: z((W, H, D), BF), "dk_taps must be torch.float32"),
    ("backward", "dv_gamma", lambda a: z((D + 1,), F32), "dv_gamma must have shape"),
    ("backward", "dstate_out", lambda a: (a["dstate_out"][0], None),
     "both be given or both be None"),
    ("backward", "dstate_in", lambda a: (z((N, W - 1, H, D), F32),) * 2,
     "dstate_in\\[0\\] must be torch.bfloat16"),
    ("backward", "workspace", lambda a: z((1024,), F32), "workspace must be torch.uint8"),
    # quantizer
    ("quantize", "codes", lambda a: z((T - 1, H, D), U8), "codes must have shape"),
    ("quantize", "scales", lambda a: z((T, H, D // 32), BF), "scales must be torch.uint8"),
]


@pytest.mark.parametrize("entry,arg,make,msg", BAD, ids=[f"{e}-{a}-{i}" for i, (e, a, _, _)
                                                          in enumerate(BAD)])
def test_malformed_argument_is_rejected_before_the_library(entry, arg, make, msg):
    args = ENTRY[entry][1]()
    args[arg] = make(args)
    with pytest.raises(ValueError, match=msg):
        call(entry, args)


def test_tensors_on_different_devices_are_rejected():
    args = prefill_args()
    args["slot_mapping"] = args["slot_mapping"].to("meta")
    with pytest.raises(ValueError, match="slot_mapping is on meta"):
        call("prefill", args)
