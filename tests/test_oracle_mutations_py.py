"""Plant plausible mistakes in the oracle's Python parts -- the speculative-verification snapshots
and commit, and the MXFP8 encoding -- and check that the pins catch each one, as
test_oracle_mutations.py does for the C oracle.

Each mutation is a text substitution in one oracle function's source; the edited function is
compiled against the oracle module's globals and installed in the module for the duration of the
test, so other oracle functions that call it see the mistake too. A pin catches a mutation when
it fails in any way (a wrong index may raise rather than assert).
"""
import inspect
import textwrap

import pytest

import oracle
import oracle_pins

PINS = [oracle_pins.pin_verify_snapshots_and_commit, oracle_pins.pin_mxfp8_codes,
        oracle_pins.pin_mxfp8_blocks]

# (name, oracle function, [(text to find, replacement), ...])
MUTATIONS = [
    ("e4m3_ties_away_from_zero", "e4m3_encode", [("m = np.rint(", "m = np.floor(0.5 + ")]),
    ("e4m3_subnormal_ties_away", "e4m3_encode",
     [("code_s = np.rint(a * 2.0 ** 9)", "code_s = np.floor(a * 2.0 ** 9 + 0.5)")]),
    ("e4m3_truncates", "e4m3_encode", [("m = np.rint(", "m = np.floor(")]),
    ("e4m3_saturates_to_nan", "e4m3_encode",
     [("code = np.where(a > E4M3_MAX, 0x7E, code)", "code = np.where(a > E4M3_MAX, 0x7F, code)"),
      ("code = np.where(code > 0x7E, 0x7E, code)", "code = np.where(code > 0x7F, 0x7F, code)")]),
    ("e4m3_no_saturation", "e4m3_encode",
     [("code = np.where(a > E4M3_MAX, 0x7E, code)", ""),
      ("code = np.where(code > 0x7E, 0x7E, code)", "")]),
    ("e4m3_exponent_bias_8", "e4m3_encode", [("((e + 7) << 3)", "((e + 8) << 3)")]),
    ("e4m3_normal_threshold", "e4m3_encode", [("normal = a >= 2.0 ** -6", "normal = a >= 2.0 ** -7")]),
    ("e4m3_decode_subnormal_scale", "e4m3_decode", [("m * 2.0 ** -9", "m * 2.0 ** -10")]),
    ("e4m3_decode_bias", "e4m3_decode", [("2.0 ** (e - 7)", "2.0 ** (e - 8)")]),
    ("mx_emax_off_by_one", "mx_scale_exponent", [("ex - 1 - 8, -127", "ex - 1 - 7, -127")]),
    ("mx_ceil_log2", "mx_scale_exponent", [("ex - 1 - 8, -127", "ex - 8, -127")]),
    ("mx_zero_block_exponent", "mx_scale_exponent", [("ex - 1 - 8, -127)", "ex - 1 - 8, 0)")]),
    ("mx_no_clamp", "mx_scale_exponent", [("np.clip(e, -127, 127)", "e")]),
    ("mx_interleaved_blocks", "mxfp8_quantize",
     [("blocks = y.reshape(*y.shape[:-1], D // MX_BLOCK, MX_BLOCK)",
       "blocks = y.reshape(*y.shape[:-1], MX_BLOCK, D // MX_BLOCK).swapaxes(-1, -2)")]),
    ("mx_scale_applied_inverted", "mxfp8_quantize",
     [("scaled = blocks / np.ldexp(1.0, e)[..., None]",
       "scaled = blocks * np.ldexp(1.0, e)[..., None]")]),
    ("mx_scale_byte_bias", "mxfp8_quantize", [("(e + 127).astype", "(e + 128).astype")]),
    ("snapshot_off_by_one", "verify_snapshots",
     [("snaps[s, i] = e[i + 1:i + 1 + R]", "snaps[s, i] = e[i:i + R]")]),
    ("snapshot_ignores_state", "verify_snapshots",
     [("z = state[idx]", "z = np.zeros((R, H, D), x.dtype)")]),
    ("snapshot_capacity_ignored", "verify_snapshots",
     [("range(min(int(cu[s + 1] - cu[s]), max_tokens))", "range(int(cu[s + 1] - cu[s]))")]),
    ("commit_one_past", "commit_state",
     [("out[idx] = snapshots[s, m - 1]", "out[idx] = snapshots[s, min(m, max_tokens - 1)]")]),
    ("commit_ignores_accepted", "commit_state",
     [("m = min(int(accepted[s]), int(cu[s + 1] - cu[s]), max_tokens)",
       "m = min(int(cu[s + 1] - cu[s]), max_tokens)")]),
    ("commit_zero_accepted", "commit_state", [("if m >= 1 and", "if m >= 0 and")]),
    ("verify_from_zero_state", "fused_verify",
     [("ones = np.ones(N, np.uint8)", "ones = np.zeros(N, np.uint8)")]),
]


def _mutant(name, edits):
    src = textwrap.dedent(inspect.getsource(getattr(oracle, name)))
    for find, repl in edits:
        assert src.count(find) == 1, f"mutation anchor not unique in {name}: {find!r}"
        src = src.replace(find, repl)
    ns = {}
    exec(compile(src, f"<mutated {name}>", "exec"), oracle.__dict__, ns)
    return ns[name]


@pytest.mark.filterwarnings("ignore::RuntimeWarning")  # some mutants overflow before a pin fails
@pytest.mark.parametrize("label,fn,edits", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_mutation(monkeypatch, label, fn, edits):
    monkeypatch.setattr(oracle, fn, _mutant(fn, edits))
    caught = []
    for pin in PINS:
        try:
            pin()
        except Exception:  # noqa: BLE001 -- any failure of a pin counts as catching it
            caught.append(pin.__name__)
            break
    assert caught, f"no pin caught the planted mistake {label}"


def test_unmutated_pins_pass():
    for pin in PINS:
        pin()
