"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that the pins catch
each one. This is what makes the pins worth trusting: a dropped term, a wrong sign or index, a
transposed operand or a misplaced eps must each fail at least one of them.

Every mutation keeps all memory accesses inside the arrays the oracle is given.
"""
import os
import subprocess

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "shortconv_oracle.c")

# (name, text to find in the oracle source, replacement, which occurrence: 0 = prefill's, -1 = last)
MUTATIONS = [
    ("tap_orientation_flipped", "taps[(k * H + h) * D + d]", "taps[((W - 1 - k) * H + h) * D + d]", 0),
    ("dropped_oldest_tap", "acc += w * e;\n                    mag", "acc += (k ? w * e : 0.0);\n                    mag", 0),
    ("wrong_sign", "acc += w * e;\n                    mag", "acc -= w * e;\n                    mag", 0),
    ("eps_outside_sqrt", "sqrt(ss / (double)D + (double)eps)", "sqrt(ss / (double)D) + (double)eps", 0),
    ("sum_instead_of_mean", "sqrt(ss / (double)D + (double)eps)", "sqrt(ss + (double)eps)", 0),
    ("gamma_reversed", "* (double)gamma[d];", "* (double)gamma[D - 1 - d];", 0),
    ("state_rows_reversed", "e = read_state ? widen(state, ((idx * R + i) * H + h)",
     "e = read_state ? widen(state, ((idx * R + (R - 1 - i)) * H + h)", 0),
    ("has_init_ignored", "read_state = slot_ok && has_init[s]", "read_state = slot_ok", 0),
    ("heads_swapped", "e = widen(x, (start + i - R) * x_stride + h * D + d, dtype);",
     "e = widen(x, (start + i - R) * x_stride + ((h + 1) % H) * D + d, dtype);", 0),
    ("token_stride_ignored", "e = widen(x, (start + i - R) * x_stride",
     "e = widen(x, (start + i - R) * (H * D)", 0),
    ("new_state_first_rows", "const int64_t i = L + j;", "const int64_t i = j < L ? j + R : j;", 0),
    ("decode_new_token_first_tap", "taps[(R * H + h) * D + d]", "taps[(0 * H + h) * D + d]", 0),
    ("decode_state_not_shifted", "((idx * R + j + 1) * H + h)", "((idx * R + j) * H + h)", 0),
    ("decode_eps_dropped", "sqrt(ss / (double)D + (double)eps)", "sqrt(ss / (double)D)", -1),
    ("cond_missing_gamma", "cond[o] = fabs((double)gamma[d]) * a[d] / r;", "cond[o] = a[d] / r;", 0),
    # the backward
    ("bwd_projection_dropped", "chat * proj) / rp;", "0.0 * proj) / rp;", 0),
    ("bwd_sum_instead_of_mean", "proj /= (double)D;", "", 0),
    ("bwd_not_divided_by_r", "chat * proj) / rp;", "chat * proj);", 0),
    ("bwd_projection_without_gamma", "proj += gd * (double)gamma[d] * chat;", "proj += gd * chat;", 0),
    ("bwd_dgamma_with_gamma", "pg[d] += gd * chat;", "pg[d] += gd * chat * (double)gamma[d];", 0),
    ("bwd_input_taps_flipped",
     "if (p >= 0 && p < L) acc += (double)taps[(k * H + h) * D + d] * dc[p * D + d];",
     "if (p >= 0 && p < L) acc += (double)taps[((W - 1 - k) * H + h) * D + d] * dc[p * D + d];", 0),
    ("bwd_dtaps_rows_flipped", "pt[k * D + d] += dc[p * D + d] * e[(p + k) * D + d];",
     "pt[k * D + d] += dc[p * D + d] * e[(p + W - 1 - k) * D + d];", 0),
    ("bwd_new_state_loss_shifted", "if (gs && i >= L)", "if (gs && i > L)", 0),
    ("bwd_dstate_ignores_has_init", "= from_state ? acc : 0.0;", "= acc;", 0),
    ("bwd_dx_shifted", "dx[((start + i - R) * H + h) * D + d] = acc;",
     "dx[((start + (i > R ? i - R - 1 : i - R)) * H + h) * D + d] = acc;", 0),
    ("bwd_dtaps_one_sequence", "acc += part_taps[((s * H + h) * W + k) * D + d];",
     "acc = part_taps[((s * H + h) * W + k) * D + d];", 0),
    ("bwd_eps_dropped", "sqrt(sumsq / (double)D + (double)eps)", "sqrt(sumsq / (double)D)", 0),
]


def _mutate(text, find, repl, which):
    hits = []
    i = text.find(find)
    while i >= 0:
        hits.append(i)
        i = text.find(find, i + 1)
    assert hits, f"mutation anchor not found: {find!r}"
    at = hits[which]
    return text[:at] + repl + text[at + len(find):]


@pytest.mark.parametrize("name,find,repl,which", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_mutation(tmp_path, name, find, repl, which):
    src = _mutate(open(SRC).read(), find, repl, which)
    c = tmp_path / "mut.c"
    c.write_text(src)
    lib = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    "-o", str(lib), str(c), "-lm"], check=True)
    caught = []
    with oracle.library(str(lib)):
        for pin in oracle_pins.ALL_PINS:
            try:
                pin()
            except AssertionError:
                caught.append(pin.__name__)
                break
    assert caught, f"no pin caught the planted mistake {name}"
