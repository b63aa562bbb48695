"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check
that the pins catch every one of them.  The real oracle is untouched: each
mutant is the C source with one textual edit, built to a temporary library.
"""
import os
import subprocess

import pytest

import oracle
from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "qmoe_oracle.c")

# (name, original text, planted mistake)
MUTANTS = [
    ("offset_minus_7", "return u - 8;", "return u - 7;"),
    ("nibble_order_swapped", "(i % 2 == 0) ? (byte & 15) : (byte >> 4)",
     "(i % 2 == 0) ? (byte >> 4) : (byte & 15)"),
    ("scale_row_stride_missing_ng", "scales[o * ng + i / gs]",
     "scales[o + i / gs]"),
    ("scale_index_modulo", "scales[o * ng + i / gs]",
     "scales[o * ng + i % ng]"),
    ("groups_round_down", "return (cols + gs - 1) / gs;",
     "return cols / gs + (cols < gs);"),
    ("row_bytes_round_down", "return (cols + 1) / 2;",
     "return cols / 2 + (cols < 2);"),
    ("pad_nibble_zero", "int lo_u = 8, hi_u = 8;", "int lo_u = 8, hi_u = 0;"),
    ("silu_sign", "return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    ("silu_on_up_instead_of_gate", "h[f] = orc_silu(g[f]) * u[f];",
     "h[f] = orc_silu(u[f]) * g[f];"),
    ("pair_wrong_scales_for_up", "orc_matvec(pu, su, rows, cols, gs, x, batch, yu);",
     "orc_matvec(pu, sg, rows, cols, gs, x, batch, yu);"),
    ("matvec_ignores_batch", "x[b * cols + i];", "x[i];"),
    ("layer_drops_routing_weight", "ot[j] += wt * y[j];", "ot[j] += y[j];"),
    ("layer_keeps_last_slot_only", "ot[j] += wt * y[j];", "ot[j] = wt * y[j];"),
    ("worklist_inv_is_expert", "inv[p] = fill[e];", "inv[p] = e;"),
    ("worklist_invalid_not_counted", "if (e < 0 || e >= experts) bad++;\n        else counts[e]++;",
     "if (e < 0 || e >= experts) {}\n        else counts[e]++;"),
    ("pack_bad_not_counted", "if (v0 < -8 || v0 > 7) bad++;", "(void)0;"),
    ("route_ties_to_highest_id", "if (best < 0 || key > best_key) {",
     "if (best < 0 || key >= best_key) {"),
    ("route_taken_flag_not_set", "taken[best] = 1;", "(void)taken;"),
    ("route_softmax_over_first_experts", "ex[s] = exp((double)l[ids[t * k + s]] - top);",
     "ex[s] = exp((double)l[s] - top);"),
    ("route_nan_not_demoted", "double key = isnan(l[e]) ? -INFINITY : (double)l[e];",
     "double key = (double)l[e];"),
    ("route_weights_not_normalised", "w[t * k + s] = (float)(ex[s] / sum);",
     "w[t * k + s] = (float)ex[s];"),
    ("import_xor_low_nibble_only", "packed[b] = (uint8_t)(twos[b] ^ 0x88);",
     "packed[b] = (uint8_t)(twos[b] ^ 0x08);"),
    ("detect_group_largest_first", "for (int c = 0; c < 8; c++)", "for (int c = 7; c >= 0; c--)"),
    ("dsilu_missing_factor", "return sg * (1.0 + z * (1.0 - sg));", "return sg * (1.0 + z * sg);"),
    ("matvec_abs_signed", "acc += fabs(orc_weight(packed, scales, cols, gs, o, i) *",
     "acc += (orc_weight(packed, scales, cols, gs, o, i) *"),
    ("layer_mag_h_once", "c[f] = 2.0 * fabs(h) +", "c[f] = fabs(h) +"),
    ("layer_mag_no_gate_term", "fabs(orc_dsilu(g[f]) * u[f]) * ag[f] +", "0.0 * ag[f] +"),
    ("layer_mag_up_uses_gate", "fabs(orc_silu(g[f])) * au[f];", "fabs(orc_silu(g[f])) * ag[f];"),
    ("layer_mag_signed_weight", "double wt = fabs((double)w[t * k + s]);",
     "double wt = (double)w[t * k + s];"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    text = open(SRC).read()
    assert text.count(old) >= 1, f"mutation anchor missing: {name}"
    bad_src = tmp_path / "mutant.c"
    bad_src.write_text(text.replace(old, new, 1))
    lib_path = str(tmp_path / "libmutant.so")
    subprocess.run(["gcc", "-O1", "-fPIC", "-shared", "-std=c99",
                    str(bad_src), "-o", lib_path, "-lm"], check=True)
    orc = oracle.Oracle(oracle.load(lib_path))
    caught = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"
