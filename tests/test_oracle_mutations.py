"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that
the pins catch each one.  The copy is compiled to a temporary library and
swapped in for the duration of one case."""
import ctypes
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "txl_oracle.c")

# (name, text in txl_oracle.c, replacement).  Every edit keeps all reads in bounds.
MUTATIONS = [
    ("dropped_u", "ac += (qe + u[e]) * k[(size_t)j * dh + e];", "ac += (qe) * k[(size_t)j * dh + e];"),
    ("dropped_vbias", "bd += (qe + vb[e]) * r[(size_t)c * dh + e];", "bd += (qe) * r[(size_t)c * dh + e];"),
    ("dropped_bd", "S[(size_t)i * K + j] = (ac + bd) * scale;", "S[(size_t)i * K + j] = (ac) * scale;"),
    ("u_on_key_side", "ac += (qe + u[e]) * k[(size_t)j * dh + e];",
     "ac += qe * (k[(size_t)j * dh + e] + u[e]);"),
    ("scale_inverted", "S[(size_t)i * K + j] = (ac + bd) * scale;", "S[(size_t)i * K + j] = (ac + bd) / scale;"),
    ("mask_off_by_one", "if (j - i > M) { S[(size_t)i * K + j] = -INFINITY; continue; }",
     "if (j - i >= M && j > 0) { S[(size_t)i * K + j] = -INFINITY; continue; }"),
    ("distance_sign", "int c = L - 1 - i + j;\n            double ac = 0.0, bd = 0.0;\n            for (int e = 0; e < dh; ++e) {\n                double qe",
     "int c = (K - 1) - (L - 1 - i + j);\n            double ac = 0.0, bd = 0.0;\n            for (int e = 0; e < dh; ++e) {\n                double qe"),
    ("pv_transposed_rows", "acc += (exp(s[j] - m) / l) * v[(size_t)j * dh + e];",
     "acc += (exp(s[j] - m) / l) * v[(size_t)(K - 1 - j) * dh + e];"),
    ("shift_direction", "y[t] = padded[(size_t)L + t];", "y[t] = padded[(size_t)t];"),
    ("tail_keeps_head", "int beg = end - mem_len > 0 ? end - mem_len : 0;", "int beg = 0; end = end < mem_len ? end : mem_len;"),
    ("pos_emb_interleaved", "out[(size_t)c * demb + half + t] = cos(p * inv_freq);",
     "out[(size_t)c * demb + half + t] = cos(p * inv_freq + 1e-3);"),
    ("ln_unbiased_var", "var /= d;", "var /= (d - 1);"),
    ("mem_valid_off_by_one", "for (int j = 0; j < M - mvalid; ++j) vis",
     "for (int j = 0; j < M - mvalid + 1 && j < K; ++j) vis"),
    ("same_length_shift", "int lower = (j - i) <= -shift;", "int lower = (j - i) < -shift;"),
    ("layer_ignores_clamp", "txo_pos_emb(K, d, clamp_len, pe);", "txo_pos_emb(K, d, 0, pe);"),
    ("bwd_dq_drops_position", "dq[(size_t)i * dh + e] += gij * (ke + re);", "dq[(size_t)i * dh + e] += gij * ke;"),
    ("bwd_dk_drops_u", "dk[(size_t)j * dh + e] += gij * (qe + u[e]);", "dk[(size_t)j * dh + e] += gij * qe;"),
    ("bwd_dr_reversed_rows", "dr[(size_t)c * dh + e] += gij * (qe + vb[e]);",
     "dr[(size_t)(K - 1 - c) * dh + e] += gij * (qe + vb[e]);"),
    ("bwd_no_softmax_centering", "P[(size_t)i * K + j] * (dS[(size_t)i * K + j] - rowdot);",
     "P[(size_t)i * K + j] * (dS[(size_t)i * K + j]);"),
    ("bwd_dv_from_g", "dv[(size_t)j * dh + e] += p * dout[(size_t)i * dh + e];",
     "dv[(size_t)j * dh + e] += gij * dout[(size_t)i * dh + e];"),
    ("bwd_scale_dropped", "double gij = dS[(size_t)i * K + j] * scale;", "double gij = dS[(size_t)i * K + j];"),
    ("bwd_du_from_r", "du[e] += gij * ke;", "du[e] += gij * re;"),
]

PINS = [
    pins.test_direct_scores_follow_golden_ids,
    lambda: pins.test_rel_shift_golden_distance_ids(5, 3),
    lambda: pins.test_relative_bias_by_naive_gather(3, 4, 8),
    lambda: pins.test_relative_bias_by_naive_gather(9, 5, 2),
    pins.test_mask_matches_printed_table,
    lambda: pins.test_mem_update_tail_over_segments(12, 8, pins.np.float32),
    pins.test_pos_emb_closed_forms,
    lambda: pins.test_layer_matches_torch_third_opinion(5),
    pins.test_rows_sum_to_one,
    pins.test_m0_zero_position_is_causal_sdpa,
    lambda: pins.test_mem_valid_equals_truncated_memory(3),
    lambda: pins.test_same_length_rows_are_windows(6, 4, 4),
    lambda: pins.test_layer_options_match_torch_third_opinion(3, 0, None),
    lambda: pins.test_backward_matches_finite_differences(1, 2, 5, 3, 4, 0, None),
    lambda: pins.test_backward_matches_torch_autograd_of_literal_form(1, 2, 5, 3, 4),
    pins.test_backward_closed_forms,
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(tmp_path, name, old, new):
    text = open(SRC).read()
    assert text.count(old) >= 1, f"mutation anchor for {name} not found"
    mutated = tmp_path / "mut.c"
    mutated.write_text(text.replace(old, new, 1))
    lib_path = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", str(mutated),
                    "-o", str(lib_path), "-lm"], check=True)
    good = oracle._load()
    try:
        oracle._lib = None
        real = oracle._LIB
        oracle._LIB = str(lib_path)
        oracle._SRC = str(mutated)
        oracle._load()
        caught = []
        for pin in PINS:
            try:
                pin()
            except AssertionError:
                caught.append(pin)
        assert caught, f"no pin caught the planted mistake {name}"
    finally:
        oracle._LIB = real
        oracle._SRC = SRC
        oracle._lib = good
