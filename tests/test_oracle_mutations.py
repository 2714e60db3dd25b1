"""The pins bite: plant one plausible mistake at a time in a copy of the
oracle (on the CPU), rebuild it, and require that at least one pin fails.

Each mutation is a textual substitution in oracle.c: a dropped term, a wrong
sign or index, a transposed operand, the wrong rounding. The mutant is a
separate shared library; the real oracle is untouched.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import test_oracle_pins as pins
import test_oracle_q40 as q40_pins
import test_oracle_sampling as sampling_pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "oracle.c")

MUTATIONS = {
    "rope_sign": ("hv[2 * j] = (float)(a * c - b * sn);", "hv[2 * j] = (float)(a * c + b * sn);"),
    "rope_freq_index": ("-(double)(2 * j) / (double)hs);\n            float ang",
                        "-(double)(j) / (double)hs);\n            float ang"),
    "rope_k_dropped": ("rope(m->k, m->nkv, hs, pos);", ";"),
    "attn_scale": ("double scale = 1.0 / sqrt((double)hs);", "double scale = 1.0 / (double)hs;"),
    "gqa_index": ("int64_t g = hd / m->kvmul;", "int64_t g = hd % m->nkv;"),
    "attn_drops_current_pos": ("for (int64_t t = 0; t <= pos; t++) {\n            const float* kt",
                               "for (int64_t t = 0; t < pos; t++) {\n            const float* kt"),
    "rmsnorm_eps_dropped": ("ss / (double)n + 1e-5", "ss / (double)n"),
    "rmsnorm_sum_not_mean": ("ss / (double)n + 1e-5", "ss + 1e-5"),
    "quant_half_even": ("return (int8_t)roundf(quotient);", "return (int8_t)rintf(quotient);"),
    "quant_scale_255": ("return amax / 127.0f;", "return amax / 255.0f;"),
    "quant_truncates": ("return (int8_t)roundf(quotient);", "return (int8_t)quotient;"),
    "q8_act_scale_dropped": ("acc += (double)dot * (double)sr[g] * (double)as[g];",
                             "acc += (double)dot * (double)sr[g];"),
    "swiglu_branches_swapped": ("double z = m->h1[i];", "double z = m->h3[i];"),
    "residual_dropped": ("matvec(m, m->y, m->o, &m->wo, l * d * d, d, d, tr ? 1 : -1);\n        residual(m->x, m->y, d);",
                         "matvec(m, m->y, m->o, &m->wo, l * d * d, d, d, tr ? 1 : -1);"),
    "matvec_transposed": ("for (int64_t j = 0; j < cols; j++) acc += (double)wr[j] * (double)x[j];",
                          "for (int64_t j = 0; j < cols; j++) acc += (double)W[j * rows + i] * (double)x[j];"),
    "kv_slot_off_by_layer": ("float* kslot = m->kc + (l * m->S + pos) * kvd;",
                             "float* kslot = m->kc + (pos) * kvd;"),
    "emb_dequant_scale_dropped": ("m->x[i] = (float)((double)qr[i] * (double)sr[i / m->gs]);",
                                  "m->x[i] = (float)((double)qr[i]);"),
    "q40_nibble_halves_swapped": ("dot += ((int32_t)(w[b] & 15) - 8) * (int32_t)xq[b];",
                                  "dot += ((int32_t)(w[b] & 15) - 8) * (int32_t)xq[b + 16];"),
    "q40_offset_7": ("dot += ((int32_t)(w[b] >> 4) - 8) * (int32_t)xq[b + 16];",
                     "dot += ((int32_t)(w[b] >> 4) - 7) * (int32_t)xq[b + 16];"),
    "q40_scale_positive": ("m / -8.0f;", "m / 8.0f;"),
    "q40_clamp_8": ("v = r < -8.0f ? -8 : r > 7.0f ? 7 : (int)r;", "v = r < -8.0f ? -8 : r > 8.0f ? 8 : (int)r;"),
    "q40_input_scale_dropped": ("acc += (double)q40_group_dot(qr + g * 16, aq + g * 32) * (double)sr[g] * (double)as[g];",
                                "acc += (double)q40_group_dot(qr + g * 16, aq + g * 32) * (double)sr[g];"),
    "q40_model_embedding_nibbles_swapped": ("const int code = (j < 16 ? (b & 15) : (b >> 4)) - 8;",
                                            "const int code = (j < 16 ? (b >> 4) : (b & 15)) - 8;"),
    "q40_model_weight_offset": ("matvec_q40_rows(out, m->aq, m->as, w->p + woff / 2, w->s + woff / 32, rows, cols);",
                                "matvec_q40_rows(out, m->aq, m->as, w->p + woff / 2, w->s + woff / 64, rows, cols);"),
    "sample_temperature_multiplies": ("return (float)((double)logit / temperature + g);",
                                      "return (float)((double)logit * temperature + g);"),
    "sample_gumbel_sign": ("const double g = -log(-log(u));", "const double g = log(-log(u));"),
    "sample_draw_constant": ("uint64_t z = seed + k * 0x9E3779B97F4A7C15ull;",
                             "uint64_t z = seed + k * 0x9E3779B97F4A7C14ull;"),
}

PIN_TESTS = [
    pins.test_quantize_handworked_golden,
    pins.test_quantize_exact_rational_bruteforce,
    pins.test_rope_unit_pair_gives_cos_sin,
    pins.test_rope_preserves_pair_norms_and_relative_position,
    lambda: pins.test_oracle_matches_full_sequence_bruteforce(pins.TINY, 0, 12),
    lambda: pins.test_oracle_matches_full_sequence_bruteforce(pins.TINY_Q8, 1, 8),
    lambda: pins.test_oracle_matches_full_sequence_bruteforce(pins.TINY_Q4, 2, 8),
    pins.test_attention_pos0_is_v_and_equal_keys_give_mean_v,
    pins.test_rmsnorm_closed_form_through_embedding,
    sampling_pins.test_splitmix64_published_outputs,
    q40_pins.test_q40_handworked_golden,
    q40_pins.test_q40_matvec_closed_form,
    lambda: sampling_pins.test_draws_follow_softmax_of_scaled_logits(0.8),
]


def _any_pin_fails(lib) -> bool:
    saved = oracle._lib
    oracle._lib = lib
    try:
        for t in PIN_TESTS:
            try:
                with np.errstate(all="ignore"):
                    t()
            except (AssertionError, ValueError, FloatingPointError):
                return True
        return False
    finally:
        oracle._lib = saved


def test_unmutated_copy_passes(tmp_path):
    so = tmp_path / "liboracle_copy.so"
    shutil.copy(SRC, tmp_path / "o.c")
    subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
                           "-o", str(so), str(tmp_path / "o.c"), "-lm"])
    assert not _any_pin_fails(oracle.bind(str(so)))


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(tmp_path, name):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique/present"
    (tmp_path / "m.c").write_text(src.replace(old, new))
    so = tmp_path / f"liboracle_{name}.so"
    subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
                           "-o", str(so), str(tmp_path / "m.c"), "-lm"])
    assert _any_pin_fails(oracle.bind(str(so))), f"no pin catches mutation {name}"
