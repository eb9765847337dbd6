"""Mutation check of the oracle's pins (CPU only).

Each case plants one plausible mistake in a temporary copy of the oracle's C
source (a reversed tap, a dropped halo, a wrong shift direction, floor
instead of ceil, a missing decay, a wrong sign, the wrong GQA map, ...),
builds it, and runs the pin tests against it: at least one pin must fail.
The oracle in the tree is never touched.
"""
import importlib.util
import os
import subprocess

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def _module(name):
    spec = importlib.util.spec_from_file_location("pins_" + name, os.path.join(HERE, name + ".py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _pins():
    ch, cv, gd = _module("test_oracle_chunks"), _module("test_oracle_conv"), _module("test_oracle_gdn")
    pins = [ch.test_tiny_lengths_5_and_13, ch.test_step_budget_two_sequences_gives_256,
            ch.test_exhaustive_small,
            cv.test_matches_numpy_correlate_with_state, cv.test_matches_torch_conv1d_zero_state,
            cv.test_identity_tap_gives_input_plus_bias,
            cv.test_oldest_tap_shifts_by_three_and_reads_state,
            cv.test_zero_weights_give_silu_of_bias, cv.test_update_equals_varlen_single_token,
            cv.test_update_window_shift, cv.test_padding_and_empty_sequences_untouched,
            gd.test_single_token_from_zero_closed_form, gd.test_identity_when_beta_zero_alpha_one,
            gd.test_zero_key_only_decays, gd.test_delta_rule_retrieval,
            gd.test_orthonormal_keys_accumulate_outer_products, gd.test_gqa_head_map,
            gd.test_padding_slot_and_no_initial_state, cv.test_round_bf16_rounds_doubles_once]
    pins += [lambda L=L: cv.test_short_sequences_state_carry(L) for L in (0, 1, 2, 3, 5, 9)]
    pins += [lambda n=n, hk=hk, hv=hv: gd.test_dense_brute_force(n, hk, hv)
             for n in (True, False) for (hk, hv) in ((2, 2), (2, 4))]
    return pins


MUTATIONS = [
    ("conv taps reversed",
     "bf16_bits_to_double(w[(int64_t)c * K + j]) *\n                         bf16_bits_to_double(e[p + j])",
     "bf16_bits_to_double(w[(int64_t)c * K + (K - 1 - j)]) *\n                         bf16_bits_to_double(e[p + j])"),
    ("carried state dropped", "e[i] = init ? st[(int64_t)i * C + c] : 0;", "e[i] = 0;"),
    ("new conv state off by one", "st[(int64_t)i * C + c] = e[L + i];",
     "st[(int64_t)i * C + c] = e[L + i - 1];"),
    ("bias dropped", "double z = bias ? bf16_bits_to_double(bias[c]) : 0.0;\n                for",
     "double z = 0.0;\n                for"),
    ("sigmoid instead of silu", "return z / (1.0 + exp(-z));", "return 1.0 / (1.0 + exp(-z));"),
    ("update shifts the wrong way",
     "st[(int64_t)j * C + c] = st[(int64_t)(j + 1) * C + c];",
     "st[(int64_t)(j + 1) * C + c] = st[(int64_t)j * C + c];"),
    ("chunks rounded down", "(len + ORACLE_CHUNK_TOKENS - 1) / ORACLE_CHUNK_TOKENS",
     "len / ORACLE_CHUNK_TOKENS"),
    ("decay missing on the erase term", "*sij = a * (*sij - b * u[i] * kh[j]) + b * vi * kh[j];",
     "*sij = a * *sij - b * u[i] * kh[j] + b * vi * kh[j];"),
    ("erase sign flipped", "*sij = a * (*sij - b * u[i] * kh[j]) + b * vi * kh[j];",
     "*sij = a * (*sij + b * u[i] * kh[j]) + b * vi * kh[j];"),
    ("g used as the decay itself", "const double a = exp((double)g[t * HV + h]);",
     "const double a = (double)g[t * HV + h];"),
    ("GQA map modulo", "const int32_t hk = h / group;", "const int32_t hk = h % num_k_heads;"),
    ("norm epsilon dropped", "const double rq = 1.0 / sqrt(nq + 1e-6);",
     "const double rq = 1.0 / sqrt(nq);"),
    ("output reads k instead of q",
     "for (int32_t j = 0; j < dk; ++j) acc += S[(int64_t)i * dk + j] * qh[j];",
     "for (int32_t j = 0; j < dk; ++j) acc += S[(int64_t)i * dk + j] * kh[j];"),
    ("initial state ignored", "            if (!init)\n", "            if (0)\n"),
    ("bf16 rounding through float32 first", "const double r = rint(d / ulp) * ulp;",
     "const double r = rint((double)(float)d / ulp) * ulp;"),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, old, new, tmp_path):
    src = open(oracle._SRC).read()
    assert src.count(old) == 1, "mutation anchor not unique: " + name
    mutant_c = tmp_path / "mutant.c"
    mutant_c.write_text(src.replace(old, new))
    so = str(tmp_path / "libmutant.so")
    subprocess.check_call(["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fPIC", "-shared",
                           "-o", so, str(mutant_c), "-lm"])
    saved = oracle._lib
    oracle._lib = oracle.bind(so)
    failed = []
    try:
        for pin in _pins():
            try:
                pin()
            except Exception as e:            # noqa: BLE001 - any failure counts
                failed.append((getattr(pin, "__name__", "pin"), type(e).__name__))
    finally:
        oracle._lib = saved
    assert failed, "no pin caught the planted mistake: " + name


def test_unmutated_oracle_passes_every_pin():
    """The harness itself: the real oracle passes every pin it runs, so a
    caught mutation is caught by the mistake, not by a broken pin."""
    for pin in _pins():
        pin()
