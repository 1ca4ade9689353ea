"""The pins catch plausible mistakes: each mutant of the oracle's C source
(one planted slip, built on the CPU into a scratch directory) must fail at
least one pin of test_oracle_pins.py."""
import ctypes
import os
import subprocess

import pytest

import oracle
import test_oracle_pins as pins

with open(oracle.SRC) as f:
    SOURCE = f.read()

CORRECTION_HEAD = "                /* 2. delta correction against the decayed state */\n"
READOUT_HEAD = "                /* 4. readout from the updated state */\n"


MUTANTS = {
    "no_decay": ("S[i * V + j] = a * S[i * V + j];", "S[i * V + j] = S[i * V + j];"),
    "exp_of_minus_g": ("const double a = exp(gd[i]);", "const double a = exp(-gd[i]);"),
    "plus_u": ("bt * (bf16_value(vt[j]) - u)", "bt * (bf16_value(vt[j]) + u)"),
    "no_beta": ("vp[j] = bt * (bf16_value(vt[j]) - u);", "vp[j] = (bf16_value(vt[j]) - u);"),
    "transposed_state": ("u += S[i * V + j] * bf16_value(kt[i]);", "u += S[j * V + i] * bf16_value(kt[i]);"),
    "update_with_q": ("const double ki = bf16_value(kt[i]);", "const double ki = bf16_value(qt[i]);"),
    "readout_with_k": ("acc += S[i * V + j] * bf16_value(qt[i]);", "acc += S[i * V + j] * bf16_value(kt[i]);"),
    "no_scale": ("o[j] = scale * acc;", "o[j] = acc;"),
    "head_modulo": ("const int64_t h = hv / heads_per_qk;", "const int64_t h = hv % H;"),
    "norm_sum_not_mean": ("sqrt(sum_sq / (double)V + eps)", "sqrt(sum_sq + eps)"),
    "norm_eps_outside": ("sqrt(sum_sq / (double)V + eps)", "(sqrt(sum_sq / (double)V) + eps)"),
    "sigmoid_not_silu": ("return x / (1.0 + exp(-x));", "return 1.0 / (1.0 + exp(-x));"),
    "no_weight": ("o[j] * r * bf16_value(w[j]) * silu", "o[j] * r * silu"),
    "gate_head0": ("gate + t * gate_stride + hv * V", "gate + t * gate_stride"),
    "drop_last_token": ("t < cu_seqlens[n + 1]; ++t)", "t + 1 < cu_seqlens[n + 1]; ++t)"),
    "beta_of_head0": ("beta[t * beta_stride + hv]", "beta[t * beta_stride]"),
    "g_of_head0": ("g + t * g_stride + hv * K", "g + t * g_stride"),
    "inter_state_of_head0": ("memcpy(inter_state + t * inter_stride + hv * K * V, S,",
                             "memcpy(inter_state + t * inter_stride, S,"),
    "softplus_even_sign": ("log1p(exp(-fabs(x)))", "log1p(exp(fabs(x)))"),
    "softplus_no_relu": ("return (x > 0.0 ? x : 0.0) + log1p", "return log1p"),
    "A_not_exponentiated": ("const double A = exp((double)A_log[hv]);", "const double A = (double)A_log[hv];"),
    "A_log_of_head0": ("exp((double)A_log[hv])", "exp((double)A_log[0])"),
    "g_positive": ("g_out[i] = -A * softplus", "g_out[i] = A * softplus"),
    "dt_bias_dropped": ("softplus(bf16_value(rg[i]) + (double)dt_bias[hv * K + i])", "softplus(bf16_value(rg[i]))"),
    "dt_bias_of_head0": ("(double)dt_bias[hv * K + i]", "(double)dt_bias[i]"),
    "raw_gate_of_head0": ("raw_gate + t * raw_gate_stride + hv * K;", "raw_gate + t * raw_gate_stride;"),
    "raw_gate_of_token0": ("raw_gate + t * raw_gate_stride + hv * K;", "raw_gate + hv * K;"),
    "sigmoid_sign": ("return 1.0 / (1.0 + exp(-r));", "return 1.0 / (1.0 + exp(r));"),
    "raw_beta_of_head0": ("raw_beta[t * raw_beta_stride + hv]", "raw_beta[t * raw_beta_stride]"),
    "readout_before_update": "READOUT_BEFORE_UPDATE",
    "decay_after_correction": "DECAY_AFTER_CORRECTION",
}


def _mutate(name):
    m = MUTANTS[name]
    if m == "READOUT_BEFORE_UPDATE":
        head = "                /* 3. rank-1 update S += k v'^T */\n"
        start = SOURCE.index(head)
        end = SOURCE.index(READOUT_HEAD)
        block3 = SOURCE[start:end]
        ro_end = SOURCE.index("                /* 5. optional gated RMSNorm")
        block4 = SOURCE[end:ro_end]
        return SOURCE[:start] + block4 + block3 + SOURCE[ro_end:]
    if m == "DECAY_AFTER_CORRECTION":
        start = SOURCE.index("                /* 1. decay")
        mid = SOURCE.index(CORRECTION_HEAD)
        end = SOURCE.index("                /* 3. rank-1 update")
        return SOURCE[:start] + SOURCE[mid:end] + SOURCE[start:mid] + SOURCE[end:]
    old, new = m
    assert SOURCE.count(old) == 1, name
    return SOURCE.replace(old, new)


PINS = [
    pins.test_hand_worked_two_tokens_exact,
    pins.test_gated_rmsnorm_sigmoid_table,
    lambda: pins.test_matrix_form_brute_force_k4(0),
    pins.test_exact_rational_k3,
    pins.test_identity_g0_beta0,
    pins.test_plain_delta_rule_g0,
    pins.test_reset_all_channels,
    pins.test_reset_subset_of_channels,
    pins.test_retrieval_unit_key,
    pins.test_pure_decay_beta0,
    pins.test_chained_single_tokens_equal_one_multi_token_call,
    pins.test_skipped_rows_and_untouched_slots,
    pins.test_value_heads_share_qk_heads,
    pins.test_norm_constant_row_closed_form,
    pins.test_norm_scale_invariance_and_gate_symmetry,
    pins.test_norm_epilogue_wiring_in_decode,
    pins.test_intermediate_states_are_the_chained_states,
    pins.test_gate_activation_logistic_closed_form,
    pins.test_gate_activation_odd_part_and_scaling,
    pins.test_gate_activation_bias_shift,
    pins.test_gate_activation_beta_logistic,
    pins.test_gate_activation_saturates_at_infinity,
    pins.test_fused_gate_decode_equals_exact_activated_inputs,
    pins.test_fused_gate_pure_decay_closed_form,
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_fails_a_pin(name, tmp_path, monkeypatch):
    src = tmp_path / "mutant.c"
    src.write_text(_mutate(name))
    lib_path = str(tmp_path / "libmutant.so")
    subprocess.run(["gcc", *oracle.CFLAGS, "-o", lib_path, str(src), "-lm"], check=True)
    original = oracle._lib
    monkeypatch.setattr(oracle, "_lib", None)
    monkeypatch.setattr(oracle, "LIB", lib_path)
    monkeypatch.setattr(oracle, "SRC", str(src))
    caught = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError):
            caught.append(pin)
    monkeypatch.setattr(oracle, "_lib", original)
    assert caught, f"mutant {name} passed every pin"


def test_unmutated_source_passes_every_pin():
    for pin in PINS:
        pin()
