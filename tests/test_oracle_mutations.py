"""The oracle's pins must catch plausible mistakes.

Each case copies oracle/rodimus_oracle.c, plants one mistake (a sign, a dropped
term, a transposed index, an off-by-one window ...), compiles the copy with gcc
into a temporary library, points the oracle wrapper at it and runs the pins of
tests/test_oracle_pins.py.  At least one pin must fail for every mutant, and
all of them must pass for the unmodified source.  CPU only.
"""
import ctypes
import os
import shutil
import subprocess

import pytest

import oracle
from tests import test_oracle_backward_pins as bpins
from tests import test_oracle_lowrank_pins as lpins
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "rodimus_oracle.c")
HDR = os.path.join(os.path.dirname(oracle.__file__), "rodimus_oracle.h")

PIN_TESTS = [
    lambda: pins.test_gates_match_power_form(),
    lambda: pins.test_gates_special_values(),
    lambda: pins.test_scan_vs_brute_force(False),
    lambda: pins.test_scan_vs_brute_force(True),
    lambda: pins.test_scan_final_state_brute_force(),
    lambda: pins.test_reduction_to_causal_linear_attention(),
    lambda: pins.test_reset_gates(),
    lambda: pins.test_skip_gates(),
    lambda: pins.test_geometric_closed_form(0.7, 0.0),
    lambda: pins.test_decode_steps_equal_scan(),
    lambda: pins.test_decode_geometric(),
    lambda: pins.test_swska_vs_sdpa(5),
    lambda: pins.test_swska_full_window_is_causal_sdpa(),
    lambda: pins.test_swska_window_one_is_identity(),
    lambda: pins.test_swska_constant_key_is_window_mean(),
    lambda: bpins.test_backward_matches_central_differences(True),
    lambda: bpins.test_backward_reduces_to_linear_attention_gradients(),
    lambda: lpins.test_lowrank_logits_match_numpy_contraction(1, (2, 3, 7, 5, 4)),
    lambda: lpins.test_lowrank_silu_values_from_the_tanh_identity(),
    lambda: lpins.test_lowrank_bias_only(),
    lambda: lpins.test_lowrank_symmetries(),
    lambda: lpins.test_lowrank_scan_geometric_closed_form(0.7, 0.3),
]

MUTATIONS = {
    "a_beta_swapped": ("log_a[i] = (tau == 0.0) ? 0.0 : -tau * softplus(-g[i]);",
                       "log_a[i] = (tau == 0.0) ? 0.0 : -tau * softplus(g[i]);"),
    "decay_dropped": ("S[i * dv + j] = a[i] * S[i * dv + j] + bk[i] * vt[j];",
                      "S[i * dv + j] = S[i * dv + j] + bk[i] * vt[j];"),
    "beta_dropped": ("bk[i] = exp(lb) * kt[i];\n        }\n        /* S <- diag(a) S",
                     "bk[i] = kt[i];\n        }\n        /* S <- diag(a) S"),
    "state_transposed_in_output": ("for (int i = 0; i < dk; ++i) acc += qt[i] * S[i * dv + j];",
                                   "for (int i = 0; i < dk; ++i) acc += qt[i] * S[j * dk + i];"),
    "output_before_update": ("        /* S <- diag(a) S + (beta*k)^T v */",
                             "        for (int j = 0; j < dv; ++j) { double acc = 0.0;"
                             " for (int i = 0; i < dk; ++i) acc += qt[i] * S[i * dv + j]; ot[j] = acc; }\n"
                             "        if (0)"),
    "sigmoid_sign": ("if (x >= 0.0) return 1.0 / (1.0 + exp(-x));",
                     "if (x >= 0.0) return 1.0 / (1.0 + exp(x));"),
    "softplus_sign": ("return (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x)));",
                      "return (x > 0.0 ? x : 0.0) - log1p(exp(-fabs(x)));"),
    "decode_decay_dropped": ("So[i * dv + j] = a[i] * Si[i * dv + j] + bk[i] * vt[j];",
                             "So[i * dv + j] = Si[i * dv + j] + bk[i] * vt[j];"),
    "window_off_by_one": ("int s0 = t - J->window + 1;", "int s0 = t - J->window + 2;"),
    "attention_scale_dropped": ("p[s - s0] = J->scale * acc;", "p[s - s0] = acc;"),
    "attention_shared_key_per_head": ("const double *kb = J->k + (size_t)b * T * dk;",
                                      "const double *kb = J->k + (size_t)(bh % J->B) * T * dk;"),
    "bwd_decay_grad_uses_new_state": ("da += G[i * dv + j] * Sp[i * dv + j];",
                                      "da += G[i * dv + j] * St[i * dv + j];"),
    "bwd_state_grad_not_decayed": ("G[i * dv + j] *= at[i];", "G[i * dv + j] *= 1.0;"),
    "bwd_dg_sign": ("dgt[i] = da * at[i] * st * sgm - dbeta * bt[i] * st * sg;",
                    "dgt[i] = da * at[i] * st * sgm + dbeta * bt[i] * st * sg;"),
    "bwd_dq_previous_state": ("for (int j = 0; j < dv; ++j) acc += dOt[j] * St[i * dv + j];",
                              "for (int j = 0; j < dv; ++j) acc += dOt[j] * Sp[i * dv + j];"),
    "bwd_dk_missing_beta": ("dkt[i] = bt[i] * d_bk;", "dkt[i] = d_bk;"),
    "lowrank_silu_as_sigmoid": ("static double silu(double x) { return x * sigmoid(x); }",
                                "static double silu(double x) { return sigmoid(x); }"),
    "lowrank_factor_transposed": ("sg += silu(zgt[r]) * ug[r];",
                                  "sg += silu(zgt[r]) * Ug[((size_t)h * R + r) * dk + c];"),
    "lowrank_bias_dropped": ("double sg = bg[(size_t)h * dk + c], st = bt[(size_t)h * dk + c];",
                             "double sg = 0.0, st = bt[(size_t)h * dk + c];"),
    "lowrank_temperature_activated": ("st += ztt[r] * ut[r];", "st += silu(ztt[r]) * ut[r];"),
    "lowrank_factor_rows_swapped": ("sg += silu(zgt[r]) * ug[r];", "sg += silu(ztt[r]) * ug[r];"),
    "lowrank_head_ignored": ("const double *ug = Ug + ((size_t)h * dk + c) * R;",
                             "const double *ug = Ug + ((size_t)0 * dk + c) * R;"),
}


def _build_variant(tmp_path, old=None, new=None):
    src = open(SRC).read()
    if old is not None:
        assert src.count(old) == 1, f"mutation anchor not unique/found: {old!r}"
        src = src.replace(old, new)
    d = tmp_path / "m"
    d.mkdir()
    (d / "rodimus_oracle.c").write_text(src)
    shutil.copy(HDR, d / "rodimus_oracle.h")
    so = d / "liboracle_variant.so"
    subprocess.check_call(["gcc", "-O1", "-std=c99", "-fPIC", "-shared", "-o", str(so),
                           str(d / "rodimus_oracle.c"), "-lm", "-lpthread"])
    return str(so)


def _use(path):
    real = oracle._load()
    lib = ctypes.CDLL(path)
    for name in ("oracle_gates", "oracle_scan", "oracle_decode", "oracle_swska", "oracle_scan_backward",
                 "oracle_lowrank_gate_logits"):
        getattr(lib, name).argtypes = getattr(real, name).argtypes
        getattr(lib, name).restype = getattr(real, name).restype
    oracle._lib = lib


def _failures():
    n = 0
    for t in PIN_TESTS:
        try:
            t()
        except AssertionError:
            n += 1
    return n


@pytest.fixture
def restore_oracle():
    saved = oracle._load()
    yield
    oracle._lib = saved


def test_unmodified_source_passes_every_pin(tmp_path, restore_oracle):
    _use(_build_variant(tmp_path))
    assert _failures() == 0


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutant_is_caught(name, tmp_path, restore_oracle):
    old, new = MUTATIONS[name]
    _use(_build_variant(tmp_path, old, new))
    assert _failures() >= 1, f"no pin caught mutation {name}"
