"""The oracle pins have teeth: plant one plausible mistake at a time in a
temporary copy of the oracle (on the CPU) and check that tests/test_oracle.py
then fails.  The real oracle is never modified."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    "no_max_subtraction": ("w = np.exp(sc - sc.max())", "w = np.exp(sc)"),
    "exp2_instead_of_exp": ("w = np.exp(sc - sc.max())", "w = np.exp2(sc - sc.max())"),
    "scale_dropped": ("sc = float(scale) * (Kd @ qrow.astype(np.float64))\n    w =",
                      "sc = (Kd @ qrow.astype(np.float64))\n    w ="),
    "head_mapping_h_mod_hk": ("for h in range(g * G, (g + 1) * G):", "for h in range(g, H, Hk):"),
    "int8_scale_group_index": ("s = np.repeat(scales.astype(np.float64), 64, axis=-1)",
                               "s = np.tile(scales.astype(np.float64), 64)"),
    "causal_off_by_one": ("Lt = int(seq_len) - (T - 1 - t)", "Lt = int(seq_len) - (T - t)"),
    "budget_width_ignores_window": ("width = min(Lt, ids_row.shape[0])", "width = ids_row.shape[0]"),
    "merge_weight_sign": ("np.exp(np.where(np.isfinite(m), m - M, 0.0))",
                          "np.exp(np.where(np.isfinite(m), M - m, 0.0))"),
    "merge_denominator_without_l": ("return num / float((e * l).sum())", "return num / float(e.sum())"),
    "k_operand_reversed": ("sc = float(scale) * (Kd @ qrow.astype(np.float64))\n    w =",
                           "sc = float(scale) * (Kd[:, ::-1] @ qrow.astype(np.float64))\n    w ="),
}


# Budget-selection oracle (oracle/select_ref.py) against tests/test_oracle_select.py.
SELECT_MUTANTS = {
    "okey_ignores_sign": ("return np.where(neg, ~bits, bits | np.uint32(0x80000000))",
                          "return np.where(neg, bits, bits | np.uint32(0x80000000))"),
    "ties_to_later_block": ('order = np.argsort(-keys, kind="stable")',
                            'order = np.argsort(-keys, kind="stable")[::-1][np.argsort(-np.sort(-keys)[::-1], kind="stable")]'),
    "last_block_counts_four": ("cells_in[-1] = n % 4", "cells_in[-1] = 4"),
    "budget_off_by_one": ("left = B\n", "left = B - 1\n"),
    "partial_block_dropped": ("nb = n // 4 + 1\n    keys", "nb = max(1, n // 4)\n    keys"),
    "ascending_scores": ('order = np.argsort(-keys, kind="stable")', 'order = np.argsort(keys, kind="stable")'),
}


# Quantize-on-append oracle (oracle/append_ref.py) against tests/test_oracle_append.py.
APPEND_MUTANTS = {
    "round_half_away": ("np.rint(g / d)", "np.trunc(g / d + np.copysign(np.float32(0.5), g))"),
    "group_of_32": ("g = x.reshape(x.shape[:-1] + (D // 64, 64))",
                    "g = x.reshape(x.shape[:-1] + (D // 32, 32))[..., ::2, :].repeat(2, axis=-2)"),
    "clamp_126": ("np.clip(q, -127.0, 127.0)", "np.clip(q, -126.0, 126.0)"),
    "code_from_f16_scale": ("np.rint(g / d)", "np.rint(g / d.astype(np.float16).astype(np.float32))"),
    "divide_by_128": ("d = (amax / np.float32(127.0))", "d = (amax / np.float32(128.0))"),
    "write_off_by_one": ("c = int(pos[s]) + i\n", "c = int(pos[s]) + i + 1\n"),
}


# Output-gate oracle (oracle/gate_ref.py) against tests/test_oracle_gate.py.
GATE_MUTANTS = {
    "exp_sign": ("return 1.0 / (1.0 + np.exp(-x))", "return 1.0 / (1.0 + np.exp(x))"),
    "tanh_gate": ("return 1.0 / (1.0 + np.exp(-x))", "return 0.5 * (1.0 + np.tanh(x))"),
    "gate_from_query_half": ("return qfull[..., :D], qfull[..., D:]",
                             "return qfull[..., :D], qfull[..., :D]"),
    "gate_added": ("return np.asarray(out, dtype=np.float64) * sigmoid(gate)",
                   "return np.asarray(out, dtype=np.float64) + sigmoid(gate)"),
}


# TurboQuant decode oracle (oracle/tq_ref.py) against tests/test_oracle_tq.py.
TQ_MUTANTS = {
    "jl_sign_flipped": ("signed_sum = 2.0 * pos_sum - q_jl.sum()", "signed_sum = q_jl.sum() - 2.0 * pos_sum"),
    "jl_factor_two_dropped": ("signed_sum = 2.0 * pos_sum - q_jl.sum()", "signed_sum = pos_sum - q_jl.sum()"),
    "jl_total_dropped": ("signed_sum = 2.0 * pos_sum - q_jl.sum()", "signed_sum = 2.0 * pos_sum"),
    "residual_norm_dropped": ("correction = norm * residual_norm * float(qjl_scale) * signed_sum",
                              "correction = norm * float(qjl_scale) * signed_sum"),
    "polar_field_order_reversed": ("idx = (w[..., :, None] >> (np.uint32(2) * k)) & np.uint32(3)",
                                   "idx = (w[..., :, None] >> (np.uint32(2) * (np.uint32(15) - k))) & np.uint32(3)"),
    "jl_bit_order_reversed": ("b = (w[..., :, None] >> k) & np.uint32(1)",
                              "b = (w[..., :, None] >> (np.uint32(31) - k)) & np.uint32(1)"),
    "rotation_unnormalised": ("(hadamard(D) @ acc) / math.sqrt(D)", "(hadamard(D) @ acc)"),
    "signs_not_undone": ("return np.asarray(signs, dtype=np.float64) * (hadamard(D) @ acc)",
                         "return (hadamard(D) @ acc)"),
    "norm_halves_swapped": ("norm, residual_norm = f16_halves(k_norms)",
                            "residual_norm, norm = f16_halves(k_norms)"),
    "polar_term_without_norm": ("return (polar_dot * norm + correction) * float(scale)",
                                "return (polar_dot + correction) * float(scale)"),
}


def run_mutant(tmp_path, module, test_file, before, after, name):
    src = open(os.path.join(ROOT, "oracle", module)).read()
    assert before in src, f"mutation site for {name} no longer exists"
    shutil.copytree(os.path.join(ROOT, "oracle"), tmp_path / "oracle")
    shutil.copytree(os.path.join(ROOT, "workloads"), tmp_path / "workloads")
    (tmp_path / "tests").mkdir()
    for f in ("conftest.py", test_file):
        shutil.copy(os.path.join(ROOT, "tests", f), tmp_path / "tests" / f)
    (tmp_path / "oracle" / module).write_text(src.replace(before, after, 1))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "tests/" + test_file], cwd=tmp_path, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 1, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    before, after = MUTANTS[name]
    run_mutant(tmp_path, "decode_ref.py", "test_oracle.py", before, after, name)


@pytest.mark.parametrize("name", sorted(SELECT_MUTANTS))
def test_select_pins_catch_mutant(name, tmp_path):
    before, after = SELECT_MUTANTS[name]
    run_mutant(tmp_path, "select_ref.py", "test_oracle_select.py", before, after, name)


@pytest.mark.parametrize("name", sorted(APPEND_MUTANTS))
def test_append_pins_catch_mutant(name, tmp_path):
    before, after = APPEND_MUTANTS[name]
    run_mutant(tmp_path, "append_ref.py", "test_oracle_append.py", before, after, name)


@pytest.mark.parametrize("name", sorted(GATE_MUTANTS))
def test_gate_pins_catch_mutant(name, tmp_path):
    before, after = GATE_MUTANTS[name]
    run_mutant(tmp_path, "gate_ref.py", "test_oracle_gate.py", before, after, name)


@pytest.mark.parametrize("name", sorted(TQ_MUTANTS))
def test_tq_pins_catch_mutant(name, tmp_path):
    before, after = TQ_MUTANTS[name]
    run_mutant(tmp_path, "tq_ref.py", "test_oracle_tq.py", before, after, name)
