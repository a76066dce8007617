"""fp64 CPU oracle for the output gate applied at the end of the merge.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or
executes this module; only the tests and the bench's CPU-baseline leg do.  It
shares no code with the HIP library.

What it computes (qsa2.metal, kernel qsa_merge2, last lines; FORWARD_MSL,
kernel attn_combine, the store): after the log-sum-exp merge of a query
row's partials, each output element is multiplied by the logistic sigmoid of
the gate element of the same (sequence, token, head, dim):

    y[s, t, h, d] = out[s, t, h, d] * 1 / (1 + exp(-gate[s, t, h, d]))

The gate comes with the query: both pages keep one [query | gate] row of
2 * D floats per (token, head), the query in the first D and the gate in the
second D.  A row with an empty window merges to 0 and stays 0.

Pinned by tests/test_oracle_gate.py (sigmoid closed forms at 0 and +-ln 3,
its limits, the [query | gate] split against hand-built rows, the empty-window
rule, and the gated decode against the ungated oracle times a hand-computed
factor).
"""
from __future__ import annotations

import numpy as np

from oracle.decode_ref import gqa_decode_ref

__all__ = ["sigmoid", "split_query_gate", "apply_gate", "gqa_decode_gated_ref"]


def sigmoid(x: np.ndarray) -> np.ndarray:
    """1 / (1 + exp(-x)) in fp64 (the form both pages write).  exp overflows
    to inf for x < -709, where the value is 0."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def split_query_gate(qfull: np.ndarray):
    """[..., 2D] rows of [query | gate] -> (query [..., D], gate [..., D])."""
    D2 = qfull.shape[-1]
    assert D2 % 2 == 0
    D = D2 // 2
    return qfull[..., :D], qfull[..., D:]


def apply_gate(out: np.ndarray, gate: np.ndarray) -> np.ndarray:
    """out * sigmoid(gate), elementwise, fp64."""
    return np.asarray(out, dtype=np.float64) * sigmoid(gate)


def gqa_decode_gated_ref(q, k, v, seq_lens, scale, gate, k_scales=None, v_scales=None,
                         ids=None) -> np.ndarray:
    """The decode output (oracle.decode_ref.gqa_decode_ref) with the gate
    applied: [S][T][H][D] fp64."""
    out = gqa_decode_ref(q, k, v, seq_lens, scale, k_scales, v_scales, ids)
    return apply_gate(out, gate)
