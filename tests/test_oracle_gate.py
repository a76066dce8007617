"""Pins of the output-gate oracle (oracle/gate_ref.py), CPU only.

The pages print no worked numbers for the gate, so the pins are closed
forms of the logistic sigmoid, its limits, the layout of a [query | gate]
row built by hand, the empty-window rule, and the gated decode against the
ungated oracle scaled by factors computed here with math.exp."""
import math

import numpy as np
import pytest

from oracle import decode_ref as DR
from oracle import gate_ref as R
from workloads import make_case


def test_sigmoid_closed_forms():
    # sigmoid(0) = 1/2, sigmoid(ln 3) = 3/4, sigmoid(-ln 3) = 1/4
    x = np.array([0.0, math.log(3.0), -math.log(3.0)])
    np.testing.assert_allclose(R.sigmoid(x), [0.5, 0.75, 0.25], rtol=0, atol=1e-15)


def test_sigmoid_limits_and_symmetry():
    assert R.sigmoid(np.array([800.0]))[0] == 1.0
    assert R.sigmoid(np.array([-800.0]))[0] == 0.0          # exp overflows to inf: value 0
    x = np.linspace(-30, 30, 61)
    np.testing.assert_allclose(R.sigmoid(x) + R.sigmoid(-x), 1.0, rtol=0, atol=1e-15)
    # increasing
    assert np.all(np.diff(R.sigmoid(x)) > 0)


def test_split_query_gate_layout():
    S, T, H, D = 2, 3, 4, 8
    q = np.arange(S * T * H * D, dtype=np.float32).reshape(S, T, H, D)
    g = -np.arange(S * T * H * D, dtype=np.float32).reshape(S, T, H, D) - 1.0
    full = np.concatenate([q, g], axis=-1)                 # [query | gate] per (t, h)
    assert full.shape == (S, T, H, 2 * D)
    # element (s, t, h, D + d) of the flat row is the gate
    flat = full.reshape(-1)
    s, t, h, d = 1, 2, 3, 5
    assert flat[((s * T + t) * H + h) * 2 * D + D + d] == g[s, t, h, d]
    qq, gg = R.split_query_gate(full)
    assert np.array_equal(qq, q) and np.array_equal(gg, g)


def test_apply_gate_elementwise():
    out = np.array([[2.0, -4.0, 8.0]])
    gate = np.array([[0.0, math.log(3.0), -math.log(3.0)]])
    np.testing.assert_allclose(R.apply_gate(out, gate), [[1.0, -3.0, 2.0]], rtol=0, atol=1e-14)


@pytest.mark.parametrize("kv", ["f16", "i8"])
def test_gated_decode_equals_ungated_times_factor(kv):
    inp = make_case(2, 2, 8, 2, 64, 50, [50, 0], kv=kv, seed=21)   # second sequence: empty windows
    rng = np.random.default_rng(5)
    gate = rng.standard_normal(inp.q.shape).astype(np.float32) * 3.0
    got = R.gqa_decode_gated_ref(inp.q, inp.k, inp.v, inp.seq_lens, inp.scale, gate,
                                 inp.k_scales, inp.v_scales)
    base = DR.gqa_decode_ref(inp.q, inp.k, inp.v, inp.seq_lens, inp.scale, inp.k_scales,
                             inp.v_scales)
    S, T, H, D = inp.q.shape
    for s in range(S):
        for t in range(T):
            for h in range(H):
                for d in (0, 17, D - 1):
                    f = 1.0 / (1.0 + math.exp(-float(gate[s, t, h, d])))
                    assert abs(got[s, t, h, d] - base[s, t, h, d] * f) <= 1e-12 * (1 + abs(base[s, t, h, d]))
    assert not got[1].any()                                  # empty windows stay 0
