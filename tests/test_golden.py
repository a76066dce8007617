"""The oracle reproduces its stored outputs (tests/golden/, written by
tests/golden/make_golden.py from the oracle alone)."""
import os

import numpy as np

from oracle.decode_ref import gqa_decode_ref
from workloads import make_inputs, make_case

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_golden(name):
    path = os.path.join(GOLDEN, name)
    with open(path) as f:
        lines = f.readlines()
    shape = [int(x) for x in lines[1].split("shape")[1].split(";")[0].split()]
    data = np.array([[float(x) for x in ln.split()] for ln in lines[2:]], dtype=np.float64)
    return data.reshape(shape)


def golden_small_i8_inputs():
    return make_case(2, 3, 4, 1, 64, 70, [70, 2], kv="i8", budget=24, seed=21, scale=1.0 / 8.0)


def test_tiny_f16_golden():
    inp = make_inputs("tiny_f16")
    out = gqa_decode_ref(inp.q, inp.k, inp.v, inp.seq_lens, inp.scale)
    np.testing.assert_allclose(out, load_golden("tiny_f16.txt"), rtol=1e-15, atol=1e-16)


def test_small_i8_ids_causal_golden():
    inp = golden_small_i8_inputs()
    out = gqa_decode_ref(inp.q, inp.k, inp.v, inp.seq_lens, inp.scale, inp.k_scales, inp.v_scales, inp.ids)
    g = load_golden("small_i8_ids_causal.txt")
    np.testing.assert_allclose(out, g, rtol=1e-15, atol=1e-16)
    assert not g[1, 0].any() and g[1, 1].any()
