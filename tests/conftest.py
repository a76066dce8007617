import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


# Tolerance for fp32 GPU output against the fp64 oracle: max absolute error
# <= 2e-3 and row-relative max error <= 1e-3, where a row is one output
# vector (s, t, h) and its relative error is max_d |g - r| / max_d |r|
# (0/0 counts as 0).
ATOL = 2e-3
RTOL_ROW = 1e-3


def parity_errors(got: np.ndarray, ref: np.ndarray):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if got.size == 0:
        return 0.0, 0.0
    D = ref.shape[-1]
    g2 = got.reshape(-1, D)
    r2 = ref.reshape(-1, D)
    diff = np.abs(g2 - r2)
    max_abs = float(diff.max())
    num = diff.max(axis=1)
    den = np.abs(r2).max(axis=1)
    rel = np.where(den > 0, num / np.where(den > 0, den, 1.0), np.where(num > 0, np.inf, 0.0))
    return max_abs, float(rel.max())


def assert_parity(got, ref, what=""):
    got = np.asarray(got)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    max_abs, max_rel = parity_errors(got, ref)
    assert max_abs <= ATOL and max_rel <= RTOL_ROW, \
        f"{what}: max_abs={max_abs:.3e} (<= {ATOL}) max_row_rel={max_rel:.3e} (<= {RTOL_ROW})"
    return max_abs, max_rel
