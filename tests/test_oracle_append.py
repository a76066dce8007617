"""Pins of the quantize-on-append oracle (oracle/append_ref.py), CPU only."""
import numpy as np
import pytest

from oracle import append_ref as R


def test_closed_form_group():
    x = np.zeros(64, dtype=np.float32)
    x[0], x[1], x[2], x[3] = 127.0, -127.0, 63.0, 0.4
    codes, scales = R.quantize_groups(x)
    assert scales[0] == np.float16(1.0)
    assert list(codes[:5]) == [127, -127, 63, 0, 0]


def test_round_half_to_even():
    x = np.zeros(64, dtype=np.float32)
    x[0] = 127.0                        # d = 1 exactly
    x[1:7] = [2.5, 3.5, -2.5, -3.5, 0.5, 1.5]
    codes, _ = R.quantize_groups(x)
    assert list(codes[1:7]) == [2, 4, -2, -4, 0, 2]


def test_zero_group_and_independence():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(256).astype(np.float32)
    x[64:128] = 0.0
    codes, scales = R.quantize_groups(x)
    assert not codes[64:128].any() and scales[1] == 0
    y = x.copy()
    y[200] *= 50.0                      # only the fourth group changes
    c2, s2 = R.quantize_groups(y)
    assert np.array_equal(c2[:192], codes[:192]) and np.array_equal(s2[:3], scales[:3])
    assert s2[3] != scales[3]


@pytest.mark.parametrize("seed", range(4))
def test_reconstruction_bound_and_extremes(seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((50, 128)) * 10.0 ** rng.uniform(-3, 3, (50, 1))).astype(np.float32)
    codes, scales = R.quantize_groups(x)
    g = x.reshape(50, 2, 64).astype(np.float64)
    c = codes.reshape(50, 2, 64).astype(np.float64)
    d = (np.max(np.abs(g), axis=-1, keepdims=True) / 127.0)
    assert np.all(np.abs(g - c * d) <= d / 2 * (1 + 1e-6))
    # the largest magnitude of every group maps to +-127
    i = np.argmax(np.abs(g), axis=-1)
    top = np.take_along_axis(c, i[..., None], axis=-1)[..., 0]
    assert np.all(np.abs(top) == 127)
    # the stored scale is the fp32 d rounded to f16
    d32 = (np.max(np.abs(x.reshape(50, 2, 64)), axis=-1) / np.float32(127)).astype(np.float32)
    assert np.array_equal(scales, d32.astype(np.float16))


def test_append_positions_and_truncation():
    rng = np.random.default_rng(5)
    S, Tn, Hk, D, Lmax = 3, 4, 2, 64, 10
    kn = rng.standard_normal((S, Tn, Hk, D)).astype(np.float32)
    vn = rng.standard_normal((S, Tn, Hk, D)).astype(np.float32)
    k = np.full((S, Lmax, Hk, D), 9, dtype=np.int8)
    v = k.copy()
    ks = np.full((S, Lmax, Hk, 1), 2.0, dtype=np.float16)
    vs = ks.copy()
    pos = np.array([0, 5, 8], dtype=np.int32)           # the last sequence runs past Lmax
    k2, v2, ks2, vs2 = R.append_i8(kn, vn, pos, k, v, ks, vs)
    kc, kss = R.quantize_groups(kn)
    for s in range(S):
        for c in range(Lmax):
            i = c - pos[s]
            if 0 <= i < Tn:
                assert np.array_equal(k2[s, c], kc[s, i]) and np.array_equal(ks2[s, c], kss[s, i])
            else:
                assert np.all(k2[s, c] == 9) and np.all(ks2[s, c] == 2.0)
    assert np.all(k == 9)                                # inputs untouched
