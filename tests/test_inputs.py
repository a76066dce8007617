"""Seeded generators: deterministic, the right shapes, dtypes and ranges, and
the algorithmic byte counts the measurements use."""
import numpy as np
import pytest

from workloads import make_case, make_inputs, kv_bytes, WORKLOADS


def test_deterministic():
    a = make_case(2, 2, 8, 2, 64, 33, [33, 5], kv="i8", budget=7, seed=9)
    b = make_case(2, 2, 8, 2, 64, 33, [33, 5], kv="i8", budget=7, seed=9)
    for x, y in [(a.q, b.q), (a.k, b.k), (a.v, b.v), (a.k_scales, b.k_scales), (a.ids, b.ids)]:
        assert np.array_equal(x, y)
    c = make_case(2, 2, 8, 2, 64, 33, [33, 5], kv="i8", budget=7, seed=10)
    assert not np.array_equal(a.q, c.q)


def test_value_ranges_and_ids():
    a = make_case(3, 2, 4, 1, 128, 300, [300, 40, 1], kv="i8", budget=64, seed=1)
    assert a.k.dtype == np.int8 and a.k.min() >= -127 and a.k.max() <= 127
    s = a.k_scales.astype(np.float32)
    assert a.k_scales.dtype == np.float16 and s.min() >= 0.0049 and s.max() <= 0.0201
    assert a.q.dtype == np.float32 and a.q.shape == (3, 2, 4, 128)
    for si, L in enumerate([300, 40, 1]):
        for t in range(2):
            Lt = max(0, L - (1 - t))
            w = min(Lt, 64)
            row = a.ids[si, t, :w]
            assert len(set(row.tolist())) == w
            assert (row >= 0).all() and (row < max(Lt, 1)).all()
            assert (np.diff(row) > 0).all()


def test_workload_shapes_and_bytes():
    tiny = make_inputs("tiny_f16")
    assert tiny.q.shape == (1, 1, 8, 64) and tiny.k.shape == (1, 256, 2, 64)
    assert kv_bytes(tiny) == 131072


@pytest.mark.parametrize("name,expect", [("i8_32k", 276824064), ("i8_budget", 17367040),
                                         ("f16_mq_causal", 2147483648)])
def test_large_workload_bytes_formula(name, expect):
    # Byte counts from the shapes alone (no tensors drawn): K + V (+ scales) per
    # visible cell and KV head, ids 4 B per budget entry.
    w = WORKLOADS[name]
    row = w.D * (1 if w.kv == "i8" else 2) + (w.D // 64 * 2 if w.kv == "i8" else 0)
    cells = w.budget if w.budget else w.Lmax
    total = w.S * 2 * row * w.Hk * cells + (4 * w.S * w.budget if w.budget else 0)
    assert total == expect


def test_f16_batch_lengths():
    from workloads import workload_seq_lens
    w = WORKLOADS["f16_batch"]
    lens = workload_seq_lens(w, np.random.SeedSequence(1000 + w.index).spawn(2)[0])
    assert lens.shape == (32,) and lens.min() >= 512 and lens.max() <= 4096
