"""Pins for the fp64 oracle (CPU only).

The source pages print no worked example values, so every pin here is a
closed form, an invariant, a brute-force evaluation, a special case that
reduces to a library routine, or an exhaustive arithmetic fact.  Each is
chosen so that a plausible slip in the oracle (a dropped max subtraction, a
wrong exp base, a missing scale, a wrong GQA head index, a transposed
operand, a wrong int8 scale group, an off-by-one causal window, a wrong
budget width, a wrong merge weight) fails at least one of them.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import decode_ref as R
from workloads import make_case, make_inputs, WORKLOADS


def _case(kv="f16", S=2, T=1, H=8, Hk=2, D=64, Lmax=40, lens=(40, 17), B=0, seed=3, scale=None):
    return make_case(S, T, H, Hk, D, Lmax, list(lens)[:S], kv=kv, budget=B, seed=seed, scale=scale)


def _ref(inp, **kw):
    return R.gqa_decode_ref(inp.q, inp.k, inp.v, inp.seq_lens, inp.scale,
                            inp.k_scales, inp.v_scales, inp.ids if "ids" not in kw else kw["ids"])


# P-1: constant V -> every output row equals that V row (normalisation).
@pytest.mark.parametrize("kv", ["f16", "i8"])
def test_constant_v_gives_v(kv):
    inp = _case(kv=kv)
    if kv == "f16":
        inp.v[...] = inp.v[:, :1, :, :]
        expect = inp.v[:, 0, :, :].astype(np.float64)
    else:
        inp.v[...] = inp.v[:, :1, :, :]
        inp.v_scales[...] = inp.v_scales[:, :1, :, :]
        expect = inp.v[:, 0, :, :].astype(np.float64) * np.repeat(
            inp.v_scales[:, 0, :, :].astype(np.float64), 64, axis=-1)
    out = _ref(inp)
    G = 4
    for s in range(2):
        for h in range(8):
            np.testing.assert_allclose(out[s, 0, h], expect[s, h // G], rtol=0, atol=1e-12)


# P-2: a single visible cell gives exactly its V row; so does a single id.
def test_single_cell_gives_row():
    inp = _case(lens=(1, 1))
    out = _ref(inp)
    for s in range(2):
        for h in range(8):
            assert np.array_equal(out[s, 0, h], inp.v[s, 0, h // 4].astype(np.float64))
    inp = _case(lens=(40, 40), B=1, kv="i8")
    out = _ref(inp)
    for s in range(2):
        c = int(inp.ids[s, 0, 0])
        for h in range(8):
            row = inp.v[s, c, h // 4].astype(np.float64) * np.repeat(
                inp.v_scales[s, c, h // 4].astype(np.float64), 64)
            assert np.array_equal(out[s, 0, h], row)


# P-3: q = 0 (or scale = 0) makes every score equal -> arithmetic mean of the
# visible V rows, checked in exact rational arithmetic.
@pytest.mark.parametrize("zero", ["q", "scale"])
def test_equal_scores_give_mean(zero):
    inp = _case(D=64, lens=(5, 3), Lmax=8, scale=0.0 if zero == "scale" else None)
    if zero == "q":
        inp.q[...] = 0
    out = _ref(inp)
    for s, L in enumerate((5, 3)):
        for h in range(8):
            for d in (0, 17, 63):
                mean = sum(Fraction(float(inp.v[s, c, h // 4, d])) for c in range(L)) / L
                assert out[s, 0, h, d] == pytest.approx(float(mean), abs=1e-15)


# P-4: two cells -> out = sigmoid(s1 - s2) V1 + sigmoid(s2 - s1) V2 with
# natural-base exp and the scale applied to q.k.
def test_two_cells_closed_form():
    inp = _case(H=2, Hk=1, D=64, Lmax=2, lens=(2, 2), scale=0.3)
    out = _ref(inp)
    for s in range(2):
        for h in range(2):
            sc = [0.3 * math.fsum(float(inp.q[s, 0, h, d]) * float(inp.k[s, c, 0, d]) for d in range(64))
                  for c in range(2)]
            a = 1.0 / (1.0 + math.exp(-(sc[0] - sc[1])))
            expect = a * inp.v[s, 0, 0].astype(np.float64) + (1 - a) * inp.v[s, 1, 0].astype(np.float64)
            np.testing.assert_allclose(out[s, 0, h], expect, rtol=0, atol=1e-12)


# Brute force on tiny inputs: nested Python loops over every (s, t, h, d)
# with math.exp, plain and independent of numpy's matrix products.
@pytest.mark.parametrize("kv,B,T", [("f16", 0, 1), ("i8", 0, 3), ("i8", 3, 2), ("f16", 4, 2)])
def test_brute_force_tiny(kv, B, T):
    inp = make_case(2, T, 4, 2, 64, 6, [6, 4], kv=kv, budget=B, seed=11, scale=0.37)
    out = _ref(inp)
    S, T, H, D = inp.q.shape
    for s in range(S):
        for t in range(T):
            Lt = max(0, min(int(inp.seq_lens[s]) - (T - 1 - t), 6))
            cells = list(range(Lt)) if B == 0 else [int(x) for x in inp.ids[s, t, :min(Lt, B)]]
            for h in range(H):
                g = h // (H // 2)

                def elem(arr, sc, c, d):
                    x = float(arr[s, c, g, d])
                    return x * float(sc[s, c, g, d // 64]) if kv == "i8" else x
                scores = [inp.scale * math.fsum(float(inp.q[s, t, h, d]) * elem(inp.k, inp.k_scales, c, d)
                                                for d in range(D)) for c in cells]
                if not cells:
                    assert not out[s, t, h].any()
                    continue
                mx = max(scores)
                w = [math.exp(x - mx) for x in scores]
                tot = math.fsum(w)
                for d in range(D):
                    val = math.fsum(wc * elem(inp.v, inp.v_scales, c, d) for wc, c in zip(w, cells)) / tot
                    assert out[s, t, h, d] == pytest.approx(val, rel=1e-12, abs=1e-14)


# P-5: permuting cells jointly in K and V (or permuting the id list) changes nothing.
def test_permutation_invariance():
    inp = _case(lens=(40, 40))
    base = _ref(inp)
    perm = np.random.default_rng(0).permutation(40)
    inp.k[:] = inp.k[:, perm]
    inp.v[:] = inp.v[:, perm]
    np.testing.assert_allclose(_ref(inp), base, rtol=0, atol=1e-12)
    inp = _case(kv="i8", lens=(40, 40), B=16)
    base = _ref(inp)
    ids = inp.ids.copy()
    ids[:, :, :] = ids[:, :, np.random.default_rng(1).permutation(16)]
    np.testing.assert_allclose(_ref(inp, ids=ids), base, rtol=0, atol=1e-12)


# P-6: split-then-merge equals the unsplit result for several chunk sizes and
# for random ragged splits; an all-empty list gives zeros.
@pytest.mark.parametrize("chunk", [1, 7, 32, 40])
def test_split_then_merge_equals_unsplit(chunk):
    for kv in ("f16", "i8"):
        inp = _case(kv=kv, T=2, lens=(40, 17))
        base = _ref(inp)
        sm = R.split_then_merge(inp.q, inp.k, inp.v, inp.seq_lens, inp.scale, chunk,
                                inp.k_scales, inp.v_scales)
        np.testing.assert_allclose(sm, base, rtol=1e-12, atol=1e-13)


def test_ragged_split_and_empty_partials():
    inp = _case(lens=(40, 40))
    rng = np.random.default_rng(5)
    Kd = R.kv_rows(inp.k, None, 0, 1, np.arange(40))
    Vd = R.kv_rows(inp.v, None, 0, 1, np.arange(40))
    base = R.attend(inp.q[0, 0, 5], Kd, Vd, inp.scale)
    for _ in range(20):
        cuts = sorted(rng.choice(np.arange(1, 40), size=rng.integers(1, 8), replace=False).tolist())
        bounds = [0] + cuts + [40]
        # an empty chunk in the middle contributes nothing
        bounds = bounds[:2] + [bounds[1]] + bounds[2:]
        parts = R.split_partials(inp.q[0, 0, 5], Kd, Vd, inp.scale, bounds)
        got = R.merge_partials([p[0] for p in parts], [p[1] for p in parts], [p[2] for p in parts])
        np.testing.assert_allclose(got, base, rtol=1e-12, atol=1e-13)
    parts = R.split_partials(inp.q[0, 0, 5], Kd[:0], Vd[:0], inp.scale, [0, 0, 0])
    z = R.merge_partials([p[0] for p in parts], [p[1] for p in parts], [p[2] for p in parts])
    assert z.shape == (64,) and not z.any()


def test_merge_weights_closed_form():
    # Two partials with m1 = m2 + ln 2 (as floats): weight of the first is twice.
    o1, o2 = np.ones(4), np.full(4, 3.0)
    m2 = 0.25
    m1 = m2 + math.log(2.0)
    got = R.merge_partials([o1, o2], [m1, m2], [1.0, 1.0])
    e1 = math.exp(m1 - m1)
    e2 = math.exp(m2 - m1)
    np.testing.assert_allclose(got, (e1 * o1 + e2 * o2) / (e1 + e2), rtol=1e-15)
    np.testing.assert_allclose(got, (2 * 1.0 + 3.0) / 3.0 * np.ones(4), rtol=1e-14)


# P-7: GQA -> MHA.  Repeating every KV head G times and running with Hk = H
# gives the same output; a wrong head mapping (h % Hk) would not.
def test_gqa_equals_repeated_mha():
    inp = _case(H=8, Hk=2, lens=(40, 23))
    base = _ref(inp)
    k_rep = np.repeat(inp.k, 4, axis=2)
    v_rep = np.repeat(inp.v, 4, axis=2)
    mha = R.gqa_decode_ref(inp.q, k_rep, v_rep, inp.seq_lens, inp.scale)
    np.testing.assert_allclose(mha, base, rtol=0, atol=1e-13)


# P-8: library cross-check against torch's scaled_dot_product_attention on the
# CPU in float64 (repeated KV heads, boolean mask for the causal windows).
@pytest.mark.parametrize("kv,T", [("f16", 1), ("f16", 3), ("i8", 2)])
def test_against_torch_sdpa(kv, T):
    inp = make_case(3, T, 12, 3, 128 if kv == "f16" else 64, 50, [50, 31, 2], kv=kv, seed=7)
    out = _ref(inp)
    S, T, H, D = inp.q.shape
    G = H // 3
    for s in range(S):
        if kv == "i8":
            Kd = R.dequant_i8(inp.k[s], inp.k_scales[s])
            Vd = R.dequant_i8(inp.v[s], inp.v_scales[s])
        else:
            Kd = inp.k[s].astype(np.float64)
            Vd = inp.v[s].astype(np.float64)
        kt = torch.from_numpy(Kd).permute(1, 0, 2).repeat_interleave(G, dim=0)  # [H][Lmax][D]
        vt = torch.from_numpy(Vd).permute(1, 0, 2).repeat_interleave(G, dim=0)
        qt = torch.from_numpy(inp.q[s].astype(np.float64)).permute(1, 0, 2)       # [H][T][D]
        pos = torch.arange(50)
        lens = torch.tensor([int(inp.seq_lens[s]) - (T - 1 - t) for t in range(T)])
        mask = pos[None, :] < lens[:, None]                                           # [T][Lmax]
        res = torch.nn.functional.scaled_dot_product_attention(
            qt, kt, vt, attn_mask=mask[None], scale=inp.scale).permute(1, 0, 2).numpy()
        for t in range(T):
            if lens[t] <= 0:
                assert not out[s, t].any()
            else:
                np.testing.assert_allclose(out[s, t], res[t], rtol=1e-10, atol=1e-12)


# P-9: ids = arange(L) equals dense; a subset of ids equals dense attention over
# the gathered rows; a budget wider than the window uses only min(L_t, B) ids.
def test_ids_identity_and_subset():
    inp = _case(kv="i8", lens=(40, 17))
    base = _ref(inp)
    ids = np.zeros((2, 1, 64), dtype=np.int32)
    ids[0, 0, :40] = np.arange(40)
    ids[1, 0, :17] = np.arange(17)
    ids[1, 0, 17:] = 5   # beyond min(L_t, B) = 17: must never be read
    np.testing.assert_allclose(_ref(inp, ids=ids), base, rtol=0, atol=1e-13)
    sub = np.array([3, 11, 12, 30], dtype=np.int32)
    ids2 = np.broadcast_to(sub, (2, 1, 4)).copy()
    got = _ref(inp, ids=ids2)
    for s in range(2):
        cells = sub[sub < [40, 17][s]]
        if s == 1:
            # width = min(17, 4) = 4: all four ids are read, even id 30 >= L_t is
            # a caller precondition violation; the oracle reads it as given.
            cells = sub
        for h in range(8):
            Kd = R.dequant_i8(inp.k[s, cells, h // 4], inp.k_scales[s, cells, h // 4])
            Vd = R.dequant_i8(inp.v[s, cells, h // 4], inp.v_scales[s, cells, h // 4])
            np.testing.assert_allclose(got[s, 0, h], R.attend(inp.q[s, 0, h], Kd, Vd, inp.scale),
                                       rtol=0, atol=1e-13)


# P-10: int8 dequantisation.  float32(i) * float32(s) equals the fp64 product
# for every int8 code and every finite positive binary16 scale, so an fp32
# kernel and the fp64 oracle define every element identically.  Plus a hand
# example and the 64-element grouping.
def test_int8_dequant_exact_in_fp32_exhaustive():
    codes = np.arange(-128, 128, dtype=np.float64)
    bits = np.arange(1, 0x7C00, dtype=np.uint16)          # +subnormals .. max finite
    sc = bits.view(np.float16)
    p64 = codes[:, None] * sc.astype(np.float64)[None, :]
    p32 = codes.astype(np.float32)[:, None] * sc.astype(np.float32)[None, :]
    assert np.array_equal(p32.astype(np.float64), p64)


def test_int8_dequant_grouping():
    codes = np.arange(256, dtype=np.int64) % 255 - 127
    codes = codes.astype(np.int8)
    scales = np.array([0.5, 0.25, 2.0, 0.125], dtype=np.float16)
    d = R.dequant_i8(codes, scales)
    for i in (0, 63, 64, 127, 128, 200, 255):
        assert d[i] == float(codes[i]) * [0.5, 0.25, 2.0, 0.125][i // 64]
    # a hand value: -127 * f16(0.0125) = -127 * 0.0124969482421875
    assert R.dequant_i8(np.array([-127] * 64, np.int8), np.array([0.0125], np.float16))[5] == \
        -127 * 0.0124969482421875


def test_int8_path_equals_dense_on_dequantised_rows():
    inp = _case(kv="i8", T=2, lens=(40, 9))
    out = _ref(inp)
    Kd = R.dequant_i8(inp.k, inp.k_scales)
    Vd = R.dequant_i8(inp.v, inp.v_scales)
    dense = R.gqa_decode_ref(inp.q, Kd, Vd, inp.seq_lens, inp.scale)
    np.testing.assert_allclose(out, dense, rtol=0, atol=1e-14)


# P-11: token t of a T-token causal window equals a single-query decode over
# its own L_t = seq_len - (T - 1 - t) cells; the count itself is pinned by
# one-hot V rows with equal scores.
def test_causal_window_equals_single_query():
    inp = _case(T=4, lens=(40, 2))
    out = _ref(inp)
    for s in range(2):
        for t in range(4):
            Lt = int(inp.seq_lens[s]) - (3 - t)
            single = R.gqa_decode_ref(inp.q[s:s + 1, t:t + 1], inp.k[s:s + 1], inp.v[s:s + 1],
                                      np.array([Lt]), inp.scale)
            np.testing.assert_allclose(out[s, t], single[0, 0], rtol=0, atol=1e-13)
    # counts: q = 0 and V[c] = c in dim 0 -> out = mean(0..L_t-1) = (L_t - 1) / 2
    inp = _case(T=4, D=64, Lmax=40, lens=(40, 2))
    inp.q[...] = 0
    inp.v[...] = 0
    inp.v[:, :, :, 0] = np.arange(40, dtype=np.float16)[None, :, None]
    out = _ref(inp)
    for s, L in enumerate((40, 2)):
        for t in range(4):
            Lt = L - (3 - t)
            want = (Lt - 1) / 2 if Lt > 0 else 0.0
            assert out[s, t, 0, 0] == pytest.approx(want, abs=1e-13)


# P-12: very large scores stay finite and tend to the V row of the argmax score.
def test_large_scores_hardmax():
    inp = _case(lens=(40, 40), scale=1e3)
    out = _ref(inp)
    assert np.isfinite(out).all()
    for s in range(2):
        for h in range(8):
            g = h // 4
            sc = inp.k[s, :40, g].astype(np.float64) @ inp.q[s, 0, h].astype(np.float64)
            top = np.argsort(sc)[-2:]
            if (sc[top[1]] - sc[top[0]]) * 1e3 > 50:
                np.testing.assert_allclose(out[s, 0, h], inp.v[s, top[1], g].astype(np.float64),
                                           rtol=0, atol=1e-12)


# P-13: an empty window (L = 0, or a token before the start of the cache) is zero.
def test_empty_window_zero():
    inp = _case(T=3, lens=(0, 1))
    out = _ref(inp)
    assert not out[0].any()
    assert not out[1, 0].any() and not out[1, 1].any() and out[1, 2].any()
    inp = _case(kv="i8", lens=(0, 3), B=8)
    assert not _ref(inp)[0].any()


def test_visible_len_rule():
    assert R.visible_len(131072, 8, 0, 131072) == 131065
    assert R.visible_len(131072, 8, 7, 131072) == 131072
    assert R.visible_len(5, 8, 0, 100) == 0
    assert R.visible_len(500, 1, 0, 100) == 100


def test_rows_variant_matches_full():
    inp = _case(kv="i8", T=2, lens=(40, 11), B=0)
    full = _ref(inp)
    rows = [(0, 0, 3), (1, 1, 7), (0, 1, 0), (1, 0, 4)]
    got = R.gqa_decode_ref_rows(inp.q, inp.k, inp.v, inp.seq_lens, inp.scale, rows,
                                inp.k_scales, inp.v_scales)
    for i, (s, t, h) in enumerate(rows):
        assert np.array_equal(got[i], full[s, t, h])
    inp = _case(kv="i8", T=2, lens=(40, 11), B=6)
    full = _ref(inp)
    got = R.gqa_decode_ref_rows(inp.q, inp.k, inp.v, inp.seq_lens, inp.scale, rows,
                                inp.k_scales, inp.v_scales, inp.ids)
    for i, (s, t, h) in enumerate(rows):
        assert np.array_equal(got[i], full[s, t, h])


def test_tiny_workload_runs():
    inp = make_inputs("tiny_f16")
    out = _ref(inp)
    assert out.shape == (1, 1, 8, 64) and np.isfinite(out).all()
    sm = R.split_then_merge(inp.q, inp.k, inp.v, inp.seq_lens, inp.scale, 32)
    np.testing.assert_allclose(sm, out, rtol=1e-12, atol=1e-13)
