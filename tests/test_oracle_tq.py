"""Pins of the TurboQuant decode oracle (oracle/tq_ref.py), CPU only.

The page prints no worked values, so the pins are: the Hadamard matrix
against scipy's; the whole path against plain softmax attention (the
separately pinned oracle/decode_ref.py) over keys and values decoded and
rotated back to the original basis by code written here (a different bit
unpacking and scipy's Hadamard), which holds exactly when the residual norm
is zero because the rotation is orthogonal; the QJL correction against the
unbiasedness of the QJL estimator for Gaussian projections (Monte Carlo);
the field / bit order and the f16 halves against hand-built words; one cell;
empty windows; and the scores and two-cell softmax of hand-built cells in
closed form, which is what pins the -sum(q_jl) term of the signed sum."""
import math

import numpy as np
import pytest
import scipy.linalg

from oracle import decode_ref as DR
from oracle import tq_ref as R
from workloads import make_tq_case


# ------------------------------------------------------------------ helpers
# (an independent unpacking: numpy's little-endian bit order on the bytes)
def unpack_fields(words: np.ndarray, D: int) -> np.ndarray:
    b = np.unpackbits(np.ascontiguousarray(words).view(np.uint8), axis=-1, bitorder="little")
    b = b.reshape(words.shape[:-1] + (D, 2)).astype(np.int64)
    return b[..., 0] + 2 * b[..., 1]


def unpack_bits(words: np.ndarray, D: int) -> np.ndarray:
    b = np.unpackbits(np.ascontiguousarray(words).view(np.uint8), axis=-1, bitorder="little")
    return b.reshape(words.shape[:-1] + (D,)).astype(np.float64)


def low_half(words):
    return (words & 0xFFFF).astype(np.uint16).view(np.float16).astype(np.float64)


def to_original_basis(x_rot: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """Inverse randomized Hadamard rotation of rows: signs * (H x) / sqrt(D)."""
    D = x_rot.shape[-1]
    H = scipy.linalg.hadamard(D).astype(np.float64)
    return (x_rot @ H.T) / math.sqrt(D) * signs.astype(np.float64)


# ------------------------------------------------------------------ pins
@pytest.mark.parametrize("D", [1, 2, 4, 32, 64, 128])
def test_hadamard_against_scipy(D):
    H = R.hadamard(D)
    assert np.array_equal(H, scipy.linalg.hadamard(D).astype(np.float64))
    np.testing.assert_array_equal(H @ H.T, D * np.eye(D))


def test_field_bit_order_and_f16_halves():
    D = 32
    polar = np.zeros((1, 2), dtype=np.uint32)
    polar[0, 0] = np.uint32(3) << np.uint32(10)        # field 5 of word 0 -> dim 5
    polar[0, 1] = np.uint32(2) << np.uint32(30)        # field 15 of word 1 -> dim 31
    idx = R.polar_indices(polar, D)[0]
    expect = np.zeros(D, dtype=np.int64)
    expect[5], expect[31] = 3, 2
    assert np.array_equal(idx, expect)
    jl = np.array([[1 << 7]], dtype=np.uint32)
    b = R.jl_bits(jl, D)[0]
    assert b[7] == 1 and b.sum() == 1
    w = np.array([np.float16(1.5).view(np.uint16) | (np.uint32(np.float16(0.25).view(np.uint16)) << 16)],
                 dtype=np.uint32)
    lo, hi = R.f16_halves(w)
    assert lo[0] == 1.5 and hi[0] == 0.25
    # against the independent unpacking on random words
    rng = np.random.default_rng(0)
    wr = rng.integers(0, 2**32, size=(5, 8), dtype=np.uint64).astype(np.uint32)
    assert np.array_equal(R.polar_indices(wr, 128), unpack_fields(wr, 128))
    assert np.array_equal(R.jl_bits(wr[:, :4], 128), unpack_bits(wr[:, :4], 128))


@pytest.mark.parametrize("T,lens", [(1, [60, 17, 0]), (3, [60, 2, 1])])
@pytest.mark.parametrize("D", [32, 64, 128])
def test_zero_residual_equals_plain_attention_in_original_basis(D, T, lens):
    S, H, Hk, Lmax = 3, 8, 2, 60
    inp = make_tq_case(S, T, H, Hk, D, Lmax, lens, seed=D + T)
    k_norms = inp.k_norms & np.uint32(0xFFFF)           # residual norm 0: no QJL term
    got = R.tq_decode_ref(inp.q_rot, inp.q_jl, inp.k_polar, inp.k_jl, k_norms, inp.v_polar,
                          inp.v_norms, inp.seq_lens, inp.signs, inp.centroids, inp.qjl_scale,
                          inp.scale)
    c = np.asarray(inp.centroids, dtype=np.float64)
    k_rot = low_half(k_norms)[..., None] * c[unpack_fields(inp.k_polar, D)]   # [S][Hk][Lmax][D]
    v_rot = low_half(inp.v_norms)[..., None] * c[unpack_fields(inp.v_polar, D)]
    k_orig = to_original_basis(k_rot, inp.signs).transpose(0, 2, 1, 3)          # [S][Lmax][Hk][D]
    v_orig = to_original_basis(v_rot, inp.signs).transpose(0, 2, 1, 3)
    # q . k is rotation invariant: the original-basis query is the inverse
    # rotation of q_rot
    q_orig = to_original_basis(inp.q_rot.astype(np.float64), inp.signs)
    ref = DR.gqa_decode_ref(q_orig, k_orig, v_orig, inp.seq_lens, inp.scale)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_qjl_correction_is_unbiased():
    # QJL: for s_i ~ N(0, I), E[(s_i . q) sign(s_i . r)] = sqrt(2/pi) q.r/|r|, so
    # sqrt(pi/2)/m * |r| * sum_i (S q)_i sign((S r)_i) estimates q . r
    D, trials = 64, 3000
    rng = np.random.default_rng(7)
    q = rng.standard_normal(D)
    r = rng.standard_normal(D)
    r /= np.linalg.norm(r)                              # |r| = 1 is exact in f16
    norms = np.array([np.float16(1.0).view(np.uint16) | (np.uint32(np.float16(1.0).view(np.uint16)) << 16)],
                     dtype=np.uint32)
    polar = np.zeros((1, D // 16), dtype=np.uint32)
    est = np.empty(trials)
    for i in range(trials):
        Smat = rng.standard_normal((D, D))
        bits = (Smat @ r > 0).astype(np.uint8)
        jl = np.packbits(bits, bitorder="little").view(np.uint32)[None, :]
        est[i] = R.tq_scores(np.zeros(D), Smat @ q, polar, jl, norms, (0.0, 0.0, 0.0, 0.0),
                             math.sqrt(math.pi / 2) / D, 1.0, D)[0]
    mean, sem = est.mean(), est.std(ddof=1) / math.sqrt(trials)
    assert abs(mean - q @ r) < 4.0 * sem, (mean, q @ r, sem)
    assert sem < 0.1 * abs(q @ r) + 0.05


def test_single_cell_gives_its_decoded_value():
    D = 64
    inp = make_tq_case(1, 1, 4, 1, D, 8, [1], seed=3)
    out = R.tq_decode_ref(inp.q_rot, inp.q_jl, inp.k_polar, inp.k_jl, inp.k_norms, inp.v_polar,
                          inp.v_norms, inp.seq_lens, inp.signs, inp.centroids, inp.qjl_scale,
                          inp.scale)
    # rotate the output forward (H (signs * out) / sqrt(D)): the cell's codes come back
    H = scipy.linalg.hadamard(D).astype(np.float64)
    back = (out[0, 0] * inp.signs) @ H.T / math.sqrt(D)
    c = np.asarray(inp.centroids, dtype=np.float64)
    expect = low_half(inp.v_norms[0, 0, :1])[0] * c[unpack_fields(inp.v_polar[0, 0, :1], D)[0]]
    for h in range(4):
        np.testing.assert_allclose(back[h], expect, rtol=0, atol=1e-12)


def test_empty_windows_and_rows_variant():
    inp = make_tq_case(2, 2, 8, 2, 64, 30, [30, 1], seed=5)
    full = R.tq_decode_ref(inp.q_rot, inp.q_jl, inp.k_polar, inp.k_jl, inp.k_norms, inp.v_polar,
                           inp.v_norms, inp.seq_lens, inp.signs, inp.centroids, inp.qjl_scale,
                           inp.scale)
    assert not full[1, 0].any() and full[1, 1].any()    # token 0 of sequence 1 sees nothing
    rows = [(0, 1, 7), (1, 0, 3), (1, 1, 0)]
    part = R.tq_decode_ref(inp.q_rot, inp.q_jl, inp.k_polar, inp.k_jl, inp.k_norms, inp.v_polar,
                           inp.v_norms, inp.seq_lens, inp.signs, inp.centroids, inp.qjl_scale,
                           inp.scale, rows=rows)
    for i, (s, t, h) in enumerate(rows):
        assert np.array_equal(part[i], full[s, t, h])


def test_residual_term_moves_scores_by_the_formula_scale():
    # two cells with identical polar codes and norms: only the JL bits differ, so
    # the softmax weight ratio is exp(score difference), and with one extra set
    # bit on dim d the difference is 2 * norm * rnorm * qjl_scale * scale * q_jl[d]
    D = 32
    inp = make_tq_case(1, 1, 1, 1, D, 2, [2], seed=9)
    inp.k_polar[0, 0, 1] = inp.k_polar[0, 0, 0]
    inp.k_norms[0, 0, 1] = inp.k_norms[0, 0, 0]
    inp.k_jl[0, 0, 0] = 0
    inp.k_jl[0, 0, 1] = 1 << 11
    sc = R.tq_scores(inp.q_rot[0, 0, 0], inp.q_jl[0, 0, 0], inp.k_polar[0, 0], inp.k_jl[0, 0],
                     inp.k_norms[0, 0], inp.centroids, inp.qjl_scale, inp.scale, D)
    n, rn = float(low_half(inp.k_norms[0, 0, :1])[0]), float(np.float16(
        (inp.k_norms[0, 0, 0] >> 16).astype(np.uint16).view(np.float16)))
    expect = 2.0 * n * rn * inp.qjl_scale * inp.scale * float(inp.q_jl[0, 0, 0, 11])
    assert abs((sc[1] - sc[0]) - expect) <= 1e-12 * (1 + abs(expect))


def _words_all_fields(index: int, D: int) -> np.ndarray:
    """D/16 polar words whose every 2-bit field holds `index`."""
    w = 0
    for k in range(16):
        w |= index << (2 * k)
    return np.full(D // 16, w, dtype=np.uint32)


def _norm_word(norm: float, residual: float) -> np.uint32:
    return np.uint32(int(np.float16(norm).view(np.uint16)) |
                     (int(np.float16(residual).view(np.uint16)) << 16))


def test_scores_and_two_cell_softmax_in_closed_form():
    # Two cells whose polar fields all hold one index (so the polar dot is
    # that centroid times sum(q_rot)), with unequal norm * residual norm.  With
    # no JL bit set the page's signed sum is -sum(q_jl); with the bits of a set
    # A set it is sum_A q_jl - sum_(not A) q_jl.  The scores, the two-cell
    # softmax weights and the rotated-back output are written out here from
    # those closed forms with the math module; every quantity is exact in f16.
    D = 32
    cent = (-0.25, -0.125, 0.125, 0.25)
    scale, qjl_scale = 0.5, 0.0625
    q_rot = np.array([0.25 if d % 2 == 0 else -0.125 for d in range(D)])
    q_jl = np.array([0.5 + 0.125 * d for d in range(D)])
    norms = [(1.0, 0.5), (0.75, 0.25)]
    k_norms = np.array([_norm_word(*n) for n in norms], dtype=np.uint32)
    k_polar = np.stack([_words_all_fields(3, D), _words_all_fields(1, D)])
    setA = [0, 5, 17, 31]
    for bits in (None, setA):
        k_jl = np.zeros((2, 1), dtype=np.uint32)
        if bits is not None:
            k_jl[1, 0] = sum(1 << d for d in bits)
        sc = R.tq_scores(q_rot, q_jl, k_polar, k_jl, k_norms, cent, qjl_scale, scale, D)
        sum_rot, sum_jl = math.fsum(q_rot), math.fsum(q_jl)
        sgn = [-sum_jl, -sum_jl]
        if bits is not None:
            in_a = math.fsum(q_jl[d] for d in bits)
            sgn[1] = in_a - (sum_jl - in_a)
        for c, (idx, (n, rn)) in enumerate(zip((3, 1), norms)):
            expect = scale * (n * cent[idx] * sum_rot + n * rn * qjl_scale * sgn[c])
            assert abs(sc[c] - expect) <= 1e-13 * (1 + abs(expect)), (bits, c, sc[c], expect)
        # two-cell attention: weights are the logistic of the score difference,
        # values are constant vectors vnorm * centroid, and the Sylvester
        # Hadamard matrix maps a constant vector a * 1 to a * D * e_0
        vnorm = (1.5, 0.5)
        v_polar = np.stack([_words_all_fields(0, D), _words_all_fields(2, D)])
        v_norms = np.array([np.float16(x).view(np.uint16) for x in vnorm], dtype=np.uint32)
        signs = np.array([-1.0] + [1.0] * (D - 1))
        out = R.tq_attend(q_rot, q_jl, k_polar, k_jl, k_norms, v_polar, v_norms, signs, cent,
                          qjl_scale, scale, D)
        s0 = scale * (norms[0][0] * cent[3] * sum_rot + norms[0][0] * norms[0][1] * qjl_scale * sgn[0])
        s1 = scale * (norms[1][0] * cent[1] * sum_rot + norms[1][0] * norms[1][1] * qjl_scale * sgn[1])
        p0 = 1.0 / (1.0 + math.exp(s1 - s0))
        a = p0 * vnorm[0] * cent[0] + (1.0 - p0) * vnorm[1] * cent[2]
        expect_out = np.zeros(D)
        expect_out[0] = -a * D / math.sqrt(D)
        np.testing.assert_allclose(out, expect_out, rtol=0, atol=1e-13)
        # the term moves the weights: with it dropped the softmax would differ
        assert abs(norms[0][0] * norms[0][1] - norms[1][0] * norms[1][1]) > 0.1


def test_decode_ref_rows_equal_single_row_attention_over_their_windows():
    # tq_decode_ref decodes each (sequence, KV head) once over the last
    # token's window; every row must equal tq_attend over exactly the cells
    # of its own causal window, sliced here by hand
    S, T, H, Hk, D, Lmax = 2, 3, 6, 2, 64, 40
    inp = make_tq_case(S, T, H, Hk, D, Lmax, [40, 2], seed=21)
    full = R.tq_decode_ref(inp.q_rot, inp.q_jl, inp.k_polar, inp.k_jl, inp.k_norms, inp.v_polar,
                           inp.v_norms, inp.seq_lens, inp.signs, inp.centroids, inp.qjl_scale,
                           inp.scale)
    G = H // Hk
    for s in range(S):
        for t in range(T):
            n = max(0, min(int(inp.seq_lens[s]) - (T - 1 - t), Lmax))
            for h in range(H):
                g = h // G
                one = R.tq_attend(inp.q_rot[s, t, h], inp.q_jl[s, t, h], inp.k_polar[s, g, :n],
                                  inp.k_jl[s, g, :n], inp.k_norms[s, g, :n], inp.v_polar[s, g, :n],
                                  inp.v_norms[s, g, :n], inp.signs, inp.centroids, inp.qjl_scale,
                                  inp.scale, D)
                assert np.array_equal(full[s, t, h], one), (s, t, h)
    rows = [(1, 0, 5), (0, 2, 0), (1, 2, 3)]
    part = R.tq_decode_ref(inp.q_rot, inp.q_jl, inp.k_polar, inp.k_jl, inp.k_norms, inp.v_polar,
                           inp.v_norms, inp.seq_lens, inp.signs, inp.centroids, inp.qjl_scale,
                           inp.scale, rows=rows)
    for i, (s, t, h) in enumerate(rows):
        assert np.array_equal(part[i], full[s, t, h])
