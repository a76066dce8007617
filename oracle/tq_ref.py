"""fp64 CPU oracle for decode attention over a TurboQuant-compressed KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or
executes this module; only the tests and the bench's CPU-baseline leg do.  It
shares no code with the HIP library.

What it computes (cera 0.4.0, flash_attention_tq.metal: the header's score
and value formulas, kernel flash_attention_tq, and its epilogue), in the
page's order and notation, for sequence s, query token t, head h (KV head
g = h // (H // Hk)) and every visible cell c of the causal window
(L_t = clamp(seq_lens[s] - (T - 1 - t), 0, Lmax), the window rule of the
other decode paths):

  key codes of (s, g, c):
    norm, residual_norm  = the f16 halves (low, high) of k_norms[s, g, c]
    idx_k[d]             = 2-bit field d % 16 of k_polar[s, g, c, d // 16]
                           (bits 2 (d % 16) and up: lowest field first)
    jl_bit[d]            = bit d % 32 of k_jl[s, g, c, d // 32]
  score (the key is never rebuilt; the query arrives rotated):
    polar_dot   = sum_d q_rot[d] * centroid[idx_k[d]]
    signed_sum  = 2 * sum_{d : jl_bit[d] = 1} q_jl[d] - sum_d q_jl[d]
    correction  = norm * residual_norm * qjl_scale * signed_sum
    score       = (polar_dot * norm + correction) * scale
  softmax over the window's cells (natural exp), p_c
  value, accumulated in the rotated basis:
    vnorm       = f16 low half of v_norms[s, g, c]
    idx_v[d]    = 2-bit field d % 16 of v_polar[s, g, c, d // 16]
    acc[d]      = sum_c p_c * vnorm_c * centroid[idx_v[c, d]]
  epilogue (the inverse randomized Hadamard transform):
    out         = signs * (H_D @ acc) / sqrt(D)
  where H_D is the D x D Walsh-Hadamard matrix in natural (Sylvester) order,
  the matrix the page's butterfly passes apply; an empty window gives 0.

Cache layout, as the page addresses its regions (slot = kv_head * cap + t):
  k_polar, v_polar [S][Hk][Lmax][D/16] uint32;  k_jl [S][Hk][Lmax][D/32]
  uint32;  k_norms, v_norms [S][Hk][Lmax] uint32.

Pinned by tests/test_oracle_tq.py: the Hadamard matrix against
scipy.linalg.hadamard; with a zero residual norm the whole path equals plain
softmax attention (oracle/decode_ref.py) over keys and values decoded and
rotated back to the original basis; the QJL correction is an unbiased
estimate of q . r for Gaussian JL projections (Monte Carlo, a property of the
estimator, not of this code); the scores, two-cell softmax weights and
rotated-back output of hand-built cells with unequal norm * residual norm,
written out in closed form with and without JL bits set (this pins the
-sum(q_jl) term of the signed sum, which the estimator's mean does not see);
field and bit order and the f16 halves against hand-built words; one cell
gives its decoded value; empty windows give 0.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = ["hadamard", "f16_halves", "polar_indices", "jl_bits", "decode_rot",
           "decode_keys", "scores_decoded", "tq_scores", "attend_decoded", "tq_attend",
           "tq_decode_ref"]


def hadamard(D: int) -> np.ndarray:
    """Sylvester Walsh-Hadamard matrix of order D (a power of two), fp64."""
    assert D >= 1 and D & (D - 1) == 0
    H = np.ones((1, 1), dtype=np.float64)
    while H.shape[0] < D:
        H = np.block([[H, H], [H, -H]])
    return H


def f16_halves(words: np.ndarray):
    """uint32 words -> (float64 of the low f16 half, float64 of the high half)."""
    w = np.asarray(words, dtype=np.uint32)
    lo = (w & np.uint32(0xFFFF)).astype(np.uint16).view(np.float16).astype(np.float64)
    hi = (w >> np.uint32(16)).astype(np.uint16).view(np.float16).astype(np.float64)
    return lo, hi


def polar_indices(words: np.ndarray, D: int) -> np.ndarray:
    """[..., D/16] uint32 -> [..., D] 2-bit indices (field k of word w is dim
    16 w + k, at bits 2k and 2k + 1)."""
    w = np.asarray(words, dtype=np.uint32)
    k = np.arange(16, dtype=np.uint32)
    idx = (w[..., :, None] >> (np.uint32(2) * k)) & np.uint32(3)
    return idx.reshape(w.shape[:-1] + (D,)).astype(np.int64)


def jl_bits(words: np.ndarray, D: int) -> np.ndarray:
    """[..., D/32] uint32 -> [..., D] sign bits (bit k of word w is dim 32 w + k)."""
    w = np.asarray(words, dtype=np.uint32)
    k = np.arange(32, dtype=np.uint32)
    b = (w[..., :, None] >> k) & np.uint32(1)
    return b.reshape(w.shape[:-1] + (D,)).astype(np.float64)


def decode_rot(polar_words: np.ndarray, norms: np.ndarray, centroids, D: int) -> np.ndarray:
    """Rotated-basis vectors norm * centroid[idx] of a set of cells:
    [n][D/16] words, [n] norms -> [n][D] fp64."""
    c = np.asarray(centroids, dtype=np.float64)
    return norms[:, None] * c[polar_indices(polar_words, D)]


def decode_keys(k_polar, k_jl, k_norms, centroids, D):
    """The per-cell key terms of n cells: centroid values c[idx_k] [n][D],
    JL bits [n][D] (0 / 1), norm [n] and residual norm [n], fp64."""
    c = np.asarray(centroids, dtype=np.float64)
    norm, residual_norm = f16_halves(k_norms)
    return c[polar_indices(k_polar, D)], jl_bits(k_jl, D), norm, residual_norm


def scores_decoded(q_rot, q_jl, kc, jl, norm, residual_norm, qjl_scale, scale):
    """Scores of one query row against cells given by their decoded key terms
    (decode_keys) -> [n] fp64."""
    q_rot = np.asarray(q_rot, dtype=np.float64)
    q_jl = np.asarray(q_jl, dtype=np.float64)
    polar_dot = kc @ q_rot
    pos_sum = jl @ q_jl
    signed_sum = 2.0 * pos_sum - q_jl.sum()
    correction = norm * residual_norm * float(qjl_scale) * signed_sum
    return (polar_dot * norm + correction) * float(scale)


def tq_scores(q_rot, q_jl, k_polar, k_jl, k_norms, centroids, qjl_scale, scale, D):
    """Scores of one query row against n cells: q_rot, q_jl [D] float;
    k_polar [n][D/16], k_jl [n][D/32], k_norms [n] uint32 -> [n] fp64."""
    return scores_decoded(q_rot, q_jl, *decode_keys(k_polar, k_jl, k_norms, centroids, D),
                          qjl_scale, scale)


def attend_decoded(q_rot, q_jl, keys, v_rot, signs, qjl_scale, scale, D) -> np.ndarray:
    """One query row over cells given by decoded key terms (decode_keys) and
    rotated-basis values v_rot [n][D] -> output [D] fp64 in the original basis."""
    if v_rot.shape[0] == 0:
        return np.zeros(D, dtype=np.float64)
    sc = scores_decoded(q_rot, q_jl, *keys, qjl_scale, scale)
    w = np.exp(sc - sc.max())
    p = w / w.sum()
    acc = p @ v_rot
    return np.asarray(signs, dtype=np.float64) * (hadamard(D) @ acc) / math.sqrt(D)


def tq_attend(q_rot, q_jl, k_polar, k_jl, k_norms, v_polar, v_norms, signs, centroids,
              qjl_scale, scale, D) -> np.ndarray:
    """One query row over n cells -> output [D] fp64 in the original basis."""
    n = k_norms.shape[0]
    if n == 0:
        return np.zeros(D, dtype=np.float64)
    vnorm, _ = f16_halves(v_norms)
    return attend_decoded(q_rot, q_jl, decode_keys(k_polar, k_jl, k_norms, centroids, D),
                          decode_rot(v_polar, vnorm, centroids, D), signs, qjl_scale, scale, D)


def tq_decode_ref(q_rot, q_jl, k_polar, k_jl, k_norms, v_polar, v_norms, seq_lens, signs,
                  centroids, qjl_scale, scale, rows=None) -> np.ndarray:
    """Decode output [S][T][H][D] fp64 (or, with rows = [(s, t, h), ...], the
    listed rows stacked [len(rows)][D]).  q_rot, q_jl [S][T][H][D]; caches as
    in the module docstring; seq_lens [S]; signs [D]; centroids [4].  The
    cells of each (sequence, KV head) are decoded once, over the window of
    its last token; every row reads the prefix its window covers."""
    S, T, H, D = q_rot.shape
    _, Hk, Lmax, _ = k_polar.shape
    G = H // Hk

    def window(s, t):
        Lt = int(seq_lens[s]) - (T - 1 - t)
        return max(0, min(Lt, Lmax))

    def slab(s, g):
        L = window(s, T - 1)
        keys = decode_keys(k_polar[s, g, :L], k_jl[s, g, :L], k_norms[s, g, :L], centroids, D)
        vnorm, _ = f16_halves(v_norms[s, g, :L])
        return keys, decode_rot(v_polar[s, g, :L], vnorm, centroids, D)

    def one(s, t, h, keys, v_rot):
        Lt = window(s, t)
        return attend_decoded(q_rot[s, t, h], q_jl[s, t, h], tuple(x[:Lt] for x in keys),
                              v_rot[:Lt], signs, qjl_scale, scale, D)

    if rows is not None:
        rows = list(rows)
        res = np.zeros((len(rows), D), dtype=np.float64)
        for sg in sorted({(s, h // G) for (s, _, h) in rows}):
            keys, v_rot = slab(*sg)
            for i, (s, t, h) in enumerate(rows):
                if (s, h // G) == sg:
                    res[i] = one(s, t, h, keys, v_rot)
        return res
    out = np.zeros((S, T, H, D), dtype=np.float64)
    for s in range(S):
        for g in range(Hk):
            keys, v_rot = slab(s, g)
            for t in range(T):
                for h in range(g * G, (g + 1) * G):
                    out[s, t, h] = one(s, t, h, keys, v_rot)
    return out
