"""fp64 CPU oracle for split-KV grouped-query decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or
executes this module; only the tests, the graft smoke check and the bench's
CPU-baseline leg do.  It shares no code with the HIP library.

What it computes (the definition every source page's kernels approximate):

  For sequence s, query token t and query head h:
    g      = h // (H // Hk)                         GQA head mapping
    L_t    = clamp(seq_lens[s] - (T - 1 - t), 0, Lmax)
                                                    causal window of token t
    cells  = [0, L_t)                 (dense)
           = ids[s, t, :min(L_t, B)]  (budgeted gather)
    K[c]   = float64(k[s, c, g, :])                 f16 cache
           = float64(int8) * float64(f16 scale[s, c, g, d // 64])
                                                    int8 cache
    score  = scale * sum_d q[s,t,h,d] * K[c, d]
    out    = sum_c exp(score_c - max score) V[c] / sum_c exp(score_c - max score)
    out    = 0 when `cells` is empty.

Sources (page title, then the part of the page):
  * GQA head mapping kv_head = head / (n_heads / n_kv_heads): cera
    attention_gqa.metal (kernel attention_gqa, setup) and cera
    flash_attention_tq.metal (header comment, "GQA").
  * Normalised softmax over the visible cells, followed by P.V: cera
    attention_gqa.metal, Phase 2 and Phase 3.
  * int8 element = float(int8) * float(f16 scale of its 64-element group):
    qsa2.metal, kernels qsa_attn2 (K and V loads) and qsa_attn3 (raw int8
    dot per 64-element group, then the group scale).
  * Budget of cell ids, width = min(n_kv, QBUDGET), row = id * QKV + kv head:
    qsa2.metal, kernel qsa_attn2 (setup and chunk ids).
  * Causal window of query t at pos0 + t sees [0, pos0 + t], clamped so bad
    parameters can only truncate: cera flash_attention_tq.metal (kernel
    flash_attention_tq, "Per-query causal window").
  * Empty window writes zeros: cera flash_attention.metal
    (flash_attention_impl, defensive early returns) and
    flash_attention_tq.metal (seq_len == 0 branch).
  * Chunk partials (unnormalised o, m, l) from a chunk-local softmax and
    their log-sum-exp merge: qsa2.metal, kernels qsa_attn2 (softmax and
    partial write) and qsa_merge2.

The softmax is natural-base exp (qsa2.metal and the cera shaders use exp;
the FORWARD_MSL page's exp2 form carries log2(e) in its scale).

Every function here is pinned by tests/test_oracle.py against closed forms,
invariants, brute force and a library attention routine; none is "parity
unpinned".
"""
from __future__ import annotations

import math
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "visible_len", "cell_list", "dequant_i8", "kv_rows", "attend",
    "gqa_decode_ref", "gqa_decode_ref_rows", "partial_over_cells", "merge_partials",
    "split_partials", "split_then_merge",
]


# --------------------------------------------------------------------------
# index rules
# --------------------------------------------------------------------------

def visible_len(seq_len: int, T: int, t: int, Lmax: int) -> int:
    """Cells visible to query token t of a T-token window whose last token
    sees `seq_len` cells: token t sits at position seq_len - T + t and sees
    [0, that position]; the count is clamped to [0, Lmax] (causal clamp of
    flash_attention_tq.metal, which only ever truncates the window)."""
    Lt = int(seq_len) - (T - 1 - t)
    return max(0, min(Lt, int(Lmax)))


def cell_list(seq_len: int, T: int, t: int, Lmax: int,
              ids_row: Optional[np.ndarray]) -> np.ndarray:
    """Cells token t attends: [0, L_t) dense, or the first min(L_t, B) entries
    of its id list (qsa2.metal: width = min(n_kv, QBUDGET))."""
    Lt = visible_len(seq_len, T, t, Lmax)
    if ids_row is None:
        return np.arange(Lt, dtype=np.int64)
    width = min(Lt, ids_row.shape[0])
    return np.asarray(ids_row[:width], dtype=np.int64)


def dequant_i8(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """float64(int8) * float64(f16 scale) with one scale per 64 consecutive
    elements of a row (qsa2.metal, qsa_attn2 / qsa_attn3).  codes [..., D],
    scales [..., D // 64]."""
    D = codes.shape[-1]
    assert scales.shape[-1] * 64 == D
    s = np.repeat(scales.astype(np.float64), 64, axis=-1)
    return codes.astype(np.float64) * s


def kv_rows(k: np.ndarray, k_scales: Optional[np.ndarray], s: int, g: int,
            cells: np.ndarray) -> np.ndarray:
    """fp64 rows [len(cells)][D] of one KV head of sequence s."""
    rows = k[s, cells, g, :]
    if k.dtype == np.int8:
        return dequant_i8(rows, k_scales[s, cells, g, :])
    return rows.astype(np.float64)


# --------------------------------------------------------------------------
# the definition
# --------------------------------------------------------------------------

def attend(qrow: np.ndarray, Kd: np.ndarray, Vd: np.ndarray, scale: float) -> np.ndarray:
    """Normalised softmax attention of one query row over fp64 rows Kd, Vd
    (cera attention_gqa.metal, Phases 1-3).  Zero rows -> zero output."""
    D = Vd.shape[1] if Vd.ndim == 2 else qrow.shape[0]
    if Kd.shape[0] == 0:
        return np.zeros(D, dtype=np.float64)
    sc = float(scale) * (Kd @ qrow.astype(np.float64))
    w = np.exp(sc - sc.max())
    return (w @ Vd) / w.sum()


def gqa_decode_ref(q: np.ndarray, k: np.ndarray, v: np.ndarray, seq_lens: np.ndarray,
                   scale: float, k_scales: Optional[np.ndarray] = None,
                   v_scales: Optional[np.ndarray] = None,
                   ids: Optional[np.ndarray] = None) -> np.ndarray:
    """Full output [S][T][H][D] in fp64.

    Per (s, g) the rows of the KV head are converted to fp64 once and every
    query row of the group reads the prefix / gather it is entitled to."""
    S, T, H, D = q.shape
    _, Lmax, Hk, _ = k.shape
    assert H % Hk == 0
    G = H // Hk
    out = np.zeros((S, T, H, D), dtype=np.float64)
    for s in range(S):
        for g in range(Hk):
            if ids is None:
                Lfull = visible_len(seq_lens[s], T, T - 1, Lmax)
                allc = np.arange(Lfull, dtype=np.int64)
                Kall = kv_rows(k, k_scales, s, g, allc)
                Vall = kv_rows(v, v_scales, s, g, allc)
            for t in range(T):
                if ids is None:
                    Lt = visible_len(seq_lens[s], T, t, Lmax)
                    Kd, Vd = Kall[:Lt], Vall[:Lt]
                else:
                    cells = cell_list(seq_lens[s], T, t, Lmax, ids[s, t])
                    Kd = kv_rows(k, k_scales, s, g, cells)
                    Vd = kv_rows(v, v_scales, s, g, cells)
                for h in range(g * G, (g + 1) * G):
                    out[s, t, h] = attend(q[s, t, h], Kd, Vd, scale)
    return out


def gqa_decode_ref_rows(q, k, v, seq_lens, scale, rows: Iterable[Tuple[int, int, int]],
                        k_scales=None, v_scales=None, ids=None) -> np.ndarray:
    """The same definition for a chosen set of output rows (s, t, h) only:
    used to check sampled outputs at sizes where the whole output would take
    the CPU too long.  Returns [len(rows)][D] fp64."""
    S, T, H, D = q.shape
    _, Lmax, Hk, _ = k.shape
    G = H // Hk
    res = []
    cache = {}
    for (s, t, h) in rows:
        g = h // G
        cells = cell_list(seq_lens[s], T, t, Lmax, None if ids is None else ids[s, t])
        if ids is None:
            kk = (s, g)
            if kk not in cache:
                cache.clear()
                Lfull = visible_len(seq_lens[s], T, T - 1, Lmax)
                allc = np.arange(Lfull, dtype=np.int64)
                cache[kk] = (kv_rows(k, k_scales, s, g, allc), kv_rows(v, v_scales, s, g, allc))
            Kall, Vall = cache[kk]
            Kd, Vd = Kall[:len(cells)], Vall[:len(cells)]
        else:
            Kd = kv_rows(k, k_scales, s, g, cells)
            Vd = kv_rows(v, v_scales, s, g, cells)
        res.append(attend(q[s, t, h], Kd, Vd, scale))
    return np.stack(res) if res else np.zeros((0, D))


# --------------------------------------------------------------------------
# split-KV partials and their log-sum-exp merge
# --------------------------------------------------------------------------

def partial_over_cells(qrow: np.ndarray, Kd: np.ndarray, Vd: np.ndarray,
                       scale: float) -> Tuple[np.ndarray, float, float]:
    """Chunk-local softmax of one query row over a chunk of rows
    (qsa2.metal, qsa_attn2): m = max score, l = sum exp(score - m),
    o = sum exp(score - m) V (unnormalised).  An empty chunk gives
    (0, -inf, 0), the state a flash loop starts from (cera
    flash_attention.metal: running max -inf, running sum 0)."""
    D = Vd.shape[1]
    if Kd.shape[0] == 0:
        return np.zeros(D, dtype=np.float64), -math.inf, 0.0
    sc = float(scale) * (Kd @ qrow.astype(np.float64))
    m = float(sc.max())
    p = np.exp(sc - m)
    return p @ Vd, m, float(p.sum())


def merge_partials(o: Sequence[np.ndarray], m: Sequence[float], l: Sequence[float]) -> np.ndarray:
    """Log-sum-exp merge (qsa2.metal, qsa_merge2): M = max m_j,
    e_j = exp(m_j - M), out = sum e_j o_j / sum e_j l_j.  Partials with
    m = -inf weigh 0 (the guarded correction of cera flash_attention.metal);
    if every partial is empty the result is zero."""
    o = [np.asarray(x, dtype=np.float64) for x in o]
    D = o[0].shape[0]
    m = np.asarray(m, dtype=np.float64)
    l = np.asarray(l, dtype=np.float64)
    if m.size == 0 or not np.isfinite(m).any():
        return np.zeros(D, dtype=np.float64)
    M = m[np.isfinite(m)].max()
    e = np.where(np.isfinite(m), np.exp(np.where(np.isfinite(m), m - M, 0.0)), 0.0)
    num = np.zeros(D, dtype=np.float64)
    for ej, oj in zip(e, o):
        num += ej * oj
    return num / float((e * l).sum())


def split_partials(qrow, Kd, Vd, scale, bounds: Sequence[int]) -> List[Tuple[np.ndarray, float, float]]:
    """Partials of the consecutive chunks [bounds[i], bounds[i+1]) of the
    cell list."""
    return [partial_over_cells(qrow, Kd[a:b], Vd[a:b], scale)
            for a, b in zip(bounds[:-1], bounds[1:])]


def split_then_merge(q, k, v, seq_lens, scale, chunk: int, k_scales=None, v_scales=None,
                     ids=None) -> np.ndarray:
    """Output [S][T][H][D] computed the split-KV way: each token's cell list
    cut into chunks of `chunk` cells, one partial per chunk, then the LSE
    merge.  Equal to gqa_decode_ref up to rounding."""
    S, T, H, D = q.shape
    _, Lmax, Hk, _ = k.shape
    G = H // Hk
    out = np.zeros((S, T, H, D), dtype=np.float64)
    for s in range(S):
        for t in range(T):
            cells = cell_list(seq_lens[s], T, t, Lmax, None if ids is None else ids[s, t])
            n = len(cells)
            bounds = list(range(0, n, chunk)) + [n]
            if n == 0:
                bounds = [0, 0]
            for h in range(H):
                g = h // G
                Kd = kv_rows(k, k_scales, s, g, cells)
                Vd = kv_rows(v, v_scales, s, g, cells)
                parts = split_partials(q[s, t, h], Kd, Vd, scale, bounds)
                out[s, t, h] = merge_partials([p[0] for p in parts], [p[1] for p in parts],
                                              [p[2] for p in parts])
    return out
