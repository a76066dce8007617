"""CPU oracle for the budget selection that produces the cell ids the
budgeted (gather) attention reads.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or
executes this module; only the tests and the bench's CPU-baseline leg do.  It
shares no code with the HIP library.

What it computes (qsa2.metal, kernel qsa_topk2):

  For sequence s and query token t of a T-token window:
    n      = L_t = clamp(seq_lens[s] - (T - 1 - t), 0, Lmax)   visible cells
    if n <= B:  ids[s, t, :n] = 0, 1, ..., n - 1                (identity)
    else:
      the cells are grouped in blocks of 4: block b holds cells 4b .. 4b+3;
      blocks 0 .. n//4 - 1 are whole, block n//4 holds the n % 4 remaining
      cells (possibly none).  Every block has one score; every cell of a
      block carries its block's score.
      Rank the cells by (block key descending, cell index ascending) and take
      the first B; emit them in ascending cell order.
    key(x) = the order-preserving map of the float's bits to an unsigned
      32-bit integer (sign bit clear: bits | 2^31; sign bit set: ~bits), so
      keys compare like the floats, with -0 below +0.

This is the plain definition of what the page's radix select reaches: it
finds the key T of the block where the running cell count, taken from the
highest key down, reaches B, takes every cell of blocks whose key exceeds T,
and fills the rest from blocks whose key equals T in block order, lowest cell
first, writing each thread's contiguous block range in order (so the output
ascends).  The key map is used but not defined on the page; the standard
order-preserving map is the reading taken.

Pinned by tests/test_oracle_select.py against an independent cell-level
formulation, closed forms (distinct scores, all-equal scores, identity below
the budget) and invariants.
"""
from __future__ import annotations

import numpy as np

__all__ = ["okey", "select_budget_ids", "blocks_per_token"]


def okey(scores: np.ndarray) -> np.ndarray:
    """Order-preserving uint32 key of float32 values."""
    bits = np.ascontiguousarray(scores, dtype=np.float32).view(np.uint32)
    neg = (bits >> np.uint32(31)) != 0
    return np.where(neg, ~bits, bits | np.uint32(0x80000000)).astype(np.uint32)


def blocks_per_token(Lmax: int) -> int:
    """Stride of the block-score rows: blocks 0 .. Lmax // 4 (the last one
    may hold no cell)."""
    return Lmax // 4 + 1


def _visible(seq_len: int, T: int, t: int, Lmax: int) -> int:
    Lt = int(seq_len) - (T - 1 - t)
    return max(0, min(Lt, int(Lmax)))


def select_one(block_scores_row: np.ndarray, n: int, B: int) -> np.ndarray:
    """Ids chosen for one token with n visible cells (ascending int64)."""
    if n <= B:
        return np.arange(n, dtype=np.int64)
    nb = n // 4 + 1
    keys = okey(block_scores_row[:nb]).astype(np.int64)
    cells_in = np.full(nb, 4, dtype=np.int64)
    cells_in[-1] = n % 4
    # blocks by key descending, block index ascending (stable sort on -key)
    order = np.argsort(-keys, kind="stable")
    chosen = []
    left = B
    for b in order:
        if left == 0:
            break
        take = min(int(cells_in[b]), left)
        chosen.extend(range(4 * int(b), 4 * int(b) + take))
        left -= take
    return np.sort(np.asarray(chosen, dtype=np.int64))


def select_budget_ids(block_scores: np.ndarray, seq_lens: np.ndarray, T: int, Lmax: int,
                      B: int) -> np.ndarray:
    """ids [S][T][B] int32.  block_scores [S][T][Lmax // 4 + 1] float32.
    Entries past min(L_t, B) of a token's row are set to -1 here (the GPU
    leaves them untouched; only the first min(L_t, B) are defined)."""
    S = block_scores.shape[0]
    assert block_scores.shape == (S, T, blocks_per_token(Lmax)), block_scores.shape
    out = np.full((S, T, B), -1, dtype=np.int32)
    for s in range(S):
        for t in range(T):
            n = _visible(seq_lens[s], T, t, Lmax)
            ids = select_one(block_scores[s, t], n, B)
            out[s, t, :len(ids)] = ids
    return out
