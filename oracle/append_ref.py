"""CPU oracle for quantize-on-append: new fp32 K/V rows written into the int8
cache with one f16 scale per 64-element group.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or
executes this module; only the tests and the bench's CPU-baseline leg do.  It
shares no code with the HIP library.

What it computes (FORWARD_MSL, kernel kv_append_q8, with the group widened
from the page's 32 elements to the 64 of the int8 cache the attention reads,
the cache format of qsa2.metal):

  for every new row r (sequence s, new token i, KV head g) and every group of
  64 consecutive elements x of that row, in fp32 as the page computes:
    d     = max |x| / 127
    code  = clamp(rint(x / d), -127, 127)   if d > 0, else 0
            (rint rounds halves to even)
    cache[s][pos[s] + i][g][group] = code (int8),  scale = f16(d)
  Rows at or past Lmax are not written (a bad position only truncates).
The code is decided with the fp32 d; the stored scale is d rounded to f16,
as on the page.  Every division and the rounding follow IEEE-754 fp32, so the
GPU, computing in the same precision, must reproduce the codes exactly.

Pinned by tests/test_oracle_append.py (closed forms, round-half-even cases,
the reconstruction bound |x - code * d| <= d / 2, group independence and the
row/position rules).
"""
from __future__ import annotations

import numpy as np

__all__ = ["quantize_groups", "append_i8"]


def quantize_groups(x: np.ndarray):
    """x [..., D] float32 with D % 64 == 0 -> (codes int8 [..., D],
    scales float16 [..., D // 64])."""
    x = np.asarray(x, dtype=np.float32)
    D = x.shape[-1]
    assert D % 64 == 0
    g = x.reshape(x.shape[:-1] + (D // 64, 64))
    amax = np.max(np.abs(g), axis=-1, keepdims=True)           # fp32
    d = (amax / np.float32(127.0)).astype(np.float32)           # fp32 division
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(d > 0, np.rint(g / d), np.float32(0.0)).astype(np.float32)
    q = np.clip(q, -127.0, 127.0)
    codes = q.astype(np.int8).reshape(x.shape)
    with np.errstate(over="ignore"):         # d past the f16 range stores inf, as f16(d) does
        scales = d[..., 0].astype(np.float16)
    return codes, scales


def append_i8(k_new, v_new, pos, k, v, k_scales, v_scales):
    """Write new rows into copies of the caches and return them.
    k_new, v_new [S][Tn][Hk][D] float32; pos [S] int32 first cell of the new
    rows; k, v [S][Lmax][Hk][D] int8; k_scales, v_scales [S][Lmax][Hk][D/64]
    float16."""
    k, v, k_scales, v_scales = k.copy(), v.copy(), k_scales.copy(), v_scales.copy()
    S, Tn = k_new.shape[:2]
    Lmax = k.shape[1]
    kc, ks = quantize_groups(k_new)
    vc, vs = quantize_groups(v_new)
    for s in range(S):
        for i in range(Tn):
            c = int(pos[s]) + i
            if c < 0 or c >= Lmax:
                continue
            k[s, c], k_scales[s, c] = kc[s, i], ks[s, i]
            v[s, c], v_scales[s, c] = vc[s, i], vs[s, i]
    return k, v, k_scales, v_scales
