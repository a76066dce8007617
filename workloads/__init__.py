"""Seeded synthetic inputs for split-KV GQA decode attention.

This module only draws random tensors of the right shapes and value
distributions; it holds none of the attention arithmetic.  Both the fp64
oracle's tests and the GPU path's tests/bench take their inputs from here, so
the two sides always see bit-identical data.

Layouts (all C-contiguous numpy arrays):
  q          [S][T][H][D]        float32
  k, v       [S][Lmax][Hk][D]    float16  (kv="f16")  or  int8 (kv="i8")
  k_scales,  [S][Lmax][Hk][D/64] float16  (kv="i8" only: one scale per 64
  v_scales                                  consecutive elements of a row)
  ids        [S][T][B]           int32    (optional budget of cell ids)
  seq_lens   [S]                 int32    cells visible to the LAST query
                                          token of each sequence

The named workloads follow the decode shapes the source pages run their
kernels on: the f16 GQA decode of the cera shaders (group 4, head_dim 64 and
128), the int8 QSA decode of qsa2.metal (12 query heads per KV head,
head_dim 256, one f16 scale per 64 elements, scale 1/16, a budget of 2048
cell ids), and the causal multi-query window of flash_attention_tq.metal.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

__all__ = ["Workload", "WORKLOADS", "WORKLOAD_ORDER", "make_inputs", "make_case",
           "Inputs", "kv_bytes", "make_block_scores", "SELECT_WORKLOADS", "APPEND_WORKLOADS",
           "make_append_rows", "TQ_WORKLOADS", "TqInputs", "make_tq_case", "make_tq_inputs",
           "tq_bytes"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int            # position in the canonical list; seeds SeedSequence(1000 + index)
    S: int
    T: int
    H: int
    Hk: int
    D: int
    Lmax: int
    kv: str               # "f16" or "i8"
    scale: float
    chunk: int            # cells per split; 0 = library's automatic choice; -P = balanced partition
    lens: str             # "full" (every sequence at Lmax) or "uniform:lo:hi" (inclusive)
    budget: int = 0       # B; 0 = dense (no ids)
    description: str = ""


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_f16", 0, S=1, T=1, H=8, Hk=2, D=64, Lmax=256, kv="f16",
                 scale=1.0 / 8.0, chunk=32, lens="full",
                 description="tiny f16 decode: 1 seq, 8 heads / 2 KV heads, hd 64, 256 cells, 32-cell chunks"),
        Workload("f16_batch", 1, S=32, T=1, H=32, Hk=8, D=128, Lmax=4096, kv="f16",
                 scale=1.0 / math.sqrt(128.0), chunk=-32, lens="uniform:512:4096",
                 description="f16 GQA decode batch: 32 seqs, lengths U[512,4096], 32/8 heads, hd 128; "
                             "balanced partition, 32 pieces per KV head"),
        Workload("i8_32k", 2, S=8, T=1, H=24, Hk=2, D=256, Lmax=32768, kv="i8",
                 scale=1.0 / 16.0, chunk=0, lens="full",
                 description="int8 KV decode: 8 seqs at context 32768, 24/2 heads (group 12), hd 256"),
        Workload("i8_budget", 3, S=8, T=1, H=24, Hk=2, D=256, Lmax=65536, kv="i8",
                 scale=1.0 / 16.0, chunk=128, lens="full", budget=2048,
                 description="budgeted sparse int8 decode: context 65536, 2048 distinct ids per token, "
                             "32-cell chunks, four per workgroup (one per wave), one partial per workgroup"),
        Workload("f16_mq_causal", 4, S=4, T=8, H=32, Hk=8, D=128, Lmax=131072, kv="f16",
                 scale=1.0 / math.sqrt(128.0), chunk=0, lens="full",
                 description="multi-query causal chunk: 4 seqs x 8 tokens at start 131064, context 131072, 32/8 heads, hd 128"),
        # not one of the pages' configurations: the int8 32K model's heads over
        # a batch of uneven lengths, where the balanced partition pays most
        Workload("i8_batch", 8, S=32, T=1, H=24, Hk=2, D=256, Lmax=16384, kv="i8",
                 scale=1.0 / 16.0, chunk=-128, lens="uniform:2048:16384",
                 description="int8 decode batch of uneven lengths: 32 seqs, lengths U[2048,16384], 24/2 heads, "
                             "hd 256; balanced partition, 128 pieces per KV head"),
    ]
}
WORKLOAD_ORDER = sorted(WORKLOADS, key=lambda n: WORKLOADS[n].index)


@dataclasses.dataclass
class Inputs:
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    seq_lens: np.ndarray
    scale: float
    k_scales: Optional[np.ndarray] = None
    v_scales: Optional[np.ndarray] = None
    ids: Optional[np.ndarray] = None

    @property
    def kv(self) -> str:
        return "i8" if self.k.dtype == np.int8 else "f16"

    @property
    def shape(self):
        S, T, H, D = self.q.shape
        _, Lmax, Hk, _ = self.k.shape
        B = 0 if self.ids is None else self.ids.shape[2]
        return dict(S=S, T=T, H=H, Hk=Hk, D=D, Lmax=Lmax, B=B)


def _normal_f16(rng: np.random.Generator, shape) -> np.ndarray:
    # Draw fp32 N(0,1), then round to binary16 (round-to-nearest-even).
    out = np.empty(shape, dtype=np.float16)
    flat = out.reshape(-1)
    step = 1 << 24
    for i in range(0, flat.size, step):
        n = min(step, flat.size - i)
        flat[i:i + n] = rng.standard_normal(n, dtype=np.float32).astype(np.float16)
    return out


def _int8_uniform(rng: np.random.Generator, shape) -> np.ndarray:
    # Uniform integers in [-127, 127] inclusive (the symmetric int8 code range).
    return rng.integers(-127, 128, size=shape, dtype=np.int8)


def _scales_f16(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.uniform(0.005, 0.02, size=shape).astype(np.float16)


def make_case(S: int, T: int, H: int, Hk: int, D: int, Lmax: int, seq_lens,
              kv: str = "f16", scale: Optional[float] = None, budget: int = 0,
              seed: int = 0, sort_ids: bool = True) -> Inputs:
    """Seeded inputs for an arbitrary shape.

    `seq_lens` is a sequence of S ints (cells visible to the last query token).
    With `budget` B > 0, token t of sequence s gets min(L_t, B) distinct ids
    drawn uniformly without replacement from [0, L_t) (L_t is the causal
    window of that token, clamped to [0, Lmax]); the remaining entries are
    padded with 0 and never read.
    """
    if kv not in ("f16", "i8"):
        raise ValueError("kv must be 'f16' or 'i8'")
    if kv == "i8" and D % 64:
        raise ValueError("int8 rows need head_dim % 64 == 0")
    seq_lens = np.asarray(seq_lens, dtype=np.int32).reshape(S)
    ss = np.random.SeedSequence(seed)
    rq, rk, rv, rks, rvs, rid = [np.random.default_rng(c) for c in ss.spawn(6)]
    q = rq.standard_normal((S, T, H, D), dtype=np.float32)
    if kv == "f16":
        k = _normal_f16(rk, (S, Lmax, Hk, D))
        v = _normal_f16(rv, (S, Lmax, Hk, D))
        ks = vs = None
    else:
        k = _int8_uniform(rk, (S, Lmax, Hk, D))
        v = _int8_uniform(rv, (S, Lmax, Hk, D))
        ks = _scales_f16(rks, (S, Lmax, Hk, D // 64))
        vs = _scales_f16(rvs, (S, Lmax, Hk, D // 64))
    ids = None
    if budget > 0:
        ids = np.zeros((S, T, budget), dtype=np.int32)
        for s in range(S):
            for t in range(T):
                Lt = int(seq_lens[s]) - (T - 1 - t)
                Lt = max(0, min(Lt, Lmax))
                w = min(Lt, budget)
                if w == 0:
                    continue
                sel = rid.choice(Lt, size=w, replace=False).astype(np.int32)
                if sort_ids:
                    sel.sort()
                ids[s, t, :w] = sel
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return Inputs(q=q, k=k, v=v, seq_lens=seq_lens, scale=float(scale),
                  k_scales=ks, v_scales=vs, ids=ids)


def workload_seq_lens(w: Workload, seed_seq: np.random.SeedSequence) -> np.ndarray:
    if w.lens == "full":
        return np.full(w.S, w.Lmax, dtype=np.int32)
    kind, lo, hi = w.lens.split(":")
    assert kind == "uniform"
    rng = np.random.default_rng(seed_seq)
    return rng.integers(int(lo), int(hi) + 1, size=w.S).astype(np.int32)


def make_inputs(name: str, sort_ids: bool = True) -> Inputs:
    """Full-size seeded inputs of a named workload (SeedSequence(1000 + index))."""
    w = WORKLOADS[name]
    root = np.random.SeedSequence(1000 + w.index)
    c_lens, c_rest = root.spawn(2)
    lens = workload_seq_lens(w, c_lens)
    seed = int(c_rest.generate_state(1)[0])
    return make_case(w.S, w.T, w.H, w.Hk, w.D, w.Lmax, lens, kv=w.kv, scale=w.scale,
                     budget=w.budget, seed=seed, sort_ids=sort_ids)


def kv_bytes(inp: Inputs) -> int:
    """Algorithmic bytes one decode step must read: K + V (+ int8 scales) rows of
    every visible cell, once per KV head and sequence (shared by all query
    heads of the group and all query tokens of a dense window), plus the ids.
    q, the output and the split partials are not counted."""
    sh = inp.shape
    S, T, Hk, D, Lmax, B = sh["S"], sh["T"], sh["Hk"], sh["D"], sh["Lmax"], sh["B"]
    row = D * inp.k.itemsize
    if inp.kv == "i8":
        row += (D // 64) * 2
    total = 0
    for s in range(S):
        if B == 0:
            cells = max(0, min(int(inp.seq_lens[s]), Lmax))
            total += 2 * row * Hk * cells
        else:
            for t in range(T):
                Lt = max(0, min(int(inp.seq_lens[s]) - (T - 1 - t), Lmax))
                w = min(Lt, B)
                total += 2 * row * Hk * w + 4 * w
    return total


# ---------------------------------------------------------------------------
# Block scores for the budget selection (one score per 4-cell block).  How
# the scores are produced is not on the source pages (qsa2.metal reads them
# from a buffer), so they are synthetic: fp32 N(0,1), or, for tie-heavy
# cases, small integers so many blocks share a score.

SELECT_WORKLOADS = {
    # the selection step of the budgeted int8 decode: 8 sequences at context
    # 65536, a budget of 2048 cells per token
    "select_64k": dict(S=8, T=1, Lmax=65536, B=2048, lens="full", index=5),
}


def make_block_scores(S: int, T: int, Lmax: int, seed: int = 0, ties: bool = False) -> np.ndarray:
    """[S][T][Lmax // 4 + 1] float32 block scores."""
    rng = np.random.default_rng(np.random.SeedSequence(seed))
    shape = (S, T, Lmax // 4 + 1)
    if ties:
        return rng.integers(-3, 4, size=shape).astype(np.float32)
    return rng.standard_normal(shape, dtype=np.float32)


# ---------------------------------------------------------------------------
# New fp32 K/V rows for quantize-on-append (fp32 N(0,1), as the projections
# that produce them would; the source pages do not say).

APPEND_WORKLOADS = {
    # a 4096-token chunk appended to the int8 32K cache shape
    "append_i8": dict(S=8, Tn=4096, Hk=2, D=256, Lmax=32768, pos=16384, index=6),
}


def make_append_rows(S: int, Tn: int, Hk: int, D: int, seed: int = 0):
    """k_new, v_new [S][Tn][Hk][D] float32."""
    ss = np.random.SeedSequence(seed)
    rk, rv = [np.random.default_rng(c) for c in ss.spawn(2)]
    return (rk.standard_normal((S, Tn, Hk, D), dtype=np.float32),
            rv.standard_normal((S, Tn, Hk, D), dtype=np.float32))


# ---------------------------------------------------------------------------
# TurboQuant-compressed caches (the cache format of cera's
# flash_attention_tq.metal).  The encoder that produces the codes is not on
# the source page, so the codes themselves are drawn: uniform 2-bit polar
# indices and JL sign bits, f16 norms, random +-1 rotation signs.  The
# centroids are the 2-bit Lloyd-Max levels of a standard normal scaled by
# 1/sqrt(D) (the spread of one coordinate of a rotated unit vector); they are
# deliberately not f16-exact.  Queries arrive already rotated (q_rot) and
# JL-projected (q_jl): fp32 N(0,1).

TQ_LLOYD_MAX_2BIT = (-1.5104, -0.4528, 0.4528, 1.5104)

TQ_WORKLOADS = {
    # 4 sequences at context 131072, 32 query / 8 KV heads, head_dim 128
    # (the page's largest head_dim)
    "tq_128k": dict(S=4, T=1, H=32, Hk=8, D=128, Lmax=131072, lens="full", index=7),
}


@dataclasses.dataclass
class TqInputs:
    q_rot: np.ndarray      # [S][T][H][D] float32
    q_jl: np.ndarray       # [S][T][H][D] float32
    k_polar: np.ndarray    # [S][Hk][Lmax][D/16] uint32
    k_jl: np.ndarray       # [S][Hk][Lmax][D/32] uint32
    k_norms: np.ndarray    # [S][Hk][Lmax] uint32: f16 norm | f16 residual norm << 16
    v_polar: np.ndarray    # [S][Hk][Lmax][D/16] uint32
    v_norms: np.ndarray    # [S][Hk][Lmax] uint32: f16 norm in the low half
    seq_lens: np.ndarray   # [S] int32
    signs: np.ndarray      # [D] float32, +-1
    centroids: tuple       # 4 floats
    qjl_scale: float       # sqrt(pi / 2) / D, as the page's header gives it
    scale: float

    @property
    def shape(self):
        S, T, H, D = self.q_rot.shape
        return dict(S=S, T=T, H=H, Hk=self.k_polar.shape[1], D=D, Lmax=self.k_polar.shape[2])


def _f16_bits(x: np.ndarray) -> np.ndarray:
    return x.astype(np.float16).view(np.uint16).astype(np.uint32)


def make_tq_case(S: int, T: int, H: int, Hk: int, D: int, Lmax: int, seq_lens, seed: int = 0,
                 scale: Optional[float] = None) -> TqInputs:
    assert D % 32 == 0 and D & (D - 1) == 0 and H % Hk == 0
    ss = np.random.SeedSequence(seed)
    r = [np.random.default_rng(c) for c in ss.spawn(10)]
    q_rot = r[0].standard_normal((S, T, H, D), dtype=np.float32)
    q_jl = r[1].standard_normal((S, T, H, D), dtype=np.float32)
    u32 = np.iinfo(np.uint32).max
    k_polar = r[2].integers(0, u32, size=(S, Hk, Lmax, D // 16), dtype=np.uint32, endpoint=True)
    k_jl = r[3].integers(0, u32, size=(S, Hk, Lmax, D // 32), dtype=np.uint32, endpoint=True)
    v_polar = r[4].integers(0, u32, size=(S, Hk, Lmax, D // 16), dtype=np.uint32, endpoint=True)
    kn = r[5].uniform(0.5, 2.0, size=(S, Hk, Lmax)).astype(np.float32)
    kr = r[6].uniform(0.0, 0.5, size=(S, Hk, Lmax)).astype(np.float32)
    vn = r[7].uniform(0.5, 2.0, size=(S, Hk, Lmax)).astype(np.float32)
    k_norms = (_f16_bits(kn) | (_f16_bits(kr) << np.uint32(16))).astype(np.uint32)
    v_norms = _f16_bits(vn).astype(np.uint32)
    signs = np.where(r[8].integers(0, 2, size=D) == 1, 1.0, -1.0).astype(np.float32)
    c = tuple(float(np.float32(x / math.sqrt(D))) for x in TQ_LLOYD_MAX_2BIT)
    return TqInputs(q_rot=q_rot, q_jl=q_jl, k_polar=k_polar, k_jl=k_jl, k_norms=k_norms,
                    v_polar=v_polar, v_norms=v_norms,
                    seq_lens=np.asarray(seq_lens, dtype=np.int32).reshape(S),
                    signs=signs, centroids=c,
                    qjl_scale=float(np.float32(math.sqrt(math.pi / 2.0) / D)),
                    scale=float(np.float32(1.0 / math.sqrt(D) if scale is None else scale)))


def make_tq_inputs(name: str) -> TqInputs:
    w = TQ_WORKLOADS[name]
    lens = [w["Lmax"]] * w["S"]
    return make_tq_case(w["S"], w["T"], w["H"], w["Hk"], w["D"], w["Lmax"], lens,
                        seed=1000 + w["index"])


def tq_bytes(inp: TqInputs) -> int:
    """Algorithmic cache bytes one decode step reads: every visible cell of
    every (sequence, KV head) once -- K polar + JL + norms, V polar + norms."""
    sh = inp.shape
    per_cell = (sh["D"] // 16 * 4) * 2 + sh["D"] // 32 * 4 + 4 + 4
    total = 0
    for s in range(sh["S"]):
        total += per_cell * sh["Hk"] * max(0, min(int(inp.seq_lens[s]), sh["Lmax"]))
    return total
