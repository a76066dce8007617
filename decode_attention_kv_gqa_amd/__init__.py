"""Split-KV flash-decoding of grouped-query attention for MI355X (gfx950).

`decode_attention` runs one decode step through the HIP library
(libgqa_decode.so): the chunk kernel writes per-split partials and the merge
kernel combines them.  PyTorch is used only for device memory and the
current stream; there is no CPU or PyTorch fallback: without the built
library (or without a GPU) the call raises.
"""
from __future__ import annotations

from typing import Optional

from . import _lib
from ._lib import (GqaDecodeError, gqa_decode_attn_f16, gqa_decode_attn_i8, gqa_decode_merge,
                   gqa_decode_merge_gated, gqa_decode_attn_tq, gqa_decode_merge_tq,
                   gqa_decode_select_ids, gqa_decode_append_i8,
                   gqa_decode_part_bytes, gqa_decode_auto_chunk, gqa_decode_auto_pieces,
                   gqa_decode_step_static,
                   gqa_bench_stream_read, strerror)

__all__ = ["decode_attention", "DecodeAttention", "GqaDecodeError", "gqa_decode_attn_f16",
           "gqa_decode_attn_i8", "gqa_decode_merge", "gqa_decode_merge_gated",
           "gqa_decode_attn_tq", "gqa_decode_merge_tq", "TqDecodeAttention", "tq_decode_attention",
           "gqa_decode_select_ids", "select_ids",
           "gqa_decode_append_i8", "append_i8",
           "gqa_decode_part_bytes", "gqa_decode_step_static",
           "gqa_decode_auto_chunk", "gqa_decode_auto_pieces", "gqa_bench_stream_read",
           "strerror"]


def _raw_stream_getter():
    """Fast lookup of the current torch stream as a raw hipStream_t."""
    import torch
    get = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if get is not None:
        return get
    return lambda dev: torch.cuda.current_stream(dev).cuda_stream


class DecodeAttention:
    """A planned decode step for fixed shapes: resolves the split size once,
    owns the partial workspace and output, and enqueues the two kernels on
    the current torch stream at each call (or on `stream`, a raw
    hipStream_t).  The per-call path is argument marshalling only."""

    def __init__(self, S, T, H, Hk, D, Lmax, kv: str, B: int = 0, chunk=0, device="cuda"):
        """chunk: cells per split; 0 picks one (gqa_decode_auto_chunk); -P
        cuts the dense windows of the whole batch, laid end to end, into P
        equal pieces per KV head (the balanced partition, for batches of
        uneven lengths); "balanced" picks P (gqa_decode_auto_pieces)."""
        import torch
        self.S, self.T, self.H, self.Hk, self.D, self.Lmax, self.B = S, T, H, Hk, D, Lmax, B
        self.kv = kv
        if chunk == "balanced":
            chunk = gqa_decode_auto_pieces(S, T, Lmax, H, Hk, D, kv == "i8")
            if chunk >= 0 or B:
                raise GqaDecodeError("gqa_decode_auto_pieces", chunk if chunk < 0 else _lib.GQA_ERR_CHUNK)
        elif chunk == 0:
            chunk = gqa_decode_auto_chunk(S, T, Lmax, B, H, Hk, D, kv == "i8")
            if chunk <= 0:
                raise GqaDecodeError("gqa_decode_auto_chunk", chunk)
        self.chunk = int(chunk)
        self.part_bytes = gqa_decode_part_bytes(S, T, Lmax, B, H, D, self.chunk)
        if self.part_bytes == 0 and Lmax > 0:
            raise GqaDecodeError("gqa_decode_part_bytes", _lib.GQA_ERR_SHAPE)
        n = max(1, (self.part_bytes + 3) // 4)
        self.part = torch.empty(n, dtype=torch.float32, device=device)
        self.out = torch.empty((S, T, H, D), dtype=torch.float32, device=device)
        self._dev = self.out.device.index
        self._stream = _raw_stream_getter()
        lib = _lib.load()
        self._f16, self._i8, self._merge = (lib.gqa_decode_attn_f16, lib.gqa_decode_attn_i8,
                                            lib.gqa_decode_merge)
        self._merge_gated = lib.gqa_decode_merge_gated

    def attn(self, q, k, v, seq_lens, scale, k_scales=None, v_scales=None, ids=None, stream=None):
        st = self._stream(self._dev) if stream is None else stream
        idp = None if ids is None else ids.data_ptr()
        B = self.B if ids is not None else 0
        if self.kv == "i8":
            rc = self._i8(q.data_ptr(), k.data_ptr(), v.data_ptr(), k_scales.data_ptr(),
                          v_scales.data_ptr(), idp, seq_lens.data_ptr(), self.part.data_ptr(),
                          self.part_bytes, self.S, self.T, self.Lmax, B, self.H, self.Hk, self.D,
                          scale, self.chunk, st)
            if rc:
                raise GqaDecodeError("gqa_decode_attn_i8", rc)
        else:
            rc = self._f16(q.data_ptr(), k.data_ptr(), v.data_ptr(), idp, seq_lens.data_ptr(),
                           self.part.data_ptr(), self.part_bytes, self.S, self.T, self.Lmax, B,
                           self.H, self.Hk, self.D, scale, self.chunk, st)
            if rc:
                raise GqaDecodeError("gqa_decode_attn_f16", rc)

    def merge(self, seq_lens, ids=None, stream=None, gate=None, gate_stride=None):
        """The merge into self.out; with `gate` (float32 on the GPU, row r of
        the S*T*H output rows at element r * gate_stride, default D) each
        output element is multiplied by sigmoid(gate)."""
        st = self._stream(self._dev) if stream is None else stream
        idp = None if ids is None else ids.data_ptr()
        B = self.B if ids is not None else 0
        if gate is None:
            rc = self._merge(self.part.data_ptr(), seq_lens.data_ptr(), idp, self.out.data_ptr(),
                             self.S, self.T, self.Lmax, B, self.H, self.D, self.chunk, st)
            if rc:
                raise GqaDecodeError("gqa_decode_merge", rc)
        else:
            gs = self.D if gate_stride is None else int(gate_stride)
            rc = self._merge_gated(self.part.data_ptr(), seq_lens.data_ptr(), idp, gate.data_ptr(),
                                   gs, self.out.data_ptr(), self.S, self.T, self.Lmax, B, self.H,
                                   self.D, self.chunk, st)
            if rc:
                raise GqaDecodeError("gqa_decode_merge_gated", rc)

    def __call__(self, q, k, v, seq_lens, scale, k_scales=None, v_scales=None, ids=None,
                 gate=None, gate_stride=None):
        self.attn(q, k, v, seq_lens, scale, k_scales, v_scales, ids)
        self.merge(seq_lens, ids, gate=gate, gate_stride=gate_stride)
        return self.out


def _validate(q, k, v, seq_lens, k_scales, v_scales, ids):
    """Dtypes and shapes first (the kernels address every array from the
    shapes, so a smaller tensor would be read past its end), then device and
    layout."""
    import torch
    tensors = [("q", q), ("k", k), ("v", v), ("seq_lens", seq_lens)]
    if k is not None and k.dtype == torch.int8:
        tensors += [("k_scales", k_scales), ("v_scales", v_scales)]
    if ids is not None:
        tensors.append(("ids", ids))
    for name, t in tensors:
        if t is None:
            raise ValueError(f"{name} is required")
    if q.dtype != torch.float32:
        raise ValueError("q must be float32 [S][T][H][D]")
    if seq_lens.dtype != torch.int32 or (ids is not None and ids.dtype != torch.int32):
        raise ValueError("seq_lens and ids must be int32")
    if k.dtype == torch.int8:
        if k_scales.dtype != torch.float16 or v_scales.dtype != torch.float16:
            raise ValueError("int8 K/V need float16 k_scales and v_scales [S][Lmax][Hk][D/64]")
    elif k.dtype != torch.float16:
        raise ValueError("K/V must be float16 or int8")
    if v.dtype != k.dtype or v.shape != k.shape:
        raise ValueError("K and V must share dtype and shape")
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [S][T][H][D] and k, v [S][Lmax][Hk][D]")
    S, T, _, D = q.shape
    _, Lmax, Hk, Dk = k.shape
    if Dk != D or k.shape[0] != S or tuple(seq_lens.shape) != (S,):
        raise ValueError("shape mismatch between q, k/v and seq_lens")
    if k.dtype == torch.int8:
        want = (S, Lmax, Hk, D // 64)
        if tuple(k_scales.shape) != want or tuple(v_scales.shape) != want:
            raise ValueError(f"k_scales and v_scales must be {list(want)}")
    if ids is not None and (ids.dim() != 3 or tuple(ids.shape[:2]) != (S, T)):
        raise ValueError("ids must be [S][T][B]")
    for name, t in tensors:
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor (there is no CPU path)")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


def decode_attention(q, k, v, seq_lens, scale: Optional[float] = None, *, k_scales=None,
                     v_scales=None, ids=None, chunk=0, gate=None):
    """One decode step.  q [S][T][H][D] float32; k, v [S][Lmax][Hk][D]
    float16, or int8 with k_scales / v_scales [S][Lmax][Hk][D/64] float16;
    seq_lens [S] int32 (cells visible to each sequence's last query token);
    chunk: cells per split, 0 for the library's choice, -P or "balanced" for
    the balanced partition of a batch of uneven lengths (dense only);
    ids None or [S][T][B] int32; gate None or float32 [S][T][H][D], possibly
    the gate half of [query | gate] rows (a view whose last dim is contiguous
    and whose head rows are evenly strided).  Returns out [S][T][H][D]
    float32, multiplied by sigmoid(gate) when a gate is given."""
    import torch
    _validate(q, k, v, seq_lens, k_scales, v_scales, ids)
    gate_stride = None
    if gate is not None:
        if not gate.is_cuda or gate.dtype != torch.float32 or tuple(gate.shape) != tuple(q.shape):
            raise ValueError("gate must be a float32 GPU tensor shaped like q")
        S_, T_, H_, D_ = gate.shape
        st = gate.stride()
        if st[3] != 1 or st[2] < D_ or st[1] != H_ * st[2] or st[0] != T_ * st[1]:
            raise ValueError("gate rows must be evenly strided with a contiguous last dim")
        gate_stride = st[2]
    S, T, H, D = q.shape
    _, Lmax, Hk, _ = k.shape
    B = 0 if ids is None else ids.shape[2]
    if scale is None:
        scale = D ** -0.5
    kv = "i8" if k.dtype == torch.int8 else "f16"
    step = _planned_step(S, T, H, Hk, D, Lmax, kv, B, chunk, q.device)
    return step(q, k, v, seq_lens, scale, k_scales, v_scales, ids, gate=gate,
                gate_stride=gate_stride).clone()


# Planned steps of decode_attention(), one per shape, device and split size:
# a repeated call reuses the resolved split, the workspace and the output
# buffer instead of planning and allocating again.  The result handed back is
# a copy, so it stays valid when the same shape runs again.  Calls on one
# device share a plan's buffers, so they must be ordered (one stream, or
# synchronised) as any reuse of a torch buffer must.
_PLANS: "dict" = {}
_PLANS_MAX = 16


def _planned_step(S, T, H, Hk, D, Lmax, kv, B, chunk, device):
    key = (S, T, H, Hk, D, Lmax, kv, B, chunk if chunk == "balanced" else int(chunk), str(device))
    step = _PLANS.get(key)
    if step is None:
        if len(_PLANS) >= _PLANS_MAX:
            _PLANS.pop(next(iter(_PLANS)))
        step = _PLANS[key] = DecodeAttention(S, T, H, Hk, D, Lmax, kv, B=B, chunk=chunk,
                                             device=device)
    return step


def select_ids(block_scores, seq_lens, B: int, out=None, Lmax: Optional[int] = None):
    """Budget selection on the GPU.  block_scores [S][T][Lmax // 4 + 1]
    float32, seq_lens [S] int32; returns ids [S][T][B] int32 whose first
    min(L_t, B) entries per token are defined (the rest keep `out`'s contents,
    -1 for a fresh output).  Lmax is the cache capacity that windows are
    clamped to; the scores' shape fixes it only up to the last block, so pass
    it unless it is a multiple of 4 (the default is 4 * (blocks - 1))."""
    import torch
    if block_scores.dtype != torch.float32 or seq_lens.dtype != torch.int32:
        raise ValueError("block_scores must be float32 and seq_lens int32")
    S, T, nbs = block_scores.shape
    if Lmax is None:
        Lmax = 4 * (nbs - 1)
    elif Lmax < 0 or Lmax // 4 + 1 != nbs:
        raise ValueError("block_scores must be [S][T][Lmax // 4 + 1]")
    if tuple(seq_lens.shape) != (S,):
        raise ValueError("seq_lens must be [S]")
    for name, t in (("block_scores", block_scores), ("seq_lens", seq_lens)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    if out is None:
        out = torch.full((S, T, B), -1, dtype=torch.int32, device=block_scores.device)
    elif tuple(out.shape) != (S, T, B) or out.dtype != torch.int32 or not out.is_contiguous():
        raise ValueError("out must be a contiguous int32 [S][T][B] tensor")
    st = torch.cuda.current_stream(block_scores.device).cuda_stream
    rc = gqa_decode_select_ids(block_scores.data_ptr(), seq_lens.data_ptr(), out.data_ptr(), S, T,
                               Lmax, B, st)
    if rc:
        raise GqaDecodeError("gqa_decode_select_ids", rc)
    return out


def append_i8(k_new, v_new, pos, k, v, k_scales, v_scales):
    """Quantize-on-append in place.  k_new, v_new [S][Tn][Hk][D] float32;
    pos [S] int32; k, v [S][Lmax][Hk][D] int8; k_scales, v_scales
    [S][Lmax][Hk][D/64] float16 (all contiguous GPU tensors)."""
    import torch
    for name, t in (("k_new", k_new), ("v_new", v_new), ("pos", pos), ("k", k), ("v", v),
                    ("k_scales", k_scales), ("v_scales", v_scales)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    if k_new.dtype != torch.float32 or v_new.dtype != torch.float32 or pos.dtype != torch.int32 \
            or k.dtype != torch.int8 or v.dtype != torch.int8 \
            or k_scales.dtype != torch.float16 or v_scales.dtype != torch.float16:
        raise ValueError("dtypes: k_new/v_new float32, pos int32, k/v int8, scales float16")
    S, Tn, Hk, D = k_new.shape
    S2, Lmax, Hk2, D2 = k.shape
    if (S2, Hk2, D2) != (S, Hk, D) or v_new.shape != k_new.shape or v.shape != k.shape \
            or tuple(pos.shape) != (S,) or tuple(k_scales.shape) != (S, Lmax, Hk, D // 64) \
            or k_scales.shape != v_scales.shape:
        raise ValueError("shape mismatch between new rows, positions, caches and scales")
    st = torch.cuda.current_stream(k.device).cuda_stream
    rc = gqa_decode_append_i8(k_new.data_ptr(), v_new.data_ptr(), pos.data_ptr(), k.data_ptr(),
                              v.data_ptr(), k_scales.data_ptr(), v_scales.data_ptr(), S, Tn, Lmax,
                              Hk, D, st)
    if rc:
        raise GqaDecodeError("gqa_decode_append_i8", rc)


class TqDecodeAttention:
    """A decode step over a TurboQuant-compressed cache with its workspace
    and output preallocated: attn() writes the rotated partials, merge() the
    merged rows rotated back to the original basis (out [S][T][H][D])."""

    def __init__(self, S, T, H, Hk, D, Lmax, chunk: int = 0, device="cuda"):
        import torch
        self.S, self.T, self.H, self.Hk, self.D, self.Lmax = S, T, H, Hk, D, Lmax
        if chunk <= 0:
            chunk = gqa_decode_auto_chunk(S, T, Lmax, 0, H, Hk, D, 2)
            if chunk <= 0:
                raise GqaDecodeError("gqa_decode_auto_chunk", chunk)
        self.chunk = int(chunk)
        self.part_bytes = gqa_decode_part_bytes(S, T, Lmax, 0, H, D, self.chunk)
        if self.part_bytes == 0 and Lmax > 0:
            raise GqaDecodeError("gqa_decode_part_bytes", _lib.GQA_ERR_SHAPE)
        self.part = torch.empty(max(1, (self.part_bytes + 3) // 4), dtype=torch.float32,
                                device=device)
        self.out = torch.empty((S, T, H, D), dtype=torch.float32, device=device)
        self._dev = self.out.device.index
        self._stream = _raw_stream_getter()
        lib = _lib.load()
        self._attn, self._merge = lib.gqa_decode_attn_tq, lib.gqa_decode_merge_tq

    def attn(self, q_rot, q_jl, k_polar, k_jl, k_norms, v_polar, v_norms, seq_lens, centroids,
             qjl_scale, scale, stream=None):
        st = self._stream(self._dev) if stream is None else stream
        c = [float(x) for x in centroids]
        rc = self._attn(q_rot.data_ptr(), q_jl.data_ptr(), k_polar.data_ptr(), k_jl.data_ptr(),
                        k_norms.data_ptr(), v_polar.data_ptr(), v_norms.data_ptr(),
                        seq_lens.data_ptr(), self.part.data_ptr(), self.part_bytes, self.S, self.T,
                        self.Lmax, self.H, self.Hk, self.D, c[0], c[1], c[2], c[3],
                        float(qjl_scale), float(scale), self.chunk, st)
        if rc:
            raise GqaDecodeError("gqa_decode_attn_tq", rc)

    def merge(self, seq_lens, signs, stream=None):
        st = self._stream(self._dev) if stream is None else stream
        rc = self._merge(self.part.data_ptr(), seq_lens.data_ptr(), signs.data_ptr(),
                         self.out.data_ptr(), self.S, self.T, self.Lmax, self.H, self.D,
                         self.chunk, st)
        if rc:
            raise GqaDecodeError("gqa_decode_merge_tq", rc)


def tq_decode_attention(q_rot, q_jl, k_polar, k_jl, k_norms, v_polar, v_norms, seq_lens, signs,
                        centroids, qjl_scale: float, scale: float, *, chunk: int = 0):
    """One decode step over a TurboQuant-compressed cache.  q_rot, q_jl
    [S][T][H][D] float32; k_polar, v_polar [S][Hk][Lmax][D/16], k_jl
    [S][Hk][Lmax][D/32], k_norms, v_norms [S][Hk][Lmax] (int32 or uint32
    words); seq_lens [S] int32; signs [D] float32; centroids: 4 floats.
    Returns out [S][T][H][D] float32 in the original basis."""
    import torch
    for name, t in (("q_rot", q_rot), ("q_jl", q_jl), ("k_polar", k_polar), ("k_jl", k_jl),
                    ("k_norms", k_norms), ("v_polar", v_polar), ("v_norms", v_norms),
                    ("seq_lens", seq_lens), ("signs", signs)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor (there is no CPU path)")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if q_rot.dtype != torch.float32 or q_jl.dtype != torch.float32 or signs.dtype != torch.float32:
        raise ValueError("q_rot, q_jl and signs must be float32")
    if q_rot.shape != q_jl.shape:
        raise ValueError("q_rot and q_jl must share a shape")
    S, T, H, D = q_rot.shape
    S2, Hk, Lmax, W = k_polar.shape
    if S2 != S or W * 16 != D or tuple(v_polar.shape) != tuple(k_polar.shape) \
            or tuple(k_jl.shape) != (S, Hk, Lmax, D // 32) \
            or tuple(k_norms.shape) != (S, Hk, Lmax) or tuple(v_norms.shape) != (S, Hk, Lmax) \
            or tuple(signs.shape) != (D,) or tuple(seq_lens.shape) != (S,):
        raise ValueError("shape mismatch between the query, the compressed cache and signs")
    step = TqDecodeAttention(S, T, H, Hk, D, Lmax, chunk=chunk, device=q_rot.device)
    step.attn(q_rot, q_jl, k_polar, k_jl, k_norms, v_polar, v_norms, seq_lens, centroids,
              qjl_scale, scale)
    step.merge(seq_lens, signs)
    return step.out.clone()
