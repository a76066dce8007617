"""ctypes binding of libgqa_decode.so (include/gqa_decode.h).

Argument marshalling only: every step of the computation runs in the HIP
library.  The functions carry the C names and take raw device pointers
(ints), sizes and a hipStream_t handle (int, 0 = null stream).
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgqa_decode.so")

GQA_OK = 0
GQA_ERR_NULL = -1
GQA_ERR_SHAPE = -2
GQA_ERR_GROUP = -3
GQA_ERR_HEAD_DIM = -4
GQA_ERR_BUDGET = -5
GQA_ERR_CHUNK = -6
GQA_ERR_WORKSPACE = -7
GQA_ERR_STATIC_LIMIT = -8
GQA_STATIC_PART_BYTES = 16 << 20

EXPORTED = ["gqa_decode_attn_f16", "gqa_decode_attn_i8", "gqa_decode_merge",
            "gqa_decode_merge_gated", "gqa_decode_attn_tq", "gqa_decode_merge_tq",
            "gqa_decode_select_ids", "gqa_decode_append_i8", "gqa_decode_part_bytes",
            "gqa_decode_auto_chunk", "gqa_decode_auto_pieces", "gqa_decode_step_static",
            "gqa_decode_strerror", "gqa_bench_stream_read"]

_lib = None


class GqaDecodeError(RuntimeError):
    def __init__(self, fn: str, code: int):
        self.code = code
        super().__init__(f"{fn} failed with {code}: {strerror(code)}")


def load() -> ctypes.CDLL:
    """Load the built library; raise if it was never built (there is no
    fallback implementation)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m decode_attention_kv_gqa_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, sz, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
    lib.gqa_decode_attn_f16.argtypes = [vp, vp, vp, vp, vp, vp, sz] + [i32] * 7 + [f32, i32, vp]
    lib.gqa_decode_attn_f16.restype = i32
    lib.gqa_decode_attn_i8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, sz] + [i32] * 7 + [f32, i32, vp]
    lib.gqa_decode_attn_i8.restype = i32
    lib.gqa_decode_merge.argtypes = [vp, vp, vp, vp] + [i32] * 7 + [vp]
    lib.gqa_decode_merge.restype = i32
    lib.gqa_decode_merge_gated.argtypes = [vp, vp, vp, vp, ctypes.c_int64, vp] + [i32] * 7 + [vp]
    lib.gqa_decode_merge_gated.restype = i32
    lib.gqa_decode_attn_tq.argtypes = [vp] * 9 + [sz] + [i32] * 6 + [f32] * 6 + [i32, vp]
    lib.gqa_decode_attn_tq.restype = i32
    lib.gqa_decode_merge_tq.argtypes = [vp] * 4 + [i32] * 6 + [vp]
    lib.gqa_decode_merge_tq.restype = i32
    lib.gqa_decode_select_ids.argtypes = [vp, vp, vp] + [i32] * 4 + [vp]
    lib.gqa_decode_select_ids.restype = i32
    lib.gqa_decode_append_i8.argtypes = [vp] * 7 + [i32] * 5 + [vp]
    lib.gqa_decode_append_i8.restype = i32
    lib.gqa_decode_part_bytes.argtypes = [i32] * 7
    lib.gqa_decode_part_bytes.restype = sz
    lib.gqa_decode_auto_chunk.argtypes = [i32] * 8
    lib.gqa_decode_auto_chunk.restype = i32
    lib.gqa_decode_auto_pieces.argtypes = [i32] * 7
    lib.gqa_decode_auto_pieces.restype = i32
    lib.gqa_decode_step_static.argtypes = [vp] * 8 + [i32] * 7 + [f32, i32, i32, vp]
    lib.gqa_decode_step_static.restype = i32
    lib.gqa_decode_strerror.argtypes = [i32]
    lib.gqa_decode_strerror.restype = ctypes.c_char_p
    lib.gqa_bench_stream_read.argtypes = [vp, sz, vp, i32, vp]
    lib.gqa_bench_stream_read.restype = i32
    _lib = lib
    return lib


def strerror(code: int) -> str:
    return load().gqa_decode_strerror(int(code)).decode()


def _p(x) -> int | None:
    return None if x is None or x == 0 else int(x)


def gqa_decode_attn_f16(q, k, v, ids, seq_lens, part, part_bytes, S, T, Lmax, B, H, Hk, D,
                        scale, chunk, stream=0) -> int:
    return load().gqa_decode_attn_f16(_p(q), _p(k), _p(v), _p(ids), _p(seq_lens), _p(part),
                                      part_bytes, S, T, Lmax, B, H, Hk, D, scale, chunk, _p(stream))


def gqa_decode_attn_i8(q, k, v, k_scales, v_scales, ids, seq_lens, part, part_bytes, S, T, Lmax,
                       B, H, Hk, D, scale, chunk, stream=0) -> int:
    return load().gqa_decode_attn_i8(_p(q), _p(k), _p(v), _p(k_scales), _p(v_scales), _p(ids),
                                     _p(seq_lens), _p(part), part_bytes, S, T, Lmax, B, H, Hk, D,
                                     scale, chunk, _p(stream))


def gqa_decode_merge(part, seq_lens, ids_or_null, out, S, T, Lmax, B, H, D, chunk, stream=0) -> int:
    return load().gqa_decode_merge(_p(part), _p(seq_lens), _p(ids_or_null), _p(out), S, T, Lmax, B,
                                   H, D, chunk, _p(stream))


def gqa_decode_merge_gated(part, seq_lens, ids_or_null, gate, gate_stride, out, S, T, Lmax, B, H,
                           D, chunk, stream=0) -> int:
    return load().gqa_decode_merge_gated(_p(part), _p(seq_lens), _p(ids_or_null), _p(gate),
                                         int(gate_stride), _p(out), S, T, Lmax, B, H, D, chunk,
                                         _p(stream))


def gqa_decode_attn_tq(q_rot, q_jl, k_polar, k_jl, k_norms, v_polar, v_norms, seq_lens, part,
                       part_bytes, S, T, Lmax, H, Hk, D, c0, c1, c2, c3, qjl_scale, scale, chunk,
                       stream=0) -> int:
    return load().gqa_decode_attn_tq(_p(q_rot), _p(q_jl), _p(k_polar), _p(k_jl), _p(k_norms),
                                     _p(v_polar), _p(v_norms), _p(seq_lens), _p(part), part_bytes,
                                     S, T, Lmax, H, Hk, D, c0, c1, c2, c3, qjl_scale, scale, chunk,
                                     _p(stream))


def gqa_decode_merge_tq(part, seq_lens, signs, out, S, T, Lmax, H, D, chunk, stream=0) -> int:
    return load().gqa_decode_merge_tq(_p(part), _p(seq_lens), _p(signs), _p(out), S, T, Lmax, H, D,
                                      chunk, _p(stream))


def gqa_decode_part_bytes(S, T, Lmax, B, H, D, chunk) -> int:
    return load().gqa_decode_part_bytes(S, T, Lmax, B, H, D, chunk)


def gqa_decode_auto_chunk(S, T, Lmax, B, H, Hk, D, kv_kind) -> int:
    """kv_kind: 0 (or False) f16, 1 (or True) int8, 2 TurboQuant."""
    return load().gqa_decode_auto_chunk(S, T, Lmax, B, H, Hk, D, int(kv_kind))


def gqa_decode_auto_pieces(S, T, Lmax, H, Hk, D, kv_kind) -> int:
    """The balanced partition's chunk argument (-P); kv_kind 0 f16, 1 int8."""
    return load().gqa_decode_auto_pieces(S, T, Lmax, H, Hk, D, int(kv_kind))


def gqa_decode_step_static(q, k, v, k_scales, v_scales, ids, seq_lens, out, S, T, Lmax, B, H, Hk,
                           D, scale, chunk, kv_kind, stream=0) -> int:
    """The whole step with the partials in the library's static buffer
    (kv_kind 0: f16, 1: int8)."""
    return load().gqa_decode_step_static(_p(q), _p(k), _p(v), _p(k_scales), _p(v_scales), _p(ids),
                                         _p(seq_lens), _p(out), S, T, Lmax, B, H, Hk, D, scale,
                                         chunk, int(kv_kind), _p(stream))


def gqa_decode_select_ids(block_scores, seq_lens, ids, S, T, Lmax, B, stream=0) -> int:
    return load().gqa_decode_select_ids(_p(block_scores), _p(seq_lens), _p(ids), S, T, Lmax, B,
                                        _p(stream))


def gqa_decode_append_i8(k_new, v_new, pos, k, v, k_scales, v_scales, S, Tn, Lmax, Hk, D,
                         stream=0) -> int:
    return load().gqa_decode_append_i8(_p(k_new), _p(v_new), _p(pos), _p(k), _p(v), _p(k_scales),
                                       _p(v_scales), S, Tn, Lmax, Hk, D, _p(stream))


def gqa_bench_stream_read(src, nbytes, sink, workgroups, stream=0) -> int:
    """Measurement aid (include/gqa_bench.h): a plain streaming read of nbytes
    at src by `workgroups` workgroups; sink[w] = XOR of the words workgroup w
    read."""
    return load().gqa_bench_stream_read(_p(src), nbytes, _p(sink), workgroups, _p(stream))
