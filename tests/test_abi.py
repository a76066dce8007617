"""The C-ABI library loads, exports every function include/gqa_decode.h
declares, and rejects bad arguments on the host before any HIP call (CPU
only: no call here reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

import decode_attention_kv_gqa_amd as gq
from decode_attention_kv_gqa_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            src = open(os.path.join(ROOT, "include", fn)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names += re.findall(r"\b(gqa_\w+)\s*\(", src)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    names = declared_functions()
    assert set(_lib.EXPORTED) <= set(names)
    for n in names:
        assert hasattr(lib, n), n
        assert ctypes.cast(getattr(lib, n), ctypes.c_void_p).value


def test_strerror_covers_codes():
    for c in range(0, -9, -1):
        assert gq.strerror(c) not in ("", "unknown error")
    assert gq.strerror(-99) == "unknown error"
    assert "HIP" in gq.strerror(98)


FAKE = 0x1000  # never dereferenced: every call below fails validation first


def attn_f16(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, ids=None, seq_lens=FAKE, part=FAKE, part_bytes=1 << 40,
             S=1, T=1, Lmax=16, B=0, H=8, Hk=2, D=64, scale=0.125, chunk=0, stream=0)
    a.update(kw)
    return gq.gqa_decode_attn_f16(a["q"], a["k"], a["v"], a["ids"], a["seq_lens"], a["part"],
                                  a["part_bytes"], a["S"], a["T"], a["Lmax"], a["B"], a["H"],
                                  a["Hk"], a["D"], a["scale"], a["chunk"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), _lib.GQA_ERR_NULL),
    (dict(k=None), _lib.GQA_ERR_NULL),
    (dict(seq_lens=None), _lib.GQA_ERR_NULL),
    (dict(part=None), _lib.GQA_ERR_NULL),
    (dict(S=0), _lib.GQA_ERR_SHAPE),
    (dict(T=0), _lib.GQA_ERR_SHAPE),
    (dict(H=0), _lib.GQA_ERR_SHAPE),
    (dict(Lmax=-1), _lib.GQA_ERR_SHAPE),
    (dict(S=1 << 20, H=4096), _lib.GQA_ERR_SHAPE),   # S*T*H output rows beyond 2^31 - 1
    (dict(H=9), _lib.GQA_ERR_GROUP),
    (dict(D=96), _lib.GQA_ERR_HEAD_DIM),
    (dict(D=32), _lib.GQA_ERR_HEAD_DIM),
    (dict(ids=FAKE, B=0), _lib.GQA_ERR_BUDGET),
    (dict(part_bytes=16), _lib.GQA_ERR_WORKSPACE),
    (dict(chunk=1, part_bytes=8 * 16 * 66 * 4 - 1), _lib.GQA_ERR_WORKSPACE),
    # balanced partition (negative chunk): dense windows only, a bounded
    # piece count and total window, a workspace holding the slot counts too
    (dict(chunk=-4, ids=FAKE, B=8), _lib.GQA_ERR_CHUNK),
    (dict(chunk=-(1 << 16) - 1), _lib.GQA_ERR_CHUNK),
    (dict(chunk=-4, S=1 << 16, Lmax=1 << 15), _lib.GQA_ERR_CHUNK),
    (dict(chunk=-4, part_bytes=8 * 4 * 66 * 4 + 15), _lib.GQA_ERR_WORKSPACE),
])
def test_attn_f16_rejects(kw, code):
    assert attn_f16(**kw) == code


def test_attn_i8_needs_scales():
    rc = gq.gqa_decode_attn_i8(FAKE, FAKE, FAKE, None, FAKE, None, FAKE, FAKE, 1 << 40,
                               1, 1, 16, 0, 8, 2, 64, 0.125, 0, 0)
    assert rc == _lib.GQA_ERR_NULL


def test_merge_rejects():
    m = gq.gqa_decode_merge
    assert m(None, FAKE, None, FAKE, 1, 1, 16, 0, 8, 64, 32, 0) == _lib.GQA_ERR_NULL
    assert m(FAKE, FAKE, None, FAKE, 1, 1, 16, 0, 8, 64, 0, 0) == _lib.GQA_ERR_CHUNK
    assert m(FAKE, FAKE, None, FAKE, 1, 1, 16, 0, 8, 96, 32, 0) == _lib.GQA_ERR_HEAD_DIM
    assert m(FAKE, FAKE, FAKE, FAKE, 1, 1, 16, 0, 8, 64, 32, 0) == _lib.GQA_ERR_BUDGET
    # the balanced partition has no ids form
    assert m(FAKE, FAKE, FAKE, FAKE, 1, 1, 16, 8, 8, 64, -4, 0) == _lib.GQA_ERR_CHUNK


def test_merge_gated_rejects():
    m = gq.gqa_decode_merge_gated
    # NULL gate, NULL workspace, gate rows narrower than D, then the merge's own checks
    assert m(FAKE, FAKE, None, None, 64, FAKE, 1, 1, 16, 0, 8, 64, 32, 0) == _lib.GQA_ERR_NULL
    assert m(None, FAKE, None, FAKE, 64, FAKE, 1, 1, 16, 0, 8, 64, 32, 0) == _lib.GQA_ERR_NULL
    assert m(FAKE, FAKE, None, FAKE, 63, FAKE, 1, 1, 16, 0, 8, 64, 32, 0) == _lib.GQA_ERR_SHAPE
    assert m(FAKE, FAKE, None, FAKE, 64, FAKE, 1, 1, 16, 0, 8, 64, 0, 0) == _lib.GQA_ERR_CHUNK
    assert m(FAKE, FAKE, None, FAKE, 96, FAKE, 1, 1, 16, 0, 8, 96, 32, 0) == _lib.GQA_ERR_HEAD_DIM


def test_tq_rejects():
    a = gq.gqa_decode_attn_tq
    args = lambda **kw: dict(dict(q_rot=FAKE, q_jl=FAKE, k_polar=FAKE, k_jl=FAKE, k_norms=FAKE,
                                  v_polar=FAKE, v_norms=FAKE, seq_lens=FAKE, part=FAKE,
                                  part_bytes=1 << 40, S=1, T=1, Lmax=64, H=8, Hk=2, D=64, c0=-1.0,
                                  c1=-0.3, c2=0.3, c3=1.0, qjl_scale=0.02, scale=0.125, chunk=32),
                             **kw)
    call = lambda **kw: a(**args(**kw), stream=0)
    assert call(k_jl=None) == _lib.GQA_ERR_NULL
    assert call(q_jl=None) == _lib.GQA_ERR_NULL
    assert call(D=256) == _lib.GQA_ERR_HEAD_DIM            # the page's limit: head_dim <= 128
    assert call(D=96) == _lib.GQA_ERR_HEAD_DIM
    assert call(H=6, Hk=4) == _lib.GQA_ERR_GROUP
    assert call(part_bytes=16) == _lib.GQA_ERR_WORKSPACE
    m = gq.gqa_decode_merge_tq
    assert m(FAKE, FAKE, None, FAKE, 1, 1, 64, 8, 64, 32, 0) == _lib.GQA_ERR_NULL
    assert m(FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 8, 256, 32, 0) == _lib.GQA_ERR_HEAD_DIM
    assert m(FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 8, 64, 0, 0) == _lib.GQA_ERR_CHUNK


def test_part_bytes_formula():
    # splits = ceil(width / chunk); one (D + 2)-float partial per query row and split
    assert gq.gqa_decode_part_bytes(8, 1, 32768, 0, 24, 256, 512) == 8 * 24 * 64 * 258 * 4
    assert gq.gqa_decode_part_bytes(8, 1, 65536, 2048, 24, 256, 32) == 8 * 24 * 64 * 258 * 4
    assert gq.gqa_decode_part_bytes(1, 1, 100, 0, 8, 64, 32) == 8 * 4 * 66 * 4
    assert gq.gqa_decode_part_bytes(1, 1, 0, 0, 8, 64, 32) == 0
    assert gq.gqa_decode_part_bytes(1, 1, 100, 0, 8, 64, 0) == 0
    # balanced partition: P slots per row, then S int32 slot counts rounded
    # up to 16 bytes; no ids form
    assert gq.gqa_decode_part_bytes(32, 1, 4096, 0, 32, 128, -32) == 32 * 32 * 32 * 130 * 4 + 128
    assert gq.gqa_decode_part_bytes(3, 2, 100, 0, 8, 64, -5) == 3 * 2 * 8 * 5 * 66 * 4 + 16
    assert gq.gqa_decode_part_bytes(3, 1, 0, 0, 8, 64, -5) == 16
    assert gq.gqa_decode_part_bytes(3, 1, 100, 8, 8, 64, -5) == 0
    assert gq.gqa_decode_part_bytes(3, 1, 100, 0, 8, 64, -(1 << 17)) == 0


def test_auto_chunk_plan():
    ac = gq.gqa_decode_auto_chunk
    # deterministic, positive, multiple of 64, never wider than the (rounded) window
    for args in [(8, 1, 32768, 0, 24, 2, 256, 1), (4, 8, 131072, 0, 32, 8, 128, 0),
                 (32, 1, 4096, 0, 32, 8, 128, 0), (1, 1, 256, 0, 8, 2, 64, 0),
                 (8, 1, 65536, 2048, 24, 2, 256, 1), (1, 1, 0, 0, 8, 2, 64, 0)]:
        c = ac(*args)
        assert c > 0 and c % 64 == 0 and c == ac(*args)
        S, T, Lmax, B = args[:4]
        w = min(B, Lmax) if B else Lmax
        assert c <= max(64, (w + 63) // 64 * 64)
    # the 32K int8 decode gets one workgroup per compute unit: 8 seqs x 2 KV
    # heads x 16 splits of 2048 cells; uneven batches get >= 8 splits per window
    assert ac(8, 1, 32768, 0, 24, 2, 256, 1) == 2048
    assert ac(32, 1, 4096, 0, 32, 8, 128, 0) == 512
    assert ac(8, 1, 32768, 0, 25, 2, 256, 1) == _lib.GQA_ERR_GROUP
    # the TurboQuant cache is planned for eight workgroups per compute unit
    assert ac(4, 1, 131072, 0, 32, 8, 128, 2) == 2048
    assert ac(4, 1, 131072, 0, 32, 8, 128, 3) == _lib.GQA_ERR_SHAPE


def test_auto_pieces_plan():
    ap = gq.gqa_decode_auto_pieces
    # one workgroup per compute unit: 256 / (KV heads x row blocks), a
    # multiple of 8 when at least 8, returned as the chunk argument (-P)
    assert ap(32, 1, 4096, 32, 8, 128, 0) == -32         # the f16 batch
    assert ap(8, 1, 32768, 24, 2, 256, 1) == -128        # int8, 2 KV heads
    assert ap(4, 4, 260, 32, 2, 256, 1) == -64           # two row blocks (64 rows at hd 256)
    assert ap(1, 1, 256, 24, 3, 64, 0) == -80            # 256 / 3 = 85 -> 80
    assert ap(1, 1, 256, 512, 512, 64, 0) == -1
    assert ap(1, 1, 256, 8, 2, 64, 2) == _lib.GQA_ERR_SHAPE          # no TurboQuant form
    assert ap(1 << 20, 1, 1 << 20, 8, 2, 64, 0) == _lib.GQA_ERR_CHUNK  # total window past 2^31
    assert ap(1, 1, 256, 9, 2, 64, 0) == _lib.GQA_ERR_GROUP
    for args in [(32, 1, 4096, 32, 8, 128, 0), (8, 1, 32768, 24, 2, 256, 1)]:
        P = -ap(*args)
        S, T, Lmax, H, Hk, D, _ = args
        assert gq.gqa_decode_part_bytes(S, T, Lmax, 0, H, D, -P) == \
            S * T * H * P * (D + 2) * 4 + (S * 4 + 15) // 16 * 16


def test_python_wrapper_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 8, 64)
    k = torch.zeros(1, 4, 2, 64, dtype=torch.float16)
    with pytest.raises(ValueError, match="GPU"):
        gq.decode_attention(q, k, k, torch.ones(1, dtype=torch.int32))


def test_select_rejects():
    f = gq.gqa_decode_select_ids
    assert f(None, FAKE, FAKE, 1, 1, 64, 8, 0) == _lib.GQA_ERR_NULL
    assert f(FAKE, FAKE, None, 1, 1, 64, 8, 0) == _lib.GQA_ERR_NULL
    assert f(FAKE, FAKE, FAKE, 0, 1, 64, 8, 0) == _lib.GQA_ERR_SHAPE
    assert f(FAKE, FAKE, FAKE, 1, 1, -4, 8, 0) == _lib.GQA_ERR_SHAPE
    assert f(FAKE, FAKE, FAKE, 1, 1, 64, 0, 0) == _lib.GQA_ERR_BUDGET


def test_append_rejects():
    f = gq.gqa_decode_append_i8
    args = [FAKE] * 7
    assert f(*args, 0, 1, 16, 2, 64, 0) == _lib.GQA_ERR_SHAPE
    assert f(*args, 1, -1, 16, 2, 64, 0) == _lib.GQA_ERR_SHAPE
    assert f(*args, 1, 1, 16, 2, 96, 0) == _lib.GQA_ERR_HEAD_DIM
    assert f(*([None] + [FAKE] * 6), 1, 1, 16, 2, 64, 0) == _lib.GQA_ERR_NULL
    assert f(*([None] * 7), 1, 0, 16, 2, 64, 0) == _lib.GQA_OK      # nothing to write
    # a grid past 2^31 - 1 workgroups (8 groups each, K and V): refused
    # before any launch; S = 2^30 overflows a 32-bit 2 * S
    assert f(*args, 1 << 30, 1, 16, 1, 64, 0) == _lib.GQA_ERR_SHAPE
    assert f(*args, 1, 1 << 30, 16, 8, 64, 0) == _lib.GQA_ERR_SHAPE


def test_stream_read_rejects():
    f = gq.gqa_bench_stream_read
    assert f(None, 64, FAKE, 4, 0) == _lib.GQA_ERR_NULL
    assert f(FAKE, 64, None, 4, 0) == _lib.GQA_ERR_NULL
    assert f(FAKE, 63, FAKE, 4, 0) == _lib.GQA_ERR_SHAPE      # not a multiple of 16 bytes
    assert f(FAKE + 8, 64, FAKE, 4, 0) == _lib.GQA_ERR_SHAPE  # misaligned
    assert f(FAKE, 64, FAKE, 0, 0) == _lib.GQA_ERR_SHAPE


@pytest.mark.parametrize("case", ["scales_short", "scales_missing", "ids_rows", "k_heads_dim",
                                  "lens_len", "v_shape"])
def test_python_wrapper_checks_shapes_before_launch(case):
    """The kernels address every array from the shapes, so the wrapper
    rejects arrays smaller than the shapes imply (checked before the device
    check, so this runs without a GPU)."""
    import torch
    S, T, H, Hk, D, Lmax = 2, 1, 8, 2, 64, 16
    q = torch.zeros(S, T, H, D)
    k = torch.zeros(S, Lmax, Hk, D, dtype=torch.int8)
    v = k.clone()
    ks = torch.zeros(S, Lmax, Hk, D // 64, dtype=torch.float16)
    vs = ks.clone()
    lens = torch.ones(S, dtype=torch.int32)
    ids = None
    if case == "scales_short":
        vs = torch.zeros(S, Lmax - 1, Hk, D // 64, dtype=torch.float16)
    elif case == "scales_missing":
        vs = None
    elif case == "ids_rows":
        ids = torch.zeros(S, T + 1, 4, dtype=torch.int32)
    elif case == "k_heads_dim":
        k = torch.zeros(S, Lmax, Hk, 2 * D, dtype=torch.int8)
        v = k.clone()
    elif case == "lens_len":
        lens = torch.ones(S + 1, dtype=torch.int32)
    elif case == "v_shape":
        v = torch.zeros(S, Lmax - 1, Hk, D, dtype=torch.int8)
    with pytest.raises(ValueError) as e:
        gq.decode_attention(q, k, v, lens, k_scales=ks, v_scales=vs, ids=ids)
    assert "GPU" not in str(e.value)


def test_select_wrapper_checks_capacity_against_scores():
    import torch
    bs = torch.zeros(1, 1, 2)                      # Lmax // 4 + 1 = 2: Lmax in 4..7
    with pytest.raises(ValueError, match="Lmax"):
        gq.select_ids(bs, torch.ones(1, dtype=torch.int32), 8, Lmax=8)


def test_static_step_rejects_before_any_gpu_call():
    # shape errors, and partials beyond the static buffer, are refused on the
    # host before the buffer's device address is looked up
    def step(**kw):
        a = dict(S=8, T=1, Lmax=32768, B=0, H=24, Hk=2, D=256, chunk=0, kv_kind=1, ids=None)
        a.update(kw)
        return gq.gqa_decode_step_static(FAKE, FAKE, FAKE, FAKE, FAKE, a["ids"], FAKE, FAKE,
                                         a["S"], a["T"], a["Lmax"], a["B"], a["H"], a["Hk"],
                                         a["D"], 0.0625, a["chunk"], a["kv_kind"], 0)
    # 8 x 24 rows x 1024 splits of 32 cells x 258 floats = 203 MB > 16 MiB
    assert step(chunk=32) == _lib.GQA_ERR_STATIC_LIMIT
    assert gq.gqa_decode_part_bytes(8, 1, 32768, 0, 24, 256, 32) > _lib.GQA_STATIC_PART_BYTES
    assert step(kv_kind=2) == _lib.GQA_ERR_SHAPE
    assert step(H=25) == _lib.GQA_ERR_GROUP
    assert step(D=96) == _lib.GQA_ERR_HEAD_DIM
    assert step(ids=FAKE, B=0) == _lib.GQA_ERR_BUDGET
    for i in (0, 6, 7):                          # q, seq_lens, out
        args = [FAKE] * 8
        args[i] = None
        assert gq.gqa_decode_step_static(*args, 1, 1, 16, 0, 8, 2, 64, 0.125, 0, 0, 0) == \
            _lib.GQA_ERR_NULL
    assert "static" in gq.strerror(_lib.GQA_ERR_STATIC_LIMIT)


def test_workspace_size_never_wraps():
    # 2^30 output rows x 2^30 one-cell splits x 258 floats is beyond any
    # address space: the size is refused (0) rather than wrapped modulo 2^64,
    # and the calls refuse the shape before looking at the workspace
    S, H, Lmax, D = 1 << 15, 1 << 15, 1 << 30, 256
    assert gq.gqa_decode_part_bytes(S, 1, Lmax, 0, H, D, 1) == 0
    assert gq.gqa_decode_part_bytes(S, 1, Lmax, 0, H, D, 1 << 20) > 0
    assert attn_f16(S=S, H=H, Hk=1, Lmax=Lmax, D=D, chunk=1, part_bytes=1 << 62) == _lib.GQA_ERR_SHAPE
    assert gq.gqa_decode_merge(FAKE, FAKE, None, FAKE, S, 1, Lmax, 0, H, D, 1, 0) == _lib.GQA_ERR_SHAPE
