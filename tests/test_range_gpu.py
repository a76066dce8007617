"""GPU parity at the edges of the f16 operand ranges, against the fp64 oracle.

The kernels feed the matrix cores f16 hi + lo operand pairs.  Such a pair
holds ~22 bits, but only between f16's subnormal step (2^-24) and its largest
value (65504).  Two operands can leave that band.
  * The softmax weights (times the int8 V scale).  A long tail of cells
    far below one dominant cell carries real mass in the softmax sum, which
    is kept in fp32, but each weight falls under f16's subnormal step.  The
    first cases check that this mass still reaches the numerator: one sink
    cell plus a long low tail, with constant V (the output must be that
    constant) and with nonzero-mean V.
  * The query.  The pages compute q . k in fp32, so |q * scale| of 1e5 or
    1e-6 is legal input.
Same bar as every parity test (tests/conftest.py)."""
import math

import numpy as np
import pytest

from conftest import assert_parity
from oracle import decode_ref as R
from oracle import tq_ref as TR
from workloads import Inputs, make_case, make_tq_case

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_attention_kv_gqa_amd  # noqa: F401  (raises if the library is missing)


def run_gpu(inp, chunk=0):
    import decode_attention_kv_gqa_amd as gq
    d = lambda x: None if x is None else torch.from_numpy(np.ascontiguousarray(x)).cuda()
    print(f"[gpu] shape={inp.shape} kv={inp.kv} chunk={chunk}", flush=True)
    out = gq.decode_attention(d(inp.q), d(inp.k), d(inp.v), d(inp.seq_lens), inp.scale,
                              k_scales=d(inp.k_scales), v_scales=d(inp.v_scales), ids=d(inp.ids),
                              chunk=chunk)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def oracle(inp):
    return R.gqa_decode_ref(inp.q, inp.k, inp.v, inp.seq_lens, inp.scale, inp.k_scales,
                            inp.v_scales, inp.ids)


# ------------------------------------------------------------ sink + low tail
def sink_case(kv, L, gap, sink_at, const_v, S=2, Hk=2, seed=0):
    """Every query row scores one sink cell `gap` natural units above all
    other cells of its window, whose scores vary by less than ~1e-2 units.
    V is one constant row (const_v) or 1 + noise."""
    D = 128 if kv == "f16" else 256
    G = 4 if kv == "f16" else 12
    H = G * Hk
    scale = 1.0 / math.sqrt(D) if kv == "f16" else 1.0 / 16.0
    rng = np.random.default_rng(seed)
    # queries: dim 0 carries the sink direction, the rest is small noise
    q = (0.01 * rng.standard_normal((S, 1, H, D), dtype=np.float32)).astype(np.float32)
    lens = np.full(S, L, dtype=np.int32)
    if kv == "f16":
        q[..., 0] = 1.0
        k = (0.05 * rng.standard_normal((S, L, Hk, D), dtype=np.float32)).astype(np.float16)
        k[..., 0] = 0
        k[:, sink_at, :, 0] = np.float16(gap / scale)           # score gap = gap
        if const_v:
            v = np.full((S, L, Hk, D), 1.0, dtype=np.float16)
        else:
            v = (1.0 + 0.1 * rng.standard_normal((S, L, Hk, D), dtype=np.float32)).astype(np.float16)
        return Inputs(q=q, k=k, v=v, seq_lens=lens, scale=scale)
    ks = np.float16(0.01)
    k = rng.integers(-3, 4, size=(S, L, Hk, D), dtype=np.int8)
    k[..., 0] = 0
    k[:, sink_at, :, 0] = 127
    k_scales = np.full((S, L, Hk, D // 64), ks, dtype=np.float16)
    q[..., 0] = np.float32(gap / (scale * 127 * float(ks)))
    if const_v:
        v = np.full((S, L, Hk, D), 100, dtype=np.int8)
        v_scales = np.full((S, L, Hk, D // 64), 0.01, dtype=np.float16)
    else:
        v = rng.integers(80, 121, size=(S, L, Hk, D), dtype=np.int8)
        v_scales = rng.uniform(0.005, 0.02, size=(S, L, Hk, D // 64)).astype(np.float16)
    return Inputs(q=q, k=k, v=v, seq_lens=lens, scale=scale, k_scales=k_scales, v_scales=v_scales)


def move_sink(inp, old, new):
    """The sink's key row moves from cell `old` to cell `new`."""
    row = inp.k[:, old, :, 0].copy()
    inp.k[:, old, :, 0] = 0
    inp.k[:, new, :, 0] = row


@pytest.mark.parametrize("kv,L,gap", [("f16", 131072, 17.5), ("i8", 32768, 13.0),
                                      ("i8", 131072, 13.0)])
@pytest.mark.parametrize("const_v", [True, False])
def test_sink_and_long_low_tail(kv, L, gap, const_v):
    inp = sink_case(kv, L, gap, 0, const_v, seed=L % 97 + int(const_v))
    where = 0
    for sink_at in (0, L // 2 + 17):
        move_sink(inp, where, sink_at)
        where = sink_at
        ref = oracle(inp)
        if const_v:
            c = 1.0 if kv == "f16" else 100 * float(np.float16(0.01))
            np.testing.assert_allclose(ref, c, rtol=1e-12)     # the definition's value
        for chunk in (0, L):                     # automatic splits, and one split of the window
            got = run_gpu(inp, chunk)
            assert_parity(got, ref, f"sink {kv} L={L} gap={gap} at {sink_at} const_v={const_v} "
                                    f"chunk={chunk}")


def test_sink_tail_budgeted_ids():
    # the gather path: 4096 of 65536 cells, the sink among them
    L, B = 65536, 4096
    inp = sink_case("i8", L, 13.0, 1000, const_v=False, seed=3)
    rng = np.random.default_rng(9)
    S = inp.q.shape[0]
    ids = np.empty((S, 1, B), dtype=np.int32)
    for s in range(S):
        others = rng.choice(L - 1, size=B - 1, replace=False)
        others = others + (others >= 1000)             # every cell but the sink
        ids[s, 0] = np.sort(np.concatenate([[1000], others]))
    inp.ids = ids
    assert all(1000 in inp.ids[s, 0] for s in range(ids.shape[0]))
    ref = oracle(inp)
    for chunk in (32, 0, B):
        assert_parity(run_gpu(inp, chunk), ref, f"sink budgeted ids chunk={chunk}")


# ------------------------------------------------------------ query range
def scaled_query_case(kv, qmag, ids, seed):
    """|q * scale| of order qmag.  With tiny queries the keys are large, so
    the scores are still of order one and the softmax depends on them."""
    D = 128 if kv == "f16" else 256
    Hk, G, L = 2, (4 if kv == "f16" else 12), 700
    scale = 1.0 / math.sqrt(D) if kv == "f16" else 1.0 / 16.0
    inp = make_case(2, 2, G * Hk, Hk, D, L, [L, 450], kv=kv, seed=seed, scale=scale,
                    budget=(200 if ids else 0))
    rng = np.random.default_rng(seed + 7)
    inp.q[...] = (rng.standard_normal(inp.q.shape) * (qmag / scale)).astype(np.float32)
    if qmag < 1e-3:
        if kv == "f16":
            inp.k[...] = rng.uniform(-6e4, 6e4, size=inp.k.shape).astype(np.float16)
        else:
            inp.k_scales[...] = rng.uniform(500.0, 2000.0, size=inp.k_scales.shape).astype(np.float16)
    return inp


@pytest.mark.parametrize("kv", ["f16", "i8"])
@pytest.mark.parametrize("qmag", [1e5, 1e-6])
@pytest.mark.parametrize("ids", [False, True])
def test_query_magnitudes(kv, qmag, ids):
    inp = scaled_query_case(kv, qmag, ids, seed=int(round(math.log10(qmag))) + 50 + 7 * ids)
    ref = oracle(inp)
    for chunk in (64, 0):
        got = run_gpu(inp, chunk)
        assert_parity(got, ref, f"|q*scale|~{qmag} kv={kv} ids={ids} chunk={chunk}")


def test_query_rows_of_different_magnitudes_in_one_group():
    # each row is normalised on its own: rows of 1e-6, 1 and 1e5 share a workgroup
    inp = scaled_query_case("i8", 1.0, False, seed=77)
    mags = np.array([1e-6, 1.0, 1e5, 3e-2] * 6, dtype=np.float64)[:inp.q.shape[2]]
    inp.q[...] = (inp.q.astype(np.float64) * mags[None, None, :, None]).astype(np.float32)
    ref = oracle(inp)
    for chunk in (64, 0):
        assert_parity(run_gpu(inp, chunk), ref, f"mixed row magnitudes chunk={chunk}")


# ------------------------------------------------------------ TurboQuant
def run_tq(inp, chunk=0):
    import decode_attention_kv_gqa_amd as gq

    def dev(x):
        x = np.ascontiguousarray(x)
        return torch.from_numpy(x.view(np.int32) if x.dtype == np.uint32 else x).cuda()
    print(f"[gpu] tq shape={inp.shape} chunk={chunk}", flush=True)
    out = gq.tq_decode_attention(dev(inp.q_rot), dev(inp.q_jl), dev(inp.k_polar), dev(inp.k_jl),
                                 dev(inp.k_norms), dev(inp.v_polar), dev(inp.v_norms),
                                 dev(inp.seq_lens), dev(inp.signs), inp.centroids, inp.qjl_scale,
                                 inp.scale, chunk=chunk)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def tq_oracle(inp):
    return TR.tq_decode_ref(inp.q_rot, inp.q_jl, inp.k_polar, inp.k_jl, inp.k_norms, inp.v_polar,
                            inp.v_norms, inp.seq_lens, inp.signs, inp.centroids, inp.qjl_scale,
                            inp.scale)


def _f16w(x):
    return np.asarray(x, dtype=np.float16).view(np.uint16).astype(np.uint32)


def test_tq_sink_and_long_low_tail():
    # every cell has the same value codes and norm (so the output is that
    # value, whatever the weights); one sink cell per (sequence, KV head)
    # scores 17.5 natural units above the rest, whose key norm is 0
    S, H, Hk, D, L = 1, 8, 2, 128, 131072
    inp = make_tq_case(S, 1, H, Hk, D, L, [L], seed=13)
    inp.q_rot[...] = np.abs(inp.q_rot)
    inp.k_polar[...] = np.uint32(0xFFFFFFFF)      # every key field on the largest centroid
    inp.v_polar[...] = inp.v_polar[:, :, :1, :]
    inp.v_norms[...] = _f16w(1.25)
    sink = 4321
    c3 = float(inp.centroids[3])
    for s in range(S):
        for g in range(Hk):
            G = H // Hk
            dots = inp.q_rot[s, 0, g * G:(g + 1) * G].astype(np.float64).sum(axis=-1) * c3
            norm = 17.5 / (inp.scale * float(dots.min()))
            inp.k_norms[s, g, :] = 0
            inp.k_norms[s, g, sink] = _f16w(norm)
    ref = tq_oracle(inp)
    for chunk in (0, L):
        assert_parity(run_tq(inp, chunk), ref, f"tq sink chunk={chunk}")


@pytest.mark.parametrize("qmag", [1e5, 3e-6])
def test_tq_query_magnitudes(qmag):
    inp = make_tq_case(2, 2, 8, 2, 128, 600, [600, 300], seed=int(round(-math.log10(qmag))) + 90,
                       scale=1.0)
    rng = np.random.default_rng(5)
    inp.q_rot[...] = (rng.standard_normal(inp.q_rot.shape) * qmag).astype(np.float32)
    inp.q_jl[...] = (rng.standard_normal(inp.q_jl.shape) * qmag).astype(np.float32)
    if qmag < 1e-3:
        # large key norms so the scores stay of order one
        kn = rng.uniform(3e4, 6e4, size=inp.k_norms.shape)
        kr = rng.uniform(0.0, 0.5, size=inp.k_norms.shape)
        inp.k_norms[...] = _f16w(kn) | (_f16w(kr) << np.uint32(16))
    ref = tq_oracle(inp)
    for chunk in (64, 0):
        assert_parity(run_tq(inp, chunk), ref, f"tq |q|~{qmag} chunk={chunk}")
