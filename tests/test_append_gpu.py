"""GPU parity of quantize-on-append (gqa_decode_append_i8) against the oracle
(oracle/append_ref.py): codes and f16 scales are decided in fp32 on both
sides, so the bar is bit-exact on every cache row, written or not.  Also
append-then-attend: rows quantised on the GPU feed the int8 attention."""
import numpy as np
import pytest

from conftest import assert_parity
from oracle import append_ref as AR
from oracle import decode_ref as DR
from workloads import make_append_rows, make_case, APPEND_WORKLOADS

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_attention_kv_gqa_amd  # noqa: F401


def run_append(kn, vn, pos, k, v, ks, vs):
    import decode_attention_kv_gqa_amd as gq
    d = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    print(f"[gpu] append new={kn.shape} cache={k.shape}", flush=True)
    kk, vv, kks, vvs = d(k), d(v), d(ks), d(vs)
    gq.append_i8(d(kn), d(vn), d(pos), kk, vv, kks, vvs)
    torch.cuda.synchronize()
    return kk.cpu().numpy(), vv.cpu().numpy(), kks.cpu().numpy(), vvs.cpu().numpy()


def check(S, Tn, Hk, D, Lmax, pos, seed, scale_rows=None):
    kn, vn = make_append_rows(S, Tn, Hk, D, seed=seed)
    if scale_rows is not None:
        kn = (kn * scale_rows).astype(np.float32)
        vn = (vn * scale_rows).astype(np.float32)
    rng = np.random.default_rng(seed + 1)
    k = rng.integers(-127, 128, (S, Lmax, Hk, D), dtype=np.int8)
    v = rng.integers(-127, 128, (S, Lmax, Hk, D), dtype=np.int8)
    ks = rng.uniform(0.005, 0.02, (S, Lmax, Hk, D // 64)).astype(np.float16)
    vs = rng.uniform(0.005, 0.02, (S, Lmax, Hk, D // 64)).astype(np.float16)
    pos = np.asarray(pos, dtype=np.int32)
    got = run_append(kn, vn, pos, k, v, ks, vs)
    ref = AR.append_i8(kn, vn, pos, k, v, ks, vs)
    for name, g, r in zip(("k", "v", "k_scales", "v_scales"), got, ref):
        assert np.array_equal(g.view(np.uint8 if g.dtype == np.int8 else np.uint16),
                              r.view(np.uint8 if r.dtype == np.int8 else np.uint16)), name


@pytest.mark.parametrize("D", [64, 128, 256, 192])
def test_append_small(D):
    check(3, 5, 2, D, 40, [0, 17, 38], seed=D)            # the last runs past Lmax


def test_append_wide_dynamic_range_and_zeros():
    S, Tn, Hk, D = 2, 7, 3, 128
    mag = (10.0 ** np.random.default_rng(0).uniform(-30, 30, (S, Tn, Hk, 1))).astype(np.float32)
    mag[0, 0, 0, 0] = 0.0                                  # an all-zero row
    check(S, Tn, Hk, D, 20, [3, -2], seed=9, scale_rows=mag)   # negative position truncates


def test_append_half_way_codes():
    # d = 1 exactly: codes of x.5 values round to even on both sides
    S, Tn, Hk, D = 1, 1, 1, 64
    import decode_attention_kv_gqa_amd as gq  # noqa: F401
    x = np.zeros((S, Tn, Hk, D), dtype=np.float32)
    x[..., 0] = 127.0
    x[..., 1:9] = [0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5, -126.5]
    k = np.zeros((S, 4, Hk, D), dtype=np.int8)
    ks = np.zeros((S, 4, Hk, 1), dtype=np.float16)
    got = run_append(x, x, np.array([1], dtype=np.int32), k, k.copy(), ks, ks.copy())
    ref = AR.append_i8(x, x, np.array([1], dtype=np.int32), k, k.copy(), ks, ks.copy())
    assert np.array_equal(got[0], ref[0]) and list(got[0][0, 1, 0, :9]) == [127, 0, 2, 2, 0, -2, -2, 126, -126]


def _append_exact(x, Lmax=4, pos=1):
    """Append x [S][Tn][Hk][D] as both K and V; codes and scales must equal
    the oracle's bit for bit."""
    S, Tn, Hk, D = x.shape
    k = np.zeros((S, Lmax, Hk, D), dtype=np.int8)
    ks = np.zeros((S, Lmax, Hk, D // 64), dtype=np.float16)
    p = np.full(S, pos, dtype=np.int32)
    got = run_append(x, x, p, k, k.copy(), ks, ks.copy())
    ref = AR.append_i8(x, x, p, k, k.copy(), ks, ks.copy())
    for name, g, r in zip(("k", "v", "k_scales", "v_scales"), got, ref):
        assert np.array_equal(g.view(np.uint8 if g.dtype == np.int8 else np.uint16),
                              r.view(np.uint8 if r.dtype == np.int8 else np.uint16)), name
    return got


def test_append_quotients_next_to_half_integers():
    # x / d within a few ulp of k + 1/2 for many k and scales: the codes
    # still follow the IEEE quotient rounded half to even
    rng = np.random.default_rng(77)
    rows = []
    for scale in (1.0, 0.37, 3.1e-3, 7.7e4, 1.3e-20):
        m = np.float32(127.0 * scale)
        d = np.float32(m / np.float32(127.0))
        for _ in range(8):
            ks = rng.integers(-127, 127, size=63) + 0.5
            x = (ks * np.float64(d)).astype(np.float32)
            steps = rng.integers(-3, 4, size=63)
            x = np.array([np.float32(v) if t == 0 else
                          np.nextafter(np.float32(v), np.float32(np.sign(t) * np.inf), dtype=np.float32)
                          if abs(t) == 1 else
                          (np.float32(v) + np.float32(t) * np.spacing(np.float32(v))).astype(np.float32)
                          for v, t in zip(x, steps)], dtype=np.float32)
            x = np.clip(x, -m, m)
            rows.append(np.concatenate([[m], x]).astype(np.float32))
    x = np.stack(rows).reshape(1, len(rows), 1, 64)
    got = _append_exact(x, Lmax=len(rows) + 2, pos=1)
    assert np.count_nonzero(got[0]) > 0


def test_append_tiny_and_subnormal_groups():
    # groups whose max |x| is subnormal, at and around 2^-100, and normal
    rng = np.random.default_rng(78)
    mags = np.array([1e-45, 3e-42, 1e-40, 1.1754942e-38, 2.0 ** -126, 2.0 ** -101,
                     2.0 ** -100 * (1 - 2.0 ** -23), 2.0 ** -100, 2.0 ** -100 * (1 + 2.0 ** -23),
                     1e-30, 1.0, 1e37], dtype=np.float64)
    x = (rng.standard_normal((1, len(mags), 1, 128)) * mags[None, :, None, None])
    x = x.astype(np.float32)
    assert np.isfinite(x).all()                    # finite inputs only (the contract)
    x[0, 0, 0, :3] = [1e-45, -1e-45, 0.0]          # the smallest subnormals
    _append_exact(x, Lmax=len(mags) + 1, pos=0)


def test_append_bench_shape():
    # the quantize-on-append workload as the bench times it: 8 sequences x
    # 4096 new rows, 2 KV heads, head_dim 256, into a 32768-cell cache at 16384
    w = APPEND_WORKLOADS["append_i8"]
    check(w["S"], w["Tn"], w["Hk"], w["D"], w["Lmax"], [w["pos"]] * w["S"],
          seed=1000 + w["index"])


def test_append_workload_full_size():
    w = APPEND_WORKLOADS["append_i8"]
    S, Tn, Hk, D, Lmax = w["S"], 512, w["Hk"], w["D"], 2048   # the workload's rows, a smaller cache
    check(S, Tn, Hk, D, Lmax, [1024] * S, seed=1000 + w["index"])


def test_append_then_attend():
    import decode_attention_kv_gqa_amd as gq
    S, T, H, Hk, D, Lmax = 2, 1, 24, 2, 256, 600
    inp = make_case(S, T, H, Hk, D, Lmax, [600, 450], kv="i8", seed=21, scale=1.0 / 16.0)
    Tn = 100
    kn, vn = make_append_rows(S, Tn, Hk, D, seed=22)
    pos = np.array([500, 350], dtype=np.int32)            # the new rows end each window
    d = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    k, v, ks, vs = d(inp.k), d(inp.v), d(inp.k_scales), d(inp.v_scales)
    gq.append_i8(d(kn), d(vn), d(pos), k, v, ks, vs)
    out = gq.decode_attention(d(inp.q), k, v, d(inp.seq_lens), inp.scale, k_scales=ks, v_scales=vs)
    torch.cuda.synchronize()
    rk, rv, rks, rvs = AR.append_i8(kn, vn, pos, inp.k, inp.v, inp.k_scales, inp.v_scales)
    ref = DR.gqa_decode_ref(inp.q, rk, rv, inp.seq_lens, inp.scale, rks, rvs)
    assert_parity(out.cpu().numpy(), ref, "append then attend")


@pytest.mark.parametrize("i", range(24))
def test_append_random_shapes(i):
    """Seeded random (S, Tn, Hk, D, capacity, positions) combinations, with
    positions that start before the cache, inside it, and run past its end;
    bit-exact against the oracle on every cache row."""
    rng = np.random.default_rng(6000 + i)
    S = int(rng.integers(1, 5))
    Tn = int(rng.integers(1, 40))
    Hk = int(rng.integers(1, 5))
    D = int(64 * rng.integers(1, 5))
    Lmax = int(rng.integers(1, 120))
    pos = [int(x) for x in rng.integers(-Tn, Lmax + 3, size=S)]
    print(f"[gpu] append sweep {i}: S={S} Tn={Tn} Hk={Hk} D={D} Lmax={Lmax} pos={pos}",
          flush=True)
    check(S, Tn, Hk, D, Lmax, pos, seed=6000 + i)
