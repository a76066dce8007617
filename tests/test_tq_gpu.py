"""GPU parity of decode attention over a TurboQuant-compressed cache
(gqa_decode_attn_tq + gqa_decode_merge_tq) against the fp64 oracle
(oracle/tq_ref.py), on identical seeded inputs.  Same bar as the other
attention paths (tests/conftest.py)."""
import numpy as np
import pytest

from conftest import assert_parity
from oracle import tq_ref as R
from workloads import make_tq_case, make_tq_inputs, TQ_WORKLOADS

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_attention_kv_gqa_amd  # noqa: F401


def dev(x):
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint32:
        x = x.view(np.int32)                     # torch has no uint32 arithmetic; bits are kept
    return torch.from_numpy(x).cuda()


def run_tq(inp, chunk=0):
    import decode_attention_kv_gqa_amd as gq
    print(f"[gpu] tq shape={inp.shape} lens={list(inp.seq_lens)[:4]} chunk={chunk}", flush=True)
    out = gq.tq_decode_attention(dev(inp.q_rot), dev(inp.q_jl), dev(inp.k_polar), dev(inp.k_jl),
                                 dev(inp.k_norms), dev(inp.v_polar), dev(inp.v_norms),
                                 dev(inp.seq_lens), dev(inp.signs), inp.centroids, inp.qjl_scale,
                                 inp.scale, chunk=chunk)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def oracle(inp, rows=None):
    return R.tq_decode_ref(inp.q_rot, inp.q_jl, inp.k_polar, inp.k_jl, inp.k_norms, inp.v_polar,
                           inp.v_norms, inp.seq_lens, inp.signs, inp.centroids, inp.qjl_scale,
                           inp.scale, rows=rows)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G", [1, 4])
@pytest.mark.parametrize("T", [1, 3])
def test_tq_small(D, G, T):
    inp = make_tq_case(3, T, 2 * G, 2, D, 700, [700, 333, 0], seed=D + 10 * G + T)
    ref = oracle(inp)
    for chunk in (32, 100, 0):
        got = run_tq(inp, chunk)
        assert_parity(got, ref, f"tq D={D} G={G} T={T} chunk={chunk}")
        assert not got[2].any()                   # empty windows give zeros


@pytest.mark.parametrize("L", [1, 31, 32, 33, 64, 129])
def test_tq_lengths_around_tiles(L):
    inp = make_tq_case(2, 1, 8, 2, 128, 200, [L, max(0, L - 1)], seed=L)
    ref = oracle(inp)
    for chunk in (32, 64, 0):
        assert_parity(run_tq(inp, chunk), ref, f"tq L={L} chunk={chunk}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G,T", [(8, 1), (4, 2), (3, 3), (9, 1)])
def test_tq_rows_around_the_packing_limit(D, G, T):
    # up to 8 rows per KV head share MFMA operands (hi parts in columns 0-7,
    # lo parts in 8-15); 9 rows take the unpacked instance
    inp = make_tq_case(2, T, 2 * G, 2, D, 260, [260, 97], seed=500 + D + 10 * G + T)
    ref = oracle(inp)
    for chunk in (64, 0):
        assert_parity(run_tq(inp, chunk), ref, f"tq rows G={G} T={T} D={D} chunk={chunk}")


def test_tq_two_row_blocks_and_many_rows():
    # 12 query heads per KV head x 2 tokens = 24 rows: two 16-row MFMA blocks;
    # 40 query heads per KV head: two workgroup row blocks
    for H, Hk, T in ((24, 2, 2), (40, 1, 1)):
        inp = make_tq_case(2, T, H, Hk, 64, 300, [300, 150], seed=H + T)
        assert_parity(run_tq(inp, 0), oracle(inp), f"tq rows H={H} Hk={Hk} T={T}")


def test_tq_large_value_norms_and_sharp_scores():
    # value norms above 255 (exact running max) and large scores (scale 4)
    inp = make_tq_case(1, 1, 8, 2, 128, 500, [500], seed=77, scale=4.0)
    v = inp.v_norms.astype(np.uint32)
    big = np.float16(1000.0).view(np.uint16)
    v[0, :, ::7] = big
    inp.v_norms[...] = v
    assert_parity(run_tq(inp, 64), oracle(inp), "tq big value norms, scale 4")


def test_tq_full_size():
    # the bench's TurboQuant workload in its launch configuration, every
    # output element (the oracle decodes each (sequence, KV head) once)
    inp = make_tq_inputs("tq_128k")
    got = run_tq(inp, 0)
    print("[gpu] tq_128k: oracle", flush=True)
    assert_parity(got, oracle(inp), "tq_128k")


def test_tq_step_replays_under_graph_capture():
    # attention + merge (with the inverse rotation) captured into a HIP graph:
    # every replay, with eager work between replays, gives the eager result
    import decode_attention_kv_gqa_amd as gq
    inp = make_tq_case(2, 1, 8, 2, 128, 400, [400, 150], seed=21)
    print("[gpu] tq graph capture", flush=True)
    x = {k: dev(getattr(inp, k)) for k in ("q_rot", "q_jl", "k_polar", "k_jl", "k_norms",
                                           "v_polar", "v_norms", "seq_lens", "signs")}
    S, T, H, D = inp.q_rot.shape
    Hk, Lmax = inp.k_polar.shape[1], inp.k_polar.shape[2]
    step = gq.TqDecodeAttention(S, T, H, Hk, D, Lmax, chunk=0, device="cuda")

    def one():
        step.attn(x["q_rot"], x["q_jl"], x["k_polar"], x["k_jl"], x["k_norms"], x["v_polar"],
                  x["v_norms"], x["seq_lens"], inp.centroids, inp.qjl_scale, inp.scale)
        step.merge(x["seq_lens"], x["signs"])

    one()
    torch.cuda.synchronize()
    eager = step.out.clone()
    assert_parity(eager.cpu().numpy(), oracle(inp), "tq eager")
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            one()
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    for r in range(4):
        step.out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(step.out, eager), f"replay {r}"
        one()
        torch.cuda.synchronize()
        assert torch.equal(step.out, eager)


def _sweep_case(i, long=False):
    """Case i of the sweep; long: windows of 800-4000 cells and splits up to
    1500, so that waves run several tiles each."""
    rng = np.random.default_rng((31000 if long else 8000) + i)
    S = int(rng.integers(1, 5))
    T = int(rng.integers(1, 4))
    Hk = int(rng.integers(1, 5))
    G = int(rng.integers(1, 13))
    D = int(rng.choice([64, 128]))
    Lmax = int(rng.integers(800, 4001)) if long else int(rng.integers(0, 801))
    lens = [int(x) for x in rng.integers(0, Lmax + 3, size=S)]
    chunk = 0 if rng.random() < 0.4 else int(rng.integers(1, 1501 if long else 301))
    return S, T, Hk, G, D, Lmax, lens, chunk


@pytest.mark.parametrize("i", range(32))
def test_tq_random_shapes(i):
    """Seeded random shapes (1-4 sequences, 1-3 causal tokens, 1-4 KV heads,
    groups of 1-12, head dim 64/128, lengths 0 to past the capacity, automatic
    or odd splits) against the oracle."""
    S, T, Hk, G, D, Lmax, lens, chunk = _sweep_case(i)
    print(f"[gpu] tq sweep {i}: S={S} T={T} Hk={Hk} G={G} D={D} Lmax={Lmax} lens={lens} "
          f"chunk={chunk}", flush=True)
    inp = make_tq_case(S, T, G * Hk, Hk, D, Lmax, lens, seed=8000 + i)
    assert_parity(run_tq(inp, chunk), oracle(inp), f"tq sweep {i}")


@pytest.mark.parametrize("i", range(16))
def test_tq_random_long_window(i):
    """Windows of 800-4000 cells against the oracle (several tiles per wave)."""
    S, T, Hk, G, D, Lmax, lens, chunk = _sweep_case(i, long=True)
    print(f"[gpu] tq long sweep {i}: S={S} T={T} Hk={Hk} G={G} D={D} Lmax={Lmax} lens={lens} "
          f"chunk={chunk}", flush=True)
    inp = make_tq_case(S, T, G * Hk, Hk, D, Lmax, lens, seed=31000 + i)
    assert_parity(run_tq(inp, chunk), oracle(inp), f"tq long sweep {i}")
