"""GPU parity: the HIP library (through the C ABI) against the fp64 oracle on
identical seeded inputs.  Bar: max |gpu - oracle| <= 2e-3 and row-relative
max error <= 1e-3 (tests/conftest.py), on every output element: the small
cases and the full-size workloads, which run in the same launch
configuration the bench times."""
import math
import sys

import numpy as np
import pytest

from conftest import assert_parity
from oracle import decode_ref as R
from workloads import make_case, make_inputs, WORKLOADS

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_attention_kv_gqa_amd  # noqa: F401  (raises if the library is missing)


def to_dev(inp):
    d = lambda x: None if x is None else torch.from_numpy(np.ascontiguousarray(x)).cuda()
    return dict(q=d(inp.q), k=d(inp.k), v=d(inp.v), seq_lens=d(inp.seq_lens),
                k_scales=d(inp.k_scales), v_scales=d(inp.v_scales), ids=d(inp.ids))


def run_gpu(inp, chunk=0, dev=None):
    import decode_attention_kv_gqa_amd as gq
    dev = dev or to_dev(inp)
    print(f"[gpu] shape={inp.shape} kv={inp.kv} chunk={chunk}", flush=True)
    out = gq.decode_attention(dev["q"], dev["k"], dev["v"], dev["seq_lens"], inp.scale,
                              k_scales=dev["k_scales"], v_scales=dev["v_scales"], ids=dev["ids"],
                              chunk=chunk)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def oracle(inp):
    return R.gqa_decode_ref(inp.q, inp.k, inp.v, inp.seq_lens, inp.scale, inp.k_scales,
                            inp.v_scales, inp.ids)


# ---------------------------------------------------------------- golden files
def test_tiny_workload_matches_golden_and_oracle():
    from test_golden import load_golden
    inp = make_inputs("tiny_f16")
    got = run_gpu(inp, chunk=WORKLOADS["tiny_f16"].chunk)
    assert_parity(got, load_golden("tiny_f16.txt"), "tiny_f16 vs golden")
    assert_parity(got, oracle(inp), "tiny_f16 vs oracle")


def test_small_i8_ids_causal_matches_golden():
    from test_golden import load_golden, golden_small_i8_inputs
    inp = golden_small_i8_inputs()
    for chunk in (0, 5, 24):
        got = run_gpu(inp, chunk=chunk)
        assert_parity(got, load_golden("small_i8_ids_causal.txt"), f"small i8 ids chunk={chunk}")
        assert not got[1, 0].any()


# ---------------------------------------------------------------- edge cases
@pytest.mark.parametrize("L", [0, 1, 31, 32, 33, 64, 65, 200])
@pytest.mark.parametrize("kv", ["f16", "i8"])
def test_lengths_around_chunk_boundaries(L, kv):
    inp = make_case(2, 1, 8, 2, 128, 256, [L, max(0, L - 1)], kv=kv, seed=100 + L)
    ref = oracle(inp)
    for chunk in (32, 0):
        got = run_gpu(inp, chunk=chunk)
        assert_parity(got, ref, f"L={L} kv={kv} chunk={chunk}")
        if L == 0:
            assert not got[0].any()


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("G", [1, 4, 6, 12])
@pytest.mark.parametrize("kv", ["f16", "i8"])
def test_head_dims_and_groups(D, G, kv):
    Hk = 2
    inp = make_case(2, 1, G * Hk, Hk, D, 300, [300, 137], kv=kv, seed=D * 31 + G)
    ref = oracle(inp)
    got = run_gpu(inp, chunk=0)
    assert_parity(got, ref, f"D={D} G={G} kv={kv}")


@pytest.mark.parametrize("chunk", [1, 7, 32, 64, 100, 0])
def test_chunk_sizes(chunk):
    inp = make_case(3, 1, 12, 1, 256, 150, [150, 77, 3], kv="i8", seed=7)
    assert_parity(run_gpu(inp, chunk=chunk), oracle(inp), f"chunk={chunk}")


@pytest.mark.parametrize("kv", ["f16", "i8"])
@pytest.mark.parametrize("T", [2, 8])
def test_multi_query_causal(kv, T):
    # seq 1 is shorter than the window: its first tokens see nothing
    inp = make_case(3, T, 16, 4, 128, 400, [400, 3, 129], kv=kv, seed=T)
    ref = oracle(inp)
    for chunk in (32, 0):
        got = run_gpu(inp, chunk=chunk)
        assert_parity(got, ref, f"T={T} kv={kv} chunk={chunk}")
        for t in range(T):
            # sequence 1 holds 3 cells: token t sees 3 - (T - 1 - t) of them
            assert got[1, t].any() == (3 - (T - 1 - t) > 0)


@pytest.mark.parametrize("Hk,G,T", [(2, 12, 1), (4, 3, 4), (4, 16, 1), (6, 2, 8), (2, 17, 1)])
def test_int8_hd256_kv_head_counts(Hk, G, T):
    # int8 head_dim 256 with 2-6 KV heads, up to 16 query rows per KV head
    # (one row block) and 17 (two), one- and four-wave splits
    inp = make_case(3, T, G * Hk, Hk, 256, 300, [300, 170, 2], kv="i8", seed=Hk * 100 + G * 10 + T)
    ref = oracle(inp)
    for chunk in (1, 32, 100, 0):
        got = run_gpu(inp, chunk=chunk)
        assert_parity(got, ref, f"Hk={Hk} G={G} T={T} chunk={chunk}")


@pytest.mark.parametrize("Hk", [1, 2])
def test_int8_large_v_scales_after_a_lagging_max(Hk):
    # Every wave's first tile scores 0 and its later tiles 7.85 (base 2): the
    # lazily moved reference max lags by less than 8, so p reaches ~230.  The
    # last KV head's V scales there are 300: p * scale would overflow f16
    # unless the kernel tracks the exact max in tiles holding scales > 255.
    # With Hk = 2 that head's rows sit at odd 256-byte offsets of the cells.
    D, L = 256, 300
    inp = make_case(1, 1, 4 * Hk, Hk, D, L, [L], kv="i8", scale=1.0 / 16.0, seed=41 + Hk)
    inp.q[...] = 1.0
    inp.k[0, :128] = 0
    inp.k[0, 128:] = 34
    inp.k_scales[...] = np.float16(0.01)
    rng = np.random.default_rng(5)
    inp.v[0, 128:, Hk - 1] = rng.integers(-1, 2, size=(L - 128, D)).astype(np.int8)
    inp.v_scales[0, 128:, Hk - 1] = np.float16(300.0)
    ref = oracle(inp)
    for chunk in (256, 0):
        got = run_gpu(inp, chunk=chunk)
        assert np.isfinite(got).all()
        assert_parity(got, ref, f"large V scales Hk={Hk} chunk={chunk}")


@pytest.mark.parametrize("kv", ["f16", "i8"])
@pytest.mark.parametrize("T", [1, 3])
def test_uneven_batch(kv, T):
    # windows of every kind in one batch (empty, one cell, short, one split,
    # full), several KV heads, splits from 64 cells to the whole window
    D = 128 if kv == "f16" else 256
    lens = [700, 0, 1, 37, 513, 699, 64, 2]
    inp = make_case(8, T, 8, 2, D, 700, lens, kv=kv, seed=31 + T)
    ref = oracle(inp)
    for chunk in (64, 100, 350, 700, 0):
        got = run_gpu(inp, chunk=chunk)
        assert_parity(got, ref, f"uneven kv={kv} T={T} chunk={chunk}")
        assert not got[1].any()


def test_many_short_sequences():
    # 520 sequences of 0..40 cells: 1040 (sequence, KV head) units
    lens = [(7 * i) % 41 for i in range(520)]
    inp = make_case(520, 1, 4, 2, 64, 40, lens, kv="f16", seed=9)
    assert_parity(run_gpu(inp, chunk=8), oracle(inp), "520 sequences")


def test_rows_beyond_one_block():
    # G * T = 64 query rows per KV head: two row blocks, each streams K/V
    inp = make_case(2, 8, 16, 2, 128, 300, [300, 190], kv="f16", seed=5)
    assert_parity(run_gpu(inp, chunk=0), oracle(inp), "64 rows per KV head")


@pytest.mark.parametrize("kv", ["f16", "i8"])
@pytest.mark.parametrize("B,lens", [(64, [500, 40]), (16, [500, 16]), (300, [300, 299])])
def test_budgeted_ids(kv, B, lens):
    inp = make_case(2, 1, 12, 2, 128 if kv == "f16" else 256, 512, lens, kv=kv, budget=B, seed=B)
    ref = oracle(inp)
    for chunk in (32, 7, 0):
        assert_parity(run_gpu(inp, chunk=chunk), ref, f"ids B={B} kv={kv} chunk={chunk}")


def test_unsorted_ids_and_multi_token_ids():
    inp = make_case(2, 3, 8, 2, 64, 256, [256, 100], kv="i8", budget=40, seed=9, sort_ids=False)
    assert_parity(run_gpu(inp, chunk=16), oracle(inp), "unsorted ids, 3 tokens")


@pytest.mark.parametrize("kv", ["f16", "i8"])
def test_out_of_range_ids_are_clamped(kv):
    # ids must lie in [0, L_t) (the header's precondition); one outside
    # [0, Lmax) is clamped on the device, so it reads cell 0 or Lmax - 1 and
    # never an address past the cache: the output equals the oracle's over
    # the clamped ids
    inp = make_case(2, 2, 8, 2, 128, 300, [300, 120], kv=kv, budget=64, seed=41)
    bad = inp.ids.copy()
    bad[0, 0, 3] = -5
    bad[0, 1, 10] = 300
    bad[1, 1, 7] = 1 << 30
    bad[1, 0, 0] = -(1 << 30)
    inp.ids = bad
    got = run_gpu(inp, chunk=16)
    inp.ids = np.clip(bad, 0, 299).astype(np.int32)
    assert_parity(got, oracle(inp), f"clamped ids kv={kv}")


def test_large_scores_stay_finite():
    inp = make_case(1, 1, 8, 2, 128, 500, [500], kv="f16", seed=3, scale=4.0)
    got = run_gpu(inp, chunk=64)
    assert np.isfinite(got).all()
    assert_parity(got, oracle(inp), "scale 4")


def test_empty_cache_capacity():
    inp = make_case(2, 2, 8, 2, 64, 0, [0, 5], kv="f16", seed=1)
    got = run_gpu(inp, chunk=0)
    assert not got.any()


def test_deterministic_and_on_side_stream():
    import decode_attention_kv_gqa_amd as gq
    inp = make_case(2, 1, 24, 2, 256, 2000, [2000, 1500], kv="i8", seed=4)
    dev = to_dev(inp)
    a = run_gpu(inp, dev=dev)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        b = gq.decode_attention(dev["q"], dev["k"], dev["v"], dev["seq_lens"], inp.scale,
                                k_scales=dev["k_scales"], v_scales=dev["v_scales"])
    s.synchronize()
    assert np.array_equal(a, b.cpu().numpy())


@pytest.mark.parametrize("kv,budget", [("i8", 0), ("f16", 0), ("i8", 48)])
def test_step_replays_under_graph_capture(kv, budget):
    # The calls allocate nothing and record no memset, so a caller can
    # capture the step (attention + merge) into a HIP graph.  Each replay,
    # with eager work and synchronisations between replays, must give the
    # eager result bit for bit, and match the oracle.
    import decode_attention_kv_gqa_amd as gq
    D = 256 if kv == "i8" else 128
    inp = make_case(2, 2, 12, 2, D, 700, [700, 300], kv=kv, budget=budget, seed=11 + budget)
    dev = to_dev(inp)
    sh = inp.shape
    step = gq.DecodeAttention(sh["S"], sh["T"], sh["H"], sh["Hk"], sh["D"], sh["Lmax"], kv,
                              B=budget, chunk=0, device="cuda")

    def one():
        step.attn(dev["q"], dev["k"], dev["v"], dev["seq_lens"], inp.scale, dev["k_scales"],
                  dev["v_scales"], dev["ids"])
        step.merge(dev["seq_lens"], dev["ids"])

    print(f"[gpu] graph capture kv={kv} budget={budget}", flush=True)
    one()
    torch.cuda.synchronize()
    eager = step.out.clone()
    assert_parity(eager.cpu().numpy(), oracle(inp), f"eager kv={kv} budget={budget}")
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            one()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for r in range(4):
        step.out.zero_()
        step.part.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(step.out, eager), f"replay {r}"
        one()                                    # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(step.out, eager)


def test_errors_do_not_launch():
    import decode_attention_kv_gqa_amd as gq
    from decode_attention_kv_gqa_amd import _lib
    inp = make_case(1, 1, 8, 2, 64, 64, [64], kv="f16", seed=1)
    dev = to_dev(inp)
    part = torch.empty(16, device="cuda")
    rc = gq.gqa_decode_attn_f16(dev["q"].data_ptr(), dev["k"].data_ptr(), dev["v"].data_ptr(), None,
                                dev["seq_lens"].data_ptr(), part.data_ptr(), 64, 1, 1, 64, 0, 8, 2,
                                64, 0.125, 32, 0)
    assert rc == _lib.GQA_ERR_WORKSPACE


# ---------------------------------------------------------------- full sizes
@pytest.mark.parametrize("name", ["f16_batch", "i8_32k", "i8_budget", "f16_mq_causal"])
def test_full_size_workload(name):
    # the bench's workloads in its launch configuration (and the automatic
    # split where the workload names another), every output element
    w = WORKLOADS[name]
    inp = make_inputs(name)
    print(f"[gpu] full-size workload {name}: oracle", flush=True)
    ref = oracle(inp)
    chunks = [w.chunk] + ([0] if w.chunk else []) + ([32] if name == "i8_budget" else [])
    dev = to_dev(inp)
    for chunk in chunks:
        got = run_gpu(inp, chunk=chunk, dev=dev)
        assert_parity(got, ref, f"{name} chunk={chunk}")


def test_full_size_budgeted_ids_in_drawn_order():
    # the budgeted workload with its ids in the order drawn (not ascending),
    # in the bench's launch configuration, every output element
    w = WORKLOADS["i8_budget"]
    inp = make_inputs("i8_budget", sort_ids=False)
    assert not all(np.all(np.diff(inp.ids[s, t]) > 0) for s in range(inp.ids.shape[0])
                   for t in range(inp.ids.shape[1]))
    print("[gpu] full-size i8_budget, ids unsorted: oracle", flush=True)
    ref = oracle(inp)
    assert_parity(run_gpu(inp, chunk=w.chunk), ref, "i8_budget unsorted ids")


@pytest.mark.parametrize("kv", ["f16", "i8"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G,T", [(8, 8), (10, 4), (16, 5)])
def test_rows_up_to_64_per_kv_head(kv, D, G, T):
    # 64, 40 and 80 query rows per KV head: one 64-row block (head_dim 64 and
    # 128 serve up to 64 rows from one workgroup, so K/V rows are read once),
    # a ragged block of 40, and two blocks for 80; one- and four-wave splits
    inp = make_case(3, T, G * 2, 2, D, 400, [400, 2, 333], kv=kv, seed=G * 10 + T + D)
    ref = oracle(inp)
    for chunk in (48, 0):
        assert_parity(run_gpu(inp, chunk=chunk), ref, f"rows={G * T} D={D} kv={kv} chunk={chunk}")


@pytest.mark.parametrize("kv", ["f16", "i8"])
def test_64_heads_per_kv_head_with_ids(kv):
    # gather mode holds one token's G query heads per workgroup: G = 64
    inp = make_case(2, 2, 64, 1, 128, 600, [600, 350], kv=kv, budget=100, seed=64)
    ref = oracle(inp)
    for chunk in (32, 0):
        assert_parity(run_gpu(inp, chunk=chunk), ref, f"G=64 ids kv={kv} chunk={chunk}")
