"""GPU parity of the balanced partition (a negative chunk: the dense windows
of the whole batch, laid end to end, cut into -chunk equal pieces per KV
head, each piece one workgroup that may cross sequence boundaries) against
the fp64 oracle, through the C ABI, on every output element."""
import numpy as np
import pytest

from conftest import assert_parity
from oracle import decode_ref as R
from workloads import make_case, make_inputs

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


def run_gpu(inp, chunk, dev=None, gate=None):
    import decode_attention_kv_gqa_amd as gq
    dev = dev or to_dev(inp)
    print(f"[gpu] balanced shape={inp.shape} kv={inp.kv} chunk={chunk}", flush=True)
    out = gq.decode_attention(dev["q"], dev["k"], dev["v"], dev["seq_lens"], inp.scale,
                              k_scales=dev["k_scales"], v_scales=dev["v_scales"], ids=dev["ids"],
                              chunk=chunk, gate=gate)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def oracle(inp):
    return R.gqa_decode_ref(inp.q, inp.k, inp.v, inp.seq_lens, inp.scale, inp.k_scales,
                            inp.v_scales, inp.ids)


@pytest.mark.parametrize("kv", ["f16", "i8"])
@pytest.mark.parametrize("T", [1, 3])
def test_uneven_batch_every_piece_count(kv, T):
    # empty, one-cell, short and full windows; from one piece for the whole
    # batch to more pieces than cells (then every cell is a piece)
    D = 128 if kv == "f16" else 256
    lens = [700, 0, 1, 37, 513, 699, 64, 2]
    inp = make_case(8, T, 8, 2, D, 700, lens, kv=kv, seed=131 + T)
    ref = oracle(inp)
    for P in (1, 2, 3, 7, 16, 64, 3000):
        got = run_gpu(inp, -P)
        assert_parity(got, ref, f"balanced kv={kv} T={T} P={P}")
        assert not got[1].any()


@pytest.mark.parametrize("kv", ["f16", "i8"])
def test_lengths_past_capacity_and_negative(kv):
    # seq_lens beyond Lmax clamp to the capacity, negative ones to empty
    D = 64 if kv == "f16" else 128
    inp = make_case(5, 2, 8, 4, D, 300, [300, 900, -5, 299, 1], kv=kv, seed=77)
    ref = oracle(inp)
    for P in (1, 5, 33):
        got = run_gpu(inp, -P)
        assert_parity(got, ref, f"capacity kv={kv} P={P}")
        assert not got[2].any()


def test_all_windows_empty():
    inp = make_case(3, 1, 8, 2, 64, 50, [0, 0, -1], kv="f16", seed=3)
    for P in (1, 8):
        got = run_gpu(inp, -P)
        assert not got.any()


def test_more_than_64_sequences():
    # the lengths are walked 64 sequences per pass
    rng = np.random.default_rng(12)
    lens = rng.integers(0, 90, size=200)
    lens[::17] = 0
    inp = make_case(200, 1, 4, 2, 64, 90, lens, kv="f16", seed=19)
    ref = oracle(inp)
    for P in (1, 13, 64, 256):
        assert_parity(run_gpu(inp, -P), ref, f"200 sequences P={P}")


@pytest.mark.parametrize("kv", ["f16", "i8"])
def test_row_blocks_with_causal_tokens(kv):
    # head_dim 256 keeps 32 rows per block: 16 heads x 4 tokens = two blocks,
    # whose windows differ by the causal clamp (a block can see nothing of a
    # segment another block sees)
    inp = make_case(4, 4, 32, 2, 256, 260, [260, 3, 2, 130], kv=kv, seed=41)
    ref = oracle(inp)
    for P in (1, 4, 9, 100):
        assert_parity(run_gpu(inp, -P), ref, f"row blocks kv={kv} P={P}")


@pytest.mark.parametrize("kv", ["f16", "i8"])
@pytest.mark.parametrize("D", [64, 128])
def test_64_rows_per_kv_head(kv, D):
    inp = make_case(3, 8, 16, 2, D, 400, [400, 17, 250], kv=kv, seed=43)
    ref = oracle(inp)
    for P in (2, 11):
        assert_parity(run_gpu(inp, -P), ref, f"64 rows kv={kv} D={D} P={P}")


def test_gated_merge():
    from oracle.gate_ref import apply_gate
    inp = make_case(6, 1, 16, 4, 128, 500, [500, 12, 0, 333, 499, 64], kv="f16", seed=51)
    g = np.random.default_rng(5).standard_normal(inp.q.shape).astype(np.float32) * 3
    ref = apply_gate(oracle(inp), g)
    got = run_gpu(inp, -10, gate=torch.from_numpy(g).cuda())
    assert_parity(got, ref, "gated balanced")


def test_agrees_with_splits_and_is_deterministic():
    inp = make_case(8, 1, 32, 8, 128, 1024, [1024, 512, 900, 7, 1, 640, 1000, 333], kv="f16",
                    seed=61)
    dev = to_dev(inp)
    a = run_gpu(inp, -24, dev=dev)
    b = run_gpu(inp, -24, dev=dev)
    assert np.array_equal(a, b)
    assert_parity(a, run_gpu(inp, 0, dev=dev), "balanced vs splits")


def test_step_replays_under_graph_capture():
    import decode_attention_kv_gqa_amd as gq
    inp = make_case(6, 1, 16, 4, 128, 700, [700, 5, 0, 321, 650, 90], kv="f16", seed=71)
    d = to_dev(inp)
    step = gq.DecodeAttention(6, 1, 16, 4, 128, 700, "f16", chunk=-16)

    def one():
        step(d["q"], d["k"], d["v"], d["seq_lens"], inp.scale)

    one()
    torch.cuda.synchronize()
    eager = step.out.clone()
    assert_parity(eager.cpu().numpy(), oracle(inp), "balanced eager")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        one()
        s.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            one()
    torch.cuda.synchronize()
    for r in range(4):
        step.out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(step.out, eager), f"replay {r}"
        one()
        torch.cuda.synchronize()
        assert torch.equal(step.out, eager)


def test_static_step_takes_the_balanced_partition():
    import decode_attention_kv_gqa_amd as gq
    inp = make_case(5, 1, 8, 2, 128, 600, [600, 0, 37, 599, 300], kv="i8", seed=81)
    d = to_dev(inp)
    out = torch.empty(inp.q.shape, dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    for P in (7, 3):
        out.fill_(float("nan"))
        rc = gq.gqa_decode_step_static(*[d[n].data_ptr() for n in ("q", "k", "v", "k_scales",
                                                                    "v_scales")],
                                       None, d["seq_lens"].data_ptr(), out.data_ptr(), 5, 1, 600,
                                       0, 8, 2, 128, inp.scale, -P, 1, st)
        assert rc == 0, gq.strerror(rc)
        torch.cuda.synchronize()
        assert_parity(out.cpu().numpy(), oracle(inp), f"static balanced P={P}")


@pytest.mark.parametrize("kv,H,Hk,D", [("i8", 24, 2, 256), ("f16", 32, 8, 128), ("i8", 16, 4, 64),
                                        ("f16", 24, 2, 256), ("i8", 32, 8, 128)])
def test_balanced_keyword_on_uneven_batches(kv, H, Hk, D):
    # chunk="balanced": the piece count the library picks (256 workgroups;
    # int8 with a piece count divisible by 8 gives each XCD a contiguous
    # eighth of the pieces, every KV head of each)
    rng = np.random.default_rng(91)
    lens = rng.integers(0, 3000, size=24)
    lens[[2, 9]] = 0
    lens[5] = 3000
    inp = make_case(24, 1, H, Hk, D, 3000, lens, kv=kv, seed=93)
    assert_parity(run_gpu(inp, "balanced"), oracle(inp), f"balanced keyword kv={kv} D={D}")


@pytest.mark.parametrize("P", [32, 64])
def test_full_size_f16_batch(P):
    inp = make_inputs("f16_batch")
    print("[gpu] full-size f16_batch: oracle", flush=True)
    ref = oracle(inp)
    assert_parity(run_gpu(inp, -P), ref, f"f16_batch P={P}")


def test_full_size_int8_batch():
    # the int8 batch of uneven lengths the bench times, in its launch
    # configuration (128 pieces per KV head) and with the automatic split
    from workloads import WORKLOADS
    inp = make_inputs("i8_batch")
    print("[gpu] full-size i8_batch: oracle", flush=True)
    ref = oracle(inp)
    dev = to_dev(inp)
    for chunk in (WORKLOADS["i8_batch"].chunk, 0):
        assert_parity(run_gpu(inp, chunk, dev=dev), ref, f"i8_batch chunk={chunk}")


@pytest.mark.parametrize("kv", ["f16", "i8"])
def test_equal_windows_and_merge_depths(kv):
    # windows all of one length (empty ones aside) take no pad; piece counts
    # from under one to 64 per sequence cover every merge prefetch depth
    D = 128
    for lens in ([777] * 4, [777, 0, 777, 777], [1] * 4):
        inp = make_case(4, 2, 16, 4, D, 777, lens, kv=kv, seed=101 + lens[1])
        ref = oracle(inp)
        for P in (1, 3, 4, 13, 24, 40, 256):
            assert_parity(run_gpu(inp, -P), ref, f"equal windows kv={kv} lens={lens} P={P}")
