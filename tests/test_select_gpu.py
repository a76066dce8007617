"""GPU parity of the budget selection (gqa_decode_select_ids) against the
oracle (oracle/select_ref.py): ids are integers, so the bar is bit-exact on
the first min(L_t, B) entries of every token; the rest of a row is untouched.
Also the budgeted decode end to end: ids chosen on the GPU feed the int8
gather attention and merge, checked against the fp64 attention oracle."""
import numpy as np
import pytest

from conftest import assert_parity
from oracle import decode_ref as DR
from oracle import select_ref as R
from workloads import make_block_scores, make_case, SELECT_WORKLOADS

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_attention_kv_gqa_amd  # noqa: F401


def run_select(bs, lens, B, Lmax=None):
    import decode_attention_kv_gqa_amd as gq
    print(f"[gpu] select shape={bs.shape} B={B} Lmax={Lmax}", flush=True)
    out = gq.select_ids(torch.from_numpy(bs).cuda(), torch.from_numpy(lens).cuda(), B,
                        Lmax=Lmax)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check(bs, lens, T, Lmax, B):
    got = run_select(bs, lens, B, Lmax)
    ref = R.select_budget_ids(bs, lens, T, Lmax, B)
    assert np.array_equal(got, ref), np.argwhere(got != ref)[:10]


@pytest.mark.parametrize("ties", [False, True])
@pytest.mark.parametrize("Lmax,lens,T,B", [
    (256, [256, 255, 254, 253], 1, 37),     # every n % 4
    (1000, [1000, 40, 3], 3, 64),          # short windows: identity and empty
    (4000, [4000, 2222], 2, 512),
    (400, [400], 1, 400),                  # window == budget: identity
    (400, [401], 1, 399),                  # clamp to Lmax, then select
])
def test_select_small(ties, Lmax, lens, T, B):
    lens = np.asarray(lens, dtype=np.int32)
    bs = make_block_scores(len(lens), T, Lmax, seed=Lmax + B, ties=ties)
    check(bs, lens, T, Lmax, B)


def test_select_signed_zero_and_infinities():
    Lmax = 64
    bs = np.zeros((1, 1, Lmax // 4 + 1), dtype=np.float32)
    bs[0, 0, ::3] = -0.0
    bs[0, 0, 5] = np.inf
    bs[0, 0, 7] = -np.inf
    check(bs, np.array([63], dtype=np.int32), 1, Lmax, 21)


@pytest.mark.parametrize("Lmax", [65536, 131072])
def test_select_long_windows(Lmax):
    # more blocks than the 16 per thread kept in registers
    bs = make_block_scores(2, 1, Lmax, seed=Lmax)
    check(bs, np.array([Lmax, Lmax - 3], dtype=np.int32), 1, Lmax, 2048)


@pytest.mark.parametrize("Lmax,B,ties", [(65536, 4096, True), (65536, 4097, False),
                                         (65536, 5000, True), (131072, 9000, False),
                                         (131072, 4097, True)])
def test_select_budgets_past_the_lds_staging(Lmax, B, ties):
    # budgets above 4096 write their ids straight to memory instead of
    # through LDS; 131072 cells also exceed the keys the kernel keeps in LDS
    bs = make_block_scores(2, 2, Lmax, seed=Lmax + B, ties=ties)
    lens = np.array([Lmax, Lmax - 5], dtype=np.int32)
    check(bs, lens, 2, Lmax, B)


def test_select_workload_full_size():
    w = SELECT_WORKLOADS["select_64k"]
    bs = make_block_scores(w["S"], w["T"], w["Lmax"], seed=1000 + w["index"])
    lens = np.full(w["S"], w["Lmax"], dtype=np.int32)
    check(bs, lens, w["T"], w["Lmax"], w["B"])


@pytest.mark.parametrize("chunk", [32, 0])
def test_budgeted_decode_end_to_end(chunk):
    import decode_attention_kv_gqa_amd as gq
    S, T, H, Hk, D, Lmax, B = 2, 2, 24, 2, 256, 3000, 256
    lens = [3000, 700]
    inp = make_case(S, T, H, Hk, D, Lmax, lens, kv="i8", seed=77, scale=1.0 / 16.0)
    bs = make_block_scores(S, T, Lmax, seed=78)
    d = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    ids_gpu = gq.select_ids(d(bs), d(inp.seq_lens), B, Lmax=Lmax)
    out = gq.decode_attention(d(inp.q), d(inp.k), d(inp.v), d(inp.seq_lens), inp.scale,
                              k_scales=d(inp.k_scales), v_scales=d(inp.v_scales), ids=ids_gpu,
                              chunk=chunk)
    torch.cuda.synchronize()
    ids_ref = R.select_budget_ids(bs, inp.seq_lens, T, Lmax, B)
    ids_ref = np.where(ids_ref < 0, 0, ids_ref).astype(np.int32)
    ref = DR.gqa_decode_ref(inp.q, inp.k, inp.v, inp.seq_lens, inp.scale, inp.k_scales,
                            inp.v_scales, ids_ref)
    assert_parity(out.cpu().numpy(), ref, f"select + gather attention chunk={chunk}")


def _sweep_case(i):
    rng = np.random.default_rng(7000 + i)
    S = int(rng.integers(1, 5))
    T = int(rng.integers(1, 4))
    # capacities on both sides of the 28672 keys the kernel stages in LDS
    # (114 688 cells), not always a multiple of 4
    Lmax = int(rng.choice([rng.integers(0, 4001), rng.integers(4001, 140001)]))
    lens = rng.integers(0, Lmax + 3, size=S).astype(np.int32)
    B = int(rng.integers(1, 3001))
    ties = bool(rng.random() < 0.4)
    return S, T, Lmax, lens, B, ties


@pytest.mark.parametrize("i", range(48))
def test_select_random_shapes(i):
    """Seeded random (S, T, capacity, lengths, budget, ties) combinations,
    bit-exact against the oracle."""
    S, T, Lmax, lens, B, ties = _sweep_case(i)
    print(f"[gpu] select sweep {i}: S={S} T={T} Lmax={Lmax} lens={lens.tolist()} B={B} "
          f"ties={ties}", flush=True)
    bs = make_block_scores(S, T, Lmax, seed=7000 + i, ties=ties)
    check(bs, lens, T, Lmax, B)
