"""GPU parity over a seeded random sweep of shapes: every combination the
grid-style tests do not pin one by one (sequence counts that are and are not
multiples of 8, 1-4 KV heads, groups of 1-20 heads, 1-4 causal query tokens,
head dims 64/128/256, f16 and int8 rows, dense or gathered through a budget
of ids, automatic or odd split sizes, lengths from 0 to past the capacity).
A second sweep covers the balanced partition (a negative chunk, or
"balanced"): batches of up to 70 sequences, some with every window of one
length, piece counts that are and are not multiples of 8.
Each case compares every output element with the fp64 oracle to the same
bar as the other parity tests (tests/conftest.py)."""
import numpy as np
import pytest

from conftest import assert_parity
from oracle import decode_ref as R
from workloads import make_case

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

N_CASES = 128
N_LONG = 32
N_BALANCED = 48


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_attention_kv_gqa_amd  # noqa: F401


def draw_case(i, long=False):
    """Case i of the sweep; long: windows of 700-4000 cells, budgets up to
    1200 and splits up to 1500, so that waves run several tiles each."""
    seed = (21000 if long else 9000) + i
    rng = np.random.default_rng(seed)
    S = int(rng.choice([1, 2, 3, 5, 8]))
    T = int(rng.integers(1, 5))
    Hk = int(rng.integers(1, 5))
    G = int(rng.integers(1, 21))
    D = int(rng.choice([64, 128, 256]))
    kv = "i8" if rng.random() < 0.5 else "f16"
    Lmax = int(rng.integers(700, 4001)) if long else int(rng.integers(0, 701))
    lens = rng.integers(0, Lmax + 4, size=S)          # past Lmax clamps to the capacity
    budget = int(rng.integers(1, 1201 if long else 301)) if rng.random() < 0.35 else 0
    chunk = 0 if rng.random() < 0.4 else int(rng.integers(1, 1501 if long else 401))
    return dict(S=S, T=T, Hk=Hk, G=G, D=D, kv=kv, Lmax=Lmax, lens=[int(x) for x in lens],
                budget=budget, chunk=chunk, seed=seed)


def draw_balanced(i):
    """Case i of the balanced-partition sweep (dense windows only)."""
    seed = 33000 + i
    rng = np.random.default_rng(seed)
    S = int(rng.choice([1, 2, 3, 5, 8, 13, 32, 70]))
    T = int(rng.integers(1, 5))
    Hk = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.integers(1, 17))
    D = int(rng.choice([64, 128, 256]))
    kv = "i8" if rng.random() < 0.5 else "f16"
    Lmax = int(rng.integers(1, 801 if S >= 32 else 3001))
    if rng.random() < 0.25:                          # one window length (no pad)
        lens = np.full(S, int(rng.integers(1, Lmax + 1)))
        lens[rng.random(S) < 0.2] = 0
    else:
        lens = rng.integers(0, Lmax + 4, size=S)
    u = rng.random()
    chunk = ("balanced" if u < 0.25 else -8 * int(rng.integers(1, 33)) if u < 0.55
             else -int(rng.integers(1, 401)))
    return dict(S=S, T=T, Hk=Hk, G=G, D=D, kv=kv, Lmax=Lmax, lens=[int(x) for x in lens],
                budget=0, chunk=chunk, seed=seed)


def run_case(c, i):
    import decode_attention_kv_gqa_amd as gq
    inp = make_case(c["S"], c["T"], c["G"] * c["Hk"], c["Hk"], c["D"], c["Lmax"], c["lens"],
                    kv=c["kv"], budget=c["budget"], seed=c["seed"])
    print(f"[gpu] sweep case {i}: {c}", flush=True)
    d = lambda x: None if x is None else torch.from_numpy(np.ascontiguousarray(x)).cuda()
    out = gq.decode_attention(d(inp.q), d(inp.k), d(inp.v), d(inp.seq_lens), inp.scale,
                              k_scales=d(inp.k_scales), v_scales=d(inp.v_scales), ids=d(inp.ids),
                              chunk=c["chunk"])
    torch.cuda.synchronize()
    ref = R.gqa_decode_ref(inp.q, inp.k, inp.v, inp.seq_lens, inp.scale, inp.k_scales,
                           inp.v_scales, inp.ids)
    assert_parity(out.cpu().numpy(), ref, f"sweep case {i} {c}")


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape(i):
    run_case(draw_case(i), i)


@pytest.mark.parametrize("i", range(N_LONG))
def test_random_long_window(i):
    """Windows of 700-4000 cells: several tiles per wave, the last one
    requesting nothing past the split."""
    run_case(draw_case(i, long=True), i)


@pytest.mark.parametrize("i", range(N_BALANCED))
def test_random_balanced(i):
    """Balanced partition: pieces crossing sequence boundaries, empty and
    equal windows, row blocks, both piece orders."""
    run_case(draw_balanced(i), i)
