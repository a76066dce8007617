"""GPU parity of gathered attention over caches whose per-sequence rows of
all KV heads span 2^31 bytes or more (past a 32-bit byte offset): the
library switches to 64-bit row addresses there.  The cache is a large
zeroed device array holding, at seeded scattered cells (many of them past
the first 2 GiB of the sequence's plane), the rows of a small seeded case;
the ids point at those cells.  The oracle runs on the small case itself,
which holds exactly the rows the ids select, in the same list order."""
import numpy as np
import pytest

from conftest import assert_parity
from oracle import decode_ref as R
from workloads import make_case

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_attention_kv_gqa_amd  # noqa: F401  (raises if the library is missing)


def spread(inp, Lbig, seed):
    """Device cache of capacity Lbig with the small case's rows at scattered
    cells (the same cells in K, V and scales); returns the device arrays and
    the ids translated to those cells."""
    S, Lc = inp.k.shape[0], inp.k.shape[1]
    rng = np.random.default_rng(seed)
    cells = np.empty((S, Lc), dtype=np.int64)
    for s in range(S):
        # half the rows in the last 2^20 cells, the rest anywhere; the very
        # last cell is always one of them
        hi = rng.choice(np.arange(Lbig - (1 << 20), Lbig - 1), size=Lc // 2, replace=False)
        lo = rng.choice(Lbig - (1 << 20), size=Lc - Lc // 2 - 1, replace=False)
        c = np.concatenate([hi, lo, [Lbig - 1]])
        rng.shuffle(c)
        cells[s] = c
    dev = {}
    for name in ("k", "v", "k_scales", "v_scales"):
        x = getattr(inp, name)
        if x is None:
            dev[name] = None
            continue
        big = torch.zeros((S, Lbig) + x.shape[2:], dtype=torch.from_numpy(x[:1, :1]).dtype,
                          device="cuda")
        for s in range(S):
            big[s, torch.from_numpy(cells[s]).cuda()] = torch.from_numpy(np.ascontiguousarray(x[s])).cuda()
        dev[name] = big
    ids = np.take_along_axis(cells[:, None, :], inp.ids.astype(np.int64), axis=2).astype(np.int32)
    return dev, ids


@pytest.mark.parametrize("kv,D", [("f16", 128), ("i8", 256)])
def test_gather_past_two_gib_of_rows(kv, D):
    import decode_attention_kv_gqa_amd as gq
    S, T, H, Hk, B = 2, 2, 32, 8, 256
    Lc = B + 64                                  # every token's window holds B ids
    row = Hk * D * (1 if kv == "i8" else 2)      # bytes between cells of one sequence
    Lbig = (1 << 31) // row + 4096               # past 2^31 bytes per sequence
    inp = make_case(S, T, H, Hk, D, Lc, [Lc] * S, kv=kv, budget=B, seed=401)
    ref = R.gqa_decode_ref(inp.q, inp.k, inp.v, inp.seq_lens, inp.scale, inp.k_scales,
                           inp.v_scales, inp.ids)
    print(f"[gpu] wide gather kv={kv} D={D} Lmax={Lbig} ({Lbig * row / 2**30:.2f} GiB per "
          f"sequence)", flush=True)
    dev, ids = spread(inp, Lbig, seed=402)
    q = torch.from_numpy(inp.q).cuda()
    lens = torch.full((S,), Lbig, dtype=torch.int32, device="cuda")
    idd = torch.from_numpy(ids).cuda()
    for chunk in (0, 32, 128, 256):
        out = gq.decode_attention(q, dev["k"], dev["v"], lens, inp.scale, k_scales=dev["k_scales"],
                                  v_scales=dev["v_scales"], ids=idd, chunk=chunk)
        torch.cuda.synchronize()
        assert_parity(out.cpu().numpy(), ref, f"wide gather kv={kv} chunk={chunk}")
    del dev
    torch.cuda.empty_cache()
