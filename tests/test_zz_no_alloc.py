"""gqa_decode_step_static (the decode step for callers that cannot allocate:
partials in the library's static per-GPU buffer) against the workspace entry
points it is a variant of, gqa_decode_attn_* + gqa_decode_merge, on the same
inputs and split: two calls in a row, the second with a smaller input, so the
second reads nothing the first left in the buffer.  Same bar as every parity
test (tests/conftest.py); the kernels and the split are the same, so the
outputs are also expected to be bit-identical."""
import numpy as np
import pytest

from conftest import assert_parity
from workloads import make_case

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_attention_kv_gqa_amd  # noqa: F401  (raises if the library is missing)


def dev(x):
    return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).cuda()


def ptr(t):
    return None if t is None else t.data_ptr()


def workspace_step(inp, d, chunk):
    """The existing entry points with a caller workspace (torch memory)."""
    import decode_attention_kv_gqa_amd as gq
    sh = inp.shape
    i8 = inp.kv == "i8"
    if chunk <= 0:
        chunk = gq.gqa_decode_auto_chunk(sh["S"], sh["T"], sh["Lmax"], sh["B"], sh["H"], sh["Hk"],
                                         sh["D"], int(i8))
    nbytes = gq.gqa_decode_part_bytes(sh["S"], sh["T"], sh["Lmax"], sh["B"], sh["H"], sh["D"],
                                      chunk)
    part = torch.empty(max(1, nbytes // 4), dtype=torch.float32, device="cuda")
    out = torch.empty(inp.q.shape, dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    if i8:
        rc = gq.gqa_decode_attn_i8(ptr(d["q"]), ptr(d["k"]), ptr(d["v"]), ptr(d["ks"]),
                                   ptr(d["vs"]), ptr(d["ids"]), ptr(d["lens"]), ptr(part), nbytes,
                                   sh["S"], sh["T"], sh["Lmax"], sh["B"], sh["H"], sh["Hk"],
                                   sh["D"], inp.scale, chunk, st)
    else:
        rc = gq.gqa_decode_attn_f16(ptr(d["q"]), ptr(d["k"]), ptr(d["v"]), ptr(d["ids"]),
                                    ptr(d["lens"]), ptr(part), nbytes, sh["S"], sh["T"],
                                    sh["Lmax"], sh["B"], sh["H"], sh["Hk"], sh["D"], inp.scale,
                                    chunk, st)
    assert rc == 0, gq.strerror(rc)
    rc = gq.gqa_decode_merge(ptr(part), ptr(d["lens"]), ptr(d["ids"]), ptr(out), sh["S"], sh["T"],
                             sh["Lmax"], sh["B"], sh["H"], sh["D"], chunk, st)
    assert rc == 0, gq.strerror(rc)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def static_step(inp, d, chunk):
    import decode_attention_kv_gqa_amd as gq
    sh = inp.shape
    out = torch.full(inp.q.shape, float("nan"), dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    rc = gq.gqa_decode_step_static(ptr(d["q"]), ptr(d["k"]), ptr(d["v"]), ptr(d["ks"]),
                                   ptr(d["vs"]), ptr(d["ids"]), ptr(d["lens"]), ptr(out), sh["S"],
                                   sh["T"], sh["Lmax"], sh["B"], sh["H"], sh["Hk"], sh["D"],
                                   inp.scale, chunk, int(inp.kv == "i8"), st)
    assert rc == 0, gq.strerror(rc)
    torch.cuda.synchronize()
    return out.cpu().numpy()


CASES = {
    # first call, then a smaller one
    "i8": [(dict(S=8, T=1, H=24, Hk=2, D=256, Lmax=32768, lens=[32768] * 8, kv="i8"), 0),
           (dict(S=3, T=2, H=12, Hk=1, D=256, Lmax=900, lens=[900, 5, 0], kv="i8"), 0)],
    "f16": [(dict(S=4, T=8, H=32, Hk=8, D=128, Lmax=8192, lens=[8192, 8000, 300, 1], kv="f16"), 0),
            (dict(S=2, T=1, H=8, Hk=2, D=64, Lmax=257, lens=[257, 31], kv="f16"), 32)],
    "i8_ids": [(dict(S=8, T=1, H=24, Hk=2, D=256, Lmax=65536, lens=[65536] * 8, kv="i8",
                     budget=2048), 32),
               (dict(S=2, T=3, H=24, Hk=2, D=256, Lmax=1000, lens=[1000, 100], kv="i8",
                     budget=64), 0)],
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_static_step_matches_workspace_step_on_two_calls(name):
    for i, (c, chunk) in enumerate(CASES[name]):
        c = dict(c)
        lens = c.pop("lens")
        inp = make_case(c["S"], c["T"], c["H"], c["Hk"], c["D"], c["Lmax"], lens, kv=c["kv"],
                        budget=c.get("budget", 0), seed=31 + i)
        print(f"[gpu] static step {name} call {i}: shape={inp.shape} chunk={chunk}", flush=True)
        d = dict(q=dev(inp.q), k=dev(inp.k), v=dev(inp.v), ks=dev(inp.k_scales),
                 vs=dev(inp.v_scales), ids=dev(inp.ids), lens=dev(inp.seq_lens))
        ref = workspace_step(inp, d, chunk)
        got = static_step(inp, d, chunk)
        assert_parity(got, ref, f"static step {name} call {i}")
        assert np.array_equal(got, ref), f"static step {name} call {i}: not bit-identical"
