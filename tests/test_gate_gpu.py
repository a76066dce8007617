"""GPU parity of the gated merge (gqa_decode_merge_gated) against the fp64
oracle (oracle/gate_ref.py): the decode output times sigmoid(gate), with
the gate as its own tensor and as the second half of [query | gate] rows.
Same bar as the attention parity tests (tests/conftest.py)."""
import numpy as np
import pytest

from conftest import assert_parity
from oracle import decode_ref as DR
from oracle import gate_ref as R
from workloads import make_case, make_inputs, WORKLOADS

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_attention_kv_gqa_amd  # noqa: F401


def dev(x):
    return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).cuda()


def run_gated(inp, gate_t, chunk=0, q_t=None):
    import decode_attention_kv_gqa_amd as gq
    print(f"[gpu] gated shape={inp.shape} kv={inp.kv} chunk={chunk} "
          f"gate_stride={gate_t.stride(2)}", flush=True)
    out = gq.decode_attention(dev(inp.q) if q_t is None else q_t, dev(inp.k), dev(inp.v),
                              dev(inp.seq_lens), inp.scale, k_scales=dev(inp.k_scales),
                              v_scales=dev(inp.v_scales), ids=dev(inp.ids), chunk=chunk,
                              gate=gate_t)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def gate_values(shape, seed, spread=3.0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(shape) * spread).astype(np.float32)


@pytest.mark.parametrize("kv", ["f16", "i8"])
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("layout", ["separate", "query_gate_rows"])
def test_gated_decode(kv, D, layout):
    inp = make_case(3, 2, 8, 2, D, 300, [300, 77, 0], kv=kv, seed=D + (kv == "i8"))
    gate = gate_values(inp.q.shape, seed=D)
    if layout == "separate":
        gate_t = dev(gate)
    else:
        # the pages' layout: one [query | gate] row of 2D floats per (token, head)
        full = dev(np.concatenate([inp.q, gate], axis=-1))
        gate_t = full[..., D:]
        assert gate_t.stride(2) == 2 * D
    ref = R.gqa_decode_gated_ref(inp.q, inp.k, inp.v, inp.seq_lens, inp.scale, gate,
                                 inp.k_scales, inp.v_scales)
    for chunk in (64, 0):
        got = run_gated(inp, gate_t, chunk)
        assert_parity(got, ref, f"gated {kv} D={D} {layout} chunk={chunk}")
        assert not got[2].any()                      # empty windows stay zero


def test_gate_extremes_and_budgeted_ids():
    inp = make_case(2, 1, 24, 2, 256, 3000, [3000, 1200], kv="i8", budget=512, seed=9,
                    scale=1.0 / 16.0)
    gate = gate_values(inp.q.shape, seed=4)
    gate[0, 0, :, :32] = 60.0                        # sigmoid -> 1
    gate[0, 0, :, 32:64] = -60.0                     # sigmoid -> 1e-26
    gate[1, 0, :, :] = 0.0                           # sigmoid = 1/2 exactly
    ref = R.gqa_decode_gated_ref(inp.q, inp.k, inp.v, inp.seq_lens, inp.scale, gate,
                                 inp.k_scales, inp.v_scales, inp.ids)
    got = run_gated(inp, dev(gate), chunk=32)
    assert_parity(got, ref, "gated ids, extreme gates")
    base = DR.gqa_decode_ref(inp.q, inp.k, inp.v, inp.seq_lens, inp.scale, inp.k_scales,
                             inp.v_scales, inp.ids)
    assert np.abs(got[0, 0, :, 32:64]).max() <= 1e-20
    np.testing.assert_allclose(got[1, 0], base[1, 0] * 0.5, rtol=0, atol=2e-3)


def test_gated_full_size_int8_32k():
    # the bench's int8 workload and launch configuration, gate as [query | gate]
    # rows, every output element
    w = WORKLOADS["i8_32k"]
    inp = make_inputs("i8_32k")
    D = inp.q.shape[-1]
    gate = gate_values(inp.q.shape, seed=1000 + w.index)
    full = dev(np.concatenate([inp.q, gate], axis=-1))
    got = run_gated(inp, full[..., D:], chunk=w.chunk)
    ref = R.apply_gate(DR.gqa_decode_ref(inp.q, inp.k, inp.v, inp.seq_lens, inp.scale,
                                         inp.k_scales, inp.v_scales, inp.ids), gate)
    assert_parity(got, ref, "gated i8_32k")


def test_gated_equals_ungated_times_sigmoid_on_device():
    # the gated merge and the plain merge read the same partials
    import decode_attention_kv_gqa_amd as gq
    inp = make_case(2, 1, 8, 2, 128, 500, [500, 260], kv="f16", seed=12)
    gate = gate_values(inp.q.shape, seed=13)
    d = {n: dev(getattr(inp, n)) for n in ("q", "k", "v", "seq_lens")}
    step = gq.DecodeAttention(2, 1, 8, 2, 128, 500, "f16", chunk=64)
    step.attn(d["q"], d["k"], d["v"], d["seq_lens"], inp.scale)
    step.merge(d["seq_lens"])
    plain = step.out.clone()
    step.merge(d["seq_lens"], gate=dev(gate))
    torch.cuda.synchronize()
    expect = plain.cpu().numpy().astype(np.float64) * R.sigmoid(gate)
    np.testing.assert_allclose(step.out.cpu().numpy(), expect, rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("i", range(24))
def test_gated_random_shapes(i):
    """Seeded random shapes (as the attention sweep, with or without budgeted
    ids), the gate as its own tensor or as the second half of [query | gate]
    rows, against the gated oracle."""
    rng = np.random.default_rng(5000 + i)
    S, T, Hk, G = int(rng.integers(1, 6)), int(rng.integers(1, 4)), int(rng.integers(1, 4)), \
        int(rng.integers(1, 13))
    D = int(rng.choice([64, 128, 256]))
    kv = "i8" if rng.random() < 0.5 else "f16"
    Lmax = int(rng.integers(0, 500))
    lens = [int(x) for x in rng.integers(0, Lmax + 3, size=S)]
    budget = int(rng.integers(1, 200)) if rng.random() < 0.3 else 0
    chunk = 0 if rng.random() < 0.5 else int(rng.integers(1, 300))
    rows_layout = bool(rng.random() < 0.5)
    print(f"[gpu] gated sweep {i}: S={S} T={T} Hk={Hk} G={G} D={D} kv={kv} Lmax={Lmax} "
          f"lens={lens} budget={budget} chunk={chunk} qg_rows={rows_layout}", flush=True)
    inp = make_case(S, T, G * Hk, Hk, D, Lmax, lens, kv=kv, budget=budget, seed=5000 + i)
    gate = gate_values(inp.q.shape, seed=5000 + i)
    if rows_layout:
        gate_t = dev(np.concatenate([inp.q, gate], axis=-1))[..., D:]
    else:
        gate_t = dev(gate)
    ref = R.gqa_decode_gated_ref(inp.q, inp.k, inp.v, inp.seq_lens, inp.scale, gate,
                                 inp.k_scales, inp.v_scales, inp.ids)
    assert_parity(run_gated(inp, gate_t, chunk), ref, f"gated sweep {i}")
