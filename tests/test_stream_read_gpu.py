"""The streaming-read reference that bench.py sets the attention's rate
beside (gqa_bench_stream_read): every workgroup stores the XOR of the words
it read, so the XOR of the sink words must equal numpy's XOR of the whole
buffer, whatever the launch shape and however ragged the last stride."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_attention_kv_gqa_amd  # noqa: F401


@pytest.mark.parametrize("nbytes", [16, 4096, 16 * 1000 + 16 * 7, 3 << 20])
@pytest.mark.parametrize("workgroups", [1, 3, 256, 2048])
def test_sink_xor_covers_every_word(nbytes, workgroups):
    import decode_attention_kv_gqa_amd as gq
    rng = np.random.default_rng(nbytes + workgroups)
    words = rng.integers(0, 2 ** 32, nbytes // 4, dtype=np.uint32)
    src = torch.from_numpy(words.view(np.int32)).cuda()
    sink = torch.full((workgroups,), -1, dtype=torch.int32, device="cuda")
    print(f"[gpu] stream_read bytes={nbytes} workgroups={workgroups}", flush=True)
    rc = gq.gqa_bench_stream_read(src.data_ptr(), nbytes, sink.data_ptr(), workgroups,
                                  torch.cuda.current_stream().cuda_stream)
    assert rc == 0, gq.strerror(rc)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(words)
