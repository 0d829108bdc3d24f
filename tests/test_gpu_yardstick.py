"""GPU check of the streaming-read yardstick behind bench.py's achievable HBM
rate: it must read every 16-byte chunk of the buffer exactly once, so the
XOR of its per-workgroup words equals the XOR of every 32-bit word of the
buffer.  Sizes cover a whole number of grid passes and ragged tails."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
mla = pytest.importorskip("head_latent_attention_fwd_amd")

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("words", [
    4,                            # one chunk: one workgroup reads, the rest are empty
    4096 * 4 * 256 * 16,          # every range a whole number of unrolled passes
    4096 * 4 * 256 * 16 * 3 + 4 * 777,  # ranges with ragged tails
    (1 << 22) + 4 * 13,           # ranges shorter than one unrolled pass
])
def test_read_sweep_reads_every_chunk_once(words):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    g = torch.Generator().manual_seed(words % 1000 + 5)
    host = torch.randint(-2 ** 31, 2 ** 31 - 1, (words,), generator=g, dtype=torch.int64).to(torch.int32)
    buf = host.to("cuda:0")
    print(f"[read_sweep] words={words}", flush=True)
    sink = mla.mla_read_sweep(buf)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    assert got == want
