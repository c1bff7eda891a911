"""dspark_read_probe, the streaming-read probe bench.py times as the
achievable read rate: every 16-byte word of the buffer is read exactly once
(the XOR of the workgroups' words equals the XOR of the whole buffer)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (1 << 20) * 33 + 16 * 7])
def test_read_probe_reads_every_word_once(nbytes):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mla_block_drafter_amd import dspark as D
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    out = torch.zeros(D.READ_PROBE_WORDS, dtype=torch.int32, device="cuda")
    D.read_probe(buf, out)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)
