"""The streaming-read probe behind bench.py's measured bandwidth ceiling reads
every byte of its buffer exactly once (each workgroup folds its own slice)."""
import numpy as np
import pytest
import torch

from self_speculative_layer_amd import binding as B

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [64, 4096 * 64 + 64 * 7, 64 << 20])
def test_probe_reads_each_byte_once(nbytes):
    rng = np.random.default_rng(nbytes)
    words = rng.integers(0, 2 ** 32, nbytes // 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(words.view(np.int32).copy()).cuda()
    sink = torch.full((2048,), -1, dtype=torch.int32, device="cuda")
    B.ssd_probe_read(src, nbytes, sink)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    n16 = nbytes // 16
    per = (n16 + 2047) // 2048
    w16 = words.reshape(n16, 4)
    for b in range(2048):
        lo, hi = min(b * per, n16), min((b + 1) * per, n16)
        ref = np.bitwise_xor.reduce(w16[lo:hi].reshape(-1)) if hi > lo else np.uint32(0)
        assert got[b] == ref, b
    with pytest.raises(B.SSDError):
        B.ssd_probe_read(src, 100, sink)
