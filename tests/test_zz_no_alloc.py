"""The allocation-free acceptance (ssd_accept_noalloc) against ssd_accept on the same inputs: the same
emitted tokens and count, bit for bit, on two calls in a row (the second smaller: fewer drafts, a
smaller vocabulary), greedy and sampled."""
import numpy as np
import pytest
import torch

import synth
from self_speculative_layer_amd import binding as B
from gpu_util import BF16_HD64, F32_GQA, dev, gpu_model

pytestmark = pytest.mark.gpu


def _accept_both(shape, d, dp, T, seed, rng):
    g = gpu_model(shape, n_layers=1)
    V = shape.vocab
    seq = B.Sequence(g, max_ctx=128, max_rows=16, max_draft=d)
    B.ssd_prefill(seq.handle, dev(synth.prompt_tokens(4, V)))        # the sequence's iteration becomes 1
    zp = (rng.standard_normal((d + 1, V)) * 3).astype(np.float32)
    zq = zp[:d] + (rng.standard_normal((d, V)) * 0.5).astype(np.float32)
    drafts = [int(np.argmax(zq[i] + rng.gumbel(size=V))) for i in range(d)]
    if T == 0:
        drafts = [int(np.argmax(zp[i])) if i < dp // 2 else int(np.argmax(zq[i])) for i in range(d)]
    seq.verify_logits[: (d + 1) * V].copy_(dev(zp.reshape(-1), torch.float32))
    seq.draft_logits[: d * V].copy_(dev(zq.reshape(-1), torch.float32))
    seq.draft_tokens[:d].copy_(dev(drafts))
    seq.n_drafted.fill_(dp)
    B.ssd_accept(seq.handle, seq.verify_logits, seq.draft_logits, seq.draft_tokens, seq.n_drafted, d, T, seed,
                 seq.out_tokens, seq.n_out)
    out2 = torch.full((d + 1,), -7, dtype=torch.int32, device="cuda")
    n2 = torch.zeros(1, dtype=torch.int32, device="cuda")
    B.ssd_accept_noalloc(seq.verify_logits, seq.draft_logits, seq.draft_tokens, seq.n_drafted, d, V, T, seed, 1,
                         out2, n2)
    torch.cuda.synchronize()
    n = int(seq.n_out.item())
    ref = seq.out_tokens[:n].cpu().numpy().tolist()
    got = out2[: int(n2.item())].cpu().numpy().tolist()
    seq.close()
    g.close()
    return ref, got, n


@pytest.mark.parametrize("T", [0.0, 1.0])
def test_accept_noalloc_equals_accept(T):
    rng = np.random.default_rng(23)
    # first call: 8 drafts over a 1000-token vocabulary; second call: 3 drafts over 777 tokens
    for shape, d, dp, seed in [(BF16_HD64, 8, 7, 101), (F32_GQA, 3, 3, 202)]:
        print("[gpu] accept_noalloc %s d=%d d'=%d T=%g" % (shape.name, d, dp, T), flush=True)
        ref, got, n = _accept_both(shape, d, dp, T, seed, rng)
        assert 1 <= n <= dp + 1
        assert got == ref


def test_accept_noalloc_rejects_long_chains():
    z = torch.zeros(40 * 10, dtype=torch.float32, device="cuda")
    t = torch.zeros(40, dtype=torch.int32, device="cuda")
    with pytest.raises(B.SSDError) as e:
        B.ssd_accept_noalloc(z, z, t, t, 33, 10, 1.0, 0, 1, t, t)
    assert e.value.code == B.SSD_ERR_CAPACITY
