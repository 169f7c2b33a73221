"""The library's failure model on the GPU: non-finite logits raise the sequence's numeric flag and emit
nothing, an out-of-range commit count raises the input flag and commits nothing, and destroyed handles are
rejected.  Every condition is forced from the host (NaN written into a buffer or a gain); every kernel
still runs to completion."""
import numpy as np
import pytest
import torch

import synth
from self_speculative_layer_amd import binding as B
from gpu_util import BF16_HD64, F32_GQA, dev, gpu_model

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T", [0.0, 1.0])
def test_nan_verify_logits_raise_numeric_and_emit_nothing(T):
    shape = BF16_HD64
    g = gpu_model(shape, n_layers=1)
    V, d = shape.vocab, 4
    seq = B.Sequence(g, max_ctx=128, max_rows=16, max_draft=d)
    B.ssd_prefill(seq.handle, dev(synth.prompt_tokens(8, V)))
    st0 = B.ssd_read_state(seq.handle)
    B.ssd_draft(seq.handle, None, 0, d, 0.0, T, 5, seq.draft_tokens, seq.draft_logits, seq.n_drafted)
    B.ssd_verify(seq.handle, None, 0, d, seq.draft_tokens, seq.n_drafted, 1, seq.verify_logits)
    torch.cuda.synchronize()
    seq.verify_logits[2 * V + 17] = float("nan")            # row 2 of the verify
    B.ssd_accept(seq.handle, seq.verify_logits, seq.draft_logits, seq.draft_tokens, seq.n_drafted, d, T, 5,
                 seq.out_tokens, seq.n_out)
    B.ssd_commit(seq.handle, seq.out_tokens, seq.n_out)
    torch.cuda.synchronize()
    assert int(seq.n_out.item()) == 0
    with pytest.raises(B.SSDError) as e:
        B.ssd_read_state(seq.handle)
    assert e.value.code == B.SSD_ERR_NUMERIC
    # nothing was committed: the sequence is where the prefill left it (read past the sticky flag)
    st = B.ssd_state()
    B.lib().ssd_read_state(seq.handle, st, None)
    assert (st.kvlen, st.n_out, st.last_token) == (st0.kvlen, st0.n_out, st0.last_token)
    seq.close()
    g.close()


def test_nan_gain_raises_numeric_at_prefill():
    shape = F32_GQA
    g = gpu_model(shape, n_layers=1)
    g.tensors["final_norm"][3] = float("nan")
    seq = B.Sequence(g, max_ctx=64, max_rows=16, max_draft=2)
    B.ssd_prefill(seq.handle, dev(synth.prompt_tokens(8, shape.vocab)))
    with pytest.raises(B.SSDError) as e:
        B.ssd_read_state(seq.handle)
    assert e.value.code == B.SSD_ERR_NUMERIC
    seq.close()
    g.close()


def test_accept_noalloc_emits_nothing_on_nan():
    V, d = 300, 3
    zp = torch.randn((d + 1) * V, device="cuda")
    zq = torch.randn(d * V, device="cuda")
    zp[V + 5] = float("inf")
    drafts = dev([1, 2, 3])
    nd = dev([3])
    out = torch.zeros(d + 1, dtype=torch.int32, device="cuda")
    n = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    for T in (0.0, 0.8):
        B.ssd_accept_noalloc(zp, zq, drafts, nd, d, V, T, 1, 1, out, n)
        torch.cuda.synchronize()
        assert int(n.item()) == 0


def test_commit_count_out_of_range_raises_input_flag():
    shape = BF16_HD64
    g = gpu_model(shape, n_layers=1)
    seq = B.Sequence(g, max_ctx=64, max_rows=16, max_draft=4)
    B.ssd_prefill(seq.handle, dev(synth.prompt_tokens(8, shape.vocab)))
    st0 = B.ssd_read_state(seq.handle)
    seq.n_out.fill_(99)                                    # more than max_draft + 1 tokens
    B.ssd_commit(seq.handle, seq.out_tokens, seq.n_out)
    with pytest.raises(B.SSDError) as e:
        B.ssd_read_state(seq.handle)
    assert e.value.code == B.SSD_ERR_ARG
    st = B.ssd_state()
    B.lib().ssd_read_state(seq.handle, st, None)
    assert (st.kvlen, st.n_out) == (st0.kvlen, st0.n_out)
    seq.close()
    g.close()


def test_destroyed_handles_are_rejected():
    shape = BF16_HD64
    g = gpu_model(shape, n_layers=1)
    seq = B.Sequence(g, max_ctx=64, max_rows=16, max_draft=4)
    with pytest.raises(B.SSDError) as e:                   # a model with a live sequence stays
        B.ssd_model_destroy(g.handle)
    assert e.value.code == B.SSD_ERR_ARG
    h = seq.handle
    seq.close()
    for call in (lambda: B.ssd_prefill(h, dev([1, 2, 3])), lambda: B.ssd_read_state(h),
                 lambda: B.ssd_seq_destroy(h)):
        with pytest.raises(B.SSDError) as e:
            call()
        assert e.value.code == B.SSD_ERR_ARG and "live sequence" in str(e.value)
    m = g.handle
    g.close()
    with pytest.raises(B.SSDError) as e:
        B.ssd_model_destroy(m)
    assert e.value.code == B.SSD_ERR_ARG and "live model" in str(e.value)


def test_scoring_beyond_1024_rows_needs_the_group_attention():
    """A scoring pass of more than 1024 rows runs only where the candidate-group attention takes it (bf16,
    head_dim 64 or 128): on an fp32 model the call is refused on the host, before any device work, and a
    pass within 1024 rows still runs."""
    shape = F32_GQA
    g = gpu_model(shape)
    L, gamma = shape.n_layers, 32
    seq = B.Sequence(g, max_ctx=128, max_rows=2048, max_draft=4)
    seq.generate_ar(dev(synth.prompt_tokens(40, shape.vocab)), gamma)
    window = dev(np.arange(gamma + 1, dtype=np.int32) % shape.vocab)
    masks = np.zeros((33, 2 * L), np.uint8)                 # 33 x 32 = 1056 rows
    scores = torch.zeros(33, dtype=torch.float32, device="cuda")
    best = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(B.SSDError) as e:
        B.ssd_score_masks(seq.handle, masks, window, 39, gamma, scores, best)
    assert e.value.code == B.SSD_ERR_UNSUPPORTED
    B.ssd_score_masks(seq.handle, masks[:32], window, 39, gamma, scores, best)
    torch.cuda.synchronize()
    assert np.all(scores[:32].cpu().numpy() == scores[0].item())   # equal plans score alike
    seq.close()
    g.close()
