"""Helpers of the GPU parity tests: build the same synthetic model on both sides."""
import numpy as np
import torch

import synth
from synth import device as sdev
from self_speculative_layer_amd import binding as B
from oracle import model as omodel
from oracle import ssd as ossd

# test shapes: several tiles, ragged tails (V and N not multiples of 16/64), GQA and MHA, hd 64 and 128
BF16_HD64 = synth.ModelShape("bf16-hd64-gqa", 4, 256, 4, 2, 64, 576, 1000, "bf16")
BF16_HD128 = synth.ModelShape("bf16-hd128", 3, 512, 4, 4, 128, 1408, 2003, "bf16")
F32_GQA = synth.ModelShape("f32-gqa", 3, 192, 6, 2, 64, 440, 777, "f32")


def gpu_model(shape, n_layers=None):
    L = shape.n_layers if n_layers is None else n_layers
    t = sdev.build_weights(shape, n_layers=L)
    return B.Model(L, shape.d_model, shape.n_heads, shape.n_kv_heads, shape.head_dim, shape.ffn_dim, shape.vocab,
                   shape.dtype, t)


def logit_tol(shape):
    return 2e-2 if shape.dtype == "bf16" else 1e-4


def oracle_ar_with_logits(m, prompt, n_gen):
    """Greedy AR with the oracle, returning tokens and each step's logits."""
    P = len(prompt)
    kv = omodel.KVCache(m.shape, P + n_gen + 2)
    z = ossd.prefill(m, kv, prompt)
    toks, zs = [int(np.argmax(z))], [z]
    while len(toks) < n_gen:
        n = P + len(toks)
        z = omodel.forward(m, [toks[-1]], [n - 1], kv)[0]
        zs.append(z)
        toks.append(int(np.argmax(z)))
    return toks, np.array(zs)


def top2_margin(z):
    s = np.sort(z)
    return float(s[-1] - s[-2])


def check_greedy_tokens(gpu, ref, ref_logits, margin=1e-2):
    """GPU tokens must equal the oracle's except where the oracle's top-2 margin
    is below `margin`; returns the index of the first excused mismatch or None."""
    gpu = [int(x) for x in gpu]
    for i, (a, b) in enumerate(zip(gpu, ref)):
        if a != b:
            mg = top2_margin(ref_logits[i])
            assert mg < margin, "token %d: gpu %d oracle %d, oracle margin %.3g" % (i, a, b, mg)
            return i
    assert len(gpu) == len(ref)
    return None


def dev(a, dtype=torch.int32):
    return torch.as_tensor(np.asarray(a), dtype=dtype).cuda()


def check_greedy_with_resync(generate, prompt, ref, ref_logits, margin=1e-2, max_events=2):
    """Greedy parity with re-synchronisation: generate(prefix, n) runs the GPU path
    from a prompt of committed tokens and returns n tokens.  A token may differ
    from the oracle's only where the oracle's top-2 margin is below `margin`; after
    such an allowed mismatch the GPU path restarts from the oracle's committed
    prefix (a fresh prefill) and the comparison goes on.  Returns the number of
    re-synchronisations (at most max_events)."""
    prompt = [int(t) for t in prompt]
    ref = [int(t) for t in ref]
    done, events = 0, 0
    while done < len(ref):
        got = [int(x) for x in generate(prompt + ref[:done], len(ref) - done)]
        mismatch = next((i for i, (a, b) in enumerate(zip(got, ref[done:])) if a != b), None)
        if mismatch is None:
            assert len(got) == len(ref) - done
            return events
        k = done + mismatch
        mg = top2_margin(ref_logits[k])
        assert mg < margin, "token %d: gpu %d oracle %d, oracle margin %.3g" % (k, got[mismatch], ref[k], mg)
        events += 1
        assert events <= max_events, "too many near-tie re-synchronisations"
        done = k + 1
    return events
