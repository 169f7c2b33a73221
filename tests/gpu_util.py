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
    """GPU tokens must equal the oracle's except where the GPU's token is within
    `margin` of the oracle's choice in the oracle's logits; returns the index of
    the first excused mismatch or None."""
    gpu = [int(x) for x in gpu]
    for i, (a, b) in enumerate(zip(gpu, ref)):
        if a != b:
            z = np.asarray(ref_logits[i])
            mg = float(z.max() - z[a])
            assert mg < margin, "token %d: gpu %d oracle %d, the oracle puts them %.3g apart" % (i, a, b, mg)
            return i
    assert len(gpu) == len(ref)
    return None


def dev(a, dtype=torch.int32):
    return torch.as_tensor(np.asarray(a), dtype=dtype).cuda()


def check_greedy_with_resync(generate, prompt, ref, ref_logits, margin=1e-2, max_events=2):
    """Greedy parity with re-synchronisation: generate(prefix, n) runs the GPU path
    from a prompt of committed tokens and returns n tokens.  A token may differ
    from the oracle's only where the GPU's token is within `margin` of the
    oracle's choice in the oracle's logits (so the oracle's top-2 margin is below
    `margin` too); after such an allowed mismatch the GPU path restarts from the
    oracle's committed prefix (a fresh prefill) and the comparison goes on.
    Returns the number of re-synchronisations (at most max_events)."""
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
        z = np.asarray(ref_logits[k])
        mg = float(z.max() - z[got[mismatch]])
        assert mg < margin, "token %d: gpu %d oracle %d, the oracle puts them %.3g apart" % (
            k, got[mismatch], ref[k], mg)
        events += 1
        assert events <= max_events, "too many near-tie re-synchronisations"
        done = k + 1
    return events


def token_sources(emitted_counts):
    """(iteration, row) of each generated token: token 0 is the prefill's (iteration 0), then iteration k
    emits emitted_counts[k - 1] tokens from its rows 0, 1, ..."""
    src = [(0, 0)]
    for k, e in enumerate(emitted_counts):
        src += [(k + 1, j) for j in range(e)]
    return src


def check_sampled_with_resync(gpu_run, oracle_run, prompt, n_gen, margin=1e-2, max_events=3):
    """Sampled parity with re-synchronisation.  The GPU path and the oracle start from the same committed
    prefix with the same random draws.  A generated token may differ only where one of the decisions that
    produced it in the oracle -- the draft draws and confidence stops, the accept decisions and the final
    draw of its iteration, at rows up to its own -- lies within `margin` of flipping (|ln(u q(y) / p(y))|
    for an accept decision, the top-2 race-key gap for a draw, |ln conf - ln tau| for a stop).  After such
    a mismatch both sides restart from the oracle's tokens up to and including the mismatched one (a fresh
    prefill each) and the comparison goes on to n_gen tokens.
    gpu_run(prefix, n) -> n tokens; oracle_run(prefix, n) -> (n tokens, stats with "emitted" and
    "decisions").  Returns the number of re-synchronisations (at most max_events)."""
    prefix = [int(t) for t in prompt]
    done, events = 0, 0
    while done < n_gen:
        n = n_gen - done
        ref, st = oracle_run(prefix, n)
        ref = [int(x) for x in ref]
        got = [int(x) for x in gpu_run(prefix, n)]
        m = next((i for i, (a, b) in enumerate(zip(got, ref)) if a != b), None)
        if m is None:
            assert len(got) == len(ref) == n
            return events
        it, row = token_sources(st["emitted"])[m]
        near = [mg for _, r, mg in st["decisions"][it] if r <= row]
        mg = min(near) if near else float("inf")
        assert mg < margin, ("token %d (iteration %d, row %d): gpu %d oracle %d; the nearest decision is %.3g from "
                             "flipping" % (done + m, it, row, got[m], ref[m], mg))
        events += 1
        assert events <= max_events, "too many near-tie re-synchronisations"
        prefix += ref[: m + 1]
        done += m + 1
    return events


def check_scores(gs, gbest, gpred, window, oscores, obest, opred, omargin, margin=1e-2):
    """Matchness scoring against the oracle, row by row: a row's prediction may differ only where the
    oracle's top-2 logit margin for that row is below `margin`; the GPU's scores are its own row matches
    (so they differ from the oracle's by at most the near-tie rows / gamma); the best plan is the oracle's
    unless the two candidates' oracle scores are within their near-tie rows of each other.  Returns the
    number of differing rows."""
    gs, gpred, opred, omargin = (np.asarray(a) for a in (gs, gpred, opred, omargin))
    targets = np.asarray(window[1:])
    gamma = len(targets)
    diff = gpred != opred
    assert np.all(omargin[diff] < margin), "rows differ from the oracle away from a near-tie: %s" % (
        np.argwhere(diff & (omargin >= margin)).tolist())
    assert np.array_equal(gs, (gpred == targets).sum(axis=1).astype(np.float32) / np.float32(gamma))
    assert gbest == int(np.argmax(gs))
    near = (omargin < margin).sum(axis=1)
    assert np.all(np.abs(gs - oscores) <= near / gamma + 1e-7)
    if gbest != obest:
        assert abs(oscores[gbest] - oscores[obest]) <= (near[gbest] + near[obest]) / gamma + 1e-7
    return int(diff.sum())


class Acc32(omodel.Model):
    """The oracle's decoder with every matrix product taken in float32 (float32 weights and float32 rounded
    inputs: products accumulated in float32, as the GPU accumulates them), all else as the oracle.  How far
    it moves from the oracle is what the accumulation precision alone does to the logits: the measuring
    instrument behind the GPU tests' full-width tolerances, not a model of its own."""

    def rnd(self, x):
        return super().rnd(x).astype(np.float32)


def acc32_twin(o):
    f = lambda a: a.astype(np.float32)
    layers = [omodel.LayerWeights(**{k: f(v) for k, v in vars(lw).items()}) for lw in o.layers]
    return Acc32(shape=o.shape, embed=o.embed, layers=layers, final_norm=o.final_norm, lm_head=f(o.lm_head))


def teacher_rows(m, prompt, iters, mask, capacity):
    """Logits of the prefill's last row, then of each iteration's draft rows and verify rows, teacher-forced
    with the given iterations' tokens: iters = [(y0, n, drafts), ...] as the SSD loop saw them.  Returns
    [z0[None], draft rows 1, verify rows 1, draft rows 2, ...]."""
    kv = omodel.KVCache(m.shape, capacity)
    rows = [ossd.prefill(m, kv, prompt)[None]]
    for y0, n, drafts in iters:
        pos = list(range(n - 1, n + len(drafts)))
        rows.append(omodel.forward(m, [y0] + list(drafts[:-1]), pos[:-1], kv.copy(), mask))
        rows.append(omodel.forward(m, [y0] + list(drafts), pos, kv))
    return rows


def max_abs_rows(a, b):
    """Per row: max |a - b|."""
    return np.abs(np.atleast_2d(a) - np.atleast_2d(b)).max(axis=1)
