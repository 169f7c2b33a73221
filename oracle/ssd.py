"""Self-speculative decoding loop, accept rule and matchness scoring (oracle).

Notation: committed tokens t[0..n-1]; the KV cache is valid for positions
0..n-2 at every layer; y0 = t[n-1]; drafts y1..yd'.  b = reuse boundary (first
layer with a skipped sub-layer).

Readings of the pages (each also listed in the design notes):
  * Exit at E runs layers 0..E-1 and verify continues at layer E (LayerSkip
    blog §3.1 prose "run only the first E layers", §3.2 "layers E+1..L, L-E in
    all"; its listing's range(E+1) is taken as an off-by-one).
  * The KV cache accumulates across draft steps (LayerSkip blog §3.1 comment);
    the listing's per-step reset is not taken.
  * Verify reuses, for the draft rows, the hidden state entering layer b (the
    listing reads "layer E's hidden state" out of a KV-cache entry; LayerSkip
    blog §3.2).  The last draft token runs layers < b itself.
  * At temperature 0 the draft is argmax and the accept rule reduces to
    "accept while equal, then emit the target's argmax"; at T > 0 the draft
    samples y ~ q so that min(1, p/q) with the norm(max(0, p - q)) correction
    is distribution-preserving (LayerSkip blog §3.3 rule; §3 "lossless").
  * Confidence = max_v q(v) of the draft distribution (SWIFT digest §4.2; the
    SpecEE notes' AdaInfer "top prob" feature); the low-confidence token is
    kept and drafting stops after it, so 1 <= d' <= d.
  * The prefill's token counts toward the number generated.
"""
import numpy as np

from . import model as mdl
from . import philox
from .numerics import argmax_lowest, softmax


# --------------------------------------------------------------------------
# Sampling primitives


def race_sample(keys_f32):
    """Exponential race / Gumbel-max: index of the largest key (lowest on ties).
    keys_v = log(weight_v) + Gumbel_v samples v with probability weight_v / sum."""
    return argmax_lowest(keys_f32)


def top2_gap(keys):
    """How far a maximum-taking decision is from flipping: the largest key minus
    the second largest (inf with a single finite key).  For race keys this is the
    log-gap of the two best candidates; for logits, the top-2 margin."""
    k = np.sort(np.asarray(keys, np.float64).ravel())
    if k.size < 2 or not np.isfinite(k[-2]):
        return float("inf")
    return float(k[-1] - k[-2])


def _log(log, kind, row, margin):
    if log is not None:
        log.append((kind, int(row), float(margin)))


def sample_logits(z, T, seed, it, row, purpose, log=None, kind="sample"):
    """Sample from softmax(z / T) by the race over float32 keys z/T + Gumbel."""
    g = philox.gumbel(seed, it, row, purpose, z.shape[-1])
    keys = (np.asarray(z, np.float64) / T).astype(np.float32) + g
    _log(log, kind, row, top2_gap(keys))
    return race_sample(keys)


def pick(z, T, seed, it, row, purpose, log=None, kind="sample"):
    """Greedy argmax at T == 0, otherwise a sample from softmax(z / T).

    log (optional list): receives (kind, row, margin) for the decision, the
    margin being how far it is from flipping (top-2 logit gap when greedy,
    top-2 race-key gap when sampling)."""
    if T == 0:
        _log(log, kind, row, top2_gap(z))
        return argmax_lowest(z)
    return sample_logits(z, T, seed, it, row, purpose, log, kind)


def log_softmax(z, T):
    zz = np.asarray(z, np.float64) / (T if T > 0 else 1.0)
    m = np.max(zz)
    return zz - (m + np.log(np.sum(np.exp(zz - m))))


def confidence(z, T):
    """max_v softmax(z / T)_v (softmax at T = 1 when decoding greedily)."""
    return float(np.exp(np.max(log_softmax(z, T))))


def accept_probability(p, q, y):
    """min(1, p(y) / q(y)) (LayerSkip blog §3.3)."""
    return min(1.0, p[y] / q[y])


def residual_distribution(p, q):
    """norm(max(0, p - q)); falls back to p when the positive part sums to 0
    (only possible when p == q, where no rejection can occur)."""
    r = np.maximum(0.0, p - q)
    s = r.sum()
    return p.copy() if s == 0 else r / s


def accept_greedy(p_logits, drafts):
    """T = 0: accept drafts while each equals the target argmax; then emit the
    target's argmax at the first mismatch (or the bonus after d' matches)."""
    k = 0
    while k < len(drafts) and argmax_lowest(p_logits[k]) == drafts[k]:
        k += 1
    return [int(t) for t in drafts[:k]] + [argmax_lowest(p_logits[k])]


def accept_sampled(p_logits, q_logits, drafts, T, seed, it, log=None):
    """T > 0 accept/reject (LayerSkip blog §3.3): for i = 1..d', accept y_i when
    u_i * q_i(y_i) < p_i(y_i) (probability min(1, p/q)); at the first rejection
    emit a sample of norm(max(0, p_i - q_i)); if all are accepted, emit a bonus
    sample of p_{d'+1}.  Decisions are taken on float32 quantities.  log: as in
    pick; an accept decision's margin is |ln(u q(y) / p(y))|."""
    dp = len(drafts)
    for i in range(dp):
        y = int(drafts[i])
        lp = log_softmax(p_logits[i], T).astype(np.float32)
        lq = log_softmax(q_logits[i], T).astype(np.float32)
        u = philox.uniforms(seed, it, i, philox.PURPOSE_ACCEPT, 1)[0]
        _log(log, "accept", i, abs(float(np.log(u) + lq[y]) - float(lp[y])))
        if np.log(u) + lq[y] < lp[y]:
            continue
        p32 = np.exp(lp)
        q32 = np.exp(lq)
        r = np.maximum(np.float32(0), p32 - q32)
        g = philox.gumbel(seed, it, i, philox.PURPOSE_SAMPLE, r.shape[0])
        if np.any(r > 0):
            with np.errstate(divide="ignore"):
                keys = np.log(r) + g
        else:
            keys = lp + g
        _log(log, "sample", i, top2_gap(keys))
        return [int(t) for t in drafts[:i]] + [race_sample(keys)]
    return [int(t) for t in drafts] + [sample_logits(p_logits[dp], T, seed, it, dp, philox.PURPOSE_SAMPLE, log)]


# --------------------------------------------------------------------------
# Prefill, draft, verify


def prefill(model, kv, prompt):
    """All prompt rows through the full model at positions 0..P-1; logits of the last row."""
    z = mdl.forward(model, prompt, range(len(prompt)), kv)
    return z[-1]


def draft(model, kv, y0, n, mask, d, tau, T, seed, it, log=None):
    """Draft phase (LayerSkip blog §3.1; SWIFT digest §3.1, §4.2).

    Feeds y0 at position n-1, then each new draft token at the next position,
    through the sub-layers the plan keeps, the shared final norm and LM head.
    Stops after step j when confidence < tau (or at j = d).  Returns
    (drafts, draft logits [d', V], hidden states entering layer b [d', D]).
    log: as in pick (kind "draft"), plus each confidence-stop decision (kind
    "stop", margin |ln conf - ln tau|) when tau > 0.
    """
    b = mdl.first_skipped_layer(mask, model.L)
    drafts, zs, hb = [], [], []
    y = int(y0)
    for j in range(1, d + 1):
        pos = [n - 2 + j]
        h = mdl.embed(model, [y])
        h = mdl.run_layers(model, h, pos, kv, None, 0, b)
        hb.append(h[0].copy())
        h = mdl.run_layers(model, h, pos, kv, mask, b, model.L)
        z = mdl.final_logits(model, h)[0]
        y = pick(z, T, seed, it, j - 1, philox.PURPOSE_DRAFT, log, "draft")
        drafts.append(y)
        zs.append(z)
        conf = np.float32(confidence(z, T))
        if tau > 0:
            _log(log, "stop", j - 1, abs(np.log(float(conf)) - np.log(float(np.float32(tau)))))
        if conf < np.float32(tau):
            break
    return drafts, np.array(zs), np.array(hb)


def verify(model, kv, y0, drafts, n, b, hb=None):
    """Verify phase (LayerSkip blog §3.2): rows y0..yd' at positions n-1..n-1+d'.

    With hb (the draft's hidden states entering layer b) only the last row runs
    layers < b; otherwise every row does (no reuse).  Layers >= b run in full
    for every row, overwriting the draft's keys/values there.  Returns the full
    model's logits [d'+1, V]; row i scores the token at position n+i.
    """
    dp = len(drafts)
    rows = [int(y0)] + [int(t) for t in drafts]
    positions = list(range(n - 1, n + dp))
    if hb is None:
        h = mdl.embed(model, rows)
        h = mdl.run_layers(model, h, positions, kv, None, 0, b)
    else:
        hl = mdl.embed(model, rows[-1:])
        hl = mdl.run_layers(model, hl, positions[-1:], kv, None, 0, b)
        h = np.concatenate([np.asarray(hb).reshape(dp, -1), hl], axis=0)
    h = mdl.run_layers(model, h, positions, kv, None, b, model.L)
    return mdl.final_logits(model, h)


# --------------------------------------------------------------------------
# Generation loops


def ar_generate(model, prompt, n_gen, T=0.0, seed=3, capacity=None):
    """Plain autoregressive decoding with the full model: the lossless reference."""
    P = len(prompt)
    kv = mdl.KVCache(model.shape, capacity or (P + n_gen + 1))
    out = [pick(prefill(model, kv, prompt), T, seed, 0, 0, philox.PURPOSE_SAMPLE)]
    it = 1
    while len(out) < n_gen:
        n = P + len(out)
        z = mdl.forward(model, [out[-1]], [n - 1], kv)[0]
        out.append(pick(z, T, seed, it, 0, philox.PURPOSE_SAMPLE))
        it += 1
    return out, kv


def exit_generate(model, prompt, n_gen, mask, T=0.0, seed=3, capacity=None):
    """Lossy early-exit decoding (LayerSkip blog §3, first inference mode): after
    the full-model prefill, every token comes from the plan's sub-layers alone
    (with the shared final norm and LM head) and is kept without verification.
    Reading: the prompt is processed by the full model (its keys/values below the
    exit are the same either way); only the tokens after the first are
    generated through the plan."""
    P = len(prompt)
    kv = mdl.KVCache(model.shape, capacity or (P + n_gen + 1))
    z = prefill(model, kv, prompt)
    out = [pick(z, T, seed, 0, 0, philox.PURPOSE_SAMPLE)]
    zs = [z]
    it = 1
    while len(out) < n_gen:
        n = P + len(out)
        z = mdl.forward(model, [out[-1]], [n - 1], kv, mask)[0]
        zs.append(z)
        out.append(pick(z, T, seed, it, 0, philox.PURPOSE_SAMPLE))
        it += 1
    return out, np.array(zs)


def ssd_generate(model, prompt, n_gen, mask, d, tau=0.0, T=0.0, seed=3, reuse=True, capacity=None,
                 on_iteration=None):
    """Self-speculative decoding loop (LayerSkip blog §3.3): draft, verify, accept,
    append the emitted tokens; output truncated to exactly n_gen tokens.
    stats["decisions"][k]: the (kind, row, margin) log of iteration k (0: the
    prefill's token) at T > 0."""
    P = len(prompt)
    L = model.L
    b = mdl.first_skipped_layer(mask, L)
    kv = mdl.KVCache(model.shape, capacity or (P + n_gen + d + 2))
    log0 = []
    out = [pick(prefill(model, kv, prompt), T, seed, 0, 0, philox.PURPOSE_SAMPLE, log0)]
    stats = {"drafted": [], "accepted": [], "emitted": [], "decisions": [log0]}
    it = 1
    while len(out) < n_gen:
        n = P + len(out)
        y0 = out[-1]
        log = []
        drafts, zq, hb = draft(model, kv, y0, n, mask, d, tau, T, seed, it, log)
        zp = verify(model, kv, y0, drafts, n, b, hb if reuse else None)
        if T == 0:
            emitted = accept_greedy(zp, drafts)
        else:
            emitted = accept_sampled(zp, zq, drafts, T, seed, it, log)
        stats["drafted"].append(len(drafts))
        stats["accepted"].append(len(emitted) - 1)
        stats["emitted"].append(len(emitted))
        stats["decisions"].append(log)
        if on_iteration is not None:
            on_iteration(it, n, drafts, zq, zp, emitted, kv)
        out.extend(emitted)
        it += 1
    return out[:n_gen], stats, kv


def score_masks(model, kv, window, pos0, masks, detail=False):
    """SWIFT matchness scoring (SWIFT digest §4.1, §4.1.2, §5.3).

    window = gamma+1 committed tokens at positions pos0..pos0+gamma; the cache
    holds the full model's keys/values for positions < pos0.  Each candidate
    plan runs ONE causal draft forward over rows window[0..gamma-1] (its own
    keys/values at the window positions, the full model's before them) and
    predicts every next token by argmax; its score is the fraction of rows whose
    prediction equals window[i+1].  Returns (scores, index of the best plan,
    lowest index on ties), and with detail=True also each row's prediction and
    its top-2 logit margin ([n_masks, gamma] each).
    """
    gamma = len(window) - 1
    rows = [int(t) for t in window[:-1]]
    targets = np.asarray(window[1:], dtype=np.int64)
    positions = list(range(pos0, pos0 + gamma))
    scores, preds, margins = [], [], []
    for mask in masks:
        kvm = kv.copy()
        z = mdl.forward(model, rows, positions, kvm, mask)
        pred = np.array([argmax_lowest(r) for r in z])
        scores.append(float(np.sum(pred == targets)) / gamma)
        preds.append(pred)
        margins.append([top2_gap(r) for r in z])
    scores = np.array(scores)
    if detail:
        return scores, int(np.argmax(scores)), np.array(preds), np.array(margins)
    return scores, int(np.argmax(scores))


def specee_features(model, h, tokens, prev_probs=None):
    """SpecEE exit features (SpecEE notes §4.3.1) of hidden states h [rows, D]
    for the speculative tokens: the speculative-token logits (the shared final
    norm and LM head restricted to those columns), their softmax (local
    probabilities) and its change against the previous layer's (zero when there
    is none).  Returns [rows, 3k]."""
    h = np.atleast_2d(np.asarray(h, np.float64))
    w = model.lm_head[[int(t) for t in tokens]]
    z = mdl.norm_input(model, h, model.final_norm) @ w.T
    p = softmax(z)
    var = np.zeros_like(p) if prev_probs is None else p - np.asarray(prev_probs, np.float64)
    return np.concatenate([z, p, var], axis=1)
