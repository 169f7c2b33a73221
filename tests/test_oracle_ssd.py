"""Pins of the oracle's self-speculative loop: the pages' invariants, exact
enumeration of the accept rule, and chi-square tests of the sampled output."""
import dataclasses
import itertools

import numpy as np
import pytest
from scipy import stats

import synth
from oracle import model as mdl
from oracle import philox, ssd
from oracle.numerics import softmax

BF16_SMALL = synth.ModelShape("bf16-small", 3, 128, 4, 2, 32, 160, 300, "bf16")
MICRO = synth.ModelShape("micro", 2, 32, 2, 2, 16, 64, 12, "f32")


def _model(shape, lm_scale=1.0):
    m = mdl.Model.synthetic(shape)
    m.lm_head = m.lm_head * lm_scale
    return m


# ---------------------------------------------------------------- greedy, lossless
@pytest.mark.parametrize("plan,d,tau", [
    ("skip2", 4, 0.0),        # the tiny workload: skip layer 2, d = 4
    ("exit1", 3, 0.0),
    ("exit3", 6, 0.0),
    ("skip2", 5, 0.004),      # confidence stop active
    ("attn_only", 4, 0.0),    # sub-layer plan: attention of layer 1 and MLP of layer 3
])
def test_greedy_ssd_equals_ar_tiny(plan, d, tau):
    """Greedy self-speculative output equals plain greedy AR output (LayerSkip blog §3
    'lossless'; SWIFT digest §1 'distribution preserved')."""
    m = _model(synth.TINY)
    prompt = synth.prompt_tokens(32, synth.TINY.vocab)
    mask = {"skip2": synth.mask_from_layers(4, [2]), "exit1": synth.mask_exit(4, 1),
            "exit3": synth.mask_exit(4, 3),
            "attn_only": np.array([0, 0, 1, 0, 0, 0, 0, 1], np.uint8)}[plan]
    ar, _ = ssd.ar_generate(m, prompt, 40)
    out, st, _ = ssd.ssd_generate(m, prompt, 40, mask, d, tau=tau)
    assert out == ar
    assert all(1 <= e <= dr + 1 for e, dr in zip(st["emitted"], st["drafted"]))
    if tau > 0:
        assert min(st["drafted"]) < d          # the stop fired at least once


def test_greedy_ssd_equals_ar_bf16():
    m = _model(BF16_SMALL)
    prompt = synth.prompt_tokens(20, BF16_SMALL.vocab)
    ar, _ = ssd.ar_generate(m, prompt, 30)
    for mask in (synth.mask_exit(3, 1), synth.mask_from_layers(3, [1])):
        out, _, _ = ssd.ssd_generate(m, prompt, 30, mask, 5)
        assert out == ar


@pytest.mark.parametrize("T", [0.0, 1.0])
def test_empty_plan_accepts_everything(T):
    """Nothing skipped: draft == target, every verify yields d'+1 tokens."""
    m = _model(MICRO, 10.0)
    prompt = synth.prompt_tokens(8, MICRO.vocab)
    out, st, _ = ssd.ssd_generate(m, prompt, 30, np.zeros(4, np.uint8), 4, T=T, seed=5)
    assert st["emitted"][:-1] == [5] * (len(st["emitted"]) - 1)
    assert all(a == dr for a, dr in zip(st["accepted"], st["drafted"]))


def test_yield_bounds_sampled():
    """Every verify yields between 1 and d'+1 tokens (LayerSkip blog §3.3)."""
    m = _model(MICRO, 10.0)
    prompt = synth.prompt_tokens(8, MICRO.vocab)
    _, st, _ = ssd.ssd_generate(m, prompt, 60, synth.mask_exit(2, 1), 3, tau=0.3, T=1.0, seed=9)
    assert all(1 <= e <= dr + 1 for e, dr in zip(st["emitted"], st["drafted"]))
    assert min(st["emitted"]) == 1 and max(st["emitted"]) > 1


# ---------------------------------------------------------------- KV reuse
@pytest.mark.parametrize("mask_layers", [[2], [1, 3], []])
def test_verify_reuse_equals_no_reuse(mask_layers):
    """Reusing the draft's prefix-layer state gives the no-reuse verify (LayerSkip blog §3.2)."""
    m = _model(synth.TINY)
    prompt = synth.prompt_tokens(16, synth.TINY.vocab)
    mask = synth.mask_from_layers(4, mask_layers)
    b = mdl.first_skipped_layer(mask, 4)
    kv = mdl.KVCache(synth.TINY, 40)
    t0 = ssd.pick(ssd.prefill(m, kv, prompt), 0, 0, 0, 0, 2)
    drafts, zq, hb = ssd.draft(m, kv, t0, 17, mask, 5, 0.0, 0.0, 0, 1)
    kv2 = kv.copy()
    z_reuse = ssd.verify(m, kv, t0, drafts, 17, b, hb)
    z_plain = ssd.verify(m, kv2, t0, drafts, 17, b, None)
    assert np.abs(z_reuse - z_plain).max() < 1e-12
    assert np.abs(kv.K[:, :23] - kv2.K[:, :23]).max() < 1e-12


def test_ssd_cache_equals_ar_cache():
    """After every SSD iteration the committed positions' keys/values equal AR's."""
    m = _model(synth.TINY)
    prompt = synth.prompt_tokens(16, synth.TINY.vocab)
    ar, kv_ar = ssd.ar_generate(m, prompt, 30)
    seen = []

    def check(it, n, drafts, zq, zp, emitted, kv):
        kvlen = n - 1 + len(emitted)          # positions 0..kvlen-1 hold committed tokens' K/V
        seen.append(kvlen)
        assert np.abs(kv.K[:, :kvlen] - kv_ar.K[:, :kvlen]).max() < 1e-12
        assert np.abs(kv.V[:, :kvlen] - kv_ar.V[:, :kvlen]).max() < 1e-12

    out, _, _ = ssd.ssd_generate(m, prompt, 30, synth.mask_from_layers(4, [1, 2]), 4, on_iteration=check)
    assert out == ar and len(seen) > 3


# ---------------------------------------------------------------- accept rule
def _tables(V, seed):
    """Deterministic conditional distributions p(.|prefix), q(.|prefix) for the enumeration."""
    cache = {}

    def get(which, prefix):
        key = (which, tuple(prefix))
        if key not in cache:
            h = abs(hash(key)) % (2 ** 32)
            r = np.random.default_rng([seed, h])
            z = r.standard_normal(V) * 1.5
            if which == "q" and len(prefix) % 2 == 0:
                z[r.integers(V)] += 2.0
            cache[key] = softmax(z)
        return cache[key]
    return get


def _ssd_law(get, V, dmax, k, prefix=()):
    """Exact law of the next k output tokens of the SSD process with d' = dmax,
    built from the oracle's accept_probability and residual_distribution."""
    out = {}

    def add(seq, pr):
        out[seq] = out.get(seq, 0.0) + pr

    def emit(prefix, drafts, pdraft, j):
        # drafts y1..yj accepted so far with probability pdraft
        if j == dmax:
            p = get("p", prefix + drafts)
            for c in range(V):
                finish(prefix, drafts + (c,), pdraft * p[c])
            return
        q = get("q", prefix + drafts)
        p = get("p", prefix + drafts)
        r = ssd.residual_distribution(p, q)
        for y in range(V):
            a = ssd.accept_probability(p, q, y)
            if a > 0:
                emit(prefix, drafts + (y,), pdraft * q[y] * a, j + 1)
            if a < 1:
                for c in range(V):
                    if r[c] > 0:
                        finish(prefix, drafts + (c,), pdraft * q[y] * (1 - a) * r[c])

    def finish(prefix, emitted, pr):
        if pr == 0:
            return
        if len(emitted) >= k:
            add(emitted[:k], pr)
        else:
            for seq, pr2 in _ssd_law(get, V, dmax, k - len(emitted), prefix + emitted).items():
                add(emitted + seq, pr * pr2)

    emit(tuple(prefix), (), 1.0, 0)
    return out


@pytest.mark.parametrize("dmax", [1, 2])
def test_accept_rule_exact_enumeration(dmax):
    """The emitted-token law equals the autoregressive law of p, exactly (to 1e-12)."""
    V, k = 8, 3
    get = _tables(V, 11)
    law = _ssd_law(get, V, dmax, k)
    assert abs(sum(law.values()) - 1) < 1e-12
    for seq in itertools.product(range(V), repeat=k):
        ar = get("p", ())[seq[0]] * get("p", seq[:1])[seq[1]] * get("p", seq[:2])[seq[2]]
        assert abs(law.get(seq, 0.0) - ar) < 1e-12


def test_accept_probability_and_residual_special_cases():
    p = softmax(np.random.default_rng(0).standard_normal(10))
    assert all(ssd.accept_probability(p, p, y) == 1.0 for y in range(10))
    assert np.array_equal(ssd.residual_distribution(p, p), p)
    a = np.zeros(6); a[1] = 1.0
    b = np.zeros(6); b[4] = 1.0
    assert ssd.accept_probability(a, b, 4) == 0.0
    assert np.array_equal(ssd.residual_distribution(a, b), a)


def test_race_sampler_law():
    """The exponential race over z/T + Gumbel samples softmax(z/T)."""
    z = np.array([0.3, -1.0, 2.0, 0.0, 1.1, -0.4, 0.7, 1.5])
    n = 20000
    counts = np.zeros(8)
    for it in range(n):
        counts[ssd.sample_logits(z, 0.8, 77, it, 0, philox.PURPOSE_SAMPLE)] += 1
    exp = softmax(z / 0.8) * n
    assert stats.chisquare(counts, exp).pvalue > 1e-4


def test_accept_sampled_frequencies():
    """accept_sampled accepts with probability min(1, p/q) and resamples from the residual."""
    V = 6
    zp = np.array([[1.0, 0.2, -0.5, 0.0, 0.3, -1.0], [0.0] * 6])
    zq = np.array([[0.0, 1.5, -0.5, 0.4, 0.3, -1.0]])
    p, q = softmax(zp[0]), softmax(zq[0])
    y = 1                                           # p(y)/q(y) < 1
    n = 20000
    acc = 0
    corr = np.zeros(V)
    for it in range(n):
        e = ssd.accept_sampled(zp, zq, [y], 1.0, 123, it)
        if len(e) == 2:
            acc += 1
        else:
            corr[e[0]] += 1
    pa = p[y] / q[y]
    assert abs(acc / n - pa) < 4 * np.sqrt(pa * (1 - pa) / n)
    r = ssd.residual_distribution(p, q)
    nz = r > 0
    assert np.all(corr[~nz] == 0)
    assert stats.chisquare(corr[nz], r[nz] * corr.sum()).pvalue > 1e-4


def _first_two_tokens(m, prompt, mask, d, trials, draft_fn=None, accept_fn=None):
    """Sample the first two tokens emitted after a fixed committed context."""
    P = len(prompt)
    kv0 = mdl.KVCache(m.shape, P + 2 * d + 8)
    t0 = ssd.pick(ssd.prefill(m, kv0, prompt), 0, 0, 0, 0, 2)     # greedy first token: fixed context
    b = mdl.first_skipped_layer(mask, m.L)
    draft_fn = draft_fn or ssd.draft
    accept_fn = accept_fn or ssd.accept_sampled
    pairs = []
    for trial in range(trials):
        kv = kv0.copy()
        out = [t0]
        it = 1
        while len(out) < 3:
            n = P + len(out)
            drafts, zq, hb = draft_fn(m, kv, out[-1], n, mask, d, 0.0, 1.0, trial, it)
            zp = ssd.verify(m, kv, out[-1], drafts, n, b, hb)
            out.extend(accept_fn(zp, zq, drafts, 1.0, trial, it))
            it += 1
        pairs.append((out[1], out[2]))
    return t0, kv0, pairs


def _target_joint(m, prompt, t0, kv0):
    V = m.shape.vocab
    P = len(prompt)
    kv = kv0.copy()
    p1 = softmax(mdl.forward(m, [t0], [P], kv)[0])
    joint = np.zeros((V, V))
    for a in range(V):
        kva = kv.copy()
        joint[a] = p1[a] * softmax(mdl.forward(m, [a], [P + 1], kva)[0])
    return p1, joint


def _chi2_pvalue(counts, expected, min_exp=5.0):
    counts, expected = counts.ravel(), expected.ravel()
    big = expected >= min_exp
    c = np.append(counts[big], counts[~big].sum())
    e = np.append(expected[big], expected[~big].sum())
    if e[-1] == 0:
        c, e = c[:-1], e[:-1]
    return stats.chisquare(c, e * c.sum() / e.sum()).pvalue


@pytest.fixture(scope="module")
def micro_setup():
    m = _model(MICRO, 12.0)       # a boosted LM head so that draft and target laws differ
    prompt = synth.prompt_tokens(6, MICRO.vocab)
    return m, prompt


def test_sampled_ssd_matches_target_law(micro_setup):
    """Chi-square: the first and the first-two-joint emitted tokens follow the target
    model's autoregressive law (LayerSkip blog §3.3 rule is distribution-preserving)."""
    m, prompt = micro_setup
    mask = synth.mask_exit(2, 1)
    n = 12000
    t0, kv0, pairs = _first_two_tokens(m, prompt, mask, 2, n)
    p1, joint = _target_joint(m, prompt, t0, kv0)
    V = MICRO.vocab
    c1 = np.bincount([a for a, _ in pairs], minlength=V).astype(float)
    cj = np.zeros((V, V))
    for a, b in pairs:
        cj[a, b] += 1
    assert _chi2_pvalue(c1, p1 * n) > 1e-4
    assert _chi2_pvalue(cj, joint * n) > 1e-4
    # the draft law differs from the target law here, so the rule is really exercised
    kv = kv0.copy()
    zq = ssd.draft(m, kv, t0, len(prompt) + 1, mask, 1, 0.0, 1.0, 0, 1)[1][0]
    assert np.abs(softmax(zq) - p1).max() > 0.05


def test_negative_control_argmax_draft_fails(micro_setup):
    """Planted mistake (the listing's literal reading): argmax drafts checked against the
    soft q.  The emitted law must then differ from the target law."""
    m, prompt = micro_setup
    mask = synth.mask_exit(2, 1)

    def argmax_draft(m_, kv, y0, n, mask_, d, tau, T, seed, it):
        drafts, zs, hb = ssd.draft(m_, kv, y0, n, mask_, d, tau, 0.0, seed, it)
        return drafts, zs, hb

    n = 4000
    t0, kv0, pairs = _first_two_tokens(m, prompt, mask, 2, n, draft_fn=argmax_draft)
    p1, _ = _target_joint(m, prompt, t0, kv0)
    c1 = np.bincount([a for a, _ in pairs], minlength=MICRO.vocab).astype(float)
    assert _chi2_pvalue(c1, p1 * n) < 1e-6


def test_negative_control_residual_without_positive_part_fails(micro_setup):
    """Planted mistake: resampling from p instead of norm(max(0, p - q))."""
    m, prompt = micro_setup
    mask = synth.mask_exit(2, 1)

    def bad_accept(zp, zq, drafts, T, seed, it):
        dp = len(drafts)
        for i in range(dp):
            y = int(drafts[i])
            lp = ssd.log_softmax(zp[i], T).astype(np.float32)
            lq = ssd.log_softmax(zq[i], T).astype(np.float32)
            u = philox.uniforms(seed, it, i, philox.PURPOSE_ACCEPT, 1)[0]
            if np.log(u) + lq[y] < lp[y]:
                continue
            return list(drafts[:i]) + [ssd.sample_logits(zp[i], T, seed, it, i, philox.PURPOSE_SAMPLE)]
        return list(drafts) + [ssd.sample_logits(zp[dp], T, seed, it, dp, philox.PURPOSE_SAMPLE)]

    n = 4000
    t0, kv0, pairs = _first_two_tokens(m, prompt, mask, 2, n, accept_fn=bad_accept)
    p1, _ = _target_joint(m, prompt, t0, kv0)
    c1 = np.bincount([a for a, _ in pairs], minlength=MICRO.vocab).astype(float)
    assert _chi2_pvalue(c1, p1 * n) < 1e-6


# ---------------------------------------------------------------- matchness scoring
@pytest.fixture(scope="module")
def scoring_setup():
    m = _model(synth.TINY)
    P, gamma = 16, 32
    prompt = synth.prompt_tokens(P, synth.TINY.vocab)
    ar, kv = ssd.ar_generate(m, prompt, gamma)
    full = list(prompt) + ar
    window = full[P - 1: P + gamma]            # gamma+1 tokens at positions P-1 .. P-1+gamma
    return m, kv, window, P - 1


def test_scoring_empty_plan_scores_one(scoring_setup):
    """A candidate that skips nothing reproduces the greedy window: matchness 1."""
    m, kv, window, pos0 = scoring_setup
    scores, best = ssd.score_masks(m, kv, window, pos0, [synth.mask_from_layers(4, [1]), np.zeros(8, np.uint8)])
    assert scores[1] == 1.0 and best == 1


def test_scoring_grid_and_parallel_equals_sequential(scoring_setup):
    """Scores are multiples of 1/gamma; the one parallel forward equals teacher-forced
    row-by-row decoding with each candidate's own cache (SWIFT digest §4.1.2)."""
    m, kv, window, pos0 = scoring_setup
    gamma = len(window) - 1
    masks = [synth.mask_from_layers(4, [2]), synth.mask_from_layers(4, [1, 3]), synth.mask_exit(4, 1)]
    scores, best = ssd.score_masks(m, kv, window, pos0, masks)
    assert np.allclose(scores * gamma, np.round(scores * gamma))
    assert best == int(np.argmax(scores))
    for mask, sc in zip(masks, scores):
        kvm = kv.copy()
        hits = 0
        for i in range(gamma):
            z = mdl.forward(m, [window[i]], [pos0 + i], kvm, mask)[0]
            hits += int(np.argmax(z) == window[i + 1])
        assert hits / gamma == sc


def test_scoring_ties_pick_lowest_index(scoring_setup):
    m, kv, window, pos0 = scoring_setup
    mk = synth.mask_from_layers(4, [2])
    scores, best = ssd.score_masks(m, kv, window, pos0, [mk, mk, np.zeros(8, np.uint8), np.zeros(8, np.uint8)])
    assert best == 2


# ---------------------------------------------------------------- lossy early exit
def test_exit_generate_empty_plan_is_ar():
    """With nothing skipped the lossy mode is plain AR (greedy and sampled)."""
    m = _model(synth.TINY)
    prompt = synth.prompt_tokens(16, synth.TINY.vocab)
    for T in (0.0, 1.0):
        ar, _ = ssd.ar_generate(m, prompt, 12, T=T)
        ex, _ = ssd.exit_generate(m, prompt, 12, np.zeros(8, np.uint8), T=T)
        assert ex == ar


def test_exit_generate_equals_truncated_model():
    """Exit at E: after the first token, each step's logits are those of a model
    holding only layers 0..E-1 (same final norm and LM head), prefilled with the
    prompt and the tokens generated so far."""
    m = _model(synth.TINY)
    E = 2
    prompt = synth.prompt_tokens(16, synth.TINY.vocab)
    ex, zs = ssd.exit_generate(m, prompt, 6, synth.mask_exit(4, E))
    trunc = mdl.Model.synthetic(dataclasses.replace(synth.TINY, n_layers=E))   # layers 0..E-1, same tensors
    for k in range(1, 6):
        seq = list(prompt) + ex[:k]
        z = ssd.prefill(trunc, mdl.KVCache(trunc.shape, len(seq) + 1), seq)
        assert np.max(np.abs(z - zs[k])) < 1e-9
        assert ex[k] == int(np.argmax(z))


# ---------------------------------------------------------------- SpecEE features
def test_specee_features_are_the_lm_head_columns():
    """The speculative-token logits are the final-norm + LM-head logits at those
    columns; the local probabilities are their softmax; the variation is the
    difference to the given previous probabilities (zero without them)."""
    m = _model(synth.TINY)
    rng = np.random.default_rng(5)
    h = rng.standard_normal((3, synth.TINY.d_model))
    toks = [7, 1000, 3, 512]
    f = ssd.specee_features(m, h, toks)
    z = mdl.final_logits(m, h)
    assert np.allclose(f[:, :4], z[:, toks], rtol=0, atol=1e-12)
    p = np.exp(z[:, toks] - z[:, toks].max(axis=1, keepdims=True))
    assert np.allclose(f[:, 4:8], p / p.sum(axis=1, keepdims=True), atol=1e-15)
    assert np.allclose(f[:, 4:8].sum(axis=1), 1.0) and not f[:, 8:].any()
    prev = rng.random((3, 4))
    g = ssd.specee_features(m, h, toks, prev)
    assert np.allclose(g[:, 8:], g[:, 4:8] - prev, atol=0)


# ---------------------------------------------------------------- decision margins (parity rule)
def test_top2_gap():
    assert ssd.top2_gap([0.0, 3.0, 1.0]) == 2.0
    assert ssd.top2_gap([5.0, -np.inf]) == float("inf")
    assert ssd.top2_gap([1.0, 1.0]) == 0.0


def test_accept_margin_is_the_distance_to_flipping():
    """The logged margin of an accept decision is |ln(u q(y) / p(y))|: moving p(y)'s logit by 0.9 of it
    toward the threshold keeps the decision, by 1.1 of it flips it."""
    rng = np.random.default_rng(3)
    V, T, seed, it = 16, 1.0, 9, 4
    for trial in range(20):
        zp = rng.standard_normal((2, V))
        zq = rng.standard_normal((1, V))
        y = int(rng.integers(V))
        log = []
        out = ssd.accept_sampled(zp, zq, [y], T, seed, it + trial, log)
        kind, row, m = log[0]
        assert (kind, row) == ("accept", 0)
        accepted = out[0] == y and len(out) == 2
        u = philox.uniforms(seed, it + trial, 0, philox.PURPOSE_ACCEPT, 1)[0]
        lp = ssd.log_softmax(zp[0], T)[y]
        lq = ssd.log_softmax(zq[0], T)[y]
        assert abs(m - abs(np.log(u) + lq - lp)) < 1e-5
        # shift the target's log-probability of y by s (renormalising keeps the others' ratios)
        for frac, flips in ((0.9, False), (1.1, True)):
            s = (-1 if accepted else 1) * frac * m
            if lp + s >= -1e-6:
                continue                  # p'(y) would reach 1
            zs = zp.copy()
            # log p'(y) = lp + s, the other entries scaled equally
            p = np.exp(ssd.log_softmax(zp[0], T))
            pn = p.copy()
            pn[y] = np.exp(lp + s)
            others = np.arange(V) != y
            pn[others] *= (1 - pn[y]) / p[others].sum()
            zs[0] = np.log(pn)
            out2 = ssd.accept_sampled(zs, zq, [y], T, seed, it + trial)
            acc2 = out2[0] == y and len(out2) == 2
            if m > 1e-3:
                assert acc2 == (accepted != flips)


def test_race_gap_is_the_distance_to_flipping():
    """A race sample's logged margin is the top-2 key gap: raising the runner-up's logit by 1.1 gaps
    (T = 1) hands it the draw, by 0.9 gaps does not."""
    rng = np.random.default_rng(8)
    V, seed = 40, 5
    for it in range(15):
        z = rng.standard_normal(V)
        log = []
        t = ssd.pick(z, 1.0, seed, it, 2, philox.PURPOSE_SAMPLE, log)
        kind, row, m = log[0]
        g = philox.gumbel(seed, it, 2, philox.PURPOSE_SAMPLE, V)
        keys = z.astype(np.float32) + g
        second = int(np.argsort(-keys, kind="stable")[1])
        for frac, winner in ((0.9, t), (1.1, second)):
            zz = z.copy()
            zz[second] += frac * m
            assert ssd.pick(zz, 1.0, seed, it, 2, philox.PURPOSE_SAMPLE) == winner


def test_sampled_generation_logs_every_decision():
    """Per iteration: one draft draw per draft row, one stop decision per row when tau > 0, an accept
    decision per tested draft, one final draw (correction or bonus)."""
    m = _model(synth.TINY)
    prompt = synth.prompt_tokens(12, synth.TINY.vocab)
    out, st, _ = ssd.ssd_generate(m, prompt, 20, synth.mask_from_layers(4, [2]), 4, tau=0.01, T=1.0, seed=7)
    assert [k for k, _, _ in st["decisions"][0]] == ["sample"]
    for k, log in enumerate(st["decisions"][1:]):
        dp, e = st["drafted"][k], st["emitted"][k]
        kinds = [x[0] for x in log]
        assert kinds.count("draft") == dp and kinds.count("stop") == dp
        assert kinds.count("accept") == min(e, dp)
        assert kinds.count("sample") == 1
        assert all(mg >= 0 for _, _, mg in log)
