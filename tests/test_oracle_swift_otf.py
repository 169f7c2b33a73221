"""Pins of SWIFT's on-the-fly alternation in the oracle (oracle/swift.py
swift_generate; SWIFT digest §4, §4.1.1, §4.1.2, §B.2, §D.2): lossless tokens,
the phase schedule, switches only on strict improvement (re-derived from the
recorded scores, and the scores re-derived from a fresh full-model cache), the
stopping rules, continuation of the step numbering, and the degenerate cases
(no optimisation = plain SSD with the starting plan; an empty candidate set =
the full model, matchness exactly 1).  CPU only."""
import numpy as np
import pytest

import synth
from oracle import model as mdl
from oracle import ssd as ossd
from oracle import swift

L4 = 4


def _model():
    return mdl.Model.synthetic(synth.TINY)


def _ar_cache(m, prompt, tokens, n):
    """The full model's cache for the positions before committed token n - 1 (tokens[:n - 1] after the prompt)."""
    seq = list(prompt) + list(tokens[:n - 1])
    kv = mdl.KVCache(synth.TINY, len(seq) + 64)
    mdl.forward(m, seq, range(len(seq)), kv)
    return kv


def _rederive(phase):
    """The plan and score a phase must end with, and its trailing unimproved run, from its recorded
    scores: the incumbent is replaced by a step's best proposal (lowest index on ties) only when that
    scores strictly higher."""
    inc, best, u = phase["before"], phase["score0"], phase["unimproved0"]
    for props, sc, _ in phase["history"]:
        k = int(np.argmax(sc))
        if sc[k] > best:
            inc, best, u = props[k], sc[k], 0
        else:
            u += 1
    return inc, best, u


def _check_schedule(tr, prompt, gamma, acc, d, max_steps, patience, target):
    """Phases run exactly after the iterations at which they are due; iterations draft with the plan
    of the last phase before them; the step count and the unimproved run carry over."""
    plan = tr["plans"][1]
    last, steps, u, done, pi = 1, 0, 0, max_steps <= 0, 0
    for k in range(1, len(tr["plans"])):
        assert np.array_equal(tr["plans"][k], plan), k
        n = tr["n_out"][k]
        due = not done and n - last >= acc and n >= gamma + 1
        if not due:
            continue
        ph = tr["phases"][pi]
        pi += 1
        assert ph["n_out"] == n and ph["pos0"] == len(prompt) + n - 1 - gamma
        assert np.array_equal(ph["before"], plan) and ph["step0"] == steps and ph["unimproved0"] == u
        assert 1 <= ph["steps"] <= max_steps - steps
        inc, best, u = _rederive(ph)
        assert np.array_equal(inc, ph["after"]) and best == ph["score"]
        plan = ph["after"]
        steps += ph["steps"]
        done = steps >= max_steps or u >= patience or best > target
        last = n
    assert pi == len(tr["phases"])
    assert (steps, u, done) == (tr["steps"], tr["unimproved"], tr["done"])
    if len(tr["n_out"]) > 1:
        assert all(1 <= b - a <= d + 1 for a, b in zip(tr["n_out"], tr["n_out"][1:]))


@pytest.fixture(scope="module")
def run():
    m = _model()
    prompt = synth.prompt_tokens(24, synth.TINY.vocab)
    kw = dict(n_skip=2, gamma=8, n_cand=3, steps_per_phase=2, max_steps=9, patience=100, target=0.95, d=3)
    toks, tr = swift.swift_generate(m, prompt, 64, **kw)
    return m, prompt, kw, toks, tr


def test_greedy_tokens_equal_ar(run):
    m, prompt, kw, toks, tr = run
    ar, _ = ossd.ar_generate(m, prompt, 64)
    assert toks == ar
    assert len(tr["phases"]) >= 3


def test_schedule_switches_and_carry(run):
    m, prompt, kw, toks, tr = run
    _check_schedule(tr, prompt, kw["gamma"], kw["gamma"], kw["d"], kw["max_steps"], kw["patience"], kw["target"])
    for ph in tr["phases"]:
        if not np.array_equal(ph["before"], ph["after"]):
            assert ph["score"] > ph["score0"]
        # the step numbering continues: a phase's first proposals are those of its global step
        for c, p in enumerate(ph["history"][0][0]):
            assert np.array_equal(p, swift.propose_mask(L4, kw["n_skip"], 3, ph["step0"], c))


def test_scores_recomputed_from_a_fresh_cache(run):
    """Every phase's first-step scores re-derived with a full-model cache built by a plain prefill."""
    m, prompt, kw, toks, tr = run
    g = kw["gamma"]
    for ph in tr["phases"]:
        n_out = ph["n_out"]
        kv = _ar_cache(m, prompt, toks, n_out - g)
        window = toks[n_out - 1 - g:n_out]
        props, sc, _ = ph["history"][0]
        got = ossd.score_masks(m, kv, window, ph["pos0"], [ph["before"]] + list(props))[0]
        assert got[0] == ph["score0"] and list(got[1:]) == list(sc)


def test_no_optimisation_is_plain_ssd():
    """max_steps = 0: no phase; the tokens (greedy and sampled) are ssd_generate's with the starting plan."""
    m = _model()
    prompt = synth.prompt_tokens(16, synth.TINY.vocab)
    plan = swift.layers_to_mask(L4, swift.uniform_skip_layers(L4, 1))
    for T, tau in ((0.0, 0.0), (1.0, 0.3)):
        toks, tr = swift.swift_generate(m, prompt, 40, 1, 8, 3, 2, 0, 10, 0.95, 3, tau=tau, T=T, seed=5)
        ref, _, _ = ossd.ssd_generate(m, prompt, 40, plan, 3, tau=tau, T=T, seed=5)
        assert toks == ref and tr["phases"] == [] and tr["done"]


def test_empty_candidates_score_one_and_stop():
    """n_skip = 0: every plan is the full model, which predicts its own greedy continuation: matchness
    exactly 1 > target, so optimisation ends after one step; every later iteration accepts all d drafts."""
    m = _model()
    prompt = synth.prompt_tokens(16, synth.TINY.vocab)
    toks, tr = swift.swift_generate(m, prompt, 48, 0, 8, 2, 4, 50, 10, 0.95, 3)
    assert len(tr["phases"]) == 1
    ph = tr["phases"][0]
    assert ph["score0"] == 1.0 and ph["score"] == 1.0 and ph["steps"] == 1 and tr["done"]
    assert not ph["after"].any()
    assert all(b - a == 4 for a, b in zip(tr["n_out"][1:], tr["n_out"][2:]))
    ar, _ = ossd.ar_generate(m, prompt, 48)
    assert toks == ar


@pytest.mark.parametrize("patience,max_steps,per", [(2, 50, 1), (100, 3, 2), (3, 7, 2)])
def test_stop_rules(patience, max_steps, per):
    m = _model()
    prompt = synth.prompt_tokens(20, synth.TINY.vocab)
    toks, tr = swift.swift_generate(m, prompt, 120, 2, 8, 2, per, max_steps, patience, 1.5, 2, seed=11)
    # target 1.5 is unreachable: only the step budget or the unimproved run can end optimisation
    _check_schedule(tr, prompt, 8, 8, 2, max_steps, patience, 1.5)
    assert tr["done"]


def test_sliding_window_schedule():
    """accumulate = steps_per_phase = 1: one optimisation step after every iteration once the window is full."""
    m = _model()
    prompt = synth.prompt_tokens(16, synth.TINY.vocab)
    toks, tr = swift.swift_generate(m, prompt, 40, 2, 8, 2, 1, 100, 100, 1.5, 2, accumulate=1)
    _check_schedule(tr, prompt, 8, 1, 2, 100, 100, 1.5)
    full = [k for k in range(1, len(tr["n_out"])) if tr["n_out"][k] >= 9]
    assert len(tr["phases"]) == len(full) and all(ph["steps"] == 1 for ph in tr["phases"])


def test_bayesian_steps_follow_the_global_count():
    """bo_every counts the steps of all phases: with one step per phase and bo_every = 3, the phases at global
    steps 3, 6, ... rank a pool (when the phase's own scores vary) or propose at random otherwise."""
    m = _model()
    prompt = synth.prompt_tokens(16, synth.TINY.vocab)
    toks, tr = swift.swift_generate(m, prompt, 80, 2, 8, 3, 2, 12, 100, 1.5, 2, bo_every=3)
    _check_schedule(tr, prompt, 8, 8, 2, 12, 100, 1.5)
    for ph in tr["phases"]:
        for t, (props, sc, _) in enumerate(ph["history"]):
            st = ph["step0"] + t
            rnd = [swift.propose_mask(L4, 2, 3, st, c) for c in range(3)]
            if st % 3 != 0 or t == 0:
                # random proposals: not a Bayesian step, or the phase has no scores yet at its first step
                assert all(np.array_equal(a, b) for a, b in zip(props, rnd))
            else:
                # a Bayesian step scores plans of its pool (or, all scores equal, the random ones)
                pool = [swift.propose_mask(L4, 2, 3, st, c) for c in range(8 * 3)]
                assert all(any(np.array_equal(p, q) for q in pool) for p in props)
