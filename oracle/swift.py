"""SWIFT layer-set search by random search (oracle; test infrastructure).

The optimisation phase of the SWIFT digest (§4.1.1, §4.1.2, §5.3, §B.2):
candidate layer sets are proposed by random search, scored by matchness on the
last context window (the scoring of oracle/ssd.py), and the best one is kept;
the phase ends at a step limit, after a number of steps without improvement, or
once the matchness passes a target (the digest's settings: 1000 steps, 300
unimproved steps, 0.95).  The periodic Bayesian-optimisation step of the pages
is not part of this search.

Readings taken (the pages give no procedure beyond the above):
  * a candidate skips n_skip whole layers (both sub-layers), or n_skip of the
    2L attention / MLP sub-layers when the search runs over sub-layers (SWIFT
    digest Appendix A, Fig. 10: the two kinds are skipped separately);
  * the uniform starting plan (SWIFT digest §1, §4.1.1: "uniform layer
    skipping") skips layers floor((2 i + 1) L / (2 n_skip)), i = 0..n_skip-1,
    i.e. the centres of n_skip equal slices of the stack;
  * a step proposes n_cand sets, each a uniformly random n_skip-subset drawn by
    Fisher-Yates: position i swaps with i + r_i, r_i = (x_i * (L - i)) >> 32
    for the Philox word x_i of key seed, counter (step, candidate, 3, i // 4),
    word i % 4 (the generator of the sampling draws, purpose 3);
  * the incumbent (at step 0 the starting plan, scored with the step's
    proposals) is replaced by the step's best proposal (lowest index on ties)
    only when that proposal scores strictly higher; a step without replacement
    counts as unimproved; the search stops when the incumbent's score exceeds
    the target, after `patience` unimproved steps in a row, or after max_steps.
"""
import numpy as np

from . import philox

PURPOSE_PROPOSE = 3


def layers_to_mask(L, layers):
    m = np.zeros(2 * L, np.uint8)
    for l in layers:
        m[2 * l] = m[2 * l + 1] = 1
    return m


def uniform_skip_layers(L, n_skip):
    """Centres of n_skip equal slices of the L layers."""
    return [((2 * i + 1) * L) // (2 * n_skip) for i in range(n_skip)]


def propose_layers(N, n_skip, seed, step, cand):
    """A uniformly random n_skip-subset of range(N) (Fisher-Yates on Philox words);
    N = L layers or 2L sub-layers."""
    x = philox.words(seed, step, cand, PURPOSE_PROPOSE, n_skip)
    idx = list(range(N))
    for i in range(n_skip):
        r = (int(x[i]) * (N - i)) >> 32
        idx[i], idx[i + r] = idx[i + r], idx[i]
    return sorted(idx[:n_skip])


def propose_mask(L, n_skip, seed, step, cand, sublayers=False):
    if sublayers:
        m = np.zeros(2 * L, np.uint8)
        m[propose_layers(2 * L, n_skip, seed, step, cand)] = 1
        return m
    return layers_to_mask(L, propose_layers(L, n_skip, seed, step, cand))


def search(score_fn, L, init_mask, n_skip, n_cand, max_steps, patience, target, seed, sublayers=False):
    """Random search.  score_fn(list of masks) -> scores.  Returns the final
    incumbent mask, its score, the number of steps run and the per-step
    history [(proposal masks, their scores, incumbent score after the step)]."""
    inc = np.asarray(init_mask, np.uint8).copy()
    inc_score = None
    unimproved = 0
    history = []
    t = 0
    while t < max_steps:
        props = [propose_mask(L, n_skip, seed, t, c, sublayers) for c in range(n_cand)]
        if t == 0:
            sc = list(score_fn([inc] + props))
            inc_score, sc = sc[0], sc[1:]
        else:
            sc = list(score_fn(props))
        k = int(np.argmax(sc))                      # lowest index among the maxima
        if sc[k] > inc_score:
            inc, inc_score = props[k].copy(), sc[k]
            unimproved = 0
        else:
            unimproved += 1
        history.append((props, sc, inc_score))
        t += 1
        if inc_score > target or unimproved >= patience:
            break
    return inc, inc_score, t, history
