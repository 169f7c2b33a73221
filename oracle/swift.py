"""SWIFT layer-set search by random search (oracle; test infrastructure).

The optimisation phase of the SWIFT digest (§4.1.1, §4.1.2, §5.3, §B.2):
candidate layer sets are proposed by random search, scored by matchness on the
last context window (the scoring of oracle/ssd.py), and the best one is kept;
the phase ends at a step limit, after a number of steps without improvement, or
once the matchness passes a target (the digest's settings: 1000 steps, 300
unimproved steps, 0.95, and a Bayesian-optimisation step every 25 steps).

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
    the target, after `patience` unimproved steps in a row, or after max_steps;
  * the Bayesian-optimisation step (every bo_every-th step, t > 0; SWIFT digest
    §4.1.2 "periodic Bayesian optimization", §B.2 every 25 steps, §5.3 the
    interval beta): a Gaussian process over the mask vectors x in {0,1}^{2L} of
    the most recent bo_window scored plans (zero-mean after subtracting the
    scores' mean and dividing by their standard deviation; squared-exponential
    kernel exp(-|x - x'|^2 / (2 l^2)) with l^2 = the number of skipped entries,
    unit signal variance, 1e-6 noise) ranks a pool of pool_factor * n_cand
    random proposals (counter (step, candidate) as above, candidates 0..pool-1)
    by expected improvement over the incumbent's score; the n_cand best (lower
    pool index first among equal values) are scored, in that order.  When the
    scores seen so far are all equal there is nothing to model and the step
    proposes at random like the others.
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


def gp_posterior(X, y, Xq, ell2, noise=1e-6):
    """Posterior mean and standard deviation at Xq of a zero-mean Gaussian
    process with kernel exp(-|x - x'|^2 / (2 ell2)) (unit signal variance) and
    observation noise `noise`, conditioned on (X, y)."""
    X = np.asarray(X, np.float64)
    Xq = np.asarray(Xq, np.float64)
    def kern(A, B):
        d2 = ((A[:, None, :] - B[None, :, :]) ** 2).sum(-1)
        return np.exp(-d2 / (2.0 * ell2))
    Kxx = kern(X, X) + noise * np.eye(len(X))
    Kqx = kern(Xq, X)
    alpha = np.linalg.solve(Kxx, np.asarray(y, np.float64))
    mu = Kqx @ alpha
    v = np.linalg.solve(Kxx, Kqx.T)
    var = np.maximum(1.0 - np.sum(Kqx * v.T, axis=1), 0.0)
    return mu, np.sqrt(var)


def expected_improvement(mu, sd, best):
    """E[max(Y - best, 0)] for Y ~ N(mu, sd^2); max(mu - best, 0) where sd = 0."""
    from math import erfc, exp, pi, sqrt
    out = []
    for m, s in zip(np.atleast_1d(mu), np.atleast_1d(sd)):
        if s <= 1e-12:
            out.append(max(m - best, 0.0))
            continue
        z = (m - best) / s
        cdf = 0.5 * erfc(-z / sqrt(2.0))
        pdf = exp(-0.5 * z * z) / sqrt(2.0 * pi)
        out.append((m - best) * cdf + s * pdf)
    return np.array(out)


def bo_proposals(obs_masks, obs_scores, inc_score, pool, n_cand):
    """The n_cand pool plans with the highest expected improvement under the GP
    of the observed (mask, score) pairs (the module's reading), best first,
    lower pool index first among equal values; None when the observed scores
    are all equal."""
    y = np.asarray(obs_scores, np.float64)
    sd = y.std()
    if not sd > 0:
        return None
    mean = y.mean()
    ell2 = float(np.asarray(pool[0]).sum())
    mu, s = gp_posterior(obs_masks, (y - mean) / sd, pool, ell2)
    ei = expected_improvement(mu, s, (inc_score - mean) / sd)
    order = sorted(range(len(pool)), key=lambda i: (-ei[i], i))
    return [pool[i] for i in order[:n_cand]]


def search(score_fn, L, init_mask, n_skip, n_cand, max_steps, patience, target, seed, sublayers=False, bo_every=0,
           pool_factor=8, bo_window=256, step0=0, unimproved0=0, out=None):
    """Random search with the periodic Bayesian-optimisation step.  score_fn(list
    of masks) -> scores.  Returns the final incumbent mask, its score, the
    number of steps run and the per-step history [(proposal masks, their
    scores, incumbent score after the step)].

    A search that continues earlier ones (the on-the-fly alternation below)
    numbers its steps from step0 (proposal counters and the Bayesian schedule
    use step0 + t) and starts its run of unimproved steps at unimproved0; the
    run at the end goes to out["unimproved"] when out is a dict (and the
    starting plan's score to out["score0"])."""
    inc = np.asarray(init_mask, np.uint8).copy()
    inc_score = None
    unimproved = unimproved0
    history = []
    obs_m, obs_s = [], []
    t = 0
    while t < max_steps:
        st = step0 + t
        props = None
        if bo_every > 0 and st > 0 and st % bo_every == 0 and obs_s:
            pool = [propose_mask(L, n_skip, seed, st, c, sublayers) for c in range(pool_factor * n_cand)]
            props = bo_proposals(obs_m[-bo_window:], obs_s[-bo_window:], inc_score, pool, n_cand)
        if props is None:
            props = [propose_mask(L, n_skip, seed, st, c, sublayers) for c in range(n_cand)]
        if t == 0:
            sc = list(score_fn([inc] + props))
            inc_score, sc = sc[0], sc[1:]
            score0 = inc_score
        else:
            sc = list(score_fn(props))
        if t == 0:
            obs_m.append(inc.copy())
            obs_s.append(inc_score)
        obs_m.extend(p.copy() for p in props)
        obs_s.extend(sc)
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
    if out is not None and t > 0:
        out["unimproved"] = unimproved
        out["score0"] = score0
    return inc, inc_score, t, history


def swift_generate(model, prompt, n_gen, n_skip, gamma, n_cand, steps_per_phase, max_steps, patience, target, d,
                   tau=0.0, T=0.0, seed=3, bo_every=0, sublayers=False, accumulate=None, init_mask=None,
                   capacity=None):
    """SWIFT's on-the-fly alternation of context accumulation and layer-set
    optimisation during generation (SWIFT digest §4, §4.1.1, §4.1.2, §5.3,
    §B.2, §D.2).

    Readings (the pages name the phases and their stopping rules, not the
    schedule between them):
      * generation starts with init_mask (default: the uniform plan of n_skip
        whole layers; a sub-layer search must be given one) and
        runs self-speculative iterations (oracle.ssd: draft, verify, accept)
        with the plan in use;
      * once `accumulate` tokens (default gamma) have been committed since the
        previous optimisation phase (for the first phase: since the prefill's
        token), and optimisation is not over, a phase runs on the window of the
        last gamma + 1 committed tokens: `search` with the plan in use as the
        starting incumbent (scored afresh on this window together with the
        phase's first proposals), steps numbered on from the earlier phases
        (proposal counters and the Bayesian schedule), the run of unimproved
        steps carried over, at most steps_per_phase steps;
      * the plan in use becomes the phase's final incumbent, which differs
        from it only when some proposal scored strictly higher on the window;
      * optimisation is over for good once max_steps steps have run in all
        phases, once the run of unimproved steps reaches patience, or once the
        incumbent's score exceeds target; generation goes on with the last plan.
    With accumulate = steps_per_phase = 1 this is one optimisation step after
    every iteration on a window that slides with the generated text.

    Returns (tokens [n_gen], trace): trace["phases"] holds, per phase, n_out
    (committed tokens when it ran), pos0, the plan before and after, the
    incumbent's score, the steps run and the per-step history;
    trace["plans"][k] is the plan iteration k (1-based) drafted with and
    trace["n_out"][k] the committed count after it; trace also has the final
    state (steps, unimproved, done).
    """
    from . import model as mdl
    from . import ssd as ossd
    P = len(prompt)
    L = model.L
    acc = gamma if accumulate is None else accumulate
    if init_mask is None:
        if sublayers:
            raise ValueError("a sub-layer search needs its starting plan")
        init_mask = layers_to_mask(L, uniform_skip_layers(L, n_skip))
    plan = np.asarray(init_mask, np.uint8).copy()
    kv = mdl.KVCache(model.shape, capacity or (P + n_gen + d + 2))
    out = [ossd.pick(ossd.prefill(model, kv, prompt), T, seed, 0, 0, philox.PURPOSE_SAMPLE)]
    trace = {"phases": [], "plans": [None], "n_out": [1]}
    steps, unimproved, done, last = 0, 0, max_steps <= 0, 1
    it = 1
    while len(out) < n_gen:
        n = P + len(out)
        b = mdl.first_skipped_layer(plan, L)
        y0 = out[-1]
        drafts, zq, hb = ossd.draft(model, kv, y0, n, plan, d, tau, T, seed, it)
        zp = ossd.verify(model, kv, y0, drafts, n, b, hb)
        emitted = ossd.accept_greedy(zp, drafts) if T == 0 else ossd.accept_sampled(zp, zq, drafts, T, seed, it)
        trace["plans"].append(plan.copy())
        out.extend(emitted)
        trace["n_out"].append(len(out))
        it += 1
        if not done and len(out) - last >= acc and len(out) >= gamma + 1:
            n_out = len(out)
            pos0 = P + n_out - 1 - gamma
            window = out[n_out - 1 - gamma:n_out]

            def score_fn(masks):
                return ossd.score_masks(model, kv, window, pos0, masks)[0]
            st = {}
            inc, sc, ran, hist = search(score_fn, L, plan, n_skip, n_cand, min(steps_per_phase, max_steps - steps),
                                        patience, target, seed, sublayers, bo_every, step0=steps,
                                        unimproved0=unimproved, out=st)
            trace["phases"].append({"n_out": n_out, "pos0": pos0, "before": plan.copy(), "after": inc.copy(),
                                    "score0": st["score0"], "score": sc, "steps": ran, "history": hist,
                                    "unimproved0": unimproved, "step0": steps})
            plan = inc.copy()
            steps += ran
            unimproved = st["unimproved"]
            done = steps >= max_steps or unimproved >= patience or sc > target
            last = n_out
    trace.update(steps=steps, unimproved=unimproved, done=done)
    return out[:n_gen], trace
