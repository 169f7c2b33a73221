"""Pins of the SWIFT layer-set search (oracle/swift.py) and of the library's
host-side helpers (uniform plan, proposals), which must equal the oracle's bit
for bit.  No GPU: the helpers make no device call."""
import itertools

import numpy as np
import pytest
from scipy import stats

from oracle import swift


@pytest.mark.parametrize("L,n,expect", [
    (40, 20, list(range(1, 40, 2))),        # every other layer, the odd ones
    (4, 1, [2]),                             # the tiny workload's "skip layer 2"
    (32, 8, list(range(2, 32, 4))),
    (5, 5, [0, 1, 2, 3, 4]),
    (6, 0, []),
])
def test_uniform_skip_closed_forms(L, n, expect):
    assert swift.uniform_skip_layers(L, n) == expect


@pytest.mark.parametrize("L,n", [(40, 16), (80, 40), (13, 5), (7, 3)])
def test_uniform_skip_is_evenly_spread(L, n):
    lay = swift.uniform_skip_layers(L, n)
    assert len(set(lay)) == n and lay == sorted(lay) and 0 <= lay[0] and lay[-1] < L
    gaps = np.diff([lay[0]] + lay + [lay[-1] + (L - lay[-1]) + lay[0]])  # including the wrap-around gap
    assert gaps[1:-1].max() - gaps[1:-1].min() <= 1 if n > 2 else True
    # each slice [i L / n, (i + 1) L / n) holds exactly one skipped layer
    for i, l in enumerate(lay):
        assert i * L <= l * n < (i + 1) * L


def test_proposals_are_uniform_subsets():
    """6000 proposals of 2 of 6 layers: every one a 2-subset, the 15 subsets
    equally likely (chi-square, p > 1e-3)."""
    L, n = 6, 2
    subsets = list(itertools.combinations(range(L), n))
    counts = np.zeros(len(subsets))
    for t in range(600):
        for c in range(10):
            p = swift.propose_layers(L, n, 2024, t, c)
            assert len(p) == n and len(set(p)) == n and all(0 <= x < L for x in p)
            counts[subsets.index(tuple(p))] += 1
    assert stats.chisquare(counts).pvalue > 1e-3


def test_proposals_depend_on_step_candidate_and_seed():
    a = swift.propose_layers(40, 20, 7, 0, 0)
    assert a == swift.propose_layers(40, 20, 7, 0, 0)
    others = [swift.propose_layers(40, 20, 7, 1, 0), swift.propose_layers(40, 20, 7, 0, 1),
              swift.propose_layers(40, 20, 8, 0, 0)]
    assert all(o != a for o in others)


def _score_table(good, n):
    def f(masks):
        return [len(good & set(np.nonzero(m[::2])[0].tolist())) / n for m in masks]
    return f


def test_search_finds_target_and_stops():
    """Score = fraction of the skipped layers inside {1, 4}: the search stops at
    the first step whose proposals contain {1, 4} (score 1 > 0.95)."""
    L, n = 6, 2
    init = swift.layers_to_mask(L, [0, 2])
    for seed in (11, 12, 13):
        best, score, steps, hist = swift.search(_score_table({1, 4}, n), L, init, n, 3, 200, 200, 0.95, seed)
        first = next(t for t in range(200)
                     if any(swift.propose_layers(L, n, seed, t, c) == [1, 4] for c in range(3)))
        assert steps == first + 1 and score == 1.0
        assert np.array_equal(best, swift.layers_to_mask(L, [1, 4]))
    # the incumbent's score never decreases and changes only on a strict improvement
    inc = [h[2] for h in hist]
    assert all(b >= a for a, b in zip(inc, inc[1:]))


def test_search_patience_and_step_limit():
    L, n = 8, 3
    init = swift.layers_to_mask(L, [0, 1, 2])
    flat = lambda masks: [0.25] * len(masks)
    best, score, steps, _ = swift.search(flat, L, init, n, 4, 50, 7, 0.95, 3)
    assert steps == 7 and score == 0.25 and np.array_equal(best, init)
    best, score, steps, _ = swift.search(flat, L, init, n, 4, 5, 7, 0.95, 3)
    assert steps == 5


def test_search_ties_take_the_lowest_index():
    """Two proposals share the best score above the incumbent: the first wins."""
    L, n, seed = 8, 3, 5
    init = swift.layers_to_mask(L, [0, 1, 2])
    props = [swift.layers_to_mask(L, swift.propose_layers(L, n, seed, 0, c)) for c in range(4)]

    def f(masks):
        if len(masks) == 5:                              # step 0: incumbent + 4 proposals
            return [0.1, 0.2, 0.5, 0.3, 0.5]
        return [0.0] * len(masks)
    best, score, steps, _ = swift.search(f, L, init, n, 4, 3, 10, 0.95, seed)
    assert np.array_equal(best, props[1]) and score == 0.5 and steps == 3


def test_library_helpers_equal_the_oracle():
    from self_speculative_layer_amd import binding as B
    for L, n in [(4, 1), (40, 20), (32, 8), (80, 40), (5, 3), (7, 7), (3, 0)]:
        assert np.array_equal(B.ssd_uniform_mask(L, n), swift.layers_to_mask(L, swift.uniform_skip_layers(L, n)))
    for L, n in [(8, 3), (40, 20), (80, 40), (5, 5), (6, 1)]:
        for t in range(4):
            for c in range(6):
                assert np.array_equal(B.ssd_swift_propose(L, n, 12345678901, t, c),
                                      swift.layers_to_mask(L, swift.propose_layers(L, n, 12345678901, t, c)))
                assert np.array_equal(B.ssd_swift_propose(L, n, 99, t, c, sublayers=True),
                                      swift.propose_mask(L, n, 99, t, c, sublayers=True))


def test_sublayer_proposals_are_uniform():
    """Sub-layer proposals: n_skip mask bits set, each of the 2L bits equally
    likely (chi-square over 4000 proposals of 3 of 8 sub-layers)."""
    L, n = 4, 3
    counts = np.zeros(2 * L)
    for t in range(400):
        for c in range(10):
            m = swift.propose_mask(L, n, 31, t, c, sublayers=True)
            assert m.sum() == n
            counts += m
    assert stats.chisquare(counts).pvalue > 1e-3


def test_library_helpers_reject_bad_arguments():
    from self_speculative_layer_amd import binding as B
    for args in [(0, 0), (4, 5), (4, -1)]:
        with pytest.raises(B.SSDError):
            B.ssd_uniform_mask(*args)
    with pytest.raises(B.SSDError):
        B.ssd_swift_propose(4, 5, 1, 0, 0)                 # more layers than there are
    with pytest.raises(B.SSDError):
        B.ssd_swift_propose(4, 9, 1, 0, 0, sublayers=True)  # more sub-layers than there are
    with pytest.raises(B.SSDError):
        B.ssd_swift_propose(4, 1, 1, -1, 0)
    assert B.ssd_swift_propose(4, 8, 1, 0, 0, sublayers=True).all()


# ---------------------------------------------------------------- Bayesian-optimisation step
def test_gp_posterior_matches_sklearn():
    """The GP of the BO step against scikit-learn's Gaussian-process regressor with
    the same fixed kernel (RBF, length scale sqrt(ell2)) and noise."""
    from sklearn.gaussian_process import GaussianProcessRegressor
    from sklearn.gaussian_process.kernels import RBF
    rng = np.random.default_rng(5)
    X = (rng.random((40, 16)) < 0.5).astype(np.float64)
    y = rng.standard_normal(40)
    Xq = (rng.random((25, 16)) < 0.5).astype(np.float64)
    ell2 = 8.0
    mu, sd = swift.gp_posterior(X, y, Xq, ell2, noise=1e-6)
    ref = GaussianProcessRegressor(kernel=RBF(length_scale=np.sqrt(ell2), length_scale_bounds="fixed"), alpha=1e-6,
                                   optimizer=None, normalize_y=False).fit(X, y)
    rmu, rsd = ref.predict(Xq, return_std=True)
    np.testing.assert_allclose(mu, rmu, rtol=0, atol=1e-8)
    np.testing.assert_allclose(sd, rsd, rtol=0, atol=1e-6)
    # interpolation: at a training point the mean is the observation and the spread vanishes
    m0, s0 = swift.gp_posterior(X, y, X[:3], ell2, noise=1e-10)
    np.testing.assert_allclose(m0, y[:3], atol=1e-6)
    assert np.all(s0 < 1e-3)


@pytest.mark.parametrize("mu,sd,best", [(0.3, 0.7, 0.1), (-1.0, 0.5, 0.2), (2.0, 1e-3, 0.5), (0.0, 2.0, 0.0),
                                        (0.4, 0.0, 0.1), (0.1, 0.0, 0.4)])
def test_expected_improvement_is_the_integral(mu, sd, best):
    from scipy import integrate, stats
    got = swift.expected_improvement([mu], [sd], best)[0]
    if sd == 0:
        assert got == max(mu - best, 0.0)
        return
    ref, _ = integrate.quad(lambda v: (v - best) * stats.norm.pdf(v, mu, sd), best, mu + 12 * sd, limit=200)
    assert abs(got - ref) < 1e-9 * max(1.0, abs(ref))


def test_bo_step_prefers_plans_the_model_expects_to_score_higher():
    """On a score that counts the skipped layers of a hidden good set, the BO
    step's picks score far above the pool they come from (a sign error in the
    improvement, a transposed kernel or a wrong ordering would not)."""
    L, n_skip, n_cand = 24, 8, 6
    good = set(range(0, 24, 2))
    score = lambda m: sum(1 for l in range(L) if m[2 * l] and l in good) / n_skip
    obs = [swift.propose_mask(L, n_skip, 9, 0, c) for c in range(60)]
    ys = [score(m) for m in obs]
    pool = [swift.propose_mask(L, n_skip, 9, 1, c) for c in range(8 * n_cand)]
    picks = swift.bo_proposals(obs, ys, max(ys), pool, n_cand)
    assert np.mean([score(m) for m in picks]) > np.mean([score(m) for m in pool]) + 0.15
    assert swift.bo_proposals(obs, [0.5] * len(obs), 0.5, pool, n_cand) is None   # nothing to model


def test_search_without_a_bo_step_in_range_is_random_search():
    L, n_skip = 12, 4
    fn = lambda ms: [float(m[::2][:6].sum()) / n_skip for m in ms]
    init = swift.layers_to_mask(L, swift.uniform_skip_layers(L, n_skip))
    a = swift.search(fn, L, init, n_skip, 5, 6, 100, 2.0, 3)
    b = swift.search(fn, L, init, n_skip, 5, 6, 100, 2.0, 3, bo_every=7)
    assert a[1] == b[1] and a[2] == b[2] and np.array_equal(a[0], b[0])
    c = swift.search(fn, L, init, n_skip, 5, 6, 100, 2.0, 3, bo_every=2)
    same = lambda ha, hb: all(np.array_equal(x, y) for x, y in zip(ha[0], hb[0]))
    assert same(a[3][0], c[3][0]) and same(a[3][1], c[3][1])   # steps 0, 1: random proposals
    assert not same(a[3][2], c[3][2])                           # step 2: the BO step's picks
