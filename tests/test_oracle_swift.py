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
