"""Pins of the oracle's draft-tree functions (SWIFT digest §4.2 dynamic
verification, with the readings R1-R4 of oracle/tree.py): closed forms of the
candidate count, brute-force ranking, hand-built acceptance cases, the leaf
logits against token-by-token decoding, and the loop against plain greedy AR
decoding (every emitted token is the full model's greedy choice)."""
import itertools

import numpy as np
import pytest

import synth
from oracle import model as mdl
from oracle import ssd, tree


# ---------------------------------------------------------------- ranking
def test_topk_lowest_matches_brute_force_with_ties():
    rng = np.random.default_rng(7)
    for _ in range(200):
        n = int(rng.integers(1, 12))
        z = rng.integers(-2, 3, size=n).astype(np.float64)      # many ties
        k = int(rng.integers(1, n + 1))
        ref = [i for _, i in sorted((-z[i], i) for i in range(n))][:k]
        assert tree.topk_lowest(z, k) == ref


# ---------------------------------------------------------------- R1 closed forms
@pytest.mark.parametrize("rho,k_max,expect", [
    (0.49, 4, 1), (0.51, 4, 2), (0.74, 4, 2), (0.76, 4, 3), (0.99, 4, 4), (0.99, 2, 2), (0.3, 1, 1),
])
def test_candidate_count_dyadic(rho, k_max, expect):
    """q = (1/2, 1/4, 1/8, 1/8): top-k mass 1/2, 3/4, 7/8, 1."""
    z = np.log(np.array([0.125, 0.5, 0.125, 0.25]))
    assert tree.candidate_count(z, rho, k_max) == expect


@pytest.mark.parametrize("V,rho,expect", [(10, 0.35, 4), (10, 0.05, 1), (20, 0.52, 11), (7, 0.99, 7)])
def test_candidate_count_uniform(V, rho, expect):
    """Equal logits: k = ceil(rho * V) (no boundary case), capped at k_max = V."""
    assert tree.candidate_count(np.zeros(V), rho, V) == expect


def test_candidate_count_confident_row_is_one():
    z = np.zeros(50)
    z[17] = 60.0
    assert tree.candidate_count(z, 0.999999, 8) == 1


# ---------------------------------------------------------------- R2/R3 leaves
def test_leaves_depth_then_rank_order_and_budget():
    V = 6
    z1 = np.log(np.array([0.05, 0.4, 0.05, 0.3, 0.1, 0.1]))      # ranks 1, 3, 4, 5 (tie: 4 first), 0, 2
    z2 = np.log(np.array([0.02, 0.02, 0.02, 0.9, 0.02, 0.02]))    # confident
    z3 = np.log(np.array([0.3, 0.3, 0.1, 0.1, 0.1, 0.1]))         # ties: 0 before 1, 2 before 3; mass < 0.85
    zq = np.stack([z1, z2, z3])
    drafts = [1, 3, 0]
    # top-k mass: z1 0.4, 0.7, 0.8, 0.9 -> k = 4; z2 -> 1; z3 0.3, 0.6, 0.7, 0.8 -> k_max
    assert tree.tree_leaves(zq, drafts, 0.85, 4, 10) == [(1, 3), (1, 4), (1, 5), (3, 1), (3, 2), (3, 3)]
    assert tree.tree_leaves(zq, drafts, 0.85, 4, 4) == [(1, 3), (1, 4), (1, 5), (3, 1)]
    assert tree.tree_leaves(zq, drafts, 0.85, 2, 10) == [(1, 3), (3, 1)]
    assert tree.tree_leaves(zq, drafts, 0.85, 4, 0) == []
    assert tree.tree_leaves(zq, drafts, 0.2, 4, 10) == []
    assert len(zq[0]) == V


# ---------------------------------------------------------------- R4 acceptance
def _onehot(V, i):
    z = np.zeros(V)
    z[i] = 1.0
    return z


def test_accept_tree_cases():
    V = 8
    drafts = [2, 5, 7]
    leaves = [(1, 4), (2, 6), (2, 1)]
    zl = np.stack([_onehot(V, 0), _onehot(V, 3), _onehot(V, 4)])
    # every draft accepted: the chain's bonus; leaves ignored
    zp = np.stack([_onehot(V, 2), _onehot(V, 5), _onehot(V, 7), _onehot(V, 6)])
    assert tree.accept_tree_greedy(zp, zl, drafts, leaves) == ([2, 5, 7, 6], None)
    # depth 2 rejected, the target's choice is the second leaf of depth 2: leaf + its own bonus
    zp = np.stack([_onehot(V, 2), _onehot(V, 1), _onehot(V, 0), _onehot(V, 0)])
    assert tree.accept_tree_greedy(zp, zl, drafts, leaves) == ([2, 1, 4], 2)
    # depth 1 rejected, the choice is the depth-1 leaf
    zp = np.stack([_onehot(V, 4), _onehot(V, 0), _onehot(V, 0), _onehot(V, 0)])
    assert tree.accept_tree_greedy(zp, zl, drafts, leaves) == ([4, 0], 0)
    # a leaf token of another depth does not count
    zp = np.stack([_onehot(V, 6), _onehot(V, 0), _onehot(V, 0), _onehot(V, 0)])
    assert tree.accept_tree_greedy(zp, zl, drafts, leaves) == ([6], None)
    # no leaves: the chain rule of ssd.accept_greedy
    for a in itertools.product(range(3), repeat=4):
        zp = np.stack([_onehot(V, [2, 0, 1][x]) if i == 0 else _onehot(V, [5, 7, 3][x]) for i, x in enumerate(a)])
        assert tree.accept_tree_greedy(zp, np.zeros((0, V)), drafts, []) == (ssd.accept_greedy(zp, drafts), None)


# ---------------------------------------------------------------- verify
BF16_SMALL = synth.ModelShape("bf16-small", 3, 128, 4, 2, 32, 160, 300, "bf16")


@pytest.mark.parametrize("shape", [synth.TINY, BF16_SMALL], ids=lambda s: s.name)
def test_leaf_logits_equal_token_by_token_decoding(shape):
    """A leaf's logits are the full model's next-token logits after its path,
    decoded one token at a time from the committed cache; the chain rows are
    ssd.verify's; the cache after verify_tree equals the cache after ssd.verify."""
    m = mdl.Model.synthetic(shape)
    P = 12
    prompt = synth.prompt_tokens(P, shape.vocab)
    kv = mdl.KVCache(shape, P + 16)
    z = ssd.prefill(m, kv, prompt)
    y0 = argmax = int(np.argmax(z))
    n = P + 1
    rng = np.random.default_rng(3)
    drafts = [int(t) for t in rng.integers(0, shape.vocab, 4)]
    leaves = [(1, int(rng.integers(shape.vocab))), (3, int(rng.integers(shape.vocab))), (3, drafts[2])]
    kv_a, kv_b = kv.copy(), kv.copy()
    zp, zl = tree.verify_tree(m, kv_a, y0, drafts, leaves, n, 0)
    zp_ref = ssd.verify(m, kv_b, y0, drafts, n, 0)
    np.testing.assert_array_equal(zp, zp_ref)
    for name in ("K", "V"):
        np.testing.assert_array_equal(getattr(kv_a, name), getattr(kv_b, name))
    for s, (j, c) in enumerate(leaves):
        kvt = kv.copy()
        path = [y0] + drafts[: j - 1] + [c]
        for i, t in enumerate(path):
            zt = mdl.forward(m, [t], [n - 1 + i], kvt)[0]
        np.testing.assert_allclose(zl[s], zt, rtol=0, atol=1e-9 * np.abs(zt).max())
    # the leaf that repeats the chain token reproduces the chain row
    np.testing.assert_allclose(zl[2], zp[3], rtol=0, atol=1e-9 * np.abs(zp[3]).max())
    assert argmax == y0


# ---------------------------------------------------------------- the loop
PLANS = {"skip2": synth.mask_from_layers(4, [2]), "mlp3": np.array([0, 0, 0, 0, 0, 0, 0, 1], np.uint8),
         "exit3": synth.mask_exit(4, 3)}


@pytest.mark.parametrize("plan", sorted(PLANS))
def test_tree_decoding_equals_greedy_ar(plan):
    """Greedy tree decoding emits the full model's greedy tokens (R4), with
    leaves accepted along the way, so the leaf logits and the cache repair
    after a leaf are exercised."""
    m = mdl.Model.synthetic(synth.TINY)
    prompt = synth.prompt_tokens(32, synth.TINY.vocab)
    out, st, _ = tree.tree_generate(m, prompt, 64, PLANS[plan], 4, 0.9, 4, 6)
    ar, _ = ssd.ar_generate(m, prompt, 64)
    assert out == ar
    assert sum(st["leaf_accepted"]) >= 5
    assert all(e <= dp + 1 for dp, e in zip(st["drafted"], st["emitted"]))


def test_tree_decoding_bf16_equals_greedy_ar():
    m = mdl.Model.synthetic(BF16_SMALL)
    prompt = synth.prompt_tokens(16, BF16_SMALL.vocab)
    mask = synth.mask_from_layers(3, [1])
    out, st, _ = tree.tree_generate(m, prompt, 40, mask, 4, 0.95, 3, 4)
    ar, _ = ssd.ar_generate(m, prompt, 40)
    assert out == ar
    assert sum(st["leaf_accepted"]) >= 1


@pytest.mark.parametrize("k_max,budget", [(1, 6), (4, 0)])
def test_no_leaves_is_the_chain_loop(k_max, budget):
    """With one candidate per step (or no room for leaves) the loop is ssd_generate's."""
    m = mdl.Model.synthetic(synth.TINY)
    prompt = synth.prompt_tokens(32, synth.TINY.vocab)
    mask = PLANS["skip2"]
    out, st, _ = tree.tree_generate(m, prompt, 48, mask, 4, 0.9, k_max, budget)
    ref, rst, _ = ssd.ssd_generate(m, prompt, 48, mask, 4)
    assert out == ref
    assert st["emitted"] == rst["emitted"]
    assert not any(st["leaf_accepted"])


# ---------------------------------------------------------------- R5: sampled trees
def test_sampled_tree_without_leaves_is_the_chain_loop():
    """k_max = 1: no leaves, and the sampled tree loop is ssd_generate's at T = 1,
    draw for draw (same tokens, same per-iteration yields)."""
    m = mdl.Model.synthetic(synth.TINY)
    prompt = synth.prompt_tokens(24, synth.TINY.vocab)
    mask = PLANS["skip2"]
    out, st, _ = tree.tree_generate(m, prompt, 40, mask, 4, 0.9, 1, 6, tau=0.002, T=1.0, seed=77)
    ref, rst, _ = ssd.ssd_generate(m, prompt, 40, mask, 4, tau=0.002, T=1.0, seed=77)
    assert out == ref
    assert st["emitted"] == rst["emitted"]


def _first_token_counts(accept_fn, leaf_fn, n, T=1.0, V=8):
    """First emitted token of one depth-1 tree (the draft's draw plus two more
    candidates) over n seeds, and the target law p_1 = softmax(zp[0] / T)."""
    from oracle import philox
    from oracle.numerics import softmax as sm
    rng = np.random.default_rng(0)
    zp = rng.standard_normal((2, V)) * 1.5
    zq = rng.standard_normal((1, V)) * 1.5
    zl = np.zeros((4, V))
    counts = np.zeros(V)
    for seed in range(n):
        y1 = ssd.sample_logits(zq[0], T, seed, 1, 0, philox.PURPOSE_DRAFT)
        leaves = leaf_fn(zq, [y1], T, seed)
        em, _ = accept_fn(zp, zq, zl, [y1], leaves, T, seed, 1)
        counts[em[0]] += 1
    return counts, sm(zp[0] / T)


def _drawn_leaves(zq, drafts, T, seed):
    return tree.tree_leaves_sampled(zq, drafts, T, 1.01, 3, 4, seed, 1)   # rho > 1: k = k_max = 3


def _mutated_accept(old, new):
    """tree.accept_tree_sampled with one planted mistake (source edit, on the CPU)."""
    import inspect
    src = inspect.getsource(tree.accept_tree_sampled)
    assert old in src
    ns = dict(tree.__dict__)
    exec(src.replace(old, new), ns)
    return ns["accept_tree_sampled"]


def test_sampled_tree_first_token_follows_the_target():
    """R5's multi-candidate rule with drawn leaves emits the target law (chi-square,
    6000 seeds); a missing residual update between candidates, a leaf tested
    against p instead of the residual, or top-k leaves instead of drawn ones each
    break it (p < 1e-6)."""
    from scipy import stats
    n = 6000
    c, p = _first_token_counts(tree.accept_tree_sampled, _drawn_leaves, n)
    assert stats.chisquare(c, n * p).pvalue > 1e-4
    no_update = _mutated_accept("cur = (r / tot).astype(np.float32)", "cur = cur")
    c, p = _first_token_counts(no_update, _drawn_leaves, n)
    assert stats.chisquare(c, n * p).pvalue < 1e-6
    against_p = _mutated_accept("lpc = lp[c] if last_r is None else", "lpc = lp[c] if True else")
    c, p = _first_token_counts(against_p, _drawn_leaves, n)
    assert stats.chisquare(c, n * p).pvalue < 1e-6
    topk = lambda zq, drafts, T, seed: [(1, t) for t in tree.topk_lowest(zq[0], 3)[:2]]
    c, p = _first_token_counts(tree.accept_tree_sampled, topk, n)
    assert stats.chisquare(c, n * p).pvalue < 1e-6


def test_sampled_tree_leaves_are_draws_of_q():
    """The extra candidates of a step are independent draws of softmax(z / T)
    (chi-square over seeds), k_j - 1 of them, depth order."""
    from scipy import stats
    from oracle.numerics import softmax as sm
    rng = np.random.default_rng(4)
    V, T = 6, 0.7
    zq = rng.standard_normal((2, V))
    counts = np.zeros(V)
    n = 4000
    for seed in range(n):
        lv = tree.tree_leaves_sampled(zq, [0, 1], T, 1.01, 3, 10, seed, 5)
        assert [j for j, _ in lv] == [1, 1, 2, 2]
        counts[lv[2][1]] += 1
    assert stats.chisquare(counts, n * sm(zq[1] / T)).pvalue > 1e-4
