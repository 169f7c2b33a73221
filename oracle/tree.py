"""Dynamic verification with confidence-sized draft trees (oracle; test
infrastructure only, like the rest of this package).

Source: SWIFT digest §4.2 "Confidence-aware inference acceleration" — the
draft's confidence decides both when drafting stops and how many candidates
are handed to the parallel verification; §3.2.1 and Figure 2 credit top-k
drafts with higher acceptance; §D.1 (Table 8) reports that dropping dynamic
verification lowers the mean accepted length.  The digest gives no formula
for the candidate count; the readings taken here (also listed in the design
notes):

  R1  Candidate count.  At draft step j, with q_j = softmax(z_j) (temperature
      1, the same distribution whose maximum is the confidence of the stop
      rule), the candidates are the k_j most probable tokens (lowest index
      first among equal logits), k_j = the least k >= 1 whose top-k mass
      reaches rho, at most k_max: a confident step hands over one candidate,
      an unsure one several.
  R2  Tree shape.  Only the top candidate y_j is drafted further; the others
      are leaves of depth j.  A leaf of depth j sits at y_j's position and
      attends to the committed prefix, y_0..y_{j-1} and itself.
  R3  Budget.  The verify pass holds at most `budget` leaf rows next to the
      chain's d'+1 rows; leaves are taken in depth order, then rank order.
  R4  Acceptance (greedy).  For j = 1..d': if the target's argmax after
      y_{j-1} is y_j, continue; otherwise, if it is a leaf of depth j, emit
      that leaf and the target's argmax after it, and stop; otherwise emit
      the target's argmax, and stop.  After d' accepted drafts the target's
      argmax after y_d' is the bonus.  Every emitted token is the full
      model's greedy choice, so the output equals greedy AR decoding.
      Only temperature 0 is covered.
"""
import numpy as np

from . import model as mdl
from . import ssd
from .numerics import argmax_lowest, softmax


def topk_lowest(z, k):
    """Indices of the k largest entries of z, largest first, the lower index
    first among equal values."""
    z = np.asarray(z)
    return [int(i) for i in np.argsort(-z, kind="stable")[:k]]


def candidate_count(z, rho, k_max):
    """R1: the least k >= 1 such that the k most probable tokens of softmax(z)
    hold at least rho of the mass, capped at k_max."""
    q = softmax(np.asarray(z, np.float64))
    top = topk_lowest(z, k_max)
    cum = np.cumsum(q[top])
    hit = np.nonzero(cum >= rho)[0]
    return int(hit[0]) + 1 if hit.size else k_max


def tree_leaves(zq, drafts, rho, k_max, budget):
    """R1-R3: leaves (depth j, token) of the draft steps' logits zq [d', V] in
    depth order, then rank order, at most `budget` of them.  drafts[j-1] must
    be the argmax of zq[j-1] (greedy drafting)."""
    leaves = []
    for j in range(1, len(drafts) + 1):
        top = topk_lowest(zq[j - 1], k_max)
        assert top[0] == int(drafts[j - 1]), "greedy draft token is the top candidate"
        k = candidate_count(zq[j - 1], rho, k_max)
        for t in top[1:k]:
            if len(leaves) < budget:
                leaves.append((j, t))
    return leaves


def verify_tree(model, kv, y0, drafts, leaves, n, b, hb=None):
    """Tree verify (R2): the chain rows as ssd.verify (rows y0..yd' at
    positions n-1..n-1+d', overwriting the cache there), and for each leaf
    (j, c) the full model's logits after the path y0, y1..y_{j-1}, c at
    positions n-1..n-1+j, computed on a copy of the cache (a leaf leaves the
    cache as it was).  Returns (chain logits [d'+1, V], leaf logits [S, V])."""
    zl = []
    for j, c in leaves:
        path = [int(y0)] + [int(t) for t in drafts[: j - 1]] + [int(c)]
        kvc = kv.copy()
        zl.append(mdl.forward(model, path, list(range(n - 1, n + j)), kvc)[-1])
    zp = ssd.verify(model, kv, y0, drafts, n, b, hb)
    V = model.shape.vocab
    return zp, (np.array(zl) if zl else np.zeros((0, V)))


def accept_tree_greedy(zp, zl, drafts, leaves):
    """R4: (emitted tokens, index of the accepted leaf or None)."""
    dp = len(drafts)
    for j in range(1, dp + 1):
        a = argmax_lowest(zp[j - 1])
        if a == int(drafts[j - 1]):
            continue
        for s, (dj, c) in enumerate(leaves):
            if dj == j and int(c) == a:
                return [int(t) for t in drafts[: j - 1]] + [a, argmax_lowest(zl[s])], s
        return [int(t) for t in drafts[: j - 1]] + [a], None
    return [int(t) for t in drafts] + [argmax_lowest(zp[dp])], None


def tree_generate(model, prompt, n_gen, mask, d, rho, k_max, budget, tau=0.0, reuse=True, capacity=None,
                  on_iteration=None):
    """Greedy self-speculative decoding with confidence-sized draft trees:
    draft (ssd.draft, T = 0), leaves (R1-R3), one tree verify, tree acceptance
    (R4).  The cache ends each iteration holding the full model's keys and
    values of every committed token: when a leaf is accepted its path is run
    through the full model into the cache.  Output truncated to n_gen tokens."""
    P = len(prompt)
    b = mdl.first_skipped_layer(mask, model.L)
    kv = mdl.KVCache(model.shape, capacity or (P + n_gen + d + 2))
    out = [argmax_lowest(ssd.prefill(model, kv, prompt))]
    stats = {"drafted": [], "leaves": [], "emitted": [], "leaf_accepted": []}
    it = 1
    while len(out) < n_gen:
        n = P + len(out)
        y0 = out[-1]
        drafts, zq, hb = ssd.draft(model, kv, y0, n, mask, d, tau, 0.0, 0, it)
        leaves = tree_leaves(zq, drafts, rho, k_max, budget)
        zp, zl = verify_tree(model, kv, y0, drafts, leaves, n, b, hb if reuse else None)
        emitted, s = accept_tree_greedy(zp, zl, drafts, leaves)
        if s is not None:
            j, c = leaves[s]
            path = [int(y0)] + [int(t) for t in drafts[: j - 1]] + [int(c)]
            mdl.forward(model, path, list(range(n - 1, n + j)), kv)
        stats["drafted"].append(len(drafts))
        stats["leaves"].append(len(leaves))
        stats["emitted"].append(len(emitted))
        stats["leaf_accepted"].append(s is not None)
        if on_iteration is not None:
            on_iteration(it, n, drafts, zq, leaves, zp, zl, emitted, s)
        out.extend(emitted)
        it += 1
    return out[:n_gen], stats, kv
