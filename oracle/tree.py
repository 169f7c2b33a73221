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
  R5  Sampling (temperature T > 0).  The top-k tokens are not draws from q,
      and the p/q rule preserves the target distribution only for drawn
      candidates, so at T > 0: k_j from R1 on softmax(z_j / T); the draft token
      y_j is the chain's draw; the leaves of depth j are k_j - 1 further
      independent draws from q_j (race keys z/T + Gumbel, purpose "leaf",
      counter row (j - 1) + 256 r for the r-th extra draw); the verify is R2's.
      Acceptance at depth j takes the candidates in order c_0 = y_j, then the
      leaves of depth j: with p' = p_j, candidate c_i is accepted when
      u_i q_j(c_i) < p'(c_i) (u_i: purpose "accept", row (j - 1) + 256 i), else
      p' becomes norm(max(0, p' - q_j)) (p' kept when that is all zero).  c_0
      accepted: go on to depth j + 1.  A leaf accepted: emit it and a draw from
      the full model after it (purpose "sample", row (j - 1) + 256 i).  All
      rejected: emit a draw from p' (purpose "sample", row j - 1).  This is the
      multi-candidate form of the speculative-sampling rule (SpecInfer, Miao et
      al. 2024): with candidates drawn independently from q_j the emitted token
      follows p_j.  Without leaves it is the chain rule of ssd.accept_sampled,
      draw for draw.
"""
import numpy as np

from . import model as mdl
from . import philox
from . import ssd
from .numerics import argmax_lowest, softmax

PURPOSE_LEAF = 4
ROW_STRIDE = 256       # counter row of the r-th candidate of draft step j: (j - 1) + 256 r


def topk_lowest(z, k):
    """Indices of the k largest entries of z, largest first, the lower index
    first among equal values."""
    z = np.asarray(z)
    return [int(i) for i in np.argsort(-z, kind="stable")[:k]]


def candidate_count(z, rho, k_max, T=0.0):
    """R1: the least k >= 1 such that the k most probable tokens of softmax(z)
    (softmax(z / T) when T > 0, R5) hold at least rho of the mass, capped at k_max."""
    q = softmax(np.asarray(z, np.float64) / (T if T > 0 else 1.0))
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


def tree_leaves_sampled(zq, drafts, T, rho, k_max, budget, seed, it, log=None):
    """R5: leaves (depth j, token) of a sampled draft, in depth order then draw
    order, at most `budget`: k_j - 1 independent draws from softmax(zq[j-1] / T).
    log: as ssd.pick, each draw logged at row j - 1 (kind "leaf")."""
    leaves = []
    for j in range(1, len(drafts) + 1):
        k = candidate_count(zq[j - 1], rho, k_max, T)
        for r in range(1, k):
            if len(leaves) < budget:
                t = ssd.sample_logits(zq[j - 1], T, seed, it, (j - 1) + ROW_STRIDE * r, PURPOSE_LEAF)
                if log is not None:
                    g = philox.gumbel(seed, it, (j - 1) + ROW_STRIDE * r, PURPOSE_LEAF, zq.shape[-1])
                    keys = (np.asarray(zq[j - 1], np.float64) / T).astype(np.float32) + g
                    log.append(("leaf", j - 1, ssd.top2_gap(keys)))
                leaves.append((j, t))
    return leaves


def accept_tree_sampled(zp, zq, zl, drafts, leaves, T, seed, it, log=None):
    """R5: (emitted tokens, index of the accepted leaf or None).  Decisions on
    float32 quantities, as ssd.accept_sampled; the final draw at a depth uses the
    last nonzero max(0, p' - q) unnormalised (log p when there was none), so that
    a depth without leaves draws exactly as the chain rule.  log: as
    ssd.accept_sampled, every decision at depth j logged at row j - 1."""
    dp = len(drafts)
    for j in range(1, dp + 1):
        lp = ssd.log_softmax(zp[j - 1], T).astype(np.float32)
        lq = ssd.log_softmax(zq[j - 1], T).astype(np.float32)
        q32 = np.exp(lq)
        cur = np.exp(lp)                      # p' (float32 probabilities)
        last_r = None                         # the last nonzero residual, unnormalised
        cands = [(int(drafts[j - 1]), None)] + [(int(c), s) for s, (dj, c) in enumerate(leaves) if dj == j]
        accepted = False
        for i, (c, s) in enumerate(cands):
            u = philox.uniforms(seed, it, (j - 1) + ROW_STRIDE * i, philox.PURPOSE_ACCEPT, 1)[0]
            lpc = lp[c] if last_r is None else (np.log(cur[c]) if cur[c] > 0 else -np.inf)
            if log is not None:
                log.append(("accept", j - 1, abs(float(np.log(u) + lq[c]) - float(lpc))))
            if np.log(u) + lq[c] < lpc:
                if s is None:
                    accepted = True           # the chain goes on
                    break
                bonus = ssd.sample_logits(zl[s], T, seed, it, (j - 1) + ROW_STRIDE * i, philox.PURPOSE_SAMPLE)
                if log is not None:
                    g = philox.gumbel(seed, it, (j - 1) + ROW_STRIDE * i, philox.PURPOSE_SAMPLE, zl.shape[-1])
                    log.append(("sample", j - 1, ssd.top2_gap((np.asarray(zl[s], np.float64) / T).astype(np.float32)
                                                             + g)))
                return [int(t) for t in drafts[: j - 1]] + [c, bonus], s
            r = np.maximum(np.float32(0), cur - q32)
            tot = np.float32(r.sum(dtype=np.float64))
            if tot > 0:
                last_r = r
                cur = (r / tot).astype(np.float32)
        if accepted:
            continue
        g = philox.gumbel(seed, it, j - 1, philox.PURPOSE_SAMPLE, cur.shape[0])
        if last_r is None:
            keys = lp + g
        else:
            with np.errstate(divide="ignore"):
                keys = np.log(last_r) + g
        if log is not None:
            log.append(("sample", j - 1, ssd.top2_gap(keys)))
        return [int(t) for t in drafts[: j - 1]] + [ssd.race_sample(keys)], None
    return [int(t) for t in drafts] + [ssd.sample_logits(zp[dp], T, seed, it, dp, philox.PURPOSE_SAMPLE, log)], None


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
                  on_iteration=None, T=0.0, seed=3):
    """Self-speculative decoding with confidence-sized draft trees: draft
    (ssd.draft), leaves (R1-R3, or R5 at T > 0), one tree verify, tree
    acceptance (R4, or R5).  The cache ends each iteration holding the full
    model's keys and values of every committed token: when a leaf is accepted
    its path is run through the full model into the cache.  Output truncated
    to n_gen tokens."""
    P = len(prompt)
    b = mdl.first_skipped_layer(mask, model.L)
    kv = mdl.KVCache(model.shape, capacity or (P + n_gen + d + 2))
    log0 = []
    out = [ssd.pick(ssd.prefill(model, kv, prompt), T, seed, 0, 0, philox.PURPOSE_SAMPLE, log0)]
    stats = {"drafted": [], "leaves": [], "emitted": [], "leaf_accepted": [], "decisions": [log0]}
    it = 1
    while len(out) < n_gen:
        n = P + len(out)
        y0 = out[-1]
        log = []
        drafts, zq, hb = ssd.draft(model, kv, y0, n, mask, d, tau, T, seed, it, log)
        if T == 0:
            leaves = tree_leaves(zq, drafts, rho, k_max, budget)
        else:
            leaves = tree_leaves_sampled(zq, drafts, T, rho, k_max, budget, seed, it, log)
        zp, zl = verify_tree(model, kv, y0, drafts, leaves, n, b, hb if reuse else None)
        if T == 0:
            emitted, s = accept_tree_greedy(zp, zl, drafts, leaves)
        else:
            emitted, s = accept_tree_sampled(zp, zq, zl, drafts, leaves, T, seed, it, log)
        stats["decisions"].append(log)
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
