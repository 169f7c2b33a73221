"""Draft trees on the GPU (through the C ABI) against the oracle's reading of
SWIFT's dynamic verification (oracle/tree.py)."""
import numpy as np
import pytest
import torch

import synth
from self_speculative_layer_amd import binding as B
from oracle import model as omodel
from oracle import ssd as ossd
from oracle import tree as otree
from oracle.numerics import softmax

from gpu_util import BF16_HD64, BF16_HD128, F32_GQA, check_greedy_tokens, check_greedy_with_resync, \
    check_sampled_with_resync, dev, gpu_model, \
    logit_tol, oracle_ar_with_logits

pytestmark = pytest.mark.gpu

# plans under which the oracle accepts leaves on these shapes (MLP of the last layer skipped)
TREE_PLANS = {"bf16-hd64-gqa": dict(mask=np.array([0, 0, 0, 0, 0, 0, 0, 1], np.uint8), d=4, max_leaves=3),
              "bf16-hd128": dict(mask=np.array([0, 0, 0, 0, 0, 1], np.uint8), d=5, max_leaves=6)}
RHO, K_MAX = 0.9, 4


@pytest.fixture(scope="module", params=[BF16_HD64, BF16_HD128], ids=lambda s: s.name)
def pair(request):
    shape = request.param
    print("[gpu] building %s" % shape.name, flush=True)
    g = gpu_model(shape)
    o = omodel.Model.synthetic(shape)
    yield shape, g, o
    g.close()


# ---------------------------------------------------------------- candidates
def _candidate_rows(V, d, seed):
    """Seeded draft-logit rows of varied confidence, one with many equal values."""
    rng = np.random.default_rng(seed)
    scales = np.linspace(0.5, 9.0, d)
    z = (rng.standard_normal((d, V)) * scales[:, None]).astype(np.float32)
    z[1] = rng.integers(0, 3, V).astype(np.float32) * 4.0          # ties: lowest index first
    z[2, int(rng.integers(V))] += 40.0                               # a confident row
    return z


def _boundary_gap(z, rho, k_max):
    """Smallest |top-k mass - rho| over the rows and k <= k_max (float64)."""
    gap = np.inf
    for row in z:
        q = softmax(np.asarray(row, np.float64))
        cum = np.cumsum(q[otree.topk_lowest(row, k_max)])
        gap = min(gap, float(np.min(np.abs(cum - rho))))
    return gap


@pytest.mark.parametrize("V,k_max,rho,max_leaves", [(1000, 4, 0.5, 15), (2003, 8, 0.3, 5), (32000, 8, 0.02, 12),
                                                    (1000, 1, 0.9, 15)])
def test_candidates_match_oracle(V, k_max, rho, max_leaves):
    shape = synth.ModelShape("vocab-%d" % V, 1, 64, 1, 1, 64, 64, V, "bf16")
    g = gpu_model(shape)
    d, dp = 8, 6
    z = _candidate_rows(V, d, seed=V + k_max)
    assert _boundary_gap(z[:dp], rho, k_max) > 1e-5           # no count decided within rounding of rho
    drafts = [int(np.argmax(r)) for r in z[:dp]]
    ref = otree.tree_leaves(z[:dp], drafts, rho, k_max, max_leaves)
    seq = B.Sequence(g, max_ctx=128, max_rows=16, max_draft=d)
    B.ssd_tree_candidates(seq.handle, dev(z.reshape(-1), torch.float32), dev([dp]), d, rho, k_max, max_leaves,
                          seq.leaf_tokens, seq.leaf_depth, seq.n_leaves)
    torch.cuda.synchronize()
    nl = int(seq.n_leaves.item())
    got = list(zip(seq.leaf_depth[:nl].cpu().tolist(), seq.leaf_tokens[:nl].cpu().tolist()))
    print("V %d k_max %d rho %.2f: %d leaves" % (V, k_max, rho, nl))
    assert got == ref
    seq.close()
    g.close()


# ---------------------------------------------------------------- verify
def test_tree_verify_matches_oracle(pair):
    """Chain rows bitwise equal to ssd_verify's and to the no-reuse pass; every row
    against the oracle's tree verify on the oracle's own draft and the same leaves."""
    shape, g, o = pair
    plan = TREE_PLANS[shape.name]
    mask, d, ml = plan["mask"], plan["d"], plan["max_leaves"]
    V = shape.vocab
    P = 24
    prompt = synth.prompt_tokens(P, V)
    # oracle: prefill, greedy draft, tree verify
    okv = omodel.KVCache(shape, P + d + 4)
    y0 = int(np.argmax(ossd.prefill(o, okv, prompt)))
    odr, _, ohb = ossd.draft(o, okv, y0, P + 1, mask, d, 0.0, 0.0, 0, 1)
    rng = np.random.default_rng(11)
    dp = len(odr)
    leaves = [(int(rng.integers(1, dp + 1)), int(rng.integers(V))) for _ in range(ml - 1)]
    leaves.append((min(2, dp), int(odr[min(2, dp) - 1])))          # a leaf repeating the chain token
    b = omodel.first_skipped_layer(mask, shape.n_layers)
    zp, zl = otree.verify_tree(o, okv, y0, odr, leaves, P + 1, b, ohb)
    outs = {}
    for reuse in (True, False):
        seq = B.Sequence(g, max_ctx=P + 4 * d + 8, max_rows=16, max_draft=d)
        B.ssd_prefill(seq.handle, dev(prompt))
        B.ssd_draft(seq.handle, mask, None, d, 0.0, 0.0, 0, seq.draft_tokens, seq.draft_logits, seq.n_drafted)
        torch.cuda.synchronize()
        gdp = int(seq.n_drafted.item())
        gdr = seq.draft_tokens[:gdp].cpu().tolist()
        assert gdr == [int(t) for t in odr], "draft differs from the oracle's (near-tie?)"
        lt, ld = dev([t for _, t in leaves] + [0] * (16 - ml)), dev([j for j, _ in leaves] + [0] * (16 - ml))
        B.ssd_verify(seq.handle, mask, None, d, seq.draft_tokens, seq.n_drafted, reuse, seq.verify_logits)
        torch.cuda.synchronize()
        chain = seq.verify_logits[: (dp + 1) * V].clone()
        B.ssd_verify_tree(seq.handle, mask, None, d, seq.draft_tokens, seq.n_drafted, lt, ld, dev([ml]), ml, reuse,
                          seq.tree_logits)
        torch.cuda.synchronize()
        tz = seq.tree_logits[: (dp + 1 + ml) * V].clone()
        assert torch.equal(tz[: (dp + 1) * V], chain), "tree chain rows differ from ssd_verify's"
        outs[reuse] = tz
        seq.close()
    assert torch.equal(outs[True], outs[False]), "reuse changed the tree verify"
    tz = outs[True].view(dp + 1 + ml, V).cpu().numpy()
    dz_chain = np.abs(tz[: dp + 1] - zp).max()
    dz_leaf = np.abs(tz[dp + 1:] - zl).max()
    print("max |dz| chain %.3g leaves %.3g" % (dz_chain, dz_leaf))
    assert dz_chain < logit_tol(shape) and dz_leaf < logit_tol(shape)
    j = min(2, dp)
    assert np.abs(tz[dp + ml] - tz[j]).max() < logit_tol(shape)     # the repeated chain token's leaf row


# ---------------------------------------------------------------- the loop
def test_tree_generation_matches_oracle(pair):
    """Greedy tree decoding: tokens equal the oracle's greedy AR tokens (margin
    rule) and the per-iteration (d', emitted) record equals the oracle's tree loop,
    in which leaves are accepted (so leaf rows, acceptance and the cache repair
    after a leaf all take part)."""
    shape, g, o = pair
    plan = TREE_PLANS[shape.name]
    mask, d, ml = plan["mask"], plan["d"], plan["max_leaves"]
    P, n_gen = 32, 48
    prompt = synth.prompt_tokens(P, shape.vocab)
    ref, ref_z = oracle_ar_with_logits(o, prompt, n_gen)
    otoks, ost, _ = otree.tree_generate(o, prompt, n_gen, mask, d, RHO, K_MAX, ml)
    assert otoks == ref and sum(ost["leaf_accepted"]) >= 1
    seq = B.Sequence(g, max_ctx=P + n_gen + 2 * d + 8, max_rows=16, max_draft=d)
    out, stats = seq.generate_tree(dev(prompt), n_gen, skip_mask=mask, d=d, rho=RHO, k_max=K_MAX, max_leaves=ml)
    print("iterations %d (oracle %d), leaf acceptances in the oracle %d" %
          (len(stats), len(ost["emitted"]), sum(ost["leaf_accepted"])))
    first = check_greedy_tokens(out, ref, ref_z)
    if first is None:
        assert [e for _, e in stats] == ost["emitted"] and [dp for dp, _ in stats] == ost["drafted"]
    seq.close()

    def gen(prefix, n):
        s2 = B.Sequence(g, max_ctx=len(prefix) + n + 2 * d + 8, max_rows=16, max_draft=d)
        toks, _ = s2.generate_tree(dev(prefix), n, skip_mask=mask, d=d, rho=RHO, k_max=K_MAX, max_leaves=ml)
        s2.close()
        return toks

    print("near-tie re-synchronisations: %d" % check_greedy_with_resync(gen, prompt, ref, ref_z))


def test_tree_arguments_rejected():
    g = gpu_model(F32_GQA)
    seq = B.Sequence(g, max_ctx=64, max_rows=16, max_draft=4)
    with pytest.raises(B.SSDError) as e:
        B.ssd_verify_tree(seq.handle, None, 1, 4, seq.draft_tokens, seq.n_drafted, seq.leaf_tokens, seq.leaf_depth,
                          seq.n_leaves, 2, 1, seq.tree_logits)
    assert e.value.code == B.SSD_ERR_UNSUPPORTED
    seq.close()
    g.close()
    g = gpu_model(BF16_HD64)
    seq = B.Sequence(g, max_ctx=64, max_rows=16, max_draft=8)
    with pytest.raises(B.SSDError) as e:
        B.ssd_verify_tree(seq.handle, None, 1, 8, seq.draft_tokens, seq.n_drafted, seq.leaf_tokens, seq.leaf_depth,
                          seq.n_leaves, 8, 1, seq.tree_logits)
    assert e.value.code == B.SSD_ERR_ARG
    with pytest.raises(B.SSDError) as e:
        B.ssd_tree_candidates(seq.handle, seq.draft_logits, seq.n_drafted, 4, 0.9, 9, 3, seq.leaf_tokens,
                              seq.leaf_depth, seq.n_leaves)
    assert e.value.code == B.SSD_ERR_ARG
    # a leaf depth outside 1..d' is flagged on the device (and clamped, so no access leaves the buffers)
    prompt = synth.prompt_tokens(8, BF16_HD64.vocab)
    B.ssd_prefill(seq.handle, dev(prompt))
    B.ssd_draft(seq.handle, None, 2, 3, 0.0, 0.0, 0, seq.draft_tokens, seq.draft_logits, seq.n_drafted)
    B.ssd_verify_tree(seq.handle, None, 2, 3, seq.draft_tokens, seq.n_drafted, dev([5] * 16), dev([7] * 16), dev([2]),
                      2, 1, seq.tree_logits)
    with pytest.raises(B.SSDError) as e:
        B.ssd_read_state(seq.handle)
    assert e.value.code == B.SSD_ERR_ARG
    seq.close()
    g.close()


@pytest.mark.parametrize("page_size", [16, 32])
def test_paged_layouts_give_identical_results(page_size):
    """Row a5's paged cache: SSD and tree decoding with small pages scattered by a
    permuted page table give the same tokens, and the same verify logits bit for
    bit, as the contiguous 64-key pages (keys are addressed per position; the
    attention's 64-key splits do not depend on the page size).  The tree run
    accepts leaves, so the repair of an accepted leaf's keys and values goes
    through the scattered pages too."""
    shape = BF16_HD64
    plan = TREE_PLANS[shape.name]
    mask, d, ml = plan["mask"], plan["d"], plan["max_leaves"]
    g = gpu_model(shape)
    P, n_gen = 70, 48
    prompt = synth.prompt_tokens(P, shape.vocab)
    max_ctx = P + n_gen + 2 * d + 16
    n_lp = (max_ctx + page_size - 1) // page_size
    perm = [(7 * i + 3) % n_lp for i in range(n_lp)]
    assert sorted(perm) == list(range(n_lp))
    runs = []
    for ps, pt in ((64, None), (page_size, perm)):
        seq = B.Sequence(g, max_ctx=max_ctx, max_rows=16, max_draft=d, page_size=ps, page_table=pt)
        out, stats = seq.generate_ssd(dev(prompt), n_gen, skip_mask=mask, d=d)
        vz = seq.verify_logits.clone()
        seq.close()
        seq = B.Sequence(g, max_ctx=max_ctx, max_rows=16, max_draft=d, page_size=ps, page_table=pt)
        tout, tstats = seq.generate_tree(dev(prompt), n_gen, skip_mask=mask, d=d, rho=RHO, k_max=K_MAX, max_leaves=ml)
        tz = seq.tree_logits.clone()
        seq.close()
        runs.append(([int(x) for x in out], stats, vz, [int(x) for x in tout], tstats, tz))
    a, b = runs
    assert a[0] == b[0] and a[1] == b[1] and torch.equal(a[2], b[2])
    assert a[3] == b[3] and a[4] == b[4] and torch.equal(a[5], b[5])
    g.close()


# ---------------------------------------------------------------- sampled trees (T > 0)
SAMPLED = dict(mask=synth.mask_exit(4, 2), d=4, max_leaves=6, T=0.5, seed=12345)   # z / 0.5 is exact on both sides


def test_sampled_candidates_match_oracle():
    """At T > 0 the leaves are draws of softmax(z / T) with the leaf purpose and the
    sequence's iteration (1 after a prefill): the same tokens as the oracle's."""
    from oracle import philox as ophilox
    V, T, seed, k_max, rho, ml = 1000, 0.5, 99, 4, 0.6, 15
    shape = synth.ModelShape("vocab-%d" % V, 1, 64, 1, 1, 64, 64, V, "bf16")
    g = gpu_model(shape)
    d, dp = 6, 5
    z = _candidate_rows(V, d, seed=7) * 0.25
    assert _boundary_gap(z[:dp] / T, rho, k_max) > 1e-5
    ref = otree.tree_leaves_sampled(z[:dp], [0] * dp, T, rho, k_max, ml, seed, 1)
    for j, _ in ref:                         # no race decided within rounding: the two best keys apart
        for r in range(1, k_max):
            keys = np.sort((np.asarray(z[j - 1], np.float64) / T).astype(np.float32) +
                           ophilox.gumbel(seed, 1, (j - 1) + 256 * r, 4, V))
            assert keys[-1] - keys[-2] > 1e-5
    seq = B.Sequence(g, max_ctx=128, max_rows=16, max_draft=d)
    B.ssd_prefill(seq.handle, dev(synth.prompt_tokens(8, V)))
    B.ssd_tree_candidates(seq.handle, dev(z.reshape(-1), torch.float32), dev([dp]), d, rho, k_max, ml,
                          seq.leaf_tokens, seq.leaf_depth, seq.n_leaves, T, seed)
    torch.cuda.synchronize()
    nl = int(seq.n_leaves.item())
    got = list(zip(seq.leaf_depth[:nl].cpu().tolist(), seq.leaf_tokens[:nl].cpu().tolist()))
    print("sampled leaves: %s" % got)
    assert got == ref and nl > 0
    seq.close()
    g.close()


def test_sampled_tree_without_leaves_is_the_chain():
    """k_max = 1: no leaves, and sampled tree decoding emits ssd_accept's tokens
    draw for draw (same tokens, same per-iteration record)."""
    shape = BF16_HD64
    g = gpu_model(shape)
    P, n_gen = 24, 40
    prompt = synth.prompt_tokens(P, shape.vocab)
    kw = dict(skip_mask=SAMPLED["mask"], d=SAMPLED["d"], temperature=SAMPLED["T"], seed=SAMPLED["seed"])
    seq = B.Sequence(g, max_ctx=P + n_gen + 32, max_rows=16, max_draft=8)
    a, sa = seq.generate_tree(dev(prompt), n_gen, k_max=1, max_leaves=SAMPLED["max_leaves"], **kw)
    seq.close()
    seq = B.Sequence(g, max_ctx=P + n_gen + 32, max_rows=16, max_draft=8)
    b, sb = seq.generate_ssd(dev(prompt), n_gen, **kw)
    seq.close()
    assert [int(x) for x in a] == [int(x) for x in b] and sa == sb
    g.close()


def test_sampled_tree_generation_matches_oracle():
    """T = 0.5 with drawn leaves: the same Philox draws on both sides, so the tokens
    agree except where a decision of the oracle (draft and leaf draws, accept
    decisions of the chain and the leaves, final draws) lies within 1e-2 of
    flipping; after such a token both restart from the oracle's prefix.  The
    oracle's run accepts leaves."""
    shape = BF16_HD64
    g = gpu_model(shape)
    o = omodel.Model.synthetic(shape)
    P, n_gen = 24, 40
    prompt = synth.prompt_tokens(P, shape.vocab)
    c = SAMPLED
    _, ost, _ = otree.tree_generate(o, prompt, n_gen, c["mask"], c["d"], RHO, K_MAX, c["max_leaves"], T=c["T"],
                                    seed=c["seed"])
    assert sum(ost["leaf_accepted"]) >= 2
    seq = B.Sequence(g, max_ctx=P + n_gen + 32, max_rows=16, max_draft=8)

    def gpu_run(prefix, n):
        return seq.generate_tree(dev(prefix), n, skip_mask=c["mask"], d=c["d"], rho=RHO, k_max=K_MAX,
                                 max_leaves=c["max_leaves"], temperature=c["T"], seed=c["seed"])[0]

    def oracle_run(prefix, n):
        toks, st, _ = otree.tree_generate(o, prefix, n, c["mask"], c["d"], RHO, K_MAX, c["max_leaves"], T=c["T"],
                                          seed=c["seed"])
        return toks, st

    events = check_sampled_with_resync(gpu_run, oracle_run, prompt, n_gen)
    print("sampled tree: %d re-synchronisations over %d tokens; oracle leaf acceptances %d" %
          (events, n_gen, sum(ost["leaf_accepted"])))
    seq.close()
    g.close()


@pytest.mark.parametrize("plan", ["empty", "skip-attention0-layer3"])
def test_tree_decoding_edge_plans(plan):
    """Reuse-boundary edge cases of the tree verify: the empty plan (b = L: y_d' and
    the leaves run every layer in the prefix block, no suffix) and a plan whose
    first sub-layer is skipped (b = 0: no prefix block; layer 3 is skipped too).
    With the empty plan
    every draft is accepted and the tokens are the GPU's AR tokens exactly; with
    the other plan the oracle's tree decoding accepts leaves (so the leaf keys
    and values beside the cache and the accepted leaf's repair are exercised) and
    the tokens are the oracle's greedy ones (margin rule with re-synchronisation)."""
    shape = BF16_HD64
    g = gpu_model(shape)
    P, n_gen, d = 24, 40, 4
    prompt = synth.prompt_tokens(P, shape.vocab)
    mask = np.zeros(2 * shape.n_layers, np.uint8)
    if plan != "empty":
        mask[[0, 6, 7]] = 1
    seq = B.Sequence(g, max_ctx=P + n_gen + 2 * d + 8, max_rows=16, max_draft=d)

    def gen(prefix, n):
        return seq.generate_tree(dev(prefix), n, skip_mask=mask, d=d, rho=0.99, k_max=4, max_leaves=3)

    if plan == "empty":
        out, stats = gen(prompt, n_gen)
        ar_seq = B.Sequence(g, max_ctx=P + n_gen + 8, max_rows=16, max_draft=2)
        ar = ar_seq.generate_ar(dev(prompt), n_gen)
        ar_seq.close()
        assert all(e == dp + 1 for dp, e in stats)
        assert [int(x) for x in out] == [int(x) for x in ar]
    else:
        o = omodel.Model.synthetic(shape)
        ref, ref_z = oracle_ar_with_logits(o, prompt, n_gen)
        otoks, ost, _ = otree.tree_generate(o, prompt, n_gen, mask, d, 0.99, 4, 3)
        assert otoks == ref and sum(ost["leaf_accepted"]) >= 1
        events = check_greedy_with_resync(lambda prefix, n: gen(prefix, n)[0], prompt, ref, ref_z)
        print("edge plan %s: %d re-synchronisations, oracle leaf acceptances %d" %
              (plan, events, sum(ost["leaf_accepted"])))
    seq.close()
    g.close()
