"""GPU path (through the C ABI) against the CPU oracle on the same seeded inputs."""
import math

import numpy as np
import pytest
import torch

import synth
from self_speculative_layer_amd import binding as B
from oracle import model as omodel
from oracle import philox as ophilox
from oracle import ssd as ossd

from synth import device as sdev
from gpu_util import (BF16_HD64, BF16_HD128, F32_GQA, check_greedy_tokens, check_greedy_with_resync,
                      check_sampled_with_resync, check_scores, dev, gpu_model,
                      logit_tol, oracle_ar_with_logits)

pytestmark = pytest.mark.gpu

SHAPES = [synth.TINY, F32_GQA, BF16_HD64, BF16_HD128]


@pytest.fixture(scope="module", params=SHAPES, ids=lambda s: s.name)
def pair(request):
    shape = request.param
    print("[gpu] building %s" % shape.name, flush=True)
    g = gpu_model(shape)
    o = omodel.Model.synthetic(shape)
    yield shape, g, o
    g.close()


def _logical(t, N, K, shape):
    """A device weight as its [N, K] row-major float matrix (bf16 weights are packed)."""
    if shape.dtype == "bf16":
        t = sdev.unpack_bf16(t, N, K)
    return t.float().cpu().numpy()


def test_device_weights_equal_host_weights(pair):
    shape, g, o = pair
    t = g.tensors
    emb = t["embed"].float().cpu().numpy().astype(np.float64)
    assert np.array_equal(emb, o.embed)
    D, F = shape.d_model, shape.ffn_dim
    wqkv = _logical(t["layers"][1]["w_qkv"], shape.qkv_dim, D, shape)
    assert np.array_equal(wqkv[:shape.q_dim], o.layers[1].wq)
    assert np.array_equal(wqkv[shape.q_dim: shape.q_dim + shape.kv_dim], o.layers[1].wk)
    assert np.array_equal(wqkv[shape.q_dim + shape.kv_dim:], o.layers[1].wv)
    wgu = _logical(t["layers"][0]["w_gate_up"], 2 * F, D, shape)
    assert np.array_equal(wgu[:F], o.layers[0].wgate)
    assert np.array_equal(wgu[F:], o.layers[0].wup)
    assert np.array_equal(_logical(t["layers"][0]["w_o"], D, shape.q_dim, shape), o.layers[0].wo)
    assert np.array_equal(_logical(t["layers"][0]["w_down"], D, F, shape), o.layers[0].wdown)
    assert np.array_equal(_logical(t["lm_head"], shape.vocab, D, shape), o.lm_head)
    for l in range(shape.n_layers):
        assert np.array_equal(t["layers"][l]["attn_norm"].cpu().numpy().astype(np.float64), o.layers[l].attn_norm)
        assert np.array_equal(t["layers"][l]["mlp_norm"].cpu().numpy().astype(np.float64), o.layers[l].mlp_norm)
    assert np.array_equal(t["final_norm"].cpu().numpy().astype(np.float64), o.final_norm)
    assert not np.array_equal(o.layers[0].attn_norm, o.layers[0].mlp_norm)


def test_prefill_logits(pair):
    shape, g, o = pair
    P = 300 if shape.dtype == "bf16" else 40          # bf16: five 64-key attention splits, ragged last
    prompt = synth.prompt_tokens(P, shape.vocab)
    # a non-identity page table: logical page i in physical page (3 i + 1) mod n
    n_lp = (P + 64 + 63) // 64
    pt = [(3 * i + 1) % (n_lp + 1) for i in range(n_lp)]
    seq = B.Sequence(g, max_ctx=n_lp * 64, max_rows=64, max_draft=4, page_table=pt)
    lg = torch.zeros(shape.vocab, dtype=torch.float32, device="cuda")
    B.ssd_prefill(seq.handle, dev(prompt), 0.0, 0, lg)
    st = B.ssd_read_state(seq.handle)
    assert st.kvlen == P and st.n_out == 1 and st.iteration == 1
    z = ossd.prefill(o, omodel.KVCache(shape, P + 1), prompt)
    err = np.abs(lg.cpu().numpy() - z).max()
    print("prefill max |dz| = %.3g" % err)
    assert err < logit_tol(shape)
    seq.close()


PLANS = {
    "tiny-f32": dict(skip_mask=synth.mask_from_layers(4, [2]), d=4),
    "f32-gqa": dict(exit_layer=1, d=3),
    "bf16-hd64-gqa": dict(skip_mask=synth.mask_from_layers(4, [1, 3]), d=5),
    "bf16-hd128": dict(exit_layer=1, d=6),
}


def _mask_of(shape, plan):
    if plan.get("skip_mask") is not None:
        return plan["skip_mask"]
    return synth.mask_exit(shape.n_layers, plan["exit_layer"])


def test_greedy_ssd_matches_oracle_and_ar(pair):
    """GPU SSD tokens == oracle AR tokens (margin rule) and == GPU AR tokens."""
    shape, g, o = pair
    plan = PLANS[shape.name]
    P, n_gen = 32, 48
    prompt = synth.prompt_tokens(P, shape.vocab)
    ref, ref_z = oracle_ar_with_logits(o, prompt, n_gen)
    seq = B.Sequence(g, max_ctx=P + n_gen + 2 * plan["d"] + 8, max_rows=64, max_draft=8)
    out, stats = seq.generate_ssd(dev(prompt), n_gen, skip_mask=plan.get("skip_mask"),
                                  exit_layer=plan.get("exit_layer"), d=plan["d"])
    print("iterations %d, mean emitted %.2f" % (len(stats), np.mean([e for _, e in stats])))
    assert all(1 <= e <= dp + 1 for dp, e in stats)
    ar = seq.generate_ar(dev(prompt), n_gen)
    assert [int(x) for x in ar] == [int(x) for x in out]
    seq.close()

    def gen(prefix, n):
        s2 = B.Sequence(g, max_ctx=len(prefix) + n + 2 * plan["d"] + 8, max_rows=64, max_draft=8)
        toks, _ = s2.generate_ssd(dev(prefix), n, skip_mask=plan.get("skip_mask"), exit_layer=plan.get("exit_layer"),
                                  d=plan["d"])
        s2.close()
        return toks

    events = check_greedy_with_resync(gen, prompt, ref, ref_z)
    print("near-tie re-synchronisations: %d" % events)


def test_verify_logits_match_oracle_per_iteration(pair):
    """Each iteration's verify logits (rows 0..d') against the oracle's verify."""
    shape, g, o = pair
    plan = PLANS[shape.name]
    mask = _mask_of(shape, plan)
    d = plan["d"]
    P, n_gen = 24, 30
    prompt = synth.prompt_tokens(P, shape.vocab)
    records = []
    ossd.ssd_generate(o, prompt, n_gen, mask, d,
                      on_iteration=lambda it, n, dr, zq, zp, em, kv: records.append((list(dr), zq, zp, em)))
    seq = B.Sequence(g, max_ctx=P + n_gen + 2 * d + 8, max_rows=64, max_draft=8)
    B.ssd_prefill(seq.handle, dev(prompt))
    V = shape.vocab
    worst = 0.0
    compared = 0
    for dr, zq, zp, em in records:
        seq.ssd_iteration(plan.get("skip_mask"), plan.get("exit_layer"), d)
        st = B.ssd_read_state(seq.handle)
        dp = st.last_n_drafted
        gd = seq.draft_tokens[:dp].cpu().numpy().tolist()
        if gd != dr:
            break          # a near-tie changed the path; later states are not comparable
        gz = seq.verify_logits[: (dp + 1) * V].view(dp + 1, V).cpu().numpy()
        gq = seq.draft_logits[: dp * V].view(dp, V).cpu().numpy()
        worst = max(worst, np.abs(gz - zp).max(), np.abs(gq - zq).max())
        compared += 1
        ge = seq.out_tokens[: st.last_n_emitted].cpu().numpy().tolist()
        if ge != em:
            break
    print("worst |dz| over %d of %d iterations %.3g" % (compared, len(records), worst))
    assert compared >= min(3, len(records))
    assert worst < logit_tol(shape)
    seq.close()


def test_reuse_equals_no_reuse(pair):
    """verify with the draft's saved state == verify recomputing every row, bitwise."""
    shape, g, o = pair
    plan = PLANS[shape.name]
    d = plan["d"]
    P = 20
    prompt = synth.prompt_tokens(P, shape.vocab)
    outs = []
    for reuse in (True, False):
        seq = B.Sequence(g, max_ctx=P + 4 * d + 8, max_rows=64, max_draft=8)
        B.ssd_prefill(seq.handle, dev(prompt))
        B.ssd_draft(seq.handle, plan.get("skip_mask"), plan.get("exit_layer"), d, 0.0, 0.0, 0, seq.draft_tokens,
                    seq.draft_logits, seq.n_drafted)
        B.ssd_verify(seq.handle, plan.get("skip_mask"), plan.get("exit_layer"), d, seq.draft_tokens, seq.n_drafted,
                     reuse, seq.verify_logits)
        torch.cuda.synchronize()
        outs.append(seq.verify_logits[: (d + 1) * shape.vocab].clone())
        seq.close()
    assert torch.equal(outs[0], outs[1])


def test_empty_plan_accepts_everything(pair):
    shape, g, o = pair
    P, n_gen, d = 16, 30, 4
    prompt = synth.prompt_tokens(P, shape.vocab)
    seq = B.Sequence(g, max_ctx=P + n_gen + 2 * d + 8, max_rows=64, max_draft=8)
    out, stats = seq.generate_ssd(dev(prompt), n_gen, skip_mask=np.zeros(2 * shape.n_layers, np.uint8), d=d)
    assert all(e == dp + 1 for dp, e in stats)
    seq.close()


def test_sampled_ssd_matches_oracle(pair):
    """T = 1 with a confidence stop: same Philox draws on both sides, so the emitted
    tokens agree except where a decision of the oracle lies within 1e-2 (log units)
    of flipping; after such a token both sides restart from the oracle's prefix
    and the comparison runs to the end."""
    shape, g, o = pair
    plan = PLANS[shape.name]
    mask = _mask_of(shape, plan)
    d, tau, T, seed = plan["d"], 0.002, 1.0, 12345
    P, n_gen = 24, 40
    prompt = synth.prompt_tokens(P, shape.vocab)
    seq = B.Sequence(g, max_ctx=P + n_gen + 2 * d + 8, max_rows=64, max_draft=8)
    drafted = []

    def gpu_run(prefix, n):
        out, stats = seq.generate_ssd(dev(prefix), n, skip_mask=plan.get("skip_mask"),
                                      exit_layer=plan.get("exit_layer"), d=d, conf_thresh=tau, temperature=T,
                                      seed=seed)
        drafted.extend(s[0] for s in stats)
        return out

    def oracle_run(prefix, n):
        toks, st, _ = ossd.ssd_generate(o, prefix, n, mask, d, tau=tau, T=T, seed=seed)
        return toks, st

    events = check_sampled_with_resync(gpu_run, oracle_run, prompt, n_gen)
    print("sampled: %d re-synchronisations over %d tokens; gpu drafted %s" % (events, n_gen, drafted[:10]))
    seq.close()


def test_row_stats_match_oracle():
    rng = np.random.default_rng(7)
    V, rows = 32000, 6
    z = (rng.standard_normal((rows, V)) * 2.0).astype(np.float32)
    z[2, 77] = z[2].max() + 1.0
    z[2, 78] = z[2, 77]                     # a tie: lowest index wins, margin 0
    zt = dev(z.reshape(-1), torch.float32)
    st = torch.zeros(rows * 6, dtype=torch.int32, device="cuda")
    for T in (0.0, 0.7):
        B.ssd_row_stats(zt, rows, V, T, 99, 5, st)
        torch.cuda.synchronize()
        raw = st.cpu().numpy()
        fl = raw.view(np.float32).reshape(rows, 6)
        it = raw.reshape(rows, 6)
        for r in range(rows):
            zz = z[r].astype(np.float64)
            assert it[r, 1] == int(np.argmax(zz))
            assert fl[r, 0] == z[r].max()
            s = np.sort(zz)
            assert fl[r, 2] == np.float32(s[-2])
            lse = ossd.log_softmax(zz, T)
            assert abs(fl[r, 3] - (np.max(zz / (T or 1.0)) - np.max(lse))) < 1e-4
            assert abs(fl[r, 4] - ossd.confidence(zz, T)) < 1e-5
            if T > 0:
                assert it[r, 5] == ossd.sample_logits(zz, T, 99, 5, r, ophilox.PURPOSE_DRAFT)
            else:
                assert it[r, 5] == it[r, 1]


@pytest.mark.parametrize("T", [0.0, 1.0, 0.6])
def test_accept_matches_oracle(T):
    """ssd_accept on constructed verify/draft logits vs the oracle's accept rule."""
    shape = BF16_HD64
    g = gpu_model(shape, n_layers=1)
    V, d = shape.vocab, 6
    rng = np.random.default_rng(11)
    seq = B.Sequence(g, max_ctx=128, max_rows=16, max_draft=8)
    B.ssd_prefill(seq.handle, dev(synth.prompt_tokens(4, V)))     # iteration becomes 1
    agree = 0
    for trial in range(12):
        zp = (rng.standard_normal((d + 1, V)) * 3).astype(np.float32)
        zq = zp[:d] + (rng.standard_normal((d, V)) * 0.5).astype(np.float32)
        drafts = [int(ossd.sample_logits(zq[i].astype(np.float64), T or 1.0, 5, trial, i, 0)) for i in range(d)]
        if T == 0:
            drafts = [int(np.argmax(zp[i])) if i < trial % (d + 1) else int(np.argmax(zq[i])) for i in range(d)]
        dp = d - trial % 3
        seq.verify_logits[: (d + 1) * V].copy_(dev(zp.reshape(-1), torch.float32))
        seq.draft_logits[: d * V].copy_(dev(zq.reshape(-1), torch.float32))
        seq.draft_tokens[:d].copy_(dev(drafts))
        seq.n_drafted.fill_(dp)
        B.ssd_accept(seq.handle, seq.verify_logits, seq.draft_logits, seq.draft_tokens, seq.n_drafted, d, T, 777,
                     seq.out_tokens, seq.n_out)
        torch.cuda.synchronize()
        n = int(seq.n_out.item())
        got = seq.out_tokens[:n].cpu().numpy().tolist()
        if T == 0:
            ref = ossd.accept_greedy(zp[: dp + 1].astype(np.float64), drafts[:dp])
        else:
            ref = ossd.accept_sampled(zp[: dp + 1].astype(np.float64), zq[:dp].astype(np.float64), drafts[:dp], T,
                                      777, 1)
        assert 1 <= n <= dp + 1
        agree += got == ref
    assert agree == 12
    seq.close()
    g.close()


def test_score_masks_match_oracle():
    shape = BF16_HD64
    g = gpu_model(shape)
    o = omodel.Model.synthetic(shape)
    P, gamma = 40, 32
    prompt = synth.prompt_tokens(P, shape.vocab)
    ref, kv = ossd.ar_generate(o, prompt, gamma)
    window = (list(prompt) + ref)[P - 1: P + gamma]
    masks = [np.zeros(8, np.uint8), synth.mask_from_layers(4, [1]), synth.mask_from_layers(4, [0, 2]),
             synth.mask_exit(4, 2), np.array([0, 1, 1, 0, 0, 0, 0, 1], np.uint8)]
    oscores, obest, opred, omargin = ossd.score_masks(o, kv, window, P - 1, masks, detail=True)
    seq = B.Sequence(g, max_ctx=P + gamma + 64, max_rows=len(masks) * gamma, max_draft=4)
    seq.generate_ar(dev(prompt), gamma)            # the cache before the window: the prompt's keys/values
    scores = torch.zeros(len(masks), dtype=torch.float32, device="cuda")
    best = torch.zeros(1, dtype=torch.int32, device="cuda")
    pred = torch.zeros(len(masks) * gamma, dtype=torch.int32, device="cuda")
    B.ssd_score_masks(seq.handle, np.stack(masks), dev(window), P - 1, gamma, scores, best, pred)
    torch.cuda.synchronize()
    gs = scores.cpu().numpy()
    print("scores gpu %s oracle %s" % (gs, oscores))
    assert gs[0] == 1.0
    nd = check_scores(gs, int(best.item()), pred.cpu().numpy().reshape(len(masks), gamma), window, oscores, obest,
                      opred, omargin)
    print("rows differing from the oracle (all near-ties): %d" % nd)
    seq.close()
    g.close()


@pytest.mark.parametrize("shape", [BF16_HD64, BF16_HD128, F32_GQA], ids=lambda s: s.name)
def test_score_masks_shared_prefixes_equal_alone(shape):
    """Plans that agree on their first sub-layers share those sub-layers' rows in a
    scoring pass (one launch per class of equal prefixes, copies where a class
    splits).  A set with long shared prefixes, splits at the first and the last
    sub-layer, a duplicate plan and the empty plan, scored together, gives every
    plan the predictions and score it gets when scored alone, bit for bit."""
    g = gpu_model(shape)
    o = omodel.Model.synthetic(shape)
    L = shape.n_layers
    P, gamma = 40, 16
    prompt = synth.prompt_tokens(P, shape.vocab)
    ref, _ = ossd.ar_generate(o, prompt, gamma)
    window = (list(prompt) + ref)[P - 1: P + gamma]
    z = np.zeros(2 * L, np.uint8)
    def sk(*i):
        m = z.copy()
        m[list(i)] = 1
        return m
    masks = [sk(2 * L - 1), z.copy(), sk(0), sk(2 * L - 1), sk(1, 2 * L - 2), sk(1), sk(0, 3), sk(0, 2 * L - 1),
             sk(*range(2 * L)), sk(2, 3), sk(2, 4)]
    seq = B.Sequence(g, max_ctx=P + gamma + 64, max_rows=len(masks) * gamma, max_draft=4)
    seq.generate_ar(dev(prompt), gamma)
    def score(ms):
        sc = torch.zeros(len(ms), dtype=torch.float32, device="cuda")
        best = torch.zeros(1, dtype=torch.int32, device="cuda")
        pred = torch.zeros(len(ms) * gamma, dtype=torch.int32, device="cuda")
        B.ssd_score_masks(seq.handle, np.stack(ms), dev(window), P - 1, gamma, sc, best, pred)
        torch.cuda.synchronize()
        return sc.cpu().numpy(), pred.cpu().numpy().reshape(len(ms), gamma)
    print("[gpu] %s: %d plans together" % (shape.name, len(masks)), flush=True)
    gs, gp = score(masks)
    for c, m in enumerate(masks):
        s1, p1 = score([m])
        assert s1[0] == gs[c] and np.array_equal(p1[0], gp[c]), c
    assert gs[0] == gs[3] and np.array_equal(gp[0], gp[3])
    assert B.ssd_read_state(seq.handle).error_flags == 0
    print("scores %s" % gs)
    seq.close()
    g.close()


@pytest.mark.parametrize("shape,P,gamma", [(BF16_HD64, 200, 12), (BF16_HD128, 150, 32), (BF16_HD64, 131, 32),
                                           (BF16_HD128, 257, 8)],
                         ids=["hd64-gqa-P200-g12", "hd128-P150-g32", "hd64-gqa-P131-g32", "hd128-P257-g8"])
def test_score_masks_long_prefix_any_pages(shape, P, gamma):
    """Mask scoring over a prompt of several 64-key chunks (the attention walks the
    cached prefix chunk by chunk before the candidates' own window keys; windows of
    8, 12 and 32 rows; grouped-query heads: 24 and 64 queries per block, one, two
    and four waves): the scores and predictions match the oracle's up to its
    near-ties, and pages of 16 or 32 positions scattered by a permuted page table
    give the same scores and predictions bit for bit as contiguous 64-position
    pages."""
    g = gpu_model(shape)
    o = omodel.Model.synthetic(shape)
    L = shape.n_layers
    prompt = synth.prompt_tokens(P, shape.vocab)
    ref, kv = ossd.ar_generate(o, prompt, gamma)
    window = (list(prompt) + ref)[P - 1: P + gamma]
    masks = [np.zeros(2 * L, np.uint8), synth.mask_from_layers(L, [1]), synth.mask_exit(L, 2),
             synth.mask_from_layers(L, [0]), np.array([0, 1] + [0] * (2 * L - 3) + [1], np.uint8)]
    oscores, obest, opred, omargin = ossd.score_masks(o, kv, window, P - 1, masks, detail=True)
    max_ctx = P + gamma + 64
    results = []
    for ps in (64, 16, 32):
        n_lp = (max_ctx + ps - 1) // ps
        mul = next(m for m in range(7, 64) if math.gcd(m, n_lp) == 1)   # (mul i + 3) mod n: a permutation
        perm = None if ps == 64 else [(mul * i + 3) % n_lp for i in range(n_lp)]
        assert perm is None or sorted(perm) == list(range(n_lp))
        seq = B.Sequence(g, max_ctx=max_ctx, max_rows=len(masks) * gamma, max_draft=4, page_size=ps, page_table=perm)
        seq.generate_ar(dev(prompt), gamma)
        scores = torch.zeros(len(masks), dtype=torch.float32, device="cuda")
        best = torch.zeros(1, dtype=torch.int32, device="cuda")
        pred = torch.zeros(len(masks) * gamma, dtype=torch.int32, device="cuda")
        B.ssd_score_masks(seq.handle, np.stack(masks), dev(window), P - 1, gamma, scores, best, pred)
        torch.cuda.synchronize()
        assert B.ssd_read_state(seq.handle).error_flags == 0
        results.append((scores.cpu().numpy(), int(best.item()), pred.cpu().numpy()))
        seq.close()
    gs, gb, gp = results[0]
    print("page 64: scores gpu %s oracle %s" % (gs, oscores))
    print("oracle top-2 margins of the full plan's rows: %s" % np.round(omargin[0], 4))
    # the full plan reproduces the window except at the oracle's near-ties
    assert gs[0] >= 1.0 - int((np.asarray(omargin[0]) < 1e-2).sum()) / gamma
    nd = check_scores(gs, gb, gp.reshape(len(masks), gamma), window, oscores, obest, opred, omargin)
    print("rows differing from the oracle (all near-ties): %d" % nd)
    for s2, b2, p2 in results[1:]:
        assert np.array_equal(s2, gs) and b2 == gb and np.array_equal(p2, gp)
    g.close()


def test_capacity_is_reported_not_faulted():
    shape = synth.TINY
    g = gpu_model(shape)
    P = 50
    seq = B.Sequence(g, max_ctx=64, max_rows=64, max_draft=8)
    B.ssd_prefill(seq.handle, dev(synth.prompt_tokens(P, shape.vocab)))
    with pytest.raises(B.SSDError) as e:
        for _ in range(10):
            seq.ssd_iteration(None, 2, 8)
            B.ssd_read_state(seq.handle)
    assert e.value.code == B.SSD_ERR_CAPACITY
    seq.close()
    g.close()


@pytest.mark.parametrize("shape", [BF16_HD64, BF16_HD128], ids=lambda s: s.name)
def test_decode_step_equals_prefill_row(shape):
    """An AR step (decode-block kernels, one row) gives the same logits, bit for
    bit, as the last row of a prefill (general kernels, many rows) at that
    position."""
    g = gpu_model(shape)
    P = 70
    prompt = synth.prompt_tokens(P, shape.vocab)
    seq1 = B.Sequence(g, max_ctx=P + 64, max_rows=64, max_draft=4)
    B.ssd_prefill(seq1.handle, dev(prompt))
    lg1 = torch.zeros(shape.vocab, dtype=torch.float32, device="cuda")
    B.ssd_decode_ar(seq1.handle, 0.0, 0, lg1)
    t_p = int(B.ssd_read_output(seq1.handle, 2)[0])
    assert B.ssd_read_state(seq1.handle).error_flags == 0
    seq1.close()
    seq2 = B.Sequence(g, max_ctx=P + 64, max_rows=32, max_draft=4)
    lg2 = torch.zeros(shape.vocab, dtype=torch.float32, device="cuda")
    B.ssd_prefill(seq2.handle, dev(list(prompt) + [t_p]), 0.0, 0, lg2)
    torch.cuda.synchronize()
    assert torch.equal(lg1, lg2)
    seq2.close()
    g.close()


@pytest.mark.parametrize("shape", [BF16_HD64, F32_GQA], ids=lambda s: s.name)
def test_prefill_chunkings_agree(shape):
    """A 1100-token prompt prefilled in chunks of 64 rows, of 1024 + 76 rows (a
    sequence of 4096 rows takes at most 1024 per prefill chunk, the split-key
    attention's capacity) and of 700 + 400 rows gives the same last-row logits
    and the same next AR step, bit for bit: a row's result does not depend on
    the rows it is processed with."""
    g = gpu_model(shape)
    P = 1100
    prompt = synth.prompt_tokens(P, shape.vocab)
    out = []
    for max_rows in (64, 4096, 700):
        print("[gpu] %s: prefill of %d tokens, max_rows %d" % (shape.name, P, max_rows), flush=True)
        seq = B.Sequence(g, max_ctx=P + 64, max_rows=max_rows, max_draft=4)
        lp = torch.zeros(shape.vocab, dtype=torch.float32, device="cuda")
        la = torch.zeros(shape.vocab, dtype=torch.float32, device="cuda")
        B.ssd_prefill(seq.handle, dev(prompt), 0.0, 0, lp)
        B.ssd_decode_ar(seq.handle, 0.0, 0, la)
        torch.cuda.synchronize()
        assert B.ssd_read_state(seq.handle).error_flags == 0
        out.append((lp.clone(), la.clone(), B.ssd_read_output(seq.handle, 2)))
        seq.close()
    for lp, la, toks in out[1:]:
        assert torch.equal(lp, out[0][0]) and torch.equal(la, out[0][1]) and list(toks) == list(out[0][2])
    g.close()


@pytest.mark.parametrize("N,K", [(16, 32), (1000, 256), (2003, 512), (48, 4096)])
def test_pack_bf16_layout(N, K):
    """ssd_pack_bf16 (device kernel) against the layout definition (element (n, k) at
    ((n / 16) * (K / 32) + k / 32) * 512 + (n % 16) * 32 + k % 32, padding rows zero)."""
    src = torch.arange(N * K, dtype=torch.float32, device="cuda").remainder(251).to(torch.bfloat16).view(N, K)
    nbytes = B.ssd_packed_bf16_bytes(N, K)
    Np = (N + 15) // 16 * 16
    assert nbytes == Np * K * 2
    dst = torch.full((Np * K,), 7.0, dtype=torch.bfloat16, device="cuda")
    B.ssd_pack_bf16(src, dst, N, K)
    torch.cuda.synchronize()
    d = dst.cpu().float().numpy()
    sv = src.cpu().float().numpy()
    n = np.arange(Np)[:, None]
    k = np.arange(K)[None, :]
    idx = ((n // 16) * (K // 32) + k // 32) * 512 + (n % 16) * 32 + k % 32
    ref = np.zeros((Np, K), np.float32)
    ref[:N] = sv
    assert np.array_equal(d[idx], ref)
    assert torch.equal(sdev.unpack_bf16(dst, N, K), src)


def test_pack_bf16_rejects_bad_k():
    src = torch.zeros(16, 48, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(B.SSDError) as e:
        B.ssd_pack_bf16(src, torch.zeros_like(src), 16, 48)
    assert e.value.code == B.SSD_ERR_SHAPE


@pytest.mark.parametrize("shape,P,ctxs", [(BF16_HD64, 2100, (2240, 4224, 8320)), (BF16_HD128, 2100, (2240, 8320)),
                                          (BF16_HD64, 4200, (4352, 8320)), (BF16_HD128, 4200, (4352, 8320))],
                         ids=["hd64-gqa-P2100", "hd128-P2100", "hd64-gqa-P4200", "hd128-P4200"])
def test_long_context_attention_paths_agree(shape, P, ctxs):
    """Contexts of 2100 and 4200 tokens (33 and 66 active 64-key splits): the
    decode attention with the merge folded in (KV pages for 2240 positions: 35
    splits; it holds up to 64) and the general partial + combine kernels (pages
    for 4224, 4352 and 8320 positions: 66, 68 and 130 splits) give the same draft
    and verify logits, bit for bit; the AR step's logits match the oracle."""
    g = gpu_model(shape)
    o = omodel.Model.synthetic(shape)
    d = 4
    prompt = synth.prompt_tokens(P, shape.vocab)
    plan = PLANS[shape.name]
    runs = []
    for max_ctx in ctxs:
        print("[gpu] %s: max_ctx %d" % (shape.name, max_ctx), flush=True)
        seq = B.Sequence(g, max_ctx=max_ctx, max_rows=64, max_draft=d)
        B.ssd_prefill(seq.handle, dev(prompt))
        lg = torch.zeros(shape.vocab, dtype=torch.float32, device="cuda")
        B.ssd_decode_ar(seq.handle, 0.0, 0, lg)
        seq.ssd_iteration(plan.get("skip_mask"), plan.get("exit_layer"), d)
        st = B.ssd_read_state(seq.handle)
        assert st.error_flags == 0
        runs.append((lg.clone(), seq.draft_logits.clone(), seq.verify_logits.clone(), st.last_n_drafted))
        seq.close()
    a0, a1, a2, n0 = runs[0]
    for b0, b1, b2, n1 in runs[1:]:
        assert n0 == n1
        assert torch.equal(a0, b0) and torch.equal(a1, b1) and torch.equal(a2, b2)
    _, ref_z = oracle_ar_with_logits(o, prompt, 2)
    err = np.abs(a0.cpu().numpy() - ref_z[1]).max()
    print("AR step at position %d: max |dz| = %.3g" % (P, err))
    assert err < logit_tol(shape)
    g.close()


@pytest.mark.parametrize("shape,sublayers,bo_every,n_sub,seed",
                         [(BF16_HD64, False, 0, 0, 5), (F32_GQA, False, 0, 0, 5), (BF16_HD64, True, 0, 0, 5),
                          (F32_GQA, True, 2, 4, 5), (BF16_HD128, True, 2, 2, 9)],
                         ids=["bf16-hd64-gqa-layers", "f32-gqa-layers", "bf16-hd64-gqa-sublayers",
                              "f32-gqa-sublayers-bo2", "bf16-hd128-sublayers-bo2"])
def test_swift_search_matches_oracle(shape, sublayers, bo_every, n_sub, seed):
    """SWIFT search (ssd_swift_search: proposals and the Bayesian-optimisation
    step on the host, batched scoring passes) against the oracle's
    search with its own scoring: same number of steps, same final plan, score
    within the scoring tolerance.  The target is out of reach, so the search runs
    until its patience ends.  In the bo2 cases (n_sub sub-layers skipped, evenly
    spaced at the start) every second step is a BO step, and on these inputs the
    BO steps change the oracle's path (final plan and score) against plain
    random search.  With rows for several steps per pass (a step and the random
    steps after it scored together) the search is the same bit for bit."""
    from oracle import swift
    g = gpu_model(shape)
    o = omodel.Model.synthetic(shape)
    P, gamma, n_cand = 40, 32, 3
    L = shape.n_layers
    prompt = synth.prompt_tokens(P, shape.vocab)
    ref, kv = ossd.ar_generate(o, prompt, gamma)
    _, ref_z = oracle_ar_with_logits(o, prompt, gamma)
    window = (list(prompt) + ref)[P - 1: P + gamma]
    n_skip = 2 if L >= 4 else 1
    init = swift.layers_to_mask(L, swift.uniform_skip_layers(L, n_skip))
    steps, patience = 6, 3
    if n_sub:
        n_skip, steps, patience = n_sub, 8, 4
        init = np.zeros(2 * L, np.uint8)
        init[[i * 2 * L // n_sub for i in range(n_sub)]] = 1
    fn = lambda ms: ossd.score_masks(o, kv, window, P - 1, ms)[0]
    obest, oscore, osteps, hist = swift.search(fn, L, init, n_skip, n_cand, steps, patience, 1.5, seed, sublayers,
                                               bo_every=bo_every)
    if bo_every:
        rbest, rscore, _, _ = swift.search(fn, L, init, n_skip, n_cand, steps, patience, 1.5, seed, sublayers)
        assert rscore != oscore and not np.array_equal(rbest, obest)
    print("oracle: %d steps, score %.4f, best %s; per step %s" % (osteps, oscore, obest[::2],
                                                                  [np.round(h[1], 3).tolist() for h in hist]))
    seq = B.Sequence(g, max_ctx=P + gamma + 64, max_rows=(n_cand + 1) * gamma, max_draft=4)
    gout = seq.generate_ar(dev(prompt), gamma)
    check_greedy_tokens(gout, ref, ref_z)     # the window itself comes from the oracle
    gbest, gscore, gsteps = B.ssd_swift_search(seq.handle, dev(window), P - 1, gamma, init, n_skip, n_cand, steps,
                                               patience, 1.5, seed, L, sublayers=sublayers, bo_every=bo_every)
    print("gpu: %d steps, score %.4f, best %s" % (gsteps, gscore, gbest[::2]))
    assert gsteps == osteps
    assert np.array_equal(gbest, obest)
    # the final plan's score may differ only by its rows that are oracle near-ties (top-2 margin < 1e-2)
    _, _, _, om = ossd.score_masks(o, kv, window, P - 1, [obest], detail=True)
    assert abs(gscore - oscore) <= int((om < 1e-2).sum()) / gamma + 1e-7
    seq.close()
    # room for several steps per scoring pass (the random steps after a step, up to the next BO step, are
    # scored with it): the same search, bit for bit
    seq = B.Sequence(g, max_ctx=P + gamma + 64, max_rows=4 * (n_cand + 1) * gamma, max_draft=4)
    seq.generate_ar(dev(prompt), gamma)
    bbest, bscore, bsteps = B.ssd_swift_search(seq.handle, dev(window), P - 1, gamma, init, n_skip, n_cand, steps,
                                               patience, 1.5, seed, L, sublayers=sublayers, bo_every=bo_every)
    assert bsteps == gsteps and bscore == gscore and np.array_equal(bbest, gbest)
    seq.close()
    g.close()


@pytest.mark.parametrize("shape", [BF16_HD64, BF16_HD128, F32_GQA], ids=lambda s: s.name)
def test_swift_search_passes_beyond_1024_rows(shape):
    """Eight random search steps of 15 proposals on a 32-token window with rows
    for all of them in one scoring pass (1 + 8 * 15 plans, 3872 rows; f32 models
    keep their passes within 1024 rows, the split attention's capacity) and with
    one step per pass: the same steps, score and plan, bit for bit.  The row
    invariance of the projections and of the scoring attention makes a candidate's
    rows independent of the pass they run in."""
    g = gpu_model(shape)
    o = omodel.Model.synthetic(shape)
    P, gamma, n_cand, steps = 40, 32, 15, 8
    L = shape.n_layers
    prompt = synth.prompt_tokens(P, shape.vocab)
    ref, _ = ossd.ar_generate(o, prompt, gamma)
    window = (list(prompt) + ref)[P - 1: P + gamma]
    init = B.ssd_uniform_mask(L, 1)
    out = []
    for max_rows in ((n_cand + 1) * gamma, (steps * n_cand + 1) * gamma):
        print("[gpu] %s: search with max_rows %d" % (shape.name, max_rows), flush=True)
        seq = B.Sequence(g, max_ctx=P + gamma + 64, max_rows=max_rows, max_draft=4)
        seq.generate_ar(dev(prompt), gamma)      # the cache holds the full model's keys and values
        out.append(B.ssd_swift_search(seq.handle, dev(window), P - 1, gamma, init, 1, n_cand, steps, 100, 1.5, 11,
                                      L, sublayers=True))
        seq.close()
    (b0, s0, n0), (b1, s1, n1) = out
    assert n0 == n1 == steps
    assert s0 == s1 and np.array_equal(b0, b1)
    g.close()


@pytest.mark.parametrize("shape", [BF16_HD64, BF16_HD128, F32_GQA], ids=lambda s: s.name)
def test_decode_exit_matches_oracle(shape):
    """Lossy early-exit decoding (ssd_decode_exit, exit at layer 1 and a skip mask)
    against the oracle's exit_generate: tokens by the margin rule, each step's
    logits within the logit tolerance up to the first excused mismatch."""
    g = gpu_model(shape)
    o = omodel.Model.synthetic(shape)
    L, V = shape.n_layers, shape.vocab
    P, n = 24, 16
    prompt = synth.prompt_tokens(P, V)
    for exit_layer, mask in ((1, None), (None, synth.mask_from_layers(L, [L - 2]))):
        om = synth.mask_exit(L, exit_layer) if mask is None else mask
        ref, ref_z = ossd.exit_generate(o, prompt, n, om)
        seq = B.Sequence(g, max_ctx=P + n + 16, max_rows=64, max_draft=2)
        B.ssd_prefill(seq.handle, dev(prompt))
        zs = []
        for _ in range(n - 1):
            lg = torch.zeros(V, dtype=torch.float32, device="cuda")
            B.ssd_decode_exit(seq.handle, mask, exit_layer, 0.0, 0, lg)
            zs.append(lg)
        out = [int(x) for x in B.ssd_read_output(seq.handle, n)]
        assert B.ssd_read_state(seq.handle).error_flags == 0
        stop = check_greedy_tokens(out, ref, ref_z)
        upto = n - 1 if stop is None else stop - 1
        for k in range(upto):
            err = np.abs(zs[k].cpu().numpy() - ref_z[k + 1]).max()
            assert err < logit_tol(shape), (k, err)
        seq.close()
    g.close()


@pytest.mark.parametrize("shape", [BF16_HD64, BF16_HD128, F32_GQA], ids=lambda s: s.name)
def test_specee_features_match_oracle(shape):
    """SpecEE exit features (ssd_specee_features) of seeded hidden states against the
    oracle: logits within the logit tolerance, probabilities and variation within
    0.005 (their error is the logits' scaled by a probability)."""
    g = gpu_model(shape)
    o = omodel.Model.synthetic(shape)
    rng = np.random.default_rng(17)
    rows, k = 5, 4
    h = rng.standard_normal((rows, shape.d_model)) * 0.5
    toks = np.array([1, shape.vocab - 1, 17, shape.vocab // 2], np.int32)
    prev = rng.random((rows, k))
    prev /= prev.sum(axis=1, keepdims=True)
    hd = torch.from_numpy(h.astype(np.float32)).cuda()
    td = torch.from_numpy(toks).cuda()
    pd = torch.from_numpy(prev.astype(np.float32)).cuda()
    for pv in (None, pd):
        out = torch.zeros(rows, 3 * k, dtype=torch.float32, device="cuda")
        B.ssd_specee_features(g.handle, hd, rows, td, k, pv, out)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        ref = ossd.specee_features(o, h.astype(np.float32).astype(np.float64), toks,
                                   None if pv is None else prev.astype(np.float32).astype(np.float64))
        assert np.abs(got[:, :k] - ref[:, :k]).max() < logit_tol(shape)
        assert np.abs(got[:, k:] - ref[:, k:]).max() < 5e-3
    g.close()
