"""Full-size parity: the 32-layer LLaMA-2-7B-shaped model of the bench, in the
bench's launch configuration (512-token prompt, exit at layer 8, d = 12,
greedy).  Checked (a) as properties of the path that hold at any size — greedy
SSD tokens equal AR tokens, the verify with the draft's saved state equals the
verify that recomputes every row, a decode step equals the last row of a
prefill, all bit for bit — and (b) against the float64 oracle at full width and
depth: the first token's logits and every draft and verify row of two SSD
iterations after the 512-token prompt (beside the oracle's float32-accumulation
twin on the same rows), 64 generated tokens against the oracle's greedy AR
tokens, and the logits of the first four tokens after an 8-token prompt."""
import numpy as np
import pytest
import torch

import synth
from self_speculative_layer_amd import binding as B
from oracle import model as omodel

from gpu_util import dev, gpu_model, oracle_ar_with_logits

pytestmark = pytest.mark.gpu

SHAPE = synth.LLAMA7B
# |dz| / max|z| per row.  Over 32 layers the bf16 rounding points make the decoder sensitive to the
# accumulation precision in front of them: the oracle with its products accumulated in float32 instead of
# float64 (same rounding points) differs from itself by up to 1.93 % of max|z| on the rows of an 8-token
# prompt at this size (0.47 % at two layers); the bound is 2^-5 (3.1 %).
REL_TOL = 2.0 ** -5


@pytest.fixture(scope="module")
def model7b():
    print("[gpu] full-size 7B: building weights", flush=True)
    g = gpu_model(SHAPE)
    yield g
    g.close()


def test_fullsize_bench_config_properties(model7b):
    g = model7b
    P, d, E = 512, 12, 8
    prompt = synth.prompt_tokens(P, SHAPE.vocab)
    n_gen = 2 * d + 4
    outs, vlog = [], []
    for reuse in (True, False):
        seq = B.Sequence(g, max_ctx=P + n_gen + 2 * d + 16, max_rows=64, max_draft=d)
        B.ssd_prefill(seq.handle, dev(prompt))
        seq.ssd_iteration(None, E, d, reuse=reuse)
        torch.cuda.synchronize()
        vlog.append(seq.verify_logits.clone())
        seq.close()
        seq = B.Sequence(g, max_ctx=P + n_gen + 2 * d + 16, max_rows=64, max_draft=d)
        out, stats = seq.generate_ssd(dev(prompt), n_gen, exit_layer=E, d=d, reuse=reuse)
        assert all(1 <= e <= dp + 1 for dp, e in stats)
        outs.append([int(x) for x in out])
        seq.close()
    assert torch.equal(vlog[0], vlog[1])
    assert outs[0] == outs[1]
    seq = B.Sequence(g, max_ctx=P + n_gen + 16, max_rows=64, max_draft=d)
    ar = [int(x) for x in seq.generate_ar(dev(prompt), n_gen)]
    seq.close()
    assert ar == outs[0]
    # a decode step (decode-block kernels) == the last row of a prefill (tiled kernels) at that position
    seq = B.Sequence(g, max_ctx=P + 16, max_rows=512, max_draft=2)
    B.ssd_prefill(seq.handle, dev(prompt))
    lg = torch.zeros(SHAPE.vocab, dtype=torch.float32, device="cuda")
    B.ssd_decode_ar(seq.handle, 0.0, 0, lg)
    t = int(B.ssd_read_output(seq.handle, 2)[1])
    seq.close()
    seq = B.Sequence(g, max_ctx=P + 16, max_rows=520, max_draft=2)
    lg2 = torch.zeros(SHAPE.vocab, dtype=torch.float32, device="cuda")
    B.ssd_prefill(seq.handle, dev(list(prompt) + [ar[0]]), 0.0, 0, lg2)
    torch.cuda.synchronize()
    seq.close()
    assert t == ar[1]
    assert torch.equal(lg, lg2)


def _rel_rows(a, b):
    """Per row: max |a - b| / max |b|."""
    a, b = np.atleast_2d(a), np.atleast_2d(b)
    return np.abs(a - b).max(axis=1) / np.abs(b).max(axis=1)


def test_fullsize_bench_prompt_parity(model7b):
    """The bench configuration itself (512-token prompt, exit 8, d = 12, greedy) against the float64
    oracle: the first token's logits and every draft and verify row of the first two SSD iterations, row
    by row, beside the same rows of the oracle's float32-accumulation twin (same rounding points; its
    drift from the oracle is what accumulation order alone does at this depth); then 64 generated tokens
    against the oracle's greedy AR tokens with re-synchronisation at near-ties."""
    from gpu_util import acc32_twin, check_greedy_with_resync
    from oracle import ssd as ossd
    g = model7b
    P, d, E, n_iter, n_gen = 512, 12, 8, 2, 64
    V = SHAPE.vocab
    prompt = synth.prompt_tokens(P, V)
    mask = synth.mask_exit(SHAPE.n_layers, E)
    print("[gpu] full-size 7B, 512-token prompt: float64 oracle prefill", flush=True)
    o = omodel.Model.synthetic(SHAPE)
    kv = omodel.KVCache(SHAPE, P + n_gen + 2 * d + 4)
    z0 = ossd.prefill(o, kv, prompt)
    kv_ar = kv.copy()
    out = [int(np.argmax(z0))]
    iters = []                                     # (y0, n, drafts, zq, zp)
    for it in range(1, n_iter + 1):
        n = P + len(out)
        y0 = out[-1]
        drafts, zq, hb = ossd.draft(o, kv, y0, n, mask, d, 0.0, 0.0, 0, it)
        zp = ossd.verify(o, kv, y0, drafts, n, E, hb)
        iters.append((y0, n, drafts, zq, zp))
        out += ossd.accept_greedy(zp, drafts)
        print("[gpu]   oracle iteration %d: %d drafts, emitted %d" % (it, len(drafts), len(out) - 1), flush=True)
    # the twin on the same rows (teacher-forced with the oracle's tokens)
    print("[gpu] float32-accumulation twin", flush=True)
    tw = acc32_twin(o)
    kvt = omodel.KVCache(SHAPE, P + n_gen + 2 * d + 4)
    tw_rows = [ossd.prefill(tw, kvt, prompt)[None]]
    for y0, n, drafts, zq, zp in iters:
        pos = list(range(n - 1, n - 1 + len(drafts) + 1))
        tw_rows.append(omodel.forward(tw, [y0] + drafts[:-1], pos[:-1], kvt.copy(), mask))
        tw_rows.append(omodel.forward(tw, [y0] + drafts, pos, kvt))
    del tw, kvt
    # the GPU path on the same steps
    seq = B.Sequence(g, max_ctx=P + n_gen + 2 * d + 16, max_rows=64, max_draft=d)
    lg0 = torch.zeros(V, dtype=torch.float32, device="cuda")
    B.ssd_prefill(seq.handle, dev(prompt), 0.0, 0, lg0)
    gpu_rows = [lg0.cpu().numpy()[None]]
    ref_rows = [z0[None]]
    tw_cmp = [tw_rows[0]]
    same_path = True
    for k_it, (y0, n, drafts, zq, zp) in enumerate(iters):
        seq.ssd_iteration(None, E, d)
        st = B.ssd_read_state(seq.handle)
        assert st.error_flags == 0
        dp = st.last_n_drafted
        gd = seq.draft_tokens[:dp].cpu().numpy().tolist()
        gq = seq.draft_logits[: dp * V].view(dp, V).cpu().numpy()
        if gd != list(drafts):
            # a draft token differs: only at an oracle near-tie; rows up to it saw the same inputs
            i = next(j for j, (a, b) in enumerate(zip(gd, drafts)) if a != b)
            assert np.sort(zq[i])[-1] - np.sort(zq[i])[-2] < 1e-2, "draft %d differs away from a near-tie" % i
            gpu_rows.append(gq[: i + 1])
            ref_rows.append(zq[: i + 1])
            tw_cmp.append(tw_rows[1 + 2 * k_it][: i + 1])
            same_path = False
            break
        gpu_rows += [gq, seq.verify_logits[: (dp + 1) * V].view(dp + 1, V).cpu().numpy()]
        ref_rows += [zq, zp]
        tw_cmp += [tw_rows[1 + 2 * k_it], tw_rows[2 + 2 * k_it]]
    seq.close()
    g_rel = np.concatenate([_rel_rows(a, b) for a, b in zip(gpu_rows, ref_rows)])
    t_rel = np.concatenate([_rel_rows(a, b) for a, b in zip(tw_cmp, ref_rows)])
    g_abs = np.concatenate([np.abs(np.atleast_2d(a) - np.atleast_2d(b)).max(axis=1) for a, b in zip(gpu_rows, ref_rows)])
    q = lambda x: "median %.3g p90 %.3g max %.3g" % (np.median(x), np.quantile(x, 0.9), x.max())
    print("rows compared: %d (same draft path: %s)" % (len(g_rel), same_path))
    print("GPU  - oracle, max|dz| / max|z| per row: %s" % q(g_rel))
    print("twin - oracle, max|dz| / max|z| per row: %s" % q(t_rel))
    print("GPU  - oracle, max|dz| absolute per row: %s (max|z| %.3g)" % (q(g_abs), np.abs(z0).max()))
    assert len(g_rel) >= 2
    # the GPU accumulates in float32 in a different order from the twin (and keeps its softmax, attention
    # and RoPE table in float32): its drift is bounded by 1.5 times the twin's, row set against row set
    # (measured: median 1.08x, max 1.15x)
    assert np.median(g_rel) <= 1.5 * np.median(t_rel)
    assert g_rel.max() <= 1.5 * t_rel.max()
    # how far an implementation as accurate as the twin can move the difference of two logits: twice its
    # largest per-logit drift on these rows.  A greedy token may differ from the oracle's only where the
    # oracle puts the two tokens closer than that (the 1e-2 margin holds at two layers, not at 32: the
    # twin itself drifts by about 0.1 per logit here)
    t_abs = np.concatenate([np.abs(np.atleast_2d(a) - np.atleast_2d(b)).max(axis=1) for a, b in zip(tw_cmp, ref_rows)])
    near = 2.0 * t_abs.max()
    print("token excuse margin from the twin: %.3g" % near)
    # 64 tokens: the GPU's SSD loop against the oracle's greedy AR
    print("[gpu] oracle greedy AR, %d tokens" % n_gen, flush=True)
    ref, ref_z = [out[0]], [z0]
    while len(ref) < n_gen:
        z = omodel.forward(o, [ref[-1]], [P + len(ref) - 1], kv_ar)[0]
        ref.append(int(np.argmax(z)))
        ref_z.append(z)
        if len(ref) % 16 == 0:
            print("[gpu]   %d tokens" % len(ref), flush=True)
    del o
    seq = B.Sequence(g, max_ctx=P + n_gen + 2 * d + 16, max_rows=64, max_draft=d)
    events = check_greedy_with_resync(lambda pre, n: seq.generate_ssd(dev(pre), n, exit_layer=E, d=d)[0], prompt,
                                      ref, np.array(ref_z), margin=near, max_events=n_gen // 4)
    seq.close()
    print("64 greedy SSD tokens: %d re-synchronisations where the oracle puts the two tokens within %.3g" %
          (events, near))


def test_fullsize_logits_match_oracle(model7b):
    g = model7b
    P, n = 8, 4
    prompt = synth.prompt_tokens(P, SHAPE.vocab)
    print("[gpu] full-size 7B: building the float64 oracle", flush=True)
    o = omodel.Model.synthetic(SHAPE)
    ref, ref_z = oracle_ar_with_logits(o, prompt, n)
    del o
    seq = B.Sequence(g, max_ctx=P + n + 16, max_rows=64, max_draft=2)
    lgs = [torch.zeros(SHAPE.vocab, dtype=torch.float32, device="cuda") for _ in range(n)]
    B.ssd_prefill(seq.handle, dev(prompt), 0.0, 0, lgs[0])
    for k in range(1, n):
        B.ssd_decode_ar(seq.handle, 0.0, 0, lgs[k])
    out = [int(x) for x in B.ssd_read_output(seq.handle, n)]
    seq.close()
    for k in range(n):
        z = lgs[k].cpu().numpy()
        rel = np.abs(z - ref_z[k]).max() / np.abs(ref_z[k]).max()
        print("token %d: gpu %d oracle %d, max |dz| / max|z| = %.3g" % (k, out[k], ref[k], rel))
        assert rel < REL_TOL
        if out[k] != ref[k]:
            break                        # a near-tie changed the path; later rows no longer correspond


def test_fullsize_tree_properties(model7b):
    """Draft trees at the bench size (tree7b: exit 8, d = 12, at most 3 leaves): the tree verify's chain
    rows equal ssd_verify's bit for bit and do not depend on reuse; a leaf that repeats the chain token
    reproduces the chain row (its own key merged after the cached splits instead of inside them); greedy
    tree decoding emits AR's tokens (a difference only where AR's top-2 margin is below 1e-2)."""
    g = model7b
    P, d, E, ml = 512, 12, 8, 3
    V = SHAPE.vocab
    prompt = synth.prompt_tokens(P, V)
    trees = []
    for reuse in (True, False):
        seq = B.Sequence(g, max_ctx=P + 4 * d + 16, max_rows=64, max_draft=d)
        B.ssd_prefill(seq.handle, dev(prompt))
        B.ssd_draft(seq.handle, None, E, d, 0.0, 0.0, 0, seq.draft_tokens, seq.draft_logits, seq.n_drafted)
        B.ssd_tree_candidates(seq.handle, seq.draft_logits, seq.n_drafted, d, 0.9, 4, ml - 1, seq.leaf_tokens,
                              seq.leaf_depth, seq.n_leaves)
        torch.cuda.synchronize()
        dp, nl = int(seq.n_drafted.item()), int(seq.n_leaves.item())
        assert dp == d and nl == ml - 1
        y2 = int(seq.draft_tokens[1].item())
        seq.leaf_tokens[nl] = y2
        seq.leaf_depth[nl] = 2
        B.ssd_verify(seq.handle, None, E, d, seq.draft_tokens, seq.n_drafted, reuse, seq.verify_logits)
        torch.cuda.synchronize()
        chain = seq.verify_logits[: (d + 1) * V].clone()
        B.ssd_verify_tree(seq.handle, None, E, d, seq.draft_tokens, seq.n_drafted, seq.leaf_tokens, seq.leaf_depth,
                          dev([ml]), ml, reuse, seq.tree_logits)
        torch.cuda.synchronize()
        tz = seq.tree_logits[: (d + 1 + ml) * V].clone()
        assert torch.equal(tz[: (d + 1) * V], chain)
        trees.append(tz)
        seq.close()
    assert torch.equal(trees[0], trees[1])
    z = trees[0].view(d + 1 + ml, V)
    rel = (z[d + ml] - z[2]).abs().max().item() / z[2].abs().max().item()
    print("leaf repeating y_2 vs chain row 2: max |dz| / max|z| = %.3g" % rel)
    # the two rows differ only in the summation order of one key per layer, which the bf16 rounding points
    # carry through 32 layers like any accumulation-order change (measured 0.51 % of max|z|)
    assert rel < REL_TOL
    n_gen = 2 * d + 4
    seq = B.Sequence(g, max_ctx=P + n_gen + 2 * d + 16, max_rows=64, max_draft=d)
    out, stats = seq.generate_tree(dev(prompt), n_gen, exit_layer=E, d=d, rho=0.9, k_max=4, max_leaves=ml)
    seq.close()
    seq = B.Sequence(g, max_ctx=P + n_gen + 16, max_rows=64, max_draft=2)
    lgs = [torch.zeros(V, dtype=torch.float32, device="cuda") for _ in range(n_gen)]
    B.ssd_prefill(seq.handle, dev(prompt), 0.0, 0, lgs[0])
    for k in range(1, n_gen):
        B.ssd_decode_ar(seq.handle, 0.0, 0, lgs[k])
    ar = [int(x) for x in B.ssd_read_output(seq.handle, n_gen)]
    seq.close()
    got = [int(x) for x in out]
    for k in range(n_gen):
        if got[k] != ar[k]:
            s = torch.sort(lgs[k], descending=True).values
            assert (s[0] - s[1]).item() < 1e-2, "token %d: tree %d AR %d" % (k, got[k], ar[k])
            break
