"""SWIFT on the fly on the GPU (ssd_swift_begin / ssd_swift_generate through the
C ABI) against the oracle's swift_generate on the same seeded model and prompt:
the committed tokens (lossless: the greedy tokens are the full model's, checked
by the margin rule), the committed count after every iteration, the plan each
iteration drafts with, and per phase the plan chosen, the steps run, the
unimproved run and the stop flag, with the matchness within the scoring
tolerance (rows that are oracle near-ties may differ)."""
import numpy as np
import pytest
import torch

import synth
from self_speculative_layer_amd import binding as B
from oracle import model as omodel
from oracle import ssd as ossd
from oracle import swift
from gpu_util import BF16_HD64, F32_GQA, check_greedy_tokens, dev, gpu_model, oracle_ar_with_logits

pytestmark = pytest.mark.gpu


def _gpu_run(g, shape, prompt, cfg, init, n_gen, rows_factor=1):
    """One iteration per call; returns (tokens, n_out after each iteration, plan each iteration drafted with,
    per-phase records).  rows_factor: the sequence's row limit in units of one search step's rows (above 1 a
    scoring pass takes several steps)."""
    seq = B.Sequence(g, max_ctx=len(prompt) + n_gen + 64, max_rows=rows_factor * (cfg.n_cand + 1) * cfg.gamma,
                     max_draft=cfg.d)
    B.ssd_prefill(seq.handle, dev(prompt))
    st = B.ssd_swift_begin(seq.handle, cfg)
    assert st.last_phase_n_out == 1 and st.phases == 0
    plan = np.ascontiguousarray(init.copy())
    n_out, nouts, plans, phases = 1, [1], [None], []
    while n_out < n_gen:
        before = plan.copy()
        B.ssd_swift_generate(seq.handle, cfg, st, plan, 1, seq.draft_tokens, seq.draft_logits, seq.n_drafted,
                             seq.verify_logits, seq.out_tokens, seq.n_out)
        n_out = B.ssd_read_state(seq.handle).n_out
        nouts.append(n_out)
        plans.append(before)
        if st.phases > len(phases):
            phases.append(dict(n_out=n_out, after=plan.copy(), score=st.score, steps=st.steps,
                               unimproved=st.unimproved, done=st.done, last=st.last_phase_n_out))
    toks = [int(x) for x in B.ssd_read_output(seq.handle, n_gen)]
    assert st.iterations == len(nouts) - 1
    seq.close()
    return toks, nouts, plans, phases, st


@pytest.mark.parametrize("shape,n_skip,acc,per,max_steps,patience,bo_every,seed", [
    (BF16_HD64, 2, 0, 2, 8, 100, 0, 3),
    (F32_GQA, 1, 0, 2, 9, 3, 0, 7),
    (BF16_HD64, 2, 1, 1, 12, 100, 3, 5),
], ids=["bf16-hd64-window", "f32-gqa-patience", "bf16-hd64-sliding-bo3"])
def test_swift_generate_matches_oracle(shape, n_skip, acc, per, max_steps, patience, bo_every, seed):
    g = gpu_model(shape)
    o = omodel.Model.synthetic(shape)
    L = shape.n_layers
    P, gamma, n_cand, d, n_gen = 40, 16, 3, 3, 112
    prompt = synth.prompt_tokens(P, shape.vocab)
    init = swift.layers_to_mask(L, swift.uniform_skip_layers(L, n_skip))
    otoks, otr = swift.swift_generate(o, prompt, n_gen, n_skip, gamma, n_cand, per, max_steps, patience, 1.5, d,
                                      seed=seed, bo_every=bo_every, accumulate=acc or None)
    print("oracle: %d iterations, %d phases, steps %d, plans %s" % (
        len(otr["plans"]) - 1, len(otr["phases"]), otr["steps"], [p["after"][::2].tolist() for p in otr["phases"]]))
    ar, ref_z = oracle_ar_with_logits(o, prompt, n_gen)
    assert otoks == ar
    cfg = B.swift_config(gamma, n_skip, n_cand, per, max_steps, patience, 1.5, d, seed, accumulate=acc,
                         bo_every=bo_every)
    toks, nouts, plans, phases, st = _gpu_run(g, shape, prompt, cfg, init, n_gen)
    print("gpu: %d iterations, %d phases, steps %d, plans %s" % (
        len(nouts) - 1, len(phases), st.steps, [p["after"][::2].tolist() for p in phases]))
    check_greedy_tokens(toks, ar, ref_z)
    assert nouts == otr["n_out"]
    assert len(phases) == len(otr["phases"]) >= 2
    kv_cache = {}
    for k, (gp, op) in enumerate(zip(phases, otr["phases"])):
        assert gp["n_out"] == op["n_out"] == gp["last"]
        assert np.array_equal(gp["after"], op["after"]), k
        assert gp["steps"] == op["step0"] + op["steps"]
        # the matchness may differ only by rows that are oracle near-ties (top-2 margin < 1e-2)
        n_out = op["n_out"]
        seq_tokens = list(prompt) + otoks[:n_out - 1 - gamma]
        kv = omodel.KVCache(shape, len(seq_tokens) + 64)
        omodel.forward(o, seq_tokens, range(len(seq_tokens)), kv)
        window = otoks[n_out - 1 - gamma:n_out]
        _, _, _, om = ossd.score_masks(o, kv, window, op["pos0"], [op["after"]], detail=True)
        assert abs(gp["score"] - op["score"]) <= int((om < 1e-2).sum()) / gamma + 1e-7
    for k in range(1, len(plans)):
        assert np.array_equal(plans[k], otr["plans"][k]), k
    assert (st.steps, st.unimproved, bool(st.done)) == (otr["steps"], otr["unimproved"], otr["done"])
    assert st.switches == sum(1 for p in otr["phases"] if not np.array_equal(p["before"], p["after"]))
    # rows for several search steps per scoring pass: the same run, bit for bit
    toks2, nouts2, plans2, phases2, st2 = _gpu_run(g, shape, prompt, cfg, init, n_gen, rows_factor=3)
    assert toks2 == toks and nouts2 == nouts
    assert all(np.array_equal(a, b) for a, b in zip(plans2[1:], plans[1:]))
    assert len(phases2) == len(phases)
    for a, b in zip(phases2, phases):
        assert np.array_equal(a["after"], b["after"]) and a["score"] == b["score"] and a["steps"] == b["steps"]
        assert (a["n_out"], a["unimproved"], a["done"]) == (b["n_out"], b["unimproved"], b["done"])
    assert (st2.steps, st2.unimproved, st2.done, st2.switches) == (st.steps, st.unimproved, st.done, st.switches)
    g.close()


def test_swift_generate_no_optimisation_is_plain_ssd():
    """max_steps = 0: no phase, the plan never changes, and the run commits exactly what plain ssd_draft /
    ssd_verify / ssd_accept / ssd_commit iterations commit with that plan (sampled, confidence stop)."""
    shape = BF16_HD64
    g = gpu_model(shape)
    L = shape.n_layers
    P, d, n_gen = 24, 3, 48
    prompt = synth.prompt_tokens(P, shape.vocab)
    init = swift.layers_to_mask(L, swift.uniform_skip_layers(L, 1))
    cfg = B.swift_config(16, 1, 3, 2, 0, 10, 0.95, d, 9, conf_thresh=0.3, temperature=1.0)
    toks, nouts, plans, phases, st = _gpu_run(g, shape, prompt, cfg, init, n_gen)
    assert phases == [] and st.done == 1 and all(np.array_equal(p, init) for p in plans[1:])
    seq = B.Sequence(g, max_ctx=P + n_gen + 64, max_rows=64, max_draft=d)
    B.ssd_prefill(seq.handle, dev(prompt))
    n_out = 1
    while n_out < n_gen:
        seq.ssd_iteration(init, None, d, conf_thresh=0.3, temperature=1.0, seed=9)
        n_out = B.ssd_read_state(seq.handle).n_out
    ref = [int(x) for x in B.ssd_read_output(seq.handle, n_gen)]
    assert toks == ref
    seq.close()
    g.close()


def test_swift_begin_rejects_bad_configurations():
    shape = BF16_HD64
    g = gpu_model(shape)
    seq = B.Sequence(g, max_ctx=256, max_rows=64, max_draft=3)
    B.ssd_prefill(seq.handle, dev(synth.prompt_tokens(8, shape.vocab)))
    for bad in (dict(gamma=0), dict(n_cand=0), dict(steps_per_phase=0), dict(d=4), dict(n_skip=5),
                dict(gamma=32, n_cand=3)):   # (n_cand + 1) * gamma > max_rows
        kw = dict(gamma=16, n_skip=2, n_cand=3, steps_per_phase=1, max_steps=4, patience=2, target=0.95, d=3, seed=1)
        kw.update(bad)
        with pytest.raises(B.SSDError) as e:
            B.ssd_swift_begin(seq.handle, B.swift_config(**kw))
        assert e.value.code == B.SSD_ERR_ARG
    seq.close()
    g.close()
