"""Benchmark of the self-speculative decoding hot path on one MI355X.

A step is one SSD iteration of the workload: draft (up to d tokens through the
plan's sub-layers, shared final norm + LM head, confidence stop), one verify
pass over the d'+1 rows, accept/reject, commit.  Inputs (weights, prompt, KV
cache after the prefill) are resident in HBM before the timed region.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
                    [--workload 7b|tiny|13b|70b|tree7b|tree13b|score13b|swift13b|swiftotf13b|exit7b]
                    [--search-steps-per-pass N] [--no-cpu-baseline]

Prints one JSON line.  value = committed tokens per second over the K timed
steps (nothing else queued).  roofline = the dominant kernel (the decode-block
gate/up projection with its fused SwiGLU epilogue, 44 % of the weight bytes of a
pass), timed live over the next K steps of the same sequence: each of its
launches carries a pair of HIP events that take the dispatch's own begin and end
timestamps; the verify pass is bracketed by events in those steps too.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0

# HBM traffic of the dominant kernel from rocprofv3 counter runs (FETCH_SIZE and
# WRITE_SIZE in KiB per dispatch, scaled by the factors a plain 1 GiB copy reads
# on the same counters).  Keyed by (kernel, workload): a record holds only for
# the workload (shapes and row counts) it was taken on, and only while the
# kernel source is the one it was taken on; otherwise the line reports null.
# The 7B gate/up launches are two instantiations, one-row blocks (104 per SSD
# step: 12 draft passes and the verify's last row over 8 layers) and 13-row
# verify blocks (24 per step, layers 8..31); the record holds each one's mean
# and the per-launch figure is their mean weighted by that mix.
PMC_TRAFFIC = {
    ("dec_gemm_kernel<DEC_SWIGLU>", "7b"): dict(
        source="self_speculative_layer_amd/csrc/decode.hip", sha1_prefix="a643b1a908b3",
        parts=[dict(launches=104, fetch_kib=88271.4, write_kib=21.5),
               dict(launches=24, fetch_kib=89262.7, write_kib=279.5)],
        fetch_scale=2.0, write_scale=1.0, profile="profiles/dec_7b_hbm_counters.md"),
    # 13B scoring gate/up, every launch of a step (the same masks every step): 23 of 129-256 rows, 12 of
    # 257-384 and 3 of 96-128 (128 x 128 tiles), 2 of at most 64 (64 x 64 tiles)
    ("gemm_bf16_tiled<EPI_SWIGLU, 4, 4>", "score13b"): dict(
        source="self_speculative_layer_amd/csrc/kernels.hip", sha1_prefix="fa9187ef4828",
        parts=[dict(launches=23, fetch_kib=165991.8, write_kib=5484.7),
               dict(launches=12, fetch_kib=215410.4, write_kib=8425.0),
               dict(launches=3, fetch_kib=142613.1, write_kib=2880.0),
               dict(launches=2, fetch_kib=140571.9, write_kib=1301.0)],
        fetch_scale=2.0, write_scale=1.0, profile="profiles/gemm_tiled_score13b_kernel_trace.md"),
}
DOMINANT = "dec_gemm_kernel<DEC_SWIGLU>"
SCORING_DOMINANT = "gemm_bf16_tiled<EPI_SWIGLU, 4, 4>"


def pmc_traffic_bytes(kernel, workload):
    """Measured HBM bytes per launch, or None (no record for this kernel and workload, or the source changed)."""
    import hashlib
    rec = PMC_TRAFFIC.get((kernel, workload))
    if rec is None:
        return None
    with open(os.path.join(ROOT, rec["source"]), "rb") as f:
        if hashlib.sha1(f.read()).hexdigest()[:12] != rec["sha1_prefix"]:
            return None
    parts = rec.get("parts") or [dict(launches=1, fetch_kib=rec["fetch_kib"], write_kib=rec["write_kib"])]
    n = sum(p["launches"] for p in parts)
    return 1024.0 * sum(p["launches"] * (p["fetch_kib"] * rec["fetch_scale"] + p["write_kib"] * rec["write_scale"])
                        for p in parts) / n

WORKLOADS = {
    "7b": dict(shape="llama2-7b-shape", prompt=512, n_gen=256, exit_layer=8, d=12, tau=0.0, T=0.0,
               desc="LLaMA-2-7B-shaped bf16 decoder, LayerSkip early-exit draft E=8, d=12, greedy, "
                    "512-token random prompt, 256 generated tokens, batch 1"),
    "tiny": dict(shape="tiny-f32", prompt=32, n_gen=64, skip_layers=[2], d=4, tau=0.0, T=0.0,
                 desc="tiny fp32 decoder (L4 D256 H4 F688 V1024), draft skips layer 2, d=4, greedy, "
                      "32-token prompt, 64 tokens"),
    "13b": dict(shape="llama2-13b-shape", prompt=1024, n_gen=256, random_skip=20, d=8, tau=0.8, T=1.0,
                desc="LLaMA-2-13B-shaped bf16 decoder, SWIFT skip mask of 20 seeded layers, d<=8, confidence "
                     "stop 0.8, T=1.0 sampling, 1024-token prompt, 256 tokens"),
    "tree7b": dict(shape="llama2-7b-shape", prompt=512, n_gen=256, exit_layer=8, d=12, tau=0.0, T=0.0,
                   tree=dict(rho=0.9, k_max=4, max_leaves=3),
                   desc="LLaMA-2-7B-shaped bf16 decoder, LayerSkip early-exit draft E=8, d=12, greedy, with SWIFT "
                        "dynamic verification: each draft step's top-k candidates (k from the top-k mass reaching "
                        "0.9, k <= 4) verified as leaves beside the chain, at most 3 leaves (16 verify rows); "
                        "512-token random prompt, batch 1"),
    "tree13b": dict(shape="llama2-13b-shape", prompt=1024, n_gen=256, random_skip=20, d=8, tau=0.8, T=1.0,
                    tree=dict(rho=0.9, k_max=4, max_leaves=7),
                    desc="LLaMA-2-13B-shaped bf16 decoder, SWIFT skip mask of 20 seeded layers, d<=8, confidence "
                         "stop 0.8, T=1.0 sampling, with sampled draft trees: each draft step's extra candidates "
                         "(k from the top-k mass of softmax(z/T) reaching 0.9, k <= 4) drawn from the draft "
                         "distribution and verified as leaves, at most 7 leaves (16 verify rows); 1024-token prompt"),
    "70b": dict(shape="llama2-70b-shape", prompt=4096, n_gen=128, random_skip=40, d=8, tau=0.0, T=0.0,
                desc="LLaMA-2-70B-shaped bf16 decoder (GQA 64/8), SWIFT skip mask of 40 seeded layers, d=8, "
                     "greedy, 4096-token prompt, 128 tokens"),
}


SCORING = {
    "score13b": dict(shape="llama2-13b-shape", prompt=1024, gamma=32, n_masks=16, skip_lo=16, skip_hi=24,
                     desc="LLaMA-2-13B-shaped bf16 decoder, SWIFT matchness scoring of 16 seeded candidate plans "
                          "(16-24 of 40 layers skipped each) over a 32-token window greedily generated after a "
                          "1024-token random prompt"),
    "swift13b": dict(shape="llama2-13b-shape", prompt=1024, gamma=32, n_masks=16, skip_lo=20, skip_hi=20, search=True,
                     desc="LLaMA-2-13B-shaped bf16 decoder, SWIFT random search: 15 proposals of 20 skipped layers per "
                          "step scored on a 32-token window greedily generated after a 1024-token random prompt, "
                          "starting from the uniform plan"),
}


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def plan_of(wl, shape):
    import synth
    if "exit_layer" in wl:
        return None, wl["exit_layer"], synth.mask_exit(shape.n_layers, wl["exit_layer"])
    if "skip_layers" in wl:
        m = synth.mask_from_layers(shape.n_layers, wl["skip_layers"])
        return m, None, m
    layers = synth.random_skip_layers(shape.n_layers, wl["random_skip"], synth.SEED_MASKS, 0)
    m = synth.mask_from_layers(shape.n_layers, layers)
    return m, None, m


def verify_bytes(shape, kvlen, rows, b):
    """Algorithmic HBM bytes of one verify pass: every layer's weights once, the
    LM head once, each layer's cached keys/values once, the new K/V written."""
    elt = 2 if shape.dtype == "bf16" else 4
    w = shape.n_layers * shape.layer_param_count() * elt + shape.vocab * shape.d_model * elt
    kv_tok = 2 * shape.kv_dim * elt
    kv = shape.n_layers * (kvlen + rows) * kv_tok + shape.n_layers * rows * kv_tok
    return w + kv


def read_ceiling_gbps(torch, B, nbytes=1 << 33, reps=5):
    """A measured streaming-read ceiling of this GPU: the best of `reps` launches of
    the library's read probe over an 8 GiB buffer (each byte read once)."""
    x = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    sink = torch.zeros(2048, dtype=torch.int32, device="cuda")
    best = float("inf")
    for _ in range(reps + 1):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        B.ssd_probe_read(x, nbytes, sink)
        b.record()
        torch.cuda.synchronize()
        best = min(best, a.elapsed_time(b))
    del x
    torch.cuda.empty_cache()
    return nbytes / (best / 1e3) / 1e9


def host_cpu():
    """The host's CPU model, its logical CPU count, and the threads the oracle's BLAS runs."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = os.cpu_count()
    return model, os.cpu_count(), threads


def cpu_baseline(shape, wl, mask, max_seconds=20.0):
    """The oracle as it stands, timed on this host on the workload itself: the prefill of the workload's own
    prompt (timed apart), then SSD iterations of the same plan from there until about max_seconds have
    passed (at most 64)."""
    import numpy as np
    import synth
    from oracle import model as omodel
    from oracle import ssd as ossd
    cpu_model, n_cpus, threads = host_cpu()
    need = shape.param_count() * 8
    mem = os.sysconf("SC_PAGE_SIZE") * os.sysconf("SC_PHYS_PAGES")
    if need > 0.6 * mem:
        return {"value": None, "unit": "tokens/s", "cores": threads, "kind": "oracle", "cpu_model": cpu_model,
                "sample": "not run: the oracle's float64 weights (%.0f GB) exceed 60%% of host RAM (%.0f GB)"
                          % (need / 1e9, mem / 1e9)}
    t0 = time.time()
    om = omodel.Model.synthetic(shape)
    log("oracle weights built in %.1fs" % (time.time() - t0))
    P, d = wl["prompt"], wl["d"]
    prompt = synth.prompt_tokens(P, shape.vocab)            # the GPU run's prompt
    kv = omodel.KVCache(shape, P + 64 * (d + 2) + 8)
    t0 = time.time()
    z = ossd.prefill(om, kv, prompt)
    prefill_s = time.time() - t0
    log("oracle prefill of %d tokens: %.1f s" % (P, prefill_s))
    out = [ossd.pick(z, wl["T"], synth.SEED_SAMPLING, 0, 0, 2)]
    b = omodel.first_skipped_layer(mask, shape.n_layers)
    tokens, iters = 0, 0
    t0 = time.time()
    while True:
        n = P + len(out)
        drafts, zq, hb = ossd.draft(om, kv, out[-1], n, mask, d, wl["tau"], wl["T"], synth.SEED_SAMPLING, iters + 1)
        if "tree" in wl:
            from oracle import tree as otree
            tr = wl["tree"]
            if wl["T"] == 0:
                leaves = otree.tree_leaves(zq, drafts, tr["rho"], tr["k_max"], tr["max_leaves"])
            else:
                leaves = otree.tree_leaves_sampled(zq, drafts, wl["T"], tr["rho"], tr["k_max"], tr["max_leaves"],
                                                   synth.SEED_SAMPLING, iters + 1)
            zp, zl = otree.verify_tree(om, kv, out[-1], drafts, leaves, n, b, hb)
            if wl["T"] == 0:
                em, s = otree.accept_tree_greedy(zp, zl, drafts, leaves)
            else:
                em, s = otree.accept_tree_sampled(zp, zq, zl, drafts, leaves, wl["T"], synth.SEED_SAMPLING, iters + 1)
            if s is not None:
                j, c = leaves[s]
                omodel.forward(om, [out[-1]] + [int(t) for t in drafts[: j - 1]] + [c], list(range(n - 1, n + j)), kv)
        else:
            zp = ossd.verify(om, kv, out[-1], drafts, n, b, hb)
            em = ossd.accept_greedy(zp, drafts) if wl["T"] == 0 else ossd.accept_sampled(
                zp, zq, drafts, wl["T"], synth.SEED_SAMPLING, iters + 1)
        out.extend(em)
        tokens += len(em)
        iters += 1
        if time.time() - t0 > max_seconds or iters >= 64:
            break
    dt = time.time() - t0
    return {"value": tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "%d SSD iterations (%d committed tokens) of the same %s model, plan and seeded %d-token prompt "
                      "as the GPU run, right after the prompt's prefill (%.1f s, not counted), float64 NumPy oracle "
                      "with %d BLAS threads, %.1f s" % (iters, tokens, shape.name, P, prefill_s, threads, dt),
            "prefill_s": round(prefill_s, 2), "cpu_model": cpu_model, "host_logical_cpus": n_cpus}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="default 64 (SSD steps), 8 (scoring steps)")
    ap.add_argument("--warmup", type=int, default=None, help="default 8 (SSD steps), 2 (scoring steps)")
    ap.add_argument("--workload", default="7b",
                    choices=sorted(WORKLOADS) + sorted(SCORING) + ["exit7b", "swiftotf13b"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--ar-steps", type=int, default=16)
    ap.add_argument("--search-steps-per-pass", type=int, default=8,
                    help="swift13b / swiftotf13b: search steps scored together in one pass (the rows allotted)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": src.numel() * 4, "copy_bytes_written": dst.numel() * 4}))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: it runs one sequence on one MI355X; --gpus %d is not supported"
              % args.gpus)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    from synth import device as sdev
    from self_speculative_layer_amd import binding as B

    if args.workload == "swiftotf13b":
        args.steps = 8 if args.steps is None else args.steps
        args.warmup = 0 if args.warmup is None else args.warmup
        run_swift_otf(args)
        return
    if args.workload == "exit7b":
        args.steps = 64 if args.steps is None else args.steps
        args.warmup = 8 if args.warmup is None else args.warmup
        run_exit(args)
        return
    if args.workload in SCORING:
        args.steps = 8 if args.steps is None else args.steps
        args.warmup = 2 if args.warmup is None else args.warmup
        run_scoring(args)
        return
    args.steps = 64 if args.steps is None else args.steps
    args.warmup = 8 if args.warmup is None else args.warmup
    wl = WORKLOADS[args.workload]
    shape = synth.SHAPES[wl["shape"]]
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    t0 = time.time()
    tensors = sdev.build_weights(shape)
    torch.cuda.synchronize()
    log("weights on device in %.1fs (%.2f GB)" % (time.time() - t0, shape.param_count() * (2 if shape.dtype == "bf16" else 4) / 1e9))
    model = B.Model(shape.n_layers, shape.d_model, shape.n_heads, shape.n_kv_heads, shape.head_dim, shape.ffn_dim,
                    shape.vocab, shape.dtype, tensors)
    skip_mask, exit_layer, mask = plan_of(wl, shape)
    d = wl["d"]
    K, W = args.steps, args.warmup
    max_ctx = wl["prompt"] + (3 * K + W + 2) * (d + 1) + 64
    seq = B.Sequence(model, max_ctx=max_ctx, max_rows=512, max_draft=max(d, 1), device=dev)
    prompt = torch.from_numpy(synth.prompt_tokens(wl["prompt"], shape.vocab)).to(dev)
    seed = synth.SEED_SAMPLING
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    B.ssd_prefill(seq.handle, prompt, wl["T"], seed)
    ev1.record()
    torch.cuda.synchronize()
    prefill_ms = ev0.elapsed_time(ev1)
    log("prefill %d tokens: %.1f ms" % (wl["prompt"], prefill_ms))

    tr = wl.get("tree")

    def iteration(vev=None, dev_=None):
        h = seq.handle
        if dev_ is not None:
            dev_[0].record()
        B.ssd_draft(h, skip_mask, exit_layer, d, wl["tau"], wl["T"], seed, seq.draft_tokens, seq.draft_logits,
                    seq.n_drafted)
        if dev_ is not None:
            dev_[1].record()
        if tr is not None:
            # dynamic verification: leaves from the draft's confidence, one tree verify, tree acceptance
            B.ssd_tree_candidates(h, seq.draft_logits, seq.n_drafted, d, tr["rho"], tr["k_max"], tr["max_leaves"],
                                  seq.leaf_tokens, seq.leaf_depth, seq.n_leaves, wl["T"], seed)
            if vev is not None:
                vev[0].record()
            B.ssd_verify_tree(h, skip_mask, exit_layer, d, seq.draft_tokens, seq.n_drafted, seq.leaf_tokens,
                              seq.leaf_depth, seq.n_leaves, tr["max_leaves"], True, seq.tree_logits)
            if vev is not None:
                vev[1].record()
            B.ssd_accept_tree(h, seq.tree_logits, seq.draft_tokens, seq.n_drafted, d, seq.leaf_tokens,
                              seq.leaf_depth, seq.n_leaves, tr["max_leaves"], seq.out_tokens, seq.n_out,
                              seq.draft_logits, wl["T"], seed)
            B.ssd_commit(h, seq.out_tokens, seq.n_out)
            return
        if vev is not None:
            vev[0].record()
        B.ssd_verify(h, skip_mask, exit_layer, d, seq.draft_tokens, seq.n_drafted, True, seq.verify_logits)
        if vev is not None:
            vev[1].record()
        B.ssd_accept(h, seq.verify_logits, seq.draft_logits, seq.draft_tokens, seq.n_drafted, d, wl["T"], seed,
                     seq.out_tokens, seq.n_out)
        B.ssd_commit(h, seq.out_tokens, seq.n_out)

    for _ in range(W):
        iteration()
    st0 = B.ssd_read_state(seq.handle)
    # timed region: K steps with nothing queued but the steps themselves
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    ev0.record()
    for k in range(K):
        iteration()
    ev1.record()
    torch.cuda.synchronize()
    t_end = time.perf_counter()
    st1 = B.ssd_read_state(seq.handle)
    elapsed_ms = ev0.elapsed_time(ev1)
    wall_ms = (t_end - t_start) * 1e3
    tokens = st1.n_out - st0.n_out
    value = tokens / (elapsed_ms / 1e3)
    # measured region: the next K steps of the same sequence, with the dominant kernel's launches carrying
    # dispatch timestamp events and the verify pass bracketed by events (both slow the stream slightly,
    # so they stay out of the timed region)
    vevs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    per_iter_swiglu = d * shape.n_layers + shape.n_layers
    B.ssd_profile_enable(B.SSD_PROF_GEMM_SWIGLU, K * per_iter_swiglu + 8)
    for k in range(K):
        iteration(vevs[k])
    torch.cuda.synchronize()
    B.ssd_profile_disable()
    st2 = B.ssd_read_state(seq.handle)
    prof_ms, prof_n, prof_bytes = B.ssd_profile_read()
    verify_ms = [a.elapsed_time(b) for a, b in vevs]
    # context during the measured steps (for the verify byte count): its mean kvlen
    kv_mid = (st1.kvlen + st2.kvlen) / 2.0
    b = int(np.argmax(mask.reshape(-1, 2).any(axis=1))) if mask.any() else shape.n_layers
    vrows = d + 1 + (tr["max_leaves"] if tr is not None else 0)
    vb = verify_bytes(shape, kv_mid, vrows, b)
    vmed = float(np.median(verify_ms))
    log("timed %d steps: %.1f ms (wall %.1f ms), %d tokens -> %.1f tok/s; verify median %.3f ms" %
        (K, elapsed_ms, wall_ms, tokens, value, vmed))
    achieved = prof_bytes / (prof_ms / 1e3) / 1e9 if prof_ms > 0 else 0.0

    # statistics pass: K more steps, each followed by a state read (d' and the emitted count), with the draft
    # phase bracketed by events (SWIFT digest §B.3: M = tokens per verify, alpha = accepted-draft fraction)
    dps, ems, draft_ms = [], [], []
    for k in range(K):
        dv = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        iteration(dev_=dv)
        st = B.ssd_read_state(seq.handle)
        dps.append(st.last_n_drafted)
        ems.append(st.last_n_emitted)
        draft_ms.append(dv[0].elapsed_time(dv[1]))
    dps, ems, draft_ms = np.array(dps), np.array(ems), np.array(draft_ms)
    acc = np.minimum(ems - 1, dps)

    # same-kernel AR decode baseline
    ar_tps = None
    if args.ar_steps > 0:
        seq2 = B.Sequence(model, max_ctx=wl["prompt"] + args.ar_steps + 64, max_rows=512, max_draft=1, device=dev)
        B.ssd_prefill(seq2.handle, prompt, wl["T"], seed)
        for _ in range(2):
            B.ssd_decode_ar(seq2.handle, wl["T"], seed)
        torch.cuda.synchronize()
        ev0.record()
        for _ in range(args.ar_steps):
            B.ssd_decode_ar(seq2.handle, wl["T"], seed)
        ev1.record()
        torch.cuda.synchronize()
        ar_tps = args.ar_steps / (ev0.elapsed_time(ev1) / 1e3)
        seq2.close()

    traffic = pmc_traffic_bytes(DOMINANT, args.workload)
    if traffic is not None:
        traffic = round(traffic)
    ceiling = read_ceiling_gbps(torch, B)
    log("measured streaming-read ceiling %.0f GB/s" % ceiling)
    result = {
        "metric": "accepted tokens/s (batch 1) + verify-pass HBM GB/s vs MI355X peak",
        "value": round(value, 3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(elapsed_ms / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if shape.dtype == "bf16" else "f32",
        "data": "synthetic (seeded random-init weights and uniform random prompt)",
        "config": {"workload": wl["desc"], "prompt_len": wl["prompt"], "d": d, "conf_thresh": wl["tau"],
                   "temperature": wl["T"], "batch": 1, "step": "one SSD iteration (draft + verify + accept + commit)"
                   if tr is None else "one SSD iteration (draft + tree candidates + tree verify + tree accept + "
                                      "commit)"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "measured": "dispatch-timestamp events on every launch of the kernel in %d further steps "
                                 "of the same sequence" % K,
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "frac_of_measured_ceiling": round(achieved / ceiling, 4),
                     "kernel": DOMINANT + " (decode-block gate/up projection + SwiGLU)",
                     "launches": prof_n, "avg_launch_us": round(prof_ms / max(prof_n, 1) * 1e3, 3),
                     "bytes_per_launch": round(prof_bytes / max(prof_n, 1))},
        "measured_read_ceiling_GBps": round(ceiling, 1),
        "verify": {"median_ms": round(vmed, 4), "algorithmic_GB": round(vb / 1e9, 4),
                   "frac_of_measured_ceiling": round(vb / (vmed / 1e3) / 1e9 / ceiling, 4),
                   "GBps": round(vb / (vmed / 1e3) / 1e9, 1),
                   "frac_of_peak": round(vb / (vmed / 1e3) / 1e9 / HBM_PEAK_GBPS, 4)},
        "mean_tokens_per_step": round(tokens / K, 4),
        "ssd_stats": {"steps": K, "M_tokens_per_verify": round(float(ems.mean()), 4),
                      "alpha_accepted_fraction": round(float(acc.sum() / max(dps.sum(), 1)), 4),
                      "d_prime_histogram": np.bincount(dps, minlength=d + 1).tolist(),
                      "draft_phase_ms_median": round(float(np.median(draft_ms)), 4),
                      "draft_ms_per_drafted_token": round(float(np.median(draft_ms / np.maximum(dps, 1))), 4),
                      "c_draft_token_over_ar_token": (None if ar_tps is None else
                                                      round(float(np.median(draft_ms / np.maximum(dps, 1)))
                                                            / (1e3 / ar_tps), 4)),
                      "measured": "%d further steps of the same sequence, a state read after each" % K},
        "ar_tokens_per_s": None if ar_tps is None else round(ar_tps, 3),
        "prefill_ms": round(prefill_ms, 2),
        "wall_ms_timed": round(wall_ms, 2),
        # what the pages report for trained models (context, not the target); under random weights the full
        # model almost never repeats a draft, so SSD runs below AR here
        "pages_context": {
            "swift_speedup_over_ar": "1.3-1.6x, LLaMA-2 and CodeLLaMA (SWIFT digest, section 5.2 and Table 2)",
            "layerskip_speedup_over_ar": "up to 2.16x (LayerSkip blog, title)",
            "hardware": "not named in the pages' text",
            "measured_ssd_over_ar": None if ar_tps is None else round(value / ar_tps, 4)},
    }
    seq.close()
    model.close()
    del tensors
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(shape, wl, mask)
    print(json.dumps(result), flush=True)


def run_exit(args):
    """Lossy early-exit decoding (no verification): one step = one token through
    layers 0..7 of the 7B shape, the shared final norm and LM head."""
    import numpy as np
    import torch

    import synth
    from synth import device as sdev
    from self_speculative_layer_amd import binding as B

    shape = synth.LLAMA7B
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    tensors = sdev.build_weights(shape)
    model = B.Model(shape.n_layers, shape.d_model, shape.n_heads, shape.n_kv_heads, shape.head_dim, shape.ffn_dim,
                    shape.vocab, shape.dtype, tensors)
    K, W, E, P = args.steps, args.warmup, 8, 512
    seq = B.Sequence(model, max_ctx=P + K + W + 64, max_rows=512, max_draft=1, device=dev)
    B.ssd_prefill(seq.handle, torch.from_numpy(synth.prompt_tokens(P, shape.vocab)).to(dev))
    for _ in range(W):
        B.ssd_decode_exit(seq.handle, None, E)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(K):
        B.ssd_decode_exit(seq.handle, None, E)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / K
    B.ssd_profile_enable(B.SSD_PROF_GEMM_SWIGLU, K * E + 8)
    for _ in range(K):
        B.ssd_decode_exit(seq.handle, None, E)
    torch.cuda.synchronize()
    B.ssd_profile_disable()
    prof_ms, prof_n, prof_bytes = B.ssd_profile_read()
    achieved = prof_bytes / (prof_ms / 1e3) / 1e9 if prof_ms > 0 else 0.0
    step_bytes = E * shape.layer_param_count() * 2 + shape.vocab * shape.d_model * 2
    # SpecEE exit features of one hidden row for 4 speculative tokens (latency-bound: 4 x 8 KB of LM-head rows)
    hrow = torch.randn(1, shape.d_model, device=dev)
    toks = torch.tensor([5, 77, 1234, 31999], dtype=torch.int32, device=dev)
    feats = torch.zeros(1, 12, device=dev)
    for _ in range(3):
        B.ssd_specee_features(model.handle, hrow, 1, toks, 4, None, feats)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(100):
        B.ssd_specee_features(model.handle, hrow, 1, toks, 4, None, feats)
    ev1.record()
    torch.cuda.synchronize()
    feat_us = ev0.elapsed_time(ev1) * 10.0
    result = {
        "metric": "lossy early-exit tokens/s (batch 1, exit at layer 8, no verification)",
        "value": round(1e3 / ms, 3), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded random-init weights and uniform random prompt)",
        "config": {"workload": "LLaMA-2-7B-shaped bf16 decoder, lossy early exit at E=8, greedy, 512-token prompt"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None,
                     "kernel": DOMINANT + " (decode-block gate/up projection + SwiGLU)", "launches": prof_n,
                     "avg_launch_us": round(prof_ms / max(prof_n, 1) * 1e3, 3)},
        "step_GBps": round(step_bytes / (ms / 1e3) / 1e9, 1),
        "specee_features_us": round(feat_us, 2),
    }
    seq.close()
    model.close()
    print(json.dumps(result), flush=True)


def run_swift_otf(args):
    """SWIFT on the fly (ssd_swift_generate): self-speculative iterations with the plan in use and, after every
    32 committed tokens, an optimisation phase of at most 8 search steps (15 proposals each) on the last 33
    committed tokens; one step = one call generating 32 tokens (its iterations and the phase that follows)."""
    import numpy as np
    import torch

    import synth
    from synth import device as sdev
    from self_speculative_layer_amd import binding as B

    shape = synth.LLAMA13B
    L = shape.n_layers
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    tensors = sdev.build_weights(shape)
    model = B.Model(shape.n_layers, shape.d_model, shape.n_heads, shape.n_kv_heads, shape.head_dim, shape.ffn_dim,
                    shape.vocab, shape.dtype, tensors)
    K, W, P, gamma, n_skip, n_cand, per, d = args.steps, args.warmup, 1024, 32, 20, 15, 8, 8
    n_gen = (K + W) * gamma
    # rows for the search steps scored together in one pass
    spp = args.search_steps_per_pass
    seq = B.Sequence(model, max_ctx=P + n_gen + 64, max_rows=(spp * n_cand + 1) * gamma, max_draft=d, device=dev)
    B.ssd_prefill(seq.handle, torch.from_numpy(synth.prompt_tokens(P, shape.vocab)).to(dev), 1.0,
                  synth.SEED_SAMPLING)
    cfg = B.swift_config(gamma, n_skip, n_cand, per, 1000, 300, 0.95, d, synth.SEED_SAMPLING, bo_every=25,
                         conf_thresh=0.8, temperature=1.0)
    st = B.ssd_swift_begin(seq.handle, cfg)
    plan = np.ascontiguousarray(B.ssd_uniform_mask(L, n_skip))

    def call():
        B.ssd_swift_generate(seq.handle, cfg, st, plan, gamma, seq.draft_tokens, seq.draft_logits, seq.n_drafted,
                             seq.verify_logits, seq.out_tokens, seq.n_out)

    for _ in range(W):
        call()
    s0 = B.ssd_read_state(seq.handle)
    it0, ph0, steps0 = st.iterations, st.phases, st.steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        call()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    s1 = B.ssd_read_state(seq.handle)
    tokens = s1.n_out - s0.n_out
    result = {
        "metric": "committed tokens/s (batch 1) with SWIFT's on-the-fly layer-set optimisation",
        "value": round(tokens / wall, 3), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(wall * 1e3 / K, 3), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded random-init weights and uniform random prompt)",
        "config": {"workload": "LLaMA-2-13B-shaped bf16 decoder, SWIFT on the fly: uniform start plan of 20 skipped "
                               "layers, a phase of <= 8 search steps (15 proposals of 20 layers, Bayesian step "
                               "every 25 steps) after every 32 committed tokens on the last 33, d<=8, confidence "
                               "stop 0.8, T=1.0, 1024-token random prompt",
                   "step": "one ssd_swift_generate call of 32 tokens (its iterations and the phase after them)",
                   "search_steps_per_pass": spp},
        "timing": "wall clock around the calls (each iteration and each optimisation step synchronises the stream)",
        "tokens": tokens, "iterations": st.iterations - it0,
        "M_tokens_per_iteration": round(tokens / max(st.iterations - it0, 1), 3),
        "phases": st.phases - ph0, "optimisation_steps": st.steps - steps0, "switches": st.switches,
        "final_score": None if st.score != st.score else round(float(st.score), 4), "optimisation_done": bool(st.done),
        "final_plan_layers": [int(l) for l in np.nonzero(plan[::2])[0]],
    }
    seq.close()
    model.close()
    print(json.dumps(result), flush=True)


def run_scoring(args):
    """One step = one ssd_score_masks call: every candidate plan's draft over the
    window rows in one batched pass (rows of the candidates that keep a sub-layer
    go through it together), the LM head, row statistics and the matchness
    scores.  The dominant kernel is the batched gate/up projection; its
    launches are timed with dispatch events in K further steps."""
    import numpy as np
    import torch

    import synth
    from synth import device as sdev
    from self_speculative_layer_amd import binding as B

    wl = SCORING[args.workload]
    shape = synth.SHAPES[wl["shape"]]
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    t0 = time.time()
    tensors = sdev.build_weights(shape)
    torch.cuda.synchronize()
    log("weights on device in %.1fs" % (time.time() - t0))
    model = B.Model(shape.n_layers, shape.d_model, shape.n_heads, shape.n_kv_heads, shape.head_dim, shape.ffn_dim,
                    shape.vocab, shape.dtype, tensors)
    P, gamma, nm = wl["prompt"], wl["gamma"], wl["n_masks"]
    masks = synth.scoring_masks(shape.n_layers, nm, wl["skip_lo"], wl["skip_hi"])
    search = wl.get("search", False)
    # the search scores a step together with the random steps after it while the rows allow: room for
    # --search-steps-per-pass steps per scoring pass, and one call runs that many steps
    per_call = args.search_steps_per_pass if search else 1
    seq = B.Sequence(model, max_ctx=P + gamma + 64, max_rows=(per_call * (nm - 1) + 1) * gamma, max_draft=1,
                     device=dev)
    prompt = torch.from_numpy(synth.prompt_tokens(P, shape.vocab)).to(dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    B.ssd_prefill(seq.handle, prompt)
    ev1.record()
    torch.cuda.synchronize()
    prefill_ms = ev0.elapsed_time(ev1)
    for _ in range(gamma - 1):
        B.ssd_decode_ar(seq.handle, 0.0, 0)
    gen = B.ssd_read_output(seq.handle, gamma)
    window = torch.tensor([int(prompt[-1])] + [int(x) for x in gen], dtype=torch.int32, device=dev)
    scores = torch.zeros(nm, dtype=torch.float32, device=dev)
    best = torch.zeros(1, dtype=torch.int32, device=dev)

    n_skip = wl["skip_lo"]
    init = B.ssd_uniform_mask(shape.n_layers, n_skip)
    search_out = {}

    used = []                                     # the masks each call scored

    def step():
        if search:
            # per_call search steps per call, scored in one pass (step 0: the starting plan and 15 proposals,
            # each later step 15 more; a new seed each call; no stop rule can end the call early)
            sd = synth.SEED_MASKS + len(used)
            bm, bs, ns = B.ssd_swift_search(seq.handle, window, P - 1, gamma, init, n_skip, nm - 1, per_call, 1000,
                                            2.0, sd, shape.n_layers)
            assert ns == per_call
            search_out.update(best=bm, score=bs)
            used.append(np.stack([init] + [B.ssd_swift_propose(shape.n_layers, n_skip, sd, st, c)
                                           for st in range(per_call) for c in range(nm - 1)]))
        else:
            B.ssd_score_masks(seq.handle, masks, window, P - 1, gamma, scores, best)
            used.append(masks)

    K, W = args.steps, args.warmup
    for _ in range(W):
        step()
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(K):
        step()
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / K / per_call          # per scoring step (search: per search step)
    # measured region: the batched gate/up launches with dispatch events
    B.ssd_profile_enable(B.SSD_PROF_GEMM_SWIGLU, K * shape.n_layers + 8)
    n_before = len(used)
    for _ in range(K):
        step()
    torch.cuda.synchronize()
    B.ssd_profile_disable()
    prof_ms, prof_n, prof_bytes = B.ssd_profile_read()
    D, F = shape.d_model, shape.ffn_dim
    flops = 0.0
    for mk in used[n_before:]:
        # a sub-layer runs once per class of candidates that run it with equal plans before it
        for sl in range(1, mk.shape[1], 2):               # each layer's MLP
            classes = {mk[c, :sl].tobytes() for c in range(mk.shape[0]) if mk[c, sl] == 0}
            flops += 2.0 * (len(classes) * gamma) * 2 * F * D
    gu_ms = prof_ms
    tflops = flops / (gu_ms / 1e3) / 1e12 if gu_ms > 0 else 0.0
    gbps = prof_bytes / (gu_ms / 1e3) / 1e9 if gu_ms > 0 else 0.0
    ai = flops / prof_bytes if prof_bytes > 0 else 0.0
    mfma_bound = ai * HBM_PEAK_GBPS * 1e9 > 2.5e15          # above the bf16 ridge: compute-bound
    log("%s step %.2f ms; gate/up launches %d, %.1f us avg, %.1f TFLOP/s, %.0f GB/s (AI %.0f flop/B)"
        % ("search" if search else "scoring", ms, prof_n, prof_ms / max(prof_n, 1) * 1e3, tflops, gbps, ai))
    roof = ({"bound": "mfma", "achieved": round(tflops, 1), "peak": 2500.0, "unit": "TFLOP/s",
             "frac": round(tflops / 2500.0, 4)} if mfma_bound else
            {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
             "frac": round(gbps / HBM_PEAK_GBPS, 4)})
    traffic = pmc_traffic_bytes(SCORING_DOMINANT, args.workload)
    roof.update({"traffic": None if traffic is None else round(traffic),
                 "kernel": SCORING_DOMINANT + " (gate/up + SwiGLU over the candidates' rows: 128 x 128 tiles, 64 x 64 below "
                           "96 rows)",
                 "launches": prof_n, "avg_launch_us": round(prof_ms / max(prof_n, 1) * 1e3, 3),
                 "flop_per_step": flops / K / per_call, "bytes_per_launch": round(prof_bytes / max(prof_n, 1)),
                 "measured": "dispatch-timestamp events on every launch of the kernel in %d further steps" % K})
    result = {
        "metric": ("SWIFT search steps/s (15 proposals x 32-token window; %d steps per call and scoring pass)"
                   % per_call if search else
                   "mask-scoring steps/s (16 candidate plans x 32-token window)"),
        "value": round(1e3 / ms, 4), "unit": "steps/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms, 3), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded random-init weights, uniform random prompt, seeded masks)",
        "config": {"workload": wl["desc"], "prompt_len": P, "gamma": gamma, "n_masks": nm},
        "roofline": roof,
        "scores": ([round(search_out.get("score", 0.0), 5)] if search else [round(float(x), 5) for x in scores.cpu()]),
        "best": (np.nonzero(search_out["best"][::2])[0].tolist() if search else int(best.item())),
        "prefill_ms": round(prefill_ms, 2),
    }
    if search:
        result["search_steps_per_call"] = per_call
        result["ms_per_call"] = round(ms * per_call, 3)
    if search:
        # a 26-step search with and without its Bayesian-optimisation step at step 25 (the pages' interval):
        # the difference is the host's GP fit and ranking of the 120-plan pool on 256 observations
        times = {}
        for bo in (0, 25):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            B.ssd_swift_search(seq.handle, window, P - 1, gamma, init, n_skip, nm - 1, 26, 1000, 2.0,
                               synth.SEED_MASKS, shape.n_layers, bo_every=bo)
            times[bo] = (time.perf_counter() - t0) * 1e3
        result["search_26_steps_ms"] = {"random": round(times[0], 2), "with_bo_step_25": round(times[25], 2)}
        log("26-step search: %.1f ms random, %.1f ms with the BO step" % (times[0], times[25]))
    seq.close()
    model.close()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
