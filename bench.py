#!/usr/bin/env python3
"""Throughput of the DFlash draft+verify step on one MI355X.

One step = drafter pass over a block of B slots + benchmark draft injection +
target verify of the block + longest-prefix accept + KV commit, captured once
as a hipGraph and replayed.  Workload (default): the 8B-class pair -- W4A16
group-64 target (36 layers, hidden 4096, 32/8 heads, FFN 12288, vocab
151936) with a 5-layer W8A16 drafter, block 32, committed context 2048,
seeded random-init weights drawn on the device, uniform-random prompt, and
injected acceptance (k = min(K, 31), K geometric of mean 23.125, so 17.9
tokens per step on average).

Prints ONE JSON line: steps/s (value), tokens/s, the roofline of the dominant
GEMM kernel variant (HIP-event timing of every launch in an eager profiled
pass), step-level HBM fraction, and the CPU oracle timed on a bounded sample.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_FP16_PEAK_TFLOPS = 2500.0      # dense fp16 MFMA (the int4 GEMMs multiply fp16)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def gemm_shapes(cfg):
    """(name, fmt, N, K, times streamed per step) of every linear of one step."""
    t, d = cfg.target, cfg.drafter
    out = []
    for l, kind in enumerate(t.kinds()):
        qkv_n = t.qkv_rows if kind == 0 else t.gdn_rows
        o_k = t.n_q_heads * t.head_dim if kind == 0 else t.gdn_heads * t.gdn_dv
        out += [("t_qkv", t.fmt, qkv_n, t.hidden, 1), ("t_o", t.fmt, t.hidden, o_k, 1),
                ("t_gu", t.fmt, 2 * t.ffn, t.hidden, 1), ("t_down", t.fmt, t.hidden, t.ffn, 1)]
    for l in range(d.n_layers):
        out += [("d_qkv", d.fmt, d.qkv_rows, d.hidden, 1), ("d_o", d.fmt, d.hidden, d.n_q_heads * d.head_dim, 1),
                ("d_gu", d.fmt, 2 * d.ffn, d.hidden, 1), ("d_down", d.fmt, d.hidden, d.ffn, 1)]
    out.append(("fc", d.fmt, d.hidden, len(cfg.sel_layers) * t.hidden, 1))
    out.append(("lm", t.fmt, t.vocab, t.hidden, 2))     # draft and verify both stream the lm-head
    return out


def weight_bytes_per_step(cfg):
    from dflash_block_diffusion_amd import binding as bn
    from ctypes import byref, c_size_t
    tot = 0
    for _, fmt, n, k, times in gemm_shapes(cfg):
        wb, sb = c_size_t(), c_size_t()
        bn.check(bn.lib().dflash_packed_bytes(fmt, n, k, byref(wb), byref(sb)))
        tot += (wb.value + sb.value) * times
    return tot


def kv_bytes_per_step(cfg, n):
    t, d = cfg.target, cfg.drafter
    eb = 4 if t.fmt == 0 else 2
    l_attn = sum(1 for k in t.kinds() if k == 0)
    kv = n * 2 * t.n_kv_heads * t.head_dim * eb * l_attn + n * 2 * d.n_kv_heads * d.head_dim * eb * d.n_layers
    n_gdn = sum(1 for k in t.kinds() if k == 1)
    gdn = 3 * n_gdn * t.gdn_heads * t.gdn_dv * t.gdn_dk * 4     # verify read, replay read + write
    return kv + gdn


def committed_traffic(kernel):
    """HBM bytes per launch of `kernel` from the rocprofv3 counter summary
    under profiles/, or None when there is none or the kernel sources have
    changed since the counters were taken."""
    import glob
    import hashlib
    for f in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        kv = {}
        hashes = []
        for line in open(f):
            line = line.strip()
            if ":" not in line:
                continue
            key, val = (t.strip() for t in line.split(":", 1))
            if key == "sources_sha256":
                hashes.append(val.split())
            else:
                kv[key] = val
        if kv.get("kernel") != kernel or "traffic_bytes_per_launch" not in kv or not hashes:
            continue
        ok = True
        for name, digest in hashes:
            path = os.path.join(ROOT, "dflash_block_diffusion_amd", "csrc", name)
            if not os.path.exists(path) or hashlib.sha256(open(path, "rb").read()).hexdigest() != digest:
                ok = False
        if ok:
            return float(kv["traffic_bytes_per_launch"])
    return None


def cpu_baseline(cfg, ctx, budget_s=30.0):
    """The oracle, as it stands, on a bounded sample of the same workload:
    one target layer, one drafter layer, the fc projection and the lm-head
    at the benchmark's widths, formats, block and context (the KV caches of
    the ctx committed positions are seeded random values instead of a host
    prefill); the full step time is extrapolated by the layer counts."""
    import numpy as np
    from dataclasses import replace
    from dflash_block_diffusion_amd import synth
    from oracle.spec import OracleDrafter, OracleTarget
    B = cfg.block
    one = replace(cfg, target=replace(cfg.target, n_layers=1, layer_kinds=cfg.target.kinds()[-1:]),
                  drafter=replace(cfg.drafter, n_layers=1), sel_layers=(0,))
    g = synth.HostSynth(cfg.seed)
    t0 = time.time()
    ck = synth.make_pair(one, g)
    fc_full = g.weight("w_fc_full", cfg.drafter.hidden, len(cfg.sel_layers) * cfg.target.hidden, cfg.drafter.fmt)
    gen_s = time.time() - t0
    cap = ctx + 2 * B
    tgt = OracleTarget(one.target, ck["target"], one.sel_layers, cap)
    drf = OracleDrafter(one.drafter, ck["drafter"], ck["target"], one.mask_token, B, cap)
    rng = np.random.default_rng(5)
    for l in tgt.K:
        tgt.K[l][:ctx] = rng.standard_normal(tgt.K[l][:ctx].shape)
        tgt.V[l][:ctx] = rng.standard_normal(tgt.V[l][:ctx].shape)
    for l in tgt.S:
        tgt.S[l] = rng.standard_normal(tgt.S[l].shape) * 0.1
    for l in range(len(drf.K)):
        drf.K[l][:ctx] = rng.standard_normal(drf.K[l][:ctx].shape)
        drf.V[l][:ctx] = rng.standard_normal(drf.V[l][:ctx].shape)
    tgt.n = ctx
    block = list(synth.prompt(cfg, B, seed=9))
    from oracle.numerics import linear
    from oracle.model import rmsnorm
    t1 = time.time()
    fwd = tgt.forward(block, layers=1)
    t_layer = time.time() - t1
    t1 = time.time()
    logits = linear(rmsnorm(fwd["x"], ck["target"]["final_norm"], 1e-6), ck["target"]["w_lm"])
    t_lm = time.time() - t1
    t1 = time.time()
    hid = np.tile(fwd["x"], (1, len(cfg.sel_layers)))
    linear(hid, fc_full)
    t_fc = time.time() - t1
    t1 = time.time()
    drf.draft(int(block[0]), ctx)
    t_draft1 = time.time() - t1 - t_lm * (B - 1) / B       # draft() includes one lm-head pass
    step_s = cfg.target.n_layers * t_layer + cfg.drafter.n_layers * max(t_draft1, 0.0) + t_fc + 2 * t_lm
    import numpy as _np
    cores = os.cpu_count()
    return {"value": 1.0 / step_s, "unit": "steps/s", "cores": cores, "kind": "oracle",
            "sample": (f"1 target layer ({t_layer:.2f} s), 1 drafter pass ({max(t_draft1, 0):.2f} s), fc "
                       f"({t_fc:.2f} s) and lm-head ({t_lm:.2f} s) of the benchmark step at ctx {ctx} with "
                       f"seeded random KV, extrapolated to {cfg.target.n_layers}+{cfg.drafter.n_layers} layers; "
                       f"float64 NumPy, BLAS threads = host cores ({cores}); weight synthesis {gen_s:.1f} s "
                       f"not timed"),
            "step_seconds": step_s}


def prefill_gemm_rate(pair, prompt, cfg, ctx):
    """MFMA throughput of the prompt pass's dense GEMMs: one profiled prompt
    pass records every launch; the dense ones are replayed back to back
    between two HIP events on the launch stream.  FLOPs = 2 * rows * the
    target's projection parameters over the rows that run as dense chunks."""
    import torch
    from dflash_block_diffusion_amd import configs
    B = cfg.block
    # rows the dense chunks run (chunks of up to 1024 rows): the whole prompt,
    # the last chunk padded to 16 rows, or, with GatedDeltaNet layers, the
    # whole blocks before the one holding the last token
    if any(k != configs.LAYER_ATTN for k in cfg.target.layer_kinds or ()):
        dense_rows = ((ctx - 1) // B) * B
    else:
        full = (ctx - 1) // 1024
        dense_rows = full * 1024 + (ctx - full * 1024 + 15) // 16 * 16
    pair.prof(True)
    pair.prefill(prompt)
    torch.cuda.synchronize()
    pair.prof(False)
    recs = {r["kernel"]: r for r in pair.prof_read()}
    names = [n for n in ("gemm_dense_w4", "gemm_dense_w4_silu") if n in recs]
    if not names or dense_rows <= 64:
        return None
    ms, launches = 0.0, 0
    for n in names:
        m, c = pair.prof_replay(n, reps=1)
        ms += m
        launches += c
    t = cfg.target
    params = (t.qkv_rows * t.hidden + t.hidden * t.n_q_heads * t.head_dim + 2 * t.ffn * t.hidden
              + t.hidden * t.ffn) * t.n_layers
    flops = 2.0 * dense_rows * params
    achieved = flops / (ms / 1e3) / 1e12
    log(f"prompt pass dense GEMMs: {launches} launches, {ms:.2f} ms back to back, {achieved:.0f} TFLOP/s")
    return {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_FP16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_FP16_PEAK_TFLOPS, 4), "kernel": "gemm_dense_w4 (+_silu)",
            "launches": launches, "dense_rows": dense_rows, "avg_launch_us": round(ms * 1e3 / launches, 2)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=16)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="8b", choices=["tiny", "4b", "8b", "27b", "hybrid"])
    ap.add_argument("--ctx", type=int, default=2048)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prof", action="store_true")
    ap.add_argument("--max-draft", type=int, default=0,
                    help="verify only the first N drafts per step (0 = the whole block)")
    ap.add_argument("--temperature", type=float, default=0.0,
                    help="speculative sampling at this temperature (drafts drawn, no injection)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="measure only the prompt pass (time to first token) and print its line")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the draft+verify step of one sequence runs on a single "
              f"MI355X (requested --gpus {args.gpus}); the library uses no second GPU.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from dflash_block_diffusion_amd import configs, synth
    from dflash_block_diffusion_amd.runtime import Pair

    cfg = configs.get(args.config)
    B, ctx = cfg.block, args.ctx
    torch.cuda.set_device(0)
    t0 = time.time()
    ck = synth.make_pair(cfg, synth.DeviceSynth(args.seed, "cuda"))
    K, W = args.steps, args.warmup
    max_ctx = ctx + (W + K + 4) * B + 64
    pair = Pair(cfg, ck, max_ctx=max_ctx)
    n_drafts = B - 1
    if args.max_draft:
        pair.set_max_draft(args.max_draft)
        n_drafts = pair.accept_block - 1
    del ck
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    log(f"model ready in {time.time() - t0:.1f} s ({cfg.name}, {(pair.t.weight_bytes() + pair.d.weight_bytes()) / 1e9:.2f} GB)")

    sampling = args.temperature > 0
    if sampling:
        pair.set_sampling(args.temperature, args.seed + 17)
    prompt = synth.prompt(cfg, ctx, seed=1)
    t0 = time.time()
    pair.prefill(prompt)
    log(f"prefill {ctx} tokens in {time.time() - t0:.2f} s (first call)")
    dense = None if args.no_prof else prefill_gemm_rate(pair, prompt, cfg, ctx)
    # time to first token: a prefill of the same prompt (the state is reset by it)
    torch.cuda.synchronize()
    t0 = time.time()
    pair.prefill(prompt)
    prefill_s = time.time() - t0
    pair.snapshot()
    log(f"prefill {ctx} tokens in {prefill_s * 1e3:.1f} ms ({ctx / prefill_s:.0f} tok/s)")
    prefill = {"tokens": ctx, "ms": round(prefill_s * 1e3, 2), "tok_per_s": round(ctx / prefill_s, 1),
               "dense_gemm_roofline": dense}
    if args.prefill_only:
        print(json.dumps({"metric": "prompt pass tokens/s (time to first token)", "value": prefill["tok_per_s"],
                          "unit": "tok/s", "n_gpus": 1, "higher_is_better": True, "data": "synthetic",
                          "config": {"workload": f"{cfg.name}: prompt of {ctx} tokens", "ctx": ctx},
                          "prefill": prefill}), flush=True)
        return
    n_sched = W + K + 8
    sched = torch.as_tensor(synth.accept_schedule(cfg, n_sched, seed=2), device="cuda")
    inj = None
    if not sampling:
        # reference greedy stream: the lossless loop itself, no injection
        need = ctx + (W + K + 3) * B
        t0 = time.time()
        while pair.query()["n"] < need:
            for _ in range(8):
                pair.step()
        n_ref = pair.query()["n"]
        ref = pair.tokens(n_ref + 1).clone()
        pair.rollback(ctx)
        log(f"reference stream of {n_ref - ctx} tokens in {time.time() - t0:.1f} s")
        filler = torch.as_tensor(synth.filler_tokens(cfg, n_sched, seed=3), device="cuda")
        inj = (ref, sched, filler)
    # capture one step
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        pair.step(inj)                      # eager warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    pair.rollback(ctx)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pair.step(inj)
    torch.cuda.synchronize()
    pair.rollback(ctx)
    for _ in range(W):
        g.replay()
    torch.cuda.synchronize()
    q0 = pair.query()
    pair.rollback(ctx)
    torch.cuda.synchronize()
    steps0 = pair.query()["steps"]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(K):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    q = pair.query()
    tokens = q["n"] - ctx
    acc = pair.acc_log().cpu().numpy()
    idx = [(steps0 + i) % len(acc) for i in range(K)]
    a_run = acc[idx]
    a_sched = np.minimum(sched.cpu().numpy()[[(steps0 + i) % n_sched for i in range(K)]], n_drafts)
    if q["status"] != 0:
        log(f"WARNING: device status word {q['status']}")
    log(f"timed {K} steps: {ms:.3f} ms, n {ctx} -> {q['n']}, accepted {a_run.tolist()}, "
        + ("drafts sampled (natural acceptance)" if sampling else f"schedule {a_sched.tolist()}"))

    steps_per_s = K / (ms / 1e3)
    tok_per_s = tokens / (ms / 1e3)
    wbytes = weight_bytes_per_step(cfg)
    n_mean = ctx + tokens / 2.0
    step_bytes = wbytes + kv_bytes_per_step(cfg, n_mean)
    step_frac = step_bytes * steps_per_s / (HBM_PEAK_GBS * 1e9)

    roof = None
    kernels = []
    if not args.no_prof:
        pair.rollback(ctx)
        pair.prof(True)
        for _ in range(K):
            pair.step(inj)
        torch.cuda.synchronize()
        pair.prof(False)
        kernels = pair.prof_read()
        kernels.sort(key=lambda r: -r["ms"])
        gem_ms = sum(r["ms"] for r in kernels)
        gem_bytes = sum(r["bytes"] for r in kernels)
        top = kernels[0]
        per_launch_bytes = top["bytes"] / top["launches"]
        # the per-launch events above carry a marker gap each; the kernel's own
        # average comes from its recorded launches replayed back to back
        # (weights of every layer in turn, so no cache holds them)
        rep_ms, rep_n = pair.prof_replay(top["kernel"], reps=3)
        avg_ms = rep_ms / rep_n
        achieved = per_launch_bytes / (avg_ms / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": committed_traffic(top["kernel"]),
                "kernel": top["kernel"], "launches_per_step": top["launches"] / K,
                "bytes_per_launch": per_launch_bytes, "avg_launch_us": round(avg_ms * 1e3, 2),
                "avg_launch_us_with_event_markers": round(top["ms"] / top["launches"] * 1e3, 2),
                "all_gemms_GBps": round(gem_bytes / (gem_ms / 1e3) / 1e9, 1),
                "gemm_ms_per_step_eager": round(gem_ms / K, 4)}
        for r in kernels:
            log(f"  {r['kernel']:18s} launches/step {r['launches'] / K:6.1f}  avg {r['ms'] / r['launches'] * 1e3:8.2f} us"
                f"  {r['bytes'] / r['launches'] / 1e6:8.2f} MB/launch  "
                f"{r['bytes'] / (r['ms'] / 1e3) / 1e9:8.1f} GB/s")

    cpu = None
    if not args.no_cpu_baseline:
        t0 = time.time()
        cpu = cpu_baseline(cfg, ctx)
        log(f"cpu baseline in {time.time() - t0:.1f} s: {cpu['value']:.5f} steps/s")
        cpu.pop("step_seconds", None)

    fmt_name = {0: "f32", 1: "bf16", 2: "w8a16", 3: "w4a16"}
    out = {
        "metric": "draft+verify steps/s & effective tok/s (block 16/32); % of HBM roofline",
        "value": round(steps_per_s, 3),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.target.fmt != 0 else "f32",
        "data": "synthetic",
        "config": {"workload": (f"{cfg.name}: {fmt_name[cfg.target.fmt]} target {cfg.target.n_layers} layers "
                                f"H{cfg.target.hidden} + {fmt_name[cfg.drafter.fmt]} drafter "
                                f"{cfg.drafter.n_layers} layers, block {B}, ctx {ctx}, "
                                + (f"temperature {args.temperature} (drafts sampled, natural acceptance)"
                                   if sampling else "injected acceptance")
                                + (f", draft cap {n_drafts} ({pair.vrows} verify rows)" if args.max_draft else "")),
                   "block": B, "ctx": ctx, "global_batch": 1, "verify_rows": pair.vrows, "drafts_verified": n_drafts,
                   "target_format": fmt_name[cfg.target.fmt], "drafter_format": fmt_name[cfg.drafter.fmt]},
        "tok_per_s": round(tok_per_s, 1),
        "tokens_per_step": round(tokens / K, 3),
        "bytes_per_step": int(step_bytes),
        "hbm_frac_step": round(step_frac, 4),
        "prefill": prefill,
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
