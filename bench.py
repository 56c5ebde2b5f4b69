#!/usr/bin/env python3
"""Throughput of the DFlash draft-and-accept hot path on one MI355X.

One step = one cycle of the whole path for every request of the batch:
dflash_draft_block (block prep, embedding, every draft layer, final norm,
lm_head, argmax) -> dflash_accept against a planted target posterior ->
dflash_project_context of the committed verify rows (fc + hidden_norm +
per-layer K/V with k-norm and RoPE into the paged cache).  The state (prefix
lengths, anchors, cache) is the same for every step: the crop is logical, so
re-running a cycle from the same committed prefix is the same work.

Inputs are seeded and synthetic (random-init weights and features
N(0, 0.02^2), random context K/V, uniform token ids), resident in HBM before
the timed region.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "draft blocks/s + drafted tokens/s at 1 GPU; % HBM/MFMA roofline (Qwen3-8B, B=16)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16, published


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def draft_pass_bytes(cfg, L):
    """Algorithmic HBM bytes of one draft pass: every weight once, the
    context K/V each layer reads (window-limited on sliding layers), the
    embedding rows of the block."""
    H, D, nq, nkv, I, V = cfg.hidden, cfg.head_dim, cfg.n_q_heads, cfg.n_kv_heads, cfg.inter, cfg.vocab
    wb = 2 if cfg.act_dtype == "bf16" else 4
    kvb = {"f32": 4, "bf16": 2, "fp8_e4m3": 1}[cfg.kv_dtype]
    layer_params = (nq + 2 * nkv) * D * H + H * nq * D + 3 * I * H + 2 * H + 2 * D
    b = cfg.n_layers * layer_params * wb + V * H * wb + H * wb
    B, S = len(L), cfg.block_size
    for l in range(cfg.n_layers):
        W = cfg.window(l)
        for Lr in L:
            keys = min(Lr, W - 1) if W else Lr
            if cfg.context_window:
                keys = min(keys, cfg.context_window)
            b += keys * nkv * D * 2 * kvb
    b += B * S * H * wb
    return b


def profiled_traffic(workload):
    """HBM bytes per lm_head launch from the committed counter summary, or None
    when there is none for this workload or the GEMM source has changed since
    the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"lm_head_gemm_{workload}.md")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith(("|", "#", "`")):
            k, _, v = line.partition(":")
            vals[k.strip()] = v.strip()
    csrc = os.path.join(ROOT, "block_diffusion_drafter_rmsnorm_amd", "csrc")
    sha = hashlib.sha256(b"".join(open(os.path.join(csrc, f), "rb").read()
                                  for f in ("gemm.hip", "common.h"))).hexdigest()
    if vals.get("kernel_source_sha256") != sha or "traffic_bytes_per_launch" not in vals:
        return None
    return int(float(vals["traffic_bytes_per_launch"]))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="qwen3_8b_b16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a 1 GiB device copy (counter calibration for profiling runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this path is measured on one MI355X and the "
              f"batch shards by request with no collectives; --gpus {args.gpus} is not run.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from workloads import synth
    from workloads.configs import get_workload
    import block_diffusion_drafter_rmsnorm_amd as dfl

    wl = get_workload(args.workload)
    cfg = wl.cfg
    B, S, P = wl.batch, cfg.block_size, cfg.page_size
    dev = "cuda"
    torch.cuda.set_device(0)
    t_setup = time.time()
    W = synth.weights(cfg, wl.seed, dev)
    cw = dfl.make_weights(W)
    L = synth.prefix_lengths(wl, "cpu").to(torch.int32)
    pt, npages = synth.page_table(L, cfg, wl.seed, 2 * S)
    K, V = synth.kv_pool_random(cfg, npages, wl.seed, dev)
    cache = dfl.KVCache(K, V, npages)
    c_cfg, c_cache = dfl.make_config(cfg), cache.c_struct()
    anchor = synth.randint(0, cfg.vocab - 1, (B,), wl.seed, "anchor").to(torch.int32).to(dev)
    Ld, ptd = L.to(dev), pt.to(dev)
    max_prefix = int(L.max())
    vfeat = synth.features(B * S, cfg, wl.seed, "verify", dev)
    positions = torch.empty((B, S), dtype=torch.int32, device=dev)
    slots = torch.empty_like(positions)
    cand = torch.empty_like(positions)
    acc = [torch.empty(B, dtype=torch.int32, device=dev) for _ in range(4)]
    out_tok = torch.empty((B, S), dtype=torch.int32, device=dev)
    dws = dfl.workspace(dfl.draft_workspace_bytes(cfg, B, max_prefix))
    cws = dfl.workspace(dfl.context_workspace_bytes(cfg, B * S))
    torch.cuda.synchronize()
    log(f"[bench] {wl.name}: setup {time.time() - t_setup:.1f}s, pages {npages}, "
        f"max prefix {max_prefix}")

    def draft():
        dfl.dflash_draft_block(cfg, cw, cache, anchor, Ld, ptd, max_prefix, positions, slots, cand,
                               dws, c_cfg=c_cfg, c_cache=c_cache)

    # planted target posterior: commit lengths as the workload states (uniform
    # in [lo, hi]) or, when it states none, 6: the pages' mean accept length
    # with a block-16 Qwen3-8B draft is 6.35-6.48.
    draft()
    torch.cuda.synchronize()
    lo, hi = wl.commit
    if hi == 0:
        commit = torch.full((B,), 6, dtype=torch.int64)
    else:
        commit = synth.randint(lo, hi, (B,), wl.seed, "commit")
    post = synth.plant_posterior(cand.cpu(), commit, cfg.vocab, wl.seed).to(dev)

    def step():
        draft()
        dfl.dflash_accept(cand, post, Ld, acc[0], acc[1], out_tok, acc[2], acc[3])
        dfl.dflash_project_context(cfg, cw, cache, vfeat, positions.view(-1), slots.view(-1),
                                   acc[1], B, S, cws, c_cfg=c_cfg, c_cache=c_cache)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    got_commit = acc[1].cpu()
    assert torch.equal(got_commit, commit.to(torch.int32)), "planted commit lengths not reproduced"

    def timed(fn, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    ms_step = timed(step, args.steps)
    ms_draft = timed(draft, args.steps)
    log(f"[bench] step {ms_step:.3f} ms, draft pass {ms_draft:.3f} ms")

    # spread of single draft passes: an event pair around each call (the mean
    # above is the back-to-back figure; these include one event gap each)
    def per_call(fn, n):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        torch.cuda.synchronize()
        for e0, e1 in evs:
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        return sorted(e0.elapsed_time(e1) for e0, e1 in evs)

    one = per_call(draft, max(args.steps, 20))
    pct = lambda q: round(one[min(len(one) - 1, int(q * len(one)))], 4)  # noqa: E731

    # dominant kernel: lm_head GEMM + argmax partials over the B*(S-1) rows,
    # timed alone on the same shapes: back-to-back calls between two events on
    # the stream they run on (the launch is the GEMM plus the ~5 us second
    # argmax stage)
    M1 = B * (S - 1)
    hid = synth.normal((M1, cfg.hidden), 1.0, wl.seed, "lm_rows", synth._DT[cfg.act_dtype], dev)
    ids = torch.empty(M1, dtype=torch.int32, device=dev)
    lws = dfl.workspace(dfl.lm_head_workspace_bytes(cfg, M1))

    def lm_call():
        dfl.dflash_lm_head_argmax(cfg, cw.packed["lm_head"], hid, ids, lws, c_cfg=c_cfg)

    lm_call()
    lm_ms = timed(lm_call, max(args.steps, 5))
    wb = 2 if cfg.act_dtype == "bf16" else 4
    lm_bytes = cfg.vocab * cfg.hidden * wb + M1 * cfg.hidden * wb + M1 * 4
    lm_avg_s = float(lm_ms) * 1e-3
    lm_gbs = lm_bytes / lm_avg_s / 1e9

    # context injection throughput (prefill of one prompt-sized chunk)
    T = min(int(L.max()), 8192) if wl.inject_rows == 0 else min(wl.inject_rows, 8192)
    T = max(T, 1)
    pf = synth.features(T, cfg, wl.seed, "prefill", dev)
    ppos = torch.arange(T, dtype=torch.int32, device=dev)
    pslot = torch.arange(T, dtype=torch.int32, device=dev) % (npages * P)
    pws = dfl.workspace(dfl.context_workspace_bytes(cfg, T))

    def inject_prefill():
        dfl.dflash_project_context(cfg, cw, cache, pf, ppos, pslot, None, 1, T, pws, c_cfg=c_cfg,
                                   c_cache=c_cache)

    inject_prefill()
    ms_inj = timed(inject_prefill, max(3, args.steps // 4))
    inj_flops = 2.0 * T * (cfg.feat_dim * cfg.hidden + cfg.hidden * cfg.n_layers * 2 *
                           cfg.n_kv_heads * cfg.head_dim)

    # rejection-sampling verify at the same batch: synthetic target logits
    # [B, S, V], the draft pass's own logits [B, S-1, V] as the proposal q
    sv = sampling_verify(dfl, synth, cfg, wl, cw, cache, anchor, Ld, ptd, max_prefix, c_cfg,
                         c_cache, timed, max(args.steps, 10), dev)
    # greedy accept reading the target's logits [B, S, V] (fused argmax)
    al = accept_from_logits(dfl, synth, cfg, wl, Ld, timed, max(args.steps, 10), dev)
    # the same pass with the DFlash 2 candidate selector (top-8, rank 64)
    sel = selector_pass(dfl, synth, cfg, wl, cw, cache, anchor, Ld, ptd, max_prefix, timed,
                        args.steps, dev, ms_draft)

    if args.copy_probe:
        # a plain copy of known size: under a counter-collection run its
        # FETCH_SIZE / WRITE_SIZE give the scale of those counters
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    pass_bytes = draft_pass_bytes(cfg, L.tolist())
    res = {
        "metric": METRIC,
        "value": round(B / (ms_step * 1e-3), 3),
        "unit": "draft blocks/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.act_dtype if cfg.kv_dtype != "fp8_e4m3" else "bf16 (fp8 e4m3 KV)",
        "data": "synthetic (seeded random-init weights, features and context K/V)",
        "config": {"workload": wl.name, "batch": B, "block_size": S,
                   "context": list(wl.ctx), "hidden": cfg.hidden, "layers": cfg.n_layers,
                   "vocab": cfg.vocab, "commit_lens": commit.tolist() if B <= 32 else "seeded",
                   "step": "draft_block + accept + project_context(committed rows)"},
        "drafted_tokens_per_s": round(B * (S - 1) / (ms_step * 1e-3), 1),
        "draft_pass": {"ms": round(ms_draft, 4), "blocks_per_s": round(B / (ms_draft * 1e-3), 2),
                       "drafted_tokens_per_s": round(B * (S - 1) / (ms_draft * 1e-3), 1),
                       "algorithmic_bytes": pass_bytes,
                       "hbm_gbs": round(pass_bytes / (ms_draft * 1e-3) / 1e9, 1),
                       "hbm_frac": round(pass_bytes / (ms_draft * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                       "single_call_ms": {"p10": pct(0.1), "p50": pct(0.5), "p90": pct(0.9),
                                          "calls": len(one)}},
        "context_injection": {"rows": T, "ms": round(ms_inj, 4),
                              "context_tokens_per_s": round(T / (ms_inj * 1e-3), 1),
                              "tflops": round(inj_flops / (ms_inj * 1e-3) / 1e12, 2),
                              "mfma_frac": round(inj_flops / (ms_inj * 1e-3) / 1e12 /
                                                 MFMA_BF16_PEAK_TFLOPS, 4)},
        "roofline": {"bound": "hbm", "achieved": round(lm_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(lm_gbs / HBM_PEAK_GBS, 4),
                     "traffic": profiled_traffic(wl.name),
                     "kernel": "gemm_rows<EpiLogits> lm_head + argmax partials "
                               "(+ argmax reduce), dflash_lm_head_argmax",
                     "bytes_per_launch": lm_bytes,
                     "avg_launch_us": round(lm_avg_s * 1e6, 2)},
        "sampling_verify": sv,
        "accept_logits": al,
        "selector_pass": sel,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, wl, L.tolist(), W, anchor.cpu().numpy(),
                                             post.cpu().numpy(), T)
    print(json.dumps(res), flush=True)


def sampling_verify(dfl, synth, cfg, wl, cw, cache, anchor, Ld, ptd, max_prefix, c_cfg, c_cache,
                    timed, n, dev):
    """Time dflash_accept_sampling on the workload's batch: argmax drafts (q a
    point mass) and drafts with q = softmax(draft logits).  Algorithmic bytes:
    every target (and draft) logit read once, plus ids, draws and outputs."""
    import torch
    B, S, V = wl.batch, cfg.block_size, cfg.vocab
    dt = synth._DT[cfg.act_dtype]
    positions = torch.empty((B, S), dtype=torch.int32, device=dev)
    slots, cand = torch.empty_like(positions), torch.empty_like(positions)
    dlog = torch.empty((B, S - 1, V), dtype=dt, device=dev)
    dws = dfl.workspace(dfl.draft_workspace_bytes(cfg, B, max_prefix))
    dfl.dflash_draft_block(cfg, cw, cache, anchor, Ld, ptd, max_prefix, positions, slots, cand, dws,
                           logits=dlog, c_cfg=c_cfg, c_cache=c_cache)
    # candidates and target rows from the verify generator (the target favours
    # the drafts, so accept lengths spread over the block)
    vc, tl, _, u = synth.verify_inputs(B, S, V, wl.seed, dtype=dt, device=dev, bump=22.0,
                                       bump_lo=13.0)
    outs = [torch.empty(B, dtype=torch.int32, device=dev) for _ in range(4)]
    ot = torch.empty((B, S), dtype=torch.int32, device=dev)
    esz = 2 if cfg.act_dtype == "bf16" else 4
    res = {}
    for mode, dl in (("argmax_drafts", None), ("draft_logits", dlog)):
        ws = dfl.workspace(dfl.accept_sampling_workspace_bytes(B, S, V, dl is not None))

        def call():
            dfl.dflash_accept_sampling(vc, tl, u, Ld, outs[0], outs[1], ot, outs[2], outs[3], ws,
                                       1.0, dl, 1.0)
        call()
        ms = timed(call, n)
        nbytes = (B * S * V + (B * (S - 1) * V if dl is not None else 0)) * esz + B * S * 12
        res[mode] = {"us": round(ms * 1e3, 2), "algorithmic_bytes": nbytes,
                     "hbm_gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
                     "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "mean_commit": round(float(outs[1].float().mean()), 3)}
    return res


def accept_from_logits(dfl, synth, cfg, wl, Ld, timed, n, dev):
    """Time dflash_accept_logits at the workload's batch on synthetic target
    logits [B, S, V].  Algorithmic bytes: every logit read once, plus ids and
    outputs."""
    import torch
    B, S, V = wl.batch, cfg.block_size, cfg.vocab
    dt = synth._DT[cfg.act_dtype]
    vc, tl, _, _ = synth.verify_inputs(B, S, V, wl.seed, dtype=dt, device=dev, bump=22.0,
                                       bump_lo=13.0)
    outs = [torch.empty(B, dtype=torch.int32, device=dev) for _ in range(4)]
    ot = torch.empty((B, S), dtype=torch.int32, device=dev)
    ws = dfl.workspace(dfl.accept_logits_workspace_bytes(B, S, V))

    def call():
        dfl.dflash_accept_logits(vc, tl, Ld, outs[0], outs[1], ot, outs[2], outs[3], ws)
    call()
    ms = timed(call, n)
    esz = 2 if cfg.act_dtype == "bf16" else 4
    nbytes = B * S * V * esz + B * S * 8 + B * 20
    return {"us": round(ms * 1e3, 2), "algorithmic_bytes": nbytes,
            "hbm_gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "mean_commit": round(float(outs[1].float().mean()), 3)}


def selector_pass(dfl, synth, cfg, wl, cw, cache, anchor, Ld, ptd, max_prefix, timed, n, dev,
                  ms_plain):
    """dflash_draft_block_selector at the workload's batch: the pass plus top-k,
    the W_h projection, the lattice and the walk (synthetic selector weights)."""
    import torch
    B, S, K, r = wl.batch, cfg.block_size, 8, 64
    dt = synth._DT[cfg.act_dtype]
    A = synth.normal((cfg.vocab, r), 0.3, wl.seed, "sel_a", dt, dev)
    Bt = synth.normal((cfg.vocab, r), 0.3, wl.seed, "sel_b", dt, dev)
    Wh = synth.normal((r, cfg.hidden), 0.02, wl.seed, "sel_wh", dt, dev)
    sel = dfl.Selector(A, Bt, Wh, K)
    ws = dfl.workspace(dfl.selector_workspace_bytes(cfg, sel, B, max_prefix))
    pos = torch.empty((B, S), dtype=torch.int32, device=dev)
    slots, cand = torch.empty_like(pos), torch.empty_like(pos)
    cids = torch.empty((B, S - 1, K), dtype=torch.int32, device=dev)
    q = torch.empty((B, S - 1, K), dtype=torch.float32, device=dev)

    def call():
        dfl.dflash_draft_block_selector(cfg, cw, cache, sel, anchor, Ld, ptd, max_prefix, pos,
                                        slots, cand, cids, q, ws)
    call()
    ms = timed(call, n)
    return {"ms": round(ms, 4), "blocks_per_s": round(B / (ms * 1e-3), 2),
            "overhead_us_vs_argmax_pass": round((ms - ms_plain) * 1e3, 1), "top_k": K,
            "rank": r}


def cpu_baseline(cfg, wl, L, W_dev, anchor, post, T_inj):
    """The oracle (numpy, unmodified steps) on the host cores, in its fp32
    timing setting, on the same units the GPU leg times: one draft pass for
    the workload's batch, one accept of that batch, and one context injection
    of the GPU leg's row count (row-local, so rows/s scales linearly).  Each
    unit is timed three times; the medians are reported.  It reads the same
    weights as the GPU run (copied to host, untimed) and random context K/V of
    the same shape."""
    import numpy as np

    import oracle
    from oracle.precision import working_precision
    from threadpoolctl import threadpool_info

    t0 = time.time()

    def host(t):
        return None if t is None else t.detach().to("cpu").float().numpy()

    W = {k: host(v) for k, v in W_dev.items() if k != "layers"}
    W["layers"] = [{k: host(v) for k, v in Lw.items()} for Lw in W_dev["layers"]]
    nkv, D, F, P, S = cfg.n_kv_heads, cfg.head_dim, cfg.feat_dim, cfg.page_size, cfg.block_size
    B = len(L)
    Ls = np.asarray(L, np.int64)
    npg = (Ls + 2 * S + P - 1) // P
    pt = np.full((B, int(npg.max())), -1, np.int64)
    off = 0
    for r in range(B):
        pt[r, :npg[r]] = off + np.arange(npg[r])
        off += int(npg[r])
    g = np.random.default_rng(wl.seed)
    cache = oracle.OracleCache.__new__(oracle.OracleCache)
    cache.k = [g.standard_normal((off * P, nkv, D), dtype=np.float32) for _ in range(cfg.n_layers)]
    cache.v = [g.standard_normal((off * P, nkv, D), dtype=np.float32) for _ in range(cfg.n_layers)]
    anc = np.asarray(anchor, np.int64)
    post = np.asarray(post, np.int64)
    feats = (g.standard_normal((T_inj, F), dtype=np.float32) * 0.02)
    pos = np.arange(T_inj)
    slots = pos % (off * P)
    copy_s = time.time() - t0

    def med3(fn):
        ts = []
        for _ in range(3):
            t = time.time()
            fn()
            ts.append(time.time() - t)
        return float(np.median(ts)), ts

    with working_precision("f32"):
        d = {}
        t_draft, r_draft = med3(lambda: d.update(oracle.draft_block(cfg, W, cache, anc, Ls, pt)))
        t_acc, r_acc = med3(lambda: oracle.accept(d["candidates"], post, Ls))
        t_inj, r_inj = med3(lambda: oracle.project_context(cfg, W, cache, feats, pos, slots))
    blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
    threads = blas[0]["num_threads"] if blas else len(os.sched_getaffinity(0))
    ctx = f"{int(Ls.min())}" if Ls.min() == Ls.max() else f"{int(Ls.min())}..{int(Ls.max())}"
    return {"value": round(B / t_draft, 5), "unit": "draft blocks/s", "cores": threads,
            "kind": "oracle",
            "sample": f"fp32 oracle, median of 3 runs per unit: one draft pass of the batch "
                      f"({B} x block {S}, {cfg.n_layers} layers, context {ctx}, vocab "
                      f"{cfg.vocab}), one accept of the batch, one {T_inj}-row context "
                      f"injection; weights copied from the GPU run ({copy_s:.1f} s, untimed)",
            "drafted_tokens_per_s": round(B * (S - 1) / t_draft, 4),
            "draft_pass_s": {"median": round(t_draft, 4), "runs": [round(t, 4) for t in r_draft]},
            "accept_s": {"median": round(t_acc, 6), "runs": [round(t, 6) for t in r_acc]},
            "injection": {"rows": T_inj, "median_s": round(t_inj, 4),
                          "runs": [round(t, 4) for t in r_inj],
                          "context_tokens_per_s": round(T_inj / t_inj, 2)}}


if __name__ == "__main__":
    main()
