#!/usr/bin/env python
"""Benchmark of the DashAttention forward pass on one MI355X.

Prints ONE JSON line on stdout:
  value      prefill tokens/s on the 128K workload (B=1, 32 query / 2 KV heads, D=128,
             bf16, alpha=1.5, planted needles calibrated to ~75% zero routing weight);
             one step = one full causal prefill (Stage 0 + Stage 1 + Stage 2), inputs
             resident in HBM;
  roofline   Stage 2 (the dominant kernel) against the bf16 dense MFMA peak, with
             algorithmic flops  sum_{b,kvh,t} G * 4 D * (64 * popcount(mask_t) + t % 64 + 1);
  decode     the 64K decode workload (B=16, 256 steps, summary appended when a chunk fills):
             us/step against the HBM roofline of its algorithmic bytes;
  dense      a dense causal flash-style kernel on the same inputs (the pages' comparator);
  topk_router  the same prefill with a top-k comparison router (k = entmax's mean active
             chunks per row) in place of entmax: Stage 1 and Stage 2 times;
  estimate_diagonal  the same prefill with the own chunk's partial summary in the entmax;
  backward   dq, dk, dv and d head_cls through all three stages (dash_prefill_backward);
  cpu_baseline  the float64 oracle timed on host cores over a bounded sample of rows.
Progress lines go to stderr.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prefill tokens/s @128K + decode us/token @64K, bf16; % MFMA/HBM roofline"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "stage2_traffic.json")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def popcount64(x):
    """Popcount of int64 tensors (two 32-bit halves, SWAR)."""
    import torch
    out = torch.zeros_like(x)
    for half in (x & 0xFFFFFFFF, (x >> 32) & 0xFFFFFFFF):
        v = half - ((half >> 1) & 0x55555555)
        v = (v & 0x33333333) + ((v >> 2) & 0x33333333)
        v = (v + (v >> 4)) & 0x0F0F0F0F
        out += (v * 0x01010101 & 0xFFFFFFFF) >> 24
    return out


# dash_prefill_stage order of one full prefill: summaries, the chunk-transposed V copy that
# bf16 Stage 2 reads, routing, sparse attention
STAGES = (0, 3, 1, 2)


def stage_times(ev):
    """Mean ms per prefill stage, keyed by dash_prefill_stage index, from per-step event
    lists [start, after STAGES[0], after STAGES[1], ...]."""
    n = len(ev)
    return {s: float(np.mean([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(n)]))
            for j, s in enumerate(STAGES)}


def source_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def bench_prefill(args, w, dash, torch):
    from long_context_sparse_stage0_amd import synth
    t0 = time.time()
    x = synth.prefill_inputs(w)
    log(f"generated {w.name} inputs in {time.time() - t0:.1f}s")
    dev = torch.device("cuda:0")
    q, k, v, hc = (torch.from_numpy(x[n]).to(torch.bfloat16).to(dev)
                   for n in ("q", "k", "v", "head_cls"))
    B, Hq, T, D = q.shape
    Hkv, G = w.Hkv, w.G
    nc = -(-T // 64)
    W = -(-nc // 64)
    out = torch.empty_like(q)
    ab = torch.empty((B, Hkv, T, W), dtype=torch.int64, device=dev)
    p = dash.make_params(B, Hq, Hkv, T, D, alpha=w.alpha, gamma=w.gamma, enable_gqa=True,
                         dtype=torch.bfloat16)
    ws = dash.alloc_workspace(dash.workspace_size("prefill", p), dev)
    kw = dict(alpha=w.alpha, gamma=w.gamma, enable_gqa=True, workspace=ws)

    # one untimed pass returning the mask, for the sparsity and the algorithmic flops
    dash.prefill(q, k, v, hc, out=out, **kw)
    dash.prefill_stage(1, q, k, v, hc, out, ws, alpha=w.alpha, gamma=w.gamma,
                       enable_gqa=True, active_blocks=ab)
    torch.cuda.synchronize()
    pc = popcount64(ab).sum(dim=-1)                       # [B, Hkv, T] active chunks per row
    t_idx = torch.arange(T, device=dev)
    routed = (t_idx // 64).to(torch.float64)
    active = pc.to(torch.float64)
    zero_frac = 1.0 - float(active.sum() / (routed.sum() * B * Hkv))
    diag = (t_idx % 64 + 1).to(torch.float64)
    flops2 = float(G * 4 * D * (64.0 * active.sum() + B * Hkv * diag.sum()))
    # executed work of the union walk: R rows per workgroup share the union of their masks
    R = min(64, 256 // G) if G >= 4 else 64
    abr = ab.view(B, Hkv, T // R, R, W) if T % R == 0 else None
    union_flops = None
    if abr is not None:
        u = abr[:, :, :, 0].clone()
        for r in range(1, R):
            u |= abr[:, :, :, r]
        upc = popcount64(u).sum(dim=-1).to(torch.float64)  # [B, Hkv, T/R]
        union_flops = float(R * G * 4 * D * 64.0 * upc.sum() + G * 4 * D * B * Hkv * 64.0 * T)
    flops_dense = float(B * Hq * 4 * D * T * (T + 1) / 2)
    log(f"zero-weight fraction {zero_frac:.4f}; stage-2 algorithmic flops {flops2:.3e}")
    k_match = max(1, int(round(float(active.sum()) / (B * Hkv * T))))   # mean active per row
    # Stage 0 and Stage 1 algorithmic work: Stage 0 reads K and writes the fp32 summaries
    # (the bf16 split planes and the chunk-transposed V are this implementation's extras);
    # Stage 1 reads Q and the summaries once, writes the mask and w_bar at set bits, and
    # does 2 D flops per (query vector, routed chunk) score (twice, for the hi and lo planes)
    nfull = T // 64
    s0_bytes = float(B * Hkv * (T * D * 2 + nfull * D * 4))
    s0_split = float(B * Hkv * nfull * D * 2 * 2)
    vt_bytes = float(B * Hkv * 2 * nc * 64 * D * 2)      # V read, V^T written
    s1_bytes = float(B * Hq * T * D * 2 + B * Hkv * nc * D * 4 + B * Hkv * T * W * 8
                     + active.sum() * 4)
    s1_flops = float(2 * D * Hq * B * routed.sum())
    del pc, active

    def step(evs=None):
        for i, s in enumerate(STAGES):
            dash.prefill_stage(s, q, k, v, hc, out, ws, alpha=w.alpha, gamma=w.gamma,
                               enable_gqa=True)
            if evs is not None:
                evs[i + 1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} done")
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(STAGES) + 1)]
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record()
        step(ev[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    st = stage_times(ev)
    log(f"prefill {ms:.2f} ms/step; summaries {st[0]:.3f}, V^T copy {st[3]:.3f}, "
        f"stage 1 {st[1]:.3f}, stage 2 {st[2]:.3f} ms")
    tokens_s = B * T / (ms / 1e3)

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        tf = json.load(open(TRAFFIC_FILE))
        src = os.path.join(ROOT, "long_context_sparse_stage0_amd", "csrc", "attend_mfma.hip")
        if tf.get("source_sha256_16") == source_hash(src) and tf.get("workload") == w.name:
            traffic = tf.get("bytes_per_launch")
    achieved = flops2 / (st[2] / 1e3) / 1e12
    roof = {"bound": "mfma", "kernel": "k_attend_mfma (Stage 2)", "achieved": achieved,
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
            "traffic": traffic, "algorithmic_flops_per_launch": flops2,
            "executed_union_flops_per_launch": union_flops,
            "kernel_ms": st[2]}
    res = dict(ms=ms, tokens_s=tokens_s, stages_ms=st, roofline=roof, zero_frac=zero_frac,
               flops2=flops2, flops_dense=flops_dense, x=x)
    res["stage0"] = {"kernel": "k_stage0", "ms": st[0], "algorithmic_bytes": s0_bytes,
                     "gbs": s0_bytes / (st[0] / 1e3) / 1e9,
                     "frac_of_hbm_peak": s0_bytes / (st[0] / 1e3) / 1e9 / PEAK_HBM_GBS,
                     "extra_bytes_split_planes": s0_split,
                     "gbs_with_split_planes": (s0_bytes + s0_split) / (st[0] / 1e3) / 1e9}
    res["vtranspose"] = {"kernel": "k_vtranspose", "ms": st[3], "bytes": vt_bytes,
                         "gbs": vt_bytes / (st[3] / 1e3) / 1e9,
                         "frac_of_hbm_peak": vt_bytes / (st[3] / 1e3) / 1e9 / PEAK_HBM_GBS}
    s1_lb = {"mfma_ms": 2 * s1_flops / (PEAK_BF16_TFLOPS * 1e12) * 1e3,
             "hbm_ms": s1_bytes / (PEAK_HBM_GBS * 1e9) * 1e3}
    res["stage1"] = {"ms": st[1], "algorithmic_bytes": s1_bytes,
                     "gbs": s1_bytes / (st[1] / 1e3) / 1e9,
                     "frac_of_hbm_peak": s1_bytes / (st[1] / 1e3) / 1e9 / PEAK_HBM_GBS,
                     "score_flops": s1_flops, "executed_score_flops_hi_lo": 2 * s1_flops,
                     "lower_bound_ms": s1_lb,
                     "frac_of_lower_bound": max(s1_lb.values()) / st[1]}

    if not args.no_topk:
        # the top-k comparison router on the same inputs, k = entmax's mean active chunks per
        # row, so that Stage 2 gets about the same work and Stage 1 compares the routers
        dash.prefill_stage(1, q, k, v, hc, out, ws, alpha=w.alpha, gamma=w.gamma,
                           enable_gqa=True, topk=k_match, active_blocks=ab)
        torch.cuda.synchronize()
        act_k = float(popcount64(ab).sum())
        evk = [[torch.cuda.Event(enable_timing=True) for _ in range(len(STAGES) + 1)]
               for _ in range(args.steps)]
        for i in range(-1, args.steps):
            if i >= 0:
                evk[i][0].record()
            for j, s in enumerate(STAGES):
                dash.prefill_stage(s, q, k, v, hc, out, ws, alpha=w.alpha, gamma=w.gamma,
                                   enable_gqa=True, topk=k_match)
                if i >= 0:
                    evk[i][j + 1].record()
        torch.cuda.synchronize()
        stk = stage_times(evk)
        res["topk"] = {"k": k_match, "stage1_ms": stk[1], "stage2_ms": stk[2],
                       "prefill_ms": sum(stk.values()),
                       "active_fraction": act_k / float(routed.sum() * B * Hkv),
                       "entmax_stage1_ms": st[1], "entmax_active_fraction": 1.0 - zero_frac}
        log(f"top-k router (k={k_match}): stage 1 {stk[1]:.2f} ms (entmax {st[1]:.2f}), "
            f"stage 2 {stk[2]:.2f} ms, active {res['topk']['active_fraction']:.3f}")

    if not args.no_diag:
        # estimate_diagonal: the own chunk's partial summary in every head's entmax
        dash.prefill_stage(1, q, k, v, hc, out, ws, alpha=w.alpha, gamma=w.gamma,
                           enable_gqa=True, estimate_diagonal=True, active_blocks=ab)
        torch.cuda.synchronize()
        act_d = float(popcount64(ab).sum())
        evd = [[torch.cuda.Event(enable_timing=True) for _ in range(len(STAGES) + 1)]
               for _ in range(args.steps)]
        for i in range(-1, args.steps):
            if i >= 0:
                evd[i][0].record()
            for j, s in enumerate(STAGES):
                dash.prefill_stage(s, q, k, v, hc, out, ws, alpha=w.alpha, gamma=w.gamma,
                                   enable_gqa=True, estimate_diagonal=True)
                if i >= 0:
                    evd[i][j + 1].record()
        torch.cuda.synchronize()
        sd = stage_times(evd)
        res["diag"] = {"stage1_ms": sd[1], "stage2_ms": sd[2], "prefill_ms": sum(sd.values()),
                       "active_fraction": act_d / float(routed.sum() * B * Hkv),
                       "without_flag_stage1_ms": st[1]}
        log(f"estimate_diagonal: stage 1 {sd[1]:.2f} ms (without {st[1]:.2f}), "
            f"stage 2 {sd[2]:.2f} ms, active {res['diag']['active_fraction']:.3f}")

    if not args.no_dense:
        pd = dash.make_params(B, Hq, Hkv, T, D, enable_gqa=True, dtype=torch.bfloat16)
        wsd = dash.alloc_workspace(dash.workspace_size("dense", pd), dev)
        dash.dense_causal(q, k, v, enable_gqa=True, out=out, workspace=wsd)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        nd = max(1, min(args.steps, 3))
        e0.record()
        for _ in range(nd):
            dash.dense_causal(q, k, v, enable_gqa=True, out=out, workspace=wsd)
        e1.record()
        torch.cuda.synchronize()
        dms = e0.elapsed_time(e1) / nd
        res["dense"] = {"ms_per_call": dms, "tflops": flops_dense / (dms / 1e3) / 1e12,
                        "frac_of_peak": flops_dense / (dms / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
                        "speedup_sparse_over_dense": dms / ms,
                        "speedup_stage2_over_dense": dms / st[2]}
        log(f"dense causal {dms:.2f} ms ({res['dense']['tflops']:.0f} TFLOP/s)")
        del wsd
    if not args.no_backward:
        # the backward pass (dash_prefill_train, then dash_prefill_backward) with a seeded
        # dL/dout: dq, dk, dv and d head_cls through all three stages
        del ws, ab
        torch.cuda.empty_cache()
        gen = torch.Generator(device=dev).manual_seed(20268000)
        do = torch.randn(q.shape, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
        out_t, lse = dash.prefill_train(q, k, v, hc, alpha=w.alpha, gamma=w.gamma, enable_gqa=True)
        pb = dash.make_params(B, Hq, Hkv, T, D, alpha=w.alpha, gamma=w.gamma, enable_gqa=True,
                              dtype=torch.bfloat16)
        wsb = dash.alloc_workspace(dash.workspace_size("backward", pb), dev)
        bkw = dict(alpha=w.alpha, gamma=w.gamma, enable_gqa=True, workspace=wsb)
        dash.prefill_backward(q, k, v, hc, out_t, do, lse, **bkw)
        torch.cuda.synchronize()
        nb = max(1, min(args.steps, 3))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(nb):
            grads = dash.prefill_backward(q, k, v, hc, out_t, do, lse, **bkw)
        e1.record()
        torch.cuda.synchronize()
        bms = e0.elapsed_time(e1) / nb
        finite = all(bool(torch.isfinite(g.float()).all()) for g in grads)
        # Stage 2 backward work: the forward's QK^T recomputed plus dP, dQ, dK and dV on the
        # same active (query, key) pairs, i.e. 2.5 times the forward's algorithmic flops
        f2b = 2.5 * flops2
        res["backward"] = {"ms_per_call": bms, "tokens_per_s": B * T / (bms / 1e3),
                           "stage2_backward_algorithmic_flops": f2b,
                           "stage2_backward_tflops_over_whole_call": f2b / (bms / 1e3) / 1e12,
                           "workspace_gib": wsb.numel() / 2 ** 30, "gradients_finite": finite,
                           "calls": nb}
        log(f"backward {bms:.1f} ms per call ({f2b / (bms / 1e3) / 1e12:.0f} TFLOP/s of Stage 2 "
            f"backward work over the whole call), gradients finite: {finite}")
        del do, out_t, lse, wsb, grads
    del q, k, v, out
    torch.cuda.empty_cache()
    return res


def bench_decode(args, w, dash, torch):
    from long_context_sparse_stage0_amd import synth
    t0 = time.time()
    x = synth.decode_inputs(w)
    log(f"generated {w.name} inputs in {time.time() - t0:.1f}s")
    dev = torch.device("cuda:0")
    kc = torch.from_numpy(x["k_cache"]).to(torch.bfloat16).to(dev)
    vc = torch.from_numpy(x["v_cache"]).to(torch.bfloat16).to(dev)
    hc = torch.from_numpy(x["head_cls"]).to(torch.bfloat16).to(dev)
    qs = torch.from_numpy(x["q_steps"]).to(torch.bfloat16).to(dev)
    del x
    B, Hkv, TT, D = kc.shape
    Hq = qs.shape[2]
    S = min(args.decode_steps, w.steps)
    nc = -(-TT // 64)
    W = -(-nc // 64)
    summ = torch.zeros((B, Hkv, nc, D), dtype=torch.float32, device=dev)
    nsum = torch.zeros(B, dtype=torch.int32, device=dev)
    lens_all = (w.T + 1 + torch.arange(S, dtype=torch.int32, device=dev))[:, None].repeat(1, B).contiguous()
    init_len = torch.full((B,), w.T, dtype=torch.int32, device=dev)
    dash.append_chunk(kc, hc, init_len, summ, nsum, Hq=Hq, enable_gqa=True)
    p = dash.make_params(B, Hq, Hkv, TT, D, alpha=w.alpha, enable_gqa=True, dtype=torch.bfloat16)
    ws = dash.alloc_workspace(dash.workspace_size("decode", p), dev)
    out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev)
    ab = torch.empty((B, Hkv, W), dtype=torch.int64, device=dev)

    def run(n, with_mask=False, diag=False):
        act = 0.0
        dkw = dict(estimate_diagonal=True, head_cls=hc) if diag else {}
        for s in range(n):
            L = w.T + 1 + s
            r = dash.decode(qs[s], kc, vc, lens_all[s], summ, alpha=w.alpha, enable_gqa=True,
                            out=out, workspace=ws, return_active_blocks=with_mask, **dkw)
            if with_mask:
                act += float(popcount64(r[1]).sum())
            if L % 64 == 0:
                dash.append_chunk(kc, hc, lens_all[s], summ, nsum, Hq=Hq, enable_gqa=True)
        return act

    # untimed pass for the algorithmic bytes
    act = run(S, with_mask=True)
    torch.cuda.synchronize()
    nsum.fill_(w.T // 64)
    # bytes: summaries of routed chunks (fp32), active K/V chunks, the diagonal tokens, q, o
    bytes_total = 0.0
    for s in range(S):
        t = w.T + s
        it = t // 64
        bytes_total += B * Hkv * (it * D * 4 + (t % 64 + 1) * D * 2 * 2) + 2 * B * Hq * D * 2
    bytes_total += act * 64 * D * 2 * 2
    for _ in range(args.warmup):
        run(min(S, 8))
    torch.cuda.synchronize()
    nsum.fill_(w.T // 64)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    run(S)
    e1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    us = e0.elapsed_time(e1) * 1e3 / S
    gbs = bytes_total / S / (us * 1e-6) / 1e9
    frac_active = act / (B * Hkv * sum((w.T + s) // 64 for s in range(S)))
    log(f"decode {us:.1f} us/step ({(t1 - t0) * 1e6 / S:.1f} wall), {gbs:.0f} GB/s, "
        f"active fraction {frac_active:.3f}")
    o_last = out.clone()

    # the same steps with estimate_diagonal (the own chunk's partial summary in the entmax)
    us_d = None
    if not args.no_diag:
        nsum.fill_(w.T // 64)
        run(min(S, 8), diag=True)
        torch.cuda.synchronize()
        nsum.fill_(w.T // 64)
        e0.record()
        run(S, diag=True)
        e1.record()
        torch.cuda.synchronize()
        us_d = e0.elapsed_time(e1) * 1e3 / S
        nsum.fill_(w.T // 64)
        log(f"decode with estimate_diagonal {us_d:.1f} us/step")

    # the same steps over paged caches: every chunk of every sequence in a shuffled page of
    # one pool [pages, Hkv, 64, D], appends through the block table
    nc_ = -(-TT // 64)
    perm = torch.randperm(B * nc_, generator=torch.Generator().manual_seed(20267000)).to(dev)

    def to_pages(cache):
        pad = torch.zeros((B, Hkv, nc_ * 64, D), dtype=cache.dtype, device=dev)
        pad[:, :, :TT] = cache
        pool = torch.empty((B * nc_, Hkv, 64, D), dtype=cache.dtype, device=dev)
        pool[perm] = pad.view(B, Hkv, nc_, 64, D).permute(0, 2, 1, 3, 4).reshape(B * nc_, Hkv, 64, D)
        return pool
    kp, vp = to_pages(kc), to_pages(vc)
    del kc, vc
    torch.cuda.empty_cache()
    table = perm.view(B, nc_).to(torch.int32).contiguous()
    summ.zero_()
    nsum.zero_()
    dash.append_chunk_paged(kp, table, hc, init_len, summ, nsum, Hq=Hq, enable_gqa=True)

    def run_paged(n):
        for s in range(n):
            L = w.T + 1 + s
            dash.decode_paged(qs[s], kp, vp, table, lens_all[s], summ, alpha=w.alpha,
                              enable_gqa=True, out=out, workspace=ws)
            if L % 64 == 0:
                dash.append_chunk_paged(kp, table, hc, lens_all[s], summ, nsum, Hq=Hq,
                                        enable_gqa=True)
    torch.cuda.synchronize()
    e0.record()
    run_paged(S)
    e1.record()
    torch.cuda.synchronize()
    us_p = e0.elapsed_time(e1) * 1e3 / S
    same = bool(torch.equal(out, o_last))
    log(f"decode (paged caches) {us_p:.1f} us/step; last step identical to contiguous: {same}")
    del kp, vp, qs, summ, ws
    torch.cuda.empty_cache()
    gbs_p = bytes_total / S / (us_p * 1e-6) / 1e9
    return {"workload": w.name, "us_per_step": us, "tokens_per_s": B / (us * 1e-6),
            "steps": S, "algorithmic_bytes_per_step": bytes_total / S,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": gbs / PEAK_HBM_GBS},
            "active_fraction": frac_active,
            "paged": {"us_per_step": us_p, "achieved_gbs": gbs_p, "frac": gbs_p / PEAK_HBM_GBS,
                      "pages": B * nc_, "identical_to_contiguous": same},
            "estimate_diagonal": {"us_per_step": us_d}}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_worker_init():
    from threadpoolctl import threadpool_limits
    global _LIMITS
    _LIMITS = threadpool_limits(limits=1)      # one BLAS thread per worker process


def _oracle_worker(task):
    """One worker's share of the sampled rows: the oracle's prefill on them, over inputs
    memory-mapped from the files the parent wrote.  Returns (rows done, seconds)."""
    d, rows, alpha = task
    from oracle import dash_oracle as O
    x = {n: np.load(os.path.join(d, n + ".npy"), mmap_mode="r")
         for n in ("q", "k", "v", "head_cls", "summ")}
    t0 = time.perf_counter()
    O.prefill(x["q"], x["k"], x["v"], np.asarray(x["head_cls"]), alpha=alpha, rows=rows,
              summaries=np.asarray(x["summ"]))
    return len(rows), time.perf_counter() - t0


def cpu_baseline(args, w, x):
    """The float64 oracle, as it stands, on the host's cores: Stage 0 over every chunk in the
    parent, then a uniformly sampled set of rows spread over one worker process per core
    (one BLAS thread each, inputs memory-mapped), timed from the moment the warmed-up pool
    gets its tasks; extrapolated to the whole sequence."""
    import multiprocessing as mp
    import shutil
    import tempfile
    from threadpoolctl import threadpool_limits
    from oracle import dash_oracle as O
    cores = max(1, min(args.cpu_workers, os.cpu_count() or 1))
    rng = np.random.default_rng(12345)
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        summ = O.chunk_summaries(x["k"], x["head_cls"], 1.0 / math.sqrt(w.D))
        t_s0 = time.perf_counter() - t0
        probe = rng.integers(0, w.T, size=2)
        t0 = time.perf_counter()
        O.prefill(x["q"], x["k"], x["v"], x["head_cls"], alpha=w.alpha, rows=probe,
                  summaries=summ)
        t_probe = (time.perf_counter() - t0) / 2
    n = int(max(cores, min(128 * cores, cores * args.cpu_seconds / max(t_probe, 1e-3))))
    rows = rng.integers(0, w.T, size=n)
    order = rng.permutation(n)
    tmp = tempfile.mkdtemp(prefix="dash_oracle_")
    try:
        for name, arr in (("q", x["q"]), ("k", x["k"]), ("v", x["v"]),
                          ("head_cls", x["head_cls"]), ("summ", summ)):
            np.save(os.path.join(tmp, name + ".npy"), arr)
        tasks = [(tmp, rows[order[i::cores]], w.alpha) for i in range(cores)]
        ctx = mp.get_context("spawn")
        with ctx.Pool(cores, initializer=_oracle_worker_init) as pool:
            pool.map(abs, range(cores))                 # workers started and imported
            t0 = time.perf_counter()
            done = pool.map(_oracle_worker, tasks)
            t_rows = time.perf_counter() - t0
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    cpu_s = sum(d[1] for d in done)
    t_full = t_s0 + t_rows / n * w.T
    log(f"oracle: stage 0 {t_s0:.1f}s; {n} rows on {cores} processes in {t_rows:.1f}s wall "
        f"({cpu_s:.0f} CPU-s) -> {t_full:.0f}s for the sequence")
    return {"value": w.B * w.T / t_full, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": _cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"{n} uniformly sampled rows of the {w.name} workload (all heads) on "
                      f"{cores} worker processes with one BLAS thread each, plus Stage 0 over "
                      f"every chunk; {t_rows:.1f}s wall for the rows, extrapolated to all "
                      f"{w.T} rows"}


def bench_sweep(args, dash, torch):
    """Sparsity sweep: the 64K, 32/8-head prefill at alpha in {1.25, 1.5, 2} x planted-needle
    count per query block ~ Poisson(2, 8, 32).  One JSON line per cell on stdout (this mode
    is a report, not the benchmark line)."""
    from long_context_sparse_stage0_amd import synth
    from long_context_sparse_stage0_amd.workloads import SWEEP
    dev = torch.device("cuda:0")
    for w in SWEEP:
        x = synth.prefill_inputs(w)
        q, k, v, hc = (torch.from_numpy(x[n]).to(torch.bfloat16).to(dev)
                       for n in ("q", "k", "v", "head_cls"))
        del x
        B, Hq, T, D = q.shape
        nc = -(-T // 64)
        W = -(-nc // 64)
        out = torch.empty_like(q)
        ab = torch.empty((B, w.Hkv, T, W), dtype=torch.int64, device=dev)
        p = dash.make_params(B, Hq, w.Hkv, T, D, alpha=w.alpha, gamma=w.gamma, enable_gqa=True,
                             dtype=torch.bfloat16)
        ws = dash.alloc_workspace(dash.workspace_size("prefill", p), dev)
        kw = dict(alpha=w.alpha, gamma=w.gamma, enable_gqa=True)
        dash.prefill_stage(0, q, k, v, hc, out, ws, **kw)
        dash.prefill_stage(3, q, k, v, hc, out, ws, **kw)
        dash.prefill_stage(1, q, k, v, hc, out, ws, active_blocks=ab, **kw)
        torch.cuda.synchronize()
        pc = popcount64(ab).sum(dim=-1).to(torch.float64)
        routed = (torch.arange(T, device=dev) // 64).to(torch.float64).sum() * B * w.Hkv
        active = float(pc.sum() / routed)
        flops2 = float(w.G * 4 * D * (64.0 * pc.sum()
                                      + B * w.Hkv * (torch.arange(T, device=dev) % 64 + 1).sum()))
        del ab, pc

        def step():
            for s in STAGES:
                dash.prefill_stage(s, q, k, v, hc, out, ws, **kw)
        for _ in range(max(1, args.warmup)):
            step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            step()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        line = {"workload": w.name, "alpha": w.alpha, "needle_lambda": w.needle_lambda,
                "active_fraction": active, "ms_per_prefill": ms, "tokens_per_s": B * T / (ms / 1e3),
                "stage2_algorithmic_flops": flops2}
        print(json.dumps(line), flush=True)
        log(f"{w.name}: active {active:.3f}, {ms:.2f} ms, {B * T / (ms / 1e3):.3e} tokens/s")
        del q, k, v, hc, out, ws
        torch.cuda.empty_cache()


def bench_short(args, dash, torch):
    """Short contexts (a report, not the benchmark line): the 16K workload's shape (32/8 heads,
    D = 128, bf16, needles +3 sigma) at T = 2K..16K; per T, the entmax prefill, the same
    prefill with the top-k comparison router at k = entmax's mean active chunks per row, and
    the dense causal kernel.  One JSON line per T on stdout."""
    import dataclasses
    from long_context_sparse_stage0_amd import synth
    from long_context_sparse_stage0_amd.workloads import PREFILL_16K_GQA as base
    dev = torch.device("cuda:0")
    for T in (2048, 4096, 8192, 16384):
        w = dataclasses.replace(base, name=f"prefill_{T // 1024}k_gqa32x8", T=T)
        x = synth.prefill_inputs(w)
        q, k, v, hc = (torch.from_numpy(x[n]).to(torch.bfloat16).to(dev)
                       for n in ("q", "k", "v", "head_cls"))
        del x
        B, Hq, _, D = q.shape
        W = -(-(-(-T // 64)) // 64)
        out = torch.empty_like(q)
        ab = torch.empty((B, w.Hkv, T, W), dtype=torch.int64, device=dev)
        p = dash.make_params(B, Hq, w.Hkv, T, D, alpha=w.alpha, enable_gqa=True,
                             dtype=torch.bfloat16)
        ws = dash.alloc_workspace(dash.workspace_size("prefill", p), dev)
        dash.prefill_stage(0, q, k, v, hc, out, ws, enable_gqa=True)
        dash.prefill_stage(1, q, k, v, hc, out, ws, enable_gqa=True, active_blocks=ab)
        torch.cuda.synchronize()
        routed = float((torch.arange(T, device=dev) // 64).sum()) * B * w.Hkv
        act = float(popcount64(ab).sum())
        kk = max(1, int(round(act / (B * w.Hkv * T))))

        def timed(fn, n):
            fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(n):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / n

        def prefill(topk):
            for s in STAGES:
                dash.prefill_stage(s, q, k, v, hc, out, ws, enable_gqa=True, topk=topk)

        def stage1(topk):
            dash.prefill_stage(1, q, k, v, hc, out, ws, enable_gqa=True, topk=topk)
        n = max(3, args.steps)
        ms_e, s1_e = timed(lambda: prefill(0), n), timed(lambda: stage1(0), n)
        ms_k, s1_k = timed(lambda: prefill(kk), n), timed(lambda: stage1(kk), n)
        pd = dash.make_params(B, Hq, w.Hkv, T, D, enable_gqa=True, dtype=torch.bfloat16)
        wsd = dash.alloc_workspace(dash.workspace_size("dense", pd), dev)
        ms_d = timed(lambda: dash.dense_causal(q, k, v, enable_gqa=True, out=out, workspace=wsd), n)
        line = {"workload": w.name, "T": T, "entmax_active_fraction": act / routed,
                "entmax_prefill_ms": ms_e, "entmax_stage1_ms": s1_e,
                "topk_k": kk, "topk_prefill_ms": ms_k, "topk_stage1_ms": s1_k,
                "dense_ms": ms_d, "speedup_entmax_over_dense": ms_d / ms_e}
        print(json.dumps(line), flush=True)
        log(f"{w.name}: entmax {ms_e:.3f} ms (stage 1 {s1_e:.3f}), top-{kk} {ms_k:.3f} ms "
            f"(stage 1 {s1_k:.3f}), dense {ms_d:.3f} ms, active {act / routed:.3f}")
        del q, k, v, hc, out, ws, wsd, ab
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--decode-steps", type=int, default=256)
    ap.add_argument("--workload", default="prefill_128k_gqa32x2")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-topk", action="store_true",
                    help="skip timing the top-k comparison router")
    ap.add_argument("--no-diag", action="store_true",
                    help="skip timing the prefill with estimate_diagonal")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip timing the backward pass")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target wall seconds of the CPU oracle's sampled rows")
    ap.add_argument("--cpu-workers", type=int, default=16,
                    help="oracle worker processes (at most the host's CPU count)")
    ap.add_argument("--short", action="store_true",
                    help="report entmax / top-k / dense at T = 2K..16K (one JSON line per T)")
    ap.add_argument("--sweep", action="store_true",
                    help="report the 64K sparsity sweep (one JSON line per cell) instead")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

    import torch
    from long_context_sparse_stage0_amd import dash
    from long_context_sparse_stage0_amd.workloads import ALL, DECODE_64K_B16
    dash.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.sweep:
        bench_sweep(args, dash, torch)
        return
    if args.short:
        bench_short(args, dash, torch)
        return
    w = ALL[args.workload]
    pre = bench_prefill(args, w, dash, torch)
    dec = None if args.no_decode else bench_decode(args, DECODE_64K_B16, dash, torch)
    cpu = None if args.no_cpu_baseline else cpu_baseline(args, w, pre["x"])

    line = {
        "metric": METRIC, "value": pre["tokens_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": pre["ms"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "T": w.T, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D,
                   "alpha": w.alpha, "needle_amp": w.needle_amp,
                   "zero_weight_fraction": pre["zero_frac"]},
        "roofline": pre["roofline"],
        "cpu_baseline": cpu,
        "stages_ms": {"stage0_summaries": pre["stages_ms"][0],
                      "vtranspose": pre["stages_ms"][3],
                      "stage1_route": pre["stages_ms"][1], "stage2_attend": pre["stages_ms"][2]},
        "stage0": pre["stage0"],
        "vtranspose": pre["vtranspose"],
        "stage1": pre["stage1"],
        "dense": pre.get("dense"),
        "topk_router": pre.get("topk"),
        "estimate_diagonal": pre.get("diag"),
        "backward": pre.get("backward"),
        "decode": dec,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
