"""HBM traffic and MFMA use of the library's kernels, from rocprofv3 hardware counters.

Run once under each of four rocprofv3 passes (one counter group per pass), then summarise:

    cd /tmp && export TMPDIR=/tmp && cd <repo>
    rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out>/traffic/fetch -o fetch \\
        -- python3 -m long_context_sparse_stage0_amd.traffic run
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d <out>/traffic/write -o write \\
        -- python3 -m long_context_sparse_stage0_amd.traffic run
    rocprofv3 --kernel-trace --output-format csv -d <out>/traffic/trace -o trace \\
        -- python3 -m long_context_sparse_stage0_amd.traffic run
    rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE \\
        --output-format csv -d <out>/traffic/mfma -o mfma \\
        -- python3 -m long_context_sparse_stage0_amd.traffic run
    python3 -m long_context_sparse_stage0_amd.traffic summarize <out>/traffic

`backward` runs the 128K backward pass three times (for a kernel-trace run), and
`ktable <stats.csv> <out.md> <title> <command> [note]` writes a rocprofv3 kernel-stats CSV
as a markdown table of the library's kernels.

`run` launches, on the 128K prefill workload, the full prefill once (to build the mask and
the weights), then Stage 2 alone three times; then, on the 64K decode workload, the bulk
summary append and kDecodeSteps decode steps; and, as the last dispatch, a plain
elementwise copy (dst = src + 1) of 1 GiB of fp32: one dispatch that reads 1 GiB and
writes 1 GiB, the calibration kernel.  `summarize` reads the per-dispatch FETCH_SIZE /
WRITE_SIZE (KiB) and scales each counter by (known copy bytes / the copy's counter
reading).  It writes profiles/stage2_traffic.json (read by bench.py, tagged with the hash
of the Stage 2 source so a changed kernel invalidates it) with a short text summary next
to it, and, when the trace and MFMA passes are present, profiles/kernels_hbm_mfma.md: per
kernel, the counted HBM bytes, the mean duration, the achieved GB/s against the 8 TB/s
peak, and for the matrix-core kernels the executed bf16 MFMA flops (512 per MOP) and the
MFMA busy fraction (busy cycles / (GPU-active cycles x 1024 SIMDs); on this part
GRBM_GUI_ACTIVE reads the sum of the 8 XCDs' cycles, so it is divided by 8).
"""
import csv
import glob
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
COPY_BYTES = 1 << 30
STAGE2_SRC = os.path.join(ROOT, "long_context_sparse_stage0_amd", "csrc", "attend_mfma.hip")
OUT_JSON = os.path.join(ROOT, "profiles", "stage2_traffic.json")
OUT_MD = os.path.join(ROOT, "profiles", "stage2_traffic_prefill128k.md")
OUT_ALL = os.path.join(ROOT, "profiles", "kernels_hbm_mfma.md")
kDecodeSteps = 16
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
SIMDS = 1024                     # 256 CUs x 4 SIMDs
XCDS = 8                         # GRBM_GUI_ACTIVE reads the sum of the 8 XCDs' busy cycles


def source_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def run():
    import torch
    sys.path.insert(0, ROOT)
    from long_context_sparse_stage0_amd import dash, synth
    from long_context_sparse_stage0_amd.workloads import PREFILL_128K_GQA as w
    dash.load()
    x = synth.prefill_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v, hc = (torch.from_numpy(x[n]).to(torch.bfloat16).to(dev)
                   for n in ("q", "k", "v", "head_cls"))
    del x
    out = torch.empty_like(q)
    p = dash.make_params(w.B, w.Hq, w.Hkv, w.T, w.D, alpha=w.alpha, gamma=w.gamma,
                         enable_gqa=True, dtype=torch.bfloat16)
    ws = dash.alloc_workspace(dash.workspace_size("prefill", p), dev)
    kw = dict(alpha=w.alpha, gamma=w.gamma, enable_gqa=True)
    dash.prefill(q, k, v, hc, out=out, workspace=ws, **kw)
    for _ in range(3):
        dash.prefill_stage(2, q, k, v, hc, out, ws, **kw)
    torch.cuda.synchronize()
    del q, k, v, hc, out, ws
    torch.cuda.empty_cache()
    _run_decode(torch, dash, synth, dev)
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.add(src, 1.0, out=dst)        # calibration: one dispatch, 1 GiB read + 1 GiB written
    torch.cuda.synchronize()
    print(f"traffic run done ({w.name})", flush=True)


def _run_decode(torch, dash, synth, dev):
    """kDecodeSteps steps of the 64K decode workload from a bulk-appended summary cache."""
    from long_context_sparse_stage0_amd.workloads import DECODE_64K_B16 as w
    x = synth.decode_inputs(w)
    kc = torch.from_numpy(x["k_cache"]).to(torch.bfloat16).to(dev)
    vc = torch.from_numpy(x["v_cache"]).to(torch.bfloat16).to(dev)
    hc = torch.from_numpy(x["head_cls"]).to(torch.bfloat16).to(dev)
    qs = torch.from_numpy(x["q_steps"][:kDecodeSteps]).to(torch.bfloat16).to(dev)
    del x
    B, Hkv, TT, D = kc.shape
    Hq = qs.shape[2]
    summ = torch.zeros((B, Hkv, -(-TT // 64), D), dtype=torch.float32, device=dev)
    nsum = torch.zeros(B, dtype=torch.int32, device=dev)
    dash.append_chunk(kc, hc, torch.full((B,), w.T, dtype=torch.int32, device=dev), summ, nsum,
                      Hq=Hq, enable_gqa=True)
    p = dash.make_params(B, Hq, Hkv, TT, D, alpha=w.alpha, enable_gqa=True, dtype=torch.bfloat16)
    ws = dash.alloc_workspace(dash.workspace_size("decode", p), dev)
    out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev)
    for s in range(kDecodeSteps):
        lens = torch.full((B,), w.T + 1 + s, dtype=torch.int32, device=dev)
        dash.decode(qs[s], kc, vc, lens, summ, alpha=w.alpha, enable_gqa=True, out=out,
                    workspace=ws)
    torch.cuda.synchronize()
    del kc, vc, qs, summ, ws
    torch.cuda.empty_cache()


def _dispatches(folder, counter):
    rows = []
    for f in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r.get("Counter_Name") != counter:
                    continue
                rows.append((int(r.get("Dispatch_Id", 0) or 0), r["Kernel_Name"],
                             float(r["Counter_Value"])))
    # one value per dispatch (counters are reported per dimension instance on some setups)
    agg = {}
    for d, name, v in rows:
        key = (d, name)
        agg[key] = agg.get(key, 0.0) + v
    return [(d, name, v) for (d, name), v in sorted(agg.items())]


def summarize(base):
    from long_context_sparse_stage0_amd.workloads import PREFILL_128K_GQA as w
    res = {}
    for counter, sub in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
        ds = _dispatches(os.path.join(base, sub), counter)
        st2 = [v for _, n, v in ds if "k_attend_mfma" in n and "true" not in n]
        other = [(d, v, n) for d, n, v in ds if "dash::" not in n]
        if not st2 or not other:
            raise SystemExit(f"{counter}: no Stage 2 or copy dispatch found in {base}/{sub}")
        _, copy_kib, copy_name = max(other)      # the last dispatch of the run
        if "elementwise" not in copy_name:
            raise SystemExit(f"{counter}: last dispatch is not the calibration copy: {copy_name}")
        factor = (COPY_BYTES / 1024.0) / copy_kib
        # the first Stage 2 dispatch belongs to the full prefill; all are the same work
        kib = sum(st2) / len(st2)
        res[counter] = dict(stage2_kib_per_dispatch=kib, dispatches=len(st2),
                            copy_kernel=copy_name[:120], copy_kib=copy_kib,
                            scale_factor=factor, stage2_bytes=kib * 1024.0 * factor)
    total = res["FETCH_SIZE"]["stage2_bytes"] + res["WRITE_SIZE"]["stage2_bytes"]
    doc = {"workload": w.name, "kernel": "k_attend_mfma (Stage 2, sparse)",
           "source_sha256_16": source_hash(STAGE2_SRC), "bytes_per_launch": total,
           "fetch_bytes": res["FETCH_SIZE"]["stage2_bytes"],
           "write_bytes": res["WRITE_SIZE"]["stage2_bytes"], "counters": res}
    os.makedirs(os.path.dirname(OUT_JSON), exist_ok=True)
    with open(OUT_JSON, "w") as f:
        json.dump(doc, f, indent=1)
    lines = [
        f"# Stage 2 HBM traffic, {w.name}",
        "",
        "Commands (repo root; rocprofv3 needs `cd /tmp && export TMPDIR=/tmp` first):",
        "",
        f"    rocprofv3 --pmc FETCH_SIZE --output-format csv -d {base}/fetch -o fetch "
        "-- python3 -m long_context_sparse_stage0_amd.traffic run",
        f"    rocprofv3 --pmc WRITE_SIZE --output-format csv -d {base}/write -o write "
        "-- python3 -m long_context_sparse_stage0_amd.traffic run",
        f"    python3 -m long_context_sparse_stage0_amd.traffic summarize {base}",
        "",
        f"Stage 2 source hash {doc['source_sha256_16']}.",
        "",
        "| counter | Stage 2 KiB/dispatch | copy kernel KiB (1 GiB moved) | scale | Stage 2 bytes/launch |",
        "|---|---|---|---|---|",
    ]
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        r = res[c]
        lines.append(f"| {c} | {r['stage2_kib_per_dispatch']:.4g} | {r['copy_kib']:.6g} | "
                     f"{r['scale_factor']:.4f} | {r['stage2_bytes']:.4g} |")
    lines += ["", f"Total HBM traffic per Stage 2 launch: {total:.4g} bytes "
              f"({total / 2**30:.2f} GiB).", ""]
    with open(OUT_MD, "w") as f:
        f.write("\n".join(lines))
    print(json.dumps(doc))
    per = report(base, {c: res[c]["scale_factor"] for c in res})
    if per:
        print(json.dumps(per))


def _rows(folder, pattern="*counter_collection.csv"):
    out = []
    for f in glob.glob(os.path.join(folder, "**", pattern), recursive=True):
        with open(f) as fh:
            out.extend(csv.DictReader(fh))
    return out


def _group(name, did, first_route):
    """Library kernel -> row label (None for other kernels)."""
    if "dash::" not in name and "_ZN4dash" not in name:
        return None
    if "k_stage0" in name:
        return "Stage 0 summaries (k_stage0, prefill)" if did < first_route \
            else "decode summary append (k_stage0)"
    for key, label in (("k_vtranspose", "Stage 0 chunk-transposed V (k_vtranspose)"),
                       ("k_route_mfma", "Stage 1 router (k_route_mfma, all launch shapes)"),
                       ("k_decode_scores", "decode scores (k_decode_scores)"),
                       ("k_decode_route", "decode route (k_decode_route)"),
                       ("k_decode_attend", "decode attend (k_decode_attend)"),
                       ("k_decode_combine", "decode combine (k_decode_combine)")):
        if key in name:
            return label
    if "k_attend_mfma" in name:
        return None if "true" in name else "Stage 2 sparse attention (k_attend_mfma)"
    return None


def report(base, factors):
    """Per-kernel table from the FETCH/WRITE, kernel-trace and MFMA passes."""
    trace = _rows(os.path.join(base, "trace"), "*kernel_trace.csv")
    if not trace:
        return None
    by_id = {}
    for r in trace:
        by_id[int(r["Dispatch_Id"])] = (r["Kernel_Name"],
                                        (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9)
    first_route = min([d for d, (n, _) in by_id.items() if "k_route_mfma" in n] or [0])
    stats = {}

    def add(label, key, v):
        st = stats.setdefault(label, {})
        st[key] = st.get(key, 0.0) + v

    for d, (n, sec) in by_id.items():
        g = _group(n, d, first_route)
        if g:
            add(g, "n", 1)
            add(g, "sec", sec)
    def first_route_of(ids_names):          # each pass numbers its own dispatches
        return min([d for d, n in ids_names if "k_route_mfma" in n] or [0])

    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        ds = _dispatches(os.path.join(base, counter.split("_")[0].lower()), counter)
        fr = first_route_of([(d, n) for d, n, _ in ds])
        for d, n, kib in ds:
            g = _group(n, d, fr)
            if g:
                add(g, counter, kib * 1024.0 * factors[counter])
    mf = {}
    for r in _rows(os.path.join(base, "mfma")):
        key = (int(r.get("Dispatch_Id", 0) or 0), r["Kernel_Name"])
        c, v = r.get("Counter_Name"), float(r["Counter_Value"])
        e = mf.setdefault(key, {})
        e[c] = max(e.get(c, 0.0), v) if c == "GRBM_GUI_ACTIVE" else e.get(c, 0.0) + v
    fr = first_route_of(list(mf.keys()))
    for (d, n), e in mf.items():
        g = _group(n, d, fr)
        if g:
            add(g, "mops", e.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0))
            add(g, "busy", e.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0))
            add(g, "gui", e.get("GRBM_GUI_ACTIVE", 0.0))
    lines = [
        "# HBM traffic and MFMA use per kernel (128K prefill, 64K decode)",
        "",
        "Commands (repo root; rocprofv3 needs `cd /tmp && export TMPDIR=/tmp` first): the four",
        "rocprofv3 passes over `python3 -m long_context_sparse_stage0_amd.traffic run` listed in",
        "that module's docstring (FETCH_SIZE; WRITE_SIZE; --kernel-trace; SQ_INSTS_VALU_MFMA_MOPS_BF16",
        "SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE), then",
        "",
        f"    python3 -m long_context_sparse_stage0_amd.traffic summarize {base}",
        "",
        f"Counter bytes are scaled by the calibration copy (FETCH_SIZE x{factors['FETCH_SIZE']:.4f}, "
        f"WRITE_SIZE x{factors['WRITE_SIZE']:.4f}).  The run holds one full 128K prefill plus three",
        f"Stage 2 launches, and {kDecodeSteps} steps of the 64K decode workload (B = 16).  GB/s =",
        "counted HBM bytes / summed kernel time; MFMA busy = busy cycles / (GPU-active cycles x",
        "1024 SIMDs), where GRBM_GUI_ACTIVE reads the sum over the 8 XCDs and is divided by 8;",
        "executed TFLOP/s = 512 x MOPs / kernel time.",
        "",
        "| kernel | dispatches | mean us | HBM bytes / dispatch | HBM GB/s | % of 8 TB/s | "
        "bf16 MFMA TFLOP/s executed | MFMA busy |",
        "|---|---|---|---|---|---|---|---|",
    ]
    order = ["Stage 0 summaries (k_stage0, prefill)", "Stage 0 chunk-transposed V (k_vtranspose)",
             "Stage 1 router (k_route_mfma, all launch shapes)",
             "Stage 2 sparse attention (k_attend_mfma)", "decode summary append (k_stage0)",
             "decode scores (k_decode_scores)", "decode route (k_decode_route)",
             "decode attend (k_decode_attend)", "decode combine (k_decode_combine)"]
    doc = {}
    for g in order:
        st = stats.get(g)
        if not st or not st.get("n"):
            continue
        n, sec = st["n"], st["sec"]
        by = st.get("FETCH_SIZE", 0.0) + st.get("WRITE_SIZE", 0.0)
        gbs = by / sec / 1e9 if sec > 0 else 0.0
        tfl = st.get("mops", 0.0) * 512 / sec / 1e12 if sec > 0 else 0.0
        busy = st["busy"] / (st["gui"] / XCDS * SIMDS) if st.get("gui") else 0.0
        doc[g] = dict(dispatches=n, mean_us=sec / n * 1e6, bytes_per_dispatch=by / n, gbs=gbs,
                      mfma_tflops=tfl, mfma_busy=busy)
        mf_cols = f"{tfl:.0f} | {100 * busy:.1f}%" if st.get("mops") else "- | -"
        lines.append(f"| {g} | {n:.0f} | {sec / n * 1e6:.1f} | {by / n:.4g} | {gbs:.0f} | "
                     f"{100 * gbs / PEAK_HBM_GBS:.1f}% | {mf_cols} |")
    lines.append("")
    with open(OUT_ALL, "w") as f:
        f.write("\n".join(lines))
    return doc


def backward():
    """The 128K backward pass: dash_prefill_train once, then dash_prefill_backward three times
    with a seeded dL/dout (for a kernel-trace run)."""
    import torch
    sys.path.insert(0, ROOT)
    from long_context_sparse_stage0_amd import dash, synth
    from long_context_sparse_stage0_amd.workloads import PREFILL_128K_GQA as w
    dash.load()
    x = synth.prefill_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v, hc = (torch.from_numpy(x[n]).to(torch.bfloat16).to(dev)
                   for n in ("q", "k", "v", "head_cls"))
    del x
    g = torch.Generator(device="cpu").manual_seed(7)
    do = torch.randn(q.shape, generator=g).to(torch.bfloat16).to(dev)
    kw = dict(alpha=w.alpha, gamma=w.gamma, enable_gqa=True)
    out, lse = dash.prefill_train(q, k, v, hc, **kw)
    p = dash.make_params(w.B, w.Hq, w.Hkv, w.T, w.D, alpha=w.alpha, gamma=w.gamma,
                         enable_gqa=True, dtype=torch.bfloat16)
    ws = dash.alloc_workspace(dash.workspace_size("backward", p), dev)
    for _ in range(3):
        dash.prefill_backward(q, k, v, hc, out, do, lse, workspace=ws, **kw)
    torch.cuda.synchronize()
    print("backward done", flush=True)


def ktable(stats_csv, out_md, title, command, note=""):
    """Write a rocprofv3 kernel-stats CSV (library kernels only) as a markdown table."""
    rows = []
    with open(stats_csv) as f:
        for r in csv.DictReader(f):
            if "dash::" not in r["Name"] and "_ZN4dash" not in r["Name"]:
                continue
            rows.append((float(r["TotalDurationNs"]), r["Name"], int(r["Calls"]),
                         float(r["AverageNs"]), float(r["MinNs"]), float(r["MaxNs"])))
    rows.sort(reverse=True)
    lines = [f"# {title}", "", "Command (repo root; `cd /tmp && export TMPDIR=/tmp` first, then back "
             "to the repo):", "", f"    {command}", "",
             f"Per-kernel statistics from `{os.path.basename(stats_csv)}` (library kernels only, by "
             "total time; torch helper kernels omitted), written by", "",
             f"    python3 -m long_context_sparse_stage0_amd.traffic ktable <csv> <md> ...", ""]
    if note:
        lines += [note, ""]
    lines += ["| kernel | calls | mean (us) | min (us) | max (us) | total (ms) |",
              "|---|---|---|---|---|---|"]
    for tot, name, calls, avg, mn, mx in rows:
        nm = name.replace("void ", "").replace("dash::", "").replace("|", "/")
        lines.append(f"| `{nm[:110]}` | {calls} | {avg / 1e3:.1f} | {mn / 1e3:.1f} | "
                     f"{mx / 1e3:.1f} | {tot / 1e6:.2f} |")
    lines.append("")
    with open(out_md, "w") as f:
        f.write("\n".join(lines))


if __name__ == "__main__":
    if len(sys.argv) >= 2 and sys.argv[1] == "run":
        run()
    elif len(sys.argv) >= 2 and sys.argv[1] == "backward":
        backward()
    elif len(sys.argv) >= 3 and sys.argv[1] == "summarize":
        summarize(sys.argv[2])
    elif len(sys.argv) >= 6 and sys.argv[1] == "ktable":
        ktable(*sys.argv[2:7])
    else:
        raise SystemExit(__doc__)
