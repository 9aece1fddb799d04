"""HBM traffic of the Stage 2 kernel, from rocprofv3 hardware counters.

Two steps, the first run twice under rocprofv3 (one counter per pass):

    cd /tmp && export TMPDIR=/tmp && cd <repo>
    rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/traffic/fetch -o fetch \\
        -- python3 -m long_context_sparse_stage0_amd.traffic run
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/traffic/write -o write \\
        -- python3 -m long_context_sparse_stage0_amd.traffic run
    python3 -m long_context_sparse_stage0_amd.traffic summarize gpurun_out/traffic

`run` launches, on the 128K prefill workload, the full prefill once (to build the mask and
the weights), then Stage 2 alone three times, then, as the last dispatch, a plain
elementwise copy (dst = src + 1) of 1 GiB of fp32: one dispatch that reads 1 GiB and
writes 1 GiB, the calibration kernel.  `summarize` reads the
per-dispatch FETCH_SIZE / WRITE_SIZE (KiB), scales each counter by (known copy bytes /
the copy's counter reading), and writes profiles/stage2_traffic.json (read by bench.py,
tagged with the hash of the Stage 2 source so a changed kernel invalidates it) and a short
text summary next to it.
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
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.add(src, 1.0, out=dst)        # calibration: one dispatch, 1 GiB read + 1 GiB written
    torch.cuda.synchronize()
    print(f"traffic run done ({w.name})", flush=True)


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
        "    rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/traffic/fetch -o fetch "
        "-- python3 -m long_context_sparse_stage0_amd.traffic run",
        "    rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/traffic/write -o write "
        "-- python3 -m long_context_sparse_stage0_amd.traffic run",
        "    python3 -m long_context_sparse_stage0_amd.traffic summarize gpurun_out/traffic",
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


if __name__ == "__main__":
    if len(sys.argv) >= 2 and sys.argv[1] == "run":
        run()
    elif len(sys.argv) >= 3 and sys.argv[1] == "summarize":
        summarize(sys.argv[2])
    else:
        raise SystemExit(__doc__)
