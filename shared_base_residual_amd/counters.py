"""HBM traffic of the split kernel (decode) or the prefill kernel from rocprofv3
hardware counters, calibrated against a plain copy of known size.

Two counter passes, each a rocprofv3 run of its own (from the repository root,
TMPDIR=/tmp), then the summary:

    rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/ctr_fetch_cfgN -o run -- \\
        python3 -m shared_base_residual_amd.counters run --config N
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/ctr_write_cfgN -o run -- \\
        python3 -m shared_base_residual_amd.counters run --config N
    python3 -m shared_base_residual_amd.counters summarize --config N \\
        --fetch gpurun_out/ctr_fetch_cfgN --write gpurun_out/ctr_write_cfgN

``run`` copies a 256 MiB device buffer once (a plain device-to-device copy:
256 MiB read and 256 MiB written), then launches the kernel of interest a few
times over rotated input sets, as bench.py does, so that each launch reads its
inputs from HBM.  ``summarize`` scales each counter's per-dispatch average for
the kernel by the copy's: bytes = counter(kernel) * (2^28 / counter(copy)),
writes the traffic per launch into profiles/counters.json (keyed by workload,
with the hash of the library sources the counters were taken on; bench.py
reports it as roofline.traffic only while the sources are unchanged) and a short
text summary beside it.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
COPY_BYTES = 256 << 20
LAUNCHES = 6

WORKLOADS = {
    1: ("decode_split_kernel", "llama8b_decode"),
    2: ("decode_split_kernel", "paged_cow_decode"),
    3: ("prefill_kernel", "baselrshared_prefill"),
    4: ("decode_split_kernel", "70b_full_depth_decode"),
}


def key_of(config: int, case) -> str:
    return (f"prefill_cfg{config}" if case.mode == "prefill" else f"decode_cfg{config}")


def run(config: int) -> None:
    sys.path.insert(0, ROOT)
    import torch

    import shared_base_residual_amd as R
    import synth

    case = synth.WORKLOADS[config]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    # calibration: one plain copy of known size
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    # the kernel of interest over rotated input sets
    if case.layers > 1:
        sets = [synth.make_inputs_torch(case, config, l, dev) for l in range(min(case.layers, 8))]
    else:
        base = synth.to_torch(synth.make_inputs(case, config), dev)
        per_set = sum(v.numel() * v.element_size() for v in base.values() if v is not None)
        reps = max(1, min(8, -(-(1 << 30) // per_set)))
        sets = [base] + [{k: (None if v is None else v.clone()) for k, v in base.items()} for _ in range(reps - 1)]
    stages = None if case.mode == "prefill" else R.STAGE_SPLIT
    torch.cuda.synchronize()
    for i in range(LAUNCHES):
        x = sets[i % len(sets)]
        R.attend(x, mode=case.mode, shared_lr=case.shared_lr, prefix_len=case.prefix_len, stages=stages)
    torch.cuda.synchronize()
    print("done", flush=True)


def _per_dispatch(d: str, counter: str):
    """(copy value, kernel values) of one pass, in KiB per dispatch."""
    paths = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not paths:
        raise SystemExit(f"no counter_collection.csv under {d}")
    copy_vals, kern_vals = [], []
    with open(paths[0]) as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") != counter:
                continue
            name, val = row.get("Kernel_Name", ""), float(row["Counter_Value"])
            if "decode_split_kernel" in name or "prefill_kernel" in name:
                kern_vals.append(val)
            elif "copy" in name.lower():
                copy_vals.append(val)
    if not copy_vals or not kern_vals:
        raise SystemExit(f"{counter}: copy or kernel dispatches missing in {paths[0]}")
    return max(copy_vals), kern_vals


def summarize(config: int, fetch_dir: str, write_dir: str) -> None:
    sys.path.insert(0, ROOT)
    import synth
    from shared_base_residual_amd.build import source_hash

    case = synth.WORKLOADS[config]
    kern, wl = WORKLOADS[config]
    cf, kf = _per_dispatch(fetch_dir, "FETCH_SIZE")
    cw, kw = _per_dispatch(write_dir, "WRITE_SIZE")
    f_fetch, f_write = COPY_BYTES / (cf * 1024.0), COPY_BYTES / (cw * 1024.0)
    fetch_b = sum(kf) / len(kf) * 1024.0 * f_fetch
    write_b = sum(kw) / len(kw) * 1024.0 * f_write
    path = os.path.join(ROOT, "profiles", "counters.json")
    data = {}
    if os.path.exists(path):
        with open(path) as f:
            data = json.load(f)
    data[key_of(config, case)] = {
        "kernel": kern, "workload": case.name, "source_hash": source_hash(),
        "bytes_per_launch": int(round(fetch_b + write_b)), "fetch_bytes": int(round(fetch_b)),
        "write_bytes": int(round(write_b)), "fetch_kib_raw": round(sum(kf) / len(kf), 1),
        "write_kib_raw": round(sum(kw) / len(kw), 1), "copy_fetch_kib": round(cf, 1), "copy_write_kib": round(cw, 1),
        "fetch_scale": round(f_fetch, 4), "write_scale": round(f_write, 4), "dispatches": len(kf),
    }
    with open(path, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
        f.write("\n")
    e = data[key_of(config, case)]
    lines = [
        f"# {kern} -- HBM traffic, {case.name}, MI355X", "",
        "Commands (repository root, TMPDIR=/tmp):", "",
        f"    rocprofv3 --pmc FETCH_SIZE --output-format csv -d {fetch_dir} -o run -- "
        f"python3 -m shared_base_residual_amd.counters run --config {config}",
        f"    rocprofv3 --pmc WRITE_SIZE --output-format csv -d {write_dir} -o run -- "
        f"python3 -m shared_base_residual_amd.counters run --config {config}",
        f"    python3 -m shared_base_residual_amd.counters summarize --config {config} --fetch {fetch_dir} "
        f"--write {write_dir}", "",
        f"Calibration: a {COPY_BYTES >> 20} MiB device-to-device copy reads FETCH_SIZE {e['copy_fetch_kib']} KiB and "
        f"WRITE_SIZE {e['copy_write_kib']} KiB; scale factors {e['fetch_scale']} (fetch) and {e['write_scale']} "
        f"(write) turn the counters into bytes.", "",
        f"Per launch ({e['dispatches']} dispatches averaged): FETCH_SIZE {e['fetch_kib_raw']} KiB -> "
        f"{e['fetch_bytes'] / 1e6:.1f} MB read; WRITE_SIZE {e['write_kib_raw']} KiB -> "
        f"{e['write_bytes'] / 1e6:.1f} MB written; traffic {e['bytes_per_launch'] / 1e6:.1f} MB.", "",
        f"Library sources hash {e['source_hash']}.", "",
    ]
    out = os.path.join(ROOT, "profiles", f"{kern}.{wl}.counters.txt")
    with open(out, "w") as f:
        f.write("\n".join(lines))
    print(json.dumps(e))


# MI355X: 256 compute units of 4 SIMDs each
SIMD_NUM = 1024


def summarize_mfma(config: int, d: str) -> None:
    """Matrix-unit utilisation of the kernel from one rocprofv3 pass with
    --pmc MfmaUtil MfmaFlopsBF16 SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE
    (MfmaUtil = MFMA-busy SIMD cycles / (GPU-active cycles x SIMDs) x 100; the
    bf16 MFMA flops are the counter's operation count x 512)."""
    sys.path.insert(0, ROOT)
    import synth
    from shared_base_residual_amd.build import source_hash

    case = synth.WORKLOADS[config]
    kern, wl = WORKLOADS[config]
    paths = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not paths:
        raise SystemExit(f"no counter_collection.csv under {d}")
    vals = {}
    with open(paths[0]) as f:
        for row in csv.DictReader(f):
            if kern not in row.get("Kernel_Name", ""):
                continue
            vals.setdefault(row["Counter_Name"], []).append(float(row["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no {kern} dispatches in {paths[0]}")
    avg = {k: sum(v) / len(v) for k, v in vals.items()}
    n = len(next(iter(vals.values())))
    util = avg.get("MfmaUtil")
    flops = avg.get("MfmaFlopsBF16")
    lines = [
        f"# {kern} -- matrix-unit (MFMA) utilisation, {case.name}, MI355X", "",
        "Commands (repository root, TMPDIR=/tmp):", "",
        f"    rocprofv3 --pmc MfmaUtil MfmaFlopsBF16 SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE --output-format csv "
        f"-d {d} -o run -- python3 -m shared_base_residual_amd.counters run --config {config}",
        f"    python3 -m shared_base_residual_amd.counters summarize-mfma --config {config} --dir {d}", "",
        f"Per dispatch ({n} dispatches averaged):", "",
        "| counter | value |", "|---|---|",
    ]
    for k in sorted(avg):
        lines.append(f"| {k} | {avg[k]:.6g} |")
    lines.append("")
    if util is not None:
        lines.append(f"MfmaUtil (rocprofv3's derived metric: SQ_VALU_MFMA_BUSY_CYCLES summed over the SIMDs / "
                     f"(GRBM_GUI_ACTIVE x {SIMD_NUM} SIMDs) x 100): **{util:.1f} %** of the SIMD cycles the matrix "
                     f"units are busy.")
    if flops is not None:
        lines.append(f"MfmaFlopsBF16: {flops / 1e12:.3f} TFLOP executed per dispatch on bf16 MFMAs "
                     f"(counted operations x 512).")
    lines += ["", f"Library sources hash {source_hash()}.", ""]
    out = os.path.join(ROOT, "profiles", f"{kern}.{wl}.mfma.txt")
    with open(out, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


def summarize_trace(config: int, d: str, bench_json: str, cmd: str) -> None:
    """Kernel durations of one rocprofv3 --kernel-trace --stats run of bench.py
    for one workload: the library's kernels from kernel_stats.csv, the average
    of the last launches of the roofline kernel (bench.py's back-to-back
    window) from kernel_trace.csv, and the bench line of the same run."""
    sys.path.insert(0, ROOT)
    import synth
    from shared_base_residual_amd.build import source_hash

    case = synth.WORKLOADS[config]
    kern, wl = WORKLOADS[config]
    with open(bench_json) as f:
        line = [l for l in f.read().splitlines() if l.startswith("{")][-1]
    rec = json.loads(line)
    roof = rec["roofline"]
    stats = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    trace = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if not stats or not trace:
        raise SystemExit(f"kernel_stats.csv / kernel_trace.csv missing under {d}")
    rows = []
    with open(stats[0]) as f:
        for r in csv.DictReader(f):
            rows.append(r)
    durs = []
    with open(trace[0]) as f:
        for r in csv.DictReader(f):
            if kern in r["Kernel_Name"]:
                durs.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    durs.sort()
    n_k = roof["launches_timed"]
    last = [x for _, x in durs[-n_k:]]
    lib_rows = [r for r in rows if "rattn" in r["Name"]]
    lines = [
        f"# {kern} -- {case.name}, MI355X", "",
        "Command (repository root, TMPDIR=/tmp):", "",
        f"    {cmd}", "",
        "Kernels of the library (kernel_stats.csv; durations in microseconds):", "",
        "| kernel | calls | avg | min | max | share of GPU time |", "|---|---|---|---|---|---|",
    ]
    for r in lib_rows:
        lines.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f} % |")
    lines += [
        "", "The bench's other kernels (input draws and copies) run outside the timed region.", "",
        f"The last {len(last)} {kern} launches in the trace (the back-to-back launches bench.py times for the "
        f"roofline) average {sum(last) / max(1, len(last)) / 1e3:.2f} us; bench.py's HIP-event average over the "
        f"same launches is {roof['avg_launch_us']} us (fraction {roof['frac']} of the {roof['peak']} "
        f"{roof['unit']} peak).", "",
        "Bench line of the same run:", "", "    " + line, "",
        f"Library sources hash {source_hash()}.", "",
    ]
    out = os.path.join(ROOT, "profiles", f"{kern}.{wl}.txt")
    with open(out, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines[:20]))


def main() -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="action", required=True)
    r = sub.add_parser("run")
    r.add_argument("--config", type=int, required=True)
    s = sub.add_parser("summarize")
    s.add_argument("--config", type=int, required=True)
    s.add_argument("--fetch", required=True)
    s.add_argument("--write", required=True)
    m = sub.add_parser("summarize-mfma")
    m.add_argument("--config", type=int, required=True)
    m.add_argument("--dir", required=True)
    t = sub.add_parser("summarize-trace")
    t.add_argument("--config", type=int, required=True)
    t.add_argument("--dir", required=True)
    t.add_argument("--bench-json", required=True)
    t.add_argument("--cmd", required=True)
    a = ap.parse_args()
    if a.action == "run":
        run(a.config)
    elif a.action == "summarize":
        summarize(a.config, a.fetch, a.write)
    elif a.action == "summarize-mfma":
        summarize_mfma(a.config, a.dir)
    else:
        summarize_trace(a.config, a.dir, a.bench_json, a.cmd)


if __name__ == "__main__":
    main()
