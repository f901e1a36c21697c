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

    case = synth.CONFIGS[config]
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

    case = synth.CONFIGS[config]
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


def main() -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    r = sub.add_parser("run")
    r.add_argument("--config", type=int, required=True)
    s = sub.add_parser("summarize")
    s.add_argument("--config", type=int, required=True)
    s.add_argument("--fetch", required=True)
    s.add_argument("--write", required=True)
    a = ap.parse_args()
    if a.cmd == "run":
        run(a.config)
    else:
        summarize(a.config, a.fetch, a.write)


if __name__ == "__main__":
    main()
