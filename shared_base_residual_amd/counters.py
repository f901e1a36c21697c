"""Hardware-counter and kernel-trace evidence for the benchmark's roofline
figures: HBM traffic of each measured kernel from rocprofv3 counters,
calibrated against a plain copy of known size, matrix-unit utilisation, and
kernel-trace summaries that tie a bench.py record to rocprofv3's own timings.

Workloads (``--workload``) are the bench.py records:

    decode_cfg1, decode_cfg2, decode_cfg4      the split kernel of a decode call
    prefill_cfg3                               the prefill kernel
    decode_cfg1_k8, decode_cfg4_k8             the split kernel over int8 base keys
    decode_cfg1_k8v3, decode_cfg4_k8v3         ... over int8 keys and 3-bit values
    recon_cfg1[_rope], recon_cfg4[_rope]       the rebuilt-key decode (split + merge)
    lr_prefill                                 the low-rank projection
    append                                     the paged append with copy-on-write

Traffic: two counter passes, each a rocprofv3 run of its own (repository root,
TMPDIR=/tmp, OUT any output folder), then the summary:

    rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/ctr_fetch_W -o run -- \\
        python3 -m shared_base_residual_amd.counters run --workload W
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT/ctr_write_W -o run -- \\
        python3 -m shared_base_residual_amd.counters run --workload W
    python3 -m shared_base_residual_amd.counters summarize --workload W \\
        --fetch OUT/ctr_fetch_W --write OUT/ctr_write_W

``run`` copies a 256 MiB device buffer once (a plain device-to-device copy:
256 MiB read and 256 MiB written), then makes a few calls of the workload over
rotated input sets, as bench.py does, so that each call reads its inputs from
HBM.  ``summarize`` scales each counter's per-dispatch average for the
workload's kernels by the copy's: bytes = counter(kernel) * (2^28 /
counter(copy)), sums them over the kernels of one call, writes the traffic per
call into profiles/counters.json (keyed by workload, with the hash of the
library sources the counters were taken on; bench.py reports it as
roofline.traffic only while the sources are unchanged) and a short text
summary beside it.

LDS and matrix-unit occupancy: one pass with the eight SQ counters of
SQ_COUNTERS, then ``summarize-sq --workload W --dir D``.

Kernel trace: one ``rocprofv3 --kernel-trace --stats`` run of bench.py, then
``summarize-trace --workload W`` per record, which finds the record's timed
launches in the trace (records are measured one after another, so each
kernel's launches fall into one stretch per record that uses it).
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
CALLS = 6
GAP_NS = 10_000_000  # launches of one kernel further apart than this (10 ms) belong to different records


def _synth():
    sys.path.insert(0, ROOT)
    import synth

    return synth


def _dec(cfg, name, k8=False, v3=False):
    def match(rec):
        return rec.get("config", {}).get("workload") == (_synth().WORKLOADS[cfg].name + (", int8 keys" if k8 else "") +
                                                         (", 3-bit values" if v3 else ""))
    return dict(kind="decode", config=cfg, k8=k8, v3=v3, kernels=["decode_split_kernel"],
                files=("decode_split_kernel", name), match=match)


def _rec(cfg, name, rope):
    def match(rec):
        w = rec.get("config", {})
        return (w.get("workload", "").startswith(_synth().WORKLOADS[cfg].name + ", one layer, residual keys rebuilt")
                and bool(w.get("rope")) == rope)
    return dict(kind="recon", config=cfg, rope=rope, kernels=["recon_split_kernel", "combine_kernel"],
                files=("recon_split_kernel", name), match=match)


SPECS = {
    "decode_cfg1": _dec(1, "llama8b_decode"),
    "decode_cfg2": _dec(2, "paged_cow_decode"),
    "decode_cfg4": _dec(4, "70b_full_depth_decode"),
    "prefill_cfg3": dict(kind="prefill", config=3, kernels=["prefill_kernel"],
                         files=("prefill_kernel", "baselrshared_prefill"),
                         match=lambda rec: rec.get("roofline", {}).get("kernel") == "prefill_kernel"),
    "decode_cfg1_k8": _dec(1, "llama8b_decode_int8_keys", k8=True),
    "decode_cfg4_k8": _dec(4, "70b_layer_int8_keys", k8=True),
    "decode_cfg1_k8v3": _dec(1, "llama8b_decode_int8_keys_3bit_values", k8=True, v3=True),
    "decode_cfg4_k8v3": _dec(4, "70b_layer_int8_keys_3bit_values", k8=True, v3=True),
    "recon_cfg1": _rec(1, "llama8b_decode_rebuilt_keys", False),
    "recon_cfg1_rope": _rec(1, "llama8b_decode_rebuilt_keys_rotated", True),
    "recon_cfg4": _rec(4, "70b_layer_rebuilt_keys", False),
    "recon_cfg4_rope": _rec(4, "70b_layer_rebuilt_keys_rotated", True),
    "lr_prefill": dict(kind="lr", kernels=["lr_project_kernel"], files=("lr_project_kernel", "lr_prefill"),
                       match=lambda rec: rec.get("config", {}).get("workload") == _synth().LR_PREFILL["name"]),
    "append": dict(kind="append", kernels=["append_kv_kernel"], files=("append_kv_kernel", "paged_append_cow"),
                   match=lambda rec: rec.get("config", {}).get("workload") == _synth().APPEND["name"]),
}


def _rotated_sets(case, seed, dev, max_sets=8):
    """Input sets of one layer shape, enough of them (up to 8) that the calls
    together read about 1 GiB, so each call finds its inputs in HBM."""
    synth = _synth()
    if case.layers > 1:
        return [synth.make_inputs_torch(case, seed, l, dev) for l in range(min(case.layers, max_sets))]
    base = synth.to_torch(synth.make_inputs(case, seed), dev)
    per_set = sum(v.numel() * v.element_size() for v in base.values() if v is not None)
    reps = max(1, min(max_sets, -(-(1 << 30) // per_set)))
    return [base] + [{k: (None if v is None else v.clone()) for k, v in base.items()} for _ in range(reps - 1)]


def run(key: str) -> None:
    synth = _synth()
    import numpy as np
    import torch

    import shared_base_residual_amd as R

    spec = SPECS[key]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    # calibration: one plain copy of known size
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    kind = spec["kind"]
    if kind in ("decode", "prefill"):
        case = synth.WORKLOADS[spec["config"]]
        sets = _rotated_sets(case, spec["config"], dev)
        scales = [None] * len(sets)
        if spec.get("k8"):
            for i, st in enumerate(sets):
                codes, sc = R.quantize_keys(st["k_base"])
                st["k_base"] = codes
                scales[i] = float(sc.cpu().numpy()[0])
        if spec.get("v3"):
            for st in sets:
                st["v_base"], st["v_scale"] = R.quantize_values(st["v_base"])
        stages = None if case.mode == "prefill" else R.STAGE_SPLIT
        torch.cuda.synchronize()
        for i in range(CALLS):
            x = sets[i % len(sets)]
            R.attend(x, mode=case.mode, shared_lr=case.shared_lr, prefix_len=case.prefix_len, stages=stages,
                     k_scale=scales[i % len(sets)])
    elif kind == "recon":
        case = synth.WORKLOADS[spec["config"]].replace(layers=1)
        sets = _rotated_sets(case, spec["config"], dev)
        theta = torch.from_numpy(synth.rope_theta(case.head_dim)).to(dev) if spec["rope"] else None
        desc = R.describe(sets[0]["q"], sets[0]["k_base"], sets[0]["lk"], sets[0]["bk"])
        ws = torch.empty(R.workspace_bytes(desc, R.RATTN_OP_RECONSTRUCT), device=dev, dtype=torch.uint8)
        out = torch.empty(tuple(sets[0]["q"].shape), device=dev, dtype=torch.float32)
        torch.cuda.synchronize()
        for i in range(CALLS):
            R.decode_reconstruct(sets[i % len(sets)], rope_theta=theta, out=out, workspace=ws)
    elif kind == "lr":
        c = synth.LR_PREFILL
        g = torch.Generator(device=dev)
        g.manual_seed(7)
        xs = [torch.randn((1, c["T"], c["d_in"]), generator=g, device=dev).to(torch.bfloat16) for _ in range(2)]
        ak = (torch.randn((c["n_sets"], c["r"], c["d_in"]), generator=g, device=dev) * 0.05).to(torch.bfloat16)
        av = (torch.randn((c["n_sets"], c["r"], c["d_in"]), generator=g, device=dev) * 0.05).to(torch.bfloat16)
        lk = torch.empty((c["n_sets"], c["T"], c["r"]), device=dev, dtype=torch.bfloat16)
        lv = torch.empty_like(lk)
        torch.cuda.synchronize()
        for i in range(CALLS):
            R.lr_project(xs[i % 2], ak, av, lk, lv)
    else:  # append
        c = synth.APPEND
        HK, D, ps, L0, T = c["HK"], c["D"], c["ps"], c["cur_len"], c["T"]
        n_phys = 2 * (-(-(L0 + T) // ps)) + 8
        pool_k = torch.zeros((n_phys, HK, ps, D), device=dev, dtype=torch.bfloat16)
        pool_v = torch.zeros_like(pool_k)
        kn = torch.randn((HK, T, D), device=dev).to(torch.bfloat16)
        vn = torch.randn((HK, T, D), device=dev).to(torch.bfloat16)
        pp = R.PagePool(n_phys)
        base = pp.alloc(-(-L0 // ps))
        pp.retain(base)  # a second sequence shares every page
        table = np.full(-(-(L0 + T) // ps), -1, np.int32)
        table[:base.size] = base
        cow = pp.plan_append(table, L0, T, ps)
        tdev = torch.from_numpy(table).to(dev)
        torch.cuda.synchronize()
        for i in range(CALLS):
            R.append_kv(pool_k, pool_v, tdev, L0, kn, vn, cow=cow)
    torch.cuda.synchronize()
    print("done", flush=True)


def _per_dispatch(d: str, counter: str, kernels):
    """(copy value, {kernel: values}) of one pass, in KiB per dispatch.  The
    calibration copy is the run's first dispatch of a copy kernel (``run``
    makes it before anything else; later copies, such as dtype conversions of
    inputs, are not calibrations)."""
    paths = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not paths:
        raise SystemExit(f"no counter_collection.csv under {d}")
    copy_vals, kern_vals = [], {k: [] for k in kernels}
    with open(paths[0]) as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") != counter:
                continue
            name, val = row.get("Kernel_Name", ""), float(row["Counter_Value"])
            hit = [k for k in kernels if k in name]
            if hit:
                kern_vals[hit[0]].append(val)
            elif "copy" in name.lower():
                copy_vals.append((int(row["Dispatch_Id"]), val))
    if not copy_vals or not all(kern_vals.values()):
        raise SystemExit(f"{counter}: copy or kernel dispatches missing in {paths[0]}")
    return min(copy_vals)[1], kern_vals


def summarize(key: str, fetch_dir: str, write_dir: str) -> None:
    sys.path.insert(0, ROOT)
    from shared_base_residual_amd.build import source_hash

    spec = SPECS[key]
    kernels = spec["kernels"]
    kern, wl = spec["files"]
    cf, kf = _per_dispatch(fetch_dir, "FETCH_SIZE", kernels)
    cw, kw = _per_dispatch(write_dir, "WRITE_SIZE", kernels)
    f_fetch, f_write = COPY_BYTES / (cf * 1024.0), COPY_BYTES / (cw * 1024.0)

    def avg(v):
        return sum(v) / len(v)

    fetch_b = sum(avg(kf[k]) for k in kernels) * 1024.0 * f_fetch
    write_b = sum(avg(kw[k]) for k in kernels) * 1024.0 * f_write
    path = os.path.join(ROOT, "profiles", "counters.json")
    data = {}
    if os.path.exists(path):
        with open(path) as f:
            data = json.load(f)
    data[key] = {
        "kernels": kernels, "source_hash": source_hash(),
        "bytes_per_launch": int(round(fetch_b + write_b)), "fetch_bytes": int(round(fetch_b)),
        "write_bytes": int(round(write_b)),
        "fetch_kib_raw": {k: round(avg(kf[k]), 1) for k in kernels},
        "write_kib_raw": {k: round(avg(kw[k]), 1) for k in kernels},
        "copy_fetch_kib": round(cf, 1), "copy_write_kib": round(cw, 1),
        "fetch_scale": round(f_fetch, 4), "write_scale": round(f_write, 4),
        "dispatches": {k: len(kf[k]) for k in kernels},
    }
    with open(path, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
        f.write("\n")
    e = data[key]
    per_k = "; ".join(f"{k}: FETCH_SIZE {e['fetch_kib_raw'][k]} KiB, WRITE_SIZE {e['write_kib_raw'][k]} KiB "
                      f"({e['dispatches'][k]} dispatches)" for k in kernels)
    lines = [
        f"# {' + '.join(kernels)} -- HBM traffic, workload {key}, MI355X", "",
        "Commands (repository root, TMPDIR=/tmp):", "",
        f"    rocprofv3 --pmc FETCH_SIZE --output-format csv -d {fetch_dir} -o run -- "
        f"python3 -m shared_base_residual_amd.counters run --workload {key}",
        f"    rocprofv3 --pmc WRITE_SIZE --output-format csv -d {write_dir} -o run -- "
        f"python3 -m shared_base_residual_amd.counters run --workload {key}",
        f"    python3 -m shared_base_residual_amd.counters summarize --workload {key} --fetch {fetch_dir} "
        f"--write {write_dir}", "",
        f"Calibration: a {COPY_BYTES >> 20} MiB device-to-device copy reads FETCH_SIZE {e['copy_fetch_kib']} KiB and "
        f"WRITE_SIZE {e['copy_write_kib']} KiB; scale factors {e['fetch_scale']} (fetch) and {e['write_scale']} "
        f"(write) turn the counters into bytes.", "",
        f"Per dispatch (averaged): {per_k}.", "",
        f"Per call: {e['fetch_bytes'] / 1e6:.1f} MB read, {e['write_bytes'] / 1e6:.1f} MB written; traffic "
        f"{e['bytes_per_launch'] / 1e6:.1f} MB.", "",
        f"Library sources hash {e['source_hash']}.", "",
    ]
    out = os.path.join(ROOT, "profiles", f"{kern}.{wl}.counters.txt")
    with open(out, "w") as f:
        f.write("\n".join(lines))
    print(json.dumps(e))


# MI355X: 256 compute units of 4 SIMDs each
SIMD_NUM = 1024


def summarize_mfma(key: str, d: str) -> None:
    """Matrix-unit utilisation of the workload's first kernel from one rocprofv3
    pass with --pmc MfmaUtil MfmaFlopsBF16 SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE
    (MfmaUtil = MFMA-busy SIMD cycles / (GPU-active cycles x SIMDs) x 100; the
    bf16 MFMA flops are the counter's operation count x 512)."""
    sys.path.insert(0, ROOT)
    from shared_base_residual_amd.build import source_hash

    spec = SPECS[key]
    kern, wl = spec["files"]
    paths = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not paths:
        raise SystemExit(f"no counter_collection.csv under {d}")
    vals = {}
    with open(paths[0]) as f:
        for row in csv.DictReader(f):
            if spec["kernels"][0] not in row.get("Kernel_Name", ""):
                continue
            vals.setdefault(row["Counter_Name"], []).append(float(row["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no {spec['kernels'][0]} dispatches in {paths[0]}")
    avg = {k: sum(v) / len(v) for k, v in vals.items()}
    n = len(next(iter(vals.values())))
    util = avg.get("MfmaUtil")
    flops = avg.get("MfmaFlopsBF16")
    lines = [
        f"# {spec['kernels'][0]} -- matrix-unit (MFMA) utilisation, workload {key}, MI355X", "",
        "Commands (repository root, TMPDIR=/tmp):", "",
        f"    rocprofv3 --pmc MfmaUtil MfmaFlopsBF16 SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE --output-format csv "
        f"-d {d} -o run -- python3 -m shared_base_residual_amd.counters run --workload {key}",
        f"    python3 -m shared_base_residual_amd.counters summarize-mfma --workload {key} --dir {d}", "",
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


SQ_COUNTERS = ("SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_ACTIVE_INST_LDS", "SQ_INSTS_LDS", "SQ_WAIT_INST_LDS",
               "SQ_BUSY_CU_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU")


def summarize_sq(key: str, d: str) -> None:
    """LDS and matrix-unit occupancy of the workload's first kernel from one
    rocprofv3 pass with --pmc SQ_COUNTERS (eight SQ counters, the most one pass
    collects).  The counters are summed over the chip: SQ_BUSY_CU_CYCLES over the
    256 compute units, SQ_VALU_MFMA_BUSY_CYCLES over the 1024 SIMDs, the LDS
    counters over the compute units."""
    sys.path.insert(0, ROOT)
    from shared_base_residual_amd.build import source_hash

    spec = SPECS[key]
    kern, wl = spec["files"]
    paths = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not paths:
        raise SystemExit(f"no counter_collection.csv under {d}")
    per = {}
    with open(paths[0]) as f:
        for row in csv.DictReader(f):
            if spec["kernels"][0] not in row.get("Kernel_Name", ""):
                continue
            dd = per.setdefault(row["Dispatch_Id"], {})
            dd[row["Counter_Name"]] = dd.get(row["Counter_Name"], 0.0) + float(row["Counter_Value"])
    if not per:
        raise SystemExit(f"no {spec['kernels'][0]} dispatches in {paths[0]}")
    ds = [per[k] for k in sorted(per, key=int)]
    avg = {c: sum(x.get(c, 0.0) for x in ds) / len(ds) for c in ds[0]}
    cu = avg["SQ_BUSY_CU_CYCLES"]
    lines = [
        f"# {spec['kernels'][0]} -- LDS and matrix-unit occupancy, workload {key}, MI355X", "",
        "Commands (repository root, TMPDIR=/tmp):", "",
        f"    rocprofv3 --pmc {' '.join(SQ_COUNTERS)} --output-format csv -d {d} -o run -- "
        f"python3 -m shared_base_residual_amd.counters run --workload {key}",
        f"    python3 -m shared_base_residual_amd.counters summarize-sq --workload {key} --dir {d}", "",
        f"Per dispatch ({len(ds)} dispatches averaged; sums over the chip):", "",
        "| counter | value |", "|---|---|",
    ]
    for k in sorted(avg):
        lines.append(f"| {k} | {avg[k]:.6g} |")
    lines += [
        "",
        f"- matrix units busy: SQ_VALU_MFMA_BUSY_CYCLES / (4 x SQ_BUSY_CU_CYCLES) = "
        f"**{avg['SQ_VALU_MFMA_BUSY_CYCLES'] / (4 * cu) * 100:.1f} %** of the SIMD cycles;",
        f"- LDS active (indexed reads and writes) {avg['SQ_LDS_IDX_ACTIVE'] / cu * 100:.1f} % of the CU cycles, "
        f"of which bank-conflict stalls {avg['SQ_LDS_BANK_CONFLICT'] / max(avg['SQ_LDS_IDX_ACTIVE'], 1) * 100:.1f} %;",
        f"- SQ_BUSY_CU_CYCLES / 256 = {cu / 256:.4g} cycles per compute unit per dispatch.",
        "", f"Library sources hash {source_hash()}.", "",
    ]
    out = os.path.join(ROOT, "profiles", f"{kern}.{wl}.sq.txt")
    with open(out, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


def _stretches(launches):
    """Split (start, duration) launches, sorted by start, where they are more
    than GAP_NS apart."""
    runs, cur = [], []
    for t, dur in launches:
        if cur and t - (cur[-1][0] + cur[-1][1]) > GAP_NS:
            runs.append(cur)
            cur = []
        cur.append((t, dur))
    if cur:
        runs.append(cur)
    return runs


def summarize_trace(key: str, d: str, bench_json: str, cmd: str) -> None:
    """Kernel durations of one rocprofv3 --kernel-trace --stats run of bench.py:
    the library's kernels from kernel_stats.csv, the average over the launches
    bench.py timed for the record (the last ones of the record's stretch of the
    trace), and the record itself."""
    sys.path.insert(0, ROOT)
    from shared_base_residual_amd.build import source_hash

    spec = SPECS[key]
    kernels = spec["kernels"]
    kern, wl = spec["files"]
    with open(bench_json) as f:
        line = [l for l in f.read().splitlines() if l.startswith("{")][-1]
    top = json.loads(line)
    recs = [top] + list(top.get("sub_records", []))
    found = [r for r in recs if spec["match"](r)]
    if not found:
        raise SystemExit(f"no record of workload {key} in {bench_json}")
    rec = found[0]
    roof = rec["roofline"]
    stats = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    trace = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if not stats or not trace:
        raise SystemExit(f"kernel_stats.csv / kernel_trace.csv missing under {d}")
    with open(stats[0]) as f:
        rows = list(csv.DictReader(f))
    launches = {k: [] for k in kernels}
    with open(trace[0]) as f:
        for r in csv.DictReader(f):
            for k in kernels:
                if k in r["Kernel_Name"]:
                    t0 = int(r["Start_Timestamp"])
                    launches[k].append((t0, int(r["End_Timestamp"]) - t0))
                    break
    for k in kernels:
        launches[k].sort()
    # the record's stretch: records run one after another, and the records whose
    # roofline names this workload's first kernel each leave one stretch of it
    users = [r for r in recs if kernels[0] in r.get("roofline", {}).get("kernel", "")]
    runs = _stretches(launches[kernels[0]])
    if len(runs) != len(users):
        raise SystemExit(f"{kernels[0]}: {len(runs)} stretches of launches for {len(users)} records")
    mine = runs[users.index(rec)]
    lo, hi = mine[0][0], mine[-1][0] + mine[-1][1]
    n_k = roof["launches_timed"]
    lines = [
        f"# {' + '.join(kernels)} -- workload {key} ({rec['config']['workload']}), MI355X", "",
        "Command (repository root, TMPDIR=/tmp):", "",
        f"    {cmd}", "",
        "Kernels of the library (kernel_stats.csv, the whole run; durations in microseconds):", "",
        "| kernel | calls | avg | min | max | share of GPU time |", "|---|---|---|---|---|---|",
    ]
    for r in rows:
        if "rattn" in r["Name"]:
            lines.append(f"| `{r['Name'][:100]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                         f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                         f"{float(r['Percentage']):.1f} % |")
    lines += ["", "The bench's other kernels (input draws, copies, the bandwidth probe) run outside the timed "
              "regions.", ""]
    total = 0.0
    for k in kernels:
        inside = [x for t, x in launches[k] if lo <= t <= hi]
        last = inside[-n_k:]
        a = sum(last) / max(1, len(last)) / 1e3
        total += a
        lines.append(f"- `{k}`: the last {len(last)} launches of this record's stretch of the trace (the launches "
                     f"bench.py timed) average {a:.2f} us.")
    lines += [
        "",
        f"Per call: {total:.2f} us; bench.py's HIP-event average over the same calls is {roof['avg_launch_us']} us "
        f"({roof.get('kernel', kernels[0])}; fraction {roof['frac']} of the {roof['peak']} {roof['unit']} peak).",
    ]
    if abs(total - roof["avg_launch_us"]) > 0.1 * total:
        lines += ["", "The two differ here because the tracer adds a fixed cost to every dispatch: for a kernel of a "
                  "few microseconds, back-to-back launches under rocprofv3 are spaced by that cost, which the "
                  "HIP-event window includes.  bench.py's line from a run without the profiler is the record of "
                  "this workload."]
    lines += [
        "", "Bench record of the same run:", "", "    " + json.dumps(rec), "",
        f"Library sources hash {source_hash()}.", "",
    ]
    out = os.path.join(ROOT, "profiles", f"{kern}.{wl}.txt")
    with open(out, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines[-12:]))


def main() -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="action", required=True)
    r = sub.add_parser("run")
    r.add_argument("--workload", required=True, choices=sorted(SPECS))
    s = sub.add_parser("summarize")
    s.add_argument("--workload", required=True, choices=sorted(SPECS))
    s.add_argument("--fetch", required=True)
    s.add_argument("--write", required=True)
    m = sub.add_parser("summarize-mfma")
    m.add_argument("--workload", required=True, choices=sorted(SPECS))
    m.add_argument("--dir", required=True)
    q = sub.add_parser("summarize-sq")
    q.add_argument("--workload", required=True, choices=sorted(SPECS))
    q.add_argument("--dir", required=True)
    t = sub.add_parser("summarize-trace")
    t.add_argument("--workload", required=True, choices=sorted(SPECS))
    t.add_argument("--dir", required=True)
    t.add_argument("--bench-json", required=True)
    t.add_argument("--cmd", required=True)
    a = ap.parse_args()
    if a.action == "run":
        run(a.workload)
    elif a.action == "summarize":
        summarize(a.workload, a.fetch, a.write)
    elif a.action == "summarize-mfma":
        summarize_mfma(a.workload, a.dir)
    elif a.action == "summarize-sq":
        summarize_sq(a.workload, a.dir)
    else:
        summarize_trace(a.workload, a.dir, a.bench_json, a.cmd)


if __name__ == "__main__":
    main()
