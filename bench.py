"""Benchmark of fused residual attention over a shared base KV cache on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 4] [--sub 1,2,3] [--no-cpu]

Headline workload (default): the 70B-shaped full-depth decode step, 80 layers of
H_q=64, H_kv=8, d=128 over a 65536-token shared prefix, 8 agents with per-agent
rank-16 residual caches, bf16 inputs, fp32 accumulation (24.2 GB of inputs,
resident in HBM, drawn on the device).  One step = the 80 layers' rattn_decode
calls (split kernel, then merge) back to back on one stream.  The other
workloads (8B-shaped decode, paged copy-on-write decode, BaseLRShared chunked
prefill) follow as sub-records in the same JSON line, each with its own
roofline, and so do the 8B- and 70B-shaped decodes over int8 keys and over
int8 keys with 3-bit values (the caches encoded outside the timed region), the
rebuilt-key decodes and the cache-write path.  For the single-layer workloads several replicas of the inputs are
rotated so that each step reads from HBM, not from the 256 MB Infinity Cache
left warm by the previous step.

Prints one JSON line.  `value` is agent x context-token pairs per second
(Gtok/s) over the timed steps (wall clock, K steps bracketed by device
synchronisations).  `roofline` is for the kernel that carries the call (the
split kernel for decode, the prefill kernel for prefill): algorithmic bytes (or
flops) per launch over its average duration, measured with HIP events on the
launch stream around K * layers back-to-back launches after a warm-up that runs
until the launch time is stable; `frac_timed_steps` is the same ratio for the
whole call over the timed steps.  `achievable` is the read rate of an HBM probe
kernel measured in the same run (libhbm_probe.so).  `traffic` is the HBM bytes
per launch read from rocprofv3 FETCH_SIZE / WRITE_SIZE counters
(profiles/counters.json, written by shared_base_residual_amd/counters.py) when
they were taken on the current library sources, else null.  `cpu_baseline`
times the fp64 oracle on the host cores over a bounded sample.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
METRIC = "agent x ctx-token attention throughput (Gtok/s) + achieved HBM GB/s, 1 GPU"
COUNTERS = os.path.join(ROOT, "profiles", "counters.json")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash() -> str:
    from shared_base_residual_amd.build import source_hash as h

    return h()


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class Hip:
    """Minimal HIP runtime access for events on an explicit stream."""

    def __init__(self):
        self.h = ctypes.CDLL("libamdhip64.so")
        self.h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.h.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        assert self.h.hipEventCreate(ctypes.byref(e)) == 0
        return e

    def record(self, e, stream):
        assert self.h.hipEventRecord(e, stream) == 0

    def elapsed_ms(self, a, b):
        t = ctypes.c_float()
        assert self.h.hipEventSynchronize(b) == 0
        assert self.h.hipEventElapsedTime(ctypes.byref(t), a, b) == 0
        return t.value

    def time_ms(self, fn, n, stream):
        """Average ms of fn() over n back-to-back calls, between two events."""
        a, b = self.event(), self.event()
        self.record(a, stream)
        for i in range(n):
            fn(i)
        self.record(b, stream)
        return self.elapsed_ms(a, b) / n


def stable_ms(hip, fn, n, stream, tol=0.01, max_batches=40):
    """Runs batches of n back-to-back calls until two consecutive batch averages
    agree within tol (clocks and caches settled); returns the batch averages."""
    hist = []
    for _ in range(max_batches):
        hist.append(hip.time_ms(fn, n, stream))
        if len(hist) >= 3 and abs(hist[-1] - hist[-2]) <= tol * hist[-1] and abs(hist[-2] - hist[-3]) <= tol * hist[-2]:
            break
    return hist


def algorithmic_bytes(c, k8=False, v3=False):
    """Bytes every input is read once plus the fp32 output written once (int8
    base keys: one byte per key element; 3-bit values: 3 d / 8 bytes of codes
    and a 4-byte scale per value vector)."""
    es = 2 if c.dtype == "bf16" else 4
    v_vec = 3 * c.head_dim // 8 + 4 if v3 else c.head_dim * es
    base = c.n_kv_heads * c.prefix_len * (c.head_dim * (1 if k8 else es) + v_vec)
    resid = 2 * c.n_lr * c.prefix_len * c.rank * es
    bmat = 2 * c.n_agents * c.rank * c.n_kv_heads * c.head_dim * es
    q = c.n_agents * c.q_len * c.n_q_heads * c.head_dim * es
    priv = 2 * c.n_agents * c.n_kv_heads * c.priv_len * c.head_dim * es
    table = 4 * c.n_table
    out = 4 * c.n_agents * c.q_len * c.n_q_heads * c.head_dim
    split = base + resid + priv + q + table + bmat // 2
    return dict(base=base, resid=resid, bmat=bmat, q=q, priv=priv, table=table, out=out,
                call=base + resid + bmat + q + priv + table + out, split=split)


def algorithmic_flops(c):
    """Multiply-adds x 2 of one call: q.K and p.V over every visible key (4d per
    query row and key), the rank-r score and value corrections over the prefix
    keys (4r), and q Bk^T and W Bv once per query row (4dr)."""
    d, r = c.head_dim, c.rank
    rows = c.n_agents * c.q_len * c.n_q_heads
    if c.mode == "prefill":
        vis_priv = c.q_len * (c.q_len + 1) / 2.0
    else:
        vis_priv = c.q_len * c.priv_len
    per_head = c.n_agents * c.n_q_heads
    flops = per_head * (c.q_len * c.prefix_len * (4 * d + 4 * r) + vis_priv * 4 * d)
    if c.prefix_len > 0 and r > 0:
        flops += rows * 4 * d * r
    return flops


def pairs_per_call(c):
    if c.mode == "prefill":
        return c.n_agents * c.q_len * (c.prefix_len + (c.q_len + 1) / 2.0)
    return c.n_agents * c.q_len * (c.prefix_len + c.priv_len)


def cpu_baseline(case, seed, budget_s=12.0):
    """The fp64 oracle, as it stands, on the host cores, over a bounded sample of
    the workload: the whole call for the decode workloads that finish in seconds,
    one agent's rows of one layer otherwise; repeated until about `budget_s`
    seconds of work have been timed.  The rate is scaled by the fraction of rows
    computed (and, for the multi-layer workload, counts one layer's pairs)."""
    import numpy as np

    import oracle
    import synth

    threads = oracle.default_threads()
    x = synth.make_inputs(case.replace(layers=1), seed)
    mask, frac, what = None, 1.0, "whole call"
    if case.mode == "prefill" or case.prefix_len * case.n_agents > 2 ** 18:
        mask = np.zeros((case.n_agents, case.q_len, case.n_q_heads), bool)
        mask[0] = True
        frac, what = 1.0 / case.n_agents, "agent 0's rows of one call"
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        oracle.attend(case, x, n_threads=threads, row_mask=mask)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > budget_s or len(times) >= 20:
            break
    t = statistics.median(times)
    return {"value": round(pairs_per_call(case) * frac / t / 1e9, 6), "unit": "Gtok/s", "cores": threads,
            "kind": "oracle", "cpu": cpu_model(),
            "sample": f"{what} ({case.name}, one layer), {len(times)} runs, median {t:.3f} s, fp64, "
                      f"{threads} threads",
            "one_thread": [one_thread_baseline(c, c) for c in (0, 1, 2)]}


def one_thread_baseline(config, seed, budget_s=3.0):
    """The oracle on one host thread for a small workload: the whole call of the
    tiny decode, else the query rows of agent 0 and KV head 0 (one materialised
    cache, its g rows), the rate scaled by the fraction of rows computed."""
    import numpy as np

    import oracle
    import synth

    case = synth.WORKLOADS[config]
    x = synth.make_inputs(case, seed)
    mask, frac, what = None, 1.0, "whole call"
    if config != 0:
        g = case.n_q_heads // case.n_kv_heads
        mask = np.zeros((case.n_agents, case.q_len, case.n_q_heads), bool)
        mask[0, :, :g] = True
        frac = float(mask.sum()) / mask.size
        what = "agent 0's rows of KV head 0"
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        oracle.attend(case, x, n_threads=1, row_mask=mask)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > budget_s or len(times) >= 9:
            break
    t = statistics.median(times)
    return {"workload": case.name, "value": round(pairs_per_call(case) * frac / t / 1e9, 7), "unit": "Gtok/s",
            "cores": 1, "sample": f"{what}, {len(times)} runs, median {t:.4f} s, fp64, 1 thread"}


def traffic_from_counters(kernel_key):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel sources."""
    if not os.path.exists(COUNTERS):
        return None
    with open(COUNTERS) as f:
        data = json.load(f)
    ent = data.get(kernel_key)
    if not ent or ent.get("source_hash") != source_hash():
        return None
    return ent.get("bytes_per_launch")


def hbm_probe(hip, stream, dev):
    """Read bandwidth two streaming readers reach over a 4 GiB buffer (each byte
    read once per launch): plain vector loads and direct loads into LDS, over a
    few launch shapes; the best is `achievable`."""
    import torch

    from shared_base_residual_amd.build import PROBE_LIB

    lib = ctypes.CDLL(PROBE_LIB)
    lib.hbm_probe_vec.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    lib.hbm_probe_lds.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_void_p]
    nbytes = 4 << 30
    buf = torch.ones(nbytes // 4, device=dev, dtype=torch.int32)
    sink = torch.zeros(1 << 16, device=dev, dtype=torch.int32)
    res = {}
    shapes = [("vec", b, 0) for b in (2048, 4096, 8192)] + [("lds", b, w) for b in (256, 512, 1024) for w in (4, 8)]
    for kind, blocks, waves in shapes:
        if kind == "vec":
            fn = lambda i: lib.hbm_probe_vec(buf.data_ptr(), nbytes, sink.data_ptr(), blocks, stream)
        else:
            fn = lambda i: lib.hbm_probe_lds(buf.data_ptr(), nbytes, sink.data_ptr(), blocks, waves, stream)
        assert fn(0) == 0
        ms = min(hip.time_ms(fn, 4, stream) for _ in range(3))
        res[f"{kind}:{blocks}" + (f"x{waves}w" if waves else "")] = round(nbytes / (ms / 1e3) / 1e9, 1)
    torch.cuda.synchronize()
    del buf, sink
    best = max(res, key=res.get)
    return {"achievable": res[best], "unit": "GB/s", "reader": best, "buffer_bytes": nbytes, "all": res}


def measure(config, K, W, dev, hip, stream, replicas=0, seed=None, probe=None, k8=False, v3=False):
    """Times one workload; returns its record (without cpu_baseline).  k8: the
    base keys are first quantised to int8 codes (rattn_quantize_keys, outside
    the timed region) and every call reads the codes; v3 (with k8): the base
    values too, to 3-bit codes and scales (rattn_quantize_values)."""
    import torch

    import shared_base_residual_amd as R
    import synth

    case = synth.WORKLOADS[config]
    seed = config if seed is None else seed
    ab = algorithmic_bytes(case, k8, v3)
    layers = case.layers
    op = R.RATTN_OP_PREFILL if case.mode == "prefill" else R.RATTN_OP_DECODE
    say(f"[bench] {case.name}: drawing inputs")

    # ---- inputs resident in HBM
    if layers > 1:
        sets = [synth.make_inputs_torch(case, seed, l, dev) for l in range(layers)]
        n_sets = layers
    else:
        x = synth.make_inputs(case, seed)
        base = synth.to_torch(x, dev)
        reps = replicas or max(1, min(8, -(-1024 * 2 ** 20 // ab["call"])))
        sets = [base] + [{k: (None if v is None else v.clone()) for k, v in base.items()} for _ in range(reps - 1)]
        n_sets = reps
    k_scale = None
    if k8:
        for st in sets:  # each set's keys become int8 codes with that set's scale
            codes, sc = R.quantize_keys(st["k_base"])
            st["k_base"] = codes
            st["k_scale"] = float(sc.cpu().numpy()[0])
        k_scale = sets[0]["k_scale"]
    if v3:
        for st in sets:  # each set's values become 3-bit codes and scales
            st["v_base"], st["v_scale"] = R.quantize_values(st["v_base"])
    desc = R.describe(sets[0]["q"], sets[0]["k_base"], sets[0]["lk"], sets[0]["bk"],
                      block_table=sets[0]["block_table"], k_priv=sets[0]["k_priv"], prefix_len=case.prefix_len,
                      shared_lr=case.shared_lr, k_scale=k_scale, v_base=sets[0]["v_base"])
    kernel = R.kernel_of(desc, op)
    wsb = R.workspace_bytes(desc, op)
    ws = torch.empty(max(wsb, 256), device=dev, dtype=torch.uint8)
    outs = [torch.empty(tuple(s["q"].shape), device=dev, dtype=torch.float32) for s in sets]
    argv, descs = [], []
    for s, o in zip(sets, outs):
        t = dict(s, out=o, lse=None)
        t.pop("k_scale", None)
        R._check_tensors(desc, t)
        argv.append(R.Args(*[None if t.get(n) is None else t[n].data_ptr() for n, _ in R.Args._fields_]))
        d_i = R.Desc.from_buffer_copy(desc)
        if k8:
            d_i.k_scale = s["k_scale"]  # one scale per set (per layer)
        descs.append(d_i)
    sp = ctypes.c_void_p(stream.cuda_stream)
    lib = R.lib()
    wsp, wss = ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(ws.numel())
    drefs = [ctypes.byref(d_i) for d_i in descs]
    arefs = [ctypes.byref(a) for a in argv]
    fn = lib.rattn_attention_stages

    def launch(i, stages):
        st = fn(drefs[i % n_sets], op, arefs[i % n_sets], wsp, wss, sp, stages)
        if st:
            raise R.RattnError(st, "rattn_attention_stages")

    # One step = all layers' calls (one call when layers == 1), each one
    # rattn_attention_stages call of all its launches.
    def step(k):
        for l in range(layers):
            launch(k * layers + l, R.STAGE_ALL)

    for k in range(W):
        step(k)
    torch.cuda.synchronize()
    # warm until the per-call time is stable (clocks settle over the first
    # launches), then the timed steps: K steps between two synchronisations
    # (wall clock), with HIP events on the launch stream around them
    per_batch = max(8, layers)
    warm = stable_ms(hip, lambda i: launch(i, R.STAGE_ALL), per_batch, sp)
    torch.cuda.synchronize()
    ev_a, ev_b = hip.event(), hip.event()
    t0 = time.perf_counter()
    hip.record(ev_a, sp)
    for k in range(K):
        step(k)
    hip.record(ev_b, sp)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms_ev = hip.elapsed_ms(ev_a, ev_b) / K

    # The kernel behind the roofline (the split kernel; for prefill the one
    # kernel of the call), launched back to back K * layers times between two
    # HIP events on the launch stream after its own stabilising warm-up, so that
    # the average is the kernel's own steady duration.
    n_k = K * layers
    stable_ms(hip, lambda i: launch(i, R.STAGE_SPLIT), per_batch, sp)
    kern_avg = hip.time_ms(lambda i: launch(i, R.STAGE_SPLIT), n_k, sp)
    torch.cuda.synchronize()

    ms_step = wall * 1e3 / K
    pairs = pairs_per_call(case) * layers
    value = pairs / (ms_step / 1e3) / 1e9
    call_ms = step_ms_ev / layers  # one call, from the timed steps' events
    if kernel[0] == "prefill":
        fl = algorithmic_flops(case)
        achieved = fl / (kern_avg / 1e3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": traffic_from_counters(f"prefill_cfg{config}"),
                "kernel": "prefill_kernel", "flops_per_launch": fl, "avg_launch_us": round(kern_avg * 1e3, 2),
                "launches_timed": n_k,
                "frac_timed_steps": round(fl / (call_ms / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
    else:
        achieved = ab["split"] / (kern_avg / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": traffic_from_counters(f"decode_cfg{config}" + ("_k8" if k8 else "") + ("v3" if v3 else "")),
                "kernel": "decode_split_kernel", "bytes_per_launch": ab["split"],
                "avg_launch_us": round(kern_avg * 1e3, 2), "launches_timed": n_k,
                # the whole call (split + merge) over the timed steps
                "frac_timed_steps": round(ab["call"] / (call_ms / 1e3) / 1e9 / HBM_PEAK_GBPS, 4)}
        if probe:
            roof["achievable"] = probe["achievable"]
            roof["frac_of_achievable"] = round(achieved / probe["achievable"], 4)
    roof["instantiation"] = list(kernel)
    rec = {
        "metric": METRIC, "value": round(value, 4), "unit": "Gtok/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": case.dtype, "data": "synthetic (seeded N(0,1) caches and queries, N(0,0.05^2) up-projections)",
        "config": {"workload": case.name + (", int8 keys" if k8 else "") + (", 3-bit values" if v3 else ""),
                   "n_agents": case.n_agents, "n_q_heads": case.n_q_heads,
                   "key_format": "int8 (per-tensor scale)" if k8 else case.dtype,
                   "value_format": "3-bit Walsh-Hadamard-rotated codes (per-vector scale)" if v3 else case.dtype,
                   "n_kv_heads": case.n_kv_heads, "head_dim": case.head_dim, "prefix_len": case.prefix_len,
                   "priv_len": case.priv_len, "q_len": case.q_len, "rank": case.rank, "page_size": case.page_size,
                   "shared_lr": case.shared_lr, "layers": layers, "mode": case.mode, "input_sets_rotated": n_sets},
        "hbm_gbps_call": round(ab["call"] * layers / (ms_step / 1e3) / 1e9, 1),
        "gpu_ms_per_step_events": round(step_ms_ev, 5),
        "warmup_call_ms": [round(x, 5) for x in warm],
        "roofline": roof,
    }
    del sets, outs, ws
    torch.cuda.empty_cache()
    say(f"[bench] {case.name}: {rec['value']} Gtok/s, kernel {roof['avg_launch_us']} us, frac {roof['frac']}")
    return rec


# The cache-write path, measured beside the attention workloads: the low-rank
# cache rows of a 32768-token shared context for 4 agents with their own
# down-projections (BaseShared "LR prefill" on an agent switch; ForkKV's base
# hit with an adapter miss), Llama-3-8B-shaped (d_in = 4096, r = 16); and a
# 4096-token append of base rows (H_kv = 8, d = 128, bf16) into a paged pool
# whose partly filled last page is shared (one copy-on-write page).


def measure_lr_prefill(K, W, dev, hip, stream, probe):
    import numpy as np
    import torch

    import shared_base_residual_amd as R
    import synth

    c = synth.LR_PREFILL
    say(f"[bench] {c['name']}: drawing inputs")
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    n_rep = 2  # X (268 MB) alternates between two replicas so each launch reads HBM
    xs = [torch.randn((1, c["T"], c["d_in"]), generator=g, device=dev).to(torch.bfloat16) for _ in range(n_rep)]
    ak = (torch.randn((c["n_sets"], c["r"], c["d_in"]), generator=g, device=dev) * 0.05).to(torch.bfloat16)
    av = (torch.randn((c["n_sets"], c["r"], c["d_in"]), generator=g, device=dev) * 0.05).to(torch.bfloat16)
    lk = torch.empty((c["n_sets"], c["T"], c["r"]), device=dev, dtype=torch.bfloat16)
    lv = torch.empty_like(lk)
    fn = lambda i: R.lr_project(xs[i % n_rep], ak, av, lk, lv, stream=stream)
    for i in range(W):
        fn(i)
    stable_ms(hip, fn, 8, ctypes.c_void_p(stream.cuda_stream))
    ms = hip.time_ms(fn, K, ctypes.c_void_p(stream.cuda_stream))
    torch.cuda.synchronize()
    nbytes = xs[0].numel() * 2 + 2 * ak.numel() * 2 + 2 * lk.numel() * 2
    achieved = nbytes / (ms / 1e3) / 1e9
    rows = c["n_sets"] * c["T"]
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic_from_counters("lr_prefill"),
            "kernel": "lr_project_kernel",
            "bytes_per_launch": nbytes, "avg_launch_us": round(ms * 1e3, 2), "launches_timed": K}
    if probe:
        roof["achievable"] = probe["achievable"]
        roof["frac_of_achievable"] = round(achieved / probe["achievable"], 4)
    say(f"[bench] {c['name']}: {ms * 1e3:.2f} us, frac {roof['frac']}")
    del xs, ak, av, lk, lv
    return {"metric": "low-rank cache rows written per second (agent x token)", "value": round(rows / ms / 1e6, 4),
            "unit": "G rows/s", "steps": K, "warmup": W, "ms_per_step": round(ms, 5), "dtype": "bf16",
            "config": {"workload": c["name"], "n_sets": c["n_sets"], "d_in": c["d_in"], "rank": c["r"],
                       "n_tokens": c["T"], "shared_x": True, "shared_a": False}, "roofline": roof}


def measure_append(K, W, dev, hip, stream, probe):
    import numpy as np
    import torch

    import shared_base_residual_amd as R
    import synth

    c = synth.APPEND
    HK, D, ps, L0, T = c["HK"], c["D"], c["ps"], c["cur_len"], c["T"]
    n_phys = 2 * (-(-(L0 + T) // ps)) + 8
    say(f"[bench] {c['name']}")
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
    fn = lambda i: R.append_kv(pool_k, pool_v, tdev, L0, kn, vn, cow=cow, stream=stream)
    for i in range(W):
        fn(i)
    sp = ctypes.c_void_p(stream.cuda_stream)
    stable_ms(hip, fn, 8, sp)
    ms = hip.time_ms(fn, K, sp)
    torch.cuda.synchronize()
    off = L0 % ps
    nbytes = 2 * (2 * HK * T * D * 2) + 2 * (2 * HK * off * D * 2) + table.size * 4
    achieved = nbytes / (ms / 1e3) / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic_from_counters("append"),
            "kernel": "append_kv_kernel",
            "bytes_per_launch": nbytes, "avg_launch_us": round(ms * 1e3, 2), "launches_timed": K}
    if probe:
        roof["achievable"] = probe["achievable"]
        roof["frac_of_achievable"] = round(achieved / probe["achievable"], 4)
    say(f"[bench] {c['name']}: {ms * 1e3:.2f} us, frac {roof['frac']}")
    del pool_k, pool_v, kn, vn
    return {"metric": "base rows appended per second (token x KV head)", "value": round(HK * T / ms / 1e6, 4),
            "unit": "G rows/s", "steps": K, "warmup": W, "ms_per_step": round(ms, 5), "dtype": "bf16",
            "config": {"workload": c["name"], "n_kv_heads": HK, "head_dim": D, "page_size": ps,
                       "cur_len": L0, "n_tokens": T, "copy_on_write_pages": int(cow[0] >= 0)}, "roofline": roof}


def measure_reconstruct(config, K, W, dev, hip, stream, probe, rope):
    """The rebuilt-key decode (rattn_decode_reconstruct) on one layer of a
    decode workload, with or without the positional rotation; timed per call
    (its split kernel and the merge), beside the factored path's roofline."""
    import torch

    import shared_base_residual_amd as R
    import synth

    case = synth.WORKLOADS[config].replace(layers=1)
    ab = algorithmic_bytes(case)
    say(f"[bench] rebuilt keys ({case.name}, rope={rope}): drawing inputs")
    x = synth.make_inputs(case, config)
    base = synth.to_torch(x, dev)
    reps = max(1, min(8, -(-1024 * 2 ** 20 // ab["call"])))
    sets = [base] + [{k: (None if v is None else v.clone()) for k, v in base.items()} for _ in range(reps - 1)]
    theta = torch.from_numpy(synth.rope_theta(case.head_dim)).to(dev) if rope else None
    outs = [torch.empty(tuple(s["q"].shape), device=dev, dtype=torch.float32) for s in sets]
    desc = R.describe(base["q"], base["k_base"], base["lk"], base["bk"])
    ws = torch.empty(R.workspace_bytes(desc, R.RATTN_OP_RECONSTRUCT), device=dev, dtype=torch.uint8)
    fn = lambda i: R.decode_reconstruct(sets[i % reps], rope_theta=theta, out=outs[i % reps], workspace=ws,
                                        stream=stream)
    for i in range(W):
        fn(i)
    sp = ctypes.c_void_p(stream.cuda_stream)
    stable_ms(hip, fn, 8, sp)
    ms = hip.time_ms(fn, K, sp)
    torch.cuda.synchronize()
    achieved = ab["call"] / (ms / 1e3) / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic_from_counters(f"recon_cfg{config}" + ("_rope" if rope else "")),
            "kernel": "recon_split_kernel + combine_kernel (whole call)", "bytes_per_launch": ab["call"],
            "avg_launch_us": round(ms * 1e3, 2), "launches_timed": K}
    if probe:
        roof["achievable"] = probe["achievable"]
        roof["frac_of_achievable"] = round(achieved / probe["achievable"], 4)
    say(f"[bench] rebuilt keys ({case.name}, rope={rope}): {ms * 1e3:.2f} us per call, frac {roof['frac']}")
    del sets, outs, ws
    return {"metric": METRIC, "value": round(pairs_per_call(case) / (ms / 1e3) / 1e9, 4), "unit": "Gtok/s",
            "steps": K, "warmup": W, "ms_per_step": round(ms, 5), "dtype": "bf16",
            "config": {"workload": f"{case.name}, one layer, residual keys rebuilt in registers" +
                                   (", rotated by position" if rope else ""), "n_agents": case.n_agents,
                       "n_q_heads": case.n_q_heads, "n_kv_heads": case.n_kv_heads, "head_dim": case.head_dim,
                       "prefix_len": case.prefix_len, "rank": case.rank, "rope": rope},
            "roofline": roof}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=4, help="headline workload (synth.WORKLOADS index)")
    ap.add_argument("--sub", default="1,2,3", help="workloads measured as sub-records ('' for none)")
    ap.add_argument("--replicas", type=int, default=0, help="input sets rotated (0: auto)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-probe", action="store_true")
    ap.add_argument("--no-cache-write", action="store_true", help="skip the cache-write sub-records")
    ap.add_argument("--no-int8", action="store_true", help="skip the int8-key sub-records")
    ap.add_argument("--no-values3", action="store_true", help="skip the int8-key + 3-bit-value sub-records")
    ap.add_argument("--no-reconstruct", action="store_true", help="skip the rebuilt-key sub-records")
    ap.add_argument("--seed", type=int, default=None)
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this build has no multi-GPU "
              "path: run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import shared_base_residual_amd as R

    R.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    hip = Hip()
    probe = None if args.no_probe else hbm_probe(hip, ctypes.c_void_p(stream.cuda_stream), dev)
    if probe:
        say(f"[bench] HBM probe: {probe['achievable']} GB/s ({probe['reader']})")
    res = measure(args.config, args.steps, args.warmup, dev, hip, stream, args.replicas, args.seed, probe)
    subs = [int(s) for s in args.sub.split(",") if s.strip() and int(s) != args.config]
    if subs:
        res["sub_records"] = [measure(c, args.steps, args.warmup, dev, hip, stream, args.replicas, None, probe)
                              for c in subs]
    if not args.no_int8:
        res.setdefault("sub_records", []).extend(
            [measure(c, args.steps, args.warmup, dev, hip, stream, args.replicas, None, probe, k8=True) for c in (1, 4)])
    if not args.no_values3:
        res.setdefault("sub_records", []).extend(
            [measure(c, args.steps, args.warmup, dev, hip, stream, args.replicas, None, probe, k8=True, v3=True)
             for c in (1, 4)])
    if not args.no_reconstruct:
        res.setdefault("sub_records", []).extend(
            [measure_reconstruct(c, args.steps, args.warmup, dev, hip, stream, probe, rope)
             for c in (1, 4) for rope in (False, True)])
    if not args.no_cache_write:
        res.setdefault("sub_records", []).extend([measure_lr_prefill(args.steps, args.warmup, dev, hip, stream, probe),
                                                  measure_append(args.steps, args.warmup, dev, hip, stream, probe)])
    if probe:
        res["hbm_probe"] = probe
    if not args.no_cpu:
        import synth

        say("[bench] cpu baseline")
        res["cpu_baseline"] = cpu_baseline(synth.WORKLOADS[args.config],
                                           args.config if args.seed is None else args.seed)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
