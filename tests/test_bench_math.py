"""The benchmark's measurement arithmetic, on the CPU: algorithmic bytes and
flops per call and agent x context-token pairs for each workload, written out
here from the shapes as literal products (each input read once, the fp32 output
written once; 4d flops per query row and visible key for q.K and p.V, 4r per
prefix key for the two rank-r corrections, 4dr per query row for q Bk^T and
W Bv), and the one-GPU guard of the command line."""
import os
import subprocess
import sys

import pytest

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
MB = 1_000_000


def test_llama8b_decode_bytes_and_flops():
    c = synth.WORKLOADS[1]  # 4 agents, 32/8 heads, d 128, L 32768, r 16, bf16
    b = bench.algorithmic_bytes(c)
    assert b["base"] == 8 * 32768 * (128 * 2 + 128 * 2)
    assert b["resid"] == 2 * 4 * 32768 * 16 * 2
    assert b["bmat"] == 2 * 4 * 16 * 8 * 128 * 2
    assert b["q"] == 4 * 32 * 128 * 2 and b["out"] == 4 * 32 * 128 * 4
    assert round(b["call"] / MB, 2) == 142.97
    assert bench.algorithmic_flops(c) == 4 * 32 * 32768 * (4 * 128 + 4 * 16) + 4 * 32 * 4 * 128 * 16
    assert bench.pairs_per_call(c) == 4 * 32768
    k8 = bench.algorithmic_bytes(c, k8=True)
    assert k8["base"] == 8 * 32768 * (128 * 1 + 128 * 2)
    v3 = bench.algorithmic_bytes(c, k8=True, v3=True)
    assert v3["base"] == 8 * 32768 * (128 + 3 * 128 // 8 + 4)


def test_paged_decode_bytes_and_flops():
    c = synth.WORKLOADS[2]  # 16 agents, 32/8 heads, L 8192 in 16-token pages, r 64, S 512
    b = bench.algorithmic_bytes(c)
    assert b["base"] == 8 * 8192 * 2 * 128 * 2
    assert b["resid"] == 2 * 16 * 8192 * 64 * 2
    assert b["priv"] == 2 * 16 * 8 * 512 * 128 * 2
    assert b["table"] == 4 * (8192 // 16)
    assert round(b["call"] / MB, 2) == 105.25
    assert bench.algorithmic_flops(c) == (16 * 32 * (8192 * (4 * 128 + 4 * 64) + 512 * 4 * 128)
                                          + 16 * 32 * 4 * 128 * 64)
    assert bench.pairs_per_call(c) == 16 * (8192 + 512)


def test_chunked_prefill_bytes_and_flops():
    c = synth.WORKLOADS[3]  # 32 agents, 256-token chunks, shared r 32, L 16384
    b = bench.algorithmic_bytes(c)
    assert b["resid"] == 2 * 1 * 16384 * 32 * 2  # one shared low-rank cache
    assert b["q"] == 32 * 256 * 32 * 128 * 2 and b["out"] == 32 * 256 * 32 * 128 * 4
    assert round(b["call"] / MB) == 308
    causal = 256 * 257 / 2
    assert bench.algorithmic_flops(c) == (32 * 32 * (256 * 16384 * (4 * 128 + 4 * 32) + causal * 4 * 128)
                                          + 32 * 256 * 32 * 4 * 128 * 32)
    assert round(bench.algorithmic_flops(c) / 1e12, 3) == 2.770
    assert bench.pairs_per_call(c) == 32 * 256 * (16384 + 257 / 2)


def test_70b_decode_bytes_per_layer():
    c = synth.WORKLOADS[4]  # 8 agents, 64/8 heads, L 65536, r 16, 80 layers
    b = bench.algorithmic_bytes(c)
    assert b["base"] == 8 * 65536 * 2 * 128 * 2
    assert round(b["call"] / MB, 1) == 302.9
    assert c.layers == 80
    assert round(80 * bench.algorithmic_flops(c) / 1e12, 2) == 1.55


def test_more_than_one_gpu_is_refused():
    """--gpus above 1 exits with status 2 and a message, before touching a GPU."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
