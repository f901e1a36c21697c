"""Calls on several streams and inside captured graphs.

rattn_decode keeps no global mutable state and launches only on the stream it
is given, with a caller-owned workspace; its kernels are deterministic.  So:
  * two input sets decoded on two streams at once (each with its own
    workspace) give the same output bits as decoded one after the other;
  * a decode captured into a graph (workspace and outputs allocated before the
    capture; the library records no memset and allocates nothing) replays to
    the eager output bit for bit, every replay, with eager work and device
    synchronisations between the replays;
  * the same holds for rattn_decode_noalloc, whose partials live in the
    library's static buffer.
"""
import os
import sys

import numpy as np
import pytest

import synth

import shared_base_residual_amd as R

pytestmark = [pytest.mark.skipif(not os.path.exists(R.LIB_PATH), reason="librattn not built"), pytest.mark.gpu]
DEV = "cuda"
CASE = synth.Case(4, 32, 8, 128, 16, 3000, name="8B-shaped heads, 3000-token prefix")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _inputs(seed):
    return synth.to_torch(synth.make_inputs(CASE, seed), DEV)


def test_two_streams_match_sequential():
    torch = pytest.importorskip("torch")
    say("[gpu] two streams")
    xs = [_inputs(61), _inputs(62)]
    ref = []
    for x in xs:
        ref.append(R.attend(x, prefix_len=CASE.prefix_len).clone())
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
    nb = R.workspace_bytes(R.describe(xs[0]["q"], xs[0]["k_base"], xs[0]["lk"], xs[0]["bk"]))
    wss = [torch.empty(nb, device=DEV, dtype=torch.uint8) for _ in streams]
    outs = [torch.full(tuple(x["q"].shape), float("nan"), device=DEV, dtype=torch.float32) for x in xs]
    torch.cuda.synchronize()
    for rep in range(3):  # interleaved launches, no synchronisation between the streams
        for x, s, ws, o in zip(xs, streams, wss, outs):
            with torch.cuda.stream(s):
                R.attend(x, prefix_len=CASE.prefix_len, out=o, workspace=ws, stream=s)
    torch.cuda.synchronize()
    for o, r in zip(outs, ref):
        assert torch.equal(o, r)


def _graph_check(run_eager, run_into, out_shape):
    torch = pytest.importorskip("torch")
    eager = run_eager().clone()
    torch.cuda.synchronize()
    out = torch.empty(out_shape, device=DEV, dtype=torch.float32)
    run_into(out)  # warm-up outside the capture (first launches set kernel attributes)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_into(out)
    torch.cuda.synchronize()
    for rep in range(4):
        out.fill_(float("nan"))  # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep}"


def test_decode_in_a_graph():
    torch = pytest.importorskip("torch")
    say("[gpu] graph capture of rattn_decode")
    x = _inputs(63)
    nb = R.workspace_bytes(R.describe(x["q"], x["k_base"], x["lk"], x["bk"]))
    ws = torch.empty(nb, device=DEV, dtype=torch.uint8)
    _graph_check(lambda: R.attend(x, prefix_len=CASE.prefix_len),
                 lambda o: R.attend(x, prefix_len=CASE.prefix_len, out=o, workspace=ws,
                                    stream=torch.cuda.current_stream()),
                 tuple(x["q"].shape))


def test_noalloc_decode_in_a_graph():
    torch = pytest.importorskip("torch")
    say("[gpu] graph capture of rattn_decode_noalloc")
    x = _inputs(64)
    _graph_check(lambda: R.attend(x, prefix_len=CASE.prefix_len),
                 lambda o: R.decode_noalloc(x, prefix_len=CASE.prefix_len, out=o,
                                            stream=torch.cuda.current_stream()),
                 tuple(x["q"].shape))
