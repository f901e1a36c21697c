"""rattn_decode_reconstruct: decode with the residual keys rebuilt per token in
registers (the ForkKV Guide's in-register kernel design), optionally rotated by
position.  Without a rotation it must match the plain oracle (the factored
path's result); with one, the rebuilt-key oracle (oracle/recon.py) over the
table that the same frequencies define.  Each of the kernel's four forms (rank
16 or 32, with or without the rotation) is exercised."""
import ctypes
import os
import sys

import numpy as np
import pytest

import oracle
import synth
from oracle import recon
from tests import parity

import shared_base_residual_amd as R

pytestmark = pytest.mark.skipif(not os.path.exists(R.LIB_PATH), reason="librattn not built")
DEV = "cuda"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.mark.parametrize("kw,status", [
    (dict(), 0),
    (dict(rank=8), -3),
    (dict(rank=64), -3),
    (dict(head_dim=64), -3),
    (dict(priv_len=4), -3),
    (dict(page_size=16, n_phys_pages=64), -3),
    (dict(n_q_heads=64, n_kv_heads=2), -3),  # 32 rows per agent and head
    (dict(dtype=R.RATTN_F32), -3),
])
def test_reconstruct_validation(kw, status):
    base = dict(n_agents=4, n_q_heads=32, n_kv_heads=8, head_dim=128, rank=16, q_len=1, prefix_len=4096)
    base.update(kw)
    d = R.make_desc(**base)
    n = ctypes.c_size_t()
    assert R.lib().rattn_workspace_bytes(ctypes.byref(d), R.RATTN_OP_RECONSTRUCT, ctypes.byref(n)) == status


def run(case, x, theta=None):
    torch = pytest.importorskip("torch")
    t = synth.to_torch(x, DEV)
    th = None if theta is None else torch.from_numpy(theta).to(DEV)
    out = torch.full(tuple(t["q"].shape), float("nan"), device=DEV, dtype=torch.float32)
    lse = torch.empty(tuple(t["q"].shape[:3]), device=DEV, dtype=torch.float32)
    R.decode_reconstruct(t, rope_theta=th, shared_lr=case.shared_lr, out=out, lse=lse)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


CASES = [
    synth.Case(4, 32, 8, 128, 16, 32768, name="8B-shaped decode"),
    synth.Case(8, 64, 8, 128, 16, 20000, name="70B-shaped heads, two agent groups"),
    synth.Case(5, 8, 2, 128, 32, 3001, name="r=32, partial agent group, ragged"),
    synth.Case(6, 16, 2, 128, 16, 777, shared_lr=True, name="shared low-rank"),
    synth.Case(3, 8, 2, 128, 16, 1000, q_len=3, name="multi-token decode"),
    synth.Case(1, 4, 1, 128, 32, 65, name="single agent, two tiles"),
    synth.Case(2, 8, 2, 128, 16, 1500, name="two agents, four token groups each"),
    synth.Case(12, 8, 2, 128, 16, 2000, name="twelve agents, two groups of six"),
]


@pytest.mark.gpu
@pytest.mark.parametrize("rope", [False, True], ids=["unrotated", "rotated"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: c.name)
def test_reconstruct_parity(case, rope):
    x = synth.make_inputs(case, 51, b_sigma=0.3, q_scale=2.0)
    theta = synth.rope_theta(case.head_dim) if rope else None
    say(f"[gpu] reconstruct {case.name} rope={rope}")
    got, got_lse = run(case, x, theta)
    if rope:
        exp, exp_lse = recon.attend(case, x, rope=recon.table_from_theta(theta, case.prefix_len))
        # the rotation must matter: the unrotated result differs by far more than the bar
        unrot, _ = oracle.attend(case, x)
        assert np.abs(unrot - exp).max() > 10 * parity.MAX_ABS * 0.1
    else:
        exp, exp_lse = oracle.attend(case, x)
    s = parity.check(got, exp, "bf16", what=f"{case.name} rope={rope}")
    assert np.abs(got_lse - exp_lse).max() <= 2e-3 * max(1.0, np.abs(exp_lse).max())
    say(f"[gpu] reconstruct {case.name} rope={rope}: ok {s}")


@pytest.mark.gpu
def test_reconstruct_without_rotation_matches_decode():
    """Same inputs, no rotation: the rebuilt-key kernel and rattn_decode agree
    within the bars (they differ only in rounding order)."""
    torch = pytest.importorskip("torch")
    c = synth.WORKLOADS[1]
    x = synth.make_inputs(c, 1, **synth.STRESS)
    got, _ = run(c, x)
    t = synth.to_torch(x, DEV)
    ref = R.attend(t)
    torch.cuda.synchronize()
    parity.check(got, ref.cpu().numpy().astype(np.float64), "bf16", what="reconstruct vs decode")
