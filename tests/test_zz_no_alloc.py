"""rattn_decode_noalloc (the entry point for callers that cannot allocate)
against rattn_decode on the same inputs, through the C ABI: two calls in a
row, the second with a smaller input, each bit-identical to rattn_decode with
a caller workspace and within the parity bars of the fp64 oracle."""
import ctypes

import numpy as np
import pytest

import oracle
import synth
from tests import parity

torch = pytest.importorskip("torch")

DEV = "cuda"


@pytest.mark.gpu
def test_noalloc_matches_workspace_entry_point_twice():
    import shared_base_residual_amd as R

    R.lib()
    cases = [synth.Case(4, 32, 8, 128, 16, 9000, priv_len=33, name="larger"),
             synth.Case(3, 8, 2, 128, 64, 1500, priv_len=10, name="smaller")]
    for i, c in enumerate(cases):
        x = synth.make_inputs(c, 900 + i, b_sigma=0.3, q_scale=2.0)
        t = synth.to_torch(x, DEV)
        desc = R.describe(t["q"], t["k_base"], t["lk"], t["bk"], k_priv=t["k_priv"])
        assert R.workspace_bytes(desc) <= R.NOALLOC_SCRATCH_BYTES
        ref = torch.full(tuple(t["q"].shape), float("nan"), device=DEV, dtype=torch.float32)
        ref_lse = torch.empty(tuple(t["q"].shape[:3]), device=DEV, dtype=torch.float32)
        R.attend(t, out=ref, lse=ref_lse)
        got = torch.full_like(ref, float("nan"))
        got_lse = torch.empty_like(ref_lse)
        R.decode_noalloc(t, out=got, lse=got_lse)
        torch.cuda.synchronize()
        assert torch.equal(got, ref) and torch.equal(got_lse, ref_lse), c.name
        exp, _ = oracle.attend(c, x)
        parity.check(got.cpu().numpy().astype(np.float64), exp, "bf16", what=f"noalloc {c.name}")


def test_noalloc_rejects_calls_beyond_the_scratch():
    """Host-only: a call whose partials exceed the static buffer returns
    RATTN_E_SCRATCH before any HIP call."""
    import shared_base_residual_amd as R

    d = R.make_desc(n_agents=64, n_q_heads=64, n_kv_heads=8, head_dim=128, rank=64, q_len=64, prefix_len=4096)
    assert R.workspace_bytes(d) > R.NOALLOC_SCRATCH_BYTES
    F = 0x10000  # never dereferenced: the call returns before any HIP call
    args = R.Args(F, F, F, None, F, F, F, F, None, None, F, None)
    assert R.lib().rattn_decode_noalloc(ctypes.byref(d), ctypes.byref(args), None) == -7
    assert R.lib().rattn_status_str(-7).startswith(b"call needs more")
