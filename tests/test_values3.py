"""Base values as 3-bit codes after a Walsh-Hadamard rotation, with int8 keys
(PolyKV, section 2B: the asymmetric scheme, int8 keys and 3-bit rotated values).

Host: validation of the descriptor, the arguments and rattn_quantize_values,
and the library's codebook against the oracle's (each derived on its own from
the Lloyd-Max conditions).  GPU: rattn_quantize_values against the oracle's
encoder (codes bit for bit except where a coordinate sits within 1e-12 of a
cell boundary, where the two codebooks may round apart; scales bit for bit for
bf16 vectors), and decode over int8 keys and 3-bit values end to end -- the
GPU encodes the seeded bf16 keys and values and attends over its codes, the
oracle encodes the same bf16 keys and values itself and attends over its own
decoded ones -- within the parity bars."""
import ctypes
import os
import sys

import numpy as np
import pytest

import oracle
import synth
from oracle import quant as Q
from oracle import values3 as V3
from tests import kernel_paths as KP
from tests import parity

import shared_base_residual_amd as R

pytestmark = pytest.mark.skipif(not os.path.exists(R.LIB_PATH), reason="librattn not built")
DEV = "cuda"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def v3_desc(**kw):
    base = dict(n_agents=4, n_q_heads=32, n_kv_heads=8, head_dim=128, rank=16, q_len=1, prefix_len=4096,
                k_format=R.RATTN_KEYS_INT8, k_scale=0.03, v_format=R.RATTN_VALUES_FWHT3)
    base.update(kw)
    return R.make_desc(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(), 0),
    (dict(k_format=R.RATTN_KEYS_DTYPE), -3),
    (dict(page_size=16, n_phys_pages=300), -3),
    (dict(priv_len=10), -3),
    (dict(v_format=4), -2),
])
def test_values3_validation(kw, status):
    n = ctypes.c_size_t()
    assert R.lib().rattn_workspace_bytes(ctypes.byref(v3_desc(**kw)), R.RATTN_OP_DECODE, ctypes.byref(n)) == status


def test_values3_not_for_prefill_or_rebuilt_keys():
    n = ctypes.c_size_t()
    d = v3_desc(q_len=8, priv_len=8)
    assert R.lib().rattn_workspace_bytes(ctypes.byref(d), R.RATTN_OP_PREFILL, ctypes.byref(n)) == -3
    d = v3_desc(k_format=R.RATTN_KEYS_DTYPE)
    assert R.lib().rattn_workspace_bytes(ctypes.byref(d), R.RATTN_OP_RECONSTRUCT, ctypes.byref(n)) == -3


def test_values3_scale_pointer_checks():
    """The scales are required with 3-bit values and refused without them;
    misaligned scales are refused.  Every check runs before any HIP call."""
    F = 0x10000
    lib = R.lib()
    fields = {n: F for n in R.ARG_NAMES}
    fields.update(block_table=None, k_priv=None, v_priv=None, lse=None)
    ws = ctypes.c_void_p(F)
    for desc, vs, want in [(v3_desc(), None, -1), (v3_desc(), F + 4, -5),
                           (v3_desc(k_format=R.RATTN_KEYS_INT8, v_format=R.RATTN_VALUES_DTYPE), F, -1)]:
        a = R.Args(*[vs if n == "v_scale" else fields[n] for n in R.ARG_NAMES])
        assert lib.rattn_decode(ctypes.byref(desc), ctypes.byref(a), ws, ctypes.c_size_t(1 << 40), None) == want


def test_quantize_values_validation():
    F = 0x10000
    lib = R.lib()
    assert lib.rattn_quantize_values(F, 0, 128, R.RATTN_BF16, F, F, None) == -2
    assert lib.rattn_quantize_values(F, 8, 96, R.RATTN_BF16, F, F, None) == -3
    assert lib.rattn_quantize_values(F, 8, 128, 7, F, F, None) == -3
    assert lib.rattn_quantize_values(None, 8, 128, R.RATTN_BF16, F, F, None) == -1
    assert lib.rattn_quantize_values(F + 1, 8, 128, R.RATTN_BF16, F, F, None) == -5
    assert lib.rattn_quantize_values(F, 8, 128, R.RATTN_BF16, F + 4, F, None) == -5


def test_library_codebook_is_the_oracles():
    c, b = R.values_codebook()
    oc, ob = V3.lloyd_max_normal()
    assert np.abs(np.array(c) - oc).max() <= 1e-13
    assert np.abs(np.array(b) - ob).max() <= 1e-13
    assert b[3] == 0.0


def test_values3_plans_and_kernels():
    """3-bit values run the int8-key kernels' own 3-bit variants, one for each."""
    for kw in (dict(), dict(n_agents=8, n_q_heads=64, rank=16), dict(n_agents=9, n_q_heads=8, n_kv_heads=2,
                                                                      rank=64), dict(rank=0)):
        k8 = R.kernel_of(v3_desc(v_format=R.RATTN_VALUES_DTYPE, **kw))
        k3 = R.kernel_of(v3_desc(**kw))
        assert R.decode_plan(v3_desc(**kw))["work_items"] >= 1
        assert k3[1] == "bf16-k8v3" and k8[1] == "bf16-k8" and k3[2:4] == k8[2:4]


# --------------------------------------------------------------------- GPU --

def _codes_match(got_packed, v, d):
    """Codes equal the oracle's except for coordinates within 1e-12 of a
    boundary, where either neighbouring code is accepted."""
    _, bnd = V3.lloyd_max_normal()
    u = V3.normalized_coords(v)
    exp = V3.codes_of(u, bnd)
    got = V3.unpack_planes(got_packed, d)
    diff = got != exp
    if not diff.any():
        return 0
    near = np.min(np.abs(u[..., None] - bnd), axis=-1) <= 1e-12
    assert np.all(near[diff]), "codes differ away from a boundary"
    assert np.all(np.abs(got[diff].astype(int) - exp[diff].astype(int)) == 1)
    return int(diff.sum())


@pytest.mark.gpu
@pytest.mark.parametrize("dtype,shape", [("bf16", (8, 4096, 128)), ("f32", (3, 333, 64)), ("bf16", (5, 77, 128)),
                                         ("bf16", (2, 50, 64))])
def test_quantize_values_matches_the_oracle(dtype, shape):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(41)
    v = rng.standard_normal(shape) * np.exp(rng.standard_normal(shape[:-1] + (1,)))
    v[0, :3] = 0.0  # zero vectors: every code at the cell of 0, scale 0
    x = synth.bf16_bits(v) if dtype == "bf16" else v.astype(np.float32)
    say(f"[gpu] quantize values {dtype} {shape}")
    t = synth.to_torch({"v": x}, DEV)["v"]
    codes, scale = R.quantize_values(t)
    torch.cuda.synchronize()
    got_c, got_s = codes.cpu().numpy(), scale.cpu().numpy()
    exp_c, exp_s = V3.quantize_values(x)
    assert got_c.shape == exp_c.shape and got_s.shape == exp_s.shape
    n_tie = _codes_match(got_c, x, shape[-1])
    if dtype == "bf16":
        assert np.array_equal(got_s, exp_s)
    else:  # ||v||^2 of fp32 vectors is rounded: the scale within one unit in the last place
        assert np.all(np.abs(got_s.view(np.int32).astype(np.int64) - exp_s.view(np.int32).astype(np.int64)) <= 1)
    assert np.all(got_s[0, :3] == 0) and np.all(V3.unpack_planes(got_c[0, :3], shape[-1]) == 4)
    say(f"[gpu] quantize values {dtype} {shape}: ok ({n_tie} boundary ties)")


def run_v3(case, x):
    """GPU: encode the bf16 keys and values, decode over the codes."""
    torch = pytest.importorskip("torch")
    t = synth.to_torch(x, DEV)
    kcodes, kscale = R.quantize_keys(t["k_base"])
    vcodes, vscale = R.quantize_values(t["v_base"])
    s = float(kscale.cpu().numpy()[0])
    t3 = dict(t, k_base=kcodes, v_base=vcodes, v_scale=vscale)
    out = torch.full(tuple(t["q"].shape), float("nan"), device=DEV, dtype=torch.float32)
    lse_t = torch.empty(tuple(t["q"].shape[:3]), device=DEV, dtype=torch.float32)
    R.attend(t3, shared_lr=case.shared_lr, prefix_len=case.prefix_len, out=out, lse=lse_t, k_scale=s)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), lse_t.cpu().numpy().astype(np.float64)


def ref_v3(case, x):
    """Oracle: its own encoding of the same bf16 keys and values, then
    attention over the dequantised keys and decoded values."""
    kc, ks = Q.quantize_keys(x["k_base"])
    vc, vs = V3.quantize_values(x["v_base"])
    return oracle.attend(case, V3.widen(x, kc, ks, vc, vs)), (kc, ks, vc, vs)


def compare_v3(case, x, what, with_b0=False):
    say(f"[gpu] 3-bit values {what}: {case}")
    got, got_lse = run_v3(case, x)
    (exp, exp_lse), enc = ref_v3(case, x)
    b0 = None
    if with_b0:
        x0 = dict(x, bk=np.zeros_like(x["bk"]), bv=np.zeros_like(x["bv"]))
        b0, _ = oracle.attend(case, V3.widen(x0, *enc))
    st = parity.check(got, exp, "bf16", b0, what)
    assert np.abs(got_lse - exp_lse).max() <= 2e-3 * max(1.0, np.abs(exp_lse).max()), what
    say(f"[gpu] 3-bit values {what}: ok {st}")
    return st


@pytest.mark.gpu
def test_values3_llama8b_decode():
    """The 8B-shaped decode (4 agents, 32768-token prefix, r = 16) over int8
    keys and 3-bit values."""
    c = synth.WORKLOADS[1]
    compare_v3(c, synth.make_inputs(c, 1), "8B-shaped decode", with_b0=True)


@pytest.mark.gpu
def test_values3_70b_layer():
    """One layer of the 70B-shaped decode (8 agents, g = 8, 65536-token prefix)."""
    c = synth.WORKLOADS[4].replace(layers=1)
    compare_v3(c, synth.make_inputs(c, 4), "70B-shaped layer", with_b0=True)


V3_EDGE = [
    synth.Case(6, 16, 2, 128, 32, 777, shared_lr=True, name="shared low-rank"),
    synth.Case(3, 8, 2, 128, 0, 1001, name="rank 0, ragged tail"),
    synth.Case(2, 8, 2, 128, 16, 290, q_len=3, name="multi-token decode"),
    synth.Case(2, 4, 1, 128, 16, 40000, name="more than 64 splits"),
    synth.Case(9, 8, 2, 128, 64, 3000, name="masked r=64"),
    synth.Case(1, 4, 1, 128, 16, 17, name="one full group and one token"),
]


@pytest.mark.gpu
@pytest.mark.parametrize("case", V3_EDGE, ids=lambda c: c.name)
def test_values3_edge(case):
    x = synth.make_inputs(case, 43, b_sigma=0.3, q_scale=2.0)
    compare_v3(case, x, case.name)


@pytest.mark.gpu
def test_values3_zero_vectors():
    """Value vectors that are zero decode to zero (scale 0)."""
    case = synth.Case(2, 8, 2, 128, 16, 500, name="zero values")
    x = synth.make_inputs(case, 44, b_sigma=0.3, q_scale=2.0)
    x["v_base"] = x["v_base"].copy()
    x["v_base"][:, 100:260] = 0
    compare_v3(case, x, case.name)


@pytest.mark.gpu
@pytest.mark.parametrize("key,case", KP.PATHS_K8, ids=[c.name for _, c in KP.PATHS_K8])
def test_values3_kernel_path(key, case):
    """Every int8-key kernel instantiation, with 3-bit values."""
    if case.page_size:
        pytest.skip("3-bit values need a contiguous base cache")
    x = synth.make_inputs(case, 79, b_sigma=0.3, q_scale=2.0)
    compare_v3(case, x, f"{case.name} {key} 3-bit values")
