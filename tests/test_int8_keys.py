"""Base keys as int8 codes with one scale per tensor (PolyKV, section 2B).

Host: validation of the int8-key descriptor.  GPU: rattn_quantize_keys
against the oracle's quantiser bit for bit (codes and scale), and decode over
int8 keys end to end -- the GPU quantises the seeded bf16 keys and attends
over its codes, the oracle quantises the same bf16 keys itself and attends
over its dequantised keys -- within the parity bars."""
import ctypes
import os
import sys

import numpy as np
import pytest

import oracle
import synth
from oracle import quant as Q
from tests import kernel_paths as KP
from tests import parity

import shared_base_residual_amd as R

pytestmark = pytest.mark.skipif(not os.path.exists(R.LIB_PATH), reason="librattn not built")
DEV = "cuda"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def k8_desc(**kw):
    base = dict(n_agents=4, n_q_heads=32, n_kv_heads=8, head_dim=128, rank=16, q_len=1, prefix_len=4096,
                k_format=R.RATTN_KEYS_INT8, k_scale=0.03)
    base.update(kw)
    return R.make_desc(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(), 0),
    (dict(dtype=R.RATTN_F32), -3),
    (dict(head_dim=64), -3),
    (dict(priv_len=10), -3),
    (dict(prefix_len=0, priv_len=10), -3),
    (dict(k_scale=0.0), -2),
    (dict(k_scale=float("nan")), -2),
    (dict(k_format=5), -2),
])
def test_int8_key_validation(kw, status):
    n = ctypes.c_size_t()
    assert R.lib().rattn_workspace_bytes(ctypes.byref(k8_desc(**kw)), R.RATTN_OP_DECODE, ctypes.byref(n)) == status


def test_int8_keys_not_for_prefill():
    d = k8_desc(q_len=8, priv_len=8)
    n = ctypes.c_size_t()
    assert R.lib().rattn_workspace_bytes(ctypes.byref(d), R.RATTN_OP_PREFILL, ctypes.byref(n)) == -3


def test_quantize_validation():
    F = 0x10000
    lib = R.lib()
    assert lib.rattn_quantize_keys(F, 0, R.RATTN_BF16, F, F, None) == -2
    assert lib.rattn_quantize_keys(F, 8, 7, F, F, None) == -3
    assert lib.rattn_quantize_keys(None, 8, R.RATTN_BF16, F, F, None) == -1
    assert lib.rattn_quantize_keys(F + 1, 8, R.RATTN_BF16, F, F, None) == -5


# --------------------------------------------------------------------- GPU --

@pytest.mark.gpu
@pytest.mark.parametrize("dtype,shape", [("bf16", (8, 32768, 128)), ("f32", (3, 1000, 64)), ("bf16", (5, 77))])
def test_quantize_keys_bit_exact(dtype, shape):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(21)
    v = rng.standard_normal(shape) * 1.7
    k = synth.bf16_bits(v) if dtype == "bf16" else v.astype(np.float32)
    say(f"[gpu] quantize {dtype} {shape}")
    t = synth.to_torch({"k": k}, DEV)["k"]
    codes, scale = R.quantize_keys(t)
    torch.cuda.synchronize()
    exp_codes, exp_scale = Q.quantize_keys(k)
    assert scale.cpu().numpy()[0] == exp_scale
    got = codes.cpu().numpy()
    assert got.shape == exp_codes.shape and np.array_equal(got, exp_codes)


def run_k8(case, x, *, lse=True):
    """GPU: quantise the bf16 keys with rattn_quantize_keys, decode over the codes."""
    torch = pytest.importorskip("torch")
    t = synth.to_torch(x, DEV)
    codes, scale = R.quantize_keys(t["k_base"])
    s = float(scale.cpu().numpy()[0])
    t8 = dict(t, k_base=codes)
    out = torch.full(tuple(t["q"].shape), float("nan"), device=DEV, dtype=torch.float32)
    lse_t = torch.empty(tuple(t["q"].shape[:3]), device=DEV, dtype=torch.float32)
    R.attend(t8, shared_lr=case.shared_lr, prefix_len=case.prefix_len, out=out, lse=lse_t, k_scale=s)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), lse_t.cpu().numpy().astype(np.float64), codes.cpu().numpy(), s


def ref_k8(case, x):
    """Oracle: its own quantisation of the same bf16 keys, then attention over
    the dequantised keys (every other input widened exactly)."""
    codes, s = Q.quantize_keys(x["k_base"])
    return oracle.attend(case, Q.widen(x, codes, s)), codes, s


def compare_k8(case, x, what, with_b0=False):
    say(f"[gpu] int8 keys {what}: {case}")
    got, got_lse, gcodes, gs = run_k8(case, x)
    (exp, exp_lse), codes, s = ref_k8(case, x)
    assert gs == s and np.array_equal(gcodes, codes), "quantised keys differ from the oracle's"
    b0 = None
    if with_b0:
        x0 = dict(x, bk=np.zeros_like(x["bk"]), bv=np.zeros_like(x["bv"]))
        b0, _ = oracle.attend(case, Q.widen(x0, codes, s))
    st = parity.check(got, exp, "bf16", b0, what)
    assert np.abs(got_lse - exp_lse).max() <= 2e-3 * max(1.0, np.abs(exp_lse).max()), what
    say(f"[gpu] int8 keys {what}: ok {st}")
    return st


@pytest.mark.gpu
@pytest.mark.parametrize("variant", ["base", "stress"])
def test_int8_keys_llama8b_decode(variant):
    """The 8B-shaped decode (4 agents, 32768-token prefix, r = 16) over int8 keys."""
    c = synth.WORKLOADS[1]
    kw = synth.STRESS if variant == "stress" else {}
    x = synth.make_inputs(c, 1 + (synth.STRESS_SEED_OFFSET if variant == "stress" else 0), **kw)
    compare_k8(c, x, f"8B-shaped decode {variant}", with_b0=(variant == "base"))


@pytest.mark.gpu
def test_int8_keys_70b_layer():
    """One layer of the 70B-shaped decode (8 agents, g = 8, 65536-token prefix)."""
    c = synth.WORKLOADS[4].replace(layers=1)
    x = synth.make_inputs(c, 4)
    compare_k8(c, x, "70B-shaped layer", with_b0=True)


K8_PAGED = synth.Case(9, 8, 2, 128, 64, 3000, page_size=16, n_phys_pages=400, name="paged, masked r=64")
K8_EDGE = [
    synth.Case(6, 16, 2, 128, 32, 777, shared_lr=True, name="shared low-rank"),
    synth.Case(3, 8, 2, 128, 0, 1001, name="rank 0"),
    synth.Case(2, 8, 2, 128, 16, 290, q_len=3, name="multi-token decode"),
    synth.Case(2, 4, 1, 128, 16, 40000, name="more than 64 splits"),
]


@pytest.mark.gpu
@pytest.mark.parametrize("case", K8_EDGE, ids=lambda c: c.name)
def test_int8_keys_edge(case):
    x = synth.make_inputs(case, 33, b_sigma=0.3, q_scale=2.0)
    compare_k8(case, x, case.name)


@pytest.mark.gpu
def test_int8_keys_paged():
    """A paged int8 pool: the codes of a shuffled pool (unused pages zero) give
    the same output bits as the codes of the identity pool."""
    torch = pytest.importorskip("torch")
    c = K8_PAGED
    x = synth.make_inputs(c, 34, b_sigma=0.3, q_scale=2.0)
    table = x["block_table"]
    used = np.zeros(c.n_phys_pages, bool)
    used[table] = True
    for key in ("k_base", "v_base"):  # the quantiser covers every page given to it: no NaN pages
        x[key] = x[key].copy()
        x[key][~used] = 0
    say("[gpu] int8 keys paged")
    got, got_lse, gcodes, gs = run_k8(c, x)
    (exp, exp_lse), codes, s = ref_k8(c, x)
    assert gs == s and np.array_equal(gcodes, codes)
    parity.check(got, exp, "bf16", what="int8 keys paged")
    # identity pool holding the same logical pages
    ident = dict(x)
    n = c.n_table
    for key in ("k_base", "v_base"):
        pool = np.zeros_like(x[key])
        pool[:n] = x[key][table]
        ident[key] = pool
    ident["block_table"] = np.arange(n, dtype=np.int32)
    got2, lse2, _, gs2 = run_k8(c, ident)
    assert gs2 == gs and np.array_equal(got, got2) and np.array_equal(got_lse, lse2)


@pytest.mark.gpu
@pytest.mark.parametrize("key,case", KP.PATHS_K8, ids=[c.name for _, c in KP.PATHS_K8])
def test_int8_key_kernel_path(key, case):
    """One workload per int8-key kernel instantiation."""
    x = synth.make_inputs(case, 78, b_sigma=0.3, q_scale=2.0)
    compare_k8(case, x, f"{case.name} {key}")
