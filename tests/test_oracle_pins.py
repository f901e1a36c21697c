"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each test names the passage or mathematical fact it relies on.  The mutant test
at the end rebuilds the oracle with one planted mistake at a time and checks
that these pins catch every one of them.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TOL = 1e-12


def _f64(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return synth.bf16_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def _sdpa(q, k, v, scale=None):
    """Library attention (torch, fp64, CPU): q [B, Hq, T, d], k/v [B, Hq, S, d]."""
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), scale=scale).numpy()


def _logical_base(case, x):
    if case.page_size:
        return (_f64(oracle.gather_base(case, x["k_base"], x["block_table"])),
                _f64(oracle.gather_base(case, x["v_base"], x["block_table"])))
    return _f64(x["k_base"]), _f64(x["v_base"])


TINY = [
    synth.Case(2, 4, 2, 4, 2, 5, dtype="bf16", name="contiguous bf16"),
    synth.Case(3, 2, 1, 3, 2, 4, priv_len=2, dtype="f32", name="suffix f32 g=2"),
    synth.Case(2, 2, 2, 4, 1, 6, page_size=2, n_phys_pages=5, dtype="bf16", name="paged"),
    synth.Case(3, 2, 1, 3, 2, 3, shared_lr=True, dtype="bf16", name="shared low-rank"),
    synth.Case(2, 2, 1, 3, 2, 3, priv_len=3, q_len=3, mode="prefill", shared_lr=True, dtype="bf16",
               name="causal chunk"),
    synth.Case(2, 3, 1, 2, 0, 4, priv_len=1, dtype="f32", name="rank 0"),
    synth.Case(1, 1, 1, 2, 1, 0, priv_len=2, dtype="f32", name="suffix only"),
]


@pytest.mark.parametrize("case", TINY, ids=lambda c: c.name)
def test_brute_force_tiny(case):
    """Pin: brute force on tiny shapes (40-digit decimal, independent code)."""
    x = synth.make_inputs(case, 7, b_sigma=0.7, q_scale=2.0)
    ob, lb = brute.to_float(*brute.attend(case, x))
    oc, lc = oracle.attend(case, x)
    assert np.abs(ob - oc).max() <= 1e-13 * max(1.0, np.abs(ob).max())
    assert np.abs(lb - lc).max() <= 1e-13 * max(1.0, np.abs(lb).max())


def test_golden_fixtures():
    """Stored 40-digit values (written by tests/golden/make_golden.py from oracle.brute)."""
    with open(os.path.join(GOLDEN, "brute_tiny.json")) as f:
        gold = json.load(f)
    assert gold["cases"], "empty fixture"
    for g in gold["cases"]:
        case = synth.Case(**g["case"])
        x = synth.make_inputs(case, g["seed"], **g["kwargs"])
        oc, lc = oracle.attend(case, x)
        ref = np.array([float(v) for v in g["out"]]).reshape(oc.shape)
        refl = np.array([float(v) for v in g["lse"]]).reshape(lc.shape)
        assert np.abs(oc - ref).max() <= 1e-13 * max(1.0, np.abs(ref).max()), g["case"]["name"]
        assert np.abs(lc - refl).max() <= 1e-13 * max(1.0, np.abs(refl).max()), g["case"]["name"]


def _gqa_expand(kv, g):
    return np.repeat(kv, g, axis=0)  # consecutive query heads share a KV head


@pytest.mark.parametrize("paged", [False, True])
def test_b_zero_is_plain_attention(paged):
    """B = 0: every agent sees the base cache only (ForkKV Guide, section 1 of the
    decomposition: K_base and V_base do not depend on the adapter), so the result is
    library attention over the base with GQA sharing and scale 1/sqrt(d)."""
    case = synth.Case(3, 8, 2, 16, 4, 40, dtype="bf16")
    if paged:
        case = case.replace(page_size=8, n_phys_pages=9)
    x = synth.make_inputs(case, 3, zero=("bk", "bv"))
    o, lse = oracle.attend(case, x)
    kb, vb = _logical_base(case, x)
    q = _f64(x["q"])                                    # [N, 1, Hq, d]
    g = case.group
    for a in range(case.n_agents):
        ref = _sdpa(q[a].transpose(1, 0, 2)[None], _gqa_expand(kb, g)[None], _gqa_expand(vb, g)[None])[0]
        assert np.abs(o[a] - ref.transpose(1, 0, 2)).max() <= TOL
    # lse closed form against numpy logsumexp of the scores
    s = np.einsum("nhd,hld->nhl", q[:, 0], _gqa_expand(kb, g)) / np.sqrt(case.head_dim)
    m = s.max(-1, keepdims=True)
    ref_lse = (m + np.log(np.exp(s - m).sum(-1, keepdims=True)))[..., 0]
    assert np.abs(lse[:, 0] - ref_lse).max() <= TOL


def test_single_agent_is_standard_attention():
    """N = 1: the call is one adapter's attention over K_1 = K_base + Lk Bk, V_1 likewise
    (the decomposition of an adapted cache into base plus low-rank residual), computed here by the
    library routine."""
    case = synth.Case(1, 4, 2, 8, 3, 33, priv_len=5, dtype="f32")
    x = synth.make_inputs(case, 4, b_sigma=0.3)
    o, _ = oracle.attend(case, x)
    d = case.head_dim
    kb, vb = _f64(x["k_base"]), _f64(x["v_base"])
    lk, lv, bk, bv = (_f64(x[n])[0] for n in ("lk", "lv", "bk", "bv"))
    ks, vs = [], []
    for k in range(case.n_kv_heads):
        kk = np.concatenate([kb[k] + lk @ bk[:, k * d:(k + 1) * d], _f64(x["k_priv"])[0, k]])
        vv = np.concatenate([vb[k] + lv @ bv[:, k * d:(k + 1) * d], _f64(x["v_priv"])[0, k]])
        ks.append(kk)
        vs.append(vv)
    K = _gqa_expand(np.stack(ks), case.group)[None]
    V = _gqa_expand(np.stack(vs), case.group)[None]
    ref = _sdpa(_f64(x["q"])[0].transpose(1, 0, 2)[None], K, V)[0].transpose(1, 0, 2)
    assert np.abs(o[0] - ref).max() <= TOL


def _factorised(case, x):
    """Independent fp64 evaluation of the fused form (contiguous base, decode):
    s = scale (q K_b^T + (q Bk^T) Lk^T)  [ForkKV Guide, AttnScore split into base and residual dot products]
    o = P V_b + (P Lv) Bv                 [LRAgent, Flash-LoRA-Attention reordering]."""
    d, g = case.head_dim, case.group
    q = _f64(x["q"])[:, 0]
    kb, vb = _logical_base(case, x)
    lk, lv, bk, bv = (_f64(x[n]) for n in ("lk", "lv", "bk", "bv"))
    out = np.zeros((case.n_agents, case.n_q_heads, d))
    for a in range(case.n_agents):
        lr = 0 if case.shared_lr else a
        for h in range(case.n_q_heads):
            k = h // g
            bkk, bvk = bk[a][:, k * d:(k + 1) * d], bv[a][:, k * d:(k + 1) * d]
            u = bkk @ q[a, h]                               # [r]
            s = (kb[k] @ q[a, h] + lk[lr] @ u) / np.sqrt(d)
            vals = [vb[k]]
            if case.priv_len:
                s = np.concatenate([s, _f64(x["k_priv"])[a, k] @ q[a, h] / np.sqrt(d)])
            p = np.exp(s - s.max())
            p /= p.sum()
            pb = p[: case.prefix_len]
            o = pb @ vb[k] + (pb @ lv[lr]) @ bvk
            if case.priv_len:
                o = o + p[case.prefix_len:] @ _f64(x["v_priv"])[a, k]
            out[a, h] = o
    return out


@pytest.mark.parametrize("shared", [False, True])
def test_factorised_identity(shared):
    """The fused (factorised) evaluation equals the materialised one (ForkKV Guide FAQ:
    the reformulation is exact; LRAgent, Flash-LoRA-Attention associativity)."""
    case = synth.Case(3, 8, 2, 16, 8, 50, priv_len=6, shared_lr=shared, page_size=8, n_phys_pages=11,
                      dtype="bf16")
    x = synth.make_inputs(case, 5, b_sigma=0.3, q_scale=2.0)
    o, _ = oracle.attend(case, x)
    assert np.abs(o[:, 0] - _factorised(case, x)).max() <= TOL


def test_zero_query_closed_form():
    """q = 0 gives uniform weights, so o = mean_j V_b[j] + (mean_j Lv[j]) Bv (plus the
    private values in the mean) and lse = ln(number of keys); no exponential involved."""
    case = synth.Case(2, 4, 2, 8, 4, 24, priv_len=3, dtype="f32")
    x = synth.make_inputs(case, 6, zero=("q",))
    o, lse = oracle.attend(case, x)
    d, g, L, S = case.head_dim, case.group, case.prefix_len, case.priv_len
    for a in range(case.n_agents):
        for h in range(case.n_q_heads):
            k = h // g
            vsum = _f64(x["v_base"])[k].sum(0) + _f64(x["lv"])[a].sum(0) @ _f64(x["bv"])[a][:, k * d:(k + 1) * d]
            vsum = vsum + _f64(x["v_priv"])[a, k].sum(0)
            assert np.abs(o[a, 0, h] - vsum / (L + S)).max() <= TOL
    assert np.abs(lse - np.log(L + S)).max() <= TOL


def test_single_key_closed_form():
    """L + S = 1: the only key gets weight one, so o = V_b[0] + Lv[0] Bv and lse = s_0."""
    case = synth.Case(2, 2, 1, 6, 3, 1, dtype="f32")
    x = synth.make_inputs(case, 8, b_sigma=0.5)
    o, lse = oracle.attend(case, x)
    d = case.head_dim
    for a in range(case.n_agents):
        bk, bv = _f64(x["bk"])[a][:, :d], _f64(x["bv"])[a][:, :d]
        k0 = _f64(x["k_base"])[0, 0] + _f64(x["lk"])[a, 0] @ bk
        v0 = _f64(x["v_base"])[0, 0] + _f64(x["lv"])[a, 0] @ bv
        for h in range(2):
            assert np.abs(o[a, 0, h] - v0).max() <= TOL
            assert abs(lse[a, 0, h] - _f64(x["q"])[a, 0, h] @ k0 / np.sqrt(d)) <= TOL


def test_split_pins():
    """Each residual separately: with Bk = 0 only the value correction acts,
    o = softmax(base scores) (V_b + Lv Bv); with Bv = 0 only the score correction acts,
    o = softmax(scores of K_b + Lk Bk) V_b.  Both evaluated with library attention."""
    case = synth.Case(2, 4, 2, 8, 4, 30, dtype="bf16")
    d, g = case.head_dim, case.group
    for zero in ("bk", "bv"):
        x = synth.make_inputs(case, 9, b_sigma=0.4, zero=(zero,))
        o, _ = oracle.attend(case, x)
        for a in range(case.n_agents):
            K = np.stack([_f64(x["k_base"])[k] + _f64(x["lk"])[a] @ _f64(x["bk"])[a][:, k * d:(k + 1) * d]
                          for k in range(case.n_kv_heads)])
            V = np.stack([_f64(x["v_base"])[k] + _f64(x["lv"])[a] @ _f64(x["bv"])[a][:, k * d:(k + 1) * d]
                          for k in range(case.n_kv_heads)])
            ref = _sdpa(_f64(x["q"])[a].transpose(1, 0, 2)[None], _gqa_expand(K, g)[None],
                        _gqa_expand(V, g)[None])[0].transpose(1, 0, 2)
            assert np.abs(o[a] - ref).max() <= TOL, zero


def test_key_permutation_invariance():
    """Without positional rotation (the pages apply none to the residual), jointly
    permuting the prefix rows of K_b, V_b, Lk, Lv, and the private rows, leaves
    every output unchanged."""
    case = synth.Case(2, 4, 2, 8, 4, 37, priv_len=5, dtype="f32")
    x = synth.make_inputs(case, 10, b_sigma=0.3)
    o, lse = oracle.attend(case, x)
    rng = np.random.default_rng(0)
    p, ps = rng.permutation(case.prefix_len), rng.permutation(case.priv_len)
    y = dict(x)
    y["k_base"], y["v_base"] = x["k_base"][:, p], x["v_base"][:, p]
    y["lk"], y["lv"] = x["lk"][:, p], x["lv"][:, p]
    y["k_priv"], y["v_priv"] = x["k_priv"][:, :, ps], x["v_priv"][:, :, ps]
    o2, lse2 = oracle.attend(case, y)
    assert np.abs(o - o2).max() <= TOL and np.abs(lse - lse2).max() <= TOL
    # ... while a permutation of Lk alone (breaking the row pairing) changes the output
    z = dict(x)
    z["lk"] = x["lk"][:, p]
    o3, _ = oracle.attend(case, z)
    assert np.abs(o - o3).max() > 1e-3


def test_agent_permutation_equivariance():
    """Agents do not interact: permuting the agents' inputs permutes the outputs."""
    case = synth.Case(4, 4, 2, 8, 4, 20, priv_len=3, dtype="bf16")
    x = synth.make_inputs(case, 11, b_sigma=0.3)
    o, _ = oracle.attend(case, x)
    p = np.array([2, 0, 3, 1])
    y = dict(x)
    for n in ("q", "lk", "lv", "bk", "bv", "k_priv", "v_priv"):
        y[n] = x[n][p]
    o2, _ = oracle.attend(case, y)
    assert np.abs(o[p] - o2).max() == 0.0


def test_shared_low_rank_cache():
    """BaseLRShared (LRAgent, Schemi di Condivisione): with shared A one low-rank cache
    serves all agents; the shared call equals the per-agent call with N identical
    copies, bit for bit, and agents with identical B and q get identical outputs."""
    base = synth.Case(3, 4, 2, 8, 4, 21, priv_len=2, dtype="bf16")
    shared = base.replace(shared_lr=True)
    x = synth.make_inputs(shared, 12, b_sigma=0.3)
    o_s, l_s = oracle.attend(shared, x)
    y = dict(x)
    y["lk"] = np.repeat(x["lk"], 3, axis=0)
    y["lv"] = np.repeat(x["lv"], 3, axis=0)
    o_p, l_p = oracle.attend(base, y)
    assert np.array_equal(o_s, o_p) and np.array_equal(l_s, l_p)
    z = dict(x)
    for n in ("q", "bk", "bv"):
        z[n] = np.repeat(x[n][:1], 3, axis=0)
    z["k_priv"] = np.repeat(x["k_priv"][:1], 3, axis=0)
    z["v_priv"] = np.repeat(x["v_priv"][:1], 3, axis=0)
    o_z, _ = oracle.attend(shared, z)
    assert np.array_equal(o_z[0], o_z[1]) and np.array_equal(o_z[0], o_z[2])


def test_prefill_matches_decode():
    """A causal chunk: query t sees the prefix and chunk tokens 0..t, so its output
    equals a decode call whose private suffix is the first t+1 chunk tokens."""
    pre = synth.Case(2, 4, 2, 8, 4, 19, priv_len=6, q_len=6, mode="prefill", shared_lr=True, dtype="bf16")
    x = synth.make_inputs(pre, 13, b_sigma=0.3)
    o, lse = oracle.attend(pre, x)
    for t in range(pre.q_len):
        dec = pre.replace(priv_len=t + 1, q_len=1, mode="decode")
        y = dict(x)
        y["q"] = x["q"][:, t:t + 1]
        y["k_priv"] = x["k_priv"][:, :, :t + 1]
        y["v_priv"] = x["v_priv"][:, :, :t + 1]
        od, ld = oracle.attend(dec, y)
        assert np.abs(o[:, t] - od[:, 0]).max() <= TOL and np.abs(lse[:, t] - ld[:, 0]).max() <= TOL


def test_paged_equals_contiguous():
    """Page translation: the pool read through a shuffled table equals the logical
    cache it describes, byte for byte, and the oracle gives identical outputs for the
    paged and the contiguous layout.  Unused pages hold NaN and stay out of the result."""
    case = synth.Case(2, 4, 2, 8, 4, 45, priv_len=2, page_size=8, n_phys_pages=12, dtype="bf16")
    x = synth.make_inputs(case, 14, b_sigma=0.3)
    kb = oracle.gather_base(case, x["k_base"], x["block_table"])
    assert kb.shape == (2, 45, 8) and kb.dtype == np.uint16
    # byte check of the gather against an explicit loop
    for j in range(case.prefix_len):
        p, s = x["block_table"][j // 8], j % 8
        assert np.array_equal(kb[:, j], x["k_base"][p, :, s])
    contig = case.replace(page_size=0, n_phys_pages=0)
    y = dict(x)
    y["k_base"], y["v_base"] = kb, oracle.gather_base(case, x["v_base"], x["block_table"])
    y["block_table"] = None
    o_p, l_p = oracle.attend(case, x)
    o_c, l_c = oracle.attend(contig, y)
    assert np.all(np.isfinite(o_p))
    assert np.array_equal(o_p, o_c) and np.array_equal(l_p, l_c)


def test_softmax_large_scores():
    """Large scores (q scaled by 40) must not overflow: compare with brute force."""
    case = synth.Case(1, 2, 1, 4, 2, 5, priv_len=1, dtype="f32")
    x = synth.make_inputs(case, 15, q_scale=40.0, b_sigma=0.5)
    ob, lb = brute.to_float(*brute.attend(case, x))
    oc, lc = oracle.attend(case, x)
    assert np.all(np.isfinite(oc))
    assert np.abs(ob - oc).max() <= 1e-12 * max(1.0, np.abs(ob).max())
    assert np.abs(lb - lc).max() <= 1e-12 * max(1.0, np.abs(lb).max())


def test_row_mask_selects_rows():
    case = synth.Case(2, 4, 2, 8, 4, 16, dtype="f32")
    x = synth.make_inputs(case, 16)
    o, _ = oracle.attend(case, x)
    m = np.zeros((2, 1, 4), bool)
    m[1, 0, 2] = True
    om, _ = oracle.attend(case, x, row_mask=m)
    assert np.array_equal(om[1, 0, 2], o[1, 0, 2])
    assert np.isnan(om[0]).all() and np.isnan(om[1, 0, 0]).all()


def test_negative_controls_fail_parity():
    """At a full-width decode shape (d=128, H_q=32, H_kv=8, r=16, 4 agents, 4k prefix),
    an 'implementation' that drops a residual term must fail the parity bars while the
    oracle itself passes them: the bars have teeth."""
    from tests import parity

    case = synth.Case(4, 32, 8, 128, 16, 4096, dtype="bf16")
    x = synth.make_inputs(case, 1)
    ref, _ = oracle.attend(case, x)
    b0, _ = oracle.attend(case, dict(x, bk=np.zeros_like(x["bk"]), bv=np.zeros_like(x["bv"])))
    assert not parity.failures(parity.stats(ref, ref, b0), "bf16")
    for drop in ("bk", "bv"):
        bad, _ = oracle.attend(case, dict(x, **{drop: np.zeros_like(x[drop])}))
        f = parity.failures(parity.stats(bad, ref, b0), "bf16")
        assert f, f"dropping {drop} passed the parity bars"


# ---------------------------------------------------------------- mutants ---

def _battery(lib_path):
    """A compact run of the pins above against a given oracle build; returns the
    number of pins that fail."""
    fails = 0

    def run(case, x, **kw):
        return oracle.attend(case, x, lib_path=lib_path, **kw)

    # brute force, incl. paged, causal, lse
    for case in TINY:
        x = synth.make_inputs(case, 7, b_sigma=0.7, q_scale=2.0)
        ob, lb = brute.to_float(*brute.attend(case, x))
        oc, lc = run(case, x)
        fails += int(not (np.abs(ob - oc).max() <= 1e-12 and np.abs(lb - lc).max() <= 1e-12))
    return fails


MUTANTS = {1: "score residual dropped", 2: "value residual dropped", 3: "residual sign",
           4: "GQA head mapping", 5: "B column layout", 6: "scale 1/d", 7: "causal off by one",
           8: "page table ignored", 9: "lse max term"}


@pytest.mark.parametrize("mutant", sorted(MUTANTS), ids=lambda m: MUTANTS[m])
def test_pins_catch_mutant(mutant, tmp_path):
    path = oracle.build(mutant=mutant, out=str(tmp_path / f"mut{mutant}.so"))
    assert oracle.load(path).rattn_oracle_version() == 1000 + mutant
    assert _battery(path) > 0, f"mutant {MUTANTS[mutant]} survived the pins"


def test_unmutated_oracle_passes_battery():
    assert _battery(None) == 0
