"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Inputs come from ``synth`` (seeded); expected values only from ``oracle``.
Bars (tests/parity.py): max-abs 2e-2, mean-abs 2e-3, relative RMS 1e-2 (bf16) or
1e-4 (fp32), and for the full workloads an error below 5 % of what the residual
terms contribute.  Indexing results (page gather, shuffled vs identity table) are
compared bit for bit.
"""
import sys

import numpy as np
import pytest

import oracle
import synth
from tests import kernel_paths as KP
from tests import parity

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def rattn():
    import shared_base_residual_amd as R

    R.lib()  # raises if the HIP library is missing
    return R


def run_gpu(case, x, lse=True):
    R = rattn()
    t = synth.to_torch(x, DEV)
    lse_t = torch.empty(t["q"].shape[:3], device=DEV, dtype=torch.float32) if lse else None
    # the output starts as NaN, so a row the kernel never writes cannot pass
    out = torch.full(tuple(t["q"].shape), float("nan"), device=DEV, dtype=torch.float32)
    R.attend(t, mode=case.mode, shared_lr=case.shared_lr, prefix_len=case.prefix_len, lse=lse_t, out=out)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), (lse_t.cpu().numpy().astype(np.float64) if lse else None)


def ref(case, x, row_mask=None, what=""):
    """The oracle's output; large workloads are computed a few agents at a time
    (row masks), with a progress line after each group."""
    rows = case.n_agents * case.q_len * case.n_q_heads
    keys = case.prefix_len + case.priv_len
    if row_mask is not None or rows * keys < 2 ** 28:
        return oracle.attend(case, x, row_mask=row_mask)
    out = np.full((case.n_agents, case.q_len, case.n_q_heads, case.head_dim), np.nan)
    lse = np.full((case.n_agents, case.q_len, case.n_q_heads), np.nan)
    step = max(1, case.n_agents // 4)
    for a0 in range(0, case.n_agents, step):
        m = np.zeros(lse.shape, bool)
        m[a0:a0 + step] = True
        o, l = oracle.attend(case, x, row_mask=m)
        out[a0:a0 + step] = o[a0:a0 + step]
        lse[a0:a0 + step] = l[a0:a0 + step]
        say(f"[gpu] {what}: oracle rows of agents {a0}..{min(a0 + step, case.n_agents) - 1} done")
    return out, lse


def compare(case, x, *, with_b0=False, what="", row_mask=None):
    say(f"[gpu] {what}: {case}")
    got, got_lse = run_gpu(case, x)
    exp, exp_lse = ref(case, x, row_mask=row_mask, what=what)
    b0 = None
    if with_b0:
        b0, _ = ref(case, dict(x, bk=np.zeros_like(x["bk"]), bv=np.zeros_like(x["bv"])), row_mask=row_mask,
                    what=what + " (B = 0)")
    s = parity.check(got, exp, case.dtype, b0, what)
    m = ~np.isnan(exp_lse)
    assert np.abs(got_lse[m] - exp_lse[m]).max() <= 2e-3 * max(1.0, np.abs(exp_lse[m]).max()), what
    say(f"[gpu] {what}: ok {s}")
    return got, s


# ------------------------------------------------------------- workloads --

@pytest.mark.parametrize("variant", ["base", "stress"])
def test_tiny_decode_fp32(variant):
    c = synth.WORKLOADS[0]
    kw = synth.STRESS if variant == "stress" else {}
    seed = 0 + (synth.STRESS_SEED_OFFSET if variant == "stress" else 0)
    compare(c, synth.make_inputs(c, seed, **kw), with_b0=True, what=f"tiny decode fp32 {variant}")


@pytest.mark.parametrize("variant", ["base", "stress"])
def test_llama8b_decode(variant):
    c = synth.WORKLOADS[1]
    kw = synth.STRESS if variant == "stress" else {}
    seed = 1 + (synth.STRESS_SEED_OFFSET if variant == "stress" else 0)
    compare(c, synth.make_inputs(c, seed, **kw), with_b0=(variant == "base"), what=f"8B decode {variant}")


@pytest.mark.parametrize("variant", ["base", "stress"])
def test_paged_cow_decode(variant):
    c = synth.WORKLOADS[2]
    kw = synth.STRESS if variant == "stress" else {}
    seed = 2 + (synth.STRESS_SEED_OFFSET if variant == "stress" else 0)
    x = synth.make_inputs(c, seed, **kw)
    got, _ = compare(c, x, with_b0=(variant == "base"), what=f"paged decode {variant}")
    assert np.all(np.isfinite(got)), "NaN-poisoned unused pages reached the output"


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("variant", ["base", "stress"])
def test_shared_lr_chunked_prefill_all_rows(variant):
    """The full BaseLRShared prefill (32 agents x 256-token chunks, L = 16384):
    every one of the 262,144 query rows against the oracle."""
    c = synth.WORKLOADS[3]
    kw = synth.STRESS if variant == "stress" else {}
    seed = 3 + (synth.STRESS_SEED_OFFSET if variant == "stress" else 0)
    x = synth.make_inputs(c, seed, **kw)
    compare(c, x, with_b0=(variant == "base"), what=f"BaseLRShared prefill {variant} (all rows)")


FULL_DEPTH_CHECKED = (0, 11, 23, 35, 47, 59, 71, 79)


@pytest.mark.timeout(1200)
def test_full_depth_decode_all_rows_of_eight_layers():
    """All 80 layers run back to back on one stream, as timed.  Every row of
    eight layers (first and last among them) is checked against the oracle,
    per layer and aggregated over the eight layers' elements, lse included."""
    R = rattn()
    c = synth.WORKLOADS[4]
    say(f"[gpu] 70B full-depth decode: generating {c.layers} layers on the device")
    layers = [synth.make_inputs_torch(c, 4, l, DEV) for l in range(c.layers)]
    outs = [torch.empty(layers[0]["q"].shape, device=DEV, dtype=torch.float32) for _ in range(c.layers)]
    lses = [torch.empty(layers[0]["q"].shape[:3], device=DEV, dtype=torch.float32) for _ in range(c.layers)]
    desc = R.describe(layers[0]["q"], layers[0]["k_base"], layers[0]["lk"], layers[0]["bk"])
    ws = torch.zeros(R.workspace_bytes(desc), device=DEV, dtype=torch.uint8)  # zero-filled once
    for l in range(c.layers):
        R.attend(layers[l], out=outs[l], lse=lses[l], workspace=ws)
    torch.cuda.synchronize()
    say("[gpu] 70B full-depth decode: ran all layers")
    gots, exps, b0s = [], [], []
    for l in FULL_DEPTH_CHECKED:
        x = {k: synth.torch_to_numpy(v) for k, v in layers[l].items()}
        exp, exp_lse = oracle.attend(c, x)
        b0, _ = oracle.attend(c, dict(x, bk=np.zeros_like(x["bk"]), bv=np.zeros_like(x["bv"])))
        got = outs[l].cpu().numpy().astype(np.float64)
        got_lse = lses[l].cpu().numpy().astype(np.float64)
        s = parity.check(got, exp, "bf16", b0, f"layer {l}")
        assert np.abs(got_lse - exp_lse).max() <= 2e-3 * max(1.0, np.abs(exp_lse).max()), f"layer {l} lse"
        say(f"[gpu] layer {l}: {s}")
        gots.append(got)
        exps.append(exp)
        b0s.append(b0)
    s = parity.check(np.stack(gots), np.stack(exps), "bf16", np.stack(b0s), "eight layers together")
    say(f"[gpu] layers {FULL_DEPTH_CHECKED} together: {s}")
    del layers


# --------------------------------------------- every kernel instantiation --

@pytest.mark.parametrize("key,case", KP.PATHS, ids=[c.name for _, c in KP.PATHS])
def test_kernel_path(key, case):
    """One workload per kernel instantiation the library can launch (the host
    test in test_kernel_paths.py pins that each reaches its instantiation)."""
    x = synth.make_inputs(case, 77, b_sigma=0.3, q_scale=2.0)
    compare(case, x, what=f"{case.name} {key}")


# ------------------------------------------------------------ edge cases --

EDGE = [
    synth.Case(3, 8, 2, 128, 16, 1000, name="ragged prefix"),
    synth.Case(2, 8, 2, 128, 16, 1, name="single prefix token"),
    synth.Case(2, 8, 2, 128, 16, 0, priv_len=37, name="private only"),
    synth.Case(2, 8, 2, 128, 16, 333, priv_len=45, name="ragged prefix and private"),
    synth.Case(5, 8, 8, 64, 8, 700, priv_len=3, name="d=64 MHA r=8"),
    synth.Case(4, 8, 2, 128, 0, 500, priv_len=20, name="rank 0"),
    synth.Case(3, 8, 2, 128, 128, 300, name="rank 128"),
    synth.Case(6, 16, 2, 128, 32, 777, shared_lr=True, name="shared low-rank decode"),
    synth.Case(2, 64, 2, 128, 16, 400, priv_len=10, name="g=32 (rows beyond one block)"),
    synth.Case(3, 8, 2, 128, 16, 290, q_len=3, priv_len=7, name="multi-token decode"),
    synth.Case(2, 8, 2, 128, 64, 600, priv_len=50, page_size=32, n_phys_pages=40, name="paged 32"),
    synth.Case(9, 8, 2, 128, 16, 2100, page_size=16, n_phys_pages=200, name="paged ragged"),
    synth.Case(2, 8, 2, 64, 16, 500, priv_len=40, q_len=40, mode="prefill", name="prefill per-agent LR"),
    synth.Case(3, 8, 2, 128, 32, 260, priv_len=33, q_len=33, mode="prefill", shared_lr=True,
               name="prefill shared ragged"),
    synth.Case(2, 4, 2, 64, 8, 300, priv_len=20, q_len=20, mode="prefill", dtype="f32", name="prefill fp32"),
    synth.Case(17, 4, 1, 128, 8, 129, name="17 agents g=4"),
    synth.Case(9, 8, 2, 128, 32, 1500, priv_len=17, name="several agents per block, r=32, ragged last block"),
    # prefill: a paged prefix (the page table leaves room for 64-key stages only),
    # padding residual columns (r = 16 in 32-column tiles), and r = 64 (two
    # contraction steps in the Bv epilogue)
    synth.Case(2, 8, 2, 128, 32, 1000, priv_len=40, q_len=40, page_size=16, n_phys_pages=80, mode="prefill",
               name="paged prefill"),
    synth.Case(2, 8, 2, 128, 16, 700, priv_len=50, q_len=50, mode="prefill", name="prefill r=16 ragged"),
    synth.Case(2, 8, 2, 128, 64, 300, priv_len=30, q_len=30, mode="prefill", name="prefill r=64"),
    # more than 64 splits per row: the merge's weight pass across waves
    synth.Case(2, 4, 1, 128, 16, 40000, name="more than 64 splits"),
    synth.Case(4, 32, 8, 128, 16, 500, priv_len=3000, name="private tokens outnumber the prefix"),
    synth.Case(12, 8, 2, 128, 64, 1000, priv_len=700, page_size=16, n_phys_pages=120,
               name="masked paged, long private suffixes"),
    # one row per agent (g = 1, r = 32): the masked ring does not fit, so blocks of
    # two agents with block-diagonal residual columns
    synth.Case(16, 4, 4, 128, 32, 600, priv_len=5, name="g=1 r=32, two agents per block"),
    # masked blocks of more than four agents: eight, then two (g = 2, r = 64, d = 64)
    synth.Case(10, 4, 2, 64, 64, 500, name="masked, 8 + 2 agents per block, d=64"),
]


@pytest.mark.parametrize("case", EDGE, ids=lambda c: c.name)
def test_edge_cases(case):
    x = synth.make_inputs(case, 31, b_sigma=0.3, q_scale=2.0)
    compare(case, x, what=case.name)


def test_run_twice_bitwise():
    c = synth.WORKLOADS[1].replace(prefix_len=8192)
    x = synth.make_inputs(c, 5)
    a, la = run_gpu(c, x)
    b, lb = run_gpu(c, x)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


# -------------------------------------------------------------- indexing --

def test_gather_base_bit_exact():
    R = rattn()
    c = synth.WORKLOADS[2]
    x = synth.make_inputs(c, 2)
    say("[gpu] gather_base on the paged workload")
    t = synth.to_torch(x, DEV)
    g = R.gather_base(t["k_base"], t["block_table"], c.prefix_len)
    torch.cuda.synchronize()
    got = synth.torch_to_numpy(g)
    exp = oracle.gather_base(c, x["k_base"], x["block_table"])
    assert got.dtype == exp.dtype and np.array_equal(got, exp)
    # ragged prefix, larger page
    c2 = synth.Case(1, 4, 4, 64, 0, 1000, page_size=32, n_phys_pages=50, dtype="f32")
    x2 = synth.make_inputs(c2, 3)
    t2 = synth.to_torch(x2, DEV)
    g2 = R.gather_base(t2["v_base"], t2["block_table"], c2.prefix_len)
    torch.cuda.synchronize()
    assert np.array_equal(g2.cpu().numpy().view(np.uint32),
                          oracle.gather_base(c2, x2["v_base"], x2["block_table"]).view(np.uint32))


def test_check_block_table():
    """The debug check counts exactly the entries outside [0, n_phys_pages)
    among the first ceil(prefix_len / page_size); entries past those are not
    read."""
    R = rattn()
    c = synth.WORKLOADS[2]
    x = synth.make_inputs(c, 2)
    say("[gpu] block-table check")
    tab = x["block_table"].astype(np.int32)
    n = c.n_table
    t = torch.from_numpy(tab.copy()).to(DEV)
    assert R.check_block_table(t, c.prefix_len, c.page_size, c.n_phys_pages) == 0
    bad = tab.copy()
    pos = [0, 7, n // 2, n - 1]
    bad[pos] = [-1, c.n_phys_pages, 2 ** 31 - 1, -(2 ** 31)]
    big = np.concatenate([bad, np.full(100, -5, np.int32)])  # a tail past the prefix's pages
    tb = torch.from_numpy(big).to(DEV)
    assert R.check_block_table(tb, c.prefix_len, c.page_size, c.n_phys_pages) == 4
    assert R.check_block_table(tb, c.prefix_len - c.page_size, c.page_size, c.n_phys_pages) == 3
    assert R.check_block_table(tb, 0, c.page_size, c.n_phys_pages) == 0
    assert R.check_block_table(tb, c.prefix_len, c.page_size, 2 ** 31 - 1) == 3
    # the count over a long table (many passes of the workgroup's stride)
    rng = np.random.default_rng(5)
    long = rng.integers(-3, 1003, 300001).astype(np.int32)
    tl = torch.from_numpy(long).to(DEV)
    exp = int(((long < 0) | (long >= 1000)).sum())
    assert R.check_block_table(tl, 300001 * 16, 16, 1000) == exp
    assert R.check_block_table(tl, 300001 * 16 - 15, 16, 1000) == exp


def test_shuffled_table_bitwise_equals_identity():
    """Output depends only on logical token order: a shuffled pool with its table and
    the identity pool give bit-identical results; unused NaN pages change nothing."""
    c = synth.WORKLOADS[2].replace(prefix_len=2048, n_phys_pages=300, priv_len=100)
    x = synth.make_inputs(c, 9)
    say("[gpu] shuffled vs identity page table")
    a, la = run_gpu(c, x)
    ident = dict(x)
    n = c.n_table
    for key in ("k_base", "v_base"):
        pool = np.full_like(x[key], synth.BF16_NAN)
        pool[:n] = x[key][x["block_table"]]
        ident[key] = pool
    ident["block_table"] = np.arange(n, dtype=np.int32)
    b, lb = run_gpu(c, ident)
    assert np.all(np.isfinite(a))
    assert np.array_equal(a, b) and np.array_equal(la, lb)
    # duplicate (aliased) table entries are legal and read the same page twice
    alias = dict(x)
    alias["block_table"] = x["block_table"].copy()
    alias["block_table"][1] = alias["block_table"][0]
    got, _ = run_gpu(c, alias)
    exp, _ = oracle.attend(c, alias)
    parity.check(got, exp, "bf16", what="aliased pages")


def test_workspace_reused_across_shapes():
    """One workspace, never cleared, serves calls of different shapes in turn (its
    contents on entry do not matter), and the stages run separately equal the call."""
    R = rattn()
    cases = [synth.Case(4, 32, 8, 128, 16, 3000, priv_len=40, name="A"),
             synth.Case(7, 8, 2, 64, 8, 900, name="B"),
             synth.Case(4, 32, 8, 128, 16, 3000, priv_len=40, name="A again")]
    xs = [synth.make_inputs(c, 40 + i, b_sigma=0.3) for i, c in enumerate(cases)]
    nbytes = max(R.workspace_bytes(R.describe(*[synth.to_torch(x, DEV)[n] for n in ("q", "k_base", "lk", "bk")],
                                              k_priv=synth.to_torch(x, DEV)["k_priv"])) for x in xs)
    ws = torch.full((nbytes,), 0x7F, device=DEV, dtype=torch.uint8)  # garbage, never cleared
    for c, x in zip(cases, xs):
        say(f"[gpu] shared workspace: {c.name}")
        t = synth.to_torch(x, DEV)
        got = R.attend(t, workspace=ws)
        torch.cuda.synchronize()
        exp, _ = oracle.attend(c, x)
        parity.check(got.cpu().numpy().astype(np.float64), exp, "bf16", what=c.name)
        o2 = torch.full_like(got, float("nan"))
        R.attend(t, workspace=ws, out=o2, stages=R.STAGE_SPLIT)
        R.attend(t, workspace=ws, out=o2, stages=R.STAGE_COMBINE)
        torch.cuda.synchronize()
        assert torch.equal(got, o2), "split then combine differs from the full call"
