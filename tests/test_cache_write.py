"""The cache-write path: the low-rank projection (rattn_lr_project), the host
page allocator with copy-on-write (rattn_pagepool_*) and the paged append
(rattn_append_kv).

Host tests (no GPU): the allocator's plans against the oracle's
copy-on-write rules (oracle/cache_write.py) over random forks, appends and
releases, and argument validation.  GPU tests: rattn_lr_project against the
fp64 X A of the oracle, rattn_append_kv bit for bit against the oracle's
logical rows (old rows then the new ones), with the other sequences that
share pages unchanged."""
import ctypes
import os
import sys

import numpy as np
import pytest

import synth
from oracle import cache_write as CW

import shared_base_residual_amd as R

pytestmark = pytest.mark.skipif(not os.path.exists(R.LIB_PATH), reason="librattn not built")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------- allocator --

class Seqs:
    """Sequences over one PagePool, driven by random forks, appends and releases;
    every append's plan is checked against the oracle's rules."""

    def __init__(self, pool, ps):
        self.pool, self.ps = pool, ps
        self.seqs = {}  # id -> (table list, length)

    def new(self, sid, length):
        n = -(-length // self.ps)
        self.seqs[sid] = (list(self.pool.alloc(n)), length)

    def fork(self, sid, src):
        table, length = self.seqs[src]
        self.pool.retain(table)
        self.seqs[sid] = (list(table), length)

    def append(self, sid, n_new):
        table, length = self.seqs[sid]
        cap = -(-(length + n_new) // self.ps)
        t = np.full(cap, -1, np.int32)
        t[:len(table)] = table
        rb = self.pool.refcounts()
        free_b = self.pool.free_pages()
        cow = self.pool.plan_append(t, length, n_new, self.ps)
        ra = self.pool.refcounts()
        bad = CW.check_append_plan(table, list(t), length, n_new, self.ps, rb, ra,
                                   None if cow[0] < 0 else cow)
        assert not bad, bad
        used = (-(-(length + n_new) // self.ps) - -(-length // self.ps)) + (1 if cow[0] >= 0 else 0)
        assert self.pool.free_pages() == free_b - used
        self.seqs[sid] = (list(t), length + n_new)
        return cow

    def release(self, sid):
        table, _ = self.seqs.pop(sid)
        self.pool.release(table)


def test_allocator_random_forks_and_appends():
    rng = np.random.default_rng(5)
    ps = 16
    pool = R.PagePool(4096)
    s = Seqs(pool, ps)
    s.new(0, 1000)
    n_cow = 0
    for step in range(400):
        op = rng.integers(0, 10)
        ids = list(s.seqs)
        if op < 2 and len(ids) < 40:
            s.fork(max(ids) + 1, int(rng.choice(ids)))
        elif op < 3 and len(ids) > 1:
            s.release(int(rng.choice(ids)))
        else:
            cow = s.append(int(rng.choice(ids)), int(rng.integers(0, 40)))
            n_cow += cow[0] >= 0
        # conservation: every page is free or held by its sequences' count
        held = np.zeros(pool.n_pages, np.int64)
        for table, length in s.seqs.values():
            for p in table[:-(-length // ps)]:
                held[p] += 1
        assert np.array_equal(held, pool.refcounts())
        assert pool.free_pages() == int((held == 0).sum())
    assert n_cow > 10  # the walk exercised copy-on-write


def test_allocator_errors_change_nothing():
    pool = R.PagePool(10)
    a = pool.alloc(3)
    with pytest.raises(R.RattnError) as e:
        pool.alloc(8)
    assert e.value.status == -8 and pool.free_pages() == 7
    pool.retain(a)  # every page of a now shared twice
    t = np.array(list(a) + [-1] * 12, np.int32)
    before = t.copy()
    with pytest.raises(R.RattnError) as e:  # 40 -> 200 tokens needs 1 copy + 10 pages; 7 free
        pool.plan_append(t, 40, 160, 16)
    assert e.value.status == -8 and np.array_equal(t, before) and pool.free_pages() == 7
    with pytest.raises(R.RattnError) as e:  # table too short for the new length
        pool.plan_append(t[:3], 40, 20, 16)
    assert e.value.status == -2
    with pytest.raises(R.RattnError) as e:  # releases beyond what is held
        pool.release([a[0]] * 3)
    assert e.value.status == -2 and pool.refcount(int(a[0])) == 2
    with pytest.raises(R.RattnError):
        pool.retain([9])  # free page
    bad = np.array([3, 99], np.int32)
    with pytest.raises(R.RattnError):
        pool.plan_append(np.concatenate([bad, [-1]]).astype(np.int32), 20, 5, 16)


def test_cache_write_validation():
    lib = R.lib()
    F = 0x10000  # never dereferenced: every call below fails validation first
    d = R.LrDesc(4, 1, 0, 4096, 16, 100, 0, 100, R.RATTN_BF16)
    ok = lambda **kw: lib.rattn_lr_project(ctypes.byref(R.LrDesc(*[kw.get(n, getattr(d, n)) for n, _ in
                                                                   R.LrDesc._fields_])), F, F, F, F, F, None)
    assert ok(d_in=4000) == -3
    assert ok(rank=12) == -3
    assert ok(dtype=R.RATTN_F32) == -3
    assert ok(pos0=10) == -2  # pos0 + T > cache_len
    assert ok(shared_a=1) == -2  # shared X and shared A need one set
    assert ok(n_sets=0) == -2
    assert lib.rattn_lr_project(ctypes.byref(d), None, F, F, F, F, None) == -1
    assert lib.rattn_lr_project(ctypes.byref(d), F + 8, F, F, F, F, None) == -5
    dd = R.make_desc(n_agents=1, n_q_heads=8, n_kv_heads=8, head_dim=128, rank=0, q_len=1, prefix_len=0,
                     page_size=16, n_phys_pages=64)
    ap = lambda *a: lib.rattn_append_kv(ctypes.byref(dd), *a)
    assert ap(F, F, F, 40, 10, F, F, 3, -1, None) == -2   # half a copy-on-write pair
    assert ap(F, F, F, 40, 10, F, F, 3, 3, None) == -2    # copy onto itself
    assert ap(F, F, F, 40, 10, F, F, 3, 64, None) == -2   # page outside the pool
    assert ap(F, F, F, 48, 10, F, F, 3, 5, None) == -2    # page-aligned length: nothing to copy
    assert ap(F, F, None, 40, 10, F, F, -1, -1, None) == -1
    dd.page_size = 8
    assert ap(F, F, F, 40, 10, F, F, -1, -1, None) == -3


# -------------------------------------------------------------- GPU: X A --

LR_CASES = [
    # (n_sets, shared_x, shared_a, d_in, r, T, pos0, cache_len)
    (4, True, False, 4096, 16, 300, 5, 400),     # LR prefill of a shared context, per-agent A
    (1, True, True, 512, 32, 1000, 0, 1000),     # BaseLRShared: one cache
    (3, False, False, 256, 8, 77, 10, 100),      # per-agent inputs, r = 8
    (2, False, True, 384, 64, 129, 0, 200),      # per-agent inputs, shared A, r = 64
    (5, True, False, 128, 128, 33, 1, 40),       # r = 128: several column blocks per X
    (2, True, False, 1024, 16, 1, 17, 18),       # one new token (a decode step)
]


@pytest.mark.gpu
@pytest.mark.parametrize("case", LR_CASES, ids=lambda c: f"n{c[0]} sx{int(c[1])} sa{int(c[2])} din{c[3]} r{c[4]} T{c[5]}")
def test_lr_project_parity(case):
    torch = pytest.importorskip("torch")
    n_sets, sx, sa, d_in, r, T, pos0, cap = case
    rng = np.random.default_rng(11)
    x = synth.bf16_bits(rng.standard_normal((1 if sx else n_sets, T, d_in)))
    ak = synth.bf16_bits(rng.standard_normal((1 if sa else n_sets, r, d_in)) * 0.05)
    av = synth.bf16_bits(rng.standard_normal((1 if sa else n_sets, r, d_in)) * 0.05)
    say(f"[gpu] lr_project {case}")
    t = synth.to_torch(dict(x=x, ak=ak, av=av), "cuda")
    sentinel = -7.0
    lk = torch.full((n_sets, cap, r), sentinel, device="cuda", dtype=torch.bfloat16)
    lv = torch.full_like(lk, sentinel)
    R.lr_project(t["x"], t["ak"], t["av"], lk, lv, pos0=pos0)
    torch.cuda.synchronize()
    for got_t, a in ((lk, ak), (lv, av)):
        got = got_t.float().cpu().numpy().astype(np.float64)
        exp = CW.lr_project(x, a)
        # rows outside [pos0, pos0 + T) untouched
        mask = np.ones(cap, bool)
        mask[pos0:pos0 + T] = False
        assert np.all(got[:, mask] == sentinel)
        g = got[:, pos0:pos0 + T]
        # bound: bf16 rounding of the result (2^-8 relative, allowing the fp32
        # sum's own rounding before it) plus the fp32 accumulation error
        xa = np.abs(CW._f64(x))
        aa = np.abs(CW._f64(a))
        mag = np.stack([xa[0 if sx else n] @ aa[0 if sa else n].T for n in range(n_sets)])
        tol = 2.0 ** -8 * np.abs(exp) + d_in * 2.0 ** -23 * mag + 1e-30
        err = np.abs(g - exp)
        assert np.all(err <= tol), f"max err {err.max()}, worst ratio {(err / tol).max()}"
        assert err.mean() <= 2.0 ** -9 * np.abs(exp).mean()


# ---------------------------------------------------------- GPU: append --

@pytest.mark.gpu
@pytest.mark.parametrize("dtype,D,ps", [("bf16", 128, 16), ("f32", 64, 32), ("bf16", 64, 16)])
def test_append_kv_copy_on_write(dtype, D, ps):
    """Three sequences share a 1000-token prefix (forks); one appends (its
    partial last page is shared: copy-on-write), then appends again (the copy is
    its own now: in place), another fork appends (copy again: the original is
    still shared), then a page-aligned sequence appends a long chunk.
    Every sequence's logical rows must equal the oracle's, bit for bit."""
    torch = pytest.importorskip("torch")
    HK, n_phys = 4, 300
    rng = np.random.default_rng(3)
    store = synth.bf16_bits if dtype == "bf16" else (lambda v: v.astype(np.float32))
    pool_np = {k: store(rng.standard_normal((n_phys, HK, ps, D))) for k in ("k", "v")}
    pool = R.PagePool(n_phys)
    seqs = Seqs(pool, ps)
    seqs.new(0, 1000)
    seqs.fork(1, 0)
    seqs.fork(2, 0)
    # the pool on the device holds the bytes the oracle keeps on the host
    dev = {k: synth.to_torch({"a": v}, "cuda")["a"] for k, v in pool_np.items()}

    def logical(pool_arr, sid):
        table, length = seqs.seqs[sid]
        return CW.logical_kv(pool_arr, table, length)

    expected = {sid: {k: logical(pool_np[k], sid) for k in ("k", "v")} for sid in seqs.seqs}
    steps = [(1, 37), (1, 5), (2, 24 + ps * 3)]
    seqs.new(3, 4 * ps)  # page-aligned, then a long chunk
    expected[3] = {k: logical(pool_np[k], 3) for k in ("k", "v")}
    steps.append((3, 700))
    n_cow = 0
    for sid, n_new in steps:
        cur = seqs.seqs[sid][1]
        new = {k: store(rng.standard_normal((HK, n_new, D))) for k in ("k", "v")}
        cow = seqs.append(sid, n_new)
        n_cow += cow[0] >= 0
        table_dev = torch.from_numpy(np.asarray(seqs.seqs[sid][0], np.int32)).cuda()
        nt = synth.to_torch(new, "cuda")
        say(f"[gpu] append seq {sid}: {cur} + {n_new} tokens, cow {cow}")
        R.append_kv(dev["k"], dev["v"], table_dev, cur, nt["k"], nt["v"], cow=cow)
        torch.cuda.synchronize()
        for k in ("k", "v"):
            expected[sid][k] = CW.append_expected(expected[sid][k], new[k])
        got_pool = {k: synth.torch_to_numpy(dev[k]) for k in ("k", "v")}
        for s2 in seqs.seqs:
            for k in ("k", "v"):
                got = logical(got_pool[k], s2)
                assert got.dtype == expected[s2][k].dtype
                assert np.array_equal(got.view(np.uint8), expected[s2][k].view(np.uint8)), (sid, s2, k)
    # copies: sequence 1's first append (page shared by 0, 1, 2) and sequence
    # 2's (still shared by 0 and 2); sequence 1's second append writes its own
    # copy in place, and sequence 3's length is page-aligned
    assert n_cow == 2
