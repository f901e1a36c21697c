"""Pins of the cache-write oracle (oracle/cache_write.py) against facts that do
not come from it: decimal brute force, closed forms, and hand-built plans that
do or do not obey copy-on-write (ForkKV Guide, "The Copy-on-Write Paradigm")."""
import numpy as np
import pytest

import synth
from oracle import brute
from oracle import cache_write as CW


def _draw(shape, seed, dtype="bf16", scale=1.0):
    rng = np.random.default_rng(seed)
    v = rng.standard_normal(shape) * scale
    return synth.bf16_bits(v) if dtype == "bf16" else v.astype(np.float32)


@pytest.mark.parametrize("nx,na,dtype", [(1, 1, "bf16"), (1, 3, "bf16"), (3, 3, "f32"), (2, 1, "f32")])
def test_lr_project_brute_force(nx, na, dtype):
    """X A against 40-digit decimal arithmetic on tiny shapes."""
    x = _draw((nx, 5, 7), 1, dtype)
    a = _draw((na, 3, 7), 2, dtype, 0.3)
    got = CW.lr_project(x, a)
    exp = np.array([[[float(v) for v in row] for row in t] for t in brute.lr_project(x, a)])
    assert got.shape == exp.shape == (max(nx, na), 5, 3)
    assert np.abs(got - exp).max() <= 1e-14 * max(1.0, np.abs(exp).max())


def test_lr_project_unit_columns_select_inputs():
    """Closed form: rows of A^T that are unit vectors e_k copy column k of X."""
    x = _draw((2, 6, 8), 3, "f32")
    a = np.zeros((2, 3, 8), np.float32)
    cols = [(5, 0, 7), (2, 2, 1)]
    for n in range(2):
        for c, k in enumerate(cols[n]):
            a[n, c, k] = 1.0
    got = CW.lr_project(x, a)
    for n in range(2):
        assert np.array_equal(got[n], x[n][:, list(cols[n])].astype(np.float64))


def test_lr_project_shared_a_equals_copies():
    """BaseLRShared: one A for all agents equals each agent holding a copy."""
    x = _draw((4, 5, 16), 4)
    a = _draw((1, 4, 16), 5, scale=0.2)
    shared = CW.lr_project(x, a)
    copies = CW.lr_project(x, np.repeat(a, 4, axis=0))
    assert np.array_equal(shared, copies)


def test_logical_kv_follows_the_table():
    pool = np.arange(5 * 2 * 4 * 3, dtype=np.int32).reshape(5, 2, 4, 3)
    table = [3, 0, 4]
    got = CW.logical_kv(pool, table, 10)
    for j in range(10):
        assert np.array_equal(got[:, j], pool[table[j // 4], :, j % 4])


def _refs(n, pairs):
    r = np.zeros(n, np.int64)
    for p, c in pairs:
        r[p] = c
    return r


def test_plan_checker_accepts_valid_plans():
    # a sequence of 10 tokens in 4-token pages [2, 5, 7]; page 7 (the partial
    # one) is shared with another sequence: the append copies it to page 1
    old = [2, 5, 7]
    rb = _refs(9, [(2, 2), (5, 2), (7, 2)])
    new = [2, 5, 1, 8]
    ra = _refs(9, [(2, 2), (5, 2), (7, 1), (1, 1), (8, 1)])
    assert CW.check_append_plan(old, new, 10, 5, 4, rb, ra, (7, 1)) == []
    # owned alone: written in place, fresh pages for the rest
    rb2 = _refs(9, [(2, 1), (5, 1), (7, 1)])
    ra2 = _refs(9, [(2, 1), (5, 1), (7, 1), (3, 1)])
    assert CW.check_append_plan(old, [2, 5, 7, 3], 10, 5, 4, rb2, ra2, None) == []
    # page-aligned length: no copy even when every page is shared
    rb3 = _refs(9, [(2, 3), (5, 3)])
    ra3 = _refs(9, [(2, 3), (5, 3), (6, 1)])
    assert CW.check_append_plan([2, 5], [2, 5, 6], 8, 3, 4, rb3, ra3, None) == []


@pytest.mark.parametrize("what", ["in place", "no decrement", "used target", "remap full", "dup fresh",
                                  "copy of owned"])
def test_plan_checker_rejects_broken_plans(what):
    old = [2, 5, 7]
    rb = _refs(9, [(2, 2), (5, 2), (7, 2), (4, 1)])
    new, ra, cow = [2, 5, 1, 8], _refs(9, [(2, 2), (5, 2), (7, 1), (1, 1), (8, 1), (4, 1)]), (7, 1)
    if what == "in place":
        new, ra, cow = [2, 5, 7, 8], _refs(9, [(2, 2), (5, 2), (7, 2), (8, 1), (4, 1)]), None
    elif what == "no decrement":
        ra = _refs(9, [(2, 2), (5, 2), (7, 2), (1, 1), (8, 1), (4, 1)])
    elif what == "used target":
        new, cow = [2, 5, 4, 8], (7, 4)
        ra = _refs(9, [(2, 2), (5, 2), (7, 1), (4, 2), (8, 1)])
    elif what == "remap full":
        new = [2, 6, 1, 8]
        ra = _refs(9, [(2, 2), (5, 2), (7, 1), (1, 1), (8, 1), (6, 1), (4, 1)])
    elif what == "dup fresh":
        new = [2, 5, 1, 8, 8]
        return_bad = CW.check_append_plan(old, new, 10, 9, 4, rb, ra, cow)
        assert return_bad
        return
    elif what == "copy of owned":
        rb = _refs(9, [(2, 1), (5, 1), (7, 1), (4, 1)])
        new, ra, cow = [2, 5, 1, 8], _refs(9, [(2, 1), (5, 1), (7, 0), (1, 1), (8, 1), (4, 1)]), (7, 1)
    assert CW.check_append_plan(old, new, 10, 5, 4, rb, ra, cow), what
