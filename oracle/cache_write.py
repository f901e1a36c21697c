"""fp64 reference ("oracle") for the cache-write path upstream of fused residual
attention: the rank-r projection that fills the low-rank caches, and the
append of new base key/value rows into a paged pool with copy-on-write pages.

TEST INFRASTRUCTURE, not part of the product: only ``tests/`` (and the smoke
check and bench baselines) import it.  It shares no code with the HIP library.

  * ``lr_project`` -- the low-rank cache rows of new tokens, L = X A, written
    out as the plain matrix product in fp64 (ForkKV Guide, "Mathematical
    Decomposition of LoRA KV Activations": the residual cache may hold the
    factored intermediate X A of rank r; "DualRadixTree", Case B: on a base hit
    with an adapter miss only the low-rank projection is computed; LRAgent,
    "Schemi di Condivisione": the LR cache stores X_i A_i after the LoRA
    down-projection, and with a shared A (BaseLRShared) one LR cache serves
    every agent).  A is given transposed, [r, d_in] (one row per rank
    component), as a linear layer from d_in to r stores its weight.
  * ``logical_kv`` -- the logical key (or value) rows a block table names in a
    paged pool (the bCache block pointers of the base lookup).
  * ``append_expected`` -- the logical rows after appending new tokens: the old
    rows followed by the new ones (nothing else may change).
  * ``check_append_plan`` -- whether a page-level plan of an append obeys
    copy-on-write (ForkKV Guide, "The Copy-on-Write Paradigm": shared pages
    are read-only; the first write to a shared page goes to a freshly
    allocated private copy, and only that writer's table points at it; pages
    the writer owns alone are written in place; new pages come from the free
    pool).  Page numbers are the allocator's choice, so the checker accepts
    any plan that obeys the rules instead of predicting one.
"""
from __future__ import annotations

from typing import List, Optional, Tuple

import numpy as np


def _f64(a: np.ndarray) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.uint16:  # bf16 bit patterns
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def lr_project(x: np.ndarray, a_t: np.ndarray) -> np.ndarray:
    """Low-rank cache rows of T new tokens for each output set n:
    out[n, t, c] = sum_k X[n_x, t, k] * A^T[n_a, c, k], with n_x = 0 when X is
    shared ([1, T, d_in]) else n, and n_a = 0 when A is shared ([1, r, d_in])
    else n.  There are max(#X sets, #A sets) output sets.  fp64, exact inputs."""
    xf, af = _f64(x), _f64(a_t)
    nx, na = xf.shape[0], af.shape[0]
    n_out = max(nx, na)
    if nx not in (1, n_out) or na not in (1, n_out):
        raise ValueError("X and A sets must be 1 or the same count")
    out = np.empty((n_out, xf.shape[1], af.shape[1]))
    for n in range(n_out):
        out[n] = xf[0 if nx == 1 else n] @ af[0 if na == 1 else n].T
    return out


def logical_kv(pool: np.ndarray, table, length: int) -> np.ndarray:
    """Logical rows [H_kv, length, d] of a paged pool [n_phys, H_kv, page, d]:
    logical token j is slot j % page of physical page table[j // page].  Pure
    indexing (bytes equal the pool's)."""
    ps = pool.shape[2]
    j = np.arange(length)
    phys = np.asarray(table, dtype=np.int64)[j // ps]
    return np.ascontiguousarray(np.transpose(pool[phys, :, j % ps, :], (1, 0, 2)))


def append_expected(old_logical: np.ndarray, new_rows: np.ndarray) -> np.ndarray:
    """Logical rows after an append: the old rows [H_kv, L, d], then the new
    ones [H_kv, T, d]."""
    return np.concatenate([old_logical, new_rows], axis=1)


def check_append_plan(old_table, new_table, cur_len: int, n_new: int, page_size: int, ref_before, ref_after,
                      cow: Optional[Tuple[int, int]]) -> List[str]:
    """Violations of copy-on-write by one append of n_new tokens to a sequence
    of cur_len tokens (empty list: the plan is valid).

    old_table / new_table: the sequence's physical pages before and after;
    ref_before / ref_after: every page's reference count before and after (0 =
    free); cow: (source page, private copy) when the plan copies a page, else
    None."""
    bad = []
    ps = page_size
    old_pages = -(-cur_len // ps)
    new_pages = -(-(cur_len + n_new) // ps)
    ref_before = np.asarray(ref_before)
    ref_after = np.asarray(ref_after)
    touched = set()
    if n_new == 0:
        if list(new_table[:old_pages]) != list(old_table[:old_pages]) or cow is not None:
            bad.append("an empty append changed the table or copied a page")
        if not np.array_equal(ref_before, ref_after):
            bad.append("an empty append changed reference counts")
        return bad
    partial = cur_len % ps != 0
    for lp in range(old_pages - (1 if partial else 0)):
        if new_table[lp] != old_table[lp]:
            bad.append(f"full page {lp} was remapped")
    expect_dec = {}
    if partial:
        lp = old_pages - 1
        src = int(old_table[lp])
        if ref_before[src] > 1:
            dst = int(new_table[lp])
            if cow is None or tuple(int(v) for v in cow) != (src, dst):
                bad.append(f"shared page {src} written without a copy (cow {cow}, new page {dst})")
            if dst == src:
                bad.append(f"shared page {src} written in place")
            elif ref_before[dst] != 0:
                bad.append(f"copy target {dst} was in use")
            expect_dec[src] = 1
            touched.add(dst)
        else:
            if new_table[lp] != src:
                bad.append(f"page {src}, owned alone, was remapped instead of written in place")
            if cow is not None:
                bad.append(f"a copy of page {src}, owned alone, was made")
    elif cow is not None:
        bad.append("a page was copied although no partial page is written")
    fresh = [int(p) for p in new_table[old_pages:new_pages]]
    if len(set(fresh)) != len(fresh):
        bad.append("a new page was given twice")
    for p in fresh:
        if ref_before[p] != 0:
            bad.append(f"new page {p} was in use")
        touched.add(p)
    if len(touched & set(int(p) for p in old_table[:old_pages])) and not bad:
        bad.append("a new page aliases one of the sequence's pages")
    for p in range(len(ref_before)):
        want = ref_before[p] - expect_dec.get(p, 0) + (1 if p in touched else 0)
        if ref_after[p] != want:
            bad.append(f"page {p}: reference count {ref_after[p]}, expected {want}")
    return bad
