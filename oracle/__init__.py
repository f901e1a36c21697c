"""fp64 reference ("oracle") for fused residual attention over a shared base KV cache.

TEST INFRASTRUCTURE, not part of the product.  Only ``tests/``, the smoke check
in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` import this
package.  The product library (``shared_base_residual_amd``) never imports, links
or calls it, and the two share no code; both only read the arrays drawn by
``synth``.

Contents
  * ``attend``      -- the plain definition in C (``rattn_oracle.c``): gather the
                       base pages, materialise each agent's keys and values,
                       textbook softmax attention, all in fp64;
  * ``gather_base`` -- logical base cache from a paged pool and its table
                       (numpy indexing, byte-exact);
  * ``brute``       -- the same definition in 40-digit decimal arithmetic, for
                       tiny shapes (pins the C code);
  * ``cache_write`` -- the cache-write path upstream of attention: the rank-r
                       projection L = X A that fills the low-rank caches, the
                       logical rows of a paged pool, and the copy-on-write
                       rules an append of new base rows must obey.
  * ``recon``       -- attention with the residual keys rebuilt per token and
                       rotated by position before the score (the pages' own
                       in-register kernel design; needed once keys are rotated
                       after the up-projection);
  * ``quant``       -- base keys as int8 codes with one scale per tensor
                       (the quantiser, the dequantised keys, and fp64 inputs
                       for ``attend`` with the keys dequantised);
  * ``values3``     -- base values as 3-bit codes after a Walsh-Hadamard
                       rotation (the 8-level Lloyd-Max quantiser of N(0, 1)
                       from its optimality conditions, the transform, the
                       codes and scales, the decoded values, and fp64 inputs
                       for ``attend`` with int8 keys and decoded values).

Every function here is pinned (``tests/test_oracle_pins.py`` and the
``tests/test_*_oracle.py`` files) against facts the pages and the mathematics fix (brute force, closed forms, invariants, library
attention for the special cases that reduce to it).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "rattn_oracle.c")
LIB = os.path.join(HERE, "librattn_oracle.so")

EL_F64, EL_F32, EL_BF16 = 0, 1, 2


class _Shape(ctypes.Structure):
    _fields_ = [
        ("n_agents", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("rank", ctypes.c_int32),
        ("prefix_len", ctypes.c_int64), ("priv_len", ctypes.c_int64),
        ("q_len", ctypes.c_int32), ("page_size", ctypes.c_int32),
        ("n_phys_pages", ctypes.c_int64),
        ("shared_lr", ctypes.c_int32), ("causal", ctypes.c_int32), ("elem", ctypes.c_int32),
        ("sm_scale", ctypes.c_double),
    ]


class _Inputs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("q", "k_base", "v_base", "block_table", "lk", "lv", "bk", "bv", "k_priv", "v_priv")]


def build(mutant: int = 0, out: Optional[str] = None) -> str:
    """Compile the C oracle (gcc, -O2, OpenMP).  ``mutant`` > 0 plants one of the
    deliberate mistakes the pin tests must catch."""
    out = out or LIB
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           f"-DORACLE_MUTANT={int(mutant)}", SRC, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


_libs = {}


def load(path: Optional[str] = None):
    path = path or LIB
    if path in _libs:
        return _libs[path]
    if not os.path.exists(path):
        if path != LIB:
            raise FileNotFoundError(path)
        build()
    lib = ctypes.CDLL(path)
    lib.rattn_oracle_attend.restype = ctypes.c_int
    lib.rattn_oracle_attend.argtypes = [ctypes.POINTER(_Shape), ctypes.POINTER(_Inputs), ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
    lib.rattn_oracle_version.restype = ctypes.c_int
    _libs[path] = lib
    return lib


def _elem(arr: np.ndarray) -> int:
    if arr.dtype == np.float64:
        return EL_F64
    if arr.dtype == np.float32:
        return EL_F32
    if arr.dtype == np.uint16:
        return EL_BF16
    raise TypeError(f"unsupported element type {arr.dtype}")


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def attend(case, inputs, *, row_mask: Optional[np.ndarray] = None, n_threads: Optional[int] = None,
           sm_scale: float = 0.0, lib_path: Optional[str] = None):
    """Reference output for one layer.

    ``case`` is a ``synth.Case``; ``inputs`` holds the arrays in ``synth``'s
    storage convention (all of one element type).  ``row_mask`` (bool,
    [N, q_len, H_q]) selects rows; unselected rows come back as NaN.
    Returns ``(out, lse)``: fp64 [N, q_len, H_q, d] and [N, q_len, H_q].
    """
    lib = load(lib_path)
    c = case
    keep = []

    def ptr(name):
        a = inputs.get(name)
        if a is None:
            return None
        a = np.ascontiguousarray(a)
        keep.append(a)
        return a.ctypes.data

    el = _elem(np.asarray(inputs["q"]))
    for name in ("k_base", "v_base", "lk", "lv", "bk", "bv", "k_priv", "v_priv"):
        a = inputs.get(name)
        if a is not None and _elem(np.asarray(a)) != el:
            raise TypeError(f"{name}: element type differs from q")
    tab = inputs.get("block_table")
    if tab is not None:
        tab = np.ascontiguousarray(tab, dtype=np.int32)
        keep.append(tab)
    shp = _Shape(c.n_agents, c.n_q_heads, c.n_kv_heads, c.head_dim, c.rank, c.prefix_len, c.priv_len,
                 c.q_len, c.page_size, c.n_phys_pages, int(c.shared_lr), int(c.mode == "prefill"), el,
                 float(sm_scale))
    ins = _Inputs(ptr("q"), ptr("k_base"), ptr("v_base"), None if tab is None else tab.ctypes.data,
                  ptr("lk"), ptr("lv"), ptr("bk"), ptr("bv"), ptr("k_priv"), ptr("v_priv"))
    out = np.full((c.n_agents, c.q_len, c.n_q_heads, c.head_dim), np.nan)
    lse = np.full((c.n_agents, c.q_len, c.n_q_heads), np.nan)
    mask_ptr = None
    if row_mask is not None:
        m = np.ascontiguousarray(row_mask, dtype=np.uint8).reshape(c.n_agents, c.q_len, c.n_q_heads)
        keep.append(m)
        mask_ptr = m.ctypes.data
    rc = lib.rattn_oracle_attend(ctypes.byref(shp), ctypes.byref(ins), mask_ptr, out.ctypes.data,
                                 lse.ctypes.data, int(n_threads or default_threads()))
    if rc != 0:
        raise ValueError(f"oracle rejected the case (status {rc})")
    return out, lse


def gather_base(case, pool: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Logical base cache [H_kv, L, d] from a paged pool [n_phys, H_kv, page, d]:
    logical token j is slot j % page of physical page table[j // page] (the page
    table plays the role of the bCache block pointers returned by the base lookup
    in the ForkKV Guide's DualRadixTree section).  Pure indexing: the result's
    bytes equal the pool's."""
    c = case
    j = np.arange(c.prefix_len)
    phys = np.asarray(table, dtype=np.int64)[j // c.page_size]
    g = pool[phys, :, j % c.page_size, :]        # [L, H_kv, d]
    return np.ascontiguousarray(np.transpose(g, (1, 0, 2)))
