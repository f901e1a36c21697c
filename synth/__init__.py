"""Seeded synthetic inputs for fused residual attention over a shared base KV cache.

This module only draws random numbers and lays them out.  It holds none of the
method's arithmetic: no score, softmax, residual product or page translation is
computed here.  Both the fp64 oracle (``oracle/``) and the HIP library read the
exact arrays produced here, so every comparison is over identical input bits.

Shapes follow the workloads of the pages:
  * ForkKV Guide (aifetchly), "Benchmark Evaluation": 4 agents on a 32k shared
    context with Llama-3-8B / 70B  -> the 8B-shaped and 70B-shaped decode cases;
  * PolyKV (gist.science), section 4: 15 agents on a shared document with
    Llama-3-8B -> the paged copy-on-write decode case (16 agents, 8k prefix);
  * LRAgent (gist.science), "Schemi di Condivisione" / BaseLRShared: shared-A
    LoRA so one low-rank cache serves every agent -> the chunked prefill case.
Values are N(0,1) activations and N(0, 0.05^2) up-projections (a small
perturbation, as LRAgent's "Decomposizione della Cache" describes the adapter
output).  No dataset item is reproduced: the pages' datasets are not used.

Storage conventions
  * bf16 tensors are numpy ``uint16`` arrays of bf16 bit patterns, rounded from
    fp32 with round-to-nearest-even; fp32 tensors are ``float32``.
  * Layouts (row-major):
      q        [N, q_len, H_q, d]
      k_base   [H_kv, L, d]                 (contiguous)  or
               [n_phys, H_kv, page, d]      (paged pool; ``block_table`` int32 [ceil(L/page)])
      lk, lv   [N or 1, L, r]               (1 when the low-rank cache is shared)
      bk, bv   [N, r, H_kv*d]
      k_priv   [N, H_kv, S, d]              (per-agent private tokens)
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

BF16_NAN = np.uint16(0x7FC0)


@dataclasses.dataclass(frozen=True)
class Case:
    """Shape of one call (one layer)."""
    n_agents: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    rank: int
    prefix_len: int
    priv_len: int = 0
    q_len: int = 1
    page_size: int = 0          # 0: contiguous base cache
    n_phys_pages: int = 0
    shared_lr: bool = False
    dtype: str = "bf16"         # "bf16" or "f32"
    mode: str = "decode"        # "decode" or "prefill"
    layers: int = 1
    name: str = ""

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def n_lr(self) -> int:
        return 1 if self.shared_lr else self.n_agents

    @property
    def n_table(self) -> int:
        if self.page_size == 0:
            return 0
        return (self.prefix_len + self.page_size - 1) // self.page_size

    def replace(self, **kw) -> "Case":
        return dataclasses.replace(self, **kw)


# The five workloads (one entry per call shape).
WORKLOADS = {
    0: Case(2, 4, 2, 64, 8, 256, dtype="f32", name="tiny decode"),
    1: Case(4, 32, 8, 128, 16, 32768, name="Llama-3-8B-shaped decode"),
    2: Case(16, 32, 8, 128, 64, 8192, priv_len=512, page_size=16, n_phys_pages=1024,
            name="paged copy-on-write decode"),
    3: Case(32, 32, 8, 128, 32, 16384, priv_len=256, q_len=256, shared_lr=True,
            mode="prefill", name="BaseLRShared chunked prefill"),
    4: Case(8, 64, 8, 128, 16, 65536, layers=80, name="70B-shaped full-depth decode"),
}


# Cache-write workloads (shapes only): the low-rank projection of a shared
# context for four agents (one X, per-agent A), and the append of new base rows
# into a paged pool whose last page is shared (so the first write copies it).
LR_PREFILL = dict(name="BaseShared LR prefill (low-rank cache write)", n_sets=4, d_in=4096, r=16, T=32768)
APPEND = dict(name="paged base append with copy-on-write", HK=8, D=128, ps=16, cur_len=8200, T=4096)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp64/fp32 -> bf16 bit patterns (uint16) via fp32, round to nearest even."""
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    b = x32.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits(x)
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(dtype)


def make_inputs(case: Case, seed: int, *, q_scale: float = 1.0, b_sigma: float = 0.05,
                zero: tuple = (), layer: int = 0) -> Dict[str, Optional[np.ndarray]]:
    """Draw one layer's inputs for ``case`` from ``PCG64(seed)``.

    Draw order: q, K_base, V_base, Lk, Lv, Bk, Bv, K_priv, V_priv, page permutation.
    ``zero`` names inputs to replace by zeros after drawing (the draw order is kept,
    so the remaining inputs are identical to the undamped draw).
    """
    c = case
    rng = np.random.Generator(np.random.PCG64(seed * 1000 + layer))
    n, hq, hkv, d, r = c.n_agents, c.n_q_heads, c.n_kv_heads, c.head_dim, c.rank
    L, S, ql = c.prefix_len, c.priv_len, c.q_len
    if hq % hkv:
        raise ValueError("H_q must be a multiple of H_kv")

    def normal(shape, sigma=1.0):
        return rng.standard_normal(shape) * sigma

    q = normal((n, ql, hq, d)) * q_scale
    if c.page_size:
        ps = c.page_size
        kb = normal((c.n_phys_pages, hkv, ps, d))
        vb = normal((c.n_phys_pages, hkv, ps, d))
    else:
        kb = normal((hkv, L, d))
        vb = normal((hkv, L, d))
    lk = normal((c.n_lr, L, r))
    lv = normal((c.n_lr, L, r))
    bk = normal((n, r, hkv * d), b_sigma)
    bv = normal((n, r, hkv * d), b_sigma)
    kp = normal((n, hkv, S, d)) if S else None
    vp = normal((n, hkv, S, d)) if S else None
    table = None
    if c.page_size:
        perm = rng.permutation(c.n_phys_pages).astype(np.int32)
        table = np.ascontiguousarray(perm[: c.n_table])

    out = dict(q=q, k_base=kb, v_base=vb, lk=lk, lv=lv, bk=bk, bv=bv, k_priv=kp, v_priv=vp)
    for name in zero:
        if out[name] is not None:
            out[name] = np.zeros_like(out[name])
    res = {k: (None if v is None else _store(v, c.dtype)) for k, v in out.items()}
    if table is not None:
        # Pages no table entry points at are poisoned with NaN: a kernel that reads
        # them (or lets them reach the output) is wrong.
        unused = np.setdiff1d(np.arange(c.n_phys_pages), table)
        nanv = BF16_NAN if c.dtype == "bf16" else np.float32(np.nan)
        for key in ("k_base", "v_base"):
            res[key][unused] = nanv
    res["block_table"] = table
    return res


# Stress variant (drawn with seed + 100): larger queries and up-projections, so
# that outputs are O(1) and an absolute error bar bites.
STRESS = dict(q_scale=4.0, b_sigma=0.25)
STRESS_SEED_OFFSET = 100


def to_torch(inputs: Dict[str, Optional[np.ndarray]], device):
    """numpy arrays -> torch tensors on ``device`` (bf16 bit patterns become bfloat16)."""
    import torch

    res = {}
    for k, v in inputs.items():
        if v is None:
            res[k] = None
        elif v.dtype == np.uint16:
            res[k] = torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).to(device)
        elif v.dtype == np.int32:
            res[k] = torch.from_numpy(v).to(device)
        else:
            res[k] = torch.from_numpy(v).to(device)
    return res


def make_inputs_torch(case: Case, seed: int, layer: int, device, *, q_scale: float = 1.0,
                      b_sigma: float = 0.05):
    """One layer's inputs drawn on the device with torch's generator (for the
    full-depth case, whose 21 GB of base cache is too large to draw on the host).
    Contiguous layout only.  Values are drawn in fp32 and rounded to bf16 with
    round-to-nearest-even (torch's conversion)."""
    import torch

    c = case
    if c.page_size:
        raise ValueError("device draw supports the contiguous layout only")
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000 + layer)
    n, hq, hkv, d, r = c.n_agents, c.n_q_heads, c.n_kv_heads, c.head_dim, c.rank
    L, S, ql = c.prefix_len, c.priv_len, c.q_len
    dt = torch.bfloat16 if c.dtype == "bf16" else torch.float32

    def normal(shape, sigma=1.0):
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        if sigma != 1.0:
            x.mul_(sigma)
        return x.to(dt)

    res = dict(
        q=normal((n, ql, hq, d), q_scale), k_base=normal((hkv, L, d)), v_base=normal((hkv, L, d)),
        lk=normal((c.n_lr, L, r)), lv=normal((c.n_lr, L, r)),
        bk=normal((n, r, hkv * d), b_sigma), bv=normal((n, r, hkv * d), b_sigma),
        k_priv=normal((n, hkv, S, d)) if S else None, v_priv=normal((n, hkv, S, d)) if S else None,
        block_table=None)
    return res


def rope_theta(head_dim: int, base: float = 10000.0) -> np.ndarray:
    """Rotation frequencies of a rotary positional table, base^(-2f/d) for
    f < d/2, as fp32 (radians per position)."""
    f = np.arange(head_dim // 2, dtype=np.float64)
    return (base ** (-2.0 * f / head_dim)).astype(np.float32)


def rope_table(length: int, head_dim: int, base: float = 10000.0) -> np.ndarray:
    """A model's positional (rotary) table for tokens 0 .. length-1: entry
    [j, f] holds (cos, sin) of the angle j * base^(-2f/d), f < d/2, as fp32.
    An input of the rebuilt-key attention (like the model's weights); the
    angles are formed in fp64 and the cosines and sines rounded once to fp32."""
    f = np.arange(head_dim // 2, dtype=np.float64)
    theta = base ** (-2.0 * f / head_dim)
    ang = np.arange(length, dtype=np.float64)[:, None] * theta[None, :]
    return np.ascontiguousarray(np.stack([np.cos(ang), np.sin(ang)], axis=-1).astype(np.float32))


def torch_to_numpy(t):
    """torch tensor (any device) -> numpy in this module's storage convention."""
    import torch

    if t is None:
        return None
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()
