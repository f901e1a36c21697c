"""fp64 reference for attention whose residual keys are rebuilt per token and
rotated by position before the score (the ForkKV Guide's kernel design,
"Fused ResidualAttention", section 2 On-the-Fly Register Fusion: the residual
key is added to the base key in registers right before the product).

TEST INFRASTRUCTURE, not part of the product: only ``tests/`` (and the smoke
check and bench baselines) import it.  It shares no code with the HIP library.

Why a rotation: the factored score q . (Lk_j Bk) = (q Bk^T) . Lk_j holds only
while the residual key is used as it comes out of the up-projection.  When a
model rotates keys by position after the projection (rotary position
embedding), the residual key of token j is rot_j(Lk_j Bk), and the product no
longer factors through one q Bk^T per query row; the key has to be rebuilt.
The pages do not describe the rotation; the reading taken here is the common
rotate-half form: for d-vector x and frequency index f < d/2,
    rot_j(x)[f]       = x[f] cos_j[f] - x[f + d/2] sin_j[f]
    rot_j(x)[f + d/2] = x[f + d/2] cos_j[f] + x[f] sin_j[f]
with the cosines and sines of token j's angles given as a table
rope[j, f] = (cos, sin) (the positional table of the model, an input like its
weights; ``table_from_theta`` forms it in fp64 from frequencies theta[f], the
angle of token j being j * theta[f]).  K_base is taken as already rotated (the base model wrote
it so); values are not rotated, so the value residual keeps its factored form.

The definition, written out for agent a, KV head k, logical token j < L:
    K_a[j] = K_base[j] + rot_j(Lk_a[j] Bk_a^(k)),   V_a[j] = V_base[j] + Lv_a[j] Bv_a^(k)
then the private tokens and textbook softmax attention exactly as in
``oracle.attend``, which computes the attention: it is called with the rebuilt
keys as an fp64 base cache and the key up-projection set to zero, one agent at
a time.  Without a table (rope None) the rotation is the identity.
"""
from __future__ import annotations

import numpy as np

import oracle


def _f64(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:  # bf16 bit patterns
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def table_from_theta(theta: np.ndarray, length: int) -> np.ndarray:
    """The (cos, sin) table [length, d/2, 2] that frequencies theta (radians
    per position, the values as given) define: angle j * theta[f], in fp64."""
    ang = np.arange(length, dtype=np.float64)[:, None] * np.asarray(theta, dtype=np.float64)[None, :]
    return np.stack([np.cos(ang), np.sin(ang)], axis=-1)


def rotate(x: np.ndarray, rope) -> np.ndarray:
    """rot_j applied to rows x[..., j, :] (d last), rope [L, d/2, 2] (cos, sin)."""
    if rope is None:
        return x
    rp = _f64(rope)
    h = x.shape[-1] // 2
    c, s = rp[..., 0], rp[..., 1]
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def rebuilt_keys(case, x: dict, agent: int, rope=None) -> np.ndarray:
    """K_a [H_kv, L, d] in fp64: base keys (logical order) plus rotated residual keys."""
    c = case
    d = c.head_dim
    if c.page_size:
        kb = _f64(oracle.gather_base(c, x["k_base"], x["block_table"]))
    else:
        kb = _f64(x["k_base"])
    lr = 0 if c.shared_lr else agent
    lk = _f64(x["lk"])[lr]                      # [L, r]
    bk = _f64(x["bk"])[agent]                   # [r, H_kv d]
    out = np.empty_like(kb)
    for k in range(c.n_kv_heads):
        dk = lk @ bk[:, k * d:(k + 1) * d]      # [L, d]
        out[k] = kb[k] + rotate(dk, rope)
    return out


def attend(case, x: dict, rope=None, row_mask=None):
    """(out, lse) fp64 with the residual keys rebuilt (and rotated when a table
    is given), each agent through ``oracle.attend`` over its rebuilt keys."""
    c = case
    out = np.full((c.n_agents, c.q_len, c.n_q_heads, c.head_dim), np.nan)
    lse = np.full((c.n_agents, c.q_len, c.n_q_heads), np.nan)
    one = c.replace(n_agents=1, page_size=0, n_phys_pages=0, shared_lr=False)
    for a in range(c.n_agents):
        if row_mask is not None and not np.any(row_mask[a]):
            continue
        lr = 0 if c.shared_lr else a
        xa = {
            "q": _f64(x["q"])[a:a + 1],
            "k_base": rebuilt_keys(c, x, a, rope),
            "v_base": _f64(oracle.gather_base(c, x["v_base"], x["block_table"])) if c.page_size else _f64(x["v_base"]),
            "lk": _f64(x["lk"])[lr:lr + 1],
            "lv": _f64(x["lv"])[lr:lr + 1],
            "bk": np.zeros_like(_f64(x["bk"])[a:a + 1]),
            "bv": _f64(x["bv"])[a:a + 1],
            "k_priv": None if x.get("k_priv") is None else _f64(x["k_priv"])[a:a + 1],
            "v_priv": None if x.get("v_priv") is None else _f64(x["v_priv"])[a:a + 1],
            "block_table": None,
        }
        m = None if row_mask is None else row_mask[a:a + 1]
        o, l = oracle.attend(one, xa, row_mask=m)
        out[a], lse[a] = o[0], l[0]
    return out, lse
