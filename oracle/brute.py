"""40-digit decimal brute force of the same definition as ``rattn_oracle.c``.

TEST INFRASTRUCTURE.  Independent of the C code: Python's ``decimal`` module,
exact widening of the input bits, plain loops, tiny shapes only.  It pins the C
oracle's arithmetic (step order as in the definition: gather, materialise
K_a = K_base + Lk_a Bk_a^(k) and V_a likewise, append private tokens, score
with 1/sqrt(d), softmax, weighted value sum; ForkKV Guide, "Mathematical
Decomposition of LoRA KV Activations" and "Mathematical Formulation of
ResidualAttention").
"""
from __future__ import annotations

import decimal
from decimal import Decimal

import numpy as np

_CTX = decimal.Context(prec=40)


def _widen(a: np.ndarray):
    """Input array -> nested Decimal values, exactly."""
    if a.dtype == np.uint16:
        f = (a.astype(np.uint32) << 16).view(np.float32)
    else:
        f = a
    return np.vectorize(lambda x: Decimal(float(x)), otypes=[object])(f)


def attend(case, inputs):
    """Returns (out, lse) as nested lists of Decimal, indexed [a][t][h][dd] and [a][t][h]."""
    c = case
    D = c.head_dim
    g = c.n_q_heads // c.n_kv_heads
    W = {k: (None if v is None else _widen(np.asarray(v))) for k, v in inputs.items() if k != "block_table"}
    table = inputs.get("block_table")
    scale = _CTX.divide(Decimal(1), _CTX.sqrt(Decimal(D)))
    with decimal.localcontext(_CTX):
        out = [[[None] * c.n_q_heads for _ in range(c.q_len)] for _ in range(c.n_agents)]
        lse = [[[None] * c.n_q_heads for _ in range(c.q_len)] for _ in range(c.n_agents)]
        for a in range(c.n_agents):
            lr = 0 if c.shared_lr else a
            for h in range(c.n_q_heads):
                k = h // g
                keys, vals = [], []
                for j in range(c.prefix_len):
                    if c.page_size:
                        p, s = int(table[j // c.page_size]), j % c.page_size
                        kb, vb = W["k_base"][p, k, s], W["v_base"][p, k, s]
                    else:
                        kb, vb = W["k_base"][k, j], W["v_base"][k, j]
                    kr, vr = [], []
                    for dd in range(D):
                        dk = sum((W["lk"][lr, j, i] * W["bk"][a, i, k * D + dd] for i in range(c.rank)), Decimal(0))
                        dv = sum((W["lv"][lr, j, i] * W["bv"][a, i, k * D + dd] for i in range(c.rank)), Decimal(0))
                        kr.append(kb[dd] + dk)
                        vr.append(vb[dd] + dv)
                    keys.append(kr)
                    vals.append(vr)
                for j in range(c.priv_len):
                    keys.append(list(W["k_priv"][a, k, j]))
                    vals.append(list(W["v_priv"][a, k, j]))
                for t in range(c.q_len):
                    nk = c.prefix_len + (t + 1 if c.mode == "prefill" else c.priv_len)
                    q = W["q"][a, t, h]
                    s = [scale * sum((q[dd] * keys[j][dd] for dd in range(D)), Decimal(0)) for j in range(nk)]
                    mx = max(s)
                    e = [(x - mx).exp() for x in s]
                    tot = sum(e, Decimal(0))
                    out[a][t][h] = [sum((e[j] * vals[j][dd] for j in range(nk)), Decimal(0)) / tot for dd in range(D)]
                    lse[a][t][h] = mx + tot.ln()
        return out, lse


def to_float(out, lse):
    o = np.array([[[[float(x) for x in row] for row in th] for th in at] for at in out])
    l = np.array([[[float(x) for x in th] for th in at] for at in lse])
    return o, l


def lr_project(x, a_t):
    """40-digit decimal L = X A for tiny shapes (the same definition as
    oracle.cache_write.lr_project: A given as [r, d_in]; one output set per
    X or A set, a single set being shared).  Returns nested lists of Decimal
    [n][t][c]."""
    X = _widen(np.asarray(x))
    A = _widen(np.asarray(a_t))
    nx, na = X.shape[0], A.shape[0]
    n_out = max(nx, na)
    with decimal.localcontext(_CTX):
        return [[[sum((X[0 if nx == 1 else n, t, k] * A[0 if na == 1 else n, c, k] for k in range(X.shape[2])),
                      Decimal(0)) for c in range(A.shape[1])] for t in range(X.shape[1])] for n in range(n_out)]
