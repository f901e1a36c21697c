"""fp64 reference for base keys stored as int8 codes with one scale per
tensor (PolyKV, section 2B, Asymmetric compression: keys quantised to int8
with per-tensor linear quantisation, because the softmax scores are sensitive
to low-bit keys; the shared pool is written once and read by every agent).

TEST INFRASTRUCTURE, not part of the product: only ``tests/`` (and the smoke
check and bench baselines) import it.  It shares no code with the HIP library.

The quantiser, written out:
  * amax = max_j |K_j| over the whole tensor (every KV head and token);
  * scale s = amax / 127, computed in fp64 and rounded once to fp32 (the
    stored scale); amax = 0 gives s = 1 (every code 0);
  * code x_j = round-half-to-even(K_j / s) in fp64, clamped to [-127, 127];
  * stored as the byte x_j + 128 (excess-128: 128 means 0);
  * dequantised key: s * x_j (exact in fp64).
Attention over int8 keys is attention over the dequantised keys: the residual
corrections and the values are unchanged (the low-rank score correction adds
to the dequantised base score).  ``widen`` turns every input into fp64
(exactly), with the keys dequantised, for the fp64 attention oracle.
"""
from __future__ import annotations

import numpy as np


def _f64(a: np.ndarray) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.uint16:  # bf16 bit patterns
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def quantize_keys(k: np.ndarray):
    """(codes, scale): codes uint8 (excess-128) of k's shape, scale np.float32."""
    kf = _f64(k)
    amax = float(np.max(np.abs(kf))) if kf.size else 0.0
    s = np.float32(amax / 127.0) if amax > 0 else np.float32(1.0)
    x = np.clip(np.rint(kf / np.float64(s)), -127, 127)
    return (x + 128).astype(np.uint8), s


def dequantize_keys(codes: np.ndarray, scale) -> np.ndarray:
    return (codes.astype(np.int64) - 128).astype(np.float64) * np.float64(np.float32(scale))


def widen(inputs: dict, codes: np.ndarray, scale) -> dict:
    """Every input as fp64 (exact widening), with k_base replaced by the
    dequantised int8 keys; the block table is kept as it is."""
    out = {}
    for name, a in inputs.items():
        if a is None or name == "block_table":
            out[name] = a
        elif name == "k_base":
            out[name] = dequantize_keys(codes, scale)
        else:
            out[name] = _f64(a)
    return out
