"""fp64 reference for base values stored as 3-bit codes after a Walsh-Hadamard
rotation (PolyKV, section 2B, "TurboQuant MSE": each value vector is rotated by
a fast Walsh-Hadamard transform so that its coordinates spread out and
approach a standard normal, every coordinate is mapped to the nearest of eight
Lloyd-Max centroids designed for N(0, 1), and decoding looks the centroids up
and applies the inverse transform).

TEST INFRASTRUCTURE, not part of the product: only ``tests/`` (and the smoke
check and bench baselines) import it.  It shares no code with the HIP library.

Readings of what the page leaves open, written out:
  * the transform is the Sylvester-ordered Hadamard matrix H_d (entries +-1,
    H_d H_d = d I) over the head dimension d of one (token, KV head) value
    vector v;
  * "converge to N(0, 1)": the rotated coordinates z = H_d v are divided by
    their root mean square, which is ||v|| (sum z_j^2 = d ||v||^2), so
    u_j = z_j / ||v|| has unit mean square; a zero vector gives u = 0;
  * the centroids are the 8-level minimum-MSE (Lloyd-Max) quantiser of N(0, 1):
    each centroid is the mean of N(0, 1) over its cell and each inner boundary
    the midpoint of its two centroids; the quantiser is symmetric, so the
    middle boundary is 0;
  * code(u) = the number of boundaries b_1 < ... < b_7 with u >= b_k (0..7);
  * stored per vector: the 3-bit codes as three bit planes (plane p holds bit
    p of every code, coordinate j at bit j % 8 of byte j / 8), 3 d / 8 bytes,
    and one fp32 scale s = fp32(||v|| / d);
  * decoded vector: v_hat = s * H_d c, with c_j the centroid of code j (since
    v = H_d z / d and z ~ ||v|| c).
The codes are decided in fp64 from the exact inputs (z and ||v||^2 are exact
in fp64 for bf16 inputs; the square root and the division are correctly
rounded).
"""
from __future__ import annotations

import math

import numpy as np

LEVELS = 8


def _pdf(x: float) -> float:
    return math.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)


def _cdf(x: float) -> float:
    return 0.5 * (1.0 + math.erf(x / math.sqrt(2.0)))


def _cell_mean(a: float, b: float) -> float:
    """E[X | a <= X < b] for X ~ N(0, 1) (a = -inf or b = +inf allowed):
    (pdf(a) - pdf(b)) / (cdf(b) - cdf(a))."""
    pa = 0.0 if math.isinf(a) else _pdf(a)
    pb = 0.0 if math.isinf(b) else _pdf(b)
    return (pa - pb) / (_cdf(b) - _cdf(a))


def lloyd_max_normal(levels: int = LEVELS, iters: int = 10000, tol: float = 1e-16):
    """(centroids, boundaries) of the minimum-MSE quantiser of N(0, 1) with an
    even number of levels, by Lloyd's alternation of the two optimality
    conditions on the non-negative half (the other half mirrors it).
    centroids: ascending, length `levels`; boundaries: the levels - 1 inner
    cell edges, ascending (the middle one is 0)."""
    h = levels // 2
    # start from equally spaced positive centroids
    c = [0.5 + i for i in range(h)]
    for _ in range(iters):
        edges = [0.0] + [0.5 * (c[i] + c[i + 1]) for i in range(h - 1)] + [math.inf]
        new = [_cell_mean(edges[i], edges[i + 1]) for i in range(h)]
        done = max(abs(x - y) for x, y in zip(new, c)) <= tol
        c = new
        if done:
            break
    pos = np.array(c, dtype=np.float64)
    cent = np.concatenate([-pos[::-1], pos])
    bpos = np.array([0.5 * (c[i] + c[i + 1]) for i in range(h - 1)], dtype=np.float64)
    bnd = np.concatenate([-bpos[::-1], [0.0], bpos])
    return cent, bnd


def fwht(x: np.ndarray) -> np.ndarray:
    """H_d x over the last axis (d a power of two), unnormalised, by the
    butterfly: at each stride h, (a, b) -> (a + b, a - b) on pairs h apart."""
    y = np.array(x, dtype=np.float64, copy=True)
    d = y.shape[-1]
    h = 1
    while h < d:
        y = y.reshape(y.shape[:-1] + (d // (2 * h), 2, h))
        a = y[..., 0, :].copy()
        b = y[..., 1, :].copy()
        y[..., 0, :] = a + b
        y[..., 1, :] = a - b
        y = y.reshape(y.shape[:-3] + (d,))
        h *= 2
    return y


def _f64(a: np.ndarray) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.uint16:  # bf16 bit patterns
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def normalized_coords(v: np.ndarray) -> np.ndarray:
    """u = H_d v / ||v|| per vector (last axis), 0 for a zero vector."""
    vf = _f64(v)
    z = fwht(vf)
    nrm = np.sqrt(np.sum(vf * vf, axis=-1, keepdims=True))
    return np.divide(z, nrm, out=np.zeros_like(z), where=nrm > 0)


def codes_of(u: np.ndarray, boundaries: np.ndarray) -> np.ndarray:
    """Number of boundaries at or below each u (0 .. levels - 1)."""
    return np.sum(u[..., None] >= boundaries, axis=-1).astype(np.uint8)


def pack_planes(codes: np.ndarray) -> np.ndarray:
    """[..., d] codes 0..7 -> [..., 3 d / 8] bytes: plane p (bytes p d/8 ..
    (p + 1) d/8 - 1) holds bit p of code j at bit j % 8 of byte j / 8."""
    d = codes.shape[-1]
    planes = []
    for p in range(3):
        bits = ((codes >> p) & 1).astype(np.uint8).reshape(codes.shape[:-1] + (d // 8, 8))
        planes.append(np.sum(bits << np.arange(8, dtype=np.uint8), axis=-1).astype(np.uint8))
    return np.concatenate(planes, axis=-1)


def unpack_planes(packed: np.ndarray, d: int) -> np.ndarray:
    out = np.zeros(packed.shape[:-1] + (d,), dtype=np.uint8)
    for p in range(3):
        plane = packed[..., p * d // 8:(p + 1) * d // 8]
        bits = (plane[..., :, None] >> np.arange(8, dtype=np.uint8)) & 1
        out |= (bits.reshape(packed.shape[:-1] + (d,)) << p).astype(np.uint8)
    return out


def quantize_values(v: np.ndarray):
    """(packed codes uint8 [..., 3 d / 8], scales float32 [...]) of value
    vectors v [..., d] (bf16 bit patterns or floats)."""
    vf = _f64(v)
    d = vf.shape[-1]
    _, bnd = lloyd_max_normal()
    u = normalized_coords(v)
    codes = codes_of(u, bnd)
    scale = (np.sqrt(np.sum(vf * vf, axis=-1)) / d).astype(np.float32)
    return pack_planes(codes), scale


def dequantize_values(packed: np.ndarray, scale: np.ndarray, d: int) -> np.ndarray:
    """v_hat = s * H_d c in fp64."""
    cent, _ = lloyd_max_normal()
    c = cent[unpack_planes(packed, d)]
    return scale.astype(np.float64)[..., None] * fwht(c)


def widen(inputs: dict, k_codes: np.ndarray, k_scale, v_packed: np.ndarray, v_scale: np.ndarray) -> dict:
    """Every input as fp64 (exact widening), with k_base the dequantised int8
    keys (see quant.py) and v_base the decoded 3-bit values."""
    from . import quant

    out = quant.widen(inputs, k_codes, k_scale)
    out["v_base"] = dequantize_values(v_packed, v_scale, inputs["v_base"].shape[-1])
    return out
