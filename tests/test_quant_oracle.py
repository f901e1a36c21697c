"""Pins of the int8-key oracle (oracle/quant.py): closed forms of the
per-tensor quantiser (PolyKV, section 2B) and the reduction of attention over
exactly representable int8 keys to attention over the same keys in bf16."""
import numpy as np

import oracle
import synth
from oracle import quant as Q


def test_integer_multiples_quantise_exactly():
    """K = j s0 with s0 = amax / 127 for integer j: codes are j, dequantised
    keys are K exactly."""
    s0 = 2.0 ** -5  # amax = 127 s0 is exact, so the stored scale is s0
    j = np.array([[-127, -3, 0, 5, 127], [64, -64, 1, -1, 100]])
    k = (j * s0).astype(np.float32)
    codes, s = Q.quantize_keys(k)
    assert s == np.float32(s0)
    assert np.array_equal(codes.astype(np.int64) - 128, j)
    assert np.array_equal(Q.dequantize_keys(codes, s), k.astype(np.float64))


def test_ties_round_to_even_and_extremes_clamp():
    s0 = 0.25
    k = np.array([127 * s0, 2.5 * s0, 3.5 * s0, -2.5 * s0, -0.5 * s0, 0.5 * s0], np.float32)
    codes, s = Q.quantize_keys(k)
    assert s == np.float32(s0)
    assert list(codes.astype(np.int64) - 128) == [127, 2, 4, -2, 0, 0]
    assert Q.quantize_keys(np.zeros(4, np.float32))[0].tolist() == [128] * 4


def test_error_bound_half_a_step():
    """|s x - K| <= s / 2 for every element, and the largest |K| maps to +-127."""
    k = synth.bf16_bits(np.random.default_rng(0).standard_normal((4, 300, 64)))
    codes, s = Q.quantize_keys(k)
    kf = Q._f64(k)
    err = np.abs(Q.dequantize_keys(codes, s) - kf)
    assert err.max() <= float(s) / 2 * (1 + 1e-6)
    i = np.unravel_index(np.argmax(np.abs(kf)), kf.shape)
    assert abs(int(codes[i]) - 128) == 127
    assert codes.min() >= 1  # excess-128 codes of -127 .. 127


def test_attention_over_representable_keys_equals_bf16_attention():
    """When every base key is an integer multiple of a power-of-two scale (so
    exact in bf16 and in int8), attention over the int8 keys (dequantised,
    fp64) equals attention over the same keys in bf16, and residual terms
    are unchanged by the key storage."""
    case = synth.Case(3, 8, 2, 16, 4, 50, priv_len=3, dtype="bf16")
    x = synth.make_inputs(case, 9, b_sigma=0.3)
    rng = np.random.default_rng(1)
    j = rng.integers(-127, 128, size=x["k_base"].shape)
    j.flat[0] = 127
    x["k_base"] = synth.bf16_bits(j * 2.0 ** -6)
    codes, s = Q.quantize_keys(x["k_base"])
    assert s == np.float32(2.0 ** -6)
    o_q, l_q = oracle.attend(case, Q.widen(x, codes, s))
    o_b, l_b = oracle.attend(case, x)
    assert np.array_equal(o_q, o_b) and np.array_equal(l_q, l_b)
