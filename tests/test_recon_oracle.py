"""Pins of the rebuilt-key oracle (oracle/recon.py): the rotation's closed
forms, a hand-worked token, and reduction to the plain oracle when the
rotation is the identity."""
import numpy as np

import oracle
import synth
from oracle import recon


def test_identity_rotation_is_the_plain_definition():
    """No table, or a table of cos = 1, sin = 0: the rebuilt keys are
    K_base + Lk Bk and the result is the plain oracle's."""
    case = synth.Case(3, 8, 2, 16, 4, 40, priv_len=3, dtype="bf16")
    x = synth.make_inputs(case, 5, b_sigma=0.3)
    o0, l0 = oracle.attend(case, x)
    o1, l1 = recon.attend(case, x)
    assert np.abs(o1 - o0).max() <= 1e-13 and np.abs(l1 - l0).max() <= 1e-13
    ident = np.zeros((case.prefix_len, case.head_dim // 2, 2), np.float32)
    ident[..., 0] = 1.0
    o2, l2 = recon.attend(case, x, rope=ident)
    assert np.array_equal(o2, o1) and np.array_equal(l2, l1)


def test_rotation_closed_forms():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 8))
    q = np.zeros((5, 4, 2), np.float32)
    q[..., 1] = 1.0  # cos 0, sin 1: a quarter turn, rot(x) = [-x2, x1]
    r = recon.rotate(x, q)
    assert np.array_equal(r, np.concatenate([-x[:, 4:], x[:, :4]], axis=1))
    t = synth.rope_table(5, 8)
    r = recon.rotate(x, t)
    # each (f, f + d/2) pair keeps its length (cos^2 + sin^2 = 1 up to fp32 rounding)
    n0 = x[:, :4] ** 2 + x[:, 4:] ** 2
    n1 = r[:, :4] ** 2 + r[:, 4:] ** 2
    assert np.abs(n1 - n0).max() <= 1e-6 * n0.max()
    # token 0 has angle 0: unchanged
    assert np.allclose(r[0], x[0], atol=0, rtol=0)


def test_hand_worked_token():
    """d = 4, r = 1, one KV head: K = K_base + rot(Lk Bk) by hand."""
    case = synth.Case(1, 1, 1, 4, 1, 1, dtype="f32")
    x = {"q": np.zeros((1, 1, 1, 4), np.float32), "k_base": np.array([[[1.0, 2.0, 3.0, 4.0]]], np.float32),
         "v_base": np.zeros((1, 1, 4), np.float32), "lk": np.array([[[2.0]]], np.float32),
         "lv": np.zeros((1, 1, 1), np.float32), "bk": np.array([[[0.5, -1.0, 0.25, 1.0]]], np.float32),
         "bv": np.zeros((1, 1, 4), np.float32), "k_priv": None, "v_priv": None, "block_table": None}
    rope = np.array([[[0.6, 0.8], [0.0, 1.0]]], np.float32)  # f = 0: (cos .6, sin .8); f = 1: quarter turn
    dk = 2.0 * np.array([0.5, -1.0, 0.25, 1.0])               # [1, -2, .5, 2]
    want = np.array([1.0 + (1 * 0.6 - 0.5 * 0.8), 2.0 + (-2 * 0.0 - 2.0 * 1.0),
                     3.0 + (0.5 * 0.6 + 1 * 0.8), 4.0 + (2.0 * 0.0 + -2 * 1.0)])
    got = recon.rebuilt_keys(case, x, 0, rope)[0, 0]
    assert np.allclose(got, want, rtol=0, atol=1e-7)


def test_table_from_theta_matches_the_fp32_table():
    """The fp64 table of the fp32 frequencies equals synth's fp32 positional
    table (angles from fp64 frequencies) up to the frequencies' rounding
    (angle error <= j * 2^-24 theta) and the table's own, and angle 0 gives (1, 0)."""
    theta = synth.rope_theta(64)
    t64 = recon.table_from_theta(theta, 300)
    t32 = synth.rope_table(300, 64)
    assert np.abs(t64 - t32).max() <= 300 * 2.0 ** -24 + 2.0 ** -23
    assert np.array_equal(t64[0, :, 0], np.ones(32)) and np.array_equal(t64[0, :, 1], np.zeros(32))
