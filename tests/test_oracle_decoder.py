"""Pins for the decoder-stack oracle (``oracle.decoder``): closed forms and
mathematical properties that a dropped term, a wrong sign, a swapped pairing
or a wrong tie rule would break.  CPU only."""
import math

import numpy as np
import pytest

import synth
from oracle import decoder as od


def _bits(x):
    return synth.bf16_bits(np.asarray(x, dtype=np.float32))


# ---- rotary embedding --------------------------------------------------------

def test_rope_position_zero_is_identity():
    x = synth.normal_bits((3, 2, 8), 0, 1, 0, "rope.id")
    got = od.rope(x, np.zeros(3, dtype=np.int32), 10000.0)
    assert np.array_equal(got, synth.bf16_to_f32(x).astype(np.float64))


def test_rope_closed_form_and_rotate_half_pairing():
    # d = 4: pair 0 is (x0, x2) at angle p, pair 1 is (x1, x3) at p * theta^(-1/2)
    theta, p = 10000.0, 7
    x = np.array([[[1.0, 0.0, 0.0, 0.0]]])
    got = od.rope(x, np.array([p]), theta)[0, 0]
    assert got == pytest.approx([math.cos(p), 0.0, math.sin(p), 0.0], abs=1e-15)
    y = np.array([[[0.0, 2.0, 0.0, 0.0]]])
    a = p * theta ** -0.5
    got = od.rope(y, np.array([p]), theta)[0, 0]
    assert got == pytest.approx([0.0, 2 * math.cos(a), 0.0, 2 * math.sin(a)], abs=1e-15)
    # the second element of a pair gets +a sin + b cos
    z = np.array([[[0.0, 0.0, 1.0, 0.0]]])
    got = od.rope(z, np.array([p]), theta)[0, 0]
    assert got == pytest.approx([-math.sin(p), 0.0, math.cos(p), 0.0], abs=1e-15)


def test_rope_is_a_rotation_group():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 3, 16))
    p1 = np.array([0, 1, 17, 300, 4095])
    p2 = np.array([5, 9, 0, 81, 1])
    twice = od.rope(od.rope(x, p1, 500000.0), p2, 500000.0)
    assert np.allclose(twice, od.rope(x, p1 + p2, 500000.0), rtol=0, atol=1e-12)
    # every (i, i + d/2) pair keeps its length
    y = od.rope(x, p1, 500000.0)
    n0 = x[..., :8] ** 2 + x[..., 8:] ** 2
    n1 = y[..., :8] ** 2 + y[..., 8:] ** 2
    assert np.allclose(n0, n1, rtol=1e-13, atol=0)


# ---- SwiGLU -------------------------------------------------------------------

def test_silu_closed_forms():
    ln3 = math.log(3.0)
    got = od.silu(np.array([0.0, ln3, -ln3, 40.0]))
    assert got[0] == 0.0
    assert got[1] == pytest.approx(0.75 * ln3, rel=1e-15)   # sigma(ln 3) = 3/4
    assert got[2] == pytest.approx(-0.25 * ln3, rel=1e-15)  # sigma(-ln 3) = 1/4
    assert got[3] == pytest.approx(40.0, rel=1e-15)


def test_swiglu_multiplies_by_up():
    ln3 = math.log(3.0)
    got = od.swiglu(np.array([ln3, ln3]), np.array([2.0, -4.0]))
    assert got == pytest.approx([1.5 * ln3, -3.0 * ln3], rel=1e-15)
    # bf16 bit-pattern inputs are widened exactly: 1.0 and 2.0
    got = od.swiglu(_bits([1.0]), _bits([2.0]))
    assert got[0] == pytest.approx(2.0 / (1.0 + math.exp(-1.0)), rel=1e-15)


# ---- add, embed, argmax -------------------------------------------------------

def test_add_exact_on_representable_values():
    assert np.array_equal(od.add(_bits([1.0, -2.5, 3.0]), _bits([0.5, 2.5, -7.0])),
                          np.array([1.5, 0.0, -4.0]))


def test_embed_gathers_and_clamps():
    table = _bits(np.arange(12, dtype=np.float32).reshape(4, 3))
    got = od.embed(np.array([2, 0, 3, -5, 9]), table)
    assert np.array_equal(got, np.array([[6, 7, 8], [0, 1, 2], [9, 10, 11], [0, 1, 2],
                                         [9, 10, 11]], dtype=np.float64))


def test_argmax_ties_nan_and_empty_rows():
    nan, inf = float("nan"), float("inf")
    x = np.array([[1.0, 3.0, 3.0, 2.0],        # tie: lowest index
                  [nan, 0.5, nan, 0.5],        # NaN never chosen, tie -> 1
                  [nan, nan, nan, nan],        # nothing to choose -> 0
                  [-inf, -inf, -inf, -inf],    # all equal -> 0
                  [-1.0, -inf, inf, inf]])     # +inf tie -> 2
    assert od.argmax(x).tolist() == [1, 1, 0, 0, 2]
