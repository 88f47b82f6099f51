"""Pins of the rotary-embedding oracle (oracle/rope.py) to things other than its own formula.

* Position 0 (angle 0) leaves every element's bits unchanged, in every dtype.
* A hand-evaluated D = 4 case at position 1, base 10000: the two pairs are (x0, x2) and (x1, x3),
  the rotate-half pairing of Llama/Mistral/Qwen, rotated by 1 rad and 0.01 rad.
* The float64 path is a rotation by the table's angle: angles add (rotating by a then by b equals
  rotating by a + b), pair norms are kept, and a query-key score after rotation depends only on
  the position difference (the property that makes it a relative position code).  A rotation
  with a flipped sign fails the first two; a wrong pairing fails the hand case.
* The float32 path (the kernel's precision) stays within float32 rounding of the float64 path,
  and rounding to bf16 / fp16 stays within half an ulp of the element type plus that.
"""
import math

import numpy as np
import pytest

from oracle import rope as R
from workloads import rope_tables


def exact_tables(positions, D, base=10000.0):
    """float64 cos/sin (no float32 rounding), for the algebraic pins."""
    i = np.arange(D // 2, dtype=np.float64)
    ang = np.arange(positions, dtype=np.float64)[:, None] * base ** (-2.0 * i / D)[None, :]
    return np.cos(ang), np.sin(ang)


def angle_tables(angles):
    """Tables whose row r rotates pair i by angles[r][i]."""
    a = np.asarray(angles, dtype=np.float64)
    return np.cos(a), np.sin(a)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_position_zero_is_identity(dtype):
    rng = np.random.default_rng(0)
    x = rng.standard_normal((3, 4, 64)).astype(np.float32)
    x[x == 0] = 1.0
    store = {"f32": x, "f16": x.astype(np.float16),
             "bf16": (x.view(np.uint32) >> 16).astype(np.uint16)}[dtype]
    c, s = rope_tables(8, 64)
    assert np.all(c[0] == 1.0) and np.all(s[0] == 0.0)
    y = R.rotate(store, dtype, np.zeros(3, dtype=np.int64), c, s)
    assert np.array_equal(np.asarray(y).view(np.uint8), np.asarray(store).view(np.uint8))


def test_hand_evaluated_d4_case():
    x = np.array([[[1.0, 2.0, 3.0, 4.0]]])
    c, s = exact_tables(2, 4)
    y = R.rotate(x, "f64", np.array([1]), c, s)[0, 0]
    c0, s0, c1, s1 = math.cos(1.0), math.sin(1.0), math.cos(0.01), math.sin(0.01)
    expect = [1 * c0 - 3 * s0, 2 * c1 - 4 * s1, 3 * c0 + 1 * s0, 4 * c1 + 2 * s1]
    assert np.allclose(y, expect, rtol=0, atol=1e-15)
    # 1 rad turns (1, 3) to about (-1.984, 2.462); 0.01 rad barely moves (2, 4)
    assert abs(y[0] + 1.98411) < 1e-5 and abs(y[2] - 2.46238) < 1e-5


def test_angles_add_and_norms_are_kept():
    rng = np.random.default_rng(1)
    D = 16
    x = rng.standard_normal((1, 3, D))
    a = rng.uniform(-4, 4, size=D // 2)
    b = rng.uniform(-4, 4, size=D // 2)
    ca, sa = angle_tables([a, b, a + b])
    y_ab = R.rotate(R.rotate(x, "f64", np.array([0]), ca, sa), "f64", np.array([1]), ca, sa)
    y_sum = R.rotate(x, "f64", np.array([2]), ca, sa)
    assert np.abs(y_ab - y_sum).max() < 1e-13
    h = D // 2
    n_in = x[..., :h] ** 2 + x[..., h:] ** 2
    n_out = y_sum[..., :h] ** 2 + y_sum[..., h:] ** 2
    assert np.abs(n_in - n_out).max() < 1e-12


def test_scores_depend_only_on_position_difference():
    rng = np.random.default_rng(2)
    D = 32
    q = rng.standard_normal((1, 1, D))
    k = rng.standard_normal((1, 1, D))
    c, s = exact_tables(200, D, base=500000.0)
    def score(m, n):
        return float((R.rotate(q, "f64", np.array([m]), c, s) *
                      R.rotate(k, "f64", np.array([n]), c, s)).sum())
    for m, n in [(7, 3), (150, 146), (40, 36), (4, 0)]:
        assert abs(score(m, n) - score(4, 0)) < 1e-12
    assert abs(score(9, 3) - score(4, 0)) > 1e-6    # a different difference scores differently


@pytest.mark.parametrize("dtype,half_ulp", [("bf16", 2.0 ** -9), ("f16", 2.0 ** -12)])
def test_float32_path_is_the_rotation_within_rounding(dtype, half_ulp):
    rng = np.random.default_rng(3)
    D, P = 128, 4096
    x = rng.standard_normal((16, 8, D)).astype(np.float32)
    c, s = rope_tables(P, D, base=500000.0)
    pos = rng.integers(0, P, size=16)
    y32 = R.rotate(x, "f32", pos, c, s).astype(np.float64)
    y64 = R.rotate(x.astype(np.float64), "f64", pos, c.astype(np.float64), s.astype(np.float64))
    mag = np.abs(x).max()
    assert np.abs(y32 - y64).max() <= 4 * 2.0 ** -24 * 2 * mag
    store = {"f16": x.astype(np.float16), "bf16": R._from_f32(x, "bf16")}[dtype]
    y = R._to_f32(R.rotate(store, dtype, pos, c, s), dtype).astype(np.float64)
    ref = R.rotate(R._to_f32(store, dtype).astype(np.float64), "f64", pos, c.astype(np.float64),
                   s.astype(np.float64))
    assert np.all(np.abs(y - ref) <= half_ulp * np.maximum(np.abs(ref), 2.0 ** -14) * 2 + 1e-6)


def test_rope_append_writes_rotated_key_and_plain_value():
    rng = np.random.default_rng(4)
    B, Hkv, D, PS, NP = 3, 2, 8, 4, 6
    kp = rng.standard_normal((NP, PS, Hkv, D)).astype(np.float32)
    vp = rng.standard_normal((NP, PS, Hkv, D)).astype(np.float32)
    kn = rng.standard_normal((B, Hkv, D)).astype(np.float32)
    vn = rng.standard_normal((B, Hkv, D)).astype(np.float32)
    q = rng.standard_normal((B, 4, D)).astype(np.float32)
    table = np.array([[0, 1], [2, 3], [4, 5]], dtype=np.int32)
    lens = np.array([5, -1, 0], dtype=np.int32)
    c, s = rope_tables(16, D)
    q2, kp2, vp2 = R.rope_kv_append(q, kp, vp, kn, vn, table, lens, c, s, "f32")
    assert np.array_equal(q2[1], q[1])                       # padding row untouched
    assert np.array_equal(q2[2], q[2])                       # position 0: identity
    assert np.array_equal(kp2[1, 1], R.rotate(kn[:1], "f32", np.array([5]), c, s)[0])
    assert np.array_equal(vp2[1, 1], vn[0])
    assert np.array_equal(kp2[4, 0], kn[2]) and np.array_equal(vp2[4, 0], vn[2])
    changed = np.zeros((NP, PS), dtype=bool)
    changed[1, 1] = changed[4, 0] = True
    assert np.array_equal(kp2[~changed], kp[~changed]) and np.array_equal(vp2[~changed], vp[~changed])
