"""Pins of the tolerance check every GPU parity test goes through.

The rules (page "mlx_backend/sparse_conv_metal.py": the kernel body
accumulates in a float and stores `(T)acc`; the wrapper returns the output in
w's dtype), with the reading of the two tolerances: fp32 outputs within
1e-5 * (S + |bias|), S = sum |f*w|; bf16 outputs within 2 bf16 ulp of the
exact value, or within the fp32 bound; S == 0 outputs equal to the rounded
bias.  Each boundary is checked on both sides with hand-chosen values.
"""
import math

import numpy as np
import pytest

from oracle.compare import STRICT_FLOOR, bf16_round, check_forward, ulp_bf16


@pytest.mark.parametrize("x, u", [
    (1.0, 2.0 ** -7), (0.75, 2.0 ** -8), (3.0, 2.0 ** -6), (-1.5, 2.0 ** -7), (0.0, 0.0),
    (2.0 ** 10, 2.0 ** 3), (1.9999, 2.0 ** -7), (2.0, 2.0 ** -6), (0.5, 2.0 ** -8),
    (-(2.0 ** -20), 2.0 ** -27), (65504.0, 2.0 ** 8),
    # smallest normal and below: bf16 subnormals are spaced 2^-133
    (2.0 ** -126, 2.0 ** -133), (2.0 ** -127, 2.0 ** -133), (2.0 ** -133, 2.0 ** -133),
    (3.0 * 2.0 ** -130, 2.0 ** -133),
])
def test_ulp_bf16_hand_values(x, u):
    assert ulp_bf16(np.array([x]))[0] == u


def test_ulp_bf16_is_the_spacing_of_bf16_values():
    # the next bf16 value above each power-of-two-bracketed x is x's bucket
    # start + ulp: 1 + 2^-7 is the bf16 after 1.0 (7 stored mantissa bits)
    for e in range(-120, 120, 7):
        lo = 2.0 ** e
        assert ulp_bf16(np.array([lo]))[0] == lo * 2.0 ** -7
        assert ulp_bf16(np.array([np.nextafter(2 * lo, 0)]))[0] == lo * 2.0 ** -7


def one(v):
    return np.array([[v]], dtype=np.float64)


def test_bf16_two_ulp_boundary():
    ref, S = 1.0, 1.0            # fp32 bound 1e-5: rescues nothing here
    ok = check_forward(one(ref + 2.0 ** -6), one(ref), one(S), None, "bf16")
    assert ok["fail"] == 0 and ok["strict_2ulp_fail"] == 0
    bad = check_forward(one(np.nextafter(ref + 2.0 ** -6, 2.0)), one(ref), one(S), None, "bf16")
    assert bad["fail"] == 1 and bad["strict_2ulp_fail"] == 1
    # below 1.0 the ulp halves: 0.75 + 2 * 2^-8 passes, a hair more fails
    ok = check_forward(one(0.75 - 2.0 ** -7), one(0.75), one(S), None, "bf16")
    assert ok["fail"] == 0
    bad = check_forward(one(np.nextafter(0.75 - 2.0 ** -7, 0.0)), one(0.75), one(S), None, "bf16")
    assert bad["fail"] == 1


def test_bf16_fp32_rule_rescues_cancelled_outputs():
    # a result that cancelled to 1e-4 with S = 1000: many ulps off, but within
    # 1e-5 * S = 1e-2
    r = check_forward(one(1e-4 + 5e-3), one(1e-4), one(1000.0), None, "bf16")
    assert r["fail"] == 0 and r["strict_2ulp_fail"] == 1 and r["max_ulp"] > 2
    r = check_forward(one(1e-4 + 1.1e-2), one(1e-4), one(1000.0), None, "bf16")
    assert r["fail"] == 1


def test_fp32_boundary_with_bias():
    # err exactly 1e-5 * (S + |b|) passes, the next double above fails; |b| is
    # used with a negative bias too
    for S, b in ((1.0, None), (0.5, 0.5), (0.5, -0.5), (0.25, -0.75)):
        bias = None if b is None else np.array([b], dtype=np.float32)
        ref = 0.0                       # keeps |g - ref| exact in float64
        tol = 1e-5 * (S + (0.0 if b is None else abs(float(np.float32(b)))))
        assert check_forward(one(ref + tol), one(ref), one(S), bias, "f32")["fail"] == 0
        assert check_forward(one(np.nextafter(ref + tol, 1.0)), one(ref), one(S), bias, "f32")["fail"] == 1
        assert check_forward(one(ref - tol), one(ref), one(S), bias, "f32")["fail"] == 0


def test_zero_S_must_equal_bias_exactly_fp32():
    b32 = np.array([0.3, -1.7, 0.0], dtype=np.float32)
    ref = b32.astype(np.float64)[None, :]
    S = np.zeros((1, 3))
    assert check_forward(ref.copy(), ref, S, b32, "f32")["fail"] == 0
    off = ref.copy()
    off[0, 0] = float(np.nextafter(b32[0], np.float32(1)))   # one fp32 ulp off
    assert check_forward(off, ref, S, b32, "f32")["fail"] == 1
    # no bias: exactly zero
    z = np.zeros((1, 3))
    assert check_forward(z, z, S, None, "f32")["fail"] == 0
    assert check_forward(z + 1e-30, z, S, None, "f32")["fail"] == 3


def test_zero_S_must_equal_bf16_bias_exactly():
    b32 = np.array([0.3, -1.7, 1.0 + 2.0 ** -8], dtype=np.float32)
    rb = bf16_round(b32)
    # round to nearest, ties to even: 0.3 -> 0.30078125, -1.7 -> -1.703125,
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 and goes to the even 1.0
    assert list(rb) == [0.30078125, -1.703125, 1.0]
    ref = b32.astype(np.float64)[None, :]
    S = np.zeros((1, 3))
    assert check_forward(rb[None, :], ref, S, b32, "bf16")["fail"] == 0
    # one bf16 ulp off the rounded bias fails although it is within 2 ulp of ref
    off = rb[None, :].copy()
    off[0, 1] -= 2.0 ** -7
    assert check_forward(off, ref, S, b32, "bf16")["fail"] == 1
    # the unrounded fp32 biases are not bf16 values and fail
    assert check_forward(ref, ref, S, b32, "bf16")["fail"] == 3


def test_strict_failure_allowance():
    n = 4000
    ref = np.ones((n, 1))
    S = np.full((n, 1), 1e6)           # the fp32 rule accepts errors up to 10
    g = ref.copy()
    allowed = max(STRICT_FLOOR, int(1e-3 * n))
    g[:allowed] += 1.0                 # 128 ulp each, rescued by the fp32 rule
    r = check_forward(g, ref, S, None, "bf16")
    assert r["strict_2ulp_fail"] == allowed and r["fail"] == 0
    g[allowed] += 1.0                  # one more than allowed
    r = check_forward(g, ref, S, None, "bf16")
    assert r["fail"] == 1


def test_reports_first_failure():
    ref = np.array([[1.0, 2.0], [3.0, 4.0]])
    g = ref.copy()
    g[1, 0] += 1.0
    r = check_forward(g, ref, np.ones_like(ref), None, "f32")
    assert r["fail"] == 1 and r["first_fail"]["row"] == 1 and r["first_fail"]["col"] == 0
    assert math.isclose(r["max_norm_err"], 1.0)
