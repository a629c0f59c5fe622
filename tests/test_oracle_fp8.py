"""Pins of the FP8 (OCP E4M3) oracle (oracle/fp8.py).

Independent of the oracle's own value table:
  * code points fixed by the OCP 8-bit floating-point format: 1.0, -1.0,
    1.5, the largest finite value 448, the smallest normal 2^-6, the
    smallest and largest subnormals, the NaN codes;
  * every finite code round-trips;
  * ties go to the even mantissa; saturation at 448; signed zero kept;
  * on random inputs the chosen code is the nearest of all 254 finite codes
    (brute force), and the relative error of normal values is at most 2^-4;
  * the FP8 projection equals a float64 product of the dequantised operands
    formed element by element from the format's definition.
"""
import numpy as np
import pytest

from oracle import fp8


def test_ocp_code_points():
    v = fp8.e4m3_values()
    assert v[0x38] == 1.0 and v[0xB8] == -1.0 and v[0x3C] == 1.5
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0
    assert v[0x08] == 2.0 ** -6                     # smallest normal
    assert v[0x01] == 2.0 ** -9 and v[0x07] == 7 * 2.0 ** -9
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert v[0x00] == 0.0 and np.signbit(v[0x80])
    assert fp8.quantize_e4m3([1.0, -1.0, 448.0, 2.0 ** -9]).tolist() == [0x38, 0xB8, 0x7E, 0x01]


def test_every_finite_code_round_trips():
    v = fp8.e4m3_values()
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    assert np.array_equal(fp8.quantize_e4m3(v[codes]), codes.astype(np.uint8))


def test_ties_to_even_and_saturation():
    q = fp8.quantize_e4m3
    # 1.0 (0x38) and 1.125 (0x39): the midpoint goes to 0x38; 1.125 and 1.25
    # (0x3A): to 0x3A
    assert q([1.0625, 1.1875, -1.0625]).tolist() == [0x38, 0x3A, 0xB8]
    # subnormal midpoint between 2^-9 and 2 2^-9 goes to the even 0x02
    assert q([1.5 * 2.0 ** -9, 0.5 * 2.0 ** -9]).tolist() == [0x02, 0x00]
    assert q([448.0, 463.9, 464.0, 1e9, np.inf, -1e9]).tolist() == [0x7E] * 5 + [0xFE]
    assert q([np.nan]).tolist() == [0x7F]
    assert q([-0.0]).tolist() == [0x80] and q([0.0]).tolist() == [0x00]


def test_nearest_code_by_brute_force():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.normal(0, 1, 2000) * np.exp2(rng.integers(-10, 9, 2000)),
                        rng.uniform(-450, 450, 500)])
    codes = fp8.quantize_e4m3(x)
    v = fp8.e4m3_values()
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    for xi, ci in zip(x, codes):
        dist = np.abs(v[finite] - xi)
        assert abs(v[ci] - xi) == dist.min()
    normal = (np.abs(x) >= 2.0 ** -6) & (np.abs(x) <= 448.0)
    rel = np.abs(v[codes[normal]] - x[normal]) / np.abs(x[normal])
    assert rel.max() <= 2.0 ** -4


def test_scaled_quantisation_and_projection():
    rng = np.random.default_rng(5)
    e = rng.normal(0, 0.02, (7, 24))
    W = rng.normal(0, 0.05, (5, 24))
    se, sw = 11, 10
    e8, W8 = fp8.quantize(e, se), fp8.quantize(W, sw)
    v = fp8.e4m3_values()
    want = np.zeros((7, 5))
    for t in range(7):
        for o in range(5):
            want[t, o] = sum((v[e8[t, j]] / 2.0 ** se) * (v[W8[o, j]] / 2.0 ** sw)
                             for j in range(24))
    assert np.allclose(fp8.project_fp8(e8, se, W8, sw), want, rtol=1e-12, atol=1e-15)
    # the quantised operands are within the format's relative bound
    assert np.all(np.abs(fp8.dequantize(e8, se) - e) <= 2.0 ** -4 * np.abs(e) + 2.0 ** -10 * 2.0 ** -se)


@pytest.mark.parametrize("bits", [0x3F80, 0xBF80, 0x0000, 0x8000, 0x7F80, 0x7FC0])
def test_bf16_inputs(bits):
    # 1.0, -1.0, +0, -0, +inf (saturates), NaN
    x = fp8.bf16_bits_to_f64([bits])
    want = {0x3F80: 0x38, 0xBF80: 0xB8, 0x0000: 0x00, 0x8000: 0x80, 0x7F80: 0x7E, 0x7FC0: 0x7F}
    assert fp8.quantize_e4m3(x).tolist() == [want[bits]]
