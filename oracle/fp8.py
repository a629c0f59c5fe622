"""CPU oracle of the FP8 projection operands.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU leg; shares no code with the HIP library. Plain numpy,
float64.

The Engram notes (§3.4) run the fused value and key projections as one
dense FP8 GEMM to raise matrix-unit use; they name neither the 8-bit format
nor its scaling. Readings taken here:
  * format: OCP 8-bit E4M3 -- sign, 4 exponent bits (bias 7), 3 mantissa
    bits; exponent field 0 holds subnormals m 2^-9; no infinities; the two
    codes with all seven low bits set are NaN; largest finite value 448;
  * scaling: one power-of-two exponent per tensor, chosen by the caller:
    q = E4M3(v 2^s), dequantised q 2^-s (v 2^s is exact in float64 for the
    bf16 and fp32 values quantised here);
  * rounding: to the nearest code, ties to the code with an even mantissa;
    magnitudes at or above 448 saturate to 448; NaN stays NaN; the sign of
    zero is kept;
  * what is quantised: e as the bf16 path stores it (signs applied, NF4
    already dequantised and rounded to bf16; fp32 e for an fp32 table) and
    W as stored. The GEMM then multiplies the dequantised values exactly and
    accumulates (here in float64).
Parity: pinned by tests/test_oracle_fp8.py (OCP code points, exhaustive
round trips, ties, saturation, brute-force nearest codes, the relative
error bound of 2^-4).
"""
import numpy as np

E4M3_MAX = 448.0


def e4m3_values():
    """float64 value of each of the 256 codes (NaN for 0x7F and 0xFF)."""
    c = np.arange(256)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    v = sign * mag
    v[(c & 0x7F) == 0x7F] = np.nan
    return v


def quantize_e4m3(x):
    """Codes (uint8) of already-scaled values x (float64 array)."""
    x = np.asarray(x, dtype=np.float64)
    pos = e4m3_values()[:0x7F]                 # codes 0..0x7E, ascending 0..448
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.clip(np.searchsorted(pos, a, side="left"), 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    d_hi = np.abs(pos[hi] - a)
    d_lo = np.abs(a - pos[lo])
    pick = np.where(d_lo < d_hi, lo, hi)
    tie = (d_lo == d_hi) & (lo != hi)
    pick = np.where(tie, np.where(lo % 2 == 0, lo, hi), pick)
    code = pick.astype(np.uint8) | np.where(np.signbit(x), 0x80, 0).astype(np.uint8)
    nan = np.isnan(x)
    code[nan] = (0x7F | np.where(np.signbit(x[nan]), 0x80, 0)).astype(np.uint8)
    return code


def quantize(v, s):
    """E4M3 codes of v 2^s."""
    return quantize_e4m3(np.asarray(v, dtype=np.float64) * 2.0 ** s)


def dequantize(codes, s):
    """float64 values q 2^-s of codes."""
    return e4m3_values()[np.asarray(codes, dtype=np.int64)] * 2.0 ** -s


def bf16_bits_to_f64(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def project_fp8(e8, se, W8, sw):
    """y = W e with both operands dequantised from E4M3 (float64)."""
    return dequantize(e8, se) @ dequantize(W8, sw).T
