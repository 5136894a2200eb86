"""FP8 (E4M3) row-wise quantisation of the logit operands, for the oracle.

TEST INFRASTRUCTURE, NOT PRODUCT CODE (like the rest of this package): only the tests, the smoke
check and the bench's CPU-baseline leg may import it. It shares no code with the HIP path.

The pages' lower-precision head is a plan, not a design ("Training — design", §8.1 "Deferred
performance levers", the W4A16 head GEMM item): half-precision operands for the head's logit GEMM, forward
first, the backward's gradient GEMMs left at the higher precision until a range probe clears them,
fp32 accumulation throughout, and the exact mode kept as the parity mode. On gfx950 the half step
below bf16 is an 8-bit float, so the reading built here is:

  * the logit operands h and W are quantised per row to OCP FP8 E4M3 (1 sign, 4 exponent bits with
    bias 7, 3 mantissa bits; no infinities; S.1111.111 is NaN; largest finite 448) with one
    power-of-two scale per row (an E8M0 byte, exponent + 127): the smallest 2^e with
    max|row| <= 448 * 2^e, so the row's largest element lands in (224, 448];
  * every element is rounded to the nearest E4M3 value after the exact scaling by 2^-e, ties to
    the even code; the sign of a value that rounds to zero is kept (code 0x80 for negatives);
  * logits (forward and the backward's recompute) come from the dequantised operands
    (code value times 2^e, exact in float64); the gradient GEMMs dh = coeff . W and
    dW = coeff^T . h keep the unquantised bf16 operands.

Pins: tests/test_oracle_fp8.py checks the code table against the OCP format's defining values and
against torch's float8_e4m3fn conversions (a library routine), rounding ties, the scale rule's
closed forms, the error bound of round-to-nearest and the identity on representable rows.
"""
from __future__ import annotations

import math

import numpy as np

E4M3_MAX = 448.0
E8M0_BIAS = 127
MIN_EXP = -127          # smallest exponent an E8M0 byte holds (byte 0)


def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3 code, in float64 (NaN for S.1111.111).

    Normal codes (exponent field E in 1..15): (-1)^s (1 + m/8) 2^(E - 7); subnormal (E = 0):
    (-1)^s (m/8) 2^-6.
    """
    c = np.asarray(codes).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    E = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(E == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(E.astype(np.float64) - 7.0))
    out = s * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


def e4m3_encode(y) -> np.ndarray:
    """Nearest E4M3 code to each value of y (ties to the even code), for finite |y| <= 448."""
    y = np.asarray(y, dtype=np.float64)
    if not np.all(np.isfinite(y)) or np.any(np.abs(y) > E4M3_MAX):
        raise ValueError("e4m3_encode takes finite values with |y| <= 448")
    a = np.abs(y)
    codes = np.zeros(a.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    # Subnormal range: the grid is n 2^-9, n = 0..8 (n = 8 is the smallest normal, code 8).
    codes[sub] = np.rint(a[sub] * 2.0 ** 9).astype(np.int64)
    nrm = ~sub
    if np.any(nrm):
        mant, ex = np.frexp(a[nrm])            # a = mant 2^ex, mant in [0.5, 1)
        E = ex - 1                             # a = (2 mant) 2^E, 2 mant in [1, 2)
        n = np.rint((2.0 * mant - 1.0) * 8.0).astype(np.int64)   # 0..8; 8 carries into E
        codes[nrm] = ((E + 7) << 3) + n
    codes |= np.where(np.signbit(y), 0x80, 0)
    return codes.astype(np.uint8)


def row_exponent(amax: float) -> int:
    """Smallest integer e >= -127 with amax <= 448 * 2^e (0 for an all-zero row)."""
    amax = float(amax)
    if not math.isfinite(amax) or amax < 0:
        raise ValueError("row maximum must be finite and non-negative")
    if amax == 0.0:
        return 0
    e = math.ceil(math.log2(amax / E4M3_MAX))   # an estimate, corrected exactly below
    while amax > math.ldexp(E4M3_MAX, e):
        e += 1
    while e - 1 >= MIN_EXP and amax <= math.ldexp(E4M3_MAX, e - 1):
        e -= 1
    return max(e, MIN_EXP)


def quantize_rows(x, block: int = 1024) -> tuple[np.ndarray, np.ndarray]:
    """Row-wise E4M3 codes [R, C] (uint8) and E8M0 row exponents [R] (uint8, exponent + 127).
    Rows are independent; `block` rows are encoded per call only to bound the memory used."""
    x = np.asarray(x)
    if x.ndim != 2:
        raise ValueError("quantize_rows takes a matrix")
    R, C = x.shape
    codes = np.zeros((R, C), dtype=np.uint8)
    exps = np.zeros(R, dtype=np.uint8)
    for r0 in range(0, R, block):
        xb = np.asarray(x[r0:r0 + block], dtype=np.float64)
        amax = np.abs(xb).max(axis=1) if C else np.zeros(len(xb))
        e = np.array([row_exponent(a) for a in amax], dtype=np.int64)
        codes[r0:r0 + block] = e4m3_encode(np.ldexp(xb, -e[:, None]))
        exps[r0:r0 + block] = (e + E8M0_BIAS).astype(np.uint8)
    return codes, exps


def dequantize_rows(codes, exps) -> np.ndarray:
    """codes [R, C] and exps [R] back to float64 values: decode(code) 2^(exp - 127)."""
    v = e4m3_decode(codes)
    e = np.asarray(exps).astype(np.int64) - E8M0_BIAS
    return np.ldexp(v, e[:, None])
