"""Number formats of the decode step, written out from their definitions.

TEST INFRASTRUCTURE (see the package docstring): only tests, the smoke check
and the benchmark's CPU-baseline leg may import this module.

* OCP FP8 E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa
  bits; exponent field 0 encodes subnormals m/8 * 2^-6; codes 0x7F and 0xFF are
  NaN; there is no infinity, so the largest finite magnitude is 1.75 * 2^8 = 448.
  The TileRT pages name FP8 as the precision of their results (SemiAnalysis
  "Ultra-High Interactivity on NVIDIA GPUs? - TileRT InferenceX", results
  section) without fixing the variant; the OCP variant is the one with hardware
  conversions on the target GPU.
* bfloat16: the upper 16 bits of an IEEE binary32 value; rounding to it is
  round-to-nearest, ties to even, on an 8-bit significand.
* MXFP4 (OCP Microscaling formats v1.0): blocks of 32 consecutive elements
  of a row share one E8M0 scale, 2^(s - 127) for s = 0..254 (255 is NaN);
  each element is FP4 E2M1: 1 sign bit, 2 exponent bits with bias 1, 1
  mantissa bit; exponent field 0 encodes the subnormal m * 0.5, no infinity
  or NaN, largest magnitude 1.5 * 2^2 = 6. The pages quote their roofline at
  4-bit weights (SemiAnalysis TileRT page, introduction: NVFP4) and state
  that TileRT itself has no FP4 yet (results section); MXFP4 is the 4-bit
  block format with hardware conversions on the target GPU. Two elements
  share a byte: element 2j in the low nibble of byte j.
"""
from __future__ import annotations

import numpy as np

BLOCK = 128


def _e4m3_table() -> np.ndarray:
    t = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        exp = (code >> 3) & 0xF
        man = code & 0x7
        if exp == 0xF and man == 0x7:
            t[code] = np.nan
        elif exp == 0:
            t[code] = sign * (man / 8.0) * 2.0 ** -6
        else:
            t[code] = sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)
    return t


E4M3 = _e4m3_table()


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Values of e4m3 codes (uint8 array) as float64."""
    return E4M3[np.asarray(codes, dtype=np.uint8)]


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) to their exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value (ties to even).

    x = m * 2^e with 0.5 <= |m| < 1; a bf16 normal number keeps 8 significant
    bits, so m * 2^8 is rounded to an integer (half to even) and scaled back.
    Values below the bf16 normal range keep the subnormal spacing 2^-133.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    e = np.maximum(e, -125)          # smallest normal bf16 is 2^-126 = 0.5 * 2^-125
    q = np.rint(np.ldexp(x, 8 - e))  # np.rint rounds half to even
    return np.ldexp(q, e - 8)


def _e2m1_table() -> np.ndarray:
    t = np.empty(16, dtype=np.float64)
    for code in range(16):
        sign = -1.0 if code & 0x8 else 1.0
        exp = (code >> 1) & 0x3
        man = code & 0x1
        t[code] = sign * (man * 0.5 if exp == 0 else (1.0 + man / 2.0) * 2.0 ** (exp - 1))
    return t


E2M1 = _e2m1_table()
MX_BLOCK = 32


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    """Values of 4-bit e2m1 codes (integer array, 0..15) as float64."""
    return E2M1[np.asarray(codes, dtype=np.uint8) & 0xF]


def e8m0_decode(bits: np.ndarray) -> np.ndarray:
    """Values of e8m0 scale bytes: 2^(s - 127), NaN for 255."""
    b = np.asarray(bits, dtype=np.int64)
    return np.where(b == 255, np.nan, np.ldexp(1.0, b - 127))


def dequant_mxfp4(codes: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """W[i, j] = e2m1(nibble j of row i) * 2^(scale[i, j // 32] - 127) in
    float64; codes [N, K/2] hold element 2j in the low nibble of byte j."""
    c = np.asarray(codes, dtype=np.uint8)
    n, kh = c.shape
    nib = np.empty((n, 2 * kh), dtype=np.uint8)
    nib[:, 0::2] = c & 0xF
    nib[:, 1::2] = c >> 4
    s = np.repeat(e8m0_decode(scale_bits), MX_BLOCK, axis=1)
    return e2m1_decode(nib) * s


def dequant_fp8(codes: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """W[i, j] = e4m3(code[i, j]) * scale[i // 128, j // 128] in float64."""
    n, k = codes.shape
    s = bf16_bits_to_f64(scale_bits)
    s_full = np.repeat(np.repeat(s, BLOCK, axis=0)[:n], BLOCK, axis=1)[:, :k]
    return e4m3_decode(codes) * s_full
