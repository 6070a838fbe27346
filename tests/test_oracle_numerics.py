"""Pins of the oracle's number formats against library casts and brute force."""
import numpy as np
import pytest
import torch

import oracle as O
from oracle import numerics as N
from synth import gen


def test_e4m3_table_matches_torch_float8():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = O.e4m3_decode(np.arange(256, dtype=np.uint8))
    nan_ref, nan_mine = np.isnan(ref), np.isnan(mine)
    assert (nan_ref == nan_mine).all()
    assert sorted(np.nonzero(nan_mine)[0].tolist()) == [0x7F, 0xFF]
    np.testing.assert_array_equal(mine[~nan_mine], ref[~nan_ref])


def test_e4m3_anchor_values():
    t = N.E4M3
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0          # largest finite
    assert t[0x38] == 1.0 and t[0xB8] == -1.0               # exponent field 7 = bias
    assert t[0x08] == 2.0 ** -6                              # smallest normal
    assert t[0x01] == 2.0 ** -9                              # smallest subnormal
    assert t[0x00] == 0.0 and t[0x80] == 0.0 and np.signbit(t[0x80])
    finite = t[np.isfinite(t)]
    assert np.nanmax(np.abs(finite)) == 448.0


def test_bf16_bits_roundtrip_torch():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 1 << 16, size=100000, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    mine = O.bf16_bits_to_f64(bits)
    same = (mine == ref) | (np.isnan(mine) & np.isnan(ref))
    assert same.all()


def test_bf16_round_matches_torch_rne():
    rng = np.random.default_rng(2)
    x = np.concatenate([
        rng.standard_normal(400000).astype(np.float32),
        (rng.standard_normal(200000) * 1e-30).astype(np.float32),
        (rng.standard_normal(200000) * 1e20).astype(np.float32),
    ])
    # exact ties: a bf16 value plus half of its ulp, both parities of the last kept bit
    base = rng.integers(0x3000, 0x5000, size=20000).astype(np.uint32) << 16
    ties = (base | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    mine = O.bf16_round(x.astype(np.float64))
    np.testing.assert_array_equal(mine, ref)


def test_dequant_is_exact_in_fp32():
    """Code value times bf16 scale needs at most 4 + 8 significant bits: fp32 holds it exactly."""
    codes = np.arange(256, dtype=np.uint8)
    finite = np.isfinite(N.E4M3[codes])
    rng = np.random.default_rng(3)
    scales = rng.integers(0x3800, 0x3D00, size=64, dtype=np.uint16)
    v32 = N.E4M3[codes][finite].astype(np.float32)
    for s in scales:
        s32 = O.bf16_bits_to_f64(np.array([s]))[0].astype(np.float32)
        p32 = (v32 * s32).astype(np.float64)
        p64 = N.E4M3[codes][finite] * float(s32)
        np.testing.assert_array_equal(p32, p64)


def test_dequant_block_indexing_bruteforce():
    rng = np.random.default_rng(4)
    n, k = 131, 260
    codes = rng.integers(0, 0x7E, size=(n, k), dtype=np.uint8)
    scales = rng.integers(0x3C00, 0x3D00, size=(2, 3), dtype=np.uint16)
    W = O.dequant_fp8(codes, scales)
    sv = O.bf16_bits_to_f64(scales)
    for i in range(0, n, 13):
        for j in range(0, k, 7):
            assert W[i, j] == N.E4M3[codes[i, j]] * sv[i // 128, j // 128]


def test_generator_quantiser_is_nearest_e4m3():
    """The storage-form codes are the round-to-nearest-even e4m3 of w/scale (brute force)."""
    g = torch.Generator().manual_seed(5)
    w = torch.randn(256, 384, generator=g) * 0.02
    w[3, 5] = 0.0
    codes, sbits = gen.quantize_blocks(w)
    codes = codes.numpy()
    s = O.bf16_bits_to_f64(sbits.numpy().view(np.uint16))
    sfull = np.repeat(np.repeat(s, 128, 0), 128, 1)
    target = np.clip(w.double().numpy() / sfull, -448, 448)
    finite_codes = np.array([c for c in range(256) if np.isfinite(N.E4M3[c])])
    vals = N.E4M3[finite_codes]
    flat_t = target.reshape(-1)[:20000]
    flat_c = codes.reshape(-1)[:20000]
    dist = np.abs(flat_t[:, None] - vals[None, :])
    best = dist.min(axis=1)
    got = np.abs(flat_t - N.E4M3[flat_c])
    # chosen code is a nearest one; among equally near, the even mantissa
    assert np.all(got <= best * (1 + 1e-12) + 1e-300)
    # block scale is bf16(amax / 448)
    amax = np.abs(w.double().numpy()).reshape(2, 128, 3, 128).max(axis=(1, 3))
    np.testing.assert_array_equal(s, O.bf16_round(amax / 448.0))


def test_quantiser_ties_to_even():
    # 1.0625 lies halfway between e4m3 1.0 (mantissa 0) and 1.125 (mantissa 1): even wins.
    w = torch.zeros(128, 128)
    w[0, 0] = 448.0 * 1.0 / 1.0  # fixes the block amax so the scale is exactly 1
    w[0, 1] = 1.0625
    w[0, 2] = 1.1875  # halfway between 1.125 (odd) and 1.25 (even)
    codes, sbits = gen.quantize_blocks(w)
    assert O.bf16_bits_to_f64(sbits.numpy().view(np.uint16))[0, 0] == 1.0
    assert N.E4M3[codes[0, 1].item()] == 1.0
    assert N.E4M3[codes[0, 2].item()] == 1.25


# --- MXFP4 (OCP Microscaling v1.0: e2m1 elements, e8m0 block scales of 32)

def _e2m1_as_e4m3_code(c: int) -> int:
    """The e4m3 code of the same value: e2m1 is (sign, exponent bias 1,
    1 mantissa bit), e4m3 (sign, exponent bias 7, 3 mantissa bits). Normal
    e2m1 values move the exponent field by +6 and the mantissa bit to the top
    of the 3-bit field; the e2m1 subnormal 0.5 is the e4m3 normal 2^-1."""
    sign, exp, man = (c >> 3) & 1, (c >> 1) & 3, c & 1
    if exp == 0:
        mag = 0 if man == 0 else (6 << 3)
    else:
        mag = ((exp + 6) << 3) | (man << 2)
    return (sign << 7) | mag


def test_e2m1_table_matches_torch_float8_values():
    # every e2m1 value is an e4m3 value: decode its e4m3 twin with torch
    twins = torch.tensor([_e2m1_as_e4m3_code(c) for c in range(16)], dtype=torch.int32).to(torch.uint8)
    ref = twins.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.e2m1_decode(np.arange(16)), ref)


def test_e2m1_invariants():
    t = N.E2M1
    assert t.shape == (16,) and np.isfinite(t).all()              # no inf / NaN codes
    np.testing.assert_array_equal(t[8:], -t[:8])                   # sign bit
    assert np.signbit(t[8]) and t[8] == 0.0
    mags = t[:8]
    assert (np.diff(mags) > 0).all() and mags.max() == 6.0         # monotone, largest 1.5 * 2^2
    assert t[1] == 0.5 and t[2] == 1.0                             # subnormal step, exponent bias 1
    # every magnitude is a multiple of the subnormal step 0.5 and below 8
    assert (np.mod(mags, 0.5) == 0).all()


def test_e8m0_scales():
    np.testing.assert_array_equal(O.e8m0_decode(np.array([127, 128, 126, 0, 254])),
                                  [1.0, 2.0, 0.5, 2.0 ** -127, 2.0 ** 127])
    assert np.isnan(O.e8m0_decode(np.array([255]))[0])


def test_mxfp4_dequant_bruteforce():
    rng = np.random.default_rng(3)
    n, k = 5, 96
    codes = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    scales = rng.integers(100, 140, size=(n, k // 32), dtype=np.uint8)
    got = O.dequant_mxfp4(codes, scales)
    for i in range(n):
        for j in range(k):
            byte = int(codes[i, j // 2])
            nib = byte & 0xF if j % 2 == 0 else byte >> 4
            sign = -1.0 if nib & 8 else 1.0
            e, m = (nib >> 1) & 3, nib & 1
            v = sign * (m / 2.0 if e == 0 else (1 + m / 2.0) * 2.0 ** (e - 1))
            assert got[i, j] == v * 2.0 ** (int(scales[i, j // 32]) - 127), (i, j)


def test_generator_mxfp4_quantiser_is_nearest():
    """The storage-form MXFP4 codes are a nearest e2m1 value of w / scale
    (ties to the even code), with scale 2^(floor(log2(block amax)) - 2)."""
    g = torch.Generator().manual_seed(7)
    w = torch.randn(64, 256, generator=g) * 0.02
    w[0, :32] = 0.0                       # an all-zero block
    w[1, 0], w[1, 1] = 6.0 * 2.0 ** -5, 5.0 * 2.0 ** -5   # 5 is halfway between 4 and 6: even code (4)
    codes, scales = gen.quantize_mxfp4(w)
    codes, scales = codes.numpy(), scales.numpy()
    deq = O.dequant_mxfp4(codes, scales)
    s = O.e8m0_decode(np.repeat(scales, 32, axis=1))
    wd = w.double().numpy()
    amax = np.abs(wd).reshape(64, 8, 32).max(axis=2)
    nz = amax > 0
    np.testing.assert_array_equal(scales[nz].astype(np.int64) - 127, np.floor(np.log2(amax[nz])) - 2)
    target = np.clip(wd / s, -6, 6)
    dist = np.abs(target.reshape(-1)[:, None] - N.E2M1[None, :])
    got = np.abs(target.reshape(-1) - deq.reshape(-1) / s.reshape(-1))
    assert np.all(got <= dist.min(axis=1) * (1 + 1e-12) + 1e-300)
    assert deq[1, 0] == 6.0 * 2.0 ** -5 and deq[1, 1] == 4.0 * 2.0 ** -5
    assert (deq[0, :32] == 0).all()
