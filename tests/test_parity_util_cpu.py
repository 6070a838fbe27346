"""The helpers the GPU parity tests compare with, pinned on the CPU."""
import numpy as np
import pytest
import torch

from parity_util import assert_bf16_rows_match, bf16_ulps, rel_l2


def _bf16(x):
    return torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).float().numpy().astype(np.float64)


def test_bf16_ulps_counts_representable_steps():
    one = _bf16([1.0])
    nxt = _bf16([1.0 + 2.0 ** -7])          # the bf16 number after 1.0
    assert bf16_ulps(one, nxt)[0] == 1
    assert bf16_ulps(nxt, one)[0] == 1
    assert bf16_ulps(_bf16([0.0]), _bf16([-0.0]))[0] == 0
    tiny = 2.0 ** -133                       # smallest positive bf16 subnormal
    assert bf16_ulps(np.array([tiny]), np.array([-tiny]))[0] == 2
    # a step across a power of two: the largest bf16 below 2 and 2 itself
    assert bf16_ulps(_bf16([2.0 - 2.0 ** -7]), _bf16([2.0]))[0] == 1
    # torch's own successor relation over many random values
    v = torch.randn(4096).to(torch.bfloat16)
    succ = torch.nextafter(v.float(), torch.full_like(v.float(), float("inf"))).to(torch.bfloat16)
    # nextafter in fp32 then rounding to bf16 may land on v itself; step the bit pattern instead
    bits = v.view(torch.int16).numpy().astype(np.int64)
    up = np.where(bits >= 0, bits + 1, bits - 1)
    up_vals = torch.from_numpy(up.astype(np.int16)).view(torch.bfloat16).float().numpy().astype(np.float64)
    finite = np.isfinite(up_vals) & (v.float().numpy() != 0)
    d = bf16_ulps(v.float().numpy().astype(np.float64)[finite], up_vals[finite])
    assert (d == 1).all()
    del succ


def test_row_match_accepts_one_step_and_rejects_two():
    rng = np.random.default_rng(3)
    want = _bf16(rng.standard_normal(576))
    bits = torch.from_numpy(want.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().astype(np.int64)
    one = bits.copy()
    one[[5, 77]] += 1
    got = torch.from_numpy(one.astype(np.int16)).view(torch.bfloat16).float().numpy().astype(np.float64)
    assert assert_bf16_rows_match(got, want) == 2
    two = bits.copy()
    two[9] += 2
    got2 = torch.from_numpy(two.astype(np.int16)).view(torch.bfloat16).float().numpy().astype(np.float64)
    with pytest.raises(AssertionError):
        assert_bf16_rows_match(got2, want)
    with pytest.raises(AssertionError):   # not bf16 values at all
        bf16_ulps(want + 1e-9, want)
    # near zero several steps are allowed within the absolute slack, not beyond
    z = want.copy()
    z[3] = _bf16([3e-6])[0]
    zg = z.copy()
    zg[3] = _bf16([3e-6 + 5e-6])[0]           # many bf16 steps, 5e-6 of a unit-rms row
    assert bf16_ulps(zg, z)[3] > 1
    assert_bf16_rows_match(zg, z)
    zg[3] = _bf16([3e-6 + 5e-3])[0]
    with pytest.raises(AssertionError):
        assert_bf16_rows_match(zg, z)


def test_rel_l2():
    a = np.array([3.0, 4.0])
    assert rel_l2(a, a) == 0.0
    assert rel_l2(a * 1.01, a) == pytest.approx(0.01)
