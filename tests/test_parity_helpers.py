"""CPU checks of the comparison rules themselves (tests/parity_helpers.py)."""

import numpy as np
import torch

from parity_helpers import assert_close, bf16_ulp


def test_bf16_ulp_is_the_spacing_of_bfloat16_values():
    assert bf16_ulp(1.0) == 2.0 ** -7
    assert bf16_ulp(0.5006) == 2.0 ** -8
    assert bf16_ulp(-3.0) == 2.0 ** -6
    assert bf16_ulp(0.0) == 0.0
    # against torch's own bfloat16 grid: the next value above a bfloat16 number
    x = torch.randn(1000, dtype=torch.float32).to(torch.bfloat16)
    up = torch.nextafter(x, torch.full_like(x, float("inf")))
    got = (up.double() - x.double()).abs().numpy()
    pos = x.double().numpy() > 0
    assert np.array_equal(got[pos], bf16_ulp(x.double().numpy())[pos])


def test_bf16_bound_is_the_stated_one_below_a_step():
    want = np.array([[0.1, -0.2, 0.15, 0.05]])
    rms = float(np.sqrt(np.mean(want ** 2)))
    ok = want + 0.019 * rms
    assert_close(torch.tensor(ok), want, torch.bfloat16, "within 2e-2 RMS")
    bad = want.copy()
    bad[0, 1] += 0.021 * rms
    try:
        assert_close(torch.tensor(bad), want, torch.bfloat16, "beyond 2e-2 RMS")
    except AssertionError:
        pass
    else:
        raise AssertionError("an error above 2e-2 * RMS passed")
    # a large element may be one bfloat16 step off, not two
    big = np.full((1, 64), 0.01)
    big[0, 0] = 8.0
    step = bf16_ulp(8.0)
    assert step > 0.02 * np.sqrt(np.mean(big ** 2))
    one, two = big.copy(), big.copy()
    one[0, 0] += step
    two[0, 0] += 2 * step
    assert_close(torch.tensor(one), big, torch.bfloat16, "one step")
    try:
        assert_close(torch.tensor(two), big, torch.bfloat16, "two steps")
    except AssertionError:
        pass
    else:
        raise AssertionError("two bfloat16 steps passed")
