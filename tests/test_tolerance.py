"""The parity comparison rule (CPU): a bf16 element passes within 1e-2 of the oracle value or as one of the two
bf16 values bracketing it; the mean bound applies as is; the fp32 rule is a plain max bound."""
import numpy as np
import pytest
import torch

from _gpu_helpers import assert_close
from oracle.compare import bf16_round_down_up


def _bf16(x):
    return torch.from_numpy(x).to(torch.float32).to(torch.bfloat16)


def test_correctly_rounded_large_outputs_pass():
    want = np.random.default_rng(0).normal(0.0, 0.1, 4096)
    want[:3] = [-4.137332183260504, 5.9, 4.4]
    got = _bf16(want)
    assert np.abs(got.double().numpy() - want).max() > 1e-2  # the rounding alone exceeds the plain bound
    assert_close(got, want, torch.bfloat16)


def test_other_bracketing_value_passes_but_the_next_one_fails():
    """At |o| in [4, 8) the bf16 spacing is 2^-5: the bf16 value on the far side of o passes (an fp32 result
    that rounds the other way), one step further does not."""
    o = np.array([4.4 + 0.003])
    lo, hi = bf16_round_down_up(o)
    assert hi - lo == 2.0 ** -5
    rest = np.linspace(-1.0, 1.0, 1023)  # exact bf16 values around the element, so the mean stays small
    rest = _bf16(rest).double().numpy()
    want = np.concatenate([o, rest])
    for g in (lo, hi, hi + 2.0 ** -5):
        got = _bf16(np.concatenate([g, rest]))
        if g[0] <= hi[0]:
            assert_close(got, want, torch.bfloat16)
        else:
            with pytest.raises(AssertionError, match="bf16 neighbour"):
                assert_close(got, want, torch.bfloat16)


def test_error_just_past_the_bound_fails_even_where_the_output_rounds():
    """o = 0.3 (bf16 rounding error 7.8e-4) with an output 0.0105 away: within 1e-2 of kernel error on top of
    the rounding (the additive reading would pass it), but neither within 1e-2 nor a bracketing value."""
    want = np.full(256, 0.3, dtype=np.float64)
    got = _bf16(want + 0.0105)
    err = float(got.double()[0]) - 0.3
    rounding = abs(float(_bf16(want)[0].double()) - 0.3)
    assert err > 1e-2 and err - rounding <= 1e-2  # passes the additive reading
    with pytest.raises(AssertionError):
        assert_close(got, want, torch.bfloat16)


def test_error_beyond_rounding_fails():
    want = np.full(256, 0.3, dtype=np.float64)
    got = _bf16(want + 0.0125)
    with pytest.raises(AssertionError):
        assert_close(got, want, torch.bfloat16)


def test_mean_bound_applies():
    want = np.linspace(-1.0, 1.0, 4096)
    got = _bf16(want + 0.0025)  # within the max bound everywhere, mean error above 2e-3
    with pytest.raises(AssertionError, match="mean"):
        assert_close(got, want, torch.bfloat16)


def test_non_finite_output_fails():
    want = np.zeros(8)
    got = _bf16(want)
    got[3] = float("nan")
    with pytest.raises(AssertionError, match="non-finite"):
        assert_close(got, want, torch.bfloat16)


def test_bracket_is_tight_on_random_values():
    rng = np.random.default_rng(1)
    o = np.concatenate([rng.normal(0.0, 3.0, 50000), rng.normal(0.0, 1e-3, 2000), [0.0, 1.0, -2.0 ** -7]])
    lo, hi = bf16_round_down_up(o)
    assert np.all(lo <= o) and np.all(hi >= o)
    for x in (lo, hi):  # both are bf16 values
        assert np.array_equal(torch.from_numpy(x).float().to(torch.bfloat16).double().numpy(), x)
    rne = torch.from_numpy(o).float().to(torch.bfloat16).double().numpy()
    assert np.all((rne == lo) | (rne == hi))
    exact = np.isin(o, [0.0, 1.0, -2.0 ** -7])
    assert np.all(lo[exact] == hi[exact])


def test_fp32_plain_bound():
    want = np.linspace(-5.0, 5.0, 1000)
    assert_close(torch.from_numpy(want).float(), want, torch.float32)
    with pytest.raises(AssertionError):
        assert_close(torch.from_numpy(want + 2e-4).float(), want, torch.float32)
