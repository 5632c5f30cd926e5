"""The parity helper's bf16 rule (CPU): the max bound applies beyond the output's own bf16 rounding, the
mean bound as is; the fp32 rule is a plain max bound."""
import numpy as np
import pytest
import torch

from _gpu_helpers import assert_close


def _bf16(x):
    return torch.from_numpy(x).to(torch.float32).to(torch.bfloat16)


def test_correctly_rounded_large_outputs_pass():
    want = np.random.default_rng(0).normal(0.0, 0.1, 4096)
    want[:3] = [-4.137332183260504, 5.9, 4.4]
    got = _bf16(want)
    assert np.abs(got.double().numpy() - want).max() > 1e-2  # the rounding alone exceeds the plain bound
    assert_close(got, want, torch.bfloat16)


def test_error_beyond_rounding_fails():
    want = np.full(256, 0.3, dtype=np.float64)
    got = _bf16(want + 0.0125)  # more than 1e-2 beyond the rounding of 0.3
    with pytest.raises(AssertionError):
        assert_close(got, want, torch.bfloat16)


def test_mean_bound_applies():
    want = np.linspace(-1.0, 1.0, 4096)
    got = _bf16(want + 0.0025)  # within the max bound everywhere, mean error above 2e-3
    with pytest.raises(AssertionError, match="mean"):
        assert_close(got, want, torch.bfloat16)


def test_fp32_plain_bound():
    want = np.linspace(-5.0, 5.0, 1000)
    assert_close(torch.from_numpy(want).float(), want, torch.float32)
    with pytest.raises(AssertionError):
        assert_close(torch.from_numpy(want + 2e-4).float(), want, torch.float32)
