"""The fp64 oracle against its pins (CPU only)."""
import numpy as np
import pytest
import torch

import _oracle_pins as pins
from oracle import paged_attention


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_sdpa_decode_both_dtypes(dtype):
    pins.pin_sdpa_decode_gqa(dtype=dtype)


def test_thread_count_does_not_change_bits():
    gen = torch.Generator().manual_seed(30)
    ctxs = [70, 3, 129, 64, 1]
    keys = [pins._randn(gen, c, 2, 16) for c in ctxs]
    values = [pins._randn(gen, c, 2, 16) for c in ctxs]
    kc, vc, bt, _ = pins.paged_from_contiguous(keys, values, 16, gen)
    q = pins._randn(gen, 5, 8, 16)
    cl = torch.tensor(ctxs, dtype=torch.int32)
    a = paged_attention(q, kc, vc, bt, cl, scale=0.25, threads=1)
    b = paged_attention(q, kc, vc, bt, cl, scale=0.25, threads=8)
    assert np.array_equal(a, b)


def test_row_subset_matches_full():
    gen = torch.Generator().manual_seed(31)
    ctxs = [20, 45]
    keys = [pins._randn(gen, c, 1, 8) for c in ctxs]
    values = [pins._randn(gen, c, 1, 8) for c in ctxs]
    kc, vc, bt, _ = pins.paged_from_contiguous(keys, values, 16, gen)
    q = pins._randn(gen, 2, 4, 8)
    cl = torch.tensor(ctxs, dtype=torch.int32)
    full = paged_attention(q, kc, vc, bt, cl, scale=0.5)
    rows = [7, 0, 5]
    sub = paged_attention(q, kc, vc, bt, cl, scale=0.5, rows=rows)
    for i, r in enumerate(rows):
        assert np.array_equal(sub[i], full[r // 4, r % 4])


@pytest.mark.parametrize("bad", ["block_id", "ctx_too_long", "qsl"])
def test_oracle_rejects_bad_inputs(bad):
    gen = torch.Generator().manual_seed(32)
    keys = [pins._randn(gen, 20, 1, 4)]
    kc, vc, bt, _ = pins.paged_from_contiguous(keys, keys, 16, gen)
    cl = torch.tensor([20], dtype=torch.int32)
    qsl = None
    if bad == "block_id":
        bt[0, 1] = kc.shape[0]
    elif bad == "ctx_too_long":
        cl[0] = bt.shape[1] * 16 + 1
    else:
        qsl = torch.tensor([1, 1], dtype=torch.int32)
    with pytest.raises(ValueError):
        paged_attention(pins._randn(gen, 1, 1, 4), kc, vc, bt, cl, qsl, scale=1.0)
