"""GPU parity for the balanced decode's slicing at full wave counts: batches whose 1024 waves each hold
several short segments, so that slice bounds fall at every position of a segment's cost (including the
charge before its first tile), next to batches that mix one-token and long contexts. Each case against the
fp64 oracle; the cases print their seeds first."""
from __future__ import annotations

import random

import pytest
import torch

from _gpu_helpers import assert_close, oracle, run_decode, run_mixed
from paged_kv_cache_168_amd import workloads as W

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)


def _short_ctx(seed, n, hi):
    r = random.Random(seed)
    return [r.randint(1, hi) for _ in range(n)]


@pytest.mark.parametrize("seed,n,hi", [(7100, 512, 48), (7101, 768, 16), (7102, 300, 40)])
def test_many_short_segments_bf16(seed, n, hi):
    # 32 query / 8 KV heads: four-head groups on the vector path, 8 segments of 1-3 tiles per request
    ctx = _short_ctx(seed, n, hi)
    print(f"short bf16 seed={seed} n={n} max_ctx={hi}", flush=True)
    wl = W.random_workload(seed, ctx=ctx, Hq=32, Hkv=8, D=128, BS=16, dtype=torch.bfloat16)
    assert_close(run_decode(wl), oracle(wl), torch.bfloat16, f"seed {seed}")


def test_many_short_segments_fp32():
    seed = 7110
    ctx = _short_ctx(seed, 400, 40)
    print(f"short fp32 seed={seed}", flush=True)
    wl = W.random_workload(seed, ctx=ctx, Hq=16, Hkv=4, D=64, BS=16, dtype=torch.float32)
    assert_close(run_decode(wl), oracle(wl), torch.float32, f"seed {seed}")


@pytest.mark.parametrize("seed", [7120, 7121])
def test_alternating_short_and_long(seed):
    r = random.Random(seed)
    ctx = [r.choice([1, r.randint(2, 20), r.randint(1500, 4096)]) for _ in range(96)]
    print(f"alternating seed={seed}", flush=True)
    wl = W.random_workload(seed, ctx=ctx, Hq=32, Hkv=8, D=128, BS=16, dtype=torch.bfloat16)
    assert_close(run_decode(wl), oracle(wl), torch.bfloat16, f"seed {seed}")


def test_short_segments_block32_mixed_step():
    # decodes of 1-3 tiles beside two chunk slices, through the mixed entry point
    seed = 7130
    r = random.Random(seed)
    ctx = [r.randint(1, 48) for _ in range(256)] + [700, 1200]
    q_lens = [1] * 256 + [64, 300]
    print(f"mixed short seed={seed}", flush=True)
    wl = W.random_workload(seed, ctx=ctx, q_lens=q_lens, Hq=32, Hkv=8, D=128, BS=32, dtype=torch.bfloat16,
                           force_qsl=True)
    assert_close(run_mixed(wl), oracle(wl), torch.bfloat16, f"seed {seed}")
