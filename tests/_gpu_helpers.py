"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI and compare it with
the fp64 oracle on the same seeded inputs."""
from __future__ import annotations

import numpy as np
import torch

from oracle import compare
from oracle import paged_attention as oracle_attention
from paged_kv_cache_168_amd import api
from paged_kv_cache_168_amd.workloads import Workload

# Tolerances against the fp64 oracle computed on the same (bf16-rounded) inputs; the rule itself is
# oracle.compare.check (within 1e-2, or one of the two bf16 values bracketing the oracle value; mean <= 2e-3).
FP32_MAX_ABS = compare.FP32_MAX_ABS
BF16_MAX_ABS = compare.BF16_MAX_ABS
BF16_MEAN_ABS = compare.BF16_MEAN_ABS


def device_inputs(wl, device="cuda"):
    d = dict(q=wl.q.to(device), k_cache=wl.k_cache.to(device), v_cache=wl.v_cache.to(device),
             block_tables=wl.block_tables.to(device), context_lens=wl.context_lens.to(device))
    if wl.query_start_loc is not None:
        d["query_start_loc"] = wl.query_start_loc.to(device)
    return d


def run_decode(wl, dev=None, **kw):
    dev = dev or device_inputs(wl)
    out = api.decode(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"], dev["context_lens"],
                     scale=wl.scale, **kw)
    torch.cuda.synchronize()
    return out


def run_mixed(wl, dev=None, **kw):
    dev = dev or device_inputs(wl)
    qsl = dev.get("query_start_loc")
    if qsl is None:
        qsl = torch.arange(wl.num_seqs + 1, dtype=torch.int32, device=dev["q"].device)
    out = api.varlen_mixed(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"], dev["context_lens"], qsl,
                           scale=wl.scale, max_query_len=max(1, wl.max_query_len), **kw)
    torch.cuda.synchronize()
    return out


def oracle(wl, rows=None):
    return oracle_attention(wl.q, wl.k_cache, wl.v_cache, wl.block_tables, wl.context_lens, wl.query_start_loc,
                            scale=wl.scale, rows=rows)


def as_f64(t):
    return t.detach().cpu().to(torch.float64).numpy()


def assert_close(got, want, dtype, what=""):
    """got: device/CPU tensor of the kernel's output dtype; want: float64 numpy oracle result."""
    return compare.check(as_f64(got).reshape(want.shape), want, dtype != torch.float32, what)


def poisoned(wl, value):
    """Copy of wl where every slot no request may read (tails of last blocks, spare and padding blocks)
    holds `value`."""
    k = wl.k_cache.clone()
    v = wl.v_cache.clone()
    NB, BS = k.shape[:2]
    live = torch.zeros(NB, BS, dtype=torch.bool)
    for s in range(wl.num_seqs):
        c = int(wl.context_lens[s])
        for i in range(c):
            live[int(wl.block_tables[s, i // BS]), i % BS] = True
    k[~live] = value
    v[~live] = value
    return Workload(wl.name, wl.q, k, v, wl.block_tables, wl.context_lens, wl.query_start_loc, wl.scale,
                    wl.poison_block, wl.meta)
