"""The read-set gate on the GPU: every path, through the C ABI, on counting inputs (zero queries, one-hot V
markers of each key's logical position, ones in every slot no row may read), against the fp64 oracle. Rows whose
visible count is a power of two must equal the oracle bit for bit and every other element must be one of the two
bf16 values bracketing it, which a dropped, repeated or extra tile, piece or token fails (tests/_readset.py and
tests/test_readset_cpu.py give the construction and its sensitivity). Each case runs both marker schemes."""
from __future__ import annotations

import pytest
import torch

from _gpu_helpers import device_inputs, oracle, run_decode, run_mixed
from _readset import SCHEMES, check_counts, counting, counting_values, logical_positions, visible_counts
from oracle import paged_attention as oracle_attention
from paged_kv_cache_168_amd import api
from paged_kv_cache_168_amd import workloads as W

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

CTX = [1, 2, 3, 15, 16, 17, 31, 32, 33, 64, 100, 256, 1000, 1024, 2048, 4096, 5000, 8192]


def _gate(wl, run, what, need_exact=True, **kw):
    n = visible_counts(wl)
    for scheme in SCHEMES:
        cw = counting(wl, scheme)
        print(f"read-set gate: {what} ({scheme})", flush=True)
        got = run(cw, **kw)
        exact = check_counts(got, oracle(cw), n, f"{what} {scheme}")
        assert exact > 0 or not need_exact, "no power-of-two row in the case"


@pytest.mark.parametrize("Hq,Hkv,D,dtype,shared", [
    (32, 8, 128, torch.bfloat16, False),   # vector path, 4-head groups, streaming loads
    (32, 8, 128, torch.bfloat16, True),    # matrix cores, 4-head groups, cached loads
    (64, 8, 128, torch.bfloat16, False),   # matrix cores, 8-head groups, K/V through LDS
    (64, 8, 64, torch.bfloat16, True),     # matrix cores, 8-head groups, cached loads, D 64
    (16, 4, 64, torch.float32, False),     # fp32 vector path
    (8, 1, 128, torch.bfloat16, False),    # matrix cores, one KV head
    (6, 2, 128, torch.bfloat16, False),    # 3-head groups (one head per wave)
], ids=["g4-stream", "g4-shared", "g8-stream", "g8-shared-d64", "fp32", "g8-one-kv", "g3"])
def test_decode_paths(Hq, Hkv, D, dtype, shared):
    wl = W.random_workload(4000 + Hq + Hkv + D, ctx=CTX + [32768], Hq=Hq, Hkv=Hkv, D=D, BS=16, dtype=dtype)
    _gate(wl, run_decode, f"decode {Hq}:{Hkv} D{D} shared={shared}", shared_blocks=shared)


@pytest.mark.parametrize("BS,pt", [(5, 0), (5, 48), (8, 16), (32, 0), (48, 0)])
def test_decode_block_sizes(BS, pt):
    wl = W.random_workload(4100 + BS + pt, ctx=CTX, Hq=32, Hkv=8, D=128, BS=BS, dtype=torch.bfloat16)
    _gate(wl, run_decode, f"decode BS={BS} pt={pt}", partition_tokens=pt)


@pytest.mark.parametrize("pt", [0, 64, 512])
@pytest.mark.parametrize("Hq,Hkv", [(32, 8), (64, 8), (16, 16)])
def test_mixed_chunks_and_decodes(pt, Hq, Hkv):
    """Chunk rows on the matrix cores (full prompts give every power-of-two row count up to 1024) beside decodes
    (the concurrent path), with and without caller-set partitions."""
    ctx = [1024, 64, 4096, 300, 2560, 1, 17]
    q_lens = [1024, 1, 512, 1, 512, 1, 17]
    wl = W.random_workload(4200 + pt + Hq + Hkv, ctx=ctx, q_lens=q_lens, Hq=Hq, Hkv=Hkv, D=128, BS=16,
                           dtype=torch.bfloat16)
    _gate(wl, run_mixed, f"mixed {Hq}:{Hkv} pt={pt}", partition_tokens=pt)


@pytest.mark.parametrize("BS", [16, 5])
def test_single_chunk(BS):
    """One request alone: the serial path and the larger chunk work-groups."""
    wl = W.random_workload(4300 + BS, ctx=[2048], q_lens=[2048], Hq=32, Hkv=8, D=128, BS=BS, dtype=torch.bfloat16)
    _gate(wl, run_mixed, f"single chunk BS={BS}")


@pytest.mark.parametrize("Hq,Hkv,dtype,BS", [(16, 4, torch.float32, 16), (6, 2, torch.bfloat16, 16),
                                             (6, 2, torch.bfloat16, 5), (16, 4, torch.float32, 7)])
def test_partition_kernel_rows(Hq, Hkv, dtype, BS):
    """Chunk rows of shapes the matrix-core kernel does not take (fp32, 3-head groups) run on the partition
    kernel; at block sizes that are not a multiple of 16 the decode rows do too."""
    ctx = [1024, 64, 700, 1, 300]
    q_lens = [1024, 1, 100, 1, 1]
    wl = W.random_workload(4350 + Hq + BS, ctx=ctx, q_lens=q_lens, Hq=Hq, Hkv=Hkv, D=64, BS=BS, dtype=dtype)
    _gate(wl, run_mixed, f"partition kernel {Hq}:{Hkv} {dtype} BS={BS}")


def _shared_runner(gs, gp):
    def run(cw, **kw):
        dev = device_inputs(cw)
        out = api.decode_shared(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"], dev["context_lens"],
                                gs.cuda(), gp.cuda(), scale=cw.scale, **kw)
        torch.cuda.synchronize()
        return out
    return run


def test_shared_prefix_entry():
    groups = [(512, [512, 1024, 600, 2048, 100]), (0, [64, 3]), (1024, [1024 + 16 * i for i in range(12)] + [4096])]
    wl = W.grouped_workload(4400, groups, Hq=32, Hkv=8, D=128, BS=16)
    _gate(wl, _shared_runner(*W.prefix_groups(wl)), "pa_decode_shared")


def test_shared_prefix_over_several_partitions():
    """Prefixes of several 1024-key prefix partitions, with members shorter than the prefix."""
    groups = [(2560, [2560, 2600, 1500, 3000, 1025, 1024, 100, 2049]), (4096, [4100, 4097, 4111, 2048])]
    wl = W.grouped_workload(4450, groups, Hq=32, Hkv=8, D=128, BS=16)
    _gate(wl, _shared_runner(*W.prefix_groups(wl)), "pa_decode_shared long prefixes")


@pytest.mark.parametrize("beams", [True, False], ids=["beam-groups", "one-group"])
def test_full_size_prefix_shared_entry(beams):
    """The prefix-shared batch through pa_decode_shared as the benchmark runs it (beam groups) and as one group."""
    wl = W.prefix_shared()
    _gate(wl, _shared_runner(*W.prefix_groups(wl, beams)), f"pa_decode_shared beams={beams}", need_exact=False)


# ---------------------------------------------------------------------------------------------
# full-size workloads, in the launch configuration the benchmark uses
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["decode64", "long", "prefix", "mixed"])
def test_full_size(name):
    wl = W.WORKLOADS[name]()
    # the drawn contexts need not hold a power of two: every element is still held to the bracketing values
    if name == "mixed":
        _gate(wl, run_mixed, name, need_exact=False, partition_tokens=wl.meta.get("partition_tokens", 0))
    else:
        _gate(wl, run_decode, name, need_exact=False, partition_tokens=wl.meta.get("partition_tokens", 0),
              shared_blocks=bool(wl.meta.get("prefix_blocks")))


def test_262144_token_context():
    """One 262144-token request (16384 blocks at the top of a shuffled pool) beside short ones, on the matrix
    cores (64:8) and the vector path (32:8)."""
    for Hq, Hkv in ((64, 8), (32, 8)):
        ctx = [262144, 5, 1024]
        g = torch.Generator().manual_seed(4500 + Hq)
        nb = [-(-c // 16) for c in ctx]
        NB = sum(nb) + 8
        ids = torch.randperm(NB, generator=g)
        bt = torch.full((len(ctx), max(nb)), int(ids[-1]), dtype=torch.int32)
        cur = 0
        for s, n in enumerate(nb):
            bt[s, :n] = ids[cur:cur + n].to(torch.int32)
            cur += n
        cl = torch.tensor(ctx, dtype=torch.int32)
        k = torch.randn(NB, 16, Hkv, 128, generator=g).to(torch.bfloat16)
        pos = logical_positions(bt, cl, NB, 16)
        n = visible_counts(W.Workload("x", torch.zeros(3, Hq, 128), k, k, bt, cl, None, 0.1, 0))
        for scheme in SCHEMES:
            v = counting_values(pos, Hkv, 128, torch.bfloat16, scheme)
            q = torch.zeros(len(ctx), Hq, 128, dtype=torch.bfloat16)
            print(f"read-set gate: 262144 tokens {Hq}:{Hkv} ({scheme})", flush=True)
            out = api.decode(q.cuda(), k.cuda(), v.cuda(), bt.cuda(), cl.cuda(), scale=0.09)
            torch.cuda.synchronize()
            want = oracle_attention(q, k, v, bt, cl, scale=0.09)
            check_counts(out, want, n, f"262144 {Hq}:{Hkv} {scheme}")
            del v
