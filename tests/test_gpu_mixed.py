"""GPU parity of pa_varlen_mixed (decodes plus causal chunked-prefill slices) against the oracle."""
from __future__ import annotations

import pytest
import torch

from _gpu_helpers import assert_close, oracle, poisoned, run_decode, run_mixed
from paged_kv_cache_168_amd import workloads as W

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("Hq,Hkv,D", [(32, 8, 128), (8, 8, 64), (16, 2, 128), (6, 2, 64)])
def test_mixed_small(dtype, Hq, Hkv, D):
    ctx = [40, 300, 1, 97, 700, 16]
    q_lens = [1, 37, 1, 97, 1, 16]
    wl = W.random_workload(1000 + Hq + D, ctx=ctx, q_lens=q_lens, Hq=Hq, Hkv=Hkv, D=D, BS=16, dtype=dtype)
    out = run_mixed(wl)
    assert_close(out, oracle(wl), dtype, f"mixed Hq={Hq} Hkv={Hkv} D={D}")


@pytest.mark.parametrize("BS,pt", [(16, 0), (16, 64), (32, 0), (1, 48), (7, 32)])
def test_mixed_block_sizes_partitions(BS, pt):
    ctx = [600, 3, 129, 64]
    q_lens = [65, 1, 129, 2]
    wl = W.random_workload(1100 + BS + pt, ctx=ctx, q_lens=q_lens, Hq=8, Hkv=2, D=128, BS=BS, dtype=torch.bfloat16)
    out = run_mixed(wl, partition_tokens=pt)
    assert_close(out, oracle(wl), torch.bfloat16, f"BS={BS} pt={pt}")


@pytest.mark.parametrize("BS,D", [(2, 128), (4, 128), (8, 128), (4, 64), (8, 64)])
def test_mixed_small_power_of_two_blocks(BS, D):
    """The chunk kernel's gather takes a block id per instruction when an instruction's key rows (4 at D 128, 8 at
    D 64) lie in one block, and each lane's row apart otherwise: block sizes on both sides of that bound."""
    ctx = [300, 3, 77, 64]
    q_lens = [130, 1, 77, 2]
    wl = W.random_workload(1150 + BS + D, ctx=ctx, q_lens=q_lens, Hq=8, Hkv=2, D=D, BS=BS, dtype=torch.bfloat16)
    out = run_mixed(wl)
    assert_close(out, oracle(wl), torch.bfloat16, f"BS={BS} D={D}")


def test_mixed_all_decode_equals_pa_decode():
    wl = W.random_workload(1200, ctx=[50, 900, 1, 4096], Hq=32, Hkv=8, D=128, BS=16, dtype=torch.bfloat16,
                           force_qsl=True)
    a = run_mixed(wl).cpu()
    wl_dec = W.Workload(wl.name, wl.q, wl.k_cache, wl.v_cache, wl.block_tables, wl.context_lens, None, wl.scale,
                        wl.poison_block)
    b = run_decode(wl_dec).cpu()
    assert torch.equal(a, b)


def _reorder(wl, order):
    """Same requests and pool, batch order permuted (query rows move with their request)."""
    qsl = wl.query_start_loc
    rows = torch.cat([torch.arange(int(qsl[s]), int(qsl[s + 1])) for s in order])
    q_lens = torch.tensor([int(qsl[s + 1] - qsl[s]) for s in order])
    new_qsl = torch.zeros(len(order) + 1, dtype=torch.int32)
    new_qsl[1:] = torch.cumsum(q_lens, 0).to(torch.int32)
    idx = torch.tensor(order)
    return W.Workload(wl.name, wl.q[rows], wl.k_cache, wl.v_cache, wl.block_tables[idx], wl.context_lens[idx],
                      new_qsl, wl.scale, wl.poison_block, dict(wl.meta))


def test_mixed_request_order_does_not_matter():
    """The chunk first, in the middle or last among the decodes: every request's rows stay the same
    (bit for bit for the chunk, within rounding for decode rows, whose balanced split depends on the
    batch)."""
    wl = W.mixed_step("first")
    S = wl.num_seqs
    base = run_mixed(wl).cpu()
    qsl = wl.query_start_loc
    for order in (list(range(1, 65)) + [0] + list(range(65, S)), list(range(1, S)) + [0], list(reversed(range(S)))):
        wl2 = _reorder(wl, order)
        out = run_mixed(wl2).cpu()
        q2 = wl2.query_start_loc
        for pos, s in enumerate(order):
            got = out[int(q2[pos]):int(q2[pos + 1])]
            want = base[int(qsl[s]):int(qsl[s + 1])]
            if int(qsl[s + 1] - qsl[s]) > 1:  # chunk rows: tiles are aligned to the request itself
                assert torch.equal(got, want), f"chunk request {s} changed when moved to position {pos}"
            else:  # decode rows: the balanced split moves with the batch, rounding may differ
                torch.testing.assert_close(got.float(), want.float(), atol=2e-2, rtol=0)


def test_future_keys_in_chunk_are_masked():
    """Huge values in keys/values beyond each chunk row's horizon must not leak into that row."""
    ctx, ql = 300, 120
    wl = W.random_workload(1300, ctx=[ctx], q_lens=[ql], Hq=8, Hkv=2, D=128, BS=16, dtype=torch.bfloat16)
    base = run_mixed(wl).cpu()
    k = wl.k_cache.clone()
    v = wl.v_cache.clone()
    # poison the last 60 keys of the chunk: rows j < ql - 60 must not change at all
    for i in range(ctx - 60, ctx):
        b = int(wl.block_tables[0, i // 16])
        k[b, i % 16] = 3e4
        v[b, i % 16] = 3e4
    wl2 = W.Workload(wl.name, wl.q, k, v, wl.block_tables, wl.context_lens, wl.query_start_loc, wl.scale,
                     wl.poison_block)
    pois = run_mixed(wl2).cpu()
    assert torch.equal(base[: ql - 60], pois[: ql - 60])


def test_config5_full_size_all_rows():
    wl = W.mixed_step()
    assert_close(run_mixed(wl), oracle(wl), torch.bfloat16, "config 5")


def test_mixed_workspace_contents_do_not_matter():
    """Mixed step with a poisoned (0xFF = NaN pattern) workspace: the same bits as a zeroed one."""
    from _gpu_helpers import device_inputs
    from paged_kv_cache_168_amd import api

    wl = W.random_workload(1300, ctx=[600, 3, 129, 5000, 64], q_lens=[65, 1, 129, 1, 2], Hq=32, Hkv=8, D=128,
                           BS=16, dtype=torch.bfloat16)
    dev = device_inputs(wl)
    p = api.make_params(dev["q"], dev["k_cache"], dev["block_tables"], scale=wl.scale)
    nbytes = api.varlen_mixed_workspace_size(p, wl.num_seqs, wl.num_tokens, wl.max_query_len)
    ref = run_mixed(wl, dev, workspace=torch.zeros(nbytes, dtype=torch.uint8, device="cuda")).cpu()
    got = run_mixed(wl, dev, workspace=torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")).cpu()
    assert torch.equal(ref, got)


# ---------------------------------------------------------------------------------------------
# chunked-prefill rows on the matrix cores: every supported GQA group size, tile remainders,
# full-prompt chunks, several chunks per step, partition sizes that cut 32-key steps
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (4, 2), (16, 4), (64, 8), (16, 1), (32, 1), (64, 1)])
def test_prefill_group_sizes(D, Hq, Hkv):
    G = Hq // Hkv
    bm = 64 // G  # query rows per work-group
    ctx = [bm + 1, 37, 1, 400, 2 * bm + 5, 90]
    q_lens = [bm + 1, 2, 1, bm - 1 if bm > 2 else 3, 2 * bm + 5, 1]  # full prompts and tile remainders
    wl = W.random_workload(1400 + G + D, ctx=ctx, q_lens=q_lens, Hq=Hq, Hkv=Hkv, D=D, BS=16, dtype=torch.bfloat16)
    out = run_mixed(wl)
    assert_close(out, oracle(wl), torch.bfloat16, f"prefill G={G} D={D}")


@pytest.mark.parametrize("pt", [16, 48, 96, 1024])
def test_prefill_partition_sizes(pt):
    wl = W.random_workload(1500 + pt, ctx=[1500, 1, 700, 64], q_lens=[300, 1, 700, 33], Hq=32, Hkv=8, D=128,
                           BS=16, dtype=torch.bfloat16)
    out = run_mixed(wl, partition_tokens=pt)
    assert_close(out, oracle(wl), torch.bfloat16, f"prefill pt={pt}")


def test_several_chunks_with_decodes():
    ctx = [2000, 5, 300, 1200, 17, 4096, 64]
    q_lens = [512, 1, 300, 77, 1, 1, 64]
    wl = W.random_workload(1600, ctx=ctx, q_lens=q_lens, Hq=32, Hkv=8, D=128, BS=32, dtype=torch.bfloat16)
    out = run_mixed(wl)
    assert_close(out, oracle(wl), torch.bfloat16, "several chunks")


@pytest.mark.parametrize("BS,D", [(16, 128), (5, 128), (4, 128), (4, 64), (8, 64)])
def test_prefill_unreferenced_slots_are_never_read_bit_exact(BS, D):
    """NaN and 1e30 in every slot no request may read give bit-identical, finite output for chunk rows."""
    wl = W.random_workload(1700 + BS + D, ctx=[130, 3, 47, 16], q_lens=[100, 1, 47, 2], Hq=16, Hkv=4, D=D, BS=BS,
                           dtype=torch.bfloat16)
    outs = [run_mixed(poisoned(wl, val)).cpu() for val in (float("nan"), 1e30, 0.0)]
    assert torch.isfinite(outs[0].float()).all()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


def test_prefill_relabelling_is_bit_exact():
    wl = W.random_workload(1800, ctx=[700, 1, 90], q_lens=[200, 1, 90], Hq=32, Hkv=8, D=128, BS=16,
                           dtype=torch.bfloat16)
    a = run_mixed(wl).cpu()
    g = torch.Generator().manual_seed(1801)
    pi = torch.randperm(wl.k_cache.shape[0], generator=g)
    k2 = torch.empty_like(wl.k_cache)
    v2 = torch.empty_like(wl.v_cache)
    k2[pi] = wl.k_cache
    v2[pi] = wl.v_cache
    bt2 = pi[wl.block_tables.long()].to(torch.int32)
    wl2 = W.Workload(wl.name, wl.q, k2, v2, bt2, wl.context_lens, wl.query_start_loc, wl.scale,
                     int(pi[wl.poison_block]))
    assert torch.equal(a, run_mixed(wl2).cpu())


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Hq,Hkv,ctx,q_len", [(32, 8, 2560, 512), (16, 16, 300, 300), (64, 8, 1000, 77),
                                              (8, 1, 130, 129)])
def test_single_request_chunk(D, Hq, Hkv, ctx, q_len):
    """A step with one request has no decode rows: its chunk runs alone, in the larger work-groups."""
    wl = W.random_workload(2000 + D + Hq + q_len, ctx=[ctx], q_lens=[q_len], Hq=Hq, Hkv=Hkv, D=D, BS=16,
                           dtype=torch.bfloat16)
    out = run_mixed(wl)
    assert_close(out, oracle(wl), torch.bfloat16, f"single chunk D={D} G={Hq // Hkv} q_len={q_len}")
    assert torch.equal(out.cpu(), run_mixed(wl).cpu())  # repeatable bit for bit
