"""GPU parity of pa_decode_shared (decode whose requests share prefix blocks: the prefix keys read once per
group on the matrix cores, each request's suffix on the decode kernel, joined by the log-sum-exp merge)
against the fp64 oracle, which reads every request through its own table."""
from __future__ import annotations

import pytest
import torch

from _gpu_helpers import assert_close, device_inputs, oracle, poisoned, run_decode
from paged_kv_cache_168_amd import api
from paged_kv_cache_168_amd import workloads as W

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)


def run_shared(wl, dev=None, beams=True, **kw):
    dev = dev or device_inputs(wl)
    gs, gp = W.prefix_groups(wl, beams)
    return api.decode_shared(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"], dev["context_lens"],
                             gs.cuda(), gp.cuda(), scale=wl.scale, **kw)


# groups: prefix tokens and member context lengths (members shorter than the prefix, equal to it, one token
# past it, singletons, a group without a prefix, a group whose first request is shorter than the declared
# prefix, which cuts the prefix to its context)
GROUPS_16 = [(512, [512, 513, 900, 2000, 17, 1030, 600, 512 + 16]), (0, [40, 3]), (64, [64]), (256, [300, 100]),
             (1024, [1024 + 5 * i for i in range(20)]), (512, [200, 700, 520])]
GROUPS_32 = [(512, [513, 700, 1600, 64]), (96, [96, 97, 128, 5])]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", [(32, 8), (64, 8), (16, 16)])
def test_groups_match_oracle(D, Hq, Hkv):
    wl = W.grouped_workload(1700 + D + Hq, GROUPS_16, Hq=Hq, Hkv=Hkv, D=D, BS=16)
    assert_close(run_shared(wl), oracle(wl), torch.bfloat16, f"{Hq}:{Hkv} D={D}")


# prefixes longer than one prefix partition (1024 keys): members longer than the prefix, shorter than it (they see
# fewer partitions of it), ending exactly on a partition bound, and a whole group of beams
GROUPS_LONG = [(2560, [2560, 2600, 1500, 3000, 1025, 1024, 100, 2049]), (1040, [1100, 1041, 1040]),
               (4096, [4100, 4097, 4100, 4111])]


@pytest.mark.parametrize("Hq,Hkv", [(32, 8), (64, 8)])
def test_prefixes_over_several_partitions(Hq, Hkv):
    wl = W.grouped_workload(1750 + Hq, GROUPS_LONG, Hq=Hq, Hkv=Hkv, D=128, BS=16)
    out = run_shared(wl)
    assert_close(out, oracle(wl), torch.bfloat16, f"long prefixes {Hq}:{Hkv}")
    dev = device_inputs(wl)
    ref = run_decode(wl, dev)
    assert (out.cpu().float() - ref.cpu().float()).abs().max().item() <= 1e-2


@pytest.mark.parametrize("BS,D", [(48, 128), (48, 64), (64, 128)])
def test_prefix_pass_block_sizes(BS, D):
    """The prefix pass takes a block id per gather instruction for power-of-two blocks and each lane's row apart
    for other sizes (48 tokens), including a prefix longer than one 1024-key partition."""
    groups = [(24 * BS, [24 * BS, 24 * BS + 3, 300, 17, 30 * BS]), (3 * BS, [3 * BS + 1, 50, 3 * BS])]
    wl = W.grouped_workload(1770 + BS + D, groups, Hq=16, Hkv=4, D=D, BS=BS)
    assert_close(run_shared(wl), oracle(wl), torch.bfloat16, f"BS={BS} D={D}")


@pytest.mark.parametrize("shared", [False, True])
def test_block_size_32_and_cached_loads(shared):
    wl = W.grouped_workload(1800, GROUPS_32, Hq=32, Hkv=8, D=128, BS=32)
    assert_close(run_shared(wl, shared_blocks=shared), oracle(wl), torch.bfloat16, f"BS=32 shared={shared}")


def test_stale_slots_are_never_read_bit_exact():
    wl = W.grouped_workload(1900, GROUPS_16, Hq=32, Hkv=8, D=128, BS=16)
    outs = [run_shared(poisoned(wl, v)).cpu() for v in (float("nan"), 1e30, 0.0)]
    assert torch.isfinite(outs[0].float()).all()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


def test_repeatable_and_workspace_contents_do_not_matter():
    wl = W.grouped_workload(2000, GROUPS_16, Hq=32, Hkv=8, D=128, BS=16)
    dev = device_inputs(wl)
    p = api.make_params(dev["q"], dev["k_cache"], dev["block_tables"], scale=wl.scale)
    n = api.decode_shared_workspace_size(p, wl.num_seqs, len(GROUPS_16))
    a = run_shared(wl, dev, workspace=torch.zeros(n, dtype=torch.uint8, device="cuda")).cpu()
    b = run_shared(wl, dev, workspace=torch.full((n,), 0xFF, dtype=torch.uint8, device="cuda")).cpu()
    assert torch.equal(a, b)


def test_fp32_runs_as_plain_decode():
    wl = W.grouped_workload(2100, GROUPS_32, Hq=8, Hkv=2, D=64, BS=32, dtype=torch.float32)
    dev = device_inputs(wl)
    assert torch.equal(run_shared(wl, dev).cpu(), run_decode(wl, dev).cpu())


@pytest.mark.parametrize("beams", [True, False], ids=["beam-groups", "one-group"])
def test_prefix_shared_batch_full_size(beams):
    """The 256-request batch whose requests share a 512-token prefix (16 groups of 4 beams among them), described
    as its 16 beam groups plus one group of the rest, or as one group of all 256 requests; every row against the
    oracle, and within the tolerance of pa_decode."""
    wl = W.prefix_shared()
    dev = device_inputs(wl)
    out = run_shared(wl, dev, beams, shared_blocks=True)
    assert_close(out, oracle(wl), torch.bfloat16, "config 4")
    ref = run_decode(wl, dev, shared_blocks=True)
    assert (out.float() - ref.float()).abs().max().item() <= 1e-2
