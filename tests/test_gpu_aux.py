"""The caller-supplied auxiliary stream (pa_varlen_mixed_ex, pa_decode_shared_ex): with the caller's stream and
events the mixed step and the shared-prefix decode give the same bits as with the library's own auxiliary stream,
on repeated calls that share one pa_aux, and on a caller stream other than the default one; with the library's own
auxiliary stream, a host copy queued on the caller's stream right after a call sees the rows written there."""
from __future__ import annotations

import pytest
import torch

from _gpu_helpers import assert_close, device_inputs, oracle
from paged_kv_cache_168_amd import api
from paged_kv_cache_168_amd import workloads as W

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)


def _aux():
    return api.make_aux()  # a new stream and two events, kept alive by the returned object


def test_mixed_step_with_caller_aux():
    wl = W.random_workload(6000, ctx=[2560, 300, 5000, 1, 4096, 17], q_lens=[512, 1, 1, 1, 1, 17], Hq=32, Hkv=8,
                           D=128, BS=16, dtype=torch.bfloat16)
    dev = device_inputs(wl)
    args = (dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"], dev["context_lens"],
            dev["query_start_loc"])
    ref = api.varlen_mixed(*args, scale=wl.scale, max_query_len=wl.max_query_len)
    torch.cuda.synchronize()
    aux = _aux()
    main = torch.cuda.Stream()
    with torch.cuda.stream(main):
        outs = [api.varlen_mixed(*args, scale=wl.scale, max_query_len=wl.max_query_len, aux=aux, stream=main)
                for _ in range(3)]
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o.cpu(), ref.cpu())
    assert_close(ref, oracle(wl), torch.bfloat16, "mixed")


def test_shared_prefix_decode_with_caller_aux():
    wl = W.grouped_workload(6100, [(512, [512, 1024, 600, 2048, 100]), (0, [64, 3])], Hq=32, Hkv=8, D=128, BS=16)
    dev = device_inputs(wl)
    gs, gp = (x.cuda() for x in W.prefix_groups(wl))
    args = (dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"], dev["context_lens"], gs, gp)
    ref = api.decode_shared(*args, scale=wl.scale)
    aux = _aux()
    outs = [api.decode_shared(*args, scale=wl.scale, aux=aux) for _ in range(2)]
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o.cpu(), ref.cpu())
    assert_close(ref, oracle(wl), torch.bfloat16, "shared prefix")


def test_host_copy_on_callers_stream_sees_chunk_rows():
    """The chunk rows are written on the auxiliary stream and the library's own fork and join events carry no
    system-scope fence: a copy to pinned host memory queued on the caller's stream right after the call (no
    device synchronisation in between) must still see them, call after call into one output buffer."""
    kw = dict(ctx=[2560, 300, 5000, 1, 4096, 17], q_lens=[512, 1, 1, 1, 1, 17], Hq=32, Hkv=8, D=128, BS=16,
              dtype=torch.bfloat16)
    wls = [W.random_workload(6200 + i, **kw) for i in range(3)]
    devs = [device_inputs(wl) for wl in wls]
    refs = []
    for wl, dev in zip(wls, devs):
        refs.append(api.varlen_mixed(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"], dev["context_lens"],
                                     dev["query_start_loc"], scale=wl.scale, max_query_len=wl.max_query_len).cpu())
    torch.cuda.synchronize()
    main = torch.cuda.Stream()
    out = torch.empty_like(devs[0]["q"])
    hosts = [torch.empty(out.shape, dtype=out.dtype, pin_memory=True) for _ in wls]
    with torch.cuda.stream(main):
        for wl, dev, h in zip(wls, devs, hosts):
            api.varlen_mixed(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"], dev["context_lens"],
                             dev["query_start_loc"], scale=wl.scale, max_query_len=wl.max_query_len, out=out,
                             stream=main)
            h.copy_(out, non_blocking=True)
    main.synchronize()
    for h, ref in zip(hosts, refs):
        assert torch.equal(h, ref)
