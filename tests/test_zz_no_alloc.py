"""pa_decode_noalloc (the decode entry point that allocates nothing: its scratch is the library's static array)
against pa_decode with a caller workspace, through the C ABI: bit-identical output on two calls in a row, the
second on a smaller batch, on the vector path, the matrix-core paths and a block size without the balanced
split; and a captured HIP graph of the call replayed several times, each replay checked against the eager
result."""
from __future__ import annotations

import pytest
import torch

from _gpu_helpers import assert_close, device_inputs, oracle, run_decode
from paged_kv_cache_168_amd import api
from paged_kv_cache_168_amd import workloads as W

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)


def _noalloc(wl, dev, out, **kw):
    api.decode_noalloc(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"], dev["context_lens"],
                       scale=wl.scale, out=out, **kw)
    torch.cuda.synchronize()
    return out.cpu()


@pytest.mark.parametrize("Hq,Hkv,BS,shared", [(32, 8, 16, False), (64, 8, 16, False), (32, 8, 16, True),
                                              (32, 8, 5, False)], ids=["vector", "mfma-g8", "shared", "bs5"])
def test_matches_pa_decode_on_two_calls(Hq, Hkv, BS, shared):
    big = W.random_workload(4600 + Hq + BS, ctx=[5000, 1, 700, 4096, 33, 2048, 17, 1024] * 4, Hq=Hq, Hkv=Hkv,
                            D=128, BS=BS, dtype=torch.bfloat16)
    small = W.random_workload(4700 + Hq + BS, ctx=[40, 3, 129], Hq=Hq, Hkv=Hkv, D=128, BS=BS,
                              dtype=torch.bfloat16)
    for wl in (big, small):  # the second call reuses the scratch the first one left behind
        print(f"noalloc {Hq}:{Hkv} BS={BS} shared={shared} S={wl.num_seqs}", flush=True)
        dev = device_inputs(wl)
        want = run_decode(wl, dev, shared_blocks=shared).cpu()
        out = torch.full_like(dev["q"], float("nan"))
        got = _noalloc(wl, dev, out, shared_blocks=shared)
        assert torch.equal(got, want)
        assert_close(got, oracle(wl), torch.bfloat16, "noalloc")


def test_full_size_long_context_then_small():
    """The 8 x 32768 long-context batch (the largest scratch of the benchmarked batches), then a small one."""
    for wl in (W.long_decode(), W.random_workload(4800, ctx=[100, 1], Hq=64, Hkv=8, D=128, BS=16)):
        print(f"noalloc {wl.name}", flush=True)
        dev = device_inputs(wl)
        want = run_decode(wl, dev).cpu()
        got = _noalloc(wl, dev, torch.empty_like(dev["q"]))
        assert torch.equal(got, want)


def test_graph_replays_match_eager():
    wl = W.random_workload(4900, ctx=[3000, 17, 900, 1, 4096], Hq=32, Hkv=8, D=128, BS=16, dtype=torch.bfloat16)
    dev = device_inputs(wl)
    eager = run_decode(wl, dev).cpu()
    out = torch.empty_like(dev["q"])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # one call before capture: the scratch address is looked up outside the graph
        api.decode_noalloc(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"], dev["context_lens"],
                           scale=wl.scale, out=out, stream=s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        api.decode_noalloc(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"], dev["context_lens"],
                           scale=wl.scale, out=out, stream=s)
    for i in range(4):
        out.fill_(float("nan"))
        other = run_decode(W.random_workload(4901 + i, ctx=[64, 9], Hq=32, Hkv=8, D=128, BS=16))  # eager work between
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.cpu(), eager), f"replay {i}"
        del other
