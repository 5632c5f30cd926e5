"""The C ABI library: loads, exports every declared symbol, validates arguments (CPU only:
every call here returns before any HIP call)."""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest
import torch

from paged_kv_cache_168_amd import api
from paged_kv_cache_168_amd.engine import ENGINE_SYMBOLS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pa.h")

OK, NULLP, INVALID, UNSUPPORTED, WS_SMALL, HIP = 0, 1, 2, 3, 4, 5


def declared_functions():
    names = set()
    for h in sorted(os.listdir(os.path.dirname(HEADER))):
        text = open(os.path.join(os.path.dirname(HEADER), h)).read()
        names |= set(re.findall(r"^\s*(?:const\s+char\*|size_t|pa_status|void)\s+(pa_\w+)\s*\(", text, re.M))
    return sorted(names)


def params(**kw):
    base = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16, num_blocks=1000, max_blocks_per_seq=256,
                dtype=1, scale=0.088, partition_tokens=0, flags=0)
    base.update(kw)
    return api.PaParams(**base)


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every case below fails validation first


def decode_status(p, num_seqs=4, ws=None, ws_bytes=0, ptrs=None):
    lib = api.library()
    ptrs = ptrs or [FAKE] * 6
    return lib.pa_decode(None if p is None else ctypes.byref(p), num_seqs, *ptrs, ws, ws_bytes, None)


def test_library_exports_every_declared_symbol():
    lib = api.library()
    names = declared_functions()
    assert set(names) == set(api.ABI_SYMBOLS) | set(ENGINE_SYMBOLS)
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", api.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (pa_\w+)", out))
    assert set(names) <= exported


def test_params_struct_matches_header_layout(tmp_path):
    """The binding's struct has the header's size and every field at the header's offset (gcc compiles the
    header and prints them)."""
    fields = [f for f, _ in api.PaParams._fields_]
    src = tmp_path / "layout.c"
    src.write_text("#include <stdio.h>\n#include <stddef.h>\n#include \"pa.h\"\nint main(void){printf(\"%zu\",sizeof(pa_params));"
                   + "".join(f'printf(" %zu",offsetof(pa_params,{f}));' for f in fields) + "return 0;}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    assert got[0] == ctypes.sizeof(api.PaParams) == 11 * 4
    assert got[1:] == [getattr(api.PaParams, f).offset for f in fields]


def test_status_strings():
    lib = api.library()
    for st in range(6):
        assert lib.pa_status_string(st).decode() not in ("", "unknown status")
    assert lib.pa_status_string(99).decode() == "unknown status"


@pytest.mark.parametrize("field,value,expect", [
    ("num_q_heads", 30, INVALID),
    ("num_kv_heads", 0, INVALID),
    ("head_dim", 96, UNSUPPORTED),
    ("head_dim", 0, INVALID),
    ("block_size", 0, INVALID),
    ("num_blocks", 0, INVALID),
    ("max_blocks_per_seq", 0, INVALID),
    ("dtype", 7, INVALID),
    ("scale", float("nan"), INVALID),
    ("scale", float("inf"), INVALID),
    ("partition_tokens", 24, INVALID),
    ("partition_tokens", 2048, INVALID),
    ("layout", 2, INVALID),
    ("layout", -1, INVALID),
    ("partition_tokens", -16, INVALID),
    ("flags", 2, INVALID),
    ("flags", -1, INVALID),
])
def test_decode_rejects_bad_scalars(field, value, expect):
    p = params(**{field: value})
    assert decode_status(p) == expect
    assert api.library().pa_last_error_detail().decode()


def test_decode_null_params_and_pointers():
    assert decode_status(None) == NULLP
    assert decode_status(params(), ptrs=[FAKE, None, FAKE, FAKE, FAKE, FAKE]) == NULLP


def test_decode_zero_sequences_is_noop():
    assert decode_status(params(), num_seqs=0, ptrs=[None] * 6) == OK
    assert decode_status(params(), num_seqs=-1) == INVALID


def test_decode_workspace_checks():
    p = params()
    need = api.decode_workspace_size(p, 4)
    assert need > 0
    assert decode_status(p, ws=None, ws_bytes=0) == NULLP
    assert decode_status(p, ws=FAKE, ws_bytes=need - 1) == WS_SMALL


def test_partition_tokens_cut_the_balanced_decode():
    """A caller-set partition size on the balanced decode (block size 16) restarts the softmax at partition bounds
    and folds the partitions in registers: the workspace (waves' partials, one piece record per request and head
    group) is the same with or without partitions."""
    lib = api.library()

    def ws(**kw):
        return lib.pa_decode_workspace_size(ctypes.byref(params(max_blocks_per_seq=2048, num_q_heads=64, **kw)), 8)

    base = ws()
    assert base > 0
    assert ws(partition_tokens=512) == ws(partition_tokens=64) == ws(partition_tokens=1024) == base


def test_noalloc_decode_argument_checks():
    """pa_decode_noalloc: the checks of pa_decode, and a batch needing more than its 32 MiB static scratch is
    refused before any HIP call."""
    lib = api.library()

    def st(p, num_seqs=4):
        return lib.pa_decode_noalloc(None if p is None else ctypes.byref(p), num_seqs, *([FAKE] * 6), None)

    assert st(None) == NULLP
    assert st(params(num_kv_heads=0)) == INVALID
    assert st(params(), num_seqs=-1) == INVALID
    assert st(params(), num_seqs=0) == OK
    assert lib.pa_decode_noalloc(ctypes.byref(params()), 4, None, *([FAKE] * 5), None) == NULLP
    # partitions of 512 tokens over 100000 blocks of 5: far more partials than 32 MiB
    big = params(block_size=5, max_blocks_per_seq=100000, num_blocks=200000)
    assert lib.pa_decode_workspace_size(ctypes.byref(big), 100) > (32 << 20)
    assert st(big, num_seqs=100) == WS_SMALL
    assert b"scratch" in lib.pa_last_error_detail()


def test_decode_workspace_sizes():
    # block sizes that are multiples of 16 take the balanced path: partial slots for every wave
    p = params(max_blocks_per_seq=32)
    assert api.decode_workspace_size(p, 8) > 0
    # ... except with at most four tiles per context, or with one partition per context and enough contexts to
    # fill the GPU four times over: one wave per context, nothing to merge
    assert api.decode_workspace_size(params(max_blocks_per_seq=4), 8) == 0
    assert api.decode_workspace_size(params(max_blocks_per_seq=5), 8) > 0
    waves_per_seq = params().num_kv_heads
    many = 4 * 1024 // waves_per_seq
    assert api.decode_workspace_size(params(max_blocks_per_seq=32), many) == 0
    assert api.decode_workspace_size(params(max_blocks_per_seq=32), many - 1) > 0
    assert api.decode_workspace_size(params(max_blocks_per_seq=33), many) > 0
    # other block sizes use context partitions: nothing to merge when one partition holds any request
    p = params(block_size=5, max_blocks_per_seq=100)  # 500 tokens <= 512
    assert api.decode_workspace_size(p, 8) == 0
    p = params(block_size=5, max_blocks_per_seq=103)  # 515 tokens: two partitions
    assert api.decode_workspace_size(p, 8) >= 8 * 32 * 2 * (128 + 2) * 4


def test_mixed_argument_checks():
    lib = api.library()
    p = params()
    ptrs = [FAKE] * 7

    def mixed(S, T, mql, ws=None, wsb=0, pp=p, ps=ptrs):
        return lib.pa_varlen_mixed(ctypes.byref(pp), S, T, mql, *ps, ws, wsb, None)

    assert mixed(0, 0, 0) == OK
    assert mixed(4, 10, 0) == INVALID
    assert mixed(4, 10, 11) == INVALID
    assert mixed(4, 10, 4, ps=[FAKE] * 6 + [None]) == NULLP
    need = api.varlen_mixed_workspace_size(p, 4, 10, 4)
    assert need > 0
    assert mixed(4, 10, 4, ws=FAKE, wsb=need - 1) == WS_SMALL


def test_host_checker():
    p = params(num_blocks=10, max_blocks_per_seq=4)
    bt = torch.tensor([[0, 1, 2, 3], [4, 5, 9, 9]], dtype=torch.int32)
    cl = torch.tensor([64, 33], dtype=torch.int32)
    assert api.check_inputs_host(p, bt, cl) == (OK, -1)
    assert api.check_inputs_host(p, bt, torch.tensor([64, 65], dtype=torch.int32))[0] == INVALID
    bt_bad = bt.clone()
    bt_bad[1, 2] = 10
    assert api.check_inputs_host(p, bt_bad, cl) == (INVALID, 1)
    # padding past the used blocks is not checked
    bt_pad = bt.clone()
    bt_pad[1, 3] = -5
    assert api.check_inputs_host(p, bt_pad, cl) == (OK, -1)
    qsl = torch.tensor([0, 1, 5], dtype=torch.int32)
    assert api.check_inputs_host(p, bt, cl, qsl) == (OK, -1)
    assert api.check_inputs_host(p, bt, torch.tensor([64, 3], dtype=torch.int32), qsl) == (INVALID, 1)
    assert api.check_inputs_host(p, bt, cl, torch.tensor([0, 2, 1], dtype=torch.int32), num_tokens=1)[0] == INVALID
    # max_query_len: request 1 has 4 query rows
    assert api.check_inputs_host(p, bt, cl, qsl, max_query_len=4) == (OK, -1)
    assert api.check_inputs_host(p, bt, cl, qsl, max_query_len=3) == (INVALID, 1)


def test_incomplete_aux_is_refused_before_any_hip_call():
    """pa_varlen_mixed_ex / pa_decode_shared_ex with a pa_aux missing an event: PA_ERR_NULL_POINTER, returned
    before the first HIP call (the pointers are never dereferenced)."""
    lib = api.library()
    p = params()
    aux = api.PaAux(stream=0x2000, fork_event=0x3000, join_event=None)
    big = 1 << 40
    st = lib.pa_varlen_mixed_ex(ctypes.byref(p), 4, 10, 4, *([FAKE] * 7), FAKE, big, None, ctypes.byref(aux))
    assert st == NULLP and b"pa_aux" in lib.pa_last_error_detail()
    st = lib.pa_decode_shared_ex(ctypes.byref(p), 4, 1, *([FAKE] * 8), FAKE, big, None, ctypes.byref(aux))
    assert st == NULLP and b"pa_aux" in lib.pa_last_error_detail()


def test_timing_hook_argument_check():
    lib = api.library()
    assert lib.pa_set_kernel_timing_events(FAKE, None) == INVALID
    assert lib.pa_set_kernel_timing_events(None, None) == OK


def test_binding_rejects_host_tensors():
    q = torch.zeros(2, 4, 128, dtype=torch.bfloat16)
    k = torch.zeros(4, 16, 2, 128, dtype=torch.bfloat16)
    bt = torch.zeros(2, 2, dtype=torch.int32)
    cl = torch.ones(2, dtype=torch.int32)
    with pytest.raises(ValueError):
        api.decode(q, k, k, bt, cl, scale=1.0, out=torch.empty_like(q))


def cache_status(p, num_seqs=4, num_tokens=4, ptrs=None, qsl=None):
    lib = api.library()
    ptrs = ptrs or [FAKE] * 6
    return lib.pa_cache_write(None if p is None else ctypes.byref(p), num_seqs, num_tokens, *ptrs, qsl, None)


def test_cache_write_argument_checks():
    assert cache_status(None) == NULLP
    assert cache_status(params(head_dim=96)) == UNSUPPORTED
    assert cache_status(params(dtype=7)) == INVALID
    assert cache_status(params(), num_seqs=-1) == INVALID
    assert cache_status(params(), num_seqs=4, num_tokens=5) == INVALID  # decode batch: one token per request
    assert cache_status(params(), num_seqs=0, num_tokens=0) == OK
    assert cache_status(params(), num_seqs=4, num_tokens=0, qsl=FAKE) == OK
    assert cache_status(params(), ptrs=[FAKE, None, FAKE, FAKE, FAKE, FAKE]) == NULLP


def test_binding_cache_write_rejects_host_tensors():
    k = torch.zeros(4, 16, 2, 128, dtype=torch.bfloat16)
    kn = torch.zeros(2, 2, 128, dtype=torch.bfloat16)
    bt = torch.zeros(2, 2, dtype=torch.int32)
    cl = torch.ones(2, dtype=torch.int32)
    with pytest.raises(ValueError):
        api.cache_write(k, k, kn, kn, bt, cl)


def copy_status(p, num_pairs=2, dst_nb=8, src_nb=8, ptrs=None):
    lib = api.library()
    d_k, d_v, s_k, s_v, m = ptrs or [FAKE] * 5
    return lib.pa_copy_blocks(None if p is None else ctypes.byref(p), num_pairs, d_k, d_v, dst_nb, s_k, s_v, src_nb,
                              m, None)


def test_copy_blocks_argument_checks():
    assert copy_status(None) == NULLP
    assert copy_status(params(head_dim=96)) == UNSUPPORTED
    assert copy_status(params(dtype=7)) == INVALID
    assert copy_status(params(), num_pairs=-1) == INVALID
    assert copy_status(params(), dst_nb=0) == INVALID
    assert copy_status(params(), src_nb=0) == INVALID
    assert copy_status(params(), num_pairs=0) == OK
    assert copy_status(params(), ptrs=[FAKE, FAKE, FAKE, FAKE, None]) == NULLP
    assert copy_status(params(), ptrs=[FAKE, None, FAKE, FAKE, FAKE]) == NULLP


def test_copy_host_checker():
    m = lambda *pairs: torch.tensor(pairs, dtype=torch.int32).reshape(-1, 2)
    assert api.check_copy_host(m([0, 3], [1, 4], [2, 5]), 8, 8, True) == (OK, -1)
    assert api.check_copy_host(m([0, 3], [1, 4]), 2, 5, False) == (OK, -1)
    assert api.check_copy_host(m([0, 3], [3, 4]), 8, 8, True) == (INVALID, 0)  # block 3 is written and read
    assert api.check_copy_host(m([0, 3], [3, 4]), 8, 8, False) == (OK, -1)  # two pools: no conflict
    assert api.check_copy_host(m([0, 3], [1, 3]), 8, 8, False) == (INVALID, 1)  # repeated destination
    assert api.check_copy_host(m([0, 1], [1, 2]), 8, 8, True) == (INVALID, 0)  # a chain within one pool
    assert api.check_copy_host(m([0, 1], [2, 8]), 8, 8, True) == (INVALID, 1)  # destination outside the pool
    assert api.check_copy_host(m([0, 1], [9, 2]), 8, 8, True) == (INVALID, 1)
    assert api.check_copy_host(m([0, 1], [-1, 2]), 8, 8, True) == (INVALID, 1)
    assert api.check_copy_host(m([0, 1]), 8, 4, True)[0] == INVALID  # one pool, two sizes
    assert api.check_copy_host(torch.zeros(0, 2, dtype=torch.int32), 1, 1, True) == (OK, -1)


def test_binding_copy_blocks_rejects_pageable_host_tensors():
    k = torch.zeros(4, 16, 2, 128, dtype=torch.bfloat16)
    m = torch.tensor([[0, 1]], dtype=torch.int32)
    with pytest.raises(ValueError):
        api.copy_blocks(k, k, k.clone(), k.clone(), m)


def test_stream_read_probe_argument_checks():
    lib = api.library()
    assert lib.pa_probe_stream_read(None, 1024, 4, FAKE, None) == NULLP
    assert lib.pa_probe_stream_read(FAKE, 1024, 4, None, None) == NULLP
    assert lib.pa_probe_stream_read(FAKE, 1000, 4, FAKE, None) == INVALID  # not a multiple of 16
    assert lib.pa_probe_stream_read(ctypes.c_void_p(0x1008), 1024, 4, FAKE, None) == INVALID  # misaligned
    assert lib.pa_probe_stream_read(FAKE, 1024, 0, FAKE, None) == INVALID
    assert lib.pa_probe_stream_read(FAKE, 1024, 70000, FAKE, None) == INVALID


def test_group_checker():
    from paged_kv_cache_168_amd import workloads as W

    wl = W.grouped_workload(77, [(64, [100, 64, 20, 300]), (0, [5]), (32, [40, 33])], Hq=8, Hkv=2, D=64, BS=16)
    p = params(num_q_heads=8, num_kv_heads=2, head_dim=64, block_size=16, num_blocks=wl.k_cache.shape[0],
               max_blocks_per_seq=wl.block_tables.shape[1])
    gs, gp = W.prefix_groups(wl)
    assert api.check_groups_host(p, gs, gp, wl.block_tables, wl.context_lens) == (OK, -1)
    bt = wl.block_tables.clone()
    bt[3, 1] = bt[3, 1] + 1 if int(bt[3, 1]) + 1 < p.num_blocks else 0  # request 3 no longer shares block 1
    assert api.check_groups_host(p, gs, gp, bt, wl.context_lens) == (INVALID, 0)
    assert api.check_groups_host(p, gs, torch.tensor([64, 0, 40]), wl.block_tables, wl.context_lens)[0] == INVALID
    assert api.check_groups_host(p, torch.tensor([0, 4, 5, 6]), gp, wl.block_tables, wl.context_lens)[0] == INVALID
    assert api.check_groups_host(p, torch.tensor([0, 4, 3, 7]), gp, wl.block_tables, wl.context_lens) == (INVALID, 1)
    # a group end past the last request, before the decrease that brings it back (never read past the tables)
    assert api.check_groups_host(p, torch.tensor([0, 9, 6, 7]), gp, wl.block_tables, wl.context_lens) == (INVALID, 0)
    # group 0 absorbing request 4, whose table does not hold group 0's prefix blocks
    assert api.check_groups_host(p, torch.tensor([0, 5, 5, 7]), gp, wl.block_tables, wl.context_lens) == (INVALID, 0)
