"""Benchmark: paged attention on one MI355X, every benchmarked workload, one JSON line.

One step is one complete library call (every kernel of the path, the log-sum-exp merge included) over the
whole batch of a synthetic workload, inputs resident in HBM. The headline (``value``) is the largest
workload: the mixed continuous-batching step of one 512-token causal chunk (offset 2048 of a 4096-token
prompt) beside 128 decodes with contexts U[256, 8192] (32 query / 8 KV heads, head_dim 128, 16-token blocks,
bf16), through ``pa_varlen_mixed``. ``value`` is its effective KV bandwidth: logical KV bytes (every context
token's K and V row of every KV head, read once; the chunk's context counted once) over the time per step.

The same line carries, under ``configs``, every other workload measured the same way: the tiny fp32 decode
(latency), the 64-request bf16 decode, the 8 x 32768 long-context decode with 512-token context partitions
merged by log-sum-exp (and, as ``long_balanced``, the same batch on the balanced split without partitions),
and the 256-request prefix-shared decode. Each entry has its step time and bandwidth, its dominant kernel
against the HBM roofline (HIP events attached to that kernel's launch), and the fp64 oracle timed on the
host cores on the same inputs. KV pools are replicated and rotated between steps so the distinct working set
exceeds the 256 MB last-level cache.

``roofline`` is the headline's decode kernel: its algorithmic bytes (the decode rows' K and V, read once)
over its launch time; the chunk runs beside it on the matrix cores (``chunk``). ``traffic`` is the calibrated
HBM traffic per launch from rocprofv3 counters (``--record-traffic``), when recorded for the current kernel
sources. Also reported: the streaming-read ceiling, the KV-cache write and block copies on the headline's
pool, and the host scheduler's block waste over a synthetic request stream.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import sys
import time

HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
METRIC = "paged-attn decode effective KV GB/s (% HBM peak); seq-steps/sec per GPU"
ROOT = os.path.dirname(os.path.abspath(__file__))
# the sources and build flags (build.py) of the kernels whose recorded traffic the line reports
KERNEL_SOURCES = ["paged_kv_cache_168_amd/csrc/pa_decode_balanced.hip", "paged_kv_cache_168_amd/csrc/pa_decode.hip",
                  "paged_kv_cache_168_amd/csrc/pa_device.h", "paged_kv_cache_168_amd/csrc/pa_api.cpp",
                  "paged_kv_cache_168_amd/csrc/pa_internal.h", "paged_kv_cache_168_amd/csrc/pa_prefill.hip",
                  "paged_kv_cache_168_amd/build.py"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")
SEED_CACHE_WRITE = 1689
HEADLINE = "mixed"
# name -> (workload, partition_tokens, what the split is, entry point ("decode", "shared" = pa_decode_shared with
# the workload's prefix groups, "shared1" = the same with the prefix-shared batch as one group, or "mixed"),
# PA_FLAG_SHARED_BLOCKS, cache layout)
TM, HM = 0, 1  # PA_LAYOUT_TOKEN_MAJOR, PA_LAYOUT_HEAD_MAJOR
CONFIGS = {
    "mixed": ("mixed", 0, "decode rows: balanced stream-K split of 16-token tiles; chunk rows: one row tile per "
                          "64 (row, head) pairs covering all its keys, on the matrix cores beside the decodes",
              "mixed", False, TM),
    "tiny": ("tiny", 0, "one wave per (request, KV head) holding the whole context (at most 3 tiles), no merge",
             "decode", False, TM),
    "decode64": ("decode64", 0, "balanced stream-K split of 16-token tiles", "decode", False, TM),
    "long": ("long", 512, "context partitions of 512 tokens (the softmax restarts at each partition bound), "
                          "balanced over the waves, log-sum-exp merge of the partitions (in registers within a "
                          "wave, by the merge kernel across waves)", "decode", False, TM),
    "long_balanced": ("long", 0, "balanced stream-K split of 16-token tiles, no fixed partitions", "decode", False,
                      TM),
    "prefix": ("prefix", 0, "each group's shared blocks read once on the matrix cores (prefix pass: the 16 beam "
                            "groups' prompt prefix and common beam blocks, the 512-token prompt prefix of the other "
                            "192 requests) beside the balanced split of the private blocks (streaming loads), "
                            "log-sum-exp merge", "shared", False, TM),
    "prefix_one_group": ("prefix", 0, "as prefix, with the batch described as one group of 256 requests sharing the "
                                      "512-token prompt prefix (the beams' common blocks go through the balanced "
                                      "split)", "shared1", False, TM),
    "prefix_plain": ("prefix", 0, "every request through its own table: balanced stream-K split, cached loads so "
                                  "that shared blocks are served from the caches", "decode", True, TM),
    # the same splits over caches stored head-major ([block][kv head][slot][head_dim])
    "mixed_head_major": ("mixed", 0, "as mixed, head-major caches", "mixed", False, HM),
    "decode64_head_major": ("decode64", 0, "as decode64, head-major caches", "decode", False, HM),
    "long_head_major": ("long", 512, "as long, head-major caches", "decode", False, HM),
    "long_balanced_head_major": ("long", 0, "as long_balanced, head-major caches", "decode", False, HM),
}


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(CONFIGS),
                    help="the headline workload (default: the mixed step, the largest)")
    ap.add_argument("--only", action="store_true",
                    help="measure the headline workload only (no other configs, probes or CPU baseline): for "
                         "profiler runs")
    ap.add_argument("--pool-copies", type=int, default=0, help="0 = enough copies for a >= 1 GB working set")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--chunk-alone", action="store_true",
                    help="time only the mixed step's chunk request as a batch of its own (the matrix-core chunk "
                         "kernel alone) and print its entry: for profiler runs")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run one 1 GiB elementwise copy first (counter calibration under rocprofv3)")
    ap.add_argument("--record-traffic", metavar="DIR",
                    help="no GPU: read the rocprofv3 counter CSVs of a --calib-copy --only run under DIR "
                         "(DIR/pmc_FETCH_SIZE and DIR/pmc_WRITE_SIZE) and store the --workload's calibrated "
                         "traffic per launch in profiles/decode_traffic.json")
    return ap.parse_args()


def kv_bytes(wl, rows: str = "all") -> int:
    """Algorithmic bytes: K and V rows of every KV head for every context token, read once. rows: "all", or
    "decode" / "chunk" for the requests with one / several query rows of a mixed step."""
    NB, BS, Hkv, D = wl.k_cache.shape
    cl = wl.context_lens.to("cpu").long()
    if rows != "all" and wl.query_start_loc is not None:
        qsl = wl.query_start_loc.to("cpu").long()
        ql = qsl[1:] - qsl[:-1]
        cl = cl[ql == 1] if rows == "decode" else cl[ql > 1]
    elif rows == "chunk":
        cl = cl[:0]
    return int(cl.sum()) * 2 * Hkv * D * wl.k_cache.element_size()


def suffix_kv_bytes(wl, beams=True) -> int:
    """Algorithmic bytes of the decode kernel when a prefix pass reads the shared prefixes: every request's K and V
    past its group's shared prefix (the workload's prefix groups), read once."""
    from paged_kv_cache_168_amd import workloads as W

    NB, BS, Hkv, D = wl.k_cache.shape
    gs, gp = W.prefix_groups(wl, beams)
    cl = wl.context_lens.tolist()
    tokens = 0
    for g in range(len(gp)):
        first = int(gs[g])
        pre = min(int(gp[g]), cl[first]) // BS * BS if int(gs[g + 1]) > first else 0
        for s in range(first, int(gs[g + 1])):
            tokens += cl[s] - min(pre, cl[s]) if pre < cl[s] else 0
    return tokens * 2 * Hkv * D * wl.k_cache.element_size()


def chunk_flops(wl) -> int:
    """Algorithmic flops of the chunk rows of a mixed step: 4 D per visible key per query head (QK^T and PV)."""
    if wl.query_start_loc is None:
        return 0
    T, Hq, D = wl.q.shape
    qsl, cl = wl.query_start_loc.tolist(), wl.context_lens.tolist()
    keys = 0
    for s in range(wl.num_seqs):
        ql = qsl[s + 1] - qsl[s]
        if ql > 1:
            keys += sum(cl[s] - ql + j + 1 for j in range(ql))
    return 4 * D * Hq * keys


def unique_kv_bytes(wl) -> int:
    """K and V bytes of the distinct (block, slot) rows the batch reads: a block shared by several requests counts
    once, with the largest fill any of them reads."""
    NB, BS, Hkv, D = wl.k_cache.shape
    fill = {}
    bt, cl = wl.block_tables.to("cpu"), wl.context_lens.to("cpu")
    for s in range(bt.shape[0]):
        c = int(cl[s])
        for b in range(-(-c // BS)):
            blk = int(bt[s, b])
            fill[blk] = max(fill.get(blk, 0), min(BS, c - b * BS))
    return sum(fill.values()) * 2 * Hkv * D * wl.k_cache.element_size()


def _visible_keys(wl):
    """Visible keys per query token (ctx, or ctx - q_len + j + 1 for row j of a slice)."""
    cl = wl.context_lens.tolist()
    if wl.query_start_loc is None:
        return cl
    qsl = wl.query_start_loc.tolist()
    n = []
    for s in range(wl.num_seqs):
        ql = qsl[s + 1] - qsl[s]
        n += [cl[s] - ql + j + 1 for j in range(ql)]
    return n


def cpu_baseline(wl, min_seconds=10.0, single_seconds=5.0):
    """The fp64 oracle over the whole workload on the host cores, repeated for about min_seconds (median), and
    on one thread over a strided sample of the rows that takes about single_seconds, scaled to the whole
    workload by the keys its rows read."""
    from oracle import paged_attention

    threads = int(os.environ.get("OMP_NUM_THREADS", 0)) or len(os.sched_getaffinity(0))
    args = (wl.q, wl.k_cache, wl.v_cache, wl.block_tables, wl.context_lens, wl.query_start_loc)
    times = []
    t_all = time.perf_counter()
    while not times or (time.perf_counter() - t_all < min_seconds and len(times) < 1000):
        t0 = time.perf_counter()
        paged_attention(*args, scale=wl.scale, threads=threads)
        times.append(time.perf_counter() - t0)
    times.sort()
    t = times[len(times) // 2]
    res = {"value": round(kv_bytes(wl) / t / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
           "seq_steps_per_s": round(wl.num_seqs / t, 2),
           "sample": f"whole workload ({wl.num_seqs} requests, {wl.num_tokens} query rows, all heads), median of "
                     f"{len(times)} runs of {t:.3f} s each, fp64 C oracle with OpenMP"}
    if single_seconds > 0:
        Hq = wl.q.shape[1]
        keys = _visible_keys(wl)
        total_keys = sum(keys) * Hq
        # one thread runs about `threads` times slower: a stride that makes the sample take ~single_seconds
        stride = max(1, math.ceil(t * threads / single_seconds))
        rows = list(range(0, wl.num_tokens * Hq, stride))
        sample_keys = sum(keys[r // Hq] for r in rows)
        t0 = time.perf_counter()
        paged_attention(*args, scale=wl.scale, threads=1, rows=rows)
        t1 = (time.perf_counter() - t0) * total_keys / max(sample_keys, 1)
        res["single_thread"] = {"value": round(kv_bytes(wl) / t1 / 1e9, 3), "unit": "GB/s", "cores": 1,
                                "seq_steps_per_s": round(wl.num_seqs / t1, 2),
                                "sample": f"one in every {stride} of the {wl.num_tokens * Hq} (query row, head) rows, "
                                          f"one run, scaled to the whole workload by the keys read"}
    return res


def timing_events(n):
    """n pairs of timing-enabled torch events, each recorded once so that its hipEvent exists (the library's
    timing hook takes the raw handles)."""
    import torch

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in ev:
        a.record()
        b.record()
    torch.cuda.synchronize()
    return ev


def _timed(call, steps, attach=True):
    """Mean microseconds of call()'s kernel by HIP events attached to its launch, each call issued on an idle
    stream (5 untimed calls first); attach=False times calls that launch no library kernel by events
    recorded around them."""
    import torch

    from paged_kv_cache_168_amd import api

    for _ in range(5):
        call()
    ev = timing_events(steps)
    for a, b in ev:
        torch.cuda.synchronize()
        if attach:
            api.set_kernel_timing_events(a, b)
        else:
            a.record()
        call()
        if not attach:
            b.record()
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in ev) / steps * 1e3


READ_CEILING_WAVES = (1024, 1536, 2048)


def read_ceiling(device, steps, gib=2):
    """The streaming-read reference (pa_probe_stream_read): a 2 GiB buffer read once per call with the decode
    kernels' 16-byte non-temporal loads; GB/s by HIP events attached to the kernel. The best of a few wave
    counts is the ceiling (1536 waves read about 8% faster than 1024 on this part)."""
    import torch

    from paged_kv_cache_168_amd import api

    buf = torch.ones(gib << 30, dtype=torch.uint8, device=device)
    sink = torch.empty(max(READ_CEILING_WAVES), dtype=torch.int32, device=device)
    best_us, best_waves, by_waves = None, None, {}
    for waves in READ_CEILING_WAVES:
        us = _timed(lambda: api.probe_stream_read(buf, sink, waves), steps)
        by_waves[str(waves)] = round((gib << 30) / (us * 1e-6) / 1e9, 1)
        if best_us is None or us < best_us:
            best_us, best_waves = us, waves
    del buf
    return {"gbps": round((gib << 30) / (best_us * 1e-6) / 1e9, 1), "bytes": gib << 30, "us": round(best_us, 2),
            "waves": best_waves, "gbps_by_waves": by_waves, "kernel": "stream_read_kernel (pa_probe_stream_read)"}


def time_cache_write(wl, q, pool, bt, cl, qsl, steps):
    """The KV-cache write of the step's new rows (one per query token) into the pool: HIP events attached to
    the kernel of each call. Bytes: the new K and V rows read once and written once."""
    import torch

    from paged_kv_cache_168_amd import api

    T = q.shape[0]
    _, _, Hkv, D = pool[0].shape
    g = torch.Generator(device="cpu").manual_seed(SEED_CACHE_WRITE)
    kn = torch.randn(T, Hkv, D, generator=g).to(pool[0].dtype).to(q.device)
    vn = torch.randn(T, Hkv, D, generator=g).to(pool[0].dtype).to(q.device)
    us = _timed(lambda: api.cache_write(pool[0], pool[1], kn, vn, bt, cl, qsl), steps)
    nbytes = 2 * 2 * T * Hkv * D * pool[0].element_size()
    return {"tokens": T, "us": round(us, 2), "bytes": nbytes, "gbps": round(nbytes / (us * 1e-6) / 1e9, 1)}


def time_block_copy(pool, bt, cl, steps):
    """Block copies on the step's pool. Copy-on-write: up to 64 blocks (a 16-group, 4-branch beam fork) into
    free blocks of the same pool; bytes = K and V blocks read once and written once. Swap: the longest
    request's blocks (up to 256) out to a pinned host pool and back into the same ids; bytes = K and V
    blocks across the host link, beside torch's contiguous copy of as many bytes (the DMA engines) for
    reference."""
    import torch

    from paged_kv_cache_168_amd import api

    NB, BS = pool[0].shape[0], pool[0].shape[1]
    bt_h, cl_h = bt.cpu(), cl.cpu()
    nblk = [-(-int(c) // BS) for c in cl_h]
    used = torch.unique(torch.cat([bt_h[s, :n] for s, n in enumerate(nblk)]))
    free_mask = torch.ones(NB, dtype=torch.bool)
    free_mask[used.long()] = False
    free = torch.nonzero(free_mask).flatten()
    block_bytes = pool[0][0].numel() * pool[0].element_size()
    res = {}
    n = min(64, free.numel(), used.numel())
    if n > 0:
        m = torch.stack([used[:n], free[:n]], 1).to(torch.int32).to(pool[0].device)
        us = _timed(lambda: api.copy_blocks(pool[0], pool[1], pool[0], pool[1], m), steps)
        nbytes = 2 * 2 * n * block_bytes
        res["cow"] = {"pairs": n, "us": round(us, 2), "bytes": nbytes, "gbps": round(nbytes / (us * 1e-6) / 1e9, 1)}
    s = max(range(len(nblk)), key=lambda i: nblk[i])
    nb = min(256, nblk[s])
    ids = bt_h[s, :nb].to(torch.int32)
    shape = (nb,) + tuple(pool[0].shape[1:])
    hk = torch.empty(shape, dtype=pool[0].dtype, pin_memory=True)
    hv = torch.empty(shape, dtype=pool[0].dtype, pin_memory=True)
    out_map = torch.stack([ids, torch.arange(nb, dtype=torch.int32)], 1).to(pool[0].device)
    in_map = out_map.flip(1).contiguous()
    nbytes = 2 * nb * block_bytes
    us_out = _timed(lambda: api.copy_blocks(hk, hv, pool[0], pool[1], out_map), steps)
    us_in = _timed(lambda: api.copy_blocks(pool[0], pool[1], hk, hv, in_map), steps)
    dev_buf = torch.empty(nbytes // 2, dtype=torch.uint8, device=pool[0].device)
    host_buf = torch.empty(nbytes // 2, dtype=torch.uint8, pin_memory=True)
    us_dma_out = _timed(lambda: (host_buf.copy_(dev_buf, non_blocking=True), host_buf.copy_(dev_buf, non_blocking=True)),
                        steps, attach=False)
    us_dma_in = _timed(lambda: (dev_buf.copy_(host_buf, non_blocking=True), dev_buf.copy_(host_buf, non_blocking=True)),
                       steps, attach=False)
    gb = lambda us: round(nbytes / (us * 1e-6) / 1e9, 1)
    res["swap"] = {"blocks": nb, "bytes": nbytes, "out_us": round(us_out, 2), "out_gbps": gb(us_out),
                   "in_us": round(us_in, 2), "in_gbps": gb(us_in), "dma_out_gbps": gb(us_dma_out),
                   "dma_in_gbps": gb(us_dma_in)}
    return res


def scheduler_summary(seed=1685, requests=512):
    """The host scheduler (pa_engine) over a synthetic request stream shaped like the 64-request decode batch:
    prompts U[128, 3840] tokens, U[16, 256] new tokens, arrivals while fewer than 64 wait, 16-token blocks in a
    pool of 9328 blocks, 64 running requests, 512-token prefill slices under a 2048-token step budget, and 4% of
    the requests forked (beam branches). Reports the mean over steps of the unfilled fraction of the blocks that
    hold tokens (the pages claim < 4%), of block utilisation (used / total), of the used blocks allocated ahead of
    their prompt slice, and the scheduler's host time per step."""
    import numpy as np

    from paged_kv_cache_168_amd.engine import Engine

    rng = np.random.default_rng(seed)
    e = Engine(num_blocks=9328, block_size=16, max_blocks_per_seq=256, max_num_seqs=64, max_num_batched_tokens=2048,
               chunk_tokens=512, reserve_blocks=2, num_host_blocks=2048)
    submitted, steps, waste, util, empty, t_step = 0, 0, [], [], [], 0.0
    while True:
        st = e.stats()
        while submitted < requests and st["waiting"] < 64:
            submitted += 1
            e.submit(submitted, int(rng.integers(128, 3841)), int(rng.integers(16, 257)))
            st["waiting"] += 1
        t0 = time.perf_counter()
        b = e.step()
        t_step += time.perf_counter() - t0
        if b.num_seqs == 0 and submitted >= requests and e.stats()["running"] == 0:
            break
        steps += 1
        st = e.stats()
        if st["used_blocks"]:
            waste.append(st["waste"])
            util.append(st["utilization"])
            empty.append(st["empty_blocks"] / st["used_blocks"])
        if b.num_seqs and rng.random() < 0.04 * b.num_seqs / 8:
            r = int(b.request_ids[int(rng.integers(0, b.num_seqs))])
            try:
                submitted_child = requests + steps
                e.fork(r, submitted_child, int(rng.integers(8, 64)))
            except Exception:
                pass
    st = e.stats()
    return {"requests": submitted, "steps": steps, "waste_mean": round(float(np.mean(waste)), 5),
            "utilization_mean": round(float(np.mean(util)), 4),
            "allocated_ahead_mean": round(float(np.mean(empty)), 4), "preemptions": st["preemptions"],
            "copies": st["copies"], "host_us_per_step": round(t_step / max(steps, 1) * 1e6, 2)}


def load_traffic(workload):
    """Calibrated HBM traffic per launch of the workload's dominant kernel, if recorded for these kernel sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        rec = json.load(f).get(workload)
    if rec and rec.get("kernel_source_hash") == kernel_source_hash():
        return rec
    return None


def measure(name, steps, warmup, dev, *, pool_copies=0, calib_copy=False, extras=False):
    """One workload: `warmup` untimed steps, then `steps` steps with HIP events attached to the dominant kernel's
    launch (each on an idle stream: the kernel's own duration), then `steps` whole steps back to back (the step
    time). Returns the result entry; with extras also the KV-cache write, block copies and the chunk alone."""
    import torch

    from paged_kv_cache_168_amd import api
    from paged_kv_cache_168_amd import workloads as W

    wname, pt, split, entry, shared, layout = CONFIGS[name]
    wl = W.WORKLOADS[wname]()
    mixed = entry == "mixed"
    use_prefix = entry in ("shared", "shared1")
    beams = entry == "shared"
    nbytes = kv_bytes(wl)
    # the dominant (decode) kernel's algorithmic bytes: the decode rows of a mixed step; past the shared prefixes
    # (which the prefix pass reads) with a prefix pass
    kbytes = kv_bytes(wl, "decode") if mixed else suffix_kv_bytes(wl, beams) if use_prefix else nbytes
    pool_bytes = 2 * wl.k_cache.numel() * wl.k_cache.element_size()
    copies = pool_copies or max(1, math.ceil(1.0e9 / pool_bytes))

    q = wl.q.to(dev)
    bt = wl.block_tables.to(dev)
    cl = wl.context_lens.to(dev)
    qsl = wl.query_start_loc.to(dev) if mixed else None
    pools = [(api.to_layout(wl.k_cache.to(dev), layout), api.to_layout(wl.v_cache.to(dev), layout))]
    for _ in range(copies - 1):
        pools.append((pools[0][0].clone(), pools[0][1].clone()))
    out = torch.empty_like(q)
    params = api.make_params(q, pools[0][0], bt, scale=wl.scale, partition_tokens=pt, shared_blocks=shared,
                             layout=layout)
    if mixed:
        ws_bytes = api.varlen_mixed_workspace_size(params, wl.num_seqs, wl.num_tokens, wl.max_query_len)
    elif use_prefix:
        groups = [x.to(dev) for x in W.prefix_groups(wl, beams)]
        ws_bytes = api.decode_shared_workspace_size(params, wl.num_seqs, int(groups[1].shape[0]))
    else:
        ws_bytes = api.decode_workspace_size(params, wl.num_seqs)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)

    def step(i):
        k, v = pools[i % copies]
        if mixed:
            api.varlen_mixed(q, k, v, bt, cl, qsl, scale=wl.scale, max_query_len=wl.max_query_len, out=out,
                             partition_tokens=pt, shared_blocks=shared, workspace=ws, layout=layout)
        elif use_prefix:
            api.decode_shared(q, k, v, bt, cl, groups[0], groups[1], scale=wl.scale, out=out, shared_blocks=shared,
                              workspace=ws, layout=layout)
        else:
            api.decode(q, k, v, bt, cl, scale=wl.scale, out=out, partition_tokens=pt, shared_blocks=shared,
                       workspace=ws, layout=layout)

    if calib_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    # Timed region 1: steps whose dominant kernel is launched with HIP events attached (hipExtLaunchKernel: they
    # bracket that kernel alone, on the stream it runs on). Each step starts on an idle stream, so the start event
    # is not held up behind the previous step's work. Only the kernel durations are taken from these steps.
    events = timing_events(steps)
    for i, (a, b) in enumerate(events):
        torch.cuda.synchronize()
        api.set_kernel_timing_events(a, b)
        step(warmup + i)
    torch.cuda.synchronize()
    kernel_ms = sum(a.elapsed_time(b) for a, b in events) / steps

    # Timed region 2: whole steps back to back, nothing recorded between the launches.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(warmup + steps + i)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / steps
    gbps = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = kbytes / (kernel_ms * 1e-3) / 1e9

    NB, BS, Hkv, D = wl.k_cache.shape
    # the balanced split always takes a workspace; one wave per context (partition kernel, one partition) none
    kernel = "decode_balanced_kernel" if int(BS) % 16 == 0 and (mixed or use_prefix or ws_bytes > 0) \
        else "decode_partition_kernel"
    res = {
        "workload": wl.name,
        "step_us": round(ms_per_step * 1e3, 2),
        "gbps": round(gbps, 2),
        "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
        "seq_steps_per_s": round(wl.num_seqs / (ms_per_step * 1e-3), 1),
        "kernel": kernel,
        "kernel_us": round(kernel_ms * 1e3, 2),
        "kernel_gbps": round(achieved, 2),
        "frac": round(achieved / HBM_PEAK_GBPS, 4),
        "algorithmic_bytes": kbytes,
        "logical_kv_bytes": nbytes,
        "split": split,
        "partition_tokens": pt or None,
        "entry_point": "pa_varlen_mixed" if mixed else "pa_decode_shared" if use_prefix else "pa_decode",
        "kv_loads": "cached (PA_FLAG_SHARED_BLOCKS)" if shared else "streaming",
        "cache_layout": "head-major" if layout == HM else "token-major",
        "bytes_basis": ("decode rows' K and V" if mixed else "K and V past the shared prefixes" if use_prefix
                        else "K and V of every context token") + ", read once",
        "pool_copies": copies,
        "dtype": "bf16" if q.dtype == torch.bfloat16 else "fp32",
        "shape": {"num_seqs": wl.num_seqs, "query_tokens": wl.num_tokens, "q_heads": int(q.shape[1]),
                  "kv_heads": int(Hkv), "head_dim": int(D), "block_size": int(BS),
                  "context_tokens": int(wl.context_lens.sum())},
    }
    if name == "tiny":
        res["note"] = "latency-bound (141 KB of KV): the HBM fraction is not meaningful"
    if mixed:
        res["query_tokens_per_s"] = round(wl.num_tokens / (ms_per_step * 1e-3), 1)
    if wl.meta.get("prefix_blocks"):  # logical bytes can exceed the HBM peak through cache hits
        ub = unique_kv_bytes(wl)
        res["unique_kv_bytes"] = ub
        res["unique_kv_gbps"] = round(ub / (ms_per_step * 1e-3) / 1e9, 1)
        res["unique_hbm_frac"] = round(ub / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)
        if shared:  # the kernel reads every request's blocks: its HBM fraction is on unique bytes
            res["frac_logical"] = res["frac"]
            res["frac"] = round(ub / (kernel_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)
            res["frac_basis"] = "unique bytes (each shared block once) over the kernel time"
    traffic = load_traffic(name)
    res["traffic"] = traffic["bytes_per_launch"] if traffic else None
    if traffic and shared:
        res["frac_fetch"] = round(traffic["read_bytes"] / (kernel_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)
    if extras:
        res["cache_write"] = time_cache_write(wl, q, pools[0], bt, cl, qsl, steps)
        res["block_copy"] = time_block_copy(pools[0], bt, cl, steps)
        if mixed:
            res["chunk"] = time_chunk_alone(wl, q, pools[0], bt, cl, qsl, steps)
    del pools, ws, out
    torch.cuda.empty_cache()
    return res


def time_chunk_alone(wl, q, pool, bt, cl, qsl, steps):
    """The step's chunk rows alone (the chunk request as a batch of its own: the MFMA tile kernel in its larger
    work-groups, no decode rows), timed by events attached to the kernel; algorithmic flops over that time against
    the bf16 matrix-core peak."""
    import torch

    from paged_kv_cache_168_amd import api

    qsl_h = wl.query_start_loc.tolist()
    s = max(range(wl.num_seqs), key=lambda i: qsl_h[i + 1] - qsl_h[i])
    r0, r1 = qsl_h[s], qsl_h[s + 1]
    q1 = q[r0:r1].contiguous()
    bt1, cl1 = bt[s:s + 1].contiguous(), cl[s:s + 1].contiguous()
    qsl1 = torch.tensor([0, r1 - r0], dtype=torch.int32, device=q.device)
    out1 = torch.empty_like(q1)
    p = api.make_params(q1, pool[0], bt1, scale=wl.scale)
    ws = torch.empty(max(api.varlen_mixed_workspace_size(p, 1, r1 - r0, r1 - r0), 1), dtype=torch.uint8,
                     device=q.device)
    call = lambda: api.varlen_mixed(q1, pool[0], pool[1], bt1, cl1, qsl1, scale=wl.scale, max_query_len=r1 - r0,
                                    out=out1, workspace=ws)
    us = _timed(call, steps)  # events attached to the chunk kernel (the call has no decode rows)
    sub = type(wl)(wl.name, wl.q[r0:r1], wl.k_cache, wl.v_cache, wl.block_tables[s:s + 1], wl.context_lens[s:s + 1],
                   torch.tensor([0, r1 - r0], dtype=torch.int32), wl.scale, wl.poison_block)
    flops = chunk_flops(sub)
    tflops = flops / (us * 1e-6) / 1e12
    return {"rows": r1 - r0, "context": int(wl.context_lens[s]), "us": round(us, 2), "flops": flops,
            "tflops": round(tflops, 1), "mfma_frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "kernel": "prefill_mfma_kernel", "timing": "HIP events attached to the kernel's launch"}


def record_traffic(workload, d):
    """Calibrated HBM bytes per launch of the workload's dominant kernel from two rocprofv3 --pmc runs of
    `bench.py --workload W --only --calib-copy` (FETCH_SIZE under d/pmc_FETCH_SIZE, WRITE_SIZE under
    d/pmc_WRITE_SIZE). Each counter is scaled by what it reads for the 1 GiB elementwise copy of --calib-copy
    (which reads 1 GiB and writes 1 GiB)."""
    def per_kernel(counter):
        files = glob.glob(os.path.join(d, f"pmc_{counter}", "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {d}/pmc_{counter}")
        vals = {}
        for fn in files:
            with open(fn) as f:
                for row in csv.DictReader(f):
                    if row.get("Counter_Name") != counter:
                        continue
                    vals.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
        return vals

    fetch, write = per_kernel("FETCH_SIZE"), per_kernel("WRITE_SIZE")
    calib = [k for k in fetch if "elementwise" in k]
    if not calib:
        raise SystemExit("the calibration copy (--calib-copy) is missing from the counters")
    ck = max(calib, key=lambda k: max(fetch[k]))
    gib = float(1 << 30)
    fetch_factor = gib / max(fetch[ck])  # bytes per counter unit
    write_factor = gib / max(write[ck])
    dk = [k for k in fetch if "decode_balanced_kernel" in k or "decode_partition_kernel" in k]
    if not dk:
        raise SystemExit("no decode kernel in the counters")
    kname = max(dk, key=lambda k: len(fetch[k]))
    rd = sum(fetch[kname]) / len(fetch[kname]) * fetch_factor
    wr = sum(write[kname]) / len(write[kname]) * write_factor
    rec = json.load(open(TRAFFIC_FILE)) if os.path.exists(TRAFFIC_FILE) else {}
    rec[workload] = {"kernel": kname, "dispatches": len(fetch[kname]), "bytes_per_launch": int(rd + wr),
                     "read_bytes": int(rd), "write_bytes": int(wr), "fetch_factor": round(fetch_factor / 1024, 4),
                     "write_factor": round(write_factor / 1024, 4), "kernel_source_hash": kernel_source_hash()}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec[workload]))


def main():
    args = parse()
    if args.record_traffic:
        record_traffic(args.workload, args.record_traffic)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    if args.chunk_alone:
        from paged_kv_cache_168_amd import workloads as W

        wl = W.WORKLOADS["mixed"]()
        pool = (wl.k_cache.to(dev), wl.v_cache.to(dev))
        print(json.dumps(time_chunk_alone(wl, wl.q.to(dev), pool, wl.block_tables.to(dev), wl.context_lens.to(dev),
                                          wl.query_start_loc.to(dev), args.steps)), flush=True)
        return
    cpu = not args.no_cpu_baseline and not args.only
    print(f"bench: headline {args.workload}", file=sys.stderr, flush=True)
    # every GPU measurement first, the oracle's CPU baselines after them, so that no host thread of the oracle is
    # still running while GPU steps are launched
    head = measure(args.workload, args.steps, args.warmup, dev, pool_copies=args.pool_copies,
                   calib_copy=args.calib_copy, extras=not args.only)
    ms = head["step_us"] / 1e3
    result = {
        "metric": METRIC,
        "value": head["gbps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic (seeded N(0,1) K/V/q, shuffled physical blocks)",
        "config": {"workload": head["workload"], **head["shape"], "split": head["split"],
                   "partition_tokens": head["partition_tokens"], "pool_copies": head["pool_copies"],
                   "entry_point": head["entry_point"], "kv_loads": head["kv_loads"]},
        "hbm_frac": head["hbm_frac"],
        "seq_steps_per_s": head["seq_steps_per_s"],
    }
    for k in ("query_tokens_per_s", "unique_kv_gbps", "unique_kv_bytes"):
        if k in head:
            result[k] = head[k]
    result["roofline"] = {"bound": "hbm", "kernel": head["kernel"], "achieved": head["kernel_gbps"],
                          "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": head["frac"], "traffic": head["traffic"],
                          "kernel_ms": round(head["kernel_us"] / 1e3, 5), "algorithmic_bytes": head["algorithmic_bytes"],
                          "bytes_basis": head["bytes_basis"]}
    if not args.only:
        ceiling = read_ceiling(dev, min(args.steps, 20))
        result["roofline"]["read_ceiling"] = ceiling
        result["roofline"]["frac_of_read_ceiling"] = round(head["kernel_gbps"] / ceiling["gbps"], 4)
        for k in ("chunk", "cache_write", "block_copy"):
            if k in head:
                result[k] = head[k]
        configs = {}
        for name in CONFIGS:
            if name == args.workload:
                continue
            print(f"bench: {name}", file=sys.stderr, flush=True)
            configs[name] = measure(name, args.steps, args.warmup, dev)
        result["configs"] = configs
        result["scheduler"] = scheduler_summary()
    if cpu:
        from paged_kv_cache_168_amd import workloads as W

        print("bench: cpu baselines", file=sys.stderr, flush=True)
        head_wl = CONFIGS[args.workload][0]
        result["cpu_baseline"] = cpu_baseline(W.WORKLOADS[head_wl](), 10.0, 5.0)
        done = {}  # one oracle run per workload, shared by the configurations over it
        for name, c in result.get("configs", {}).items():
            wname = CONFIGS[name][0]
            if wname not in done:
                done[wname] = result["cpu_baseline"] if wname == head_wl else cpu_baseline(W.WORKLOADS[wname](), 2.0, 0.0)
            c["cpu_baseline"] = done[wname]
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
