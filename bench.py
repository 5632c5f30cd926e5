"""Benchmark: paged-attention decode on one MI355X.

One step = one complete ``pa_decode`` call (the balanced decode kernel, which splits the batch's
16-token tiles evenly over a fixed set of waves, plus the log-sum-exp merge of segments that several
waves shared) over the whole batch of a synthetic workload, inputs resident in HBM. The default workload is the bf16
decode batch at a Llama-3-8B layer shape (64 requests, contexts U[128, 4096], 32 query / 8 KV
heads, head_dim 128, 16-token blocks). KV pools are replicated and rotated between steps so the
distinct working set exceeds the 256 MB Infinity Cache.

Prints ONE JSON line. ``value`` is the effective KV bandwidth: logical KV bytes (every context
token's K and V row of every KV head, read once) divided by the measured time per step. The line also
reports the dominant kernel against the HBM roofline, the KV-cache write of the step's new rows
(``cache_write``) and block copies on the step's pool (``block_copy``: copy-on-write within the pool, swap
to and from a pinned host pool), each timed separately and not part of ``value``, the host scheduler's
block waste and utilisation over a synthetic request stream (``scheduler``), and, unless disabled, the
fp64 oracle on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

HBM_PEAK_GBPS = 8000.0
METRIC = "paged-attn decode effective KV GB/s (% HBM peak); seq-steps/sec per GPU"
ROOT = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = ["paged_kv_cache_168_amd/csrc/pa_decode_balanced.hip", "paged_kv_cache_168_amd/csrc/pa_decode.hip",
                  "paged_kv_cache_168_amd/csrc/pa_device.h", "paged_kv_cache_168_amd/csrc/pa_api.cpp",
                  "paged_kv_cache_168_amd/csrc/pa_internal.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")
SEED_CACHE_WRITE = 1689


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
    ap.add_argument("--workload", default="decode64", choices=["decode64", "long", "prefix", "mixed", "tiny"],
                    help="decode64 (default): 64-request decode; long: 8 x 32768; prefix: 256 requests sharing a "
                         "prefix; mixed: 512-row chunk + 128 decodes; tiny: 4 requests (latency)")
    ap.add_argument("--partition-tokens", type=int, default=0)
    ap.add_argument("--prefix-pass", action="store_true",
                    help="decode a prefix-shared batch with pa_decode_shared (prefix read once per group) instead "
                         "of pa_decode; measured slower on the 256-request batch, whose prefix stays in the caches")
    ap.add_argument("--pool-copies", type=int, default=0, help="0 = enough copies for a >= 1 GB working set")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run one 1 GiB elementwise copy first (counter calibration under rocprofv3)")
    return ap.parse_args()


def kv_bytes(wl) -> int:
    """Algorithmic bytes: K and V rows of every KV head for every context token, read once."""
    NB, BS, Hkv, D = wl.k_cache.shape
    return int(wl.context_lens.to("cpu").long().sum()) * 2 * Hkv * D * wl.k_cache.element_size()


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


def cpu_baseline(wl, min_seconds=10.0):
    """The fp64 oracle over the whole workload on the host cores, repeated for ~min_seconds."""
    from oracle import paged_attention

    threads = int(os.environ.get("OMP_NUM_THREADS", 0)) or len(os.sched_getaffinity(0))
    times = []
    t_all = time.perf_counter()
    while not times or (time.perf_counter() - t_all < min_seconds and len(times) < 1000):
        t0 = time.perf_counter()
        paged_attention(wl.q, wl.k_cache, wl.v_cache, wl.block_tables, wl.context_lens, wl.query_start_loc,
                        scale=wl.scale, threads=threads)
        times.append(time.perf_counter() - t0)
    times.sort()
    t = times[len(times) // 2]
    # the same oracle on one thread: up to 3 runs within about min_seconds
    t1s = []
    t_all = time.perf_counter()
    while not t1s or (time.perf_counter() - t_all + t1s[-1] < min_seconds and len(t1s) < 3):
        t0 = time.perf_counter()
        paged_attention(wl.q, wl.k_cache, wl.v_cache, wl.block_tables, wl.context_lens, wl.query_start_loc,
                        scale=wl.scale, threads=1)
        t1s.append(time.perf_counter() - t0)
    t1s.sort()
    t1 = t1s[len(t1s) // 2]
    return {"value": round(kv_bytes(wl) / t / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "seq_steps_per_s": round(wl.num_seqs / t, 2),
            "sample": f"whole workload ({wl.num_seqs} requests, all heads), median of {len(times)} runs of "
                      f"{t:.3f} s each, fp64 C oracle with OpenMP",
            "single_thread": {"value": round(kv_bytes(wl) / t1 / 1e9, 3), "unit": "GB/s", "cores": 1,
                              "seq_steps_per_s": round(wl.num_seqs / t1, 2),
                              "sample": f"median of {len(t1s)} runs of {t1:.3f} s each"}}


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


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from paged_kv_cache_168_amd import api
    from paged_kv_cache_168_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    wl = W.WORKLOADS[args.workload]()
    mixed = wl.query_start_loc is not None
    pt = args.partition_tokens or wl.meta.get("partition_tokens", 0)
    # a batch whose requests share blocks says so: K/V loads then stay cached for the other readers
    shared = bool(wl.meta.get("prefix_blocks"))
    # with --prefix-pass a batch whose requests share a prefix reads it once per group (pa_decode_shared)
    use_prefix = shared and not mixed and args.prefix_pass
    nbytes = kv_bytes(wl)
    pool_bytes = 2 * wl.k_cache.numel() * wl.k_cache.element_size()
    copies = args.pool_copies or max(1, math.ceil(1.0e9 / pool_bytes))

    q = wl.q.to(dev)
    bt = wl.block_tables.to(dev)
    cl = wl.context_lens.to(dev)
    qsl = wl.query_start_loc.to(dev) if mixed else None
    pools = [(wl.k_cache.to(dev), wl.v_cache.to(dev))]
    for _ in range(copies - 1):
        pools.append((pools[0][0].clone(), pools[0][1].clone()))
    out = torch.empty_like(q)
    params = api.make_params(q, pools[0][0], bt, scale=wl.scale, partition_tokens=pt, shared_blocks=shared)
    if mixed:
        ws_bytes = api.varlen_mixed_workspace_size(params, wl.num_seqs, wl.num_tokens, wl.max_query_len)
    elif use_prefix:
        groups = [x.to(dev) for x in W.prefix_groups(wl)]
        ws_bytes = api.decode_shared_workspace_size(params, wl.num_seqs, int(groups[1].shape[0]))
    else:
        ws_bytes = api.decode_workspace_size(params, wl.num_seqs)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)

    def step(i):
        k, v = pools[i % copies]
        if mixed:
            api.varlen_mixed(q, k, v, bt, cl, qsl, scale=wl.scale, max_query_len=wl.max_query_len, out=out,
                             partition_tokens=pt, shared_blocks=shared, workspace=ws)
        elif use_prefix:
            api.decode_shared(q, k, v, bt, cl, groups[0], groups[1], scale=wl.scale, out=out, shared_blocks=shared,
                              workspace=ws)
        else:
            api.decode(q, k, v, bt, cl, scale=wl.scale, out=out, partition_tokens=pt, shared_blocks=shared,
                       workspace=ws)

    if args.calib_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Timed region 1: steps whose dominant kernel is launched with HIP events attached (hipExtLaunchKernel:
    # they bracket that kernel alone, on the stream it runs on). Each step starts on an idle stream, so the
    # start event is not held up behind the previous step's work. Only the kernel durations are taken from
    # these steps; they also finish warming the clocks up for region 2.
    events = timing_events(args.steps)
    for i, (a, b) in enumerate(events):
        torch.cuda.synchronize()
        api.set_kernel_timing_events(a, b)
        step(args.warmup + i)
    torch.cuda.synchronize()
    kernel_ms = sum(a.elapsed_time(b) for a, b in events) / args.steps

    # Timed region 2: whole steps back to back, nothing recorded between the launches. `value` and
    # `ms_per_step` come from here.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + args.steps + i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    gbps = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / (kernel_ms * 1e-3) / 1e9

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(args.workload)
        if rec and rec.get("kernel_source_hash") == kernel_source_hash():
            traffic = rec.get("bytes_per_launch")

    NB, BS, Hkv, D = wl.k_cache.shape
    result = {
        "metric": METRIC,
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if q.dtype == torch.bfloat16 else "fp32",
        "data": "synthetic (seeded N(0,1) K/V/q, shuffled physical blocks)",
        "config": {
            "workload": wl.name,
            "num_seqs": wl.num_seqs,
            "query_tokens": wl.num_tokens,
            "q_heads": int(q.shape[1]),
            "kv_heads": int(Hkv),
            "head_dim": int(D),
            "block_size": int(BS),
            "context_tokens": int(wl.context_lens.sum()),
            "partition_tokens": pt or 512,  # applies to the partition kernel (chunk rows, other block sizes)
            "pool_copies": copies,
            "entry_point": "pa_varlen_mixed" if mixed else "pa_decode_shared" if use_prefix else "pa_decode",
            "kv_loads": "cached (PA_FLAG_SHARED_BLOCKS)" if shared else "streaming",
        },
        "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
        **({"unique_kv_gbps": round(unique_kv_bytes(wl) / (ms_per_step * 1e-3) / 1e9, 1),
            "unique_kv_bytes": unique_kv_bytes(wl)} if shared else {}),
        "seq_steps_per_s": round(wl.num_seqs / (ms_per_step * 1e-3), 1),
        "roofline": {
            "bound": "hbm",
            "kernel": "decode_balanced_kernel" if int(BS) % 16 == 0 else "decode_partition_kernel",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "kernel_ms": round(kernel_ms, 5),
            "algorithmic_bytes": nbytes,
        },
    }
    if mixed:
        result["query_tokens_per_s"] = round(wl.num_tokens / (ms_per_step * 1e-3), 1)
    ceiling = read_ceiling(dev, min(args.steps, 20))
    result["roofline"]["read_ceiling"] = ceiling
    result["roofline"]["frac_of_read_ceiling"] = round(achieved / ceiling["gbps"], 4)
    result["cache_write"] = time_cache_write(wl, q, pools[0], bt, cl, qsl, args.steps)
    result["block_copy"] = time_block_copy(pools[0], bt, cl, args.steps)
    result["scheduler"] = scheduler_summary()
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
