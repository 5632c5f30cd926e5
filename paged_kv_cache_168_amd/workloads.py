"""Seeded synthetic inputs for paged attention.

This module builds block pools, block tables, context lengths and queries. It
holds none of the attention arithmetic: both the HIP path and the fp64 oracle
consume what it returns, and neither is imported here.

Recipe (all draws from one ``torch.Generator`` seeded per workload, in this
order: context lengths -> physical-block permutation -> q -> K pool -> V pool):

* values are N(0, 1) float32; bf16 workloads cast them with round-to-nearest-
  even. Every pool block is filled, spare blocks included.
* a request's table takes the next unused ids of the permutation in request
  order, so physical ids are scattered and never reused across requests except
  where sharing is the point (prefix and beam sharing).
* the pool holds the blocks the requests need plus 10% spare; padding entries
  of a table (beyond its last used block) hold one spare id, the "poison"
  block, so a kernel that reads padding reads that block.

Shapes follow the pages' workloads: 16-token blocks, 512-token prefill chunks
mixed with decodes, 64-256 concurrent requests, contexts up to 32768, a shared
~500-token system prompt, beam-style branches sharing all but their last block.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

SEED_BASE = 1680


@dataclass
class Workload:
    name: str
    q: torch.Tensor  # [T, Hq, D]
    k_cache: torch.Tensor  # [NB, BS, Hkv, D]
    v_cache: torch.Tensor  # [NB, BS, Hkv, D]
    block_tables: torch.Tensor  # int32 [S, W]
    context_lens: torch.Tensor  # int32 [S]
    query_start_loc: torch.Tensor | None  # int32 [S+1]; None for pure decode
    scale: float
    poison_block: int
    meta: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.block_tables.shape[0])

    @property
    def num_tokens(self) -> int:
        return int(self.q.shape[0])

    @property
    def max_query_len(self) -> int:
        if self.query_start_loc is None:
            return 1
        return int((self.query_start_loc[1:] - self.query_start_loc[:-1]).max().item()) if self.num_seqs else 0

    @property
    def block_size(self) -> int:
        return int(self.k_cache.shape[1])

    @property
    def dims(self) -> dict:
        T, Hq, D = self.q.shape
        NB, BS, Hkv, _ = self.k_cache.shape
        return dict(T=T, Hq=Hq, D=D, NB=NB, BS=BS, Hkv=Hkv, S=self.num_seqs, W=int(self.block_tables.shape[1]))


def blocks_for(n_tokens: int, block_size: int) -> int:
    """Blocks a request of n_tokens cached tokens occupies (allocation on demand)."""
    return -(-n_tokens // block_size)


def pool_with_spare(needed_blocks: int) -> int:
    """Needed blocks plus 10% spare, rounded up, at least one spare (the poison block)."""
    return max(needed_blocks + 1, (11 * needed_blocks + 9) // 10)


def _randn_pool(gen: torch.Generator, shape, dtype: torch.dtype, chunk_blocks: int = 4096) -> torch.Tensor:
    out = torch.empty(shape, dtype=dtype)
    for b0 in range(0, shape[0], chunk_blocks):
        b1 = min(shape[0], b0 + chunk_blocks)
        out[b0:b1] = torch.randn((b1 - b0,) + tuple(shape[1:]), generator=gen, dtype=torch.float32).to(dtype)
    return out


def _tables_from_lists(lists, width: int, pad_id: int) -> torch.Tensor:
    bt = torch.full((len(lists), max(width, 1)), pad_id, dtype=torch.int32)
    for s, ids in enumerate(lists):
        if ids:
            bt[s, : len(ids)] = torch.tensor(ids, dtype=torch.int32)
    return bt


def make_workload(name, gen, ctx, *, Hq, Hkv, D, BS, dtype, q_lens=None, num_blocks=None,
                  table_lists=None, scale=None, meta=None) -> Workload:
    """Assemble a workload once context lengths are drawn.

    ``table_lists`` (list of physical-id lists) may be given for structured
    sharing; otherwise each request takes fresh ids from a seeded permutation.
    """
    ctx = [int(c) for c in ctx]
    S = len(ctx)
    if q_lens is None:
        q_lens = [1] * S
    needed = sum(blocks_for(c, BS) for c in ctx) if table_lists is None else None
    if table_lists is None:
        NB = num_blocks if num_blocks is not None else pool_with_spare(needed)
        perm = torch.randperm(NB, generator=gen).tolist()
        if needed >= NB:
            raise ValueError("pool has no spare block for the poison id")
        lists, cur = [], 0
        for c in ctx:
            nb = blocks_for(c, BS)
            lists.append(perm[cur:cur + nb])
            cur += nb
        poison = perm[-1]
    else:
        NB = num_blocks
        lists = table_lists["lists"]
        poison = table_lists["poison"]
    W = max([len(x) for x in lists] + [1])
    bt = _tables_from_lists(lists, W, poison)
    T = sum(q_lens)
    q = torch.randn((T, Hq, D), generator=gen, dtype=torch.float32).to(dtype)
    k = _randn_pool(gen, (NB, BS, Hkv, D), dtype)
    v = _randn_pool(gen, (NB, BS, Hkv, D), dtype)
    qsl = None
    if any(ql != 1 for ql in q_lens) or (meta or {}).get("force_qsl"):
        qsl = torch.zeros(S + 1, dtype=torch.int32)
        qsl[1:] = torch.cumsum(torch.tensor(q_lens, dtype=torch.int64), 0).to(torch.int32)
    return Workload(name=name, q=q, k_cache=k, v_cache=v, block_tables=bt,
                    context_lens=torch.tensor(ctx, dtype=torch.int32), query_start_loc=qsl,
                    scale=float(scale if scale is not None else 1.0 / math.sqrt(D)),
                    poison_block=int(poison), meta=dict(meta or {}))


def tiny_decode() -> Workload:
    """Tiny fp32 MHA decode: contexts {1, 15, 16, 37}, Hq=Hkv=4, D=64, BS=16, pool of 64 blocks."""
    g = torch.Generator().manual_seed(SEED_BASE + 1)
    return make_workload("tiny fp32 decode (4 seqs, ctx 1/15/16/37, 4:4 heads, D64)", g, [1, 15, 16, 37],
                         Hq=4, Hkv=4, D=64, BS=16, dtype=torch.float32, num_blocks=64)


def decode_64() -> Workload:
    """bf16 decode at a Llama-3-8B layer shape: 64 requests, ctx U[128, 4096], GQA 32:8, D=128."""
    g = torch.Generator().manual_seed(SEED_BASE + 2)
    ctx = torch.randint(128, 4097, (64,), generator=g).tolist()
    return make_workload("bf16 decode 64 seqs ctx U[128,4096] 32:8 heads D128", g, ctx,
                         Hq=32, Hkv=8, D=128, BS=16, dtype=torch.bfloat16)


def long_decode() -> Workload:
    """Long-context bf16 decode: 8 requests x 32768 tokens, GQA 64:8, D=128 (split-K 512)."""
    g = torch.Generator().manual_seed(SEED_BASE + 3)
    return make_workload("bf16 long decode 8 seqs x 32768, 64:8 heads D128", g, [32768] * 8,
                         Hq=64, Hkv=8, D=128, BS=16, dtype=torch.bfloat16, meta={"partition_tokens": 512})


def prefix_shared() -> Workload:
    """Prefix-shared bf16 decode: 256 requests share a 32-block (512-token) prefix; requests 0-63
    form 16 beam groups of 4 that share their suffix except a private last block."""
    g = torch.Generator().manual_seed(SEED_BASE + 4)
    BS, prefix_blocks = 16, 32
    group_len = torch.randint(16, 2049, (16,), generator=g).tolist()
    indep_len = torch.randint(16, 2049, (192,), generator=g).tolist()
    suffix = [group_len[s // 4] for s in range(64)] + indep_len
    needed = prefix_blocks
    for L in group_len:
        needed += (blocks_for(L, BS) - 1) + 4
    for L in indep_len:
        needed += blocks_for(L, BS)
    NB = pool_with_spare(needed)
    perm = torch.randperm(NB, generator=g).tolist()
    prefix = perm[:prefix_blocks]
    cur = prefix_blocks
    lists = []
    for grp in range(16):
        nb = blocks_for(group_len[grp], BS)
        shared = perm[cur:cur + nb - 1]
        cur += nb - 1
        for _ in range(4):
            lists.append(prefix + shared + [perm[cur]])
            cur += 1
    for L in indep_len:
        nb = blocks_for(L, BS)
        lists.append(prefix + perm[cur:cur + nb])
        cur += nb
    ctx = [prefix_blocks * BS + L for L in suffix]
    # what a beam-search scheduler knows: each beam group shares the prompt prefix and its own blocks but the last;
    # the other 192 requests share the prompt prefix
    beam_start = [4 * grp for grp in range(16)] + [64, 256]
    beam_prefix = [(prefix_blocks + blocks_for(group_len[grp], BS) - 1) * BS for grp in range(16)] + [prefix_blocks * BS]
    return make_workload("bf16 prefix-shared decode 256 seqs (512-token shared prefix, 16x4 beams)", g, ctx,
                         Hq=32, Hkv=8, D=128, BS=BS, dtype=torch.bfloat16, num_blocks=NB,
                         table_lists={"lists": lists, "poison": perm[-1]},
                         meta={"unique_blocks": needed, "prefix_blocks": prefix_blocks,
                               "beam_group_start": beam_start, "beam_group_prefix": beam_prefix})


def mixed_step(chunk_position: str = "first") -> Workload:
    """Mixed chunked-prefill step: one 512-token causal chunk at offset 2048 of a 4096-token
    prompt (ctx 2560 once its own K/V is cached) plus 128 decodes with ctx U[256, 8192]."""
    g = torch.Generator().manual_seed(SEED_BASE + 5)
    dec = torch.randint(256, 8193, (128,), generator=g).tolist()
    chunk_ctx, chunk_q = 2048 + 512, 512
    pos = {"first": 0, "middle": 64, "last": 128}[chunk_position]
    ctx = dec[:pos] + [chunk_ctx] + dec[pos:]
    q_lens = [1] * pos + [chunk_q] + [1] * (128 - pos)
    return make_workload(f"bf16 mixed step: 512-token causal chunk ({chunk_position}) + 128 decodes", g, ctx,
                         Hq=32, Hkv=8, D=128, BS=16, dtype=torch.bfloat16, q_lens=q_lens,
                         meta={"chunk_seq": pos})


# The benchmarked workloads by name (bench.py --workload).
WORKLOADS = {"tiny": tiny_decode, "decode64": decode_64, "long": long_decode, "prefix": prefix_shared,
             "mixed": mixed_step}


def prefix_groups(wl: Workload, beams: bool = True):
    """(group_start, group_prefix) int32 tensors describing the shared prefixes of a workload built with them.
    The prefix-shared batch: with beams, its 16 beam groups (each sharing the prompt prefix and its beams' common
    blocks) and one group of the other 192 requests; without, one group of all 256 requests sharing the 512-token
    prompt prefix. grouped_workload: its groups."""
    if beams and "beam_group_start" in wl.meta:
        return (torch.tensor(wl.meta["beam_group_start"], dtype=torch.int32),
                torch.tensor(wl.meta["beam_group_prefix"], dtype=torch.int32))
    if "group_start" in wl.meta:
        return (torch.tensor(wl.meta["group_start"], dtype=torch.int32),
                torch.tensor(wl.meta["group_prefix"], dtype=torch.int32))
    bs = wl.k_cache.shape[1]
    return (torch.tensor([0, wl.num_seqs], dtype=torch.int32),
            torch.tensor([wl.meta.get("prefix_blocks", 0) * bs], dtype=torch.int32))


def grouped_workload(seed: int, groups, *, Hq=32, Hkv=8, D=128, BS=16, dtype=torch.bfloat16) -> Workload:
    """Requests in groups that share the blocks of a common prefix. groups: [(prefix_tokens, [ctx, ...]), ...]
    with prefix_tokens a multiple of BS; a request whose context is shorter than its group's prefix uses the
    prefix blocks that cover it. Every other block is private."""
    g = torch.Generator().manual_seed(seed)
    needed = 0
    for pre, ctxs in groups:
        needed += pre // BS + sum(max(0, blocks_for(c, BS) - pre // BS) for c in ctxs)
    NB = pool_with_spare(needed)
    perm = torch.randperm(NB, generator=g).tolist()
    lists, ctx_all, starts, prefixes, cur = [], [], [0], [], 0
    for pre, ctxs in groups:
        shared = perm[cur:cur + pre // BS]
        cur += pre // BS
        for c in ctxs:
            own = max(0, blocks_for(c, BS) - pre // BS)
            lists.append((shared + perm[cur:cur + own])[:max(1, blocks_for(c, BS))])
            cur += own
            ctx_all.append(c)
        starts.append(len(ctx_all))
        prefixes.append(pre)
    return make_workload(f"grouped seed={seed}", g, ctx_all, Hq=Hq, Hkv=Hkv, D=D, BS=BS, dtype=dtype, num_blocks=NB,
                         table_lists={"lists": lists, "poison": perm[-1]},
                         meta={"group_start": starts, "group_prefix": prefixes})


def random_workload(seed: int, *, ctx, q_lens=None, Hq=4, Hkv=1, D=128, BS=16, dtype=torch.bfloat16,
                    spare: int | None = None, force_qsl: bool = False) -> Workload:
    """Small seeded workload with explicit context lengths (and optional query lengths)."""
    g = torch.Generator().manual_seed(seed)
    needed = sum(blocks_for(int(c), BS) for c in ctx)
    nb = needed + (spare if spare is not None else max(1, needed // 10 + 1))
    return make_workload(f"random seed={seed}", g, ctx, Hq=Hq, Hkv=Hkv, D=D, BS=BS, dtype=dtype,
                         q_lens=q_lens, num_blocks=nb, meta={"force_qsl": force_qsl})
