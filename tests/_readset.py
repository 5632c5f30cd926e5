"""The read-set gate: inputs whose attention output is an exact count of the keys each row reads.

With every query zero, every score is zero, so every visible key gets weight exactly 1 (exp of 0) on any
correct path, and the output of a row with n visible keys is (sum of their V rows) / n. V marks each logical
token i of KV head h with a one-hot row at a dimension that depends on i, by one of two schemes (a case runs
both):

* "tile": the token's 16-token tile, d = (i // 16 + 5h) mod D, so a dropped or repeated tile or piece moves
  16 keys of one dimension at once (a relative change of 1/16 of a dimension's tiles: 6% at 32768 keys, 0.8% at
  262144);
* "token": the token's slot and tile class, d = i % 16 + 16 * ((i // 16 + h) mod (D / 16)), so a dropped,
  repeated or extra single token moves a dimension of its own (1 of n / D keys: visible in bf16 up to about
  4096 keys).

Slots no row may read (past a context, spare and padding blocks) hold 1 in every dimension, so reading one
raises every dimension. The output is then count / n for integer counts: exact in fp32 on every path
(sums of ones, the log-sum-exp merge of partials whose maxima are all 0), and a bf16 value when n is a power of
two. The gate asks for bit equality with the oracle on those rows and, on every other row, for one of the two
bf16 values bracketing the oracle value (fp32 outputs: within two fp32 spacings): far tighter than the accuracy
bound, and tight enough that a missing or extra key (a relative change of at least 1/count) fails it.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle.compare import bf16_round_down_up
from paged_kv_cache_168_amd.workloads import Workload


SCHEMES = ("tile", "token")


def marker_dims(pos: torch.Tensor, h: int, D: int, scheme: str) -> torch.Tensor:
    """The one-hot dimension of logical token positions `pos` (int64 tensor) in KV head h."""
    tile = pos // 16
    if scheme == "tile":
        return (tile + 5 * h) % D
    assert scheme == "token"
    return pos % 16 + 16 * ((tile + h) % (D // 16))


def logical_positions(block_tables, context_lens, num_blocks, block_size) -> torch.Tensor:
    """pos[block, slot] = the logical position every request reading that slot gives it (-1: read by none).
    Raises if two requests read one slot at different positions (the markers could not tell them apart)."""
    pos = torch.full((num_blocks, block_size), -1, dtype=torch.int64)
    bt = block_tables.cpu().long()
    for s, c in enumerate(context_lens.cpu().tolist()):
        if c <= 0:
            continue
        i = torch.arange(c, dtype=torch.int64)
        b = bt[s, i // block_size]
        sl = i % block_size
        prev = pos[b, sl]
        if bool(((prev >= 0) & (prev != i)).any()):
            raise ValueError(f"request {s} reads a slot another request reads at another position")
        pos[b, sl] = i
    return pos


def counting_values(pos: torch.Tensor, num_kv_heads: int, head_dim: int, dtype, scheme: str) -> torch.Tensor:
    """V pool [NB, BS, Hkv, D] of markers for the live slots of `pos` and ones elsewhere."""
    NB, BS = pos.shape
    v = torch.ones((NB, BS, num_kv_heads, head_dim), dtype=dtype)
    live = pos >= 0
    b, sl = torch.nonzero(live, as_tuple=True)
    p = pos[b, sl]
    for h in range(num_kv_heads):
        v[b, sl, h] = 0
        v[b, sl, h, marker_dims(p, h, head_dim, scheme)] = 1
    return v


def counting(wl: Workload, scheme: str = "tile") -> Workload:
    """wl with zero queries and counting values (K, tables, lengths and query layout unchanged)."""
    NB, BS, Hkv, D = wl.k_cache.shape
    pos = logical_positions(wl.block_tables, wl.context_lens, NB, BS)
    v = counting_values(pos, Hkv, D, wl.v_cache.dtype, scheme)
    meta = dict(wl.meta, readset_scheme=scheme)
    return Workload(f"{wl.name} (read-set gate, {scheme})", torch.zeros_like(wl.q), wl.k_cache, v, wl.block_tables,
                    wl.context_lens, wl.query_start_loc, wl.scale, wl.poison_block, meta)


def visible_counts(wl: Workload) -> np.ndarray:
    """n per query token: the keys its rows see (ctx for decode, ctx - q_len + j + 1 for row j of a slice)."""
    ctx = wl.context_lens.cpu().numpy().astype(np.int64)
    if wl.query_start_loc is None:
        return ctx
    qsl = wl.query_start_loc.cpu().numpy().astype(np.int64)
    n = np.zeros(wl.num_tokens, dtype=np.int64)
    for s in range(wl.num_seqs):
        ql = qsl[s + 1] - qsl[s]
        n[qsl[s]:qsl[s + 1]] = ctx[s] - ql + np.arange(ql) + 1
    return n


def closed_form(wl: Workload) -> np.ndarray:
    """The exact output of a counting workload, from the markers alone: out[t, h, d] = count / n, where count is
    the number of positions i < n whose marker in h's KV head is d (float64, no attention arithmetic)."""
    T, Hq, D = wl.q.shape
    Hkv = wl.k_cache.shape[2]
    G = Hq // Hkv
    scheme = wl.meta["readset_scheme"]
    n = visible_counts(wl)
    out = np.zeros((T, Hq, D), dtype=np.float64)
    for t in range(T):
        if n[t] <= 0:
            continue
        i = torch.arange(int(n[t]), dtype=torch.int64)
        for kvh in range(Hkv):
            c = np.bincount(marker_dims(i, kvh, D, scheme).numpy(), minlength=D).astype(np.float64)
            out[t, kvh * G:(kvh + 1) * G] = c / n[t]
    return out


def check_counts(got: torch.Tensor, want: np.ndarray, n: np.ndarray, what: str = "") -> int:
    """The gate: rows whose visible count is a power of two equal to the oracle value bit for bit; every other
    element one of the two bf16 values bracketing it (bf16 output), or within two fp32 spacings of it (fp32
    output, where the reciprocal of the weight sum may be rounded once more). Returns the number of exactly
    checked rows."""
    g = got.detach().cpu().to(torch.float64).numpy().reshape(want.shape)
    if got.dtype == torch.float32:
        bad = np.abs(g - want) > 2 * np.spacing(np.abs(want).astype(np.float32)).astype(np.float64)
        kind = "within two fp32 spacings of"
    else:
        lo, hi = bf16_round_down_up(want)
        bad = ~((g == lo) | (g == hi))
        kind = "a bf16 neighbour of"
    if bad.any():
        t, h, d = (int(x[0]) for x in np.nonzero(bad))
        raise AssertionError(f"{what}: {int(bad.sum())} elements are not {kind} the count (first: token {t} head {h} "
                             f"dim {d}, n {int(n[t])}: got {g[t, h, d]!r}, oracle {want[t, h, d]!r})")
    pow2 = (n > 0) & ((n & (n - 1)) == 0)
    exact_rows = want[pow2]
    assert np.array_equal(*bf16_round_down_up(exact_rows)), f"{what}: a power-of-two row is not a bf16 value"
    mism = g[pow2] != exact_rows
    assert not mism.any(), f"{what}: {int(mism.sum())} elements of power-of-two rows differ from the oracle"
    return int(pow2.sum())
