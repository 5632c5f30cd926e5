"""Pins for the fp64 oracle: each checks it against something other than itself.

Every pin takes ``lib_path`` (None = the built oracle) so that the mutation
tests can run the same battery against deliberately broken copies of the
oracle's C source. A pin raises AssertionError (or ValueError from the oracle)
when the oracle disagrees with what the pages or the mathematics fix.

Kinds of pin used here:
* library routine: torch's scaled_dot_product_attention in float64 on the
  contiguous (never paged) keys and values, with an explicit bottom-right
  causal mask for chunk rows;
* closed forms: one visible key returns its value exactly; a zero query
  returns the mean of the visible values; constant values are returned
  unchanged; two keys with scores 0 and 1 give (e^-1 v0 + v1) / (1 + e^-1);
* invariants: relabelling physical blocks, changing the block size and
  sharing prefix blocks leave the output bit-identical; a chunk row equals a
  decode row with the truncated context;
* the pages' worked tables: which physical (block, slot) pairs a request reads;
* poison: every slot that must not be read holds NaN.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

from oracle import bf16_to_float64, paged_attention, read_counts

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------------------------------------
# input construction: start from contiguous per-request K/V and scatter them into a shuffled pool
# ----------------------------------------------------------------------------------------------
def paged_from_contiguous(keys, values, block_size, gen, *, dtype=torch.float32, spare=3, poison=float("nan"),
                          table_width=None):
    """keys[s], values[s]: float32 [ctx_s, Hkv, D]. Returns (k_cache, v_cache, block_tables, poison_id).

    Logical token i of request s goes to physical block table[s][i // BS], slot i % BS (the pages'
    logical-block definition). Slots that hold no token, spare blocks and the padding block are
    filled with ``poison``.
    """
    Hkv, D = keys[0].shape[1:] if len(keys) else (1, 1)
    nbs = [-(-k.shape[0] // block_size) for k in keys]
    NB = sum(nbs) + spare
    perm = torch.randperm(NB, generator=gen).tolist()
    pool_k = torch.full((NB, block_size, Hkv, D), poison, dtype=torch.float32)
    pool_v = torch.full((NB, block_size, Hkv, D), poison, dtype=torch.float32)
    W = table_width or max(nbs + [1])
    pad_id = perm[-1]
    bt = torch.full((len(keys), W), pad_id, dtype=torch.int32)
    cur = 0
    for s, (k, v) in enumerate(zip(keys, values)):
        ids = perm[cur:cur + nbs[s]]
        cur += nbs[s]
        bt[s, : len(ids)] = torch.tensor(ids, dtype=torch.int32)
        for i in range(k.shape[0]):
            pool_k[ids[i // block_size], i % block_size] = k[i]
            pool_v[ids[i // block_size], i % block_size] = v[i]
    return pool_k.to(dtype), pool_v.to(dtype), bt, pad_id


def _randn(gen, *shape, dtype=torch.float32):
    # values are rounded to the storage dtype first so both sides see identical numbers
    return torch.randn(*shape, generator=gen).to(dtype).to(torch.float32)


def _sdpa_reference(q_rows, keys, values, n_vis, scale, G):
    """float64 SDPA for one request: q_rows [n_q, Hq, D]; keys/values [ctx, Hkv, D];
    row r sees keys 0 .. n_vis[r]-1 (explicit boolean mask)."""
    q = q_rows.to(torch.float64).permute(1, 0, 2).unsqueeze(0)  # [1, Hq, n_q, D]
    k = keys.to(torch.float64).repeat_interleave(G, dim=1).permute(1, 0, 2).unsqueeze(0).contiguous()
    v = values.to(torch.float64).repeat_interleave(G, dim=1).permute(1, 0, 2).unsqueeze(0).contiguous()
    n_q, ctx = q_rows.shape[0], keys.shape[0]
    mask = torch.arange(ctx).unsqueeze(0) < torch.tensor(n_vis).unsqueeze(1)  # [n_q, ctx]
    out = F.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=scale)
    return out.squeeze(0).permute(1, 0, 2).numpy()  # [n_q, Hq, D]


# ----------------------------------------------------------------------------------------------
# pins
# ----------------------------------------------------------------------------------------------
def pin_sdpa_decode_gqa(lib_path=None, dtype=torch.float32):
    """Decode batch, GQA 4:1 plus MHA-like heads, ragged contexts, vs float64 SDPA."""
    gen = torch.Generator().manual_seed(11)
    ctxs = [1, 5, 16, 17, 40, 33]
    Hq, Hkv, D, BS = 8, 2, 16, 16
    keys = [_randn(gen, c, Hkv, D, dtype=dtype) for c in ctxs]
    values = [_randn(gen, c, Hkv, D, dtype=dtype) for c in ctxs]
    q = _randn(gen, len(ctxs), Hq, D, dtype=dtype)
    kc, vc, bt, _ = paged_from_contiguous(keys, values, BS, gen, dtype=dtype)
    scale = 1.0 / math.sqrt(D)
    got = paged_attention(q.to(dtype), kc, vc, bt, torch.tensor(ctxs, dtype=torch.int32), scale=scale,
                          lib_path=lib_path)
    for s, c in enumerate(ctxs):
        ref = _sdpa_reference(q[s:s + 1], keys[s], values[s], [c], float(np.float32(scale)), Hq // Hkv)
        err = np.abs(got[s] - ref[0]).max()
        assert err <= 1e-12, f"decode row {s}: |oracle - sdpa| = {err}"


def pin_sdpa_mixed_causal(lib_path=None, dtype=torch.bfloat16):
    """Mixed batch: chunk rows with a bottom-right causal mask next to decode rows, vs SDPA."""
    gen = torch.Generator().manual_seed(12)
    ctxs = [21, 9, 50, 3]
    qls = [1, 6, 19, 3]
    Hq, Hkv, D, BS = 4, 2, 8, 4
    keys = [_randn(gen, c, Hkv, D, dtype=dtype) for c in ctxs]
    values = [_randn(gen, c, Hkv, D, dtype=dtype) for c in ctxs]
    T = sum(qls)
    q = _randn(gen, T, Hq, D, dtype=dtype)
    kc, vc, bt, _ = paged_from_contiguous(keys, values, BS, gen, dtype=dtype)
    qsl = torch.tensor([0] + list(np.cumsum(qls)), dtype=torch.int32)
    scale = 0.3
    got = paged_attention(q.to(dtype), kc, vc, bt, torch.tensor(ctxs, dtype=torch.int32), qsl, scale=scale,
                          lib_path=lib_path)
    for s, (c, ql) in enumerate(zip(ctxs, qls)):
        t0 = int(qsl[s])
        n_vis = [c - ql + j + 1 for j in range(ql)]
        ref = _sdpa_reference(q[t0:t0 + ql], keys[s], values[s], n_vis, float(np.float32(scale)), Hq // Hkv)
        err = np.abs(got[t0:t0 + ql] - ref).max()
        assert err <= 1e-12, f"request {s}: |oracle - sdpa| = {err}"


def pin_sdpa_compact_pool(lib_path=None):
    """SDPA agreement with used blocks packed into the low ids of a large pool and a table wider
    than the block size, so that a wrong table column or kv-head stride still reads in-bounds
    (wrong) data and fails on value rather than by crashing."""
    gen = torch.Generator().manual_seed(10)
    ctxs = [29, 7, 32]
    Hq, Hkv, D, BS = 4, 2, 8, 4
    keys = [_randn(gen, c, Hkv, D) for c in ctxs]
    values = [_randn(gen, c, Hkv, D) for c in ctxs]
    q = _randn(gen, len(ctxs), Hq, D)
    kc, vc, bt, _ = paged_from_contiguous(keys, values, BS, gen, spare=0, table_width=8)
    used = kc.shape[0]
    NB = 4 * used
    kc = torch.cat([kc, torch.zeros((NB - used,) + tuple(kc.shape[1:]))])
    vc = torch.cat([vc, torch.zeros((NB - used,) + tuple(vc.shape[1:]))])
    got = paged_attention(q, kc, vc, bt, torch.tensor(ctxs, dtype=torch.int32), scale=0.5, lib_path=lib_path)
    for s, c in enumerate(ctxs):
        ref = _sdpa_reference(q[s:s + 1], keys[s], values[s], [c], 0.5, Hq // Hkv)
        assert np.abs(got[s] - ref[0]).max() <= 1e-12, f"compact-pool row {s} disagrees with sdpa"


def pin_one_token_context_is_v(lib_path=None):
    """With one visible key the weight is exp(0)/exp(0) = 1: the output is that value, exactly."""
    gen = torch.Generator().manual_seed(13)
    Hq, Hkv, D, BS = 4, 2, 32, 16
    keys = [_randn(gen, 1, Hkv, D, dtype=torch.bfloat16) for _ in range(3)]
    values = [_randn(gen, 1, Hkv, D, dtype=torch.bfloat16) for _ in range(3)]
    q = _randn(gen, 3, Hq, D, dtype=torch.bfloat16)
    kc, vc, bt, _ = paged_from_contiguous(keys, values, BS, gen, dtype=torch.bfloat16)
    got = paged_attention(q.to(torch.bfloat16), kc, vc, bt, torch.ones(3, dtype=torch.int32), scale=0.125,
                          lib_path=lib_path)
    for s in range(3):
        for h in range(Hq):
            want = values[s][0, h // (Hq // Hkv)].to(torch.float64).numpy()
            assert np.array_equal(got[s, h], want), f"seq {s} head {h}: one-token output is not V"


def pin_zero_query_is_mean(lib_path=None):
    """q = 0 makes every score 0, so the output is the plain mean of the visible values."""
    gen = torch.Generator().manual_seed(14)
    ctxs = [7, 31, 64]
    Hq, Hkv, D, BS = 2, 1, 8, 16
    keys = [_randn(gen, c, Hkv, D) for c in ctxs]
    values = [_randn(gen, c, Hkv, D) for c in ctxs]
    kc, vc, bt, _ = paged_from_contiguous(keys, values, BS, gen)
    got = paged_attention(torch.zeros(3, Hq, D), kc, vc, bt, torch.tensor(ctxs, dtype=torch.int32), scale=1.0,
                          lib_path=lib_path)
    for s, c in enumerate(ctxs):
        want = values[s][:, 0].to(torch.float64).mean(0).numpy()
        for h in range(Hq):
            assert np.abs(got[s, h] - want).max() <= 1e-14, f"seq {s}: zero-query output is not the mean"


def pin_constant_values(lib_path=None):
    """If every visible value equals c, the output is c whatever the scores are."""
    gen = torch.Generator().manual_seed(15)
    ctxs = [3, 45]
    Hq, Hkv, D, BS = 4, 4, 8, 16
    keys = [_randn(gen, c, Hkv, D) * 3 for c in ctxs]
    c_vec = _randn(gen, Hkv, D)
    values = [c_vec.unsqueeze(0).repeat(c, 1, 1) for c in ctxs]
    q = _randn(gen, 2, Hq, D)
    kc, vc, bt, _ = paged_from_contiguous(keys, values, BS, gen)
    got = paged_attention(q, kc, vc, bt, torch.tensor(ctxs, dtype=torch.int32), scale=0.7, lib_path=lib_path)
    for s in range(2):
        assert np.abs(got[s] - c_vec.to(torch.float64).numpy()).max() <= 1e-14


def pin_two_keys_closed_form(lib_path=None):
    """Scores 0 and 1: out = (e^-1 v0 + v1) / (1 + e^-1). (The pages' printed loop, which adds the
    second weight without rescaling the running sum, would divide by 2 instead.)"""
    D = 4
    q = torch.zeros(1, 1, D)
    q[0, 0, 0] = 1.0
    k0 = torch.zeros(1, 1, D)
    k1 = torch.zeros(1, 1, D)
    k1[0, 0, 0] = 1.0
    v0 = torch.tensor([[[1.0, -2.0, 0.5, 3.0]]])
    v1 = torch.tensor([[[-1.0, 4.0, 0.25, 0.0]]])
    gen = torch.Generator().manual_seed(16)
    kc, vc, bt, _ = paged_from_contiguous([torch.cat([k0, k1])], [torch.cat([v0, v1])], 16, gen)
    got = paged_attention(q, kc, vc, bt, torch.tensor([2], dtype=torch.int32), scale=1.0, lib_path=lib_path)[0, 0]
    e = math.exp(-1.0)
    want = (e * v0[0, 0].double().numpy() + v1[0, 0].double().numpy()) / (1.0 + e)
    assert np.abs(got - want).max() <= 1e-15, f"two-key closed form violated: {got} vs {want}"


def pin_large_scores_stay_finite(lib_path=None):
    """Scores near +-1000: softmax is shift invariant, so the result must stay finite and pick the
    top-scoring key's value (the others are e^-(>=100) smaller)."""
    D, n = 4, 6
    gen = torch.Generator().manual_seed(17)
    q = torch.zeros(1, 1, D)
    q[0, 0, 0] = 1.0
    scores = torch.tensor([900.0, 1000.0, -1000.0, 700.0, 850.0, 600.0])
    keys = torch.zeros(n, 1, D)
    keys[:, 0, 0] = scores
    values = _randn(gen, n, 1, D)
    kc, vc, bt, _ = paged_from_contiguous([keys], [values], 16, gen)
    got = paged_attention(q, kc, vc, bt, torch.tensor([n], dtype=torch.int32), scale=1.0, lib_path=lib_path)[0, 0]
    assert np.all(np.isfinite(got)), "overflow: scores were not shifted by their maximum"
    assert np.abs(got - values[1, 0].double().numpy()).max() <= 1e-15


def pin_permutation_invariance(lib_path=None):
    """Relabel physical blocks by a permutation and move the data with them: bit-identical output."""
    gen = torch.Generator().manual_seed(18)
    ctxs = [40, 1, 17, 64]
    Hq, Hkv, D, BS = 4, 2, 16, 16
    keys = [_randn(gen, c, Hkv, D) for c in ctxs]
    values = [_randn(gen, c, Hkv, D) for c in ctxs]
    q = _randn(gen, 4, Hq, D)
    kc, vc, bt, _ = paged_from_contiguous(keys, values, BS, gen, poison=0.0)
    cl = torch.tensor(ctxs, dtype=torch.int32)
    a = paged_attention(q, kc, vc, bt, cl, scale=0.25, lib_path=lib_path)
    NB = kc.shape[0]
    pi = torch.randperm(NB, generator=gen)
    kc2 = torch.empty_like(kc)
    vc2 = torch.empty_like(vc)
    kc2[pi] = kc
    vc2[pi] = vc
    bt2 = pi[bt.long()].to(torch.int32)
    b = paged_attention(q, kc2, vc2, bt2, cl, scale=0.25, lib_path=lib_path)
    assert np.array_equal(a, b), "output changed when physical ids were relabelled"


def pin_block_size_invariance(lib_path=None):
    """The same logical K/V stored with block size 1, 16 and 32: bit-identical output."""
    gen = torch.Generator().manual_seed(19)
    ctxs = [1, 16, 33, 70]
    Hq, Hkv, D = 6, 3, 8
    keys = [_randn(gen, c, Hkv, D) for c in ctxs]
    values = [_randn(gen, c, Hkv, D) for c in ctxs]
    q = _randn(gen, 4, Hq, D)
    cl = torch.tensor(ctxs, dtype=torch.int32)
    outs = []
    for BS in (1, 16, 32):
        kc, vc, bt, _ = paged_from_contiguous(keys, values, BS, gen)
        outs.append(paged_attention(q, kc, vc, bt, cl, scale=0.5, lib_path=lib_path))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2]), "block size changed the output"


def pin_shared_prefix(lib_path=None):
    """Request A reads shared prefix blocks, request B private copies of the same data: identical."""
    gen = torch.Generator().manual_seed(20)
    Hq, Hkv, D, BS = 4, 1, 8, 4
    prefix_k = _randn(gen, 12, Hkv, D)
    prefix_v = _randn(gen, 12, Hkv, D)
    suffix_k = _randn(gen, 5, Hkv, D)
    suffix_v = _randn(gen, 5, Hkv, D)
    keys = [torch.cat([prefix_k, suffix_k])] * 2
    values = [torch.cat([prefix_v, suffix_v])] * 2
    kc, vc, bt, _ = paged_from_contiguous(keys, values, BS, gen)
    # third request shares the first request's prefix blocks (3 blocks) and has its own suffix copy
    bt3 = bt[0].clone()
    NB = kc.shape[0]
    extra_k = torch.full((2, BS, Hkv, D), float("nan"))
    extra_v = torch.full((2, BS, Hkv, D), float("nan"))
    extra_k[:, :] = kc[bt[0, 3:5].long()]
    extra_v[:, :] = vc[bt[0, 3:5].long()]
    kc = torch.cat([kc, extra_k])
    vc = torch.cat([vc, extra_v])
    bt3[3:5] = torch.tensor([NB, NB + 1], dtype=torch.int32)
    bt = torch.cat([bt, bt3.unsqueeze(0)])
    q1 = _randn(gen, 1, Hq, D)
    q = q1.repeat(3, 1, 1)
    out = paged_attention(q, kc, vc, bt, torch.tensor([17, 17, 17], dtype=torch.int32), scale=0.4,
                          lib_path=lib_path)
    assert np.array_equal(out[0], out[1]) and np.array_equal(out[0], out[2]), "shared and private copies differ"


def pin_chunk_row_is_truncated_decode(lib_path=None):
    """Row j of a causal chunk equals a decode with context ctx - q_len + j + 1, bit for bit."""
    gen = torch.Generator().manual_seed(21)
    Hq, Hkv, D, BS = 4, 2, 8, 8
    ctx, ql = 30, 7
    keys = [_randn(gen, ctx, Hkv, D)]
    values = [_randn(gen, ctx, Hkv, D)]
    kc, vc, bt, _ = paged_from_contiguous(keys, values, BS, gen)
    q = _randn(gen, ql, Hq, D)
    chunk = paged_attention(q, kc, vc, bt, torch.tensor([ctx], dtype=torch.int32),
                            torch.tensor([0, ql], dtype=torch.int32), scale=0.6, lib_path=lib_path)
    for j in range(ql):
        dec = paged_attention(q[j:j + 1], kc, vc, bt, torch.tensor([ctx - ql + j + 1], dtype=torch.int32),
                              scale=0.6, lib_path=lib_path)
        assert np.array_equal(chunk[j], dec[0]), f"chunk row {j} differs from the truncated decode"


def pin_zero_context_gives_zeros(lib_path=None):
    gen = torch.Generator().manual_seed(22)
    keys = [_randn(gen, 5, 1, 4), _randn(gen, 1, 1, 4)]
    values = [_randn(gen, 5, 1, 4), _randn(gen, 1, 1, 4)]
    kc, vc, bt, _ = paged_from_contiguous(keys, values, 4, gen)
    out = paged_attention(_randn(gen, 2, 2, 4), kc, vc, bt, torch.tensor([0, 1], dtype=torch.int32), scale=1.0,
                          lib_path=lib_path)
    assert np.array_equal(out[0], np.zeros_like(out[0])) and np.all(np.isfinite(out))


def pin_worked_block_table(lib_path=None):
    """The pages' example table 0->7, 1->12, 2->3, 3->19: exactly those slots are read."""
    with open(os.path.join(GOLDEN, "worked_block_table.json")) as f:
        g = json.load(f)
    BS, NB = g["block_size"], g["num_blocks"]
    for case in g["cases"]:
        bt = torch.tensor([g["block_table"]], dtype=torch.int32)
        cnt = read_counts(bt, torch.tensor([case["context_len"]], dtype=torch.int32), num_tokens=1,
                          num_q_heads=1, num_kv_heads=1, block_size=BS, num_blocks=NB, lib_path=lib_path)
        want = np.zeros((NB, BS), dtype=np.int64)
        for blk, (lo, hi) in case["reads"].items():
            want[int(blk), lo:hi + 1] = 1
        assert np.array_equal(cnt, want), f"context {case['context_len']}: wrong (block, slot) reads"
        # and the values read are the ones at those slots: a zero query averages exactly them
        gen = torch.Generator().manual_seed(23)
        vc = torch.full((NB, BS, 1, 2), float("nan"))
        kc = torch.zeros((NB, BS, 1, 2))
        vals = []
        for blk, (lo, hi) in case["reads"].items():
            x = _randn(gen, hi - lo + 1, 1, 2)
            vc[int(blk), lo:hi + 1] = x
            vals.append(x)
        out = paged_attention(torch.zeros(1, 1, 2), kc, vc, bt, torch.tensor([case["context_len"]], dtype=torch.int32),
                              scale=1.0, lib_path=lib_path)
        want_mean = torch.cat(vals).double().mean(0)[0].numpy()
        assert np.abs(out[0, 0] - want_mean).max() <= 1e-15


def pin_logical_blocks_48(lib_path=None):
    """48 tokens with 16-token blocks are logical blocks 0..2 covering tokens 0-15, 16-31, 32-47."""
    with open(os.path.join(GOLDEN, "logical_blocks_48_tokens.json")) as f:
        g = json.load(f)
    BS, ctx = g["block_size"], g["context_len"]
    table = [5, 0, 9]
    cnt = read_counts(torch.tensor([table], dtype=torch.int32), torch.tensor([ctx], dtype=torch.int32),
                      num_tokens=1, num_q_heads=1, num_kv_heads=1, block_size=BS, num_blocks=10, lib_path=lib_path)
    for b, (lo, hi) in enumerate(g["logical_blocks"]):
        assert hi - lo + 1 == BS
        assert cnt[table[b]].tolist() == [1] * BS, f"logical block {b} not read in full from physical {table[b]}"
    assert cnt.sum() == ctx


def pin_block_reuse_tables(lib_path=None):
    """The pages' allocate/free/reuse figure: reads follow the tables before and after the reuse."""
    with open(os.path.join(GOLDEN, "block_reuse_after_free.json")) as f:
        g = json.load(f)
    BS, NB = g["block_size"], g["num_blocks"]
    for phase in ("before", "after"):
        tabs, ctxs = g[phase]["tables"], g[phase]["context_lens"]
        W = max(len(t) for t in tabs)
        bt = torch.tensor([t + [t[-1]] * (W - len(t)) for t in tabs], dtype=torch.int32)
        cnt = read_counts(bt, torch.tensor(ctxs, dtype=torch.int32), num_tokens=len(tabs), num_q_heads=1,
                          num_kv_heads=1, block_size=BS, num_blocks=NB, lib_path=lib_path)
        want = np.zeros((NB, BS), dtype=np.int64)
        for t, c in zip(tabs, ctxs):
            for i in range(c):
                want[t[i // BS], i % BS] += 1
        assert np.array_equal(cnt, want)
        assert cnt[7].sum() == 0


def pin_poison_never_read(lib_path=None):
    """NaN in every slot outside the contexts (tails of last blocks, spare and padding blocks):
    the output must be finite and equal to the same run with the NaNs replaced by 1e30."""
    gen = torch.Generator().manual_seed(24)
    ctxs = [13, 16, 2, 50]
    qls = [1, 4, 1, 9]
    Hq, Hkv, D, BS = 4, 2, 8, 16
    keys = [_randn(gen, c, Hkv, D, dtype=torch.bfloat16) for c in ctxs]
    values = [_randn(gen, c, Hkv, D, dtype=torch.bfloat16) for c in ctxs]
    q = _randn(gen, sum(qls), Hq, D, dtype=torch.bfloat16).to(torch.bfloat16)
    qsl = torch.tensor([0] + list(np.cumsum(qls)), dtype=torch.int32)
    cl = torch.tensor(ctxs, dtype=torch.int32)
    outs = []
    for poison in (float("nan"), 1e30):
        g2 = torch.Generator().manual_seed(25)
        kc, vc, bt, _ = paged_from_contiguous(keys, values, BS, g2, dtype=torch.bfloat16, poison=poison,
                                              table_width=6)
        outs.append(paged_attention(q, kc, vc, bt, cl, qsl, scale=0.35, lib_path=lib_path))
    assert np.all(np.isfinite(outs[0])), "a poisoned slot was read"
    assert np.array_equal(outs[0], outs[1])


def pin_bf16_widening(lib_path=None):
    """bf16 inputs are widened exactly: a single-key context returns the bf16 value as a double."""
    v = torch.tensor([[[[1.0078125, -3.140625, 65280.0, 1.1754944e-38]]]], dtype=torch.bfloat16)
    k = torch.zeros_like(v)
    out = paged_attention(torch.zeros(1, 1, 4, dtype=torch.bfloat16), k, v, torch.tensor([[0]], dtype=torch.int32),
                          torch.tensor([1], dtype=torch.int32), scale=1.0, lib_path=lib_path)
    assert np.array_equal(out[0, 0], bf16_to_float64(v)[0, 0, 0])
    assert out[0, 0, 0] == 1.0078125 and out[0, 0, 2] == 65280.0


def pin_mixed_query_rows_are_tokens(lib_path=None):
    """In a mixed batch, query row t belongs to the request whose [qsl[s], qsl[s+1]) contains t:
    permuting the request order (and the query rows with it) permutes the output rows."""
    gen = torch.Generator().manual_seed(26)
    ctxs = [9, 30, 4]
    qls = [1, 5, 2]
    Hq, Hkv, D, BS = 2, 1, 8, 8
    keys = [_randn(gen, c, Hkv, D) for c in ctxs]
    values = [_randn(gen, c, Hkv, D) for c in ctxs]
    qs = [_randn(gen, ql, Hq, D) for ql in qls]
    outs = {}
    for order in ([0, 1, 2], [2, 0, 1]):
        g2 = torch.Generator().manual_seed(27)
        kc, vc, bt, _ = paged_from_contiguous([keys[i] for i in order], [values[i] for i in order], BS, g2)
        qsl = torch.tensor([0] + list(np.cumsum([qls[i] for i in order])), dtype=torch.int32)
        out = paged_attention(torch.cat([qs[i] for i in order]), kc, vc, bt,
                              torch.tensor([ctxs[i] for i in order], dtype=torch.int32), qsl, scale=0.5,
                              lib_path=lib_path)
        for pos, i in enumerate(order):
            outs.setdefault(i, []).append(out[int(qsl[pos]):int(qsl[pos + 1])])
    for i in outs:
        assert np.array_equal(outs[i][0], outs[i][1])


ALL_PINS = [
    pin_sdpa_compact_pool,
    pin_sdpa_decode_gqa,
    pin_sdpa_mixed_causal,
    pin_one_token_context_is_v,
    pin_zero_query_is_mean,
    pin_constant_values,
    pin_two_keys_closed_form,
    pin_large_scores_stay_finite,
    pin_permutation_invariance,
    pin_block_size_invariance,
    pin_shared_prefix,
    pin_chunk_row_is_truncated_decode,
    pin_zero_context_gives_zeros,
    pin_worked_block_table,
    pin_logical_blocks_48,
    pin_block_reuse_tables,
    pin_poison_never_read,
    pin_bf16_widening,
    pin_mixed_query_rows_are_tokens,
]


# ----------------------------------------------------------------------------------------------
# KV-cache write
# ----------------------------------------------------------------------------------------------
def _cache_case(gen, ctx, q_lens, BS, Hkv=2, D=8, dtype=torch.float32, spare=4):
    """A shuffled pool holding each request's cached tokens before this step, plus the step's new rows.

    Returns (k_pool, v_pool, block_tables, context_lens, qsl, k_new, v_new, k_logical, v_logical) where
    k_logical[s] is the request's whole context after the step [ctx, Hkv, D] (old prefix, then new rows)."""
    S = len(ctx)
    k_log = [_randn(gen, c, Hkv, D, dtype=dtype) for c in ctx]
    v_log = [_randn(gen, c, Hkv, D, dtype=dtype) for c in ctx]
    nblk = [-(-c // BS) for c in ctx]
    NB = sum(nblk) + spare
    W = max(nblk)
    perm = torch.randperm(NB, generator=gen)
    k_pool = _randn(gen, NB, BS, Hkv, D, dtype=dtype)  # stale data everywhere
    v_pool = _randn(gen, NB, BS, Hkv, D, dtype=dtype)
    bt = torch.full((S, W), int(perm[-1]), dtype=torch.int32)
    used = 0
    for s in range(S):
        ids = perm[used:used + nblk[s]]
        used += nblk[s]
        bt[s, :nblk[s]] = ids.to(torch.int32)
        old = ctx[s] - q_lens[s]
        for i in range(old):  # the prefix is already cached
            k_pool[int(ids[i // BS]), i % BS] = k_log[s][i]
            v_pool[int(ids[i // BS]), i % BS] = v_log[s][i]
    k_new = torch.cat([k_log[s][ctx[s] - q_lens[s]:] for s in range(S)])
    v_new = torch.cat([v_log[s][ctx[s] - q_lens[s]:] for s in range(S)])
    qsl = torch.tensor([0] + list(np.cumsum(q_lens)), dtype=torch.int32)
    cast = lambda x: x.to(dtype)  # stored in the element type (exact: the values are already rounded to it)
    return (cast(k_pool), cast(v_pool), bt, torch.tensor(ctx, dtype=torch.int32), qsl, cast(k_new), cast(v_new),
            [cast(x) for x in k_log], [cast(x) for x in v_log])


def _gather(pool, table_row, n, BS):
    """Contiguous [n, Hkv, D] view of a request's logical tokens, by one vectorised index."""
    i = torch.arange(n)
    return pool[table_row.long()[i // BS], i % BS]


def _as_torch(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.view(torch.bfloat16) if dtype == torch.bfloat16 else t


def pin_cache_write_gather(lib_path=None):
    """After the write, gathering every request's context through its table gives the old prefix
    followed by the new rows, bit for bit (decode batch and mixed batch, fp32 and bf16)."""
    from oracle import cache_write

    for dtype, q_lens, ctx, BS in ((torch.float32, [1, 1, 1, 1], [1, 16, 17, 40], 16),
                                   (torch.bfloat16, [3, 1, 20, 1], [3, 9, 50, 33], 16),
                                   (torch.float32, [5, 2, 1], [12, 7, 30], 5)):
        gen = torch.Generator().manual_seed(4100 + BS + len(ctx))
        kp, vp, bt, cl, qsl, kn, vn, k_log, v_log = _cache_case(gen, ctx, q_lens, BS, dtype=dtype)
        decode = all(x == 1 for x in q_lens)
        k2, v2 = cache_write(kp, vp, kn, vn, bt, cl, None if decode else qsl, lib_path=lib_path)
        k2, v2 = _as_torch(k2, dtype), _as_torch(v2, dtype)
        for s in range(len(ctx)):
            assert torch.equal(_gather(k2, bt[s], ctx[s], BS), k_log[s]), f"K of request {s}"
            assert torch.equal(_gather(v2, bt[s], ctx[s], BS), v_log[s]), f"V of request {s}"


def pin_cache_write_untouched(lib_path=None):
    """Only the (block, slot) rows of the new tokens change; every other row keeps its bits."""
    from oracle import cache_write

    gen = torch.Generator().manual_seed(4200)
    ctx, q_lens, BS = [20, 7, 33], [4, 1, 16], 8
    kp, vp, bt, cl, qsl, kn, vn, _, _ = _cache_case(gen, ctx, q_lens, BS)
    k2, v2 = cache_write(kp, vp, kn, vn, bt, cl, qsl, lib_path=lib_path)
    changed = (torch.from_numpy(k2) != kp).any(dim=(2, 3)) | (torch.from_numpy(v2) != vp).any(dim=(2, 3))
    want = torch.zeros_like(changed)
    for s in range(len(ctx)):
        for pos in range(ctx[s] - q_lens[s], ctx[s]):
            want[int(bt[s, pos // BS]), pos % BS] = True
    assert torch.equal(changed, want)


def pin_cache_write_worked_table(lib_path=None):
    """The continuous-batching page's table 0->7, 1->12, 2->3, 3->19 with 16-token blocks: a decode
    token at position p lands in physical block table[p // 16], slot p % 16."""
    from oracle import cache_write

    g = json.load(open(os.path.join(GOLDEN, "worked_block_table.json")))
    BS, NB = g["block_size"], g["num_blocks"]
    table = torch.tensor([g["block_table"]], dtype=torch.int32)
    for pos, (blk, slot) in {0: (7, 0), 16: (12, 0), 40: (3, 8), 63: (19, 15), 17: (12, 1)}.items():
        kp = torch.zeros(NB, BS, 1, 1)
        kn = torch.ones(1, 1, 1)
        k2, _ = cache_write(kp, kp.clone(), kn, kn.clone(), table, torch.tensor([pos + 1], dtype=torch.int32),
                            lib_path=lib_path)
        hit = np.argwhere(k2[..., 0, 0] != 0).tolist()
        assert hit == [[blk, slot]], f"position {pos}: wrote {hit}, expected {(blk, slot)}"


def pin_cache_write_relabelling(lib_path=None):
    """Relabelling physical blocks (moving their contents) relabels the written pool the same way."""
    from oracle import cache_write

    gen = torch.Generator().manual_seed(4300)
    ctx, q_lens, BS = [30, 5, 18], [10, 1, 2], 4
    kp, vp, bt, cl, qsl, kn, vn, _, _ = _cache_case(gen, ctx, q_lens, BS)
    pi = torch.randperm(kp.shape[0], generator=gen)
    kq, vq = torch.empty_like(kp), torch.empty_like(vp)
    kq[pi], vq[pi] = kp, vp
    a, _ = cache_write(kp, vp, kn, vn, bt, cl, qsl, lib_path=lib_path)
    b, _ = cache_write(kq, vq, kn, vn, pi[bt.long()].to(torch.int32), cl, qsl, lib_path=lib_path)
    assert torch.equal(torch.from_numpy(b)[pi], torch.from_numpy(a))


ALL_PINS += [
    pin_cache_write_gather,
    pin_cache_write_untouched,
    pin_cache_write_worked_table,
    pin_cache_write_relabelling,
]


# ----------------------------------------------------------------------------------------------
# Block copy: copy-on-write within one pool, swap between a GPU pool and a host pool
# ----------------------------------------------------------------------------------------------
def _bits(x):
    """Raw bytes of a torch tensor or numpy array, for bit-for-bit comparison."""
    a = x.contiguous().view(torch.uint8).numpy() if hasattr(x, "detach") else np.ascontiguousarray(x).view(np.uint8)
    return a.reshape(-1)


def pin_copy_blocks_indexed_assignment(lib_path=None):
    """Pool to pool (different pool sizes) and within one pool (sources and destinations disjoint): the
    result equals torch's indexed assignment dst[to] = src[from] bit for bit, fp32 and bf16, any block
    shape; the source pool of a pool-to-pool copy keeps its bits."""
    from oracle import copy_blocks

    for dtype, BS, Hkv, D in ((torch.float32, 16, 2, 8), (torch.bfloat16, 5, 3, 4)):
        gen = torch.Generator().manual_seed(4400 + BS)
        sk, sv = (_randn(gen, 11, BS, Hkv, D, dtype=dtype).to(dtype) for _ in range(2))
        dk, dv = (_randn(gen, 7, BS, Hkv, D, dtype=dtype).to(dtype) for _ in range(2))
        src_bits = _bits(sk), _bits(sv)
        frm, to = torch.randperm(11, generator=gen)[:5], torch.randperm(7, generator=gen)[:5]
        k2, v2 = copy_blocks(dk, dv, sk, sv, torch.stack([frm, to], 1).to(torch.int32), lib_path=lib_path)
        wk, wv = dk.clone(), dv.clone()
        wk[to], wv[to] = sk[frm], sv[frm]
        assert np.array_equal(_bits(k2), _bits(wk)) and np.array_equal(_bits(v2), _bits(wv)), "pool to pool"
        assert np.array_equal(_bits(sk), src_bits[0]) and np.array_equal(_bits(sv), src_bits[1]), "source changed"
        perm = torch.randperm(11, generator=gen)
        frm, to = perm[:4], perm[4:8]
        k3, v3 = copy_blocks(sk, sv, sk, sv, torch.stack([frm, to], 1).to(torch.int32), lib_path=lib_path)
        wk, wv = sk.clone(), sv.clone()
        wk[to], wv[to] = sk[frm], sv[frm]
        assert np.array_equal(_bits(k3), _bits(wk)) and np.array_equal(_bits(v3), _bits(wv)), "within one pool"


def pin_copy_on_write_beam_fork(lib_path=None):
    """A beam fork: two branches share all blocks of a 21-token context (8-token blocks, the last one
    partly filled). Before branch B writes its next token the shared last block is copied to a free block
    and B's table points there; then both branches write their token (position 21). Each branch's decode
    attention then equals float64 SDPA over its own logical sequence: the 21 shared tokens followed by its
    own new token."""
    from oracle import cache_write, copy_blocks

    gen = torch.Generator().manual_seed(4500)
    Hq, Hkv, D, BS, old = 4, 2, 8, 8, 21
    shared_k, shared_v = _randn(gen, old, Hkv, D), _randn(gen, old, Hkv, D)
    new_k, new_v = _randn(gen, 2, Hkv, D), _randn(gen, 2, Hkv, D)
    NB = 9
    ids = torch.randperm(NB, generator=gen)
    kc, vc = _randn(gen, NB, BS, Hkv, D), _randn(gen, NB, BS, Hkv, D)  # stale data
    for i in range(old):
        kc[ids[i // BS], i % BS], vc[ids[i // BS], i % BS] = shared_k[i], shared_v[i]
    bt = torch.stack([ids[:3], ids[:3]]).to(torch.int32)
    fresh = int(ids[3])
    k1, v1 = copy_blocks(kc, vc, kc, vc, torch.tensor([[int(ids[2]), fresh]], dtype=torch.int32), lib_path=lib_path)
    bt[1, 2] = fresh
    ctx = torch.tensor([old + 1, old + 1], dtype=torch.int32)
    k2, v2 = cache_write(torch.from_numpy(k1), torch.from_numpy(v1), new_k, new_v, bt, ctx, lib_path=lib_path)
    q = _randn(gen, 2, Hq, D)
    got = paged_attention(q, torch.from_numpy(k2), torch.from_numpy(v2), bt, ctx, scale=0.35, lib_path=lib_path)
    for b in range(2):
        keys = torch.cat([shared_k, new_k[b:b + 1]])
        values = torch.cat([shared_v, new_v[b:b + 1]])
        ref = _sdpa_reference(q[b:b + 1], keys, values, [old + 1], float(np.float32(0.35)), Hq // Hkv)
        err = np.abs(got[b] - ref[0]).max()
        assert err <= 1e-12, f"branch {b}: |oracle - sdpa| = {err}"


def pin_swap_round_trip(lib_path=None):
    """Preemption by swapping: a request's blocks go to a host pool, its GPU blocks are reused (their data
    overwritten), and on resumption the blocks come back into other free GPU blocks. With the table
    relabelled to the new ids the request's attention is bit-identical to its attention before the swap,
    fp32 and bf16."""
    from oracle import copy_blocks

    for dtype in (torch.float32, torch.bfloat16):
        gen = torch.Generator().manual_seed(4600)
        Hq, Hkv, D, BS = 4, 2, 8, 4
        ctxs = [13, 6]
        keys = [_randn(gen, c, Hkv, D, dtype=dtype) for c in ctxs]
        values = [_randn(gen, c, Hkv, D, dtype=dtype) for c in ctxs]
        kc, vc, bt, _ = paged_from_contiguous(keys, values, BS, gen, dtype=dtype, poison=0.0)
        q = _randn(gen, 1, Hq, D, dtype=dtype).to(dtype)
        cl = torch.tensor(ctxs[:1], dtype=torch.int32)
        before = paged_attention(q, kc, vc, bt[:1], cl, scale=0.5, lib_path=lib_path)
        used = bt[0, :4].long()  # ceil(13 / 4) blocks
        hk, hv = torch.zeros(6, BS, Hkv, D, dtype=dtype), torch.zeros(6, BS, Hkv, D, dtype=dtype)
        host_ids = torch.tensor([5, 0, 3, 1])
        out_map = torch.stack([used, host_ids], 1).to(torch.int32)
        hk, hv = copy_blocks(hk, hv, kc, vc, out_map, lib_path=lib_path)
        kc2 = torch.cat([kc, torch.full((4, BS, Hkv, D), float("nan"), dtype=dtype)])
        vc2 = torch.cat([vc, torch.full((4, BS, Hkv, D), float("nan"), dtype=dtype)])
        kc2[used] = _randn(gen, 4, BS, Hkv, D, dtype=dtype).to(dtype)  # reused by another request
        new_ids = torch.arange(kc.shape[0], kc.shape[0] + 4)
        in_map = torch.stack([host_ids, new_ids], 1).to(torch.int32)
        k3, v3 = copy_blocks(kc2, vc2, _as_torch(hk, dtype), _as_torch(hv, dtype), in_map, lib_path=lib_path)
        bt2 = bt[:1].clone()
        bt2[0, :4] = new_ids.to(torch.int32)
        after = paged_attention(q, _as_torch(k3, dtype), _as_torch(v3, dtype), bt2, cl, scale=0.5,
                                lib_path=lib_path)
        assert np.array_equal(before, after), f"{dtype}: attention changed across the swap"


def pin_copy_blocks_rejects_foreign_ids(lib_path=None):
    """A block id outside its pool is rejected and nothing is copied."""
    from oracle import copy_blocks

    k = torch.zeros(3, 2, 1, 2)
    for pair in ([3, 0], [0, 3], [-1, 0], [0, -1]):
        try:
            copy_blocks(k, k.clone(), k.clone(), k.clone(), torch.tensor([[0, 1], pair], dtype=torch.int32),
                        lib_path=lib_path)
        except ValueError:
            continue
        raise AssertionError(f"pair {pair} was accepted")


ALL_PINS += [
    pin_copy_blocks_indexed_assignment,
    pin_copy_on_write_beam_fork,
    pin_swap_round_trip,
    pin_copy_blocks_rejects_foreign_ids,
]
