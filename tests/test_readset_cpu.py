"""The read-set gate on the CPU: the oracle's output on counting inputs equals the closed form from the markers
alone (bit for bit), and the gate's comparison fails for the read mistakes it exists to catch: a dropped,
repeated or shifted tile and a dropped or repeated piece at contexts of 592 to 262144 tokens (the "tile"
markers), and one dropped, extra or misplaced token or one stale slot read up to 4096 keys (the "token"
markers; beyond that a single key is under half a bf16 spacing of its dimension's count, and the masking code
those mistakes come from runs the same at every length, so the short contexts of every case cover it)."""
import numpy as np
import pytest
import torch

from _readset import SCHEMES, check_counts, closed_form, counting, marker_dims, visible_counts
from oracle import paged_attention
from paged_kv_cache_168_amd import workloads as W


def _oracle(wl):
    return paged_attention(wl.q, wl.k_cache, wl.v_cache, wl.block_tables, wl.context_lens, wl.query_start_loc,
                           scale=wl.scale)


@pytest.mark.parametrize("scheme", SCHEMES)
@pytest.mark.parametrize("BS", [1, 5, 16, 32])
def test_oracle_equals_the_closed_form_decode(BS, scheme):
    wl = counting(W.random_workload(3100 + BS, ctx=[1, 2, 15, 16, 17, 64, 100, 513, 1024], Hq=16, Hkv=4, D=64,
                                    BS=BS, dtype=torch.bfloat16), scheme)
    want = _oracle(wl)
    assert np.array_equal(want, closed_form(wl))
    assert check_counts(torch.from_numpy(want).float().to(torch.bfloat16), want, visible_counts(wl), "self") == 5


@pytest.mark.parametrize("scheme", SCHEMES)
def test_oracle_equals_the_closed_form_mixed_and_shared_prefix(scheme):
    wl = counting(W.random_workload(3200, ctx=[300, 1, 1024, 40], q_lens=[120, 1, 1024, 1], Hq=32, Hkv=8, D=128,
                                    BS=16, dtype=torch.bfloat16), scheme)
    assert np.array_equal(_oracle(wl), closed_form(wl))
    wl = counting(W.grouped_workload(3201, [(64, [64, 100, 300]), (0, [17, 5])], Hq=8, Hkv=2, D=128, BS=16), scheme)
    assert np.array_equal(_oracle(wl), closed_form(wl))


def test_fp32_inputs_count_the_same():
    wl = counting(W.random_workload(3300, ctx=[7, 64, 200], Hq=4, Hkv=2, D=64, BS=16, dtype=torch.float32))
    assert np.array_equal(_oracle(wl), closed_form(wl))


def _row(positions, h, D, scheme, stale=0):
    """Output of one row that read the keys at `positions` (with repeats) and `stale` unreadable slots."""
    d = marker_dims(torch.as_tensor(positions, dtype=torch.int64), h, D, scheme).numpy()
    c = np.bincount(d, minlength=D).astype(np.float64) + stale
    return c / (len(positions) + stale)


def _gate(positions, n, h, D, scheme, stale=0):
    want = _row(np.arange(n), h, D, scheme)[None, None, :]
    got = torch.from_numpy(_row(positions, h, D, scheme, stale)[None, None, :]).float().to(torch.bfloat16)
    check_counts(got, want, np.array([n]), "planted")


@pytest.mark.parametrize("n", [16 * 37, 4096, 32768, 262144])
@pytest.mark.parametrize("h", [0, 1, 6, 7])
@pytest.mark.parametrize("scheme", SCHEMES)
def test_gate_catches_read_mistakes(n, h, scheme):
    D = 128
    full = np.arange(n)
    _gate(full, n, h, D, scheme)  # the correct read set passes
    tiles = n // 16
    if scheme == "tile":  # whole tiles and pieces, at every size
        mistakes = {
            "dropped tile": np.delete(full, np.arange(16 * (tiles // 3), 16 * (tiles // 3) + 16)),
            "repeated tile": np.concatenate([full, full[16 * (tiles // 2):16 * (tiles // 2) + 16]]),
            "repeated piece": np.concatenate([full, full[: max(16, (n // 24) // 16 * 16)]]),
            "dropped piece": full[max(16, (n // 24) // 16 * 16):],
            "tile shifted by one block": np.concatenate([full[:-16], full[-32:-16]]),
        }
    else:  # single tokens, up to 4096 keys (n / D keys per dimension: one key is 3% of 32 at 4096)
        mistakes = {} if n > 4096 else {
            "dropped token": full[:-1],
            "extra token": np.concatenate([full, [n // 2]]),
            "token read from the wrong slot": np.concatenate([full[:-1], [n - 2]]),
        }
    for what, pos in mistakes.items():
        with pytest.raises(AssertionError):
            _gate(pos, n, h, D, scheme)
            pytest.fail(f"{what} passed at n={n}")  # pragma: no cover
    if n <= 4096:  # one stale slot among n keys moves a dimension by about 1/count; past 4096 keys that is under
        # half a bf16 spacing, and the NaN / 1e30 poison tests (bit-exact) are the gate for stale reads
        with pytest.raises(AssertionError):
            _gate(full, n, h, D, scheme, stale=1)


def test_gate_rejects_a_wrong_tile_at_a_non_power_of_two_count():
    n, D = 3000, 128
    for h in (0, 1):
        for scheme in SCHEMES:
            full = np.arange(n)
            _gate(full, n, h, D, scheme)
            wrong = full.copy()
            wrong[1600:1616] = np.arange(2400, 2416)  # one tile read twice, another never
            with pytest.raises(AssertionError):
                _gate(wrong, n, h, D, scheme)
