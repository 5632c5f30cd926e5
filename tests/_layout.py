"""Cache pools rewritten between the two layouts, element by element (test helpers, apart from the binding's own
conversion): token-major [NB, BS, Hkv, D] and head-major [NB, Hkv, BS, D]."""
from __future__ import annotations

import torch


def head_major(pool):
    """[NB, BS, Hkv, D] -> [NB, Hkv, BS, D], contiguous (written out here, apart from the binding's helper)."""
    NB, BS, Hkv, D = pool.shape
    out = torch.empty(NB, Hkv, BS, D, dtype=pool.dtype, device=pool.device)
    for h in range(Hkv):
        out[:, h] = pool[:, :, h]
    return out


def token_major(pool):
    NB, Hkv, BS, D = pool.shape
    out = torch.empty(NB, BS, Hkv, D, dtype=pool.dtype, device=pool.device)
    for h in range(Hkv):
        out[:, :, h] = pool[:, h]
    return out
