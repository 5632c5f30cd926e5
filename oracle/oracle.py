"""ctypes entry to the fp64 C oracle in ``pa_oracle.c`` (test infrastructure only).

The C file is the definition; this module only marshals arrays. The attention
returns float64 numpy arrays, the cache write returns the written caches in
their own element type; everything is computed on the CPU. It never touches a
GPU and never imports the product package.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

STATUS = {
    0: "ok",
    -1: "bad argument",
    -2: "bad query_start_loc",
    -3: "bad context length",
    -4: "block id out of range",
    -5: "out of memory",
}


def build(src: str = _SRC, out: str = _LIB_PATH, sanitize: bool = False) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no FP contraction); sanitize: under AddressSanitizer and
    UndefinedBehaviorSanitizer (the sanitizer tier of the CPU tests)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-shared", "-fPIC", "-o", out, src, "-lm"]
    if sanitize:
        cmd[1:1] = ["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]
    subprocess.run(cmd, check=True)
    return out


def _load(path: str | None = None):
    global _lib
    if path is None and os.environ.get("ORACLE_LIBRARY"):  # another build of this file (the sanitizer build)
        path = os.environ["ORACLE_LIBRARY"]
    if path is not None:
        lib = ctypes.CDLL(path)
    else:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        lib = _lib = ctypes.CDLL(_LIB_PATH)
    p, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    lib.pa_oracle_attention.argtypes = [i32] * 9 + [ctypes.c_float] + [p] * 6 + [p, i64, p, i32]
    lib.pa_oracle_attention.restype = i32
    lib.pa_oracle_read_counts.argtypes = [i32] * 7 + [p, p, p, p]
    lib.pa_oracle_read_counts.restype = i32
    lib.pa_oracle_cache_write.argtypes = [i32] * 8 + [p] * 7
    lib.pa_oracle_cache_write.restype = i32
    lib.pa_oracle_copy_blocks.argtypes = [i32] * 7 + [p] * 5
    lib.pa_oracle_copy_blocks.restype = i32
    return lib


def _as_numpy(x):
    """torch CPU tensor or numpy array -> (contiguous numpy array, dtype code)."""
    if hasattr(x, "detach"):  # torch tensor
        import torch

        x = x.detach().cpu().contiguous()
        if x.dtype == torch.bfloat16:
            return x.view(torch.int16).numpy().view(np.uint16), 1
        x = x.numpy()
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x, 0
    if x.dtype == np.uint16:  # raw bf16 bit patterns
        return x, 1
    if x.dtype == np.int32:
        return x, None
    raise TypeError(f"unsupported dtype {x.dtype}")


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def paged_attention(q, k_cache, v_cache, block_tables, context_lens, query_start_loc=None, *,
                    scale, rows=None, threads=None, lib_path=None) -> np.ndarray:
    """Paged attention in fp64.

    q [T, Hq, D]; k_cache, v_cache [NB, BS, Hkv, D] (fp32, or bf16 as torch
    bfloat16 / raw uint16); block_tables int32 [S, W]; context_lens int32 [S];
    query_start_loc int32 [S+1] or None (decode: T == S). ``rows`` lists flat
    row ids t*Hq + h to compute; the result is then [len(rows), D], otherwise
    [T, Hq, D].
    """
    lib = _load(lib_path)
    qn, dt = _as_numpy(q)
    kn, dk = _as_numpy(k_cache)
    vn, dv = _as_numpy(v_cache)
    if not (dt == dk == dv) or dt is None:
        raise TypeError("q, k_cache and v_cache must share one float dtype")
    bt = np.ascontiguousarray(_as_numpy(block_tables)[0], dtype=np.int32)
    cl = np.ascontiguousarray(_as_numpy(context_lens)[0], dtype=np.int32)
    qsl = None if query_start_loc is None else np.ascontiguousarray(_as_numpy(query_start_loc)[0], dtype=np.int32)
    T, Hq, D = qn.shape
    NB, BS, Hkv, D2 = kn.shape
    if D2 != D or vn.shape != kn.shape:
        raise ValueError("shape mismatch between q and the caches")
    S, W = bt.shape
    if cl.shape != (S,) or (qsl is not None and qsl.shape != (S + 1,)):
        raise ValueError("context_lens / query_start_loc shape mismatch")
    if rows is None:
        rows_arr, nrows = None, 0
        out = np.zeros((T, Hq, D), dtype=np.float64)
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows = rows_arr.size
        out = np.zeros((nrows, D), dtype=np.float64)
    if threads is None:
        threads = os.cpu_count() or 1
    st = lib.pa_oracle_attention(dt, S, T, Hq, Hkv, D, BS, NB, W, ctypes.c_float(scale),
                                 _ptr(qn), _ptr(kn), _ptr(vn), _ptr(bt), _ptr(cl), _ptr(qsl),
                                 _ptr(rows_arr), nrows, _ptr(out), int(threads))
    if st != 0:
        raise ValueError(f"oracle rejected the inputs: {STATUS.get(st, st)}")
    return out


def read_counts(block_tables, context_lens, query_start_loc=None, *, num_tokens, num_q_heads,
                num_kv_heads, block_size, num_blocks, lib_path=None) -> np.ndarray:
    """counts[block, slot] = number of (query token, query head) rows reading that slot."""
    lib = _load(lib_path)
    bt = np.ascontiguousarray(_as_numpy(block_tables)[0], dtype=np.int32)
    cl = np.ascontiguousarray(_as_numpy(context_lens)[0], dtype=np.int32)
    qsl = None if query_start_loc is None else np.ascontiguousarray(_as_numpy(query_start_loc)[0], dtype=np.int32)
    S, W = bt.shape
    counts = np.zeros((num_blocks, block_size), dtype=np.int64)
    st = lib.pa_oracle_read_counts(S, num_tokens, num_q_heads, num_kv_heads, block_size, num_blocks, W,
                                   _ptr(bt), _ptr(cl), _ptr(qsl), _ptr(counts))
    if st != 0:
        raise ValueError(f"oracle rejected the inputs: {STATUS.get(st, st)}")
    return counts


def cache_write(k_cache, v_cache, k_new, v_new, block_tables, context_lens, query_start_loc=None, *,
                lib_path=None):
    """The caches after storing this step's new K/V rows (copies; the inputs are not modified).

    k_cache, v_cache [NB, BS, Hkv, D] and k_new, v_new [T, Hkv, D] share one dtype (fp32, or bf16 as
    torch bfloat16 / raw uint16). Returns (k, v) numpy arrays in that representation.
    """
    lib = _load(lib_path)
    kc, dk = _as_numpy(k_cache)
    vc, dv = _as_numpy(v_cache)
    kn, dkn = _as_numpy(k_new)
    vn, dvn = _as_numpy(v_new)
    if not (dk == dv == dkn == dvn) or dk is None:
        raise TypeError("caches and new rows must share one float dtype")
    kc, vc = kc.copy(), vc.copy()
    bt = np.ascontiguousarray(_as_numpy(block_tables)[0], dtype=np.int32)
    cl = np.ascontiguousarray(_as_numpy(context_lens)[0], dtype=np.int32)
    qsl = None if query_start_loc is None else np.ascontiguousarray(_as_numpy(query_start_loc)[0], dtype=np.int32)
    NB, BS, Hkv, D = kc.shape
    T = kn.shape[0]
    S, W = bt.shape
    if kn.shape != (T, Hkv, D) or vn.shape != kn.shape or vc.shape != kc.shape:
        raise ValueError("shape mismatch between the caches and the new rows")
    st = lib.pa_oracle_cache_write(kc.itemsize, S, T, Hkv, D, BS, NB, W, _ptr(kc), _ptr(vc), _ptr(kn), _ptr(vn),
                                   _ptr(bt), _ptr(cl), _ptr(qsl))
    if st != 0:
        raise ValueError(f"oracle rejected the inputs: {STATUS.get(st, st)}")
    return kc, vc


def copy_blocks(dst_k, dst_v, src_k, src_v, mapping, *, lib_path=None):
    """The destination pools after copying source block mapping[i][0] to destination block mapping[i][1]
    for every pair, in order (copies; the inputs are not modified).

    Pools are [NB, BS, Hkv, D] of one dtype (fp32, or bf16 as torch bfloat16 / raw uint16); the source
    and destination pools may have different NB. For copy-on-write within one pool pass that pool as both
    source and destination. Returns (k, v) numpy arrays in the pools' representation.
    """
    lib = _load(lib_path)
    sk, dsk = _as_numpy(src_k)
    sv, dsv = _as_numpy(src_v)
    dk, ddk = _as_numpy(dst_k)
    dv, ddv = _as_numpy(dst_v)
    if not (dsk == dsv == ddk == ddv) or dsk is None:
        raise TypeError("pools must share one float dtype")
    if sk.shape != sv.shape or dk.shape != dv.shape or sk.shape[1:] != dk.shape[1:]:
        raise ValueError("K and V pools must match and share [BS, Hkv, D]")
    same = dst_k is src_k
    dk, dv = dk.copy(), dv.copy()
    if same:  # copy-on-write: the copies read the pool as the earlier pairs left it
        sk, sv = dk, dv
    m = np.ascontiguousarray(_as_numpy(mapping)[0], dtype=np.int32).reshape(-1, 2)
    _, BS, Hkv, D = dk.shape
    st = lib.pa_oracle_copy_blocks(dk.itemsize, m.shape[0], BS, Hkv, D, sk.shape[0], dk.shape[0], _ptr(sk),
                                   _ptr(sv), _ptr(dk), _ptr(dv), _ptr(m))
    if st != 0:
        raise ValueError(f"oracle rejected the inputs: {STATUS.get(st, st)}")
    return dk, dv


def bf16_to_float64(x) -> np.ndarray:
    """Exact widening of bf16 (torch bfloat16 or raw uint16) to float64."""
    a, code = _as_numpy(x)
    if code == 1:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)
