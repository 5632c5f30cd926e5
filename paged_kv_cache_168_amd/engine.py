"""ctypes binding of the host block manager and continuous-batching scheduler (``pa_engine.h``).

Argument marshalling only: the scheduling runs in ``libpa.so``. Each step's batch is copied out into numpy
arrays (the engine's own buffers are reused by the next step)."""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import numpy as np

from .api import PA_OK, PagedAttentionError, host_library

ENGINE_SYMBOLS = (
    "pa_engine_create",
    "pa_engine_destroy",
    "pa_engine_submit",
    "pa_engine_fork",
    "pa_engine_finish",
    "pa_engine_step",
    "pa_engine_get_stats",
)

_i32, _i64 = ctypes.c_int32, ctypes.c_int64
_P32, _P64 = ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)


class EngineConfig(ctypes.Structure):
    _fields_ = [(n, _i32) for n in ("num_blocks", "block_size", "max_blocks_per_seq", "max_num_seqs",
                                    "max_num_batched_tokens", "chunk_tokens", "reserve_blocks", "num_host_blocks")]


class _Batch(ctypes.Structure):
    _fields_ = [("num_seqs", _i32), ("num_tokens", _i32), ("max_query_len", _i32),
                ("request_ids", _P64), ("query_lens", _P32), ("context_lens", _P32), ("query_start_loc", _P32),
                ("block_tables", _P32),
                ("num_copies", _i32), ("copies", _P32),
                ("num_swap_out", _i32), ("swap_out", _P32),
                ("num_swap_in", _i32), ("swap_in", _P32),
                ("num_finished", _i32), ("finished", _P64),
                ("num_preempted", _i32), ("preempted", _P64)]


class _Stats(ctypes.Structure):
    _fields_ = [(n, _i32) for n in ("free_blocks", "used_blocks", "free_host_blocks", "empty_blocks", "waiting",
                                    "running", "swapped")] + \
               [(n, _i64) for n in ("stored_tokens", "preemptions", "swaps", "recomputes", "copies")]


@dataclass
class Batch:
    request_ids: np.ndarray      # int64 [S]
    query_lens: np.ndarray       # int32 [S]
    context_lens: np.ndarray     # int32 [S]
    query_start_loc: np.ndarray  # int32 [S + 1]
    block_tables: np.ndarray     # int32 [S, W], -1 past the used blocks
    copies: np.ndarray           # int32 [n, 2] GPU -> GPU (copy-on-write)
    swap_out: np.ndarray         # int32 [n, 2] GPU -> host
    swap_in: np.ndarray          # int32 [n, 2] host -> GPU
    finished: np.ndarray         # int64
    preempted: np.ndarray        # int64
    max_query_len: int

    @property
    def num_seqs(self) -> int:
        return int(self.request_ids.shape[0])

    @property
    def num_tokens(self) -> int:
        return int(self.query_start_loc[-1])


def _arr(ptr, n, dtype, shape=None):
    """A copy of n elements of the engine's buffer at ptr (valid until the next step), as a writable array. The
    dtype is the buffer's own (int32 or int64), so one memmove does it."""
    if n == 0:
        return np.zeros(shape if shape is not None else (0,), dtype=dtype)
    a = np.empty(n, dtype=dtype)
    ctypes.memmove(a.ctypes.data, ptr, n * a.itemsize)
    return a.reshape(shape) if shape is not None else a


def _lib():
    lib = host_library()
    if not getattr(lib, "_pa_engine_bound", False):
        P = ctypes.c_void_p
        lib.pa_engine_create.argtypes = [ctypes.POINTER(EngineConfig), ctypes.POINTER(P)]
        lib.pa_engine_destroy.argtypes = [P]
        lib.pa_engine_destroy.restype = None
        lib.pa_engine_submit.argtypes = [P, _i64, _i32, _i32]
        lib.pa_engine_fork.argtypes = [P, _i64, _i64, _i32]
        lib.pa_engine_finish.argtypes = [P, _i64]
        lib.pa_engine_step.argtypes = [P, ctypes.POINTER(_Batch)]
        lib.pa_engine_get_stats.argtypes = [P, ctypes.POINTER(_Stats)]
        for n in ("pa_engine_create", "pa_engine_submit", "pa_engine_fork", "pa_engine_finish", "pa_engine_step",
                  "pa_engine_get_stats"):
            getattr(lib, n).restype = _i32
        lib._pa_engine_bound = True
    return lib


def _check(st, what):
    if st != PA_OK:
        raise PagedAttentionError(st, what)


class Engine:
    """Block manager + continuous-batching scheduler. See ``include/pa_engine.h`` for the step semantics."""

    def __init__(self, *, num_blocks, block_size, max_blocks_per_seq, max_num_seqs, max_num_batched_tokens,
                 chunk_tokens=512, reserve_blocks=2, num_host_blocks=0):
        self.config = EngineConfig(num_blocks, block_size, max_blocks_per_seq, max_num_seqs, max_num_batched_tokens,
                                   chunk_tokens, reserve_blocks, num_host_blocks)
        self._lib = _lib()
        self._h = ctypes.c_void_p()
        _check(self._lib.pa_engine_create(ctypes.byref(self.config), ctypes.byref(self._h)), "engine config")

    def close(self):
        if self._h:
            self._lib.pa_engine_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:  # pragma: no cover - interpreter shutdown
            pass

    def submit(self, request_id: int, prompt_tokens: int, max_new_tokens: int):
        _check(self._lib.pa_engine_submit(self._h, request_id, prompt_tokens, max_new_tokens), "submit")

    def fork(self, parent_id: int, child_id: int, max_new_tokens: int):
        _check(self._lib.pa_engine_fork(self._h, parent_id, child_id, max_new_tokens), "fork")

    def finish(self, request_id: int):
        _check(self._lib.pa_engine_finish(self._h, request_id), "finish")

    def step(self) -> Batch:
        b = _Batch()
        _check(self._lib.pa_engine_step(self._h, ctypes.byref(b)), "step")
        S, W = b.num_seqs, self.config.max_blocks_per_seq
        return Batch(
            request_ids=_arr(b.request_ids, S, np.int64),
            query_lens=_arr(b.query_lens, S, np.int32),
            context_lens=_arr(b.context_lens, S, np.int32),
            query_start_loc=_arr(b.query_start_loc, S + 1, np.int32),
            block_tables=_arr(b.block_tables, S * W, np.int32, (S, W)),
            copies=_arr(b.copies, 2 * b.num_copies, np.int32, (b.num_copies, 2)),
            swap_out=_arr(b.swap_out, 2 * b.num_swap_out, np.int32, (b.num_swap_out, 2)),
            swap_in=_arr(b.swap_in, 2 * b.num_swap_in, np.int32, (b.num_swap_in, 2)),
            finished=_arr(b.finished, b.num_finished, np.int64),
            preempted=_arr(b.preempted, b.num_preempted, np.int64),
            max_query_len=int(b.max_query_len),
        )

    def stats(self) -> dict:
        s = _Stats()
        _check(self._lib.pa_engine_get_stats(self._h, ctypes.byref(s)), "stats")
        d = {n: getattr(s, n) for n, _ in _Stats._fields_}
        # waste: unfilled slots of the blocks that hold tokens (internal fragmentation of the partly filled
        # blocks); prompt blocks allocated ahead of their prefill slice are counted apart, as empty_blocks
        bs = self.config.block_size
        holding = d["used_blocks"] - d["empty_blocks"]
        d["waste"] = 0.0 if holding == 0 else 1.0 - d["stored_tokens"] / (holding * bs)
        d["utilization"] = d["used_blocks"] / self.config.num_blocks
        return d
