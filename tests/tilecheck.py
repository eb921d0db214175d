"""ctypes access to tests/native/libpkv_tilecheck.so: the decode kernels' address functions and
the plan's cut rules, run on the host (see tests/native/tile_check.hip)."""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "native", "libpkv_tilecheck.so")
_lib = None

_i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
_u32p = np.ctypeslib.ndpointer(np.uint32, flags="C_CONTIGUOUS")


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"{LIB} is missing: run python __graft_entry__.py build")
        L = ctypes.CDLL(LIB)
        L.pkv_tilecheck_partition.restype = ctypes.c_int
        L.pkv_tilecheck_partition.argtypes = [ctypes.c_int] * 4
        L.pkv_tilecheck_tail_chunk.restype = ctypes.c_int
        L.pkv_tilecheck_tail_chunk.argtypes = [ctypes.c_int] * 2
        L.pkv_tilecheck_items_offset.restype = ctypes.c_int64
        L.pkv_tilecheck_items_offset.argtypes = [ctypes.c_int] * 5
        L.pkv_tilecheck_counts_offset.restype = ctypes.c_int64
        L.pkv_tilecheck_counts_offset.argtypes = [ctypes.c_int] * 5
        L.pkv_tilecheck_plan.restype = ctypes.c_int64
        L.pkv_tilecheck_plan.argtypes = [_i32p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_int, ctypes.c_int, _u32p,
                                         ctypes.c_int64, _i32p]
        L.pkv_tilecheck_loads.restype = ctypes.c_int64
        L.pkv_tilecheck_loads.argtypes = [ctypes.c_int, ctypes.c_int, _i32p, ctypes.c_int,
                                          ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int, _u32p, ctypes.c_int64, ctypes.c_char_p,
                                          ctypes.c_int]
        _lib = L
    return _lib


def partition(kv8: bool, block_size: int, max_context_len: int, partition_size: int = 0) -> int:
    return lib().pkv_tilecheck_partition(int(kv8), block_size, max_context_len, partition_size)


def plan(lens, block_size: int, P: int, len_limit: int, group_starts=None, prefix_lens=None,
         per_item: int = 1):
    """(items uint32 [n, 4], np_of int32 [B]) of the host planner."""
    L = lib()
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    B = len(lens)
    Q = L.pkv_tilecheck_tail_chunk(P, block_size)
    gs = pl = None
    ng = 0
    if group_starts is not None:
        gs = np.ascontiguousarray(group_starts, dtype=np.int32)
        pl = np.ascontiguousarray(prefix_lens, dtype=np.int32)
        ng = len(pl)
    np_of = np.zeros(max(B, 1), dtype=np.int32)
    cap = 16
    while True:
        items = np.zeros((cap, 4), dtype=np.uint32)
        n = L.pkv_tilecheck_plan(lens, B, len_limit, P, Q, block_size,
                                 None if gs is None else gs.ctypes.data,
                                 None if pl is None else pl.ctypes.data, ng, per_item,
                                 items, cap, np_of)
        if n <= cap:
            return items[:n], np_of[:B]
        cap = int(n)


def bad_loads(kernel: str, tables, num_blocks: int, num_kv_heads: int, head_size: int,
              block_size: int, P: int, items, planted: bool = False):
    """(number of loads outside the pool or the pad, first violation) for kernel '16' or '8'."""
    tables = np.ascontiguousarray(tables, dtype=np.int32)
    items = np.ascontiguousarray(items, dtype=np.uint32).reshape(-1, 4)
    msg = ctypes.create_string_buffer(512)
    n = lib().pkv_tilecheck_loads(0 if kernel == "16" else 1, int(planted), tables,
                                  tables.shape[1], num_blocks, num_kv_heads, head_size, block_size,
                                  P, items, len(items), msg, len(msg))
    if n < 0:
        raise ValueError("shape not built by the kernels")
    return int(n), msg.value.decode()


def items_offset(num_seqs: int, num_heads: int, head_size: int, max_context_len: int,
                 partition_size: int) -> int:
    return int(lib().pkv_tilecheck_items_offset(num_seqs, num_heads, head_size, max_context_len,
                                                partition_size))


def counts_offset(num_seqs: int, num_heads: int, head_size: int, max_context_len: int,
                  partition_size: int) -> int:
    return int(lib().pkv_tilecheck_counts_offset(num_seqs, num_heads, head_size, max_context_len,
                                                 partition_size))
