"""CPU reference for the three KV-cache operations, on raw storage bits.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.  Every function works on numpy arrays of unsigned integers
(the bit patterns of the stored elements), so results compare byte for byte.

* reshape_and_cache -- nano-vLLM's KV-cache write (cybasar.com nano-vLLM
  article, section 5.2.3 "KV Cache 写入"): token i goes to slot
  slot_mapping[i]; a slot of -1 means "do not write".  Here the slot is
  resolved in the block layout of the "Vllm" page ("CacheEngine"): block
  slot // block_size, offset slot % block_size.  Any negative slot is read
  as "skip".
* copy_blocks -- CacheEngine's copy (the "Vllm" page, "CacheEngine"): each
  (src, dst) pair copies a whole key block and value block, in every layer.
  The pairs come from the block manager's copy-on-write (the AIGC interview
  book section 23, ``append_slots``), whose dst is always a freshly
  allocated block; all pairs read the state before the call.
* swap_blocks -- CacheEngine's swap_in / swap_out (same section): block
  ``src`` of one cache becomes block ``dst`` of the other.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np


def slot_of(table_row: Sequence[int], pos: int, block_size: int) -> int:
    """Slot of token ``pos``: physical block table[pos // bs], offset pos % bs."""
    return int(table_row[pos // block_size]) * block_size + pos % block_size


def reshape_and_cache(key_cache: np.ndarray, value_cache: np.ndarray, key: np.ndarray,
                      value: np.ndarray, slot_mapping: Sequence[int]) -> None:
    """In place: key_cache[blk, h, d // x, off, d % x] = key[i, h, d];
    value_cache[blk, h, d, off] = value[i, h, d] for every token i with slot >= 0."""
    N, H, D = key.shape
    bs = key_cache.shape[3]
    x = key_cache.shape[4]
    assert x * key_cache.dtype.itemsize == 16
    for i in range(N):
        slot = int(slot_mapping[i])
        if slot < 0:
            continue
        blk, off = slot // bs, slot % bs
        for h in range(H):
            for d in range(D):
                key_cache[blk, h, d // x, off, d % x] = key[i, h, d]
                value_cache[blk, h, d, off] = value[i, h, d]


def reshape_and_cache_fp8(key_cache: np.ndarray, value_cache: np.ndarray, key_bits: np.ndarray,
                          value_bits: np.ndarray, dtype: str, slot_mapping: Sequence[int],
                          k_scale: float, v_scale: float) -> None:
    """The same scatter into an 8-bit (E4M3) cache: each new element (raw bits of the model's
    16-bit ``dtype``) is quantised with oracle.fp8.quantize and its cache's scale first."""
    from oracle.attention import widen
    from oracle.fp8 import quantize
    kq = quantize(widen(key_bits, dtype).astype(np.float32), k_scale)
    vq = quantize(widen(value_bits, dtype).astype(np.float32), v_scale)
    reshape_and_cache(key_cache, value_cache, kq, vq, slot_mapping)


def reshape_and_cache_int8(key_cache: np.ndarray, value_cache: np.ndarray, key_bits: np.ndarray,
                           value_bits: np.ndarray, dtype: str, slot_mapping: Sequence[int],
                           k_scale: float, v_scale: float) -> None:
    """The same scatter into an 8-bit integer cache: each new element is quantised with
    oracle.int8.quantize and its cache's scale first."""
    from oracle.attention import widen
    from oracle.int8 import quantize
    kq = quantize(widen(key_bits, dtype).astype(np.float32), k_scale)
    vq = quantize(widen(value_bits, dtype).astype(np.float32), v_scale)
    reshape_and_cache(key_cache, value_cache, kq, vq, slot_mapping)


def copy_blocks(caches: List[np.ndarray], mapping: Sequence[Tuple[int, int]]) -> None:
    """In place, for each cache array (every layer's K and V): cache[dst] = old cache[src]."""
    for cache in caches:
        before = cache.copy()
        for src, dst in mapping:
            cache[int(dst)] = before[int(src)]


def swap_blocks(dst: np.ndarray, src: np.ndarray, mapping: Sequence[Tuple[int, int]]) -> None:
    """In place: dst[d] = src[s] for each (s, d)."""
    for s, d in mapping:
        dst[int(d)] = src[int(s)]


def memory_waste(context_lens: Sequence[int], block_size: int) -> float:
    """Fraction of allocated slots left empty: only the last block of a sequence is partial."""
    lens = np.asarray(context_lens, dtype=np.int64)
    alloc = ((lens + block_size - 1) // block_size) * block_size
    return float((alloc - lens).sum() / alloc.sum())


def kv_cache_bytes(batch: int, seq_len: int, layers: int, heads: int, head_dim: int,
                   elem_bytes: int) -> int:
    """KV-cache size: 2 (K and V) x batch x seq_len x layers x heads x head_dim x bytes
    (mlqm.cn explainer, KV-cache memory formula)."""
    return 2 * batch * seq_len * layers * heads * head_dim * elem_bytes
