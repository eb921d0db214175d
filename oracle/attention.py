"""fp64 oracle for single-query decode attention over a block-paged KV cache.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

Sources for each step:

* Block layout -- "Vllm" agent-guide page, section "CacheEngine": a key block
  has shape [num_heads, head_size // x, block_size, x] with
  x = 16 // sizeof(dtype); a value block has shape [num_heads, head_size,
  block_size].  The pool of blocks is the outer dimension (the pages give
  only the per-block shape; the plainest reading puts the block index first).
* Addressing -- mlqm.cn vLLM explainer, section "1、PagedAttention": a
  sequence's block table lists its physical blocks in logical order, 16
  tokens per block, so token t sits in table[t // block_size] at offset
  t % block_size.
* Attention -- "Vllm" page, section "transformer":
  softmax(Q K^T / sqrt(d_k)) V.  The caller's ``scale`` replaces
  1 / sqrt(d_k) (every workload passes 1 / sqrt(head_size)).
* Decode -- "Vllm" page, section "transformer" (decoding paragraph): the new
  token's K, V are appended to the cache and its query attends to the whole
  cache, so ``context_lens`` counts the new token.
* Gather-then-dense -- mlqm.cn explainer, nano-vLLM "Attention 计算的妥协
  Gather 机制": collect the blocks named by the block table into one dense
  tensor, then run ordinary attention.
* Grouped-query attention (GQA is only named on the pages, "推理优化" on the
  "Vllm" page): query head h reads KV head h // (num_heads // num_kv_heads).
* A sequence of length 0 attends to nothing; its output is defined as 0.
"""
from __future__ import annotations

from typing import Iterable, Optional, Tuple

import numpy as np


def widen(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of stored elements given as raw bits.

    ``dtype`` is 'f32' (uint32 bits), 'f16' (uint16, IEEE binary16),
    'bf16' (uint16: the upper half of an IEEE binary32, so shifting the bits
    left by 16 gives the binary32 with the same value), 'e4m3' (uint8, the
    8-bit float of oracle.fp8, without its scale) or 'i8' (uint8 bytes of the
    signed integer codes of oracle.int8, without their scale).
    """
    if dtype == "f32":
        return bits.view(np.float32).astype(np.float64)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float64)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == "e4m3":
        from oracle.fp8 import e4m3_decode
        return e4m3_decode(bits)
    if dtype == "i8":
        from oracle.int8 import i8_decode
        return i8_decode(bits)
    raise ValueError(dtype)


def chunk_width(bits: np.ndarray) -> int:
    """x = 16 bytes / element size."""
    return 16 // bits.dtype.itemsize


def gather_kv(key_bits: np.ndarray, value_bits: np.ndarray, dtype: str, table_row: np.ndarray,
              L: int, kv_head: int, k_scale: float = 1.0,
              v_scale: float = 1.0) -> Tuple[np.ndarray, np.ndarray]:
    """Dense K[t, d], V[t, d] (float64, t < L) of one sequence and one KV head.

    K[t, d] = key_cache[table[t // bs], kv_head, d // x, t % bs, d % x] * k_scale
    V[t, d] = value_cache[table[t // bs], kv_head, d, t % bs] * v_scale
    (the scales are 1 except for an 8-bit cache; they are taken as the float32 the kernel gets)
    """
    bs = key_bits.shape[3]
    x = key_bits.shape[4]
    D = value_bits.shape[2]
    assert x == chunk_width(key_bits) and key_bits.shape[2] * x == D
    t = np.arange(L)
    d = np.arange(D)
    blk = np.asarray(table_row, dtype=np.int64)[t // bs]
    off = t % bs
    K = key_bits[blk[:, None], kv_head, (d // x)[None, :], off[:, None], (d % x)[None, :]]
    V = value_bits[blk[:, None], kv_head, d[None, :], off[:, None]]
    return widen(K, dtype) * as_scale(k_scale), widen(V, dtype) * as_scale(v_scale)


def dense_decode(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * K q) V for one query vector, in float64.  Empty context -> 0."""
    if K.shape[0] == 0:
        return np.zeros(V.shape[1], dtype=np.float64)
    s = scale * (K @ q)
    m = s.max()
    p = np.exp(s - m)
    return (p @ V) / p.sum()


def as_scale(scale: float) -> float:
    """The float32 value the kernel receives, widened exactly."""
    return float(np.float32(scale))


def paged_decode(query_bits: np.ndarray, key_bits: np.ndarray, value_bits: np.ndarray,
                 dtype: str, block_tables: np.ndarray, context_lens: np.ndarray, scale: float,
                 pairs: Optional[Iterable[Tuple[int, int]]] = None, kv_dtype: Optional[str] = None,
                 k_scale: float = 1.0, v_scale: float = 1.0) -> np.ndarray:
    """Output [B, Hq, D] in float64 (or only the (b, h) in ``pairs``; other rows stay NaN).

    ``query_bits`` [B, Hq, D], ``key_bits`` [NB, Hkv, D/x, bs, x],
    ``value_bits`` [NB, Hkv, D, bs] hold raw storage bits of ``dtype`` (the caches of
    ``kv_dtype`` when given, e.g. 'e4m3' with its per-cache scales).
    """
    B, Hq, D = query_bits.shape
    Hkv = key_bits.shape[1]
    assert Hq % Hkv == 0
    group = Hq // Hkv
    sc = as_scale(scale)
    out = np.full((B, Hq, D), np.nan)
    if pairs is None:
        pairs = [(b, h) for b in range(B) for h in range(Hq)]
    by_seq_head = {}
    for b, h in pairs:
        by_seq_head.setdefault((b, h // group), []).append(h)
    for (b, g), heads in sorted(by_seq_head.items()):
        L = int(context_lens[b])
        K, V = gather_kv(key_bits, value_bits, kv_dtype or dtype, block_tables[b], L, g,
                         k_scale, v_scale)
        for h in heads:
            q = widen(query_bits[b, h], dtype)
            out[b, h] = dense_decode(q, K, V, sc)
    return out


def partition_stats(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float, start: int,
                    stop: int) -> Tuple[float, float, np.ndarray]:
    """(m_p, l_p, acc_p) of tokens [start, stop): max logit, sum of exp(s - m_p), sum of exp(s - m_p) V."""
    s = scale * (K[start:stop] @ q)
    m = s.max()
    p = np.exp(s - m)
    return float(m), float(p.sum()), p @ V[start:stop]


def combine_partitions(stats) -> np.ndarray:
    """Log-sum-exp combination of per-partition (m_p, l_p, acc_p):
    out = sum_p e^(m_p - M) acc_p / sum_p e^(m_p - M) l_p with M = max_p m_p."""
    M = max(m for m, _, _ in stats)
    num = sum(np.exp(m - M) * acc for m, _, acc in stats)
    den = sum(np.exp(m - M) * l for m, l, _ in stats)
    return num / den


def partitioned_decode(query_bits: np.ndarray, key_bits: np.ndarray, value_bits: np.ndarray,
                       dtype: str, block_tables: np.ndarray, context_lens: np.ndarray,
                       scale: float, partition_size: int) -> np.ndarray:
    """The same output computed over ``partition_size``-token slices of each context, then combined."""
    B, Hq, D = query_bits.shape
    Hkv = key_bits.shape[1]
    group = Hq // Hkv
    sc = as_scale(scale)
    out = np.zeros((B, Hq, D))
    for b in range(B):
        L = int(context_lens[b])
        if L == 0:
            continue
        for g in range(Hkv):
            K, V = gather_kv(key_bits, value_bits, dtype, block_tables[b], L, g)
            for h in range(g * group, (g + 1) * group):
                q = widen(query_bits[b, h], dtype)
                stats = [partition_stats(q, K, V, sc, s0, min(s0 + partition_size, L))
                         for s0 in range(0, L, partition_size)]
                out[b, h] = combine_partitions(stats)
    return out


def shared_prefix_length(context_lens: np.ndarray, start: int, stop: int, prefix_len: int,
                         block_size: int) -> int:
    """Tokens that the sequences [start, stop) read from shared blocks: the caller's prefix
    length, capped by every member's context length and rounded down to whole blocks (a
    block is either shared by all members or owned by one, as with copy-on-write in the
    mlqm.cn explainer's example); a group of one shares nothing."""
    if stop - start < 2:
        return 0
    pre = min([max(int(prefix_len), 0)] + [int(L) for L in context_lens[start:stop]])
    return pre - pre % block_size


def check_shared_prefix_groups(block_tables: np.ndarray, context_lens: np.ndarray, group_starts,
                               prefix_lens, block_size: int) -> None:
    """Raise ValueError unless the groups satisfy the shared-prefix contract.

    Groups are consecutive runs of sequences [group_starts[g], group_starts[g + 1]) that cover
    [0, B) once, in order (an empty group is allowed).  Members of a group hold the same physical blocks for their shared tokens
    [0, pre), pre = shared_prefix_length(...): the block table entries of every member equal
    the first member's for the pre / block_size logical blocks (PagedAttention's block sharing:
    beams or samples forked from one prompt point at the prompt's blocks, mlqm.cn explainer,
    "PagedAttention", and the fork of the AIGC interview book, section 23).  Entries past the
    rounded prefix may differ (a partial last block is copied on write)."""
    starts = [int(s) for s in group_starts]
    B = len(context_lens)
    if len(starts) != len(prefix_lens) + 1 or starts[0] != 0 or starts[-1] != B or any(
            b < a for a, b in zip(starts, starts[1:])):
        raise ValueError("group_starts must be non-decreasing from 0 to num_seqs")
    for g in range(len(prefix_lens)):
        s0, s1 = starts[g], starts[g + 1]
        pre = shared_prefix_length(context_lens, s0, s1, int(prefix_lens[g]), block_size)
        n = pre // block_size
        for b in range(s0 + 1, s1):
            if not np.array_equal(block_tables[b, :n], block_tables[s0, :n]):
                raise ValueError(f"sequence {b} does not share group {g}'s first {n} blocks")


def shared_prefix_decode(query_bits: np.ndarray, key_bits: np.ndarray, value_bits: np.ndarray,
                         dtype: str, block_tables: np.ndarray, context_lens: np.ndarray,
                         scale: float, group_starts, prefix_lens) -> np.ndarray:
    """Decode of sequences grouped by a shared prompt prefix.

    Reading the shared blocks once per group is a change of memory traffic, not of the result:
    inside the contract (check_shared_prefix_groups, which raises outside it) every member's
    output is the plain paged decode of its own table and length.  So the oracle checks the
    contract and then computes that definition."""
    check_shared_prefix_groups(block_tables, context_lens, group_starts, prefix_lens,
                               key_bits.shape[3])
    return paged_decode(query_bits, key_bits, value_bits, dtype, block_tables, context_lens,
                        scale)
