"""fp64 oracle for multi-query paged attention: chunked prefill and mixed batches.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix, and the reading taken where they stop:

* Flattened queries with start offsets -- the tiemojia.cn vLLM run-flow
  article, section 3.5 (the Attention module's metadata): Q is the flattened
  token sequence of all requests in the batch; ``query_start_loc`` marks where
  each request's query tokens start, next to the block table and slot mapping.
  So request b owns query rows [query_start_loc[b], query_start_loc[b + 1]).
* Chunked prefill -- the AIGC interview book's scheduler section (the note on
  chunked prefill): a long prompt is not prefilled at once; each iteration
  carries the next piece of it beside the decode tokens.  Reading: a request
  whose context holds L tokens (its earlier chunks plus this one, already
  written to the cache) and whose chunk has n query tokens places those
  queries at positions L - n, ..., L - 1; the query at position p attends to
  cache positions 0..p (causal attention, "Vllm" page, "transformer").  A
  decode token is the case n = 1; n = 0 contributes no rows.
* Everything else -- block layout, gather, scale, GQA head map -- as in
  ``oracle.attention``, whose helpers this module uses.
"""
from __future__ import annotations

from typing import Iterable, Optional, Tuple

import numpy as np

from .attention import as_scale, dense_decode, gather_kv, widen


def query_positions(context_len: int, num_queries: int) -> np.ndarray:
    """Cache positions of a request's query tokens: the last ``num_queries`` of its context."""
    return np.arange(context_len - num_queries, context_len)


def request_of_rows(query_start_loc: np.ndarray, rows: np.ndarray) -> np.ndarray:
    """Request index of each flattened query row."""
    return np.searchsorted(np.asarray(query_start_loc), rows, side="right") - 1


def chunked_prefill(query_bits: np.ndarray, key_bits: np.ndarray, value_bits: np.ndarray,
                    dtype: str, block_tables: np.ndarray, context_lens: np.ndarray,
                    query_start_loc: np.ndarray, scale: float,
                    pairs: Optional[Iterable[Tuple[int, int]]] = None,
                    kv_dtype: Optional[str] = None, k_scale: float = 1.0,
                    v_scale: float = 1.0) -> np.ndarray:
    """Output [T, Hq, D] in float64 (only the (row, head) in ``pairs`` when given; other
    entries stay NaN).  ``query_bits`` [T, Hq, D] holds the flattened query rows; the caches
    hold ``kv_dtype`` when given (e.g. 'e4m3' codes with their per-cache scales)."""
    T, Hq, D = query_bits.shape
    Hkv = key_bits.shape[1]
    assert Hq % Hkv == 0
    group = Hq // Hkv
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    B = len(qsl) - 1
    assert qsl[0] == 0 and qsl[-1] == T and np.all(np.diff(qsl) >= 0)
    sc = as_scale(scale)
    out = np.full((T, Hq, D), np.nan)
    if pairs is None:
        pairs = [(r, h) for r in range(T) for h in range(Hq)]
    wanted = {}
    for r, h in pairs:
        b = int(request_of_rows(qsl, np.array([r]))[0])
        wanted.setdefault((b, h // group), []).append((r, h))
    for (b, kvh), items in sorted(wanted.items()):
        n, L = int(qsl[b + 1] - qsl[b]), int(context_lens[b])
        assert 0 <= n <= L, "a request's chunk cannot exceed its context"
        K, V = gather_kv(key_bits, value_bits, kv_dtype or dtype, block_tables[b], L, kvh,
                         k_scale, v_scale)
        pos = query_positions(L, n)
        for r, h in items:
            p = int(pos[r - qsl[b]])
            out[r, h] = dense_decode(widen(query_bits[r, h], dtype), K[:p + 1], V[:p + 1], sc)
    return out


def attention_flops(context_lens: np.ndarray, query_start_loc: np.ndarray, num_heads: int,
                    head_size: int) -> int:
    """Useful flops of the causal attention: 4 * D per (query, visible key, head)
    (2 for q.k and 2 for the weighted sum of v)."""
    total = 0
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    for b in range(len(qsl) - 1):
        n, L = int(qsl[b + 1] - qsl[b]), int(context_lens[b])
        # positions L-n .. L-1 see L-n+1 .. L keys
        total += n * (L - n) + n * (n + 1) // 2
    return 4 * head_size * num_heads * total
