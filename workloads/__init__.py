"""Seeded synthetic inputs for paged decode attention and the cache operations.

This module only draws random numbers and lays them out in the paged-cache
storage format.  It holds none of the attention arithmetic: both the fp64
oracle (``oracle/``) and the HIP path take their inputs from here, and
neither is imported by it.

Storage layout (the "Vllm" page of the yang20150702 agent guide, section
"CacheEngine"): a key block is ``[num_kv_heads, head_size // x, block_size, x]``
with ``x = 16 // sizeof(dtype)``; a value block is
``[num_kv_heads, head_size, block_size]``.  The pool of physical blocks is the
outermost dimension.  A sequence reaches its blocks through one row of
``block_tables`` (logical block -> physical block id); token ``t`` of a
sequence lives in logical block ``t // block_size`` at offset
``t % block_size`` (the mlqm.cn vLLM explainer, "PagedAttention" block-table
example).

Random streams: ``numpy.random.default_rng([seed, stream])`` with
``seed = 1000 + config_index`` and one stream per quantity, so changing one
draw never shifts another.  Values are drawn as float32 N(0, 1) and rounded
to the storage dtype with round-to-nearest-even (torch's cast).  Slots a
sequence does not own (the tail of its last block, unused pool blocks) are
NaN when ``poison`` is set, so that a kernel that reads them without masking
produces NaN.  Unused block-table entries are -1.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

# stream ids for default_rng([seed, stream])
S_LENS, S_PERM, S_Q, S_K, S_V, S_OUTLIER, S_SLOTS, S_NEWKV, S_COW, S_SWAP = range(10)

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def x_of(dtype: str) -> int:
    """Elements per 16-byte key chunk: 16 // sizeof(dtype) (fp32 -> 4, fp16/bf16 -> 8)."""
    return 16 // torch.tensor([], dtype=DTYPES[dtype]).element_size()


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    key: str
    name: str
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_size: int
    block_size: int
    dtype: str
    lens: tuple            # ("uniform", lo, hi) | ("lognormal", median, sigma, lo, hi) | ("fixed", L)
    pool: tuple            # ("fixed", n) | ("times", k) | ("plus", n)
    partition_size: int = 512
    outlier_p: float = 0.0
    outlier_scale: float = 1.0
    seed: int = 0

    @property
    def x(self) -> int:
        return x_of(self.dtype)


CONFIGS: Dict[str, DecodeConfig] = {
    "c1": DecodeConfig("c1", "tiny paged decode fp32", 4, 8, 8, 64, 16, "f32",
                       ("uniform", 1, 256), ("fixed", 128), seed=1001),
    "c2": DecodeConfig("c2", "MHA 7B-like layer fp16", 64, 32, 32, 128, 16, "f16",
                       ("uniform", 512, 4096), ("times", 2), seed=1002),
    "c3": DecodeConfig("c3", "GQA batch-256 bf16", 256, 32, 8, 128, 16, "bf16",
                       ("lognormal", 2048, 0.8, 16, 32768), ("plus", 64), seed=1003),
    "c4": DecodeConfig("c4", "long-context split-K bf16", 8, 64, 8, 128, 32, "bf16",
                       ("fixed", 131072), ("fixed", 32768), outlier_p=0.01,
                       outlier_scale=8.0, seed=1004),
}


def rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([seed, stream])


def draw_lengths(cfg: DecodeConfig, num_seqs: int) -> np.ndarray:
    g = rng(cfg.seed, S_LENS)
    kind = cfg.lens[0]
    if kind == "uniform":
        _, lo, hi = cfg.lens
        lens = g.integers(lo, hi + 1, size=num_seqs)
    elif kind == "lognormal":
        _, median, sigma, lo, hi = cfg.lens
        lens = np.clip(np.rint(g.lognormal(math.log(median), sigma, size=num_seqs)), lo, hi)
    elif kind == "fixed":
        lens = np.full(num_seqs, cfg.lens[1])
    else:
        raise ValueError(kind)
    return lens.astype(np.int64)


def _normal_to(shape, g: np.random.Generator, dtype: str) -> torch.Tensor:
    a = g.standard_normal(size=shape, dtype=np.float32)
    return torch.from_numpy(a).to(DTYPES[dtype])


def storage_bits(t: torch.Tensor) -> np.ndarray:
    """Raw storage of a CPU tensor as unsigned integers (uint8 for 8-bit codes, uint16 for 2-byte
    dtypes, uint32 for fp32)."""
    t = t.contiguous()
    if t.element_size() == 1:
        return t.view(torch.uint8).numpy()
    if t.element_size() == 2:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.element_size() == 4:
        return t.view(torch.int32).numpy().view(np.uint32)
    if t.element_size() == 8:
        return t.view(torch.int64).numpy().view(np.uint64)
    raise ValueError(t.dtype)


@dataclasses.dataclass
class DecodeCase:
    """One decode step's inputs, all on the CPU in storage dtype.

    ``key_cache``/``value_cache`` are the state *before* the step: the slot of
    each sequence's newest token (position ``context_lens[b] - 1``) is still
    unwritten (NaN when poisoned).  The step first scatters ``new_key`` /
    ``new_value`` into ``slot_mapping`` and then attends over
    ``context_lens[b]`` tokens, so ``context_lens`` counts the new token.
    """
    cfg: DecodeConfig
    query: torch.Tensor         # [B, Hq, D]
    key_cache: torch.Tensor     # [NB, Hkv, D/x, bs, x]
    value_cache: torch.Tensor   # [NB, Hkv, D, bs]
    block_tables: torch.Tensor  # int32 [B, max_blocks]
    context_lens: torch.Tensor  # int32 [B]
    new_key: torch.Tensor       # [B, Hkv, D]
    new_value: torch.Tensor     # [B, Hkv, D]
    slot_mapping: torch.Tensor  # int64 [B]
    scale: float
    used_blocks: np.ndarray     # physical ids in use, in assignment order
    free_blocks: np.ndarray     # physical ids not referenced by any table
    kv_dtype: Optional[str] = None  # 'e4m3' / 'i8': caches hold 8-bit codes (new K/V stay 16-bit)
    k_scale: float = 1.0
    v_scale: float = 1.0

    @property
    def num_seqs(self) -> int:
        return self.query.shape[0]

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max().item()) if self.num_seqs else 0

    @property
    def max_num_blocks_per_seq(self) -> int:
        return self.block_tables.shape[1]


def _pool_size(cfg: DecodeConfig, n_used: int) -> int:
    kind, n = cfg.pool
    if kind == "fixed":
        return max(int(n), n_used)
    if kind == "times":
        return int(n) * n_used
    if kind == "plus":
        return n_used + int(n)
    raise ValueError(kind)


def fill_pool(key_cache: torch.Tensor, value_cache: torch.Tensor, ids: np.ndarray,
              cfg: DecodeConfig, chunk: int = 2048) -> None:
    """Draw N(0,1) K and V for the physical blocks ``ids`` (in that order), chunk by chunk."""
    gk, gv = rng(cfg.seed, S_K), rng(cfg.seed, S_V)
    go = rng(cfg.seed, S_OUTLIER) if cfg.outlier_p > 0 else None
    kshape = tuple(key_cache.shape[1:])
    vshape = tuple(value_cache.shape[1:])
    Hkv, _, bs, _ = kshape
    for s in range(0, len(ids), chunk):
        sel = torch.from_numpy(np.ascontiguousarray(ids[s:s + chunk]))
        n = len(sel)
        k = gk.standard_normal(size=(n,) + kshape, dtype=np.float32)
        if go is not None:
            # one Bernoulli draw per (block, kv head, token): the whole key
            # vector of an outlier token is scaled before rounding
            hit = go.random(size=(n, Hkv, 1, bs, 1)) < cfg.outlier_p
            k = np.where(hit, k * np.float32(cfg.outlier_scale), k)
        key_cache[sel] = torch.from_numpy(k).to(key_cache.dtype)
        v = gv.standard_normal(size=(n,) + vshape, dtype=np.float32)
        value_cache[sel] = torch.from_numpy(v).to(value_cache.dtype)


def poison_slots(key_cache: torch.Tensor, value_cache: torch.Tensor, block_id: int,
                 first_off: int, last_off: Optional[int] = None) -> None:
    """NaN-fill token slots [first_off, last_off) of one physical block (all heads, all dims)."""
    if last_off is None:
        last_off = key_cache.shape[3]
    key_cache[block_id, :, :, first_off:last_off, :] = float("nan")
    value_cache[block_id, :, :, first_off:last_off] = float("nan")


@dataclasses.dataclass
class DecodeLayout:
    """Lengths and block tables of a decode step, without any cache contents."""
    cfg: DecodeConfig
    lens: np.ndarray        # int64 [B]
    tables: np.ndarray      # int32 [B, max_blocks], -1 past each sequence's blocks
    num_blocks: int         # pool size
    used: np.ndarray        # physical ids in use, in assignment order
    free: np.ndarray        # physical ids not referenced by any table


def decode_layout(key: str, *, num_seqs: Optional[int] = None, len_cap: Optional[int] = None,
                  lens: Optional[Sequence[int]] = None, **overrides) -> DecodeLayout:
    """The lengths and block tables make_decode_case draws (same arguments, same streams)."""
    cfg = dataclasses.replace(CONFIGS[key], **overrides) if overrides else CONFIGS[key]
    if lens is not None:
        lens = np.asarray(lens, dtype=np.int64)
    else:
        B_full = cfg.num_seqs
        B = B_full if num_seqs is None else int(num_seqs)
        lens = draw_lengths(cfg, max(B, B_full))[:B]
    if len_cap is not None:
        lens = np.minimum(lens, len_cap)
    B = len(lens)
    bs = cfg.block_size
    nblk = (lens + bs - 1) // bs
    n_used = int(nblk.sum())
    NB = _pool_size(cfg, n_used)
    perm = rng(cfg.seed, S_PERM).permutation(NB)
    used = perm[:n_used]
    free = np.sort(perm[n_used:])
    max_blocks = int(nblk.max()) if B else 1
    tables = np.full((B, max(max_blocks, 1)), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        tables[b, :nblk[b]] = used[off:off + nblk[b]]
        off += nblk[b]
    return DecodeLayout(cfg, lens, tables, NB, used, free)


def make_decode_case(key: str, *, num_seqs: Optional[int] = None, len_cap: Optional[int] = None,
                     lens: Optional[Sequence[int]] = None, poison: bool = True,
                     **overrides) -> DecodeCase:
    """Build one decode step of config ``key`` (c1..c4).

    ``num_seqs`` keeps the first sequences of the full draw (same lengths);
    ``len_cap`` clips lengths, for oracle-sized parity cases; ``lens`` replaces
    the drawn lengths outright; ``overrides`` replace config fields (shapes,
    dtype, pool) for variants outside the five workloads.
    """
    lay = decode_layout(key, num_seqs=num_seqs, len_cap=len_cap, lens=lens, **overrides)
    cfg, lens, tables, NB, used, free = lay.cfg, lay.lens, lay.tables, lay.num_blocks, lay.used, lay.free
    B = len(lens)
    bs, Hq, Hkv, D, x = cfg.block_size, cfg.num_heads, cfg.num_kv_heads, cfg.head_size, cfg.x

    tdt = DTYPES[cfg.dtype]
    fill = float("nan") if poison else 0.0
    key_cache = torch.full((NB, Hkv, D // x, bs, x), fill, dtype=tdt)
    value_cache = torch.full((NB, Hkv, D, bs), fill, dtype=tdt)
    fill_pool(key_cache, value_cache, used, cfg)

    slot = np.full(B, -1, dtype=np.int64)   # an empty context gets no new token
    for b in range(B):
        L = int(lens[b])
        if L == 0:
            continue
        last = L - 1
        blk = int(tables[b, last // bs])
        slot[b] = blk * bs + last % bs
        if poison:
            # the tail of the last block and the new token's slot are not yet written
            poison_slots(key_cache, value_cache, blk, last % bs)

    q = _normal_to((B, Hq, D), rng(cfg.seed, S_Q), cfg.dtype)
    gn = rng(cfg.seed, S_NEWKV)
    new_k = _normal_to((B, Hkv, D), gn, cfg.dtype)
    new_v = _normal_to((B, Hkv, D), gn, cfg.dtype)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    return DecodeCase(cfg, q, key_cache, value_cache, torch.from_numpy(tables),
                      torch.from_numpy(lens.astype(np.int32)), new_k, new_v,
                      torch.from_numpy(slot), scale, used.astype(np.int64), free.astype(np.int64))


def to_e4m3_codes(t: torch.Tensor, scale: float) -> torch.Tensor:
    """uint8 FP8 E4M3 codes of t / scale, rounded by torch's float8_e4m3fn cast after clamping
    to the format's range (NaN stays NaN)."""
    y = t.to(torch.float32) / torch.tensor(scale, dtype=torch.float32)
    y = torch.where(torch.isnan(y), y, y.clamp(-448.0, 448.0))
    return y.to(torch.float8_e4m3fn).view(torch.uint8)


def to_i8_codes(t: torch.Tensor, scale: float) -> torch.Tensor:
    """uint8 bytes of the INT8 codes of t / scale (torch's round half to even, clamped to
    +-127); NaN elements (the unused slots of a poisoned cache) become -128, a code the cache
    write never produces."""
    y = t.to(torch.float32) / torch.tensor(scale, dtype=torch.float32)
    q = torch.round(torch.nan_to_num(y, nan=0.0)).clamp(-127, 127).to(torch.int8)
    q = torch.where(torch.isnan(y), torch.full_like(q, -128), q)
    return q.view(torch.uint8)


# per-cache scales of the 8-bit workloads: N(0, 1) keys and values span about +-6 within E4M3's
# +-448 and about +-4 within INT8's +-127
KV8_SCALES = {"e4m3": (0.0137, 0.0211), "i8": (0.0313, 0.0297)}


def with_8bit_cache(case, code: str = "e4m3", k_scale: Optional[float] = None,
                    v_scale: Optional[float] = None):
    """The same step with an 8-bit cache: every stored key / value (NaN in unused slots) as its
    ``code`` ('e4m3' or 'i8') with the given per-cache scales.  Queries and the step's new
    tokens keep the model's 16-bit type."""
    ks0, vs0 = KV8_SCALES[code]
    k_scale = ks0 if k_scale is None else k_scale
    v_scale = vs0 if v_scale is None else v_scale
    enc = to_e4m3_codes if code == "e4m3" else to_i8_codes
    NB, H, Dx, bs, x = case.key_cache.shape
    D = Dx * x
    # the 16-bit key layout [.., D/8, bs, 8] as [.., D/16, bs, 16] (x = 16 / sizeof(code) = 16)
    k = case.key_cache.permute(0, 1, 3, 2, 4).reshape(NB, H, bs, D // 16, 16).permute(0, 1, 3, 2, 4)
    return dataclasses.replace(case, key_cache=enc(k.contiguous(), k_scale),
                               value_cache=enc(case.value_cache, v_scale),
                               kv_dtype=code, k_scale=float(np.float32(k_scale)),
                               v_scale=float(np.float32(v_scale)))


def with_fp8_cache(case, k_scale: float = 0.0137, v_scale: float = 0.0211):
    """with_8bit_cache with E4M3 codes."""
    return with_8bit_cache(case, "e4m3", k_scale, v_scale)


def random_free_slots(case: DecodeCase, n: int, stream_seed: int = 0) -> np.ndarray:
    """``n`` distinct slots drawn uniformly from the blocks no table references."""
    g = rng(case.cfg.seed, S_SLOTS + 100 * stream_seed)
    bs = case.cfg.block_size
    all_slots = (case.free_blocks[:, None] * bs + np.arange(bs)[None, :]).reshape(-1)
    return g.choice(all_slots, size=n, replace=False).astype(np.int64)


# ---------------------------------------------------------------------------
# Shared-prefix beam search (32 prompts x 4 beams)
# ---------------------------------------------------------------------------

BEAM_CFG = DecodeConfig("c5", "shared-prefix beam search fp16", 128, 40, 40, 128, 16, "f16",
                        ("uniform", 1, 512), ("times", 1), seed=1005)


@dataclasses.dataclass
class BeamCase:
    """Prompts whose blocks are shared by all beams of the prompt, plus private blocks per beam.

    ``ref_count[block]`` is the number of block-table rows referencing the
    block (the reference counter of the mlqm.cn explainer's copy-on-write
    example).  ``free_blocks`` is the free list, in pop order.
    """
    cfg: DecodeConfig
    num_prompts: int
    beams: int
    prompt_len: int
    query: torch.Tensor
    key_cache: torch.Tensor
    value_cache: torch.Tensor
    block_tables: np.ndarray   # int32 [B, max_blocks], -1 padded
    context_lens: np.ndarray   # int32 [B]
    ref_count: np.ndarray      # int32 [NB]
    free_blocks: List[int]
    scale: float


def make_beam_case(num_prompts: int = 32, beams: int = 4, prompt_len: int = 2048,
                   max_private: int = 512, num_heads: Optional[int] = None,
                   poison: bool = True) -> BeamCase:
    cfg = BEAM_CFG
    if num_heads is not None:
        cfg = dataclasses.replace(cfg, num_heads=num_heads, num_kv_heads=num_heads)
    bs, H, D, x = cfg.block_size, cfg.num_heads, cfg.head_size, cfg.x
    B = num_prompts * beams
    priv = rng(cfg.seed, S_LENS).integers(1, max_private + 1, size=B).astype(np.int64)
    lens = prompt_len + priv
    p_blocks = (prompt_len + bs - 1) // bs
    priv_blocks = (priv + bs - 1) // bs
    n_unique = num_prompts * p_blocks + int(priv_blocks.sum())
    NB = int(math.ceil(1.5 * n_unique)) + B   # 1.5x the unique blocks + copy-on-write headroom
    perm = rng(cfg.seed, S_PERM).permutation(NB)
    used = perm[:n_unique]
    max_blocks = int(p_blocks + priv_blocks.max()) + 1
    tables = np.full((B, max_blocks), -1, dtype=np.int32)
    ref = np.zeros(NB, dtype=np.int32)
    off = 0
    prompt_ids = []
    for p in range(num_prompts):
        ids = used[off:off + p_blocks]
        off += p_blocks
        prompt_ids.append(ids)
    tdt = DTYPES[cfg.dtype]
    fill = float("nan") if poison else 0.0
    key_cache = torch.full((NB, H, D // x, bs, x), fill, dtype=tdt)
    value_cache = torch.full((NB, H, D, bs), fill, dtype=tdt)
    for b in range(B):
        p = b // beams
        tables[b, :p_blocks] = prompt_ids[p]
        n = int(priv_blocks[b])
        tables[b, p_blocks:p_blocks + n] = used[off:off + n]
        off += n
        for blk in tables[b, :p_blocks + n]:
            ref[blk] += 1
    fill_pool(key_cache, value_cache, used, cfg)
    if prompt_len % bs and poison:
        for p in range(num_prompts):
            poison_slots(key_cache, value_cache, int(prompt_ids[p][-1]), prompt_len % bs)
    for b in range(B):
        tail = int(priv[b]) % bs
        if tail and poison:
            poison_slots(key_cache, value_cache, int(tables[b, p_blocks + priv_blocks[b] - 1]), tail)
    q = _normal_to((B, H, D), rng(cfg.seed, S_Q), cfg.dtype)
    free = [int(i) for i in perm[n_unique:]]
    scale = float(np.float32(1.0 / math.sqrt(D)))
    return BeamCase(cfg, num_prompts, beams, prompt_len, q, key_cache, value_cache, tables,
                    lens.astype(np.int32), ref, free, scale)


def draw_normal(shape, dtype: str, seed: int, stream: int) -> torch.Tensor:
    """N(0,1) float32 draws rounded to ``dtype`` (for ad-hoc test tensors)."""
    return _normal_to(tuple(shape), rng(seed, stream), dtype)


# ---------------------------------------------------------------------------
# General shared-prefix groups (for the shared-prefix decode)
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class PrefixCase:
    """Groups of sequences that share their first ``prefix_lens[g]`` tokens.

    Whole blocks of a group's prefix are one set of physical blocks referenced by every
    member's table.  When the prefix ends inside a block, that block is copied into a block
    of each member (as copy-on-write leaves it), so the tables share only the whole blocks.
    """
    cfg: DecodeConfig
    query: torch.Tensor
    key_cache: torch.Tensor
    value_cache: torch.Tensor
    block_tables: np.ndarray   # int32 [B, max_blocks], -1 padded
    context_lens: np.ndarray   # int32 [B]
    group_starts: np.ndarray   # int32 [G + 1]
    prefix_lens: np.ndarray    # int32 [G]
    scale: float


def make_prefix_case(group_sizes: Sequence[int], prefix_lens: Sequence[int],
                     private: tuple = (0, 64), *, seed: int = 1105, poison: bool = True,
                     **overrides) -> PrefixCase:
    """Members of group g have prefix_lens[g] shared tokens plus U[private] tokens of their own.
    ``overrides`` replace fields of the beam configuration (heads, head size, block size,
    dtype)."""
    cfg = dataclasses.replace(BEAM_CFG, seed=seed, **overrides)
    bs, Hq, Hkv, D, x = cfg.block_size, cfg.num_heads, cfg.num_kv_heads, cfg.head_size, cfg.x
    g_len = rng(seed, S_LENS)
    lens, nshared, nown = [], [], []
    for n, pre in zip(group_sizes, prefix_lens):
        for _ in range(n):
            L = int(pre) + int(g_len.integers(private[0], private[1] + 1))
            lens.append(L)
            nshared.append(int(pre) // bs)
            nown.append((L + bs - 1) // bs - int(pre) // bs)
    B = len(lens)
    n_unique = sum(int(p) // bs for p in prefix_lens) + sum(nown)
    NB = n_unique + 8
    perm = rng(seed, S_PERM).permutation(NB)
    tdt = DTYPES[cfg.dtype]
    fill = float("nan") if poison else 0.0
    key_cache = torch.full((NB, Hkv, D // x, bs, x), fill, dtype=tdt)
    value_cache = torch.full((NB, Hkv, D, bs), fill, dtype=tdt)
    fill_pool(key_cache, value_cache, perm[:n_unique], cfg)
    max_blocks = max([s + o for s, o in zip(nshared, nown)] + [1])
    tables = np.full((B, max_blocks), -1, dtype=np.int32)
    off, b = 0, 0
    for n, pre in zip(group_sizes, prefix_lens):
        shared = perm[off:off + int(pre) // bs]
        off += len(shared)
        first_copy = None
        for _ in range(n):
            own = perm[off:off + nown[b]]
            off += nown[b]
            tables[b, :len(shared)] = shared
            tables[b, len(shared):len(shared) + len(own)] = own
            if pre % bs and len(own):
                # the prefix's partial block: every member holds a copy of the same tokens
                if first_copy is None:
                    first_copy = int(own[0])
                else:
                    key_cache[int(own[0]), :, :, :pre % bs] = key_cache[first_copy, :, :, :pre % bs]
                    value_cache[int(own[0]), :, :, :pre % bs] = value_cache[first_copy, :, :, :pre % bs]
            L = lens[b]
            if poison and L % bs and L > 0:
                poison_slots(key_cache, value_cache, int(tables[b, (L - 1) // bs]), L % bs)
            b += 1
    q = _normal_to((B, Hq, D), rng(seed, S_Q), cfg.dtype)
    starts = np.concatenate([[0], np.cumsum(group_sizes)]).astype(np.int32)
    return PrefixCase(cfg, q, key_cache, value_cache, tables, np.asarray(lens, dtype=np.int32),
                      starts, np.asarray(prefix_lens, dtype=np.int32),
                      float(np.float32(1.0 / math.sqrt(D))))


# ---------------------------------------------------------------------------
# Multi-query steps: chunked prefill and mixed batches (query_start_loc)
# ---------------------------------------------------------------------------

S_PF_LENS, S_PF_Q, S_PF_NEWKV = 20, 21, 22

PREFILL_CFG = DecodeConfig("c6", "chunked prefill bf16", 16, 32, 8, 128, 16, "bf16",
                           ("uniform", 0, 7168), ("plus", 64), seed=1006)


@dataclasses.dataclass
class PrefillCase:
    """One multi-query step: request b has ``query_lens[b]`` new tokens (its chunk) at the end
    of a context of ``context_lens[b]`` tokens.  The caches hold every earlier token; the
    chunk's own slots are still unwritten (NaN when poisoned): the step scatters ``new_key`` /
    ``new_value`` [T, Hkv, D] into ``slot_mapping`` [T] and then attends."""
    cfg: DecodeConfig
    query: torch.Tensor            # [T, Hq, D], the requests' rows one after another
    key_cache: torch.Tensor        # [NB, Hkv, D/x, bs, x]
    value_cache: torch.Tensor      # [NB, Hkv, D, bs]
    block_tables: np.ndarray       # int32 [B, max_blocks]
    context_lens: np.ndarray       # int32 [B]
    query_start_loc: np.ndarray    # int32 [B + 1]
    new_key: torch.Tensor          # [T, Hkv, D]
    new_value: torch.Tensor        # [T, Hkv, D]
    slot_mapping: np.ndarray       # int64 [T]
    scale: float
    kv_dtype: Optional[str] = None  # 'e4m3' / 'i8': caches hold 8-bit codes (new K/V stay 16-bit)
    k_scale: float = 1.0
    v_scale: float = 1.0

    @property
    def num_tokens(self) -> int:
        return int(self.query_start_loc[-1])

    @property
    def query_lens(self) -> np.ndarray:
        return np.diff(self.query_start_loc)

    @property
    def max_query_len(self) -> int:
        return int(self.query_lens.max()) if len(self.context_lens) else 0

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if len(self.context_lens) else 0


def draw_prefill_requests(cfg: DecodeConfig = PREFILL_CFG, chunk: int = 1024):
    """The chunked-prefill workload: cfg.num_seqs requests, each a ``chunk``-token piece of a
    prompt whose earlier pieces (U[lo, hi] tokens) are already cached."""
    _, lo, hi = cfg.lens
    prefix = rng(cfg.seed, S_PF_LENS).integers(lo, hi + 1, size=cfg.num_seqs)
    return [(int(p), chunk) for p in prefix]


def make_prefill_case(requests: Sequence[Tuple[int, int]], *, cfg: DecodeConfig = PREFILL_CFG,
                      poison: bool = True, **overrides) -> PrefillCase:
    """``requests`` = [(cached tokens, new query tokens)] per request; a decode token is
    (L - 1, 1).  ``overrides`` replace configuration fields (heads, head size, block size,
    dtype, seed)."""
    if overrides:
        cfg = dataclasses.replace(cfg, **overrides)
    bs, Hq, Hkv, D, x = cfg.block_size, cfg.num_heads, cfg.num_kv_heads, cfg.head_size, cfg.x
    pre = np.array([p for p, _ in requests], dtype=np.int64)
    nq = np.array([n for _, n in requests], dtype=np.int64)
    lens = pre + nq
    B = len(requests)
    nblk = (lens + bs - 1) // bs
    n_used = int(nblk.sum())
    NB = _pool_size(cfg, n_used)
    perm = rng(cfg.seed, S_PERM).permutation(NB)
    used = perm[:n_used]
    max_blocks = max(int(nblk.max()) if B else 1, 1)
    tables = np.full((B, max_blocks), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        tables[b, :nblk[b]] = used[off:off + nblk[b]]
        off += nblk[b]
    tdt = DTYPES[cfg.dtype]
    fill = float("nan") if poison else 0.0
    key_cache = torch.full((NB, Hkv, D // x, bs, x), fill, dtype=tdt)
    value_cache = torch.full((NB, Hkv, D, bs), fill, dtype=tdt)
    fill_pool(key_cache, value_cache, used, cfg)
    qsl = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    T = int(qsl[-1])
    slots = np.empty(T, dtype=np.int64)
    for b in range(B):
        for i, p in enumerate(range(int(pre[b]), int(lens[b]))):
            slots[qsl[b] + i] = int(tables[b, p // bs]) * bs + p % bs
        if poison and nq[b] > 0:
            # the chunk's slots (and the tail of its last block) are not yet written
            first = int(pre[b])
            for j in range(first // bs, int(nblk[b])):
                poison_slots(key_cache, value_cache, int(tables[b, j]),
                             first % bs if j == first // bs else 0)
    q = _normal_to((T, Hq, D), rng(cfg.seed, S_PF_Q), cfg.dtype)
    gn = rng(cfg.seed, S_PF_NEWKV)
    new_k = _normal_to((T, Hkv, D), gn, cfg.dtype)
    new_v = _normal_to((T, Hkv, D), gn, cfg.dtype)
    return PrefillCase(cfg, q, key_cache, value_cache, tables, lens.astype(np.int32), qsl,
                       new_k, new_v, slots, float(np.float32(1.0 / math.sqrt(D))))
