"""Multi-query paged attention (chunked prefill, mixed prefill / decode batches) on the GPU
against the fp64 oracle: the step scatters each chunk's new keys and values
(reshape_and_cache) and then attends with query_start_loc."""
import numpy as np
import pytest
import torch

import paged_kv_cache_164_amd as pkv
from gpu_cases import DEV, log, within_tolerance
from oracle import cache_ops as OC
from oracle import prefill as OP
from workloads import draw_prefill_requests, make_prefill_case, storage_bits

pytestmark = pytest.mark.gpu

MIXED = [(0, 1), (0, 37), (100, 300), (513, 64), (40, 1), (0, 0), (1000, 1), (31, 33),
         (2048, 200), (7, 1), (255, 257)]
SHAPES = [
    dict(num_heads=8, num_kv_heads=2, head_size=64, block_size=8),
    dict(num_heads=8, num_kv_heads=8, head_size=128, block_size=16),
    dict(num_heads=12, num_kv_heads=4, head_size=128, block_size=32),   # G = 3: ragged columns
    dict(num_heads=16, num_kv_heads=1, head_size=64, block_size=16),    # G = 16
]


def _gpu_step(case, partition_size=0, out=None, ws=None):
    """reshape_and_cache of the chunk, then the multi-query attention; returns (out, caches)."""
    kc, vc = case.key_cache.to(DEV), case.value_cache.to(DEV)
    pkv.reshape_and_cache(case.new_key.to(DEV), case.new_value.to(DEV), kc, vc,
                          torch.from_numpy(case.slot_mapping).to(DEV))
    q = case.query.to(DEV)
    out = torch.full_like(q, float("nan")) if out is None else out
    pkv.paged_attention_prefill(out, q, kc, vc, torch.from_numpy(case.block_tables).to(DEV),
                                torch.from_numpy(case.context_lens).to(DEV),
                                torch.from_numpy(case.query_start_loc).to(DEV), case.scale,
                                case.max_context_len, partition_size, ws)
    return out, kc, vc


def _oracle(case, pairs=None):
    kb, vb = storage_bits(case.key_cache).copy(), storage_bits(case.value_cache).copy()
    OC.reshape_and_cache(kb, vb, storage_bits(case.new_key), storage_bits(case.new_value),
                         case.slot_mapping)
    ref = OP.chunked_prefill(storage_bits(case.query), kb, vb, case.cfg.dtype, case.block_tables,
                             case.context_lens, case.query_start_loc, case.scale, pairs)
    return ref, kb, vb


def _as_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("shape", range(len(SHAPES)))
@pytest.mark.parametrize("P", [0, 32, 96, 1024])
def test_mixed_batch_matches_oracle(dtype, shape, P):
    kw = SHAPES[shape]
    log(f"prefill mixed {dtype} {kw} P={P}")
    case = make_prefill_case(MIXED, dtype=dtype, seed=300 + shape, **kw)
    out, kc, vc = _gpu_step(case, P)
    torch.cuda.synchronize()
    ref, kb, vb = _oracle(case)
    assert np.array_equal(storage_bits(kc.cpu()), kb) and np.array_equal(storage_bits(vc.cpu()), vb)
    ok, err, ratio = within_tolerance(_as_f64(out), ref, dtype)
    assert ok, f"max err {err}, worst ratio {ratio}"


def test_single_tokens_and_whole_prompts():
    """Only decode rows; then only whole prompts (no cached prefix), lengths around the tile
    size (64 query tokens at G = 4) and the 32-key stage."""
    kw = dict(num_heads=16, num_kv_heads=4, head_size=128, block_size=16)
    for reqs in ([(L - 1, 1) for L in (1, 2, 31, 32, 33, 700, 4096)],
                 [(0, n) for n in (1, 2, 31, 32, 33, 63, 64, 65, 128, 129, 500)]):
        log(f"prefill {reqs}")
        case = make_prefill_case(reqs, seed=311, **kw)
        out, _, _ = _gpu_step(case)
        torch.cuda.synchronize()
        ref, _, _ = _oracle(case)
        ok, err, ratio = within_tolerance(_as_f64(out), ref, "bf16")
        assert ok, f"{reqs}: max err {err}, worst ratio {ratio}"


def test_empty_requests_leave_rows_and_skip():
    """Requests with no query tokens add no rows; with every request empty nothing runs."""
    kw = dict(num_heads=8, num_kv_heads=8, head_size=64, block_size=16)
    case = make_prefill_case([(50, 0), (10, 5), (70, 0)], seed=312, **kw)
    out, _, _ = _gpu_step(case, 32)
    torch.cuda.synchronize()
    ref, _, _ = _oracle(case)
    ok, err, _ = within_tolerance(_as_f64(out), ref, "bf16")
    assert ok, err
    empty = make_prefill_case([(50, 0), (70, 0)], seed=313, **kw)
    q = empty.query.to(DEV)
    assert q.shape[0] == 0
    pkv.paged_attention_prefill(torch.empty_like(q), q, empty.key_cache.to(DEV),
                                empty.value_cache.to(DEV),
                                torch.from_numpy(empty.block_tables).to(DEV),
                                torch.from_numpy(empty.context_lens).to(DEV),
                                torch.from_numpy(empty.query_start_loc).to(DEV), empty.scale,
                                empty.max_context_len)


def test_deterministic_and_split_consistent():
    """Two runs give the same bits; splitting the keys (P = 64) stays within tolerance of the
    unsplit result and of the oracle."""
    kw = dict(num_heads=32, num_kv_heads=8, head_size=128, block_size=16)
    case = make_prefill_case([(300, 200), (0, 129), (1500, 1)], seed=314, **kw)
    a, _, _ = _gpu_step(case)
    b, _, _ = _gpu_step(case)
    c, _, _ = _gpu_step(case, 64)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    ref, _, _ = _oracle(case)
    for got in (a, c):
        ok, err, _ = within_tolerance(_as_f64(got), ref, "bf16")
        assert ok, err


@pytest.mark.parametrize("P", [0, 2048])
def test_full_chunked_prefill_workload_sampled(P):
    """The chunked-prefill workload at full size (16 requests x 1024 new tokens after
    U[0, 7168] cached ones, 32 / 8 heads, head 128, block 16, bf16): sampled (row, head)
    pairs against the oracle, including each request's first and last rows."""
    reqs = draw_prefill_requests()
    case = make_prefill_case(reqs)
    log(f"chunked prefill workload: {case.num_tokens} rows, max context {case.max_context_len}, P={P}")
    out, _, _ = _gpu_step(case, P)
    torch.cuda.synchronize()
    g = np.random.default_rng(5)
    Hq = case.cfg.num_heads
    pairs = set()
    for b in range(len(reqs)):
        s0, s1 = int(case.query_start_loc[b]), int(case.query_start_loc[b + 1])
        for r in (s0, s0 + 63, s0 + 64, s1 - 1):
            pairs.add((r, int(g.integers(Hq))))
        for r in g.integers(s0, s1, size=6):
            pairs.add((int(r), int(g.integers(Hq))))
    pairs = sorted(pairs)
    ref, _, _ = _oracle(case, pairs)
    got = _as_f64(out)
    rows = np.array([p[0] for p in pairs])
    heads = np.array([p[1] for p in pairs])
    ok, err, ratio = within_tolerance(got[rows, heads], ref[rows, heads], "bf16")
    assert ok, f"max err {err}, worst ratio {ratio}"
    assert np.isfinite(got).all()


@pytest.mark.parametrize("code", ["e4m3", "i8"])
def test_full_chunked_prefill_workload_kv8_sampled(code):
    """The chunked-prefill workload at full size over an 8-bit cache (E4M3 or INT8 codes with
    per-cache scales): the chunk quantised into the cache, then the multi-query call; sampled
    (row, head) pairs against the oracle over the codes, including each request's first and
    last rows and both sides of a 64-row tile boundary."""
    from workloads import with_8bit_cache
    reqs = draw_prefill_requests()
    case = with_8bit_cache(make_prefill_case(reqs), code)
    log(f"chunked prefill workload over {code}: {case.num_tokens} rows, max context {case.max_context_len}")
    kc, vc = case.key_cache.to(DEV), case.value_cache.to(DEV)
    pkv.reshape_and_cache_fp8(case.new_key.to(DEV), case.new_value.to(DEV), kc, vc,
                              torch.from_numpy(case.slot_mapping).to(DEV), case.k_scale, case.v_scale,
                              code=code)
    q = case.query.to(DEV)
    out = torch.full_like(q, float("nan"))
    pkv.paged_attention_prefill(out, q, kc, vc, torch.from_numpy(case.block_tables).to(DEV),
                                torch.from_numpy(case.context_lens).to(DEV),
                                torch.from_numpy(case.query_start_loc).to(DEV), case.scale,
                                case.max_context_len, 0, k_scale=case.k_scale, v_scale=case.v_scale,
                                code=code)
    torch.cuda.synchronize()
    g = np.random.default_rng(6)
    Hq = case.cfg.num_heads
    pairs = set()
    for b in range(len(reqs)):
        s0, s1 = int(case.query_start_loc[b]), int(case.query_start_loc[b + 1])
        for r in (s0, s0 + 63, s0 + 64, s1 - 1):
            pairs.add((r, int(g.integers(Hq))))
        for r in g.integers(s0, s1, size=4):
            pairs.add((int(r), int(g.integers(Hq))))
    pairs = sorted(pairs)
    from oracle import cache_ops as OC8
    kb, vb = storage_bits(case.key_cache).copy(), storage_bits(case.value_cache).copy()
    write = OC8.reshape_and_cache_fp8 if code == "e4m3" else OC8.reshape_and_cache_int8
    write(kb, vb, storage_bits(case.new_key), storage_bits(case.new_value), "bf16",
          case.slot_mapping, case.k_scale, case.v_scale)
    assert np.array_equal(kc.cpu().numpy(), kb) and np.array_equal(vc.cpu().numpy(), vb)
    ref = OP.chunked_prefill(storage_bits(case.query), kb, vb, "bf16", case.block_tables,
                             case.context_lens, case.query_start_loc, case.scale, pairs,
                             kv_dtype=code, k_scale=case.k_scale, v_scale=case.v_scale)
    got = _as_f64(out)
    rows = np.array([p[0] for p in pairs])
    heads = np.array([p[1] for p in pairs])
    ok, err, ratio = within_tolerance(got[rows, heads], ref[rows, heads], "bf16")
    assert ok, f"max err {err}, worst ratio {ratio}"
    assert np.isfinite(got).all()


@pytest.mark.parametrize("code", ["e4m3", "i8"])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("shape", [0, 2, 3])
@pytest.mark.parametrize("P", [0, 96])
def test_kv8_cache_mixed_batch_matches_oracle(dtype, shape, P, code):
    """The multi-query call over an 8-bit cache (E4M3 or INT8 codes): the chunk quantised into
    the cache by the 8-bit cache write (bit-exact), then attention against the oracle over the
    codes."""
    from oracle import cache_ops as OC8
    from workloads import with_8bit_cache
    kw = SHAPES[shape]
    log(f"prefill {code} mixed {dtype} {kw} P={P}")
    case = with_8bit_cache(make_prefill_case(MIXED, dtype=dtype, seed=400 + shape, **kw), code)
    kc, vc = case.key_cache.to(DEV), case.value_cache.to(DEV)
    pkv.reshape_and_cache_fp8(case.new_key.to(DEV), case.new_value.to(DEV), kc, vc,
                              torch.from_numpy(case.slot_mapping).to(DEV), case.k_scale, case.v_scale,
                              code=code)
    q = case.query.to(DEV)
    out = torch.full_like(q, float("nan"))
    pkv.paged_attention_prefill(out, q, kc, vc, torch.from_numpy(case.block_tables).to(DEV),
                                torch.from_numpy(case.context_lens).to(DEV),
                                torch.from_numpy(case.query_start_loc).to(DEV), case.scale,
                                case.max_context_len, P, k_scale=case.k_scale, v_scale=case.v_scale,
                                code=code)
    torch.cuda.synchronize()
    kb, vb = storage_bits(case.key_cache).copy(), storage_bits(case.value_cache).copy()
    write = OC8.reshape_and_cache_fp8 if code == "e4m3" else OC8.reshape_and_cache_int8
    write(kb, vb, storage_bits(case.new_key), storage_bits(case.new_value), dtype,
          case.slot_mapping, case.k_scale, case.v_scale)
    assert np.array_equal(kc.cpu().numpy(), kb) and np.array_equal(vc.cpu().numpy(), vb)
    ref = OP.chunked_prefill(storage_bits(case.query), kb, vb, dtype, case.block_tables,
                             case.context_lens, case.query_start_loc, case.scale,
                             kv_dtype=code, k_scale=case.k_scale, v_scale=case.v_scale)
    ok, err, ratio = within_tolerance(_as_f64(out), ref, dtype)
    assert ok, f"max err {err}, worst ratio {ratio}"


@pytest.mark.parametrize("code", [None, "e4m3"])
def test_stage_count_sweep(code):
    """Requests whose keys take 1..14 stages of 32, each with a partial last stage at another
    offset, over a cache poisoned (NaN) past every context: every position of the unrolled
    stage loop and its tail, the stores of the prologue and of the loop, and the zeroing of
    the last stage's values (in LDS for the prologue's stages, in registers for the loop's)."""
    from oracle import cache_ops as OC8
    from workloads import with_8bit_cache
    reqs = []
    for nst in range(1, 15):
        L = 32 * (nst - 1) + 1 + (nst * 11) % 32    # the last stage holds 1..32 keys
        n = 1 + (nst * 5) % min(L, 9)               # a few query rows: one tile
        reqs.append((L - n, n))
    kw = dict(num_heads=8, num_kv_heads=2, head_size=128, block_size=16)
    case = make_prefill_case(reqs, seed=420, **kw)
    log(f"stage sweep {code}: {reqs}")
    if code is None:
        out, _, _ = _gpu_step(case)
        torch.cuda.synchronize()
        ref, _, _ = _oracle(case)
    else:
        case = with_8bit_cache(case, code)
        kc, vc = case.key_cache.to(DEV), case.value_cache.to(DEV)
        pkv.reshape_and_cache_fp8(case.new_key.to(DEV), case.new_value.to(DEV), kc, vc,
                                  torch.from_numpy(case.slot_mapping).to(DEV), case.k_scale,
                                  case.v_scale, code=code)
        q = case.query.to(DEV)
        out = torch.full_like(q, float("nan"))
        pkv.paged_attention_prefill(out, q, kc, vc, torch.from_numpy(case.block_tables).to(DEV),
                                    torch.from_numpy(case.context_lens).to(DEV),
                                    torch.from_numpy(case.query_start_loc).to(DEV), case.scale,
                                    case.max_context_len, 0, k_scale=case.k_scale,
                                    v_scale=case.v_scale, code=code)
        torch.cuda.synchronize()
        kb, vb = storage_bits(case.key_cache).copy(), storage_bits(case.value_cache).copy()
        OC8.reshape_and_cache_fp8(kb, vb, storage_bits(case.new_key), storage_bits(case.new_value),
                                  "bf16", case.slot_mapping, case.k_scale, case.v_scale)
        ref = OP.chunked_prefill(storage_bits(case.query), kb, vb, "bf16", case.block_tables,
                                 case.context_lens, case.query_start_loc, case.scale,
                                 kv_dtype=code, k_scale=case.k_scale, v_scale=case.v_scale)
    got = _as_f64(out)
    assert np.isfinite(got).all()
    ok, err, ratio = within_tolerance(got, ref, "bf16")
    assert ok, f"max err {err}, worst ratio {ratio}"
