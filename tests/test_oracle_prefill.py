"""Pins of the multi-query (chunked prefill) oracle: a library causal SDPA, chunked-vs-whole
prefill, decode rows, closed forms, invariants and a planted alignment mistake."""
import numpy as np
import pytest
import torch

from oracle import attention as OA
from oracle import cache_ops as OC
from oracle import prefill as OP
from workloads import make_prefill_case, storage_bits


def _step(case):
    """The caches after the step's scatter of the chunk's K/V, as raw bits."""
    kb, vb = storage_bits(case.key_cache).copy(), storage_bits(case.value_cache).copy()
    OC.reshape_and_cache(kb, vb, storage_bits(case.new_key), storage_bits(case.new_value),
                         case.slot_mapping)
    return kb, vb


def _run(case, pairs=None):
    kb, vb = _step(case)
    return OP.chunked_prefill(storage_bits(case.query), kb, vb, case.cfg.dtype, case.block_tables,
                              case.context_lens, case.query_start_loc, case.scale, pairs)


SMALL = dict(num_heads=4, num_kv_heads=2, head_size=32, block_size=8)


@pytest.mark.parametrize("kv_heads", [4, 2, 1])
def test_whole_prompt_equals_causal_sdpa(kv_heads):
    """A request with no cached tokens (n = L) is causal self-attention: equal to torch's
    scaled_dot_product_attention(is_causal=True) in float64 on the gathered dense K, V."""
    case = make_prefill_case([(0, 37), (0, 1), (0, 16)], **{**SMALL, "num_kv_heads": kv_heads})
    out = _run(case)
    kb, vb = _step(case)
    G = case.cfg.num_heads // kv_heads
    for b in range(3):
        s0, s1 = case.query_start_loc[b], case.query_start_loc[b + 1]
        L = int(case.context_lens[b])
        q = torch.from_numpy(OA.widen(storage_bits(case.query)[s0:s1], "bf16")).permute(1, 0, 2)
        Ks, Vs = [], []
        for h in range(kv_heads):
            K, V = OA.gather_kv(kb, vb, "bf16", case.block_tables[b], L, h)
            Ks.append(K)
            Vs.append(V)
        K = torch.from_numpy(np.stack(Ks)).repeat_interleave(G, 0)
        V = torch.from_numpy(np.stack(Vs)).repeat_interleave(G, 0)
        ref = torch.nn.functional.scaled_dot_product_attention(
            q, K, V, is_causal=True, scale=OA.as_scale(case.scale)).permute(1, 0, 2).numpy()
        np.testing.assert_allclose(out[s0:s1], ref, rtol=0, atol=1e-12)


def test_chunks_equal_whole_prompt():
    """Prefilling a prompt in chunks (each chunk's queries at the end of the context cached so
    far) gives every row the output of the whole-prompt prefill: this pins the bottom-right
    placement of a chunk's queries."""
    L, cuts = 70, [0, 23, 40, 41, 70]
    whole = make_prefill_case([(0, L)], **SMALL, seed=7)
    ref = _run(whole)
    kb, vb = _step(whole)
    qb = storage_bits(whole.query)
    for c0, c1 in zip(cuts[:-1], cuts[1:]):
        got = OP.chunked_prefill(qb[c0:c1], kb, vb, "bf16", whole.block_tables,
                                 np.array([c1], np.int32), np.array([0, c1 - c0], np.int32),
                                 whole.scale)
        assert np.array_equal(got, ref[c0:c1]), (c0, c1)


def test_planted_top_left_alignment_is_caught(monkeypatch):
    """Queries placed at the start of the context (top-left) instead of its end fail the
    chunk equivalence."""
    whole = make_prefill_case([(0, 30)], **SMALL, seed=8)
    ref = _run(whole)
    kb, vb = _step(whole)
    monkeypatch.setattr(OP, "query_positions", lambda L, n: np.arange(0, n))
    got = OP.chunked_prefill(storage_bits(whole.query)[20:30], kb, vb, "bf16", whole.block_tables,
                             np.array([30], np.int32), np.array([0, 10], np.int32), whole.scale)
    assert not np.allclose(got, ref[20:30])


def test_decode_rows_equal_paged_decode():
    """A request with one query token is the decode step of the single-query path."""
    case = make_prefill_case([(40, 1), (0, 9), (100, 1), (7, 1)], **SMALL, seed=9)
    out = _run(case)
    kb, vb = _step(case)
    rows = [int(case.query_start_loc[b]) for b in (0, 2, 3)]
    dec = OA.paged_decode(storage_bits(case.query)[rows], kb, vb, "bf16",
                          case.block_tables[[0, 2, 3]], case.context_lens[[0, 2, 3]], case.scale)
    assert np.array_equal(out[rows], dec)


def test_first_query_of_a_prompt_returns_its_value():
    """The query at position 0 sees one key: its output is V[0] exactly, whatever q and K."""
    case = make_prefill_case([(0, 12), (0, 5)], **SMALL, seed=10)
    out = _run(case)
    kb, vb = _step(case)
    G = case.cfg.num_heads // case.cfg.num_kv_heads
    for b in range(2):
        r = int(case.query_start_loc[b])
        for h in range(case.cfg.num_heads):
            _, V = OA.gather_kv(kb, vb, "bf16", case.block_tables[b], 1, h // G)
            assert np.array_equal(out[r, h], V[0])


def test_two_token_closed_form():
    """Position 1 of a prompt: w = 1 / (1 + exp(scale (q.k0 - q.k1))), out = w v1 + (1-w) v0."""
    case = make_prefill_case([(0, 2)], **SMALL, seed=11)
    out = _run(case)
    kb, vb = _step(case)
    K, V = OA.gather_kv(kb, vb, "bf16", case.block_tables[0], 2, 0)
    q = OA.widen(storage_bits(case.query)[1, 0], "bf16")
    sc = OA.as_scale(case.scale)
    w1 = 1.0 / (1.0 + np.exp(sc * (q @ K[0] - q @ K[1])))
    np.testing.assert_allclose(out[1, 0], w1 * V[1] + (1 - w1) * V[0], rtol=1e-13, atol=1e-14)


def test_empty_query_and_block_permutation():
    """A request with no query tokens contributes no rows; relabelling physical blocks
    changes nothing."""
    reqs = [(17, 5), (30, 0), (0, 8), (5, 1)]
    case = make_prefill_case(reqs, **SMALL, seed=12)
    out = _run(case)
    assert out.shape[0] == 14 and np.all(np.isfinite(out))
    kb, vb = _step(case)
    NB = kb.shape[0]
    perm = np.random.default_rng(0).permutation(NB)
    kp, vp = np.empty_like(kb), np.empty_like(vb)
    kp[perm], vp[perm] = kb, vb
    tables = np.where(case.block_tables >= 0, perm[np.maximum(case.block_tables, 0)], -1)
    got = OP.chunked_prefill(storage_bits(case.query), kp, vp, "bf16", tables, case.context_lens,
                             case.query_start_loc, case.scale)
    assert np.array_equal(got, out)


def test_sampled_pairs_match_full():
    case = make_prefill_case([(9, 20), (0, 3), (50, 1)], **SMALL, seed=13)
    full = _run(case)
    pairs = [(0, 1), (19, 3), (21, 0), (23, 2)]
    part = _run(case, pairs)
    for r, h in pairs:
        assert np.array_equal(part[r, h], full[r, h])
    assert np.isnan(part[5, 0]).all()


def test_flop_count_closed_form():
    # positions L-n..L-1 see L-n+1..L keys: n (L-n) + n (n+1) / 2 visible pairs
    qsl, lens = np.array([0, 4, 5]), np.array([10, 3])
    pairs = (4 * 6 + 10) + (1 * 2 + 1)
    assert OP.attention_flops(lens, qsl, 2, 8) == 4 * 8 * 2 * pairs


def _kv8_step(case):
    """The caches after the step's scatter into an 8-bit cache (the chunk quantised)."""
    kb, vb = storage_bits(case.key_cache).copy(), storage_bits(case.value_cache).copy()
    write = OC.reshape_and_cache_fp8 if case.kv_dtype == "e4m3" else OC.reshape_and_cache_int8
    write(kb, vb, storage_bits(case.new_key), storage_bits(case.new_value),
          case.cfg.dtype, case.slot_mapping, case.k_scale, case.v_scale)
    return kb, vb


@pytest.mark.parametrize("code", ["e4m3", "i8"])
def test_kv8_whole_prompt_equals_sdpa_on_dequantised_kv(code):
    """Over an 8-bit cache: whole prompts equal causal SDPA on K, V dequantised by torch's own
    casts (float8_e4m3fn or int8 to float64, independent of the oracle's codecs), times the
    scales."""
    from workloads import with_8bit_cache
    case = with_8bit_cache(make_prefill_case([(0, 29), (0, 8)], **SMALL, seed=20), code)
    kb, vb = _kv8_step(case)
    out = OP.chunked_prefill(storage_bits(case.query), kb, vb, "bf16", case.block_tables,
                             case.context_lens, case.query_start_loc, case.scale,
                             kv_dtype=code, k_scale=case.k_scale, v_scale=case.v_scale)
    tdt = torch.float8_e4m3fn if code == "e4m3" else torch.int8
    G = case.cfg.num_heads // case.cfg.num_kv_heads
    x = kb.shape[-1]
    for b in range(2):
        s0, s1 = case.query_start_loc[b], case.query_start_loc[b + 1]
        L = int(case.context_lens[b])
        t = np.arange(L)
        blk = case.block_tables[b][t // case.cfg.block_size]
        off = t % case.cfg.block_size
        Ks, Vs = [], []
        for h in range(case.cfg.num_kv_heads):
            d = np.arange(case.cfg.head_size)
            kcode = kb[blk[:, None], h, (d // x)[None, :], off[:, None], (d % x)[None, :]]
            vcode = vb[blk[:, None], h, d[None, :], off[:, None]]
            deq = lambda c, sc: (torch.from_numpy(np.ascontiguousarray(c)).view(tdt)
                                 .to(torch.float64) * float(np.float32(sc)))
            Ks.append(deq(kcode, case.k_scale))
            Vs.append(deq(vcode, case.v_scale))
        K = torch.stack(Ks).repeat_interleave(G, 0)
        V = torch.stack(Vs).repeat_interleave(G, 0)
        q = torch.from_numpy(OA.widen(storage_bits(case.query)[s0:s1], "bf16")).permute(1, 0, 2)
        ref = torch.nn.functional.scaled_dot_product_attention(
            q, K, V, is_causal=True, scale=OA.as_scale(case.scale)).permute(1, 0, 2).numpy()
        np.testing.assert_allclose(out[s0:s1], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("code", ["e4m3", "i8"])
def test_kv8_decode_rows_equal_kv8_paged_decode(code):
    from workloads import with_8bit_cache
    case = with_8bit_cache(make_prefill_case([(40, 1), (0, 9), (100, 1)], **SMALL, seed=21), code)
    kb, vb = _kv8_step(case)
    out = OP.chunked_prefill(storage_bits(case.query), kb, vb, "bf16", case.block_tables,
                             case.context_lens, case.query_start_loc, case.scale,
                             kv_dtype=code, k_scale=case.k_scale, v_scale=case.v_scale)
    rows = [int(case.query_start_loc[b]) for b in (0, 2)]
    dec = OA.paged_decode(storage_bits(case.query)[rows], kb, vb, "bf16", case.block_tables[[0, 2]],
                          case.context_lens[[0, 2]], case.scale, kv_dtype=code,
                          k_scale=case.k_scale, v_scale=case.v_scale)
    assert np.array_equal(out[rows], dec)
