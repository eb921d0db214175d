"""Pins for the cache-operation oracle and the closed forms (CPU only)."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import attention as OA
from oracle import cache_ops as OC
from workloads import storage_bits, draw_normal, DTYPES

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _cache(NB, H, D, bs, dtype, fill=float("nan")):
    x = 16 // torch.tensor([], dtype=DTYPES[dtype]).element_size()
    kc = torch.full((NB, H, D // x, bs, x), fill, dtype=DTYPES[dtype])
    vc = torch.full((NB, H, D, bs), fill, dtype=DTYPES[dtype])
    return kc, vc


@pytest.mark.parametrize("dtype,bs", [("f32", 16), ("f16", 8), ("bf16", 32)])
def test_reshape_and_cache_matches_slot_view(dtype, bs):
    """Against torch indexing on a slot-major view: permute the key cache to
    [block, token, head, chunk, x], flatten to [slot, head, dim] and assign rows."""
    NB, H, D, N = 7, 3, 16, 20
    kc, vc = _cache(NB, H, D, bs, dtype)
    key = draw_normal((N, H, D), dtype, 1, 0)
    val = draw_normal((N, H, D), dtype, 1, 1)
    slots = np.random.default_rng(2).choice(NB * bs, size=N, replace=False)
    slots[3] = -1
    slots[11] = -5
    kb, vb = storage_bits(kc).copy(), storage_bits(vc).copy()
    OC.reshape_and_cache(kb, vb, storage_bits(key), storage_bits(val), slots)

    kview = kc.clone().permute(0, 3, 1, 2, 4).reshape(NB * bs, H, D)    # copy: [slot, head, dim]
    vview = vc.clone().permute(0, 3, 1, 2).reshape(NB * bs, H, D)
    keep = torch.from_numpy(slots >= 0)
    idx = torch.from_numpy(slots[slots >= 0])
    kview[idx] = key[keep]
    vview[idx] = val[keep]
    x = kc.shape[4]
    kref = kview.reshape(NB, bs, H, D // x, x).permute(0, 2, 3, 1, 4).contiguous()
    vref = vview.reshape(NB, bs, H, D).permute(0, 2, 3, 1).contiguous()
    assert np.array_equal(kb, storage_bits(kref))
    assert np.array_equal(vb, storage_bits(vref))


def test_reshape_then_gather_round_trip():
    """Scatter a sequence's tokens through its block table, gather them back with the attention
    oracle's gather: the dense K and V come back unchanged."""
    H, D, bs, L = 2, 16, 8, 29
    kc, vc = _cache(9, H, D, bs, "bf16")
    table = np.array([6, 2, 8, 0], dtype=np.int32)
    key = draw_normal((L, H, D), "bf16", 3, 0)
    val = draw_normal((L, H, D), "bf16", 3, 1)
    slots = [OC.slot_of(table, t, bs) for t in range(L)]
    kb, vb = storage_bits(kc).copy(), storage_bits(vc).copy()
    OC.reshape_and_cache(kb, vb, storage_bits(key), storage_bits(val), slots)
    for h in range(H):
        K, V = OA.gather_kv(kb, vb, "bf16", table, L, h)
        assert np.array_equal(K, key[:, h].to(torch.float64).numpy())
        assert np.array_equal(V, val[:, h].to(torch.float64).numpy())


def test_negative_slot_writes_nothing():
    kc, vc = _cache(3, 2, 8, 4, "f16", fill=0.0)
    kb, vb = storage_bits(kc).copy(), storage_bits(vc).copy()
    key = draw_normal((2, 2, 8), "f16", 4, 0)
    OC.reshape_and_cache(kb, vb, storage_bits(key), storage_bits(key), [-1, -1])
    assert not kb.any() and not vb.any()


def test_cow_worked_example():
    """The copy-on-write walk-through of the mlqm.cn explainer (golden/cow_worked_example.json)."""
    spec = json.load(open(os.path.join(GOLDEN, "cow_worked_example.json")))
    bs = spec["block_size"]
    prompt = spec["prompt_tokens"]
    H, D = 1, 8
    NB = 4
    kc, vc = _cache(NB, H, D, bs, "f16", fill=0.0)
    # prompt tokens: value = token index + 1 in every dim
    kb, vb = storage_bits(kc).copy(), storage_bits(vc).copy()
    pk = torch.arange(1, prompt + 1, dtype=torch.float16)[:, None, None].expand(prompt, H, D).contiguous()
    OC.reshape_and_cache(kb, vb, storage_bits(pk), storage_bits(pk),
                         [OC.slot_of([0, 1], t, bs) for t in range(prompt)])
    tables = {k: list(v) for k, v in spec["initial_tables"].items()}
    ref = {int(k): v for k, v in spec["initial_ref_count"].items()}
    free = list(spec["free_list"])
    copies, slots, refs = [], {}, []
    new_tok = {"A": 100.0, "B": 200.0, "C": 300.0}
    for seq in ("A", "B", "C"):
        last = tables[seq][-1]
        if ref[last] > 1:                      # shared: copy the block before writing
            new = free.pop(0)
            OC.copy_blocks([kb, vb], [(last, new)])
            copies.append([last, new])
            ref[last] -= 1
            ref[new] = 1
            tables[seq][-1] = new
            refs.append({str(last): ref[last], str(new): 1})
        else:
            refs.append({str(last): ref[last]})
        s = OC.slot_of(tables[seq], prompt, bs)
        slots[seq] = s
        t = torch.full((1, H, D), new_tok[seq], dtype=torch.float16)
        OC.reshape_and_cache(kb, vb, storage_bits(t), storage_bits(t), [s])
    exp = spec["expected"]
    assert copies == exp["copies"]
    assert tables == exp["tables"]
    assert slots == exp["new_token_slots"]
    assert refs == exp["ref_count_after_each_write"]
    # contents: every copy carries block 1's 10 prompt tokens, then the sequence's own token
    V = OA.widen(vb, "f16")
    for seq, blk in (("A", 2), ("B", 3), ("C", 1)):
        assert np.array_equal(V[blk, 0, 0, :10], np.arange(17, 27))
        assert V[blk, 0, 0, 10] == new_tok[seq]
        assert not V[blk, 0, 0, 11:].any()
    assert np.array_equal(V[0, 0, 0, :], np.arange(1, 17))


def test_copy_blocks_reads_pre_call_state_and_spares_others():
    kc, vc = _cache(6, 2, 8, 4, "bf16", fill=0.0)
    kc[:] = draw_normal(kc.shape, "bf16", 6, 0)
    vc[:] = draw_normal(vc.shape, "bf16", 6, 1)
    kb, vb = storage_bits(kc).copy(), storage_bits(vc).copy()
    before_k, before_v = kb.copy(), vb.copy()
    OC.copy_blocks([kb, vb], [(1, 4), (1, 5), (3, 0)])
    assert np.array_equal(kb[4], before_k[1]) and np.array_equal(kb[5], before_k[1])
    assert np.array_equal(vb[0], before_v[3])
    for blk in (1, 2, 3):
        assert np.array_equal(kb[blk], before_k[blk]) and np.array_equal(vb[blk], before_v[blk])


def test_swap_out_then_in_is_identity():
    dev = storage_bits(draw_normal((8, 2, 2, 4, 8), "f16", 7, 0)).copy()
    host = np.zeros((5, 2, 2, 4, 8), dtype=np.uint16)
    out_map = [(1, 0), (6, 3), (2, 4)]
    OC.swap_blocks(host, dev, out_map)
    dev2 = dev.copy()
    dev2[[1, 6, 2]] = 0
    back = [(0, 1), (3, 6), (4, 2)]
    OC.swap_blocks(dev2, host, back)
    assert np.array_equal(dev2, dev)


# ---------------------------------------------------------------- closed forms

def test_memory_waste_bound():
    """At most the last block is partial: at most bs-1 = 15 empty slots per sequence at bs 16
    (mlqm.cn explainer, section '1、PagedAttention')."""
    assert OC.memory_waste([16, 17], 16) == 15 / 48
    lens = np.random.default_rng(0).integers(1, 5000, size=500)
    alloc = ((lens + 15) // 16) * 16
    assert np.all(alloc - lens <= 15)
    assert OC.memory_waste(lens, 16) <= 15 * len(lens) / alloc.sum()


def test_kv_bytes_llama13b():
    """LLaMA-13B (40 layers, 40 heads, head dim 128), one 8192-token request in fp16: the page says
    about 6 GB; the closed form gives 6,710,886,400 B = 6.25 GiB."""
    b = OC.kv_cache_bytes(1, 8192, 40, 40, 128, 2)
    assert b == 6710886400
    assert round(b / 2 ** 30) == 6
