"""Shared-prefix beam search: 4 beams per prompt share the prompt's physical blocks.

Copy-on-write of each beam's partial last block (copy_blocks), the new token written into
the fresh block (reshape_and_cache), decode over the shared blocks; then 25% of the blocks
in use are swapped out to pinned host memory, the device copies poisoned, swapped back
into different block ids and every table remapped: the decode output must be bit-identical
to the one before the swap, and both must match the fp64 oracle.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_164_amd as pkv
from gpu_cases import DEV, log, within_tolerance
from oracle import attention as OA
from oracle import cache_ops as OC
from workloads import S_COW, S_SWAP, draw_normal, make_beam_case, rng, storage_bits

pytestmark = pytest.mark.gpu


def _decode(q, kc, vc, tables, lens, scale):
    out = torch.empty_like(q)
    lmax = int(lens.max())
    pkv.paged_attention_decode(out, q, kc, vc, torch.from_numpy(tables).to(DEV),
                               torch.from_numpy(lens).to(DEV), scale, lmax)
    return out


def _decode_shared(q, kc, vc, tables, lens, scale, beams, prompt_len):
    """The beams of one prompt are one group sharing the prompt's blocks."""
    out = torch.empty_like(q)
    B = q.shape[0]
    gs = torch.arange(0, B + 1, beams, dtype=torch.int32, device=DEV)
    pl = torch.full((B // beams,), prompt_len, dtype=torch.int32, device=DEV)
    pkv.paged_attention_decode_shared(out, q, kc, vc, torch.from_numpy(tables).to(DEV),
                                      torch.from_numpy(lens).to(DEV), gs, pl, scale, int(lens.max()))
    return out


def _cow_step(bc):
    """One beam step's bookkeeping: copy-on-write of each beam's partial last block into a
    free block, and the slot of its next token there.  Returns the new tables and lengths,
    the copy pairs, the slots, the new keys and values and the remaining free list."""
    bs = bc.cfg.block_size
    B, H, D = bc.query.shape
    tables, lens = bc.block_tables.copy(), bc.context_lens.copy()
    free, ref = list(bc.free_blocks), bc.ref_count.copy()
    pairs, slots = [], np.full(B, -1, dtype=np.int64)
    for b in range(B):
        L = int(lens[b])
        if L % bs:
            j = (L - 1) // bs
            last, new = int(tables[b, j]), free.pop(0)
            pairs.append((last, new))
            tables[b, j] = new
            ref[last] -= 1
            ref[new] = 1
            slots[b] = new * bs + L % bs
            lens[b] = L + 1
    nk = draw_normal((B, H, D), "f16", bc.cfg.seed, S_COW)
    nv = draw_normal((B, H, D), "f16", bc.cfg.seed, S_COW + 100)
    mapping = np.array(pairs, dtype=np.int64).reshape(-1, 2)
    return tables, lens, pairs, mapping, slots, nk, nv, free


def _beam_run(num_prompts, n_pairs=None):
    bc = make_beam_case(num_prompts=num_prompts)
    B, H, D = bc.query.shape
    log(f"beam: {num_prompts} prompts x {bc.beams} beams, H={H}, pool={bc.key_cache.shape[0]}")
    kc, vc = bc.key_cache.to(DEV), bc.value_cache.to(DEV)
    q = bc.query.to(DEV)
    # (i) copy-on-write of each beam's partial last block, then its next token
    tables, lens, pairs, mapping, slots, nk, nv, free = _cow_step(bc)
    pkv.copy_blocks([kc], [vc], torch.from_numpy(mapping).to(DEV))
    pkv.reshape_and_cache(nk.to(DEV), nv.to(DEV), kc, vc, torch.from_numpy(slots).to(DEV))
    out1 = _decode(q, kc, vc, tables, lens, bc.scale)
    sh1 = _decode_shared(q, kc, vc, tables, lens, bc.scale, bc.beams, bc.prompt_len)
    torch.cuda.synchronize()
    log(f"beam: {len(pairs)} copy-on-write pairs")

    kb, vb = storage_bits(bc.key_cache).copy(), storage_bits(bc.value_cache).copy()
    OC.copy_blocks([kb, vb], mapping)
    OC.reshape_and_cache(kb, vb, storage_bits(nk), storage_bits(nv), slots)
    assert np.array_equal(storage_bits(kc.cpu()), kb) and np.array_equal(storage_bits(vc.cpu()), vb)
    all_pairs = None
    if n_pairs is not None:
        g = np.random.default_rng(0)
        all_pairs = sorted({(int(g.integers(B)), int(g.integers(H))) for _ in range(n_pairs)})
    ref_out = OA.paged_decode(storage_bits(bc.query), kb, vb, "f16", tables, lens, bc.scale,
                              pairs=all_pairs)
    for name, o in (("plain", out1), ("shared-prefix", sh1)):
        got = o.cpu().to(torch.float64).numpy()
        ref_sel = ref_out
        if all_pairs is not None:
            idx = tuple(np.array(all_pairs).T)
            got, ref_sel = got[idx], ref_out[idx]
        ok, err, ratio = within_tolerance(got, ref_sel, "f16")
        log(f"beam {name} decode vs oracle: max|err|={err:.3e} ratio={ratio:.3f}")
        assert ok

    # (ii) swap 25% of the blocks in use out to pinned host memory and back into new ids
    in_use = np.unique(tables[tables >= 0])
    g = rng(bc.cfg.seed, S_SWAP)
    chosen = np.sort(g.choice(in_use, size=len(in_use) // 4, replace=False))
    n = len(chosen)
    host_k = torch.empty((n,) + tuple(kc.shape[1:]), dtype=kc.dtype).pin_memory()
    host_v = torch.empty((n,) + tuple(vc.shape[1:]), dtype=vc.dtype).pin_memory()
    out_map = np.stack([chosen, np.arange(n)], axis=1)
    pkv.swap_blocks(kc, host_k, out_map)
    pkv.swap_blocks(vc, host_v, out_map)
    torch.cuda.synchronize()
    kc[torch.from_numpy(chosen).to(DEV)] = float("nan")
    vc[torch.from_numpy(chosen).to(DEV)] = float("nan")
    new_ids = np.array([free.pop(0) for _ in range(n)], dtype=np.int64)
    in_map = np.stack([np.arange(n), new_ids], axis=1)
    pkv.swap_blocks(host_k, kc, in_map)
    pkv.swap_blocks(host_v, vc, in_map)
    remap = dict(zip(chosen.tolist(), new_ids.tolist()))
    tables2 = np.vectorize(lambda t: remap.get(int(t), int(t)))(tables).astype(np.int32)
    out2 = _decode(q, kc, vc, tables2, lens, bc.scale)
    sh2 = _decode_shared(q, kc, vc, tables2, lens, bc.scale, bc.beams, bc.prompt_len)
    torch.cuda.synchronize()
    log(f"beam: swapped {n} blocks out and back")
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(sh1.view(torch.int16), sh2.view(torch.int16))


def test_beam_small_all_outputs():
    _beam_run(num_prompts=4)


def test_beam_full_size_all_outputs():
    """32 prompts x 4 beams at full size: every (sequence, head) output against the oracle."""
    _beam_run(num_prompts=32)


@pytest.mark.parametrize("num_prompts,P", [(8, 0), (32, 512)])
def test_beam_step_with_fused_plan_and_cache(num_prompts, P):
    """The beam step as bench.py runs it: copy-on-write, then the new tokens' cache write and the
    shared-prefix plan in one launch, the planned kernel and the reduce.  Caches and output
    bit-identical to copy_blocks + reshape_and_cache + the one-call shared-prefix decode."""
    bc = make_beam_case(num_prompts=num_prompts)
    B = bc.query.shape[0]
    tables, lens, pairs, mapping, slots, nk, nv, _ = _cow_step(bc)
    q = bc.query.to(DEV)
    bt, cl = torch.from_numpy(tables).to(DEV), torch.from_numpy(lens).to(DEV)
    gs = torch.arange(0, B + 1, bc.beams, dtype=torch.int32, device=DEV)
    pl = torch.full((B // bc.beams,), bc.prompt_len, dtype=torch.int32, device=DEV)
    mp, sl = torch.from_numpy(mapping).to(DEV), torch.from_numpy(slots).to(DEV)
    nkd, nvd = nk.to(DEV), nv.to(DEV)
    L = int(lens.max())
    log(f"beam fused step: {num_prompts} prompts, {len(pairs)} copy-on-write pairs, P={P}")
    kc1, vc1 = bc.key_cache.to(DEV), bc.value_cache.to(DEV)
    pkv.copy_blocks([kc1], [vc1], mp)
    pkv.reshape_and_cache(nkd, nvd, kc1, vc1, sl)
    ref = torch.full_like(q, float("nan"))
    pkv.paged_attention_decode_shared(ref, q, kc1, vc1, bt, cl, gs, pl, bc.scale, L, P)
    kc2, vc2 = bc.key_cache.to(DEV), bc.value_cache.to(DEV)
    pkv.copy_blocks([kc2], [vc2], mp)
    out = torch.full_like(q, float("nan"))
    ws = pkv.paged_attention_plan_and_cache_shared(out, q, kc2, vc2, bt, cl, gs, pl, bc.scale, L,
                                                   nkd, nvd, sl, P)
    pkv.paged_attention_partitions_planned_shared(out, q, kc2, vc2, bt, cl, gs, pl, bc.scale, L,
                                                  P, ws)
    pkv.paged_attention_reduce(out, cl, L, ws, P)
    torch.cuda.synchronize()
    assert torch.equal(kc1.view(torch.int16), kc2.view(torch.int16))
    assert torch.equal(vc1.view(torch.int16), vc2.view(torch.int16))
    assert torch.equal(ref.view(torch.int16), out.view(torch.int16))
