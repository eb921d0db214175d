"""Decode steps and multi-query calls captured in a HIP graph (torch.cuda.graph): every replay,
with eager work and synchronisations between replays, must give the eager result bit for bit.
The entry points record kernels only (no memset or copy nodes)."""
import numpy as np
import pytest
import torch

import paged_kv_cache_164_amd as pkv
from gpu_cases import DEV, log
from workloads import make_decode_case, make_prefill_case

pytestmark = pytest.mark.gpu


def _check_replays(step, out, n=3):
    """step() launches the work into `out`; returns after comparing n graph replays to eager."""
    step()
    torch.cuda.synchronize()
    ref = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on a side stream before capture, as torch advises
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(n):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {r} differs from the eager result"
        step()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out, ref)


def test_decode_step_graph_replays():
    case = make_decode_case("c3", num_seqs=48, len_cap=5000)
    log(f"graph decode: {case.num_seqs} sequences, max {case.max_context_len}")
    q, kc, vc = case.query.to(DEV), case.key_cache.to(DEV), case.value_cache.to(DEV)
    bt, cl = case.block_tables.to(DEV), case.context_lens.to(DEV)
    nk, nv, slots = case.new_key.to(DEV), case.new_value.to(DEV), case.slot_mapping.to(DEV)
    out = torch.empty_like(q)
    ws = torch.empty(pkv.paged_attention_workspace_size(case.num_seqs, 32, 128, case.max_context_len),
                     dtype=torch.uint8, device=DEV)

    def step():
        pkv.reshape_and_cache(nk, nv, kc, vc, slots)  # same slots, same values: idempotent
        pkv.paged_attention_decode(out, q, kc, vc, bt, cl, case.scale, case.max_context_len, 0, ws)

    _check_replays(step, out)


@pytest.mark.parametrize("P", [0, 64])
def test_multi_query_graph_replays(P):
    case = make_prefill_case([(300, 130), (0, 77), (1000, 1), (40, 200)], poison=False,
                             num_heads=16, num_kv_heads=4, head_size=128, block_size=16)
    log(f"graph multi-query: {case.num_tokens} rows, P={P}")
    kc, vc = case.key_cache.to(DEV), case.value_cache.to(DEV)
    pkv.reshape_and_cache(case.new_key.to(DEV), case.new_value.to(DEV), kc, vc,
                          torch.from_numpy(case.slot_mapping).to(DEV))
    q = case.query.to(DEV)
    bt = torch.from_numpy(case.block_tables).to(DEV)
    cl = torch.from_numpy(case.context_lens).to(DEV)
    qsl = torch.from_numpy(case.query_start_loc).to(DEV)
    out = torch.empty_like(q)
    B = len(case.context_lens)
    ws = torch.empty(max(pkv.paged_attention_prefill_workspace_size(
        B, case.num_tokens, 16, 4, 128, case.max_context_len, P), 256), dtype=torch.uint8, device=DEV)

    def step():
        pkv.paged_attention_prefill(out, q, kc, vc, bt, cl, qsl, case.scale, case.max_context_len,
                                    P, ws)

    _check_replays(step, out)


def test_planned_step_graph_replays():
    """Plan, cache write, attention on the plan and reduce, captured as one graph."""
    case = make_decode_case("c3", num_seqs=40, len_cap=6000)
    q, kc, vc = case.query.to(DEV), case.key_cache.to(DEV), case.value_cache.to(DEV)
    bt, cl = case.block_tables.to(DEV), case.context_lens.to(DEV)
    nk, nv, slots = case.new_key.to(DEV), case.new_value.to(DEV), case.slot_mapping.to(DEV)
    out = torch.empty_like(q)
    ws = torch.empty(pkv.paged_attention_workspace_size(case.num_seqs, 32, 128, case.max_context_len),
                     dtype=torch.uint8, device=DEV)
    log(f"graph planned decode: {case.num_seqs} sequences")

    def step():
        pkv.paged_attention_plan(out, q, kc, vc, bt, cl, case.scale, case.max_context_len, 0, ws)
        pkv.reshape_and_cache(nk, nv, kc, vc, slots)
        pkv.paged_attention_partitions_planned(out, q, kc, vc, bt, cl, case.scale,
                                               case.max_context_len, 0, ws)
        pkv.paged_attention_reduce(out, cl, case.max_context_len, ws, 0)

    _check_replays(step, out)


@pytest.mark.parametrize("code", ["e4m3", "i8"])
def test_8bit_decode_and_multi_query_graph_replays(code):
    from workloads import with_8bit_cache
    case = with_8bit_cache(make_decode_case("c3", num_seqs=24, len_cap=4000), code)
    q, kc, vc = case.query.to(DEV), case.key_cache.to(DEV), case.value_cache.to(DEV)
    bt, cl = case.block_tables.to(DEV), case.context_lens.to(DEV)
    nk, nv, slots = case.new_key.to(DEV), case.new_value.to(DEV), case.slot_mapping.to(DEV)
    out = torch.empty_like(q)
    ws = torch.empty(pkv.paged_attention_workspace_size(case.num_seqs, 32, 128, case.max_context_len),
                     dtype=torch.uint8, device=DEV)
    log(f"graph 8-bit decode {code}")

    def step():
        pkv.reshape_and_cache_fp8(nk, nv, kc, vc, slots, case.k_scale, case.v_scale, code=code)
        pkv.paged_attention_decode_fp8(out, q, kc, vc, bt, cl, case.scale, case.k_scale,
                                       case.v_scale, case.max_context_len, 0, ws, code=code)

    _check_replays(step, out)

    pcase = with_8bit_cache(make_prefill_case([(300, 130), (0, 77), (1000, 1)], poison=False,
                                              num_heads=16, num_kv_heads=4, head_size=128,
                                              block_size=16), code)
    pkc, pvc = pcase.key_cache.to(DEV), pcase.value_cache.to(DEV)
    pkv.reshape_and_cache_fp8(pcase.new_key.to(DEV), pcase.new_value.to(DEV), pkc, pvc,
                              torch.from_numpy(pcase.slot_mapping).to(DEV), pcase.k_scale,
                              pcase.v_scale, code=code)
    pq = pcase.query.to(DEV)
    pbt = torch.from_numpy(pcase.block_tables).to(DEV)
    pcl = torch.from_numpy(pcase.context_lens).to(DEV)
    pqsl = torch.from_numpy(pcase.query_start_loc).to(DEV)
    pout = torch.empty_like(pq)
    B = len(pcase.context_lens)
    pws = torch.empty(max(pkv.paged_attention_prefill_workspace_size(
        B, pcase.num_tokens, 16, 4, 128, pcase.max_context_len, 64), 256), dtype=torch.uint8,
        device=DEV)
    log(f"graph 8-bit multi-query {code}")

    def pstep():
        pkv.paged_attention_prefill(pout, pq, pkc, pvc, pbt, pcl, pqsl, pcase.scale,
                                    pcase.max_context_len, 64, pws, k_scale=pcase.k_scale,
                                    v_scale=pcase.v_scale, code=code)

    _check_replays(pstep, pout)


@pytest.mark.parametrize("kind", ["16-bit", "e4m3", "i8", "beam"])
def test_fused_plan_and_cache_steps_graph_replays(kind):
    """The steps bench.py times, captured as one graph: the fused plan + cache-write launch
    (16-bit, 8-bit, or shared-prefix after a beam step's copy-on-write), the planned kernel and
    the reduce.  Replays must equal the eager step bit for bit."""
    from workloads import make_beam_case, with_8bit_cache
    if kind == "beam":
        from test_gpu_beam import _cow_step
        bc = make_beam_case(num_prompts=8)
        B = bc.query.shape[0]
        tables, lens, pairs, mapping, slots, nk, nv, _ = _cow_step(bc)
        q, kc, vc = bc.query.to(DEV), bc.key_cache.to(DEV), bc.value_cache.to(DEV)
        bt, cl = torch.from_numpy(tables).to(DEV), torch.from_numpy(lens).to(DEV)
        gs = torch.arange(0, B + 1, bc.beams, dtype=torch.int32, device=DEV)
        pl = torch.full((B // bc.beams,), bc.prompt_len, dtype=torch.int32, device=DEV)
        mp, sl = torch.from_numpy(mapping).to(DEV), torch.from_numpy(slots).to(DEV)
        nkd, nvd = nk.to(DEV), nv.to(DEV)
        L, scale = int(lens.max()), bc.scale
        ptrs = pkv.copy_blocks([kc], [vc], mp)  # device pointer tables made outside the capture
        H, D = q.shape[1], q.shape[2]
        ws = torch.empty(pkv.paged_attention_workspace_size(B, H, D, L), dtype=torch.uint8,
                         device=DEV)
        log(f"graph fused beam step: {B} sequences, {len(pairs)} copy-on-write pairs")

        def step():
            pkv.copy_blocks([kc], [vc], mp, _ptr_buffers=ptrs)
            pkv.paged_attention_plan_and_cache_shared(out, q, kc, vc, bt, cl, gs, pl, scale, L,
                                                      nkd, nvd, sl, 0, ws)
            pkv.paged_attention_partitions_planned_shared(out, q, kc, vc, bt, cl, gs, pl, scale,
                                                          L, 0, ws)
            pkv.paged_attention_reduce(out, cl, L, ws, 0)
    else:
        case = make_decode_case("c3", num_seqs=40, len_cap=6000)
        if kind != "16-bit":
            case = with_8bit_cache(case, kind)
        q, kc, vc = case.query.to(DEV), case.key_cache.to(DEV), case.value_cache.to(DEV)
        bt, cl = case.block_tables.to(DEV), case.context_lens.to(DEV)
        nk, nv, sl = case.new_key.to(DEV), case.new_value.to(DEV), case.slot_mapping.to(DEV)
        L = case.max_context_len
        ws = torch.empty(pkv.paged_attention_workspace_size(case.num_seqs, 32, 128, L),
                         dtype=torch.uint8, device=DEV)
        log(f"graph fused {kind} step: {case.num_seqs} sequences")

        def step():
            if kind == "16-bit":
                pkv.paged_attention_plan_and_cache(out, q, kc, vc, bt, cl, case.scale, L, nk, nv,
                                                   sl, 0, ws)
                pkv.paged_attention_partitions_planned(out, q, kc, vc, bt, cl, case.scale, L, 0,
                                                       ws)
            else:
                pkv.paged_attention_plan_and_cache_fp8(out, q, kc, vc, bt, cl, case.scale,
                                                       case.k_scale, case.v_scale, L, nk, nv, sl,
                                                       0, ws, code=kind)
                pkv.paged_attention_partitions_planned_fp8(out, q, kc, vc, bt, cl, case.scale,
                                                           case.k_scale, case.v_scale, L, 0, ws,
                                                           code=kind)
            pkv.paged_attention_reduce(out, cl, L, ws, 0)
    out = torch.empty_like(q)
    _check_replays(step, out)
