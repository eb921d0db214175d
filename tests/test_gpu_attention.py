"""GPU parity of paged decode attention (reshape_and_cache of the step's new tokens, then
decode) against the fp64 oracle, through the C ABI.

Sizes: every workload at a size the oracle covers in a few seconds (several partitions, a
ragged last block), and every workload at its full size with every (sequence, head) output
compared, in the launch configuration the benchmark times (auto partition size).
"""
import dataclasses

import numpy as np
import pytest
import torch

import paged_kv_cache_164_amd as pkv
from gpu_cases import (DEV, GpuDecode, log, oracle_after_write, oracle_decode,
                       within_tolerance)
import tilecheck as TC
from workloads import DTYPES, decode_layout, make_decode_case

pytestmark = pytest.mark.gpu


def _run_and_check(case, P=0, pairs=None, tag=""):
    log(f"[{tag}] B={case.num_seqs} Hq={case.query.shape[1]} Hkv={case.key_cache.shape[1]} "
        f"D={case.query.shape[2]} bs={case.key_cache.shape[3]} {case.cfg.dtype} P={P} "
        f"Lmax={case.max_context_len}")
    g = GpuDecode(case, P)
    out = g.step()
    torch.cuda.synchronize()
    got = out.cpu().to(torch.float64).numpy()
    kb, vb = oracle_after_write(case)
    ref = oracle_decode(case, kb, vb, pairs)
    if pairs is not None:
        idx = tuple(np.array(pairs).T)
        got, ref = got[idx], ref[idx]
    ok, err, ratio = within_tolerance(got, ref, case.cfg.dtype)
    log(f"[{tag}] max|err|={err:.3e} worst err/bound={ratio:.3f}")
    assert ok, f"{tag}: max|err| {err} exceeds tolerance (ratio {ratio})"
    return g, got


# ---------------------------------------------------------------- oracle-sized, every output

@pytest.mark.parametrize("P", [0, 16, 64])
def test_c1_tiny_fp32(P):
    _run_and_check(make_decode_case("c1"), P, tag=f"c1 P={P}")


def test_c2_mha_fp16_small():
    _run_and_check(make_decode_case("c2", num_seqs=6), tag="c2 small")


def test_c3_gqa_bf16_small():
    _run_and_check(make_decode_case("c3", num_seqs=16), tag="c3 small")


@pytest.mark.parametrize("P", [0, 512])
def test_c4_long_splitk_bf16_small(P):
    """Long contexts, 1% outlier keys; 512-token partitions as the workload states, and auto."""
    case = make_decode_case("c4", num_seqs=2, len_cap=20000, pool=("fixed", 0))
    _run_and_check(case, P, tag=f"c4 small P={P}")


@pytest.mark.parametrize("P", [16, 48, 80, 256, 512, 1024, 2048])
def test_partition_sizes(P):
    """Whole partitions of P tokens and remainder chunks of at most ceil(P / 2) rounded up to
    whole blocks (48 -> chunks of 32, 80 -> chunks of 48: two per remainder)."""
    _run_and_check(make_decode_case("c3", num_seqs=6, len_cap=5000), P, tag=f"c3 P={P}")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("heads", [(4, 4), (8, 2), (8, 1)])
def test_edge_lengths(dtype, heads):
    """Empty context, one token, a block, a remainder chunk or a partition exactly full, one
    past it (auto partition: 2048 tokens in chunks of 512 on the matrix cores, 1024 in chunks
    of 256 for fp32)."""
    lens = [0, 1, 15, 16, 17, 511, 512, 513, 1024, 1025, 33, 2047, 2048, 2049, 2560, 2561, 4095]
    case = make_decode_case("c3", lens=lens, dtype=dtype, num_heads=heads[0], num_kv_heads=heads[1])
    g, got = _run_and_check(case, tag=f"edges {dtype} {heads}")
    assert np.all(got[0] == 0.0)   # empty context -> zero output


@pytest.mark.parametrize("dtype,D,bs,heads", [
    ("bf16", 64, 8, (8, 4)), ("f16", 128, 32, (6, 6)), ("f32", 128, 8, (4, 2)),
    ("f16", 64, 16, (16, 2)), ("bf16", 128, 32, (16, 2)), ("f32", 64, 32, (8, 8)),
    ("f16", 64, 16, (16, 1)), ("bf16", 128, 8, (12, 4)), ("f16", 128, 16, (40, 8)),
])
def test_shape_variants(dtype, D, bs, heads):
    case = make_decode_case("c3", num_seqs=5, len_cap=1800, dtype=dtype, head_size=D,
                            block_size=bs, num_heads=heads[0], num_kv_heads=heads[1])
    _run_and_check(case, tag=f"variant {dtype} D{D} bs{bs} {heads}")


# ---------------------------------------------------------------- full size, every output

# One full-size case and its oracle output at a time: c4's two partition sizes share them.
# The oracle's cache write lands in the CPU case tensors; a second GPU step on the same case
# writes the same new tokens to the same slots again, so it sees the same cache.
_FULL = {}


def _full_case_and_oracle(key):
    if key not in _FULL:
        _FULL.clear()
        case = make_decode_case(key)
        log(f"[{key} full] oracle over all {case.num_seqs} x {case.query.shape[1]} outputs")
        kb, vb = oracle_after_write(case)
        _FULL[key] = (case, oracle_decode(case, kb, vb))
    return _FULL[key]


@pytest.mark.parametrize("key,P", [("c2", 0), ("c3", 0), ("c4", 0), ("c4", 512)])
def test_full_size_all_outputs(key, P):
    """Each workload at its full size, every (sequence, head) output against the oracle, in the
    launch configuration the benchmark times (auto partitions) and, for the long-context
    workload, the 512-token partitions it states."""
    case, ref = _full_case_and_oracle(key)
    log(f"[{key} full P={P}] B={case.num_seqs} Lmax={case.max_context_len}")
    out = GpuDecode(case, P).step()
    torch.cuda.synchronize()
    got = out.cpu().to(torch.float64).numpy()
    ok, err, ratio = within_tolerance(got, ref, case.cfg.dtype)
    log(f"[{key} full P={P}] max|err|={err:.3e} worst err/bound={ratio:.3f} over {got.size} elements")
    assert ok, f"{key} full P={P}: max|err| {err} exceeds tolerance (ratio {ratio})"
    if key == "c4" and P == 512:
        _FULL.clear()


# ---------------------------------------------------------------- properties on the GPU

def test_run_to_run_bit_determinism():
    g = GpuDecode(make_decode_case("c3", num_seqs=32), 0)
    a = g.step().clone()
    b = g.decode(torch.empty_like(g.out)).clone()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_block_permutation_bit_equal():
    """Relabel every physical block on the GPU and remap the tables: bit-identical output."""
    case = make_decode_case("c2", num_seqs=8)
    g = GpuDecode(case, 0)
    base = g.step().clone()
    NB = g.kc.shape[0]
    perm = torch.from_numpy(np.random.default_rng(5).permutation(NB)).to(DEV)
    kc2, vc2 = torch.empty_like(g.kc), torch.empty_like(g.vc)
    kc2[perm] = g.kc
    vc2[perm] = g.vc
    bt = g.bt.long()
    bt2 = torch.where(bt >= 0, perm[bt.clamp(min=0)], bt).to(torch.int32)
    out2 = torch.empty_like(base)
    pkv.paged_attention_decode(out2, g.q, kc2, vc2, bt2.contiguous(), g.cl, case.scale,
                               case.max_context_len, 0, g.ws)
    torch.cuda.synchronize()
    assert torch.equal(base.view(torch.int16), out2.view(torch.int16))


def test_two_phase_entry_points_equal_fused_call():
    case = make_decode_case("c3", num_seqs=24)
    g = GpuDecode(case, 0)
    fused = g.step().clone()
    out2 = torch.empty_like(fused)
    ws = pkv.paged_attention_partitions(out2, g.q, g.kc, g.vc, g.bt, g.cl, case.scale,
                                        case.max_context_len, 0, g.ws)
    pkv.paged_attention_reduce(out2, g.cl, case.max_context_len, ws, 0)
    torch.cuda.synchronize()
    assert torch.equal(fused.view(torch.int16), out2.view(torch.int16))


@pytest.mark.parametrize("key,dtype", [("c3", None), ("c2", None), ("c1", None), ("c3", "f32")])
def test_plan_reused_across_layers(key, dtype):
    """One plan serves several layers: per layer a different query and cache, the same block
    tables and lengths.  Planned attention + reduce must equal the one-call decode of each layer
    bit for bit."""
    over = {} if dtype is None else {"dtype": dtype}
    c0 = make_decode_case(key, num_seqs=4 if key == "c1" else 24, len_cap=3000, **over)
    # layers: the same tables and lengths, other queries and cache contents (rolled and
    # rescaled copies of the first layer's; NaN poison stays NaN)
    cases = [c0] + [dataclasses.replace(
        c0, query=torch.roll(c0.query, layer, dims=1) * (1.0 + 0.5 * layer),
        key_cache=c0.key_cache * (1.0 - 0.25 * layer), value_cache=c0.value_cache + layer,
        new_key=c0.new_key * 0.5, new_value=c0.new_value - layer) for layer in (1, 2)]
    gs = [GpuDecode(c, 0) for c in cases]
    base = [g.step().clone() for g in gs]   # also writes each layer's new token
    g0 = gs[0]
    ws = torch.zeros_like(g0.ws)
    pkv.paged_attention_plan(torch.empty_like(base[0]), g0.q, g0.kc, g0.vc, g0.bt, g0.cl,
                             c0.scale, c0.max_context_len, 0, ws)
    for layer, (c, g) in enumerate(zip(cases, gs)):
        out = torch.full_like(base[layer], float("nan"))
        pkv.paged_attention_partitions_planned(out, g.q, g.kc, g.vc, g0.bt, g0.cl, c.scale,
                                               c.max_context_len, 0, ws)
        pkv.paged_attention_reduce(out, g0.cl, c.max_context_len, ws, 0)
        torch.cuda.synchronize()
        log(f"plan reuse {key} {dtype} layer {layer}")
        assert torch.equal(out.view(torch.int16 if out.element_size() == 2 else torch.int32),
                           base[layer].view(torch.int16 if out.element_size() == 2 else torch.int32))


def test_planned_call_on_an_unplanned_workspace_writes_nothing():
    case = make_decode_case("c3", num_seqs=8, len_cap=2000)
    g = GpuDecode(case, 0)
    ws = torch.zeros_like(g.ws)   # no plan since it was zeroed: an empty list
    out = torch.full_like(g.q, 7.0)
    pkv.paged_attention_partitions_planned(out, g.q, g.kc, g.vc, g.bt, g.cl, case.scale,
                                           case.max_context_len, 0, ws)
    pkv.paged_attention_reduce(out, g.cl, case.max_context_len, ws, 0)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())


def test_gqa_matches_mha_with_repeated_kv_on_gpu():
    """The GQA path on G heads per KV head == the MHA path on the KV heads repeated G times, bit
    for bit: both run the matrix-core kernel with the same cuts, and each MFMA column (query
    head) is computed the same way whichever other columns share its item."""
    case = make_decode_case("c3", num_seqs=6, len_cap=3000)
    g = GpuDecode(case, 0)
    gqa = g.step().clone().to(torch.float64)
    G = case.query.shape[1] // case.key_cache.shape[1]
    kc = g.kc.repeat_interleave(G, dim=1).contiguous()
    vc = g.vc.repeat_interleave(G, dim=1).contiguous()
    mha = torch.empty_like(g.out)
    pkv.paged_attention_decode(mha, g.q, kc, vc, g.bt, g.cl, case.scale, case.max_context_len, 0,
                               g.ws)
    torch.cuda.synchronize()
    diff = (gqa - mha.to(torch.float64)).abs().max().item()
    log(f"GQA vs repeated-KV MHA: max diff {diff:.3e}")
    assert torch.equal(gqa.to(torch.bfloat16).view(torch.int16), mha.view(torch.int16))


@pytest.mark.parametrize("key,over,P,groups", [
    ("c3", {}, 0, None), ("c4", {}, 512, None), ("c4", {}, 0, None), ("c2", {}, 0, None),
    ("c3", dict(num_seqs=6, len_cap=5000), 80, None),
    ("c3", dict(lens=[0, 1, 15, 16, 17, 2047, 2048, 2049, 4095], block_size=8), 0, None),
    ("c3", dict(lens=[300, 300, 290, 500, 40, 40, 2100, 2200, 2300, 0]), 256,
     ([0, 3, 4, 6, 9, 10], [288, 0, 32, 2048, 0])),
])
def test_device_plan_matches_host_planner(key, over, P, groups):
    """The plan kernel's work list equals, as a set, the host planner's that the address check
    (tests/test_tile_addresses.py) runs over; the per-sequence item counts agree too."""
    lay = decode_layout(key, **over)
    cfg = lay.cfg
    B, Hq, Hkv, D, bs = len(lay.lens), cfg.num_heads, cfg.num_kv_heads, cfg.head_size, cfg.block_size
    lens = lay.lens.astype(np.int32)
    Lmax = int(lens.max())
    dt = DTYPES[cfg.dtype]
    x = cfg.x
    q = torch.zeros((B, Hq, D), dtype=dt, device=DEV)
    kc = torch.zeros((1, Hkv, D // x, bs, x), dtype=dt, device=DEV)   # the plan reads no cache
    vc = torch.zeros((1, Hkv, D, bs), dtype=dt, device=DEV)
    bt = torch.from_numpy(lay.tables).to(DEV)
    cl = torch.from_numpy(lens).to(DEV)
    need = pkv.paged_attention_workspace_size(B, Hq, D, Lmax, P)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    log(f"plan {key} {over} P={P} groups={groups is not None}: B={B} Lmax={Lmax}")
    per_item = 1
    if groups is None:
        pkv.paged_attention_plan(torch.empty_like(q), q, kc, vc, bt, cl, 1.0, Lmax, P, ws)
        gs = pl = None
    else:
        gs, pl = groups
        per_item = 16 // (Hq // Hkv)
        pkv.paged_attention_plan_shared(torch.empty_like(q), q, kc, vc, bt, cl,
                                        torch.tensor(gs, dtype=torch.int32, device=DEV),
                                        torch.tensor(pl, dtype=torch.int32, device=DEV), 1.0, Lmax,
                                        P, ws)
    torch.cuda.synchronize()
    host = ws.cpu().numpy()
    n = int(host[4:8].view(np.uint32)[0])
    off = TC.items_offset(B, Hq, D, Lmax, P)
    dev_items = host[off:off + 16 * n].view(np.uint32).reshape(n, 4)
    coff = TC.counts_offset(B, Hq, D, Lmax, P)
    dev_counts = host[coff:coff + 4 * B].view(np.int32)
    P_eff = TC.partition(False, bs, Lmax, P)
    items, counts = TC.plan(lens, bs, P_eff, min(Lmax, lay.tables.shape[1] * bs), gs, pl, per_item)
    assert sorted(map(tuple, dev_items.tolist())) == sorted(map(tuple, items.tolist()))
    assert dev_counts.tolist() == counts.tolist()


@pytest.mark.parametrize("key,over,P", [
    ("c3", dict(num_seqs=64, len_cap=6000), 0), ("c1", {}, 0), ("c2", dict(num_seqs=12), 512),
    ("c3", dict(lens=[0, 1, 15, 16, 17, 2047, 2048, 2049, 4095], block_size=8), 0),
])
def test_plan_and_cache_equals_write_then_plan(key, over, P):
    """The fused launch (cache write + work-list plan) then the planned kernel and the reduce:
    caches and output bit-identical to reshape_and_cache followed by the one-call decode."""
    case = make_decode_case(key, **over)
    ref = GpuDecode(case, P)
    base = ref.step().clone()
    g = GpuDecode(case, P)
    out = torch.full_like(g.out, float("nan"))
    ws = pkv.paged_attention_plan_and_cache(out, g.q, g.kc, g.vc, g.bt, g.cl, case.scale,
                                            case.max_context_len, g.nk, g.nv, g.slots, P, g.ws)
    pkv.paged_attention_partitions_planned(out, g.q, g.kc, g.vc, g.bt, g.cl, case.scale,
                                           case.max_context_len, P, ws)
    pkv.paged_attention_reduce(out, g.cl, case.max_context_len, ws, P)
    torch.cuda.synchronize()
    iv = torch.int16 if out.element_size() == 2 else torch.int32
    assert torch.equal(ref.kc.view(iv), g.kc.view(iv)) and torch.equal(ref.vc.view(iv), g.vc.view(iv))
    assert torch.equal(base.view(iv), out.view(iv))
    kb, vb = oracle_after_write(case)
    ok, err, _ = within_tolerance(out.cpu().to(torch.float64).numpy(), oracle_decode(case, kb, vb),
                                  case.cfg.dtype)
    assert ok, err
