"""GPU parity of the shared-prefix decode (pkv_paged_attention_decode_shared) through the C ABI.

Groups of sequences share the physical blocks of a prompt prefix; the kernel reads each shared
block once per group with the members' query rows as matrix columns.  Checked against the fp64
oracle on every output, and bit for bit against the plain decode where both take the same
partitions on the same kernel (group size >= 2, prefixes on partition boundaries).
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_164_amd as pkv
from gpu_cases import DEV, log, within_tolerance
from oracle import attention as OA
from workloads import make_prefix_case, storage_bits

pytestmark = pytest.mark.gpu


def _gpu_inputs(c):
    return (c.query.to(DEV), c.key_cache.to(DEV), c.value_cache.to(DEV),
            torch.from_numpy(c.block_tables).to(DEV), torch.from_numpy(c.context_lens).to(DEV))


def _shared(c, P, inputs=None, workspace=None):
    q, kc, vc, bt, cl = inputs or _gpu_inputs(c)
    out = torch.full_like(q, float("nan"))
    gs = torch.from_numpy(c.group_starts).to(DEV)
    pl = torch.from_numpy(c.prefix_lens).to(DEV)
    pkv.paged_attention_decode_shared(out, q, kc, vc, bt, cl, gs, pl, c.scale,
                                      int(c.context_lens.max()), P, workspace)
    return out


def _plain(c, P, inputs=None):
    q, kc, vc, bt, cl = inputs or _gpu_inputs(c)
    out = torch.full_like(q, float("nan"))
    pkv.paged_attention_decode(out, q, kc, vc, bt, cl, c.scale, int(c.context_lens.max()), P)
    return out


def _check_vs_oracle(c, got, tag):
    ref = OA.paged_decode(storage_bits(c.query), storage_bits(c.key_cache),
                          storage_bits(c.value_cache), c.cfg.dtype, c.block_tables,
                          c.context_lens, c.scale)
    got = got.cpu().to(torch.float64).numpy()
    ok, err, ratio = within_tolerance(got, ref, c.cfg.dtype)
    log(f"[{tag}] max|err|={err:.3e} worst err/bound={ratio:.3f}")
    assert ok, f"{tag}: max|err| {err} (ratio {ratio})"
    return got


# (dtype, head_size, block_size, Hq, Hkv, group sizes, prefix lengths, private range, P)
CASES = [
    ("f16", 128, 16, 8, 8, [4, 4, 1], [256, 100, 0], (0, 40), 0),        # MHA, 4 beams
    ("bf16", 128, 16, 8, 2, [5, 3, 2], [512, 48, 17], (1, 300), 256),    # G=4: 4 + 1 members
    ("bf16", 64, 8, 16, 1, [2, 2], [64, 40], (0, 20), 16),               # G=16: one per item
    ("f16", 64, 32, 4, 4, [17, 1], [96, 0], (0, 70), 64),                # 17 members: 16 + 1
    ("bf16", 128, 32, 16, 8, [3, 2], [1024, 2048], (0, 1500), 0),        # several partitions
    ("f16", 128, 8, 12, 4, [6], [1000], (0, 33), 512),                   # G=3, prefix in a partition
]


@pytest.mark.parametrize("dtype,D,bs,Hq,Hkv,sizes,prefixes,private,P", CASES)
def test_shared_prefix_vs_oracle(dtype, D, bs, Hq, Hkv, sizes, prefixes, private, P):
    tag = f"shared {dtype} D={D} bs={bs} {Hq}/{Hkv} groups={sizes} pre={prefixes} P={P}"
    log(tag)
    c = make_prefix_case(sizes, prefixes, private, num_heads=Hq, num_kv_heads=Hkv,
                         head_size=D, block_size=bs, dtype=dtype)
    out = _shared(c, P)
    torch.cuda.synchronize()
    _check_vs_oracle(c, out, tag)


def test_shared_prefix_edge_lengths():
    """Members whose whole context is the prefix (no own tokens), empty contexts, a group of
    empty contexts."""
    c = make_prefix_case([2, 1, 2, 3], [32, 0, 0, 48], (0, 0), num_heads=8, num_kv_heads=4,
                         head_size=64, block_size=16, dtype="bf16")
    assert list(c.context_lens) == [32, 32, 0, 0, 0, 48, 48, 48]
    for P in (16, 32, 0):
        log(f"shared edges P={P}")
        out = _shared(c, P)
        torch.cuda.synchronize()
        got = _check_vs_oracle(c, out, f"edges P={P}")
        assert np.all(got[2:5] == 0.0)


@pytest.mark.parametrize("dtype,Hq,Hkv", [("bf16", 32, 8), ("f16", 8, 8)])
def test_shared_prefix_bitwise_equals_plain_decode(dtype, Hq, Hkv):
    """Prefixes on partition boundaries (auto partition: 2048 tokens): both calls cut every
    sequence at the same tokens and run the same kernel; only the columns of an item come from
    several sequences, so the results agree bit for bit."""
    c = make_prefix_case([4, 4, 3, 1], [2048, 4096, 2048, 0], (1, 2600), num_heads=Hq,
                         num_kv_heads=Hkv, head_size=128, block_size=16, dtype=dtype)
    inputs = _gpu_inputs(c)
    for P in (0, 1024, 512):
        log(f"shared vs plain bitwise {dtype} {Hq}/{Hkv} P={P}")
        a = _shared(c, P, inputs)
        b = _plain(c, P, inputs)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_shared_prefix_repeatable_and_workspace_reuse():
    """Two calls with one workspace (stale items and counts from the first) give identical bits."""
    c = make_prefix_case([4, 2], [512, 160], (0, 700), num_heads=8, num_kv_heads=8,
                         head_size=128, block_size=16, dtype="f16")
    inputs = _gpu_inputs(c)
    need = pkv.paged_attention_workspace_size(len(c.context_lens), 8, 128,
                                                     int(c.context_lens.max()), 256)
    ws = torch.full((need,), 0xAB, dtype=torch.uint8, device=DEV)
    a = _shared(c, 256, inputs, ws)
    b = _shared(c, 256, inputs, ws)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    _check_vs_oracle(c, a, "workspace reuse")


def _planned_layers(c, P, layers):
    """One shared-prefix plan, then for each layer's (query, caches) the attention kernel on it
    and the reduce."""
    _, _, _, bt, cl = _gpu_inputs(c)
    gs = torch.from_numpy(c.group_starts).to(DEV)
    pl = torch.from_numpy(c.prefix_lens).to(DEV)
    L = int(c.context_lens.max())
    q0, kc0, vc0 = layers[0]
    need = pkv.paged_attention_workspace_size(len(c.context_lens), q0.shape[1], q0.shape[2], L, P)
    ws = torch.full((max(need, 256),), 0xCD, dtype=torch.uint8, device=DEV)
    pkv.paged_attention_plan_shared(torch.empty_like(q0), q0, kc0, vc0, bt, cl, gs, pl, c.scale,
                                    L, P, ws)
    outs = []
    for q, kc, vc in layers:
        out = torch.full_like(q, float("nan"))
        pkv.paged_attention_partitions_planned_shared(out, q, kc, vc, bt, cl, gs, pl, c.scale, L,
                                                      P, ws)
        pkv.paged_attention_reduce(out, cl, L, ws, P)
        outs.append(out)
    return outs


@pytest.mark.parametrize("dtype,D,bs,Hq,Hkv,sizes,prefixes,private,P",
                         [CASES[0], CASES[1], CASES[4], CASES[5]])
def test_shared_plan_reused_across_layers(dtype, D, bs, Hq, Hkv, sizes, prefixes, private, P):
    """One plan_shared, three layers (other queries and caches over the same tables, groups and
    lengths): each layer's planned kernel + reduce equals decode_shared bit for bit, and the first
    layer matches the oracle."""
    c = make_prefix_case(sizes, prefixes, private, num_heads=Hq, num_kv_heads=Hkv, head_size=D,
                         block_size=bs, dtype=dtype)
    q, kc, vc, bt, cl = _gpu_inputs(c)
    layers = [(q, kc, vc), (q.flip(-1).contiguous(), -kc, vc * 2), (q * 0.5, kc * 2, -vc)]
    log(f"shared plan reuse {dtype} D={D} bs={bs} {Hq}/{Hkv} P={P}")
    got = _planned_layers(c, P, layers)
    for i, (lq, lk, lv) in enumerate(layers):
        ref = _shared(c, P, (lq, lk, lv, bt, cl))
        torch.cuda.synchronize()
        assert torch.equal(got[i].view(torch.int16), ref.view(torch.int16)), f"layer {i}"
    _check_vs_oracle(c, got[0], "planned shared, layer 0")


def test_shared_planned_call_on_an_unplanned_workspace_writes_nothing():
    c = make_prefix_case([4, 2], [512, 160], (0, 700), num_heads=8, num_kv_heads=8,
                         head_size=128, block_size=16, dtype="f16")
    q, kc, vc, bt, cl = _gpu_inputs(c)
    gs = torch.from_numpy(c.group_starts).to(DEV)
    pl = torch.from_numpy(c.prefix_lens).to(DEV)
    L = int(c.context_lens.max())
    need = pkv.paged_attention_workspace_size(len(c.context_lens), 8, 128, L, 256)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=DEV)
    out = torch.full_like(q, float("nan"))
    pkv.paged_attention_partitions_planned_shared(out, q, kc, vc, bt, cl, gs, pl, c.scale, L, 256,
                                                  ws)
    pkv.paged_attention_reduce(out, cl, L, ws, 256)
    torch.cuda.synchronize()
    assert torch.isnan(out).all()
