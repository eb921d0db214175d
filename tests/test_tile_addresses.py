"""Every key and value load of the decode kernels stays inside the block pool or the
workspace's prefetch pad.  CPU only: the kernels' own address functions (pkv_tile_addr.h) run
on the host over the work items of the test workloads and of the full-size GQA and long-context
workloads, with table entries past each sequence's blocks set to -1 (not block ids: a lane that
used one would read below the pool).

The block table and the block layout are those of the pages: token t of a sequence is in
block_tables[b][t / block_size] (the mlqm.cn explainer, "PagedAttention"), and a (block, KV
head) tile is [D/x][bs][x] keys and [D][bs] values (the "Vllm" page, "CacheEngine").  A planted
pick without the guard for lanes past an item's last block must fail the check: that mistake
once faulted the GPU.
"""
import numpy as np
import pytest

import tilecheck as TC
from workloads import decode_layout


def _check(kernel, lay, P=0):
    cfg = lay.cfg
    lens = lay.lens.astype(np.int32)
    Lmax = int(lens.max())
    P = TC.partition(kernel == "8", cfg.block_size, Lmax, P)
    len_limit = min(Lmax, lay.tables.shape[1] * cfg.block_size)
    items, _ = TC.plan(lens, cfg.block_size, P, len_limit)
    n, msg = TC.bad_loads(kernel, lay.tables, lay.num_blocks, cfg.num_kv_heads, cfg.head_size,
                          cfg.block_size, P, items)
    assert n == 0, msg
    return items, P


# the workloads of the decode parity tests (16-bit kernel: fp16 / bf16 caches)
LAYOUTS_16 = [
    ("c1", dict(dtype="bf16"), 0), ("c2", dict(num_seqs=6), 0), ("c3", dict(num_seqs=16), 0),
    ("c4", dict(num_seqs=2, len_cap=20000, pool=("fixed", 0)), 0),
    ("c4", dict(num_seqs=2, len_cap=20000, pool=("fixed", 0)), 512),
] + [("c3", dict(num_seqs=6, len_cap=5000), P) for P in (16, 48, 80, 256, 512, 1024, 2048)] + [
    ("c3", dict(num_seqs=5, len_cap=1800, head_size=D, block_size=bs, num_heads=h, num_kv_heads=k), 0)
    for D, bs, (h, k) in [(64, 8, (8, 4)), (128, 32, (6, 6)), (64, 16, (16, 2)), (128, 32, (16, 2)),
                          (64, 16, (16, 1)), (128, 8, (12, 4)), (128, 16, (40, 8))]
]

EDGE_LENS = [0, 1, 15, 16, 17, 511, 512, 513, 1024, 1025, 33, 2047, 2048, 2049, 2560, 2561, 4095]


@pytest.mark.parametrize("key,over,P", LAYOUTS_16)
def test_16bit_kernel_loads_stay_in_bounds(key, over, P):
    _check("16", decode_layout(key, **over), P)


@pytest.mark.parametrize("bs", [8, 16, 32])
@pytest.mark.parametrize("P", [0, 8 * 32, 1024])
def test_16bit_kernel_edge_lengths(bs, P):
    lay = decode_layout("c3", lens=[L for L in EDGE_LENS], block_size=bs, num_heads=8, num_kv_heads=2)
    _check("16", lay, P)


@pytest.mark.parametrize("bs", [8, 16, 32])
@pytest.mark.parametrize("P", [0, 256, 2048, 4096])
def test_8bit_kernel_loads_stay_in_bounds(bs, P):
    """Edge lengths (every tile position relative to block and item ends) and lengths just past
    32-token tiles at each block size and partition size."""
    if P > 256 * bs:
        pytest.skip("an 8-bit item spans at most 256 blocks")
    lens = EDGE_LENS + [31, 33, 63, 65, 40, 72, 4097, 9000]
    lay = decode_layout("c3", lens=lens, block_size=bs, num_heads=8, num_kv_heads=2)
    _check("8", lay, P)


@pytest.mark.parametrize("key,P", [("c3", 0), ("c4", 0), ("c4", 512), ("c2", 0)])
def test_full_size_loads_stay_in_bounds(key, P):
    """Full-size workloads in the launch configuration the benchmark times (auto partitions),
    for both kernels (the 8-bit cache has the same tables)."""
    lay = decode_layout(key)
    items, P16 = _check("16", lay, P)
    assert len(items) > 0
    _check("8", lay, P)


def test_planted_unguarded_pick_fails():
    """The check has the power to catch the mistake it guards: without the guard, lanes past an
    item's last block take table entries that are not block ids."""
    lay = decode_layout("c3", lens=[40, 33, 65, 72, 200], block_size=8, num_heads=8, num_kv_heads=2)
    lens = lay.lens.astype(np.int32)
    for kernel, bs in (("16", 8), ("8", 8)):
        P = TC.partition(kernel == "8", bs, int(lens.max()))
        items, _ = TC.plan(lens, bs, P, int(lens.max()))
        good, _ = TC.bad_loads(kernel, lay.tables, lay.num_blocks, 2, 128, bs, P, items)
        bad, msg = TC.bad_loads(kernel, lay.tables, lay.num_blocks, 2, 128, bs, P, items, planted=True)
        assert good == 0 and bad > 0, (kernel, good, bad)
        assert "out of the pool" in msg, msg
    lay16 = decode_layout("c3", lens=[40, 33, 72], block_size=16, num_heads=8, num_kv_heads=2)
    items, _ = TC.plan(lay16.lens.astype(np.int32), 16, 2048, 72)
    bad, msg = TC.bad_loads("8", lay16.tables, lay16.num_blocks, 2, 128, 16, 2048, items, planted=True)
    assert bad > 0, "an 8-bit tile at block size 16 reaches past a 40-token item's blocks"


def test_host_plan_cuts():
    """The planner's cut rule on hand-worked lengths: P = 64, Q = 32 at block size 16: whole
    partitions, then chunks of at most 32 tokens; an empty sequence gets one empty item."""
    items, np_of = TC.plan([150, 0, 64, 20], 16, 64, 4096)
    got = sorted(tuple(int(v) for v in it) for it in items)
    want = sorted([(0, 1 | 0 << 8, 0, 64), (0, 1 | 1 << 8, 64, 128), (0, 1 | 2 << 8, 128, 150),
                   (1, 1, 0, 0), (2, 1, 0, 64), (3, 1, 0, 20)])
    assert got == want
    assert np_of.tolist() == [3, 1, 1, 1]
    # shared prefix: a group of three with a 100-token prefix (96 after rounding), one item per
    # pair of members (per_item 2), then each member's own tokens after the prefix
    items, np_of = TC.plan([130, 96, 100], 16, 64, 4096, group_starts=[0, 3], prefix_lens=[100],
                           per_item=2)
    got = sorted(tuple(int(v) for v in it) for it in items)
    want = sorted([(0, 2 | 0 << 8, 0, 64), (0, 2 | 1 << 8, 64, 96), (2, 1 | 0 << 8, 0, 64),
                   (2, 1 | 1 << 8, 64, 96), (0, 1 | 2 << 8, 96, 128), (0, 1 | 3 << 8, 128, 130),
                   (2, 1 | 2 << 8, 96, 100)])
    assert got == want
    assert np_of.tolist() == [4, 2, 3]
