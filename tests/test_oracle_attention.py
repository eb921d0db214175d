"""Pins for the fp64 attention oracle (CPU only).

Each test ties the oracle to something other than itself: hand-enumerated
addresses from the pages' block-layout statement, a library SDPA on dense
inputs, closed forms and invariants of softmax attention.  A plausible slip
in the oracle (wrong chunk index, transposed cache dims, a wrong GQA head
map, a missing max-subtraction or normalisation, a wrong partition
combine) breaks at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention as OA
from workloads import storage_bits, DTYPES

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bits(t):
    return storage_bits(t)


# ---------------------------------------------------------------- widening

@pytest.mark.parametrize("dtype,bits,value", [
    ("bf16", 0x3F80, 1.0), ("bf16", 0xC000, -2.0), ("bf16", 0x4049, 3.140625),
    ("bf16", 0x0001, 2.0 ** -133), ("bf16", 0x8000, -0.0), ("bf16", 0x7F80, math.inf),
    ("f16", 0x3C00, 1.0), ("f16", 0x0001, 2.0 ** -24), ("f16", 0xC248, -3.140625),
    ("f16", 0x7BFF, 65504.0), ("f32", 0x3F800000, 1.0), ("f32", 0x00000001, 2.0 ** -149),
])
def test_widen_known_patterns(dtype, bits, value):
    npdt = np.uint32 if dtype == "f32" else np.uint16
    got = OA.widen(np.array([bits], dtype=npdt), dtype)[0]
    assert got == value and math.copysign(1, got) == math.copysign(1, value)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_widen_matches_torch_cast(dtype):
    g = torch.Generator().manual_seed(5)
    t = (torch.randn(4096, generator=g) * 100).to(DTYPES[dtype])
    assert np.array_equal(OA.widen(_bits(t), dtype), t.to(torch.float64).numpy())


# ---------------------------------------------------------------- layout

def test_layout_addresses_from_golden():
    """Hand-enumerated flat offsets inside one block (golden/layout_addresses.json)."""
    spec = json.load(open(os.path.join(GOLDEN, "layout_addresses.json")))
    c = spec["case"]
    H, D, x, bs = c["num_kv_heads"], c["head_size"], c["x"], c["block_size"]
    # one block whose elements hold their own flat offset (as fp32 bit patterns)
    kblk = np.arange(H * D * bs, dtype=np.float32).reshape(1, H, D // x, bs, x)
    vblk = np.arange(H * D * bs, dtype=np.float32).reshape(1, H, D, bs)
    K, V = OA.gather_kv(kblk.view(np.uint32), vblk.view(np.uint32), "f32", np.array([0]), bs, 0)
    for e in spec["entries"]:
        assert K[e["t"], e["d"]] == e["key_offset"]
        assert V[e["t"], e["d"]] == e["value_offset"]


def test_block_table_maps_token_ranges():
    """Tokens 1-16 sit in block A and 17-32 in block D (mlqm.cn explainer block-table example)."""
    bs, D, x = 16, 8, 4
    NB = 6
    A, Dblk = 1, 4
    kc = np.zeros((NB, 1, D // x, bs, x), dtype=np.float32)
    vc = np.zeros((NB, 1, D, bs), dtype=np.float32)
    # tag every slot with (block id * 100 + offset)
    for b in range(NB):
        for t in range(bs):
            kc[b, 0, :, t, :] = b * 100 + t
            vc[b, 0, :, t] = b * 100 + t
    K, V = OA.gather_kv(kc.view(np.uint32), vc.view(np.uint32), "f32", np.array([A, Dblk]), 32, 0)
    for tok1 in range(1, 33):          # 1-based token numbers as on the page
        blk = A if tok1 <= 16 else Dblk
        assert K[tok1 - 1, 0] == blk * 100 + (tok1 - 1) % 16
        assert V[tok1 - 1, 3] == blk * 100 + (tok1 - 1) % 16


# ---------------------------------------------------------------- helpers

def _scatter_dense(Kd, Vd, tables, lens, NB, bs, x, Hkv, dtype, poison=True):
    """Write dense per-sequence K/V [B][Hkv][L, D] into a paged cache, slot by slot.

    Written independently of the oracle's vectorised gather: one explicit loop
    over (sequence, head, token, dim)."""
    D = Kd[0].shape[-1]
    fill = float("nan") if poison else 0.0
    kc = torch.full((NB, Hkv, D // x, bs, x), fill, dtype=DTYPES[dtype])
    vc = torch.full((NB, Hkv, D, bs), fill, dtype=DTYPES[dtype])
    for b in range(len(lens)):
        for t in range(int(lens[b])):
            blk = int(tables[b][t // bs])
            off = t % bs
            for h in range(Hkv):
                for d in range(D):
                    kc[blk, h, d // x, off, d % x] = Kd[b][h, t, d]
                    vc[blk, h, d, off] = Vd[b][h, t, d]
    return kc, vc


def _random_paged(seed, B=3, Hq=4, Hkv=2, D=16, bs=4, dtype="f32", lens=None, pool_extra=5):
    rng = np.random.default_rng(seed)
    x = 16 // torch.tensor([], dtype=DTYPES[dtype]).element_size()
    if lens is None:
        lens = rng.integers(1, 23, size=B)
    nblk = [(int(L) + bs - 1) // bs for L in lens]
    NB = sum(nblk) + pool_extra
    perm = rng.permutation(NB)
    tables = np.full((B, max(nblk)), -1, dtype=np.int32)
    o = 0
    for b in range(B):
        tables[b, :nblk[b]] = perm[o:o + nblk[b]]
        o += nblk[b]
    Kd = [torch.from_numpy(rng.standard_normal((Hkv, int(L), D)).astype(np.float32)).to(DTYPES[dtype])
          for L in lens]
    Vd = [torch.from_numpy(rng.standard_normal((Hkv, int(L), D)).astype(np.float32)).to(DTYPES[dtype])
          for L in lens]
    q = torch.from_numpy(rng.standard_normal((B, Hq, D)).astype(np.float32)).to(DTYPES[dtype])
    kc, vc = _scatter_dense(Kd, Vd, tables, lens, NB, bs, x, Hkv, dtype)
    return dict(q=q, kc=kc, vc=vc, tables=tables, lens=np.asarray(lens, dtype=np.int32),
                Kd=Kd, Vd=Vd, dtype=dtype, scale=1.0 / math.sqrt(D))


def _oracle(c, **kw):
    return OA.paged_decode(_bits(c["q"]), _bits(c["kc"]), _bits(c["vc"]), c["dtype"], c["tables"],
                           c["lens"], c["scale"], **kw)


# ---------------------------------------------------------------- attention math

@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (4, 2), (8, 1)])
def test_dense_equivalence_vs_sdpa(dtype, Hq, Hkv):
    """Oracle over the paged cache == torch SDPA (float64) over the dense K/V it was scattered from."""
    c = _random_paged(11 + Hq + Hkv, Hq=Hq, Hkv=Hkv, dtype=dtype)
    out = _oracle(c)
    G = Hq // Hkv
    sc = float(np.float32(c["scale"]))
    for b in range(len(c["lens"])):
        q = c["q"][b].to(torch.float64)[:, None, :]                      # [Hq, 1, D]
        K = c["Kd"][b].to(torch.float64).repeat_interleave(G, dim=0)     # [Hq, L, D]
        V = c["Vd"][b].to(torch.float64).repeat_interleave(G, dim=0)
        ref = torch.nn.functional.scaled_dot_product_attention(q, K, V, scale=sc)[:, 0, :]
        assert np.max(np.abs(out[b] - ref.numpy())) <= 1e-12


def test_gqa_equals_mha_with_repeated_kv():
    """G query heads sharing KV head g == an MHA run whose heads g*G..g*G+G-1 all hold KV head g."""
    c = _random_paged(3, Hq=8, Hkv=2, dtype="bf16")
    G = 4
    Kd = [k.repeat_interleave(G, dim=0) for k in c["Kd"]]
    Vd = [v.repeat_interleave(G, dim=0) for v in c["Vd"]]
    NB = c["kc"].shape[0]
    kc, vc = _scatter_dense(Kd, Vd, c["tables"], c["lens"], NB, 4, 8, 8, "bf16")
    mha = dict(c, kc=kc, vc=vc)
    assert np.array_equal(_oracle(c), _oracle(mha))


def test_block_permutation_invariance():
    """Relabelling physical blocks (and remapping the tables) leaves the output bit-identical."""
    c = _random_paged(21, dtype="f16")
    NB = c["kc"].shape[0]
    pi = np.random.default_rng(99).permutation(NB)
    kc = torch.empty_like(c["kc"])
    vc = torch.empty_like(c["vc"])
    kc[torch.from_numpy(pi)] = c["kc"]
    vc[torch.from_numpy(pi)] = c["vc"]
    tables = np.where(c["tables"] >= 0, pi[np.maximum(c["tables"], 0)], -1).astype(np.int32)
    moved = dict(c, kc=kc, vc=vc, tables=tables)
    assert np.array_equal(_oracle(c), _oracle(moved))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_length_one_returns_v0(dtype):
    c = _random_paged(5, lens=[1, 1, 1], dtype=dtype)
    out = _oracle(c)
    G = 2
    for b in range(3):
        for h in range(4):
            assert np.array_equal(out[b, h], c["Vd"][b][h // G, 0].to(torch.float64).numpy())


def test_identical_keys_return_mean_of_v():
    c = _random_paged(6, lens=[7, 16, 21], dtype="f32")
    for b in range(3):
        c["Kd"][b][:] = c["Kd"][b][:, :1, :]
    NB = c["kc"].shape[0]
    c["kc"], c["vc"] = _scatter_dense(c["Kd"], c["Vd"], c["tables"], c["lens"], NB, 4, 4, 2, "f32")
    out = _oracle(c)
    for b in range(3):
        for h in range(4):
            mean = c["Vd"][b][h // 2].to(torch.float64).numpy().mean(axis=0)
            assert np.max(np.abs(out[b, h] - mean)) <= 1e-15


def test_convex_hull_and_finite_with_poisoned_slots():
    """Output lies inside [min_t V, max_t V] per dim; NaN tails / free blocks never leak in."""
    c = _random_paged(8, lens=[5, 13, 22], dtype="f16")
    out = _oracle(c)
    assert np.all(np.isfinite(out))
    for b in range(3):
        for h in range(4):
            V = c["Vd"][b][h // 2].to(torch.float64).numpy()
            assert np.all(out[b, h] >= V.min(axis=0) - 1e-15)
            assert np.all(out[b, h] <= V.max(axis=0) + 1e-15)


def test_key_shift_invariance():
    """Adding one vector c to every key shifts all logits by scale*q.c: softmax, hence output, is unchanged."""
    rng = np.random.default_rng(4)
    c = _random_paged(9, lens=[9, 17, 6], dtype="f32")
    # integer-valued keys and shift: every sum stays exact in fp32 storage
    for b in range(3):
        c["Kd"][b][:] = torch.from_numpy(rng.integers(-3, 4, size=c["Kd"][b].shape).astype(np.float32))
    NB = c["kc"].shape[0]
    c["kc"], c["vc"] = _scatter_dense(c["Kd"], c["Vd"], c["tables"], c["lens"], NB, 4, 4, 2, "f32")
    base = _oracle(c)
    shift = torch.from_numpy(rng.integers(-5, 6, size=16).astype(np.float32))
    Ks = [k + shift for k in c["Kd"]]
    kc, vc = _scatter_dense(Ks, c["Vd"], c["tables"], c["lens"], NB, 4, 4, 2, "f32")
    shifted = _oracle(dict(c, kc=kc, vc=vc))
    assert np.max(np.abs(base - shifted)) <= 1e-12


def test_empty_context_is_zero():
    c = _random_paged(10, lens=[3, 5, 2], dtype="f32")
    c["lens"] = np.array([3, 0, 2], dtype=np.int32)
    out = _oracle(c)
    assert np.all(out[1] == 0)
    assert np.all(np.isfinite(out))


def test_sampled_pairs_match_full():
    c = _random_paged(12, dtype="bf16")
    full = _oracle(c)
    part = _oracle(c, pairs=[(0, 1), (2, 3)])
    assert np.array_equal(part[0, 1], full[0, 1]) and np.array_equal(part[2, 3], full[2, 3])
    assert np.isnan(part[1, 0]).all()


# ---------------------------------------------------------------- split-K algebra

@pytest.mark.parametrize("P", [4, 8, 16, 512])
def test_partitioned_equals_monolithic(P):
    c = _random_paged(13, B=4, lens=[1, 4, 17, 61], dtype="bf16")
    mono = _oracle(c)
    part = OA.partitioned_decode(_bits(c["q"]), _bits(c["kc"]), _bits(c["vc"]), "bf16", c["tables"],
                                 c["lens"], c["scale"], P)
    assert np.max(np.abs(mono - part)) <= 1e-12


def test_combine_is_not_a_plain_average():
    """The log-sum-exp combine weights partitions by e^(m_p - M) l_p: two partitions with very
    different logit scales must not be averaged."""
    q = np.array([1.0, 0.0])
    K = np.array([[10.0, 0.0], [10.0, 0.0], [0.0, 0.0], [0.0, 0.0]])
    V = np.array([[1.0, 0.0], [1.0, 0.0], [0.0, 1.0], [0.0, 1.0]])
    st = [OA.partition_stats(q, K, V, 1.0, 0, 2), OA.partition_stats(q, K, V, 1.0, 2, 4)]
    ref = OA.dense_decode(q, K, V, 1.0)
    assert np.max(np.abs(OA.combine_partitions(st) - ref)) <= 1e-15
    w = 1.0 / (1.0 + math.exp(-10.0))
    assert abs(ref[0] - w) <= 1e-15


# ---------------------------------------------------------------- shared-prefix decode

def _random_shared(seed, sizes=(3, 1, 2), prefixes=(8, 0, 12), Hq=4, Hkv=2, D=16, bs=4,
                   dtype="bf16", max_priv=9):
    """Groups of sequences whose first `prefix` tokens are the same dense K/V in the same
    physical blocks (one table prefix per group), followed by private tokens."""
    rng = np.random.default_rng(seed)
    x = 16 // torch.tensor([], dtype=DTYPES[dtype]).element_size()
    lens, pre_of = [], []
    for n, pre in zip(sizes, prefixes):
        for _ in range(n):
            lens.append(pre + int(rng.integers(0, max_priv + 1)))
            pre_of.append(pre)
    B = len(lens)
    nblk = [(L + bs - 1) // bs for L in lens]
    NB = sum(nblk) + 4
    perm = list(rng.permutation(NB))
    tables = np.full((B, max(nblk)), -1, dtype=np.int32)
    Kd, Vd, b = [], [], 0
    for n, pre in zip(sizes, prefixes):
        assert pre % bs == 0
        shared_ids = [perm.pop() for _ in range(pre // bs)]
        Kp = rng.standard_normal((Hkv, pre, D)).astype(np.float32)
        Vp = rng.standard_normal((Hkv, pre, D)).astype(np.float32)
        for _ in range(n):
            L = lens[b]
            own = [perm.pop() for _ in range(nblk[b] - pre // bs)]
            tables[b, :nblk[b]] = shared_ids + own
            Ko = rng.standard_normal((Hkv, L - pre, D)).astype(np.float32)
            Vo = rng.standard_normal((Hkv, L - pre, D)).astype(np.float32)
            Kd.append(torch.from_numpy(np.concatenate([Kp, Ko], axis=1)).to(DTYPES[dtype]))
            Vd.append(torch.from_numpy(np.concatenate([Vp, Vo], axis=1)).to(DTYPES[dtype]))
            b += 1
    q = torch.from_numpy(rng.standard_normal((B, Hq, D)).astype(np.float32)).to(DTYPES[dtype])
    kc, vc = _scatter_dense(Kd, Vd, tables, lens, NB, bs, x, Hkv, dtype)
    starts = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    return dict(q=q, kc=kc, vc=vc, tables=tables, lens=np.asarray(lens, dtype=np.int32),
                dtype=dtype, scale=1.0 / math.sqrt(D), starts=starts,
                prefixes=np.asarray(prefixes, dtype=np.int32))


def _shared(c, prefixes=None, starts=None):
    return OA.shared_prefix_decode(_bits(c["q"]), _bits(c["kc"]), _bits(c["vc"]), c["dtype"],
                                   c["tables"], c["lens"], c["scale"],
                                   c["starts"] if starts is None else starts,
                                   c["prefixes"] if prefixes is None else prefixes)


def test_shared_prefix_length_rule():
    lens = np.array([10, 7, 30, 5], dtype=np.int32)
    assert OA.shared_prefix_length(lens, 0, 2, 9, 4) == 4     # min(9, 10, 7) = 7 -> whole blocks: 4
    assert OA.shared_prefix_length(lens, 0, 2, 100, 1) == 7   # capped by the shortest member
    assert OA.shared_prefix_length(lens, 2, 3, 16, 4) == 0    # a group of one shares nothing
    assert OA.shared_prefix_length(lens, 0, 4, -3, 4) == 0
    assert OA.shared_prefix_length(lens, 2, 4, 8, 4) == 4     # capped by L = 5, rounded down


def test_shared_prefix_decode_is_the_plain_decode():
    """Inside the contract the grouped call has the plain decode's result (prefix lengths that
    end inside a block are cut back to whole blocks and still qualify)."""
    c = _random_shared(21)
    mono = _oracle(c)
    assert np.array_equal(_shared(c), mono)
    assert np.array_equal(_shared(c, np.array([10, 3, 15], dtype=np.int32)), mono)


def test_shared_prefix_contract_refuses_diverging_tables():
    """A member whose table points elsewhere below the rounded prefix breaks the contract: the
    oracle refuses it (what the kernel does with such input is unspecified)."""
    c = _random_shared(23, sizes=(2,), prefixes=(8,), max_priv=6)
    bs = c["kc"].shape[3]
    assert 2 * bs == 8
    # member 1's second prefix block moved to a fresh copy holding other keys
    alt = c["tables"].copy()
    NB = c["kc"].shape[0]
    c2 = dict(c, kc=torch.cat([c["kc"], -c["kc"][alt[1, 1:2]]]),
              vc=torch.cat([c["vc"], c["vc"][alt[1, 1:2]]]), tables=alt)
    alt[1, 1] = NB
    with pytest.raises(ValueError, match="does not share"):
        _shared(c2)
    # a divergence at or past the rounded prefix is allowed: with prefix 7 only block 0 is
    # shared (7 rounds down to 4 tokens), so member 1 may own block 1
    got = _shared(c2, np.array([7], dtype=np.int32))
    assert np.all(np.isfinite(got)) and np.array_equal(got, _oracle(c2))


@pytest.mark.parametrize("starts", [[0, 1], [1, 2], [0, 2, 1, 2], [0, 3]])
def test_shared_prefix_contract_refuses_bad_groups(starts):
    """Groups must cover the sequences once, in order."""
    c = _random_shared(24, sizes=(2,), prefixes=(8,), max_priv=6)
    prefixes = np.zeros(len(starts) - 1, dtype=np.int32)
    with pytest.raises(ValueError, match="group_starts"):
        _shared(c, prefixes, np.asarray(starts, dtype=np.int32))


def test_shared_prefix_contract_allows_empty_groups_and_singletons():
    c = _random_shared(25, sizes=(1, 2, 1), prefixes=(0, 8, 4), max_priv=6)
    starts = np.array([0, 1, 1, 3, 4], dtype=np.int32)   # an empty group between 0 and 1
    prefixes = np.array([0, 64, 8, 4], dtype=np.int32)
    assert np.array_equal(_shared(c, prefixes, starts), _oracle(c))
