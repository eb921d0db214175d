"""The C-ABI library loads, exports every entry point of include/pkv.h, and rejects bad
arguments on the host before touching the GPU (CPU only: no kernel is launched)."""
import ctypes
import glob
import os
import re

import pytest
import torch

import paged_kv_cache_164_amd as pkv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    if not os.path.exists(pkv.library_path()):
        pytest.fail("libpkv.so is not built (run python -m paged_kv_cache_164_amd.build)")
    return pkv.library()


def test_exports_every_header_symbol():
    lib = _lib()
    declared = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        declared |= set(re.findall(r"\b(pkv_\w+)\s*\(", open(h).read()))
    assert declared == set(pkv.EXPORTED_SYMBOLS)
    assert len(declared) == 47
    for name in declared:
        assert hasattr(lib, name), name


def test_every_header_symbol_has_a_ctypes_signature():
    """Each declared entry point has its argument types set before a call (a float or a 64-bit
    argument marshalled as a default int would be read wrongly)."""
    from paged_kv_cache_164_amd import _binding
    assert set(_binding._SIGNATURES) == set(pkv.EXPORTED_SYMBOLS)


def test_single_hip_runtime_shared_with_torch():
    _lib()
    paths = {line.split()[-1] for line in open("/proc/self/maps") if "libamdhip64" in line}
    assert len(paths) == 1, paths


def test_workspace_size():
    _lib()
    a256 = lambda v: (v + 255) // 256 * 256

    def expect(B, H, D, L, P):
        # header, prefetch pad, partial counts, then S items of 16 B and S partial slots
        # per (sequence, head) with S = ceil(L / P') + 4, P' = P or 1024 for auto
        S = -(-L // (P or 1024)) + 4
        n = B * H * S
        return 256 + 8192 + a256(4 * B) + a256(16 * B * S) + 2 * a256(4 * n) + a256(4 * n * D)

    for L, P in [(512, 512), (0, 0), (1025, 512), (2049, 0), (131072, 2048), (1, 16)]:
        assert pkv.paged_attention_workspace_size(4, 8, 64, L, P) == expect(4, 8, 64, L, P), (L, P)
    assert pkv.paged_attention_workspace_size(0, 8, 64, 100, 0) == 0
    assert pkv.paged_attention_workspace_size(4, 8, 64, 100, 8192) == 0   # partition too large
    assert pkv.paged_attention_workspace_size(4, 8, 64, 100, -1) == 0


def test_noalloc_refuses_oversized_calls_on_the_host():
    """The allocation-free decode checks its sizes against its static scratch before any HIP
    call: 256 sequences x 32 heads at 512-token partitions of a 10236-token context need more
    than 64 MiB."""
    lib = _lib()
    assert lib.pkv_paged_attention_noalloc_scratch_bytes() == 64 << 20
    rc = lib.pkv_paged_attention_decode_noalloc(1, 1, 1, 1, 1, 1, 0.125, 256, 32, 8, 128, 16, 640,
                                                10236, 2, 512, None)
    assert rc == -4 and b"scratch" in lib.pkv_last_error()
    # invalid sizes are reported as for the workspace call
    rc = lib.pkv_paged_attention_decode_noalloc(1, 1, 1, 1, 1, 1, 0.125, 2, 8, 3, 64, 16, 4, 64,
                                                1, 0, None)
    assert rc == -1


def _shared(lib, entry="pkv_paged_attention_decode_shared", **over):
    args = dict(out=1, query=1, key_cache=1, value_cache=1, block_tables=1, context_lens=1,
                group_starts=1, prefix_lens=1, num_groups=1, scale=0.125, num_seqs=2, num_heads=8,
                num_kv_heads=8, head_size=64, block_size=16, max_blocks=4, max_context_len=64,
                dtype=1, partition_size=0, workspace=None, ws_bytes=0, stream=None)
    args.update(over)
    return getattr(lib, entry)(*args.values())


@pytest.mark.parametrize("over,code", [
    (dict(dtype=0), -2),                          # fp32 has no matrix-core path
    (dict(num_heads=8 * 17, num_kv_heads=8), -2),  # group size above 16
    (dict(group_starts=None), -3),
    (dict(prefix_lens=None), -3),
    (dict(num_groups=0), -1),
    (dict(num_groups=3), -1),                    # more groups than sequences
    (dict(), -4),                                # needs a workspace
])
@pytest.mark.parametrize("entry", ["pkv_paged_attention_decode_shared",
                                   "pkv_paged_attention_plan_shared",
                                   "pkv_paged_attention_partitions_planned_shared"])
def test_shared_decode_argument_errors(entry, over, code):
    lib = _lib()
    assert _shared(lib, entry, **over) == code
    assert lib.pkv_last_error().decode() != ""


def _decode(lib, entry="pkv_paged_attention_decode", **over):
    args = dict(out=1, query=1, key_cache=1, value_cache=1, block_tables=1, context_lens=1,
                scale=0.125, num_seqs=2, num_heads=8, num_kv_heads=8, head_size=64, block_size=16,
                max_blocks=4, max_context_len=64, dtype=0, partition_size=0, workspace=None,
                ws_bytes=0, stream=None)
    args.update(over)
    return getattr(lib, entry)(*args.values())


@pytest.mark.parametrize("over,code", [
    (dict(head_size=96), -2),
    (dict(block_size=12), -2),
    (dict(num_heads=12), -1),            # not a multiple of num_kv_heads
    (dict(dtype=7), -1),
    (dict(partition_size=24), -1),       # not a multiple of block_size
    (dict(partition_size=8192), -1),     # above 4096
    (dict(dtype=1, block_size=8, partition_size=2048), -1),   # more than 128 blocks per item
    (dict(dtype=1, block_size=16, partition_size=4096), -1),  # more than 128 blocks per item
    (dict(scale=float("nan")), -1),
    (dict(query=None), -3),
    (dict(max_context_len=4096), -4),    # needs a workspace
    (dict(num_heads=24, num_kv_heads=8, dtype=0), -2),   # group 3 unsupported for fp32
])
@pytest.mark.parametrize("entry", ["pkv_paged_attention_decode", "pkv_paged_attention_plan",
                                   "pkv_paged_attention_partitions_planned",
                                   "pkv_paged_attention_partitions"])
def test_decode_argument_errors(entry, over, code):
    lib = _lib()
    assert _decode(lib, entry, **over) == code
    assert lib.pkv_last_error().decode() != ""


def test_cache_op_argument_errors():
    lib = _lib()
    # reshape: bad dtype, stride too small
    assert lib.pkv_reshape_and_cache(1, 1, 1, 1, 1, 4, 2, 64, 16, 10, 128, 128, 9, None) == -1
    assert lib.pkv_reshape_and_cache(1, 1, 1, 1, 1, 4, 2, 64, 16, 10, 100, 128, 1, None) == -1
    # copy: block bytes not a multiple of 16
    assert lib.pkv_copy_blocks(1, 1, 1, 1, 1, 40, 10, None) == -1
    # swap: bad direction; ids out of range are found before any copy is issued
    m = (ctypes.c_int64 * 2)(0, 5)
    assert lib.pkv_swap_blocks(1, 1, m, 1, 64, 4, 4, 3, None) == -1
    # zero-sized calls are no-ops
    assert lib.pkv_copy_blocks(None, None, 1, None, 0, 64, 10, None) == 0
    assert lib.pkv_reshape_and_cache(None, None, None, None, None, 0, 2, 64, 16, 10, 128, 128, 1, None) == 0


def test_binding_refuses_cpu_tensors():
    q = torch.zeros(1, 8, 64)
    with pytest.raises(pkv.PKVError):
        pkv.paged_attention_decode(q, q, torch.zeros(1, 8, 16, 16, 4), torch.zeros(1, 8, 64, 16),
                                   torch.zeros(1, 1, dtype=torch.int32),
                                   torch.zeros(1, dtype=torch.int32), 0.125, 16)


def test_decode_bytes_formula():
    # two sequences of 17 and 16 tokens, MHA 2 heads, D 8, bs 16, 2-byte elements
    b = pkv.decode_bytes([17, 16], 2, 2, 8, 16, 2)
    assert b == 33 * 2 * 8 * 2 * 2 + 2 * 2 * 2 * 8 * 2 + 4 * 3 + 4 * 2


def test_prefill_workspace_size():
    _lib()
    a256 = lambda v: (v + 255) // 256 * 256

    def expect(B, T, Hq, Hkv, D, L, P):
        # header, work items (tiles x pieces), per-row piece counts, then partials when split
        P = P or 8192
        qt = 256 // (Hq // Hkv)
        S = -(-L // P) if L > 0 else 1
        cap = (T // qt + B) * S
        base = 256 + a256(16 * cap) + a256(4 * T)
        if S <= 1:
            return base
        n = T * Hq * S
        return base + 2 * a256(4 * n) + a256(4 * n * D)

    for args in [(4, 100, 8, 2, 64, 300, 0), (16, 16384, 32, 8, 128, 8192, 0),
                 (3, 40, 16, 1, 128, 5000, 64), (1, 1, 4, 4, 64, 131072, 4096)]:
        assert pkv.paged_attention_prefill_workspace_size(*args) == expect(*args), args
    assert pkv.paged_attention_prefill_workspace_size(0, 10, 8, 8, 64, 100, 0) == 0
    assert pkv.paged_attention_prefill_workspace_size(2, 10, 8, 8, 64, 100, 48) == 0   # not x32
    assert pkv.paged_attention_prefill_workspace_size(2, 10, 8, 8, 64, 100, 16384) == 0
    assert pkv.paged_attention_prefill_workspace_size(2, 10, 68, 4, 64, 100, 0) == 0   # G 17


def _prefill(lib, **over):
    args = dict(out=1, query=1, key_cache=1, value_cache=1, block_tables=1, context_lens=1,
                query_start_loc=1, scale=0.125, num_seqs=2, num_tokens=10, num_heads=8,
                num_kv_heads=2, head_size=128, block_size=16, max_blocks=4, max_context_len=64,
                dtype=2, partition_size=0, workspace=None, ws_bytes=0, stream=None)
    args.update(over)
    return lib.pkv_paged_attention_prefill(*args.values())


@pytest.mark.parametrize("over,code", [
    (dict(dtype=0), -2),                          # fp32: matrix cores only
    (dict(dtype=7), -1),
    (dict(num_heads=7), -1),                      # not a multiple of num_kv_heads
    (dict(num_heads=34), -2),                     # group size 17
    (dict(head_size=96), -2),
    (dict(block_size=64), -2),
    (dict(scale=0.0), -1),
    (dict(scale=float("inf")), -1),
    (dict(partition_size=48), -1),
    (dict(partition_size=16384), -1),
    (dict(max_blocks=3), -1),                     # 3 x 16 < max_context_len 64
    (dict(query_start_loc=None), -3),
    (dict(), -4),                                 # needs a workspace
    (dict(num_tokens=-1), -1),
])
def test_prefill_argument_errors(over, code):
    lib = _lib()
    assert _prefill(lib, **over) == code
    assert lib.pkv_last_error().decode() != ""


def test_prefill_nothing_to_do():
    lib = _lib()
    assert _prefill(lib, num_tokens=0) == 0
    assert _prefill(lib, num_seqs=0, num_tokens=0) == 0


@pytest.mark.parametrize("entry", [f"pkv_paged_attention_{stage}_{fmt}" for fmt in ("fp8", "int8")
                                   for stage in ("decode", "plan", "partitions_planned")])
@pytest.mark.parametrize("over,code", [
    (dict(k_scale=0.0), -1),
    (dict(v_scale=float("nan")), -1),
    (dict(k_scale=float("inf")), -1),
    (dict(dtype=0), -2),                  # the queries of an 8-bit cache are 16-bit
    (dict(head_size=96), -2),
    (dict(query=None), -3),
])
def test_kv8_decode_argument_errors(entry, over, code):
    lib = _lib()
    args = dict(out=1, query=1, key_cache=1, value_cache=1, block_tables=1, context_lens=1,
                scale=0.125, k_scale=0.02, v_scale=0.03, num_seqs=2, num_heads=8, num_kv_heads=2,
                head_size=128, block_size=16, max_blocks=4, max_context_len=64, dtype=2,
                partition_size=0, workspace=None, ws_bytes=0, stream=None)
    args.update(over)
    assert getattr(lib, entry)(*args.values()) == code
    assert lib.pkv_last_error().decode() != ""


@pytest.mark.parametrize("entry", ["pkv_paged_attention_prefill_fp8", "pkv_paged_attention_prefill_int8"])
def test_kv8_prefill_argument_errors(entry):
    lib = _lib()
    base = dict(out=1, query=1, key_cache=1, value_cache=1, block_tables=1, context_lens=1,
                query_start_loc=1, scale=0.125, k_scale=0.02, v_scale=0.03, num_seqs=2,
                num_tokens=10, num_heads=8, num_kv_heads=2, head_size=128, block_size=16,
                max_blocks=4, max_context_len=64, dtype=2, partition_size=0, workspace=None,
                ws_bytes=0, stream=None)
    for over, code in [(dict(k_scale=-1.0), -1), (dict(v_scale=0.0), -1), (dict(dtype=0), -2),
                       (dict(), -4)]:
        args = dict(base, **over)
        assert getattr(lib, entry)(*args.values()) == code, over


@pytest.mark.parametrize("entry", ["pkv_reshape_and_cache_fp8", "pkv_reshape_and_cache_int8"])
def test_kv8_cache_write_argument_errors(entry):
    lib = _lib()
    f = getattr(lib, entry)
    #               key value kc vc slots N  H  D   bs NB  kstr vstr dtype ks    vs    stream
    assert f(1, 1, 1, 1, 1, 4, 2, 64, 16, 10, 128, 128, 0, 0.02, 0.03, None) == -1   # fp32 input
    assert f(1, 1, 1, 1, 1, 4, 2, 40, 16, 10, 128, 128, 2, 0.02, 0.03, None) == -1   # D % 16
    assert f(1, 1, 1, 1, 1, 4, 2, 64, 16, 10, 128, 128, 2, 0.0, 0.03, None) == -1    # scale 0
    assert f(1, 1, 1, 1, 1, 4, 2, 64, 16, 10, 128, 100, 2, 0.02, 0.03, None) == -1   # stride
    assert f(None, None, None, None, None, 0, 2, 64, 16, 10, 128, 128, 2, 0.02, 0.03, None) == 0


def _plan_and_cache(lib, fmt="", **over):
    """The fused plan + cache-write entries; fmt '' (16-bit), 'fp8', 'int8' or 'shared'."""
    args = dict(out=1, query=1, key_cache=1, value_cache=1, block_tables=1, context_lens=1)
    if fmt == "shared":
        args.update(group_starts=1, prefix_lens=1, num_groups=1)
    args.update(scale=0.125)
    if fmt in ("fp8", "int8"):
        args.update(k_scale=0.02, v_scale=0.03)
    args.update(num_seqs=0, num_heads=8, num_kv_heads=2, head_size=128, block_size=16,
                max_blocks=4, max_context_len=64, dtype=2, partition_size=0, workspace=None,
                ws_bytes=0, key=1, value=1, slot_mapping=1, num_tokens=0, num_blocks=10,
                key_stride=256, value_stride=256, stream=None)
    args.update(over)
    name = "pkv_paged_attention_plan_and_cache" + (f"_{fmt}" if fmt else "")
    return getattr(lib, name)(*args.values())


@pytest.mark.parametrize("fmt", ["", "fp8", "int8", "shared"])
def test_plan_and_cache_argument_errors(fmt):
    """Every fused plan + cache-write entry validates both halves on the host and enqueues
    nothing on error; with no sequences and no tokens it has nothing to do."""
    lib = _lib()
    assert _plan_and_cache(lib, fmt) == 0
    for over, code in [(dict(num_tokens=-1), -1),
                       (dict(num_blocks=-5), -1),
                       (dict(num_tokens=3, key_stride=100), -1),   # stride < Hkv * D
                       (dict(num_tokens=3, key=None), -3),
                       (dict(num_tokens=3, slot_mapping=None), -3),
                       (dict(head_size=96), -2),
                       (dict(num_seqs=2), -4)]:                    # the plan needs a workspace
        if fmt == "shared" and over.get("num_seqs") == 2:
            over = dict(over, num_groups=1)
        assert _plan_and_cache(lib, fmt, **over) == code, (fmt, over)
        assert lib.pkv_last_error().decode() != ""
    if fmt in ("fp8", "int8"):
        assert _plan_and_cache(lib, fmt, k_scale=0.0) == -1
        assert _plan_and_cache(lib, fmt, dtype=0) == -2           # 16-bit queries only
    if fmt == "shared":
        assert _plan_and_cache(lib, fmt, num_seqs=2, num_groups=3) == -1
        assert _plan_and_cache(lib, fmt, num_seqs=2, group_starts=None) == -3
