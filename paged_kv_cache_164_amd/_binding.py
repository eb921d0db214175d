"""ctypes binding of libpkv (argument marshalling only; every step runs in the HIP kernels).

The library is loaded after torch so that it binds to the same HIP runtime
(``libamdhip64.so.7``) that torch already loaded: device pointers and stream
handles from torch are then valid for the library.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import List, Optional, Sequence

import torch

PKV_F32, PKV_F16, PKV_BF16 = 0, 1, 2
PKV_SWAP_IN, PKV_SWAP_OUT = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))
# PKV_LIBRARY may name another build of the same library (e.g. one compiled with other tuning knobs).
_LIB_PATH = os.environ.get("PKV_LIBRARY") or os.path.join(_HERE, "libpkv.so")
_INCLUDE = os.path.join(os.path.dirname(_HERE), "include")
_HEADERS = [os.path.join(_INCLUDE, h) for h in ("pkv.h", "pkv_block_manager.h")]
_lib: Optional[ctypes.CDLL] = None

_DTYPE_CODE = {torch.float32: PKV_F32, torch.float16: PKV_F16, torch.bfloat16: PKV_BF16}

_c_int, _c_i64, _c_sz, _c_p, _c_f = (ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t,
                                     ctypes.c_void_p, ctypes.c_float)
_DECODE_ARGTYPES = [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_f, _c_int, _c_int, _c_int, _c_int,
                    _c_int, _c_int, _c_int, _c_int, _c_int, _c_p, _c_sz, _c_p]
_SIGNATURES = {
    "pkv_paged_attention_decode": (_c_int, _DECODE_ARGTYPES),
    "pkv_paged_attention_partitions": (_c_int, _DECODE_ARGTYPES),
    "pkv_paged_attention_plan": (_c_int, _DECODE_ARGTYPES),
    "pkv_paged_attention_partitions_planned": (_c_int, _DECODE_ARGTYPES),
    "pkv_paged_attention_reduce": (_c_int, [_c_p, _c_p, _c_int, _c_int, _c_int, _c_int, _c_int,
                                            _c_int, _c_p, _c_sz, _c_p]),
    "pkv_paged_attention_workspace_size": (_c_sz, [_c_int, _c_int, _c_int, _c_int, _c_int]),
    "pkv_paged_attention_decode_noalloc": (_c_int, _DECODE_ARGTYPES[:16] + [_c_p]),
    "pkv_paged_attention_plan_and_cache": (_c_int, _DECODE_ARGTYPES[:18] + [_c_p, _c_p, _c_p, _c_int,
                                                                           _c_i64, _c_i64, _c_i64, _c_p]),
    "pkv_paged_attention_noalloc_scratch_bytes": (_c_sz, []),
    "pkv_paged_attention_decode_shared": (_c_int, _DECODE_ARGTYPES[:6] + [_c_p, _c_p, _c_int]
                                          + _DECODE_ARGTYPES[6:]),
    "pkv_paged_attention_plan_shared": (_c_int, _DECODE_ARGTYPES[:6] + [_c_p, _c_p, _c_int]
                                        + _DECODE_ARGTYPES[6:]),
    "pkv_paged_attention_partitions_planned_shared": (_c_int, _DECODE_ARGTYPES[:6]
                                                      + [_c_p, _c_p, _c_int]
                                                      + _DECODE_ARGTYPES[6:]),
    "pkv_paged_attention_plan_and_cache_shared": (_c_int, _DECODE_ARGTYPES[:6] + [_c_p, _c_p, _c_int]
                                                  + _DECODE_ARGTYPES[6:18]
                                                  + [_c_p, _c_p, _c_p, _c_int, _c_i64, _c_i64,
                                                     _c_i64, _c_p]),
    "pkv_paged_attention_decode_fp8": (_c_int, _DECODE_ARGTYPES[:7] + [_c_f, _c_f]
                                       + _DECODE_ARGTYPES[7:]),
    "pkv_paged_attention_decode_int8": (_c_int, _DECODE_ARGTYPES[:7] + [_c_f, _c_f]
                                        + _DECODE_ARGTYPES[7:]),
    "pkv_paged_attention_plan_fp8": (_c_int, _DECODE_ARGTYPES[:7] + [_c_f, _c_f]
                                        + _DECODE_ARGTYPES[7:]),
    "pkv_paged_attention_partitions_planned_fp8": (_c_int, _DECODE_ARGTYPES[:7] + [_c_f, _c_f]
                                        + _DECODE_ARGTYPES[7:]),
    "pkv_paged_attention_plan_int8": (_c_int, _DECODE_ARGTYPES[:7] + [_c_f, _c_f]
                                        + _DECODE_ARGTYPES[7:]),
    "pkv_paged_attention_partitions_planned_int8": (_c_int, _DECODE_ARGTYPES[:7] + [_c_f, _c_f]
                                        + _DECODE_ARGTYPES[7:]),
    "pkv_paged_attention_plan_and_cache_fp8": (_c_int, _DECODE_ARGTYPES[:7] + [_c_f, _c_f]
                                               + _DECODE_ARGTYPES[7:18]
                                               + [_c_p, _c_p, _c_p, _c_int, _c_i64, _c_i64,
                                                  _c_i64, _c_p]),
    "pkv_paged_attention_plan_and_cache_int8": (_c_int, _DECODE_ARGTYPES[:7] + [_c_f, _c_f]
                                                + _DECODE_ARGTYPES[7:18]
                                                + [_c_p, _c_p, _c_p, _c_int, _c_i64, _c_i64,
                                                   _c_i64, _c_p]),
    "pkv_paged_attention_prefill_workspace_size": (_c_sz, [_c_int] * 7),
    "pkv_paged_attention_prefill": (_c_int, [_c_p] * 7 + [_c_f] + [_c_int] * 10
                                    + [_c_p, _c_sz, _c_p]),
    "pkv_paged_attention_prefill_fp8": (_c_int, [_c_p] * 7 + [_c_f] * 3 + [_c_int] * 10
                                        + [_c_p, _c_sz, _c_p]),
    "pkv_paged_attention_prefill_int8": (_c_int, [_c_p] * 7 + [_c_f] * 3 + [_c_int] * 10
                                         + [_c_p, _c_sz, _c_p]),
    "pkv_stream_read": (_c_int, [_c_p, _c_sz, _c_p, _c_p]),
    "pkv_reshape_and_cache_fp8": (_c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_int, _c_int, _c_int,
                                           _c_int, _c_i64, _c_i64, _c_i64, _c_int, _c_f, _c_f, _c_p]),
    "pkv_reshape_and_cache_int8": (_c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_int, _c_int, _c_int,
                                            _c_int, _c_i64, _c_i64, _c_i64, _c_int, _c_f, _c_f, _c_p]),
    "pkv_reshape_and_cache": (_c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_int, _c_int, _c_int, _c_int,
                                       _c_i64, _c_i64, _c_i64, _c_int, _c_p]),
    "pkv_copy_blocks": (_c_int, [_c_p, _c_p, _c_int, _c_p, _c_int, _c_i64, _c_i64, _c_p]),
    "pkv_swap_blocks": (_c_int, [_c_p, _c_p, _c_p, _c_int, _c_i64, _c_i64, _c_i64, _c_int, _c_p]),
    "pkv_last_error": (ctypes.c_char_p, []),
    # host block manager (include/pkv_block_manager.h); the manager is an opaque pointer
    "pkv_bm_create": (_c_p, [_c_int, _c_int, _c_int, _c_f]),
    "pkv_bm_destroy": (None, [_c_p]),
    "pkv_bm_can_allocate": (_c_int, [_c_p, _c_int]),
    "pkv_bm_allocate": (_c_int, [_c_p, _c_i64, _c_int]),
    "pkv_bm_fork": (_c_int, [_c_p, _c_i64, _c_i64]),
    "pkv_bm_can_append": (_c_int, [_c_p, _c_int]),
    "pkv_bm_append": (_c_int, [_c_p, _c_i64, _c_p, _c_p, _c_p]),
    "pkv_bm_free": (_c_int, [_c_p, _c_i64]),
    "pkv_bm_swap_out": (_c_int, [_c_p, _c_p, _c_int, _c_p, _c_int, _c_p]),
    "pkv_bm_swap_in": (_c_int, [_c_p, _c_p, _c_int, _c_p, _c_int, _c_p]),
    "pkv_bm_block_table": (_c_int, [_c_p, _c_i64, _c_p, _c_int, _c_p]),
    "pkv_bm_seq_len": (_c_i64, [_c_p, _c_i64]),
    "pkv_bm_seq_device": (_c_int, [_c_p, _c_i64]),
    "pkv_bm_num_free": (_c_int, [_c_p, _c_int]),
    "pkv_bm_ref_count": (_c_int, [_c_p, _c_int, _c_int]),
}


def _header_symbols() -> List[str]:
    """Every function the public headers declare."""
    names = set()
    for h in _HEADERS:
        names.update(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(pkv_\w+)\s*\(", open(h).read(), re.M))
    return sorted(names)


EXPORTED_SYMBOLS = (_header_symbols() if all(os.path.exists(h) for h in _HEADERS)
                    else sorted(_SIGNATURES))


class PKVError(RuntimeError):
    pass


def library_path() -> str:
    return _LIB_PATH


def library() -> ctypes.CDLL:
    """Load libpkv.so (raises if it was never built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise PKVError(f"{_LIB_PATH} is missing: build it with `python -m paged_kv_cache_164_amd.build`")
        lib = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(rc: int, what: str) -> None:
    if rc != 0:
        msg = library().pkv_last_error().decode(errors="replace")
        raise PKVError(f"{what} failed with code {rc}: {msg}")


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _torch_stream(stream):
    """The torch stream object of `stream` (None: torch's current stream; a raw handle is wrapped
    as an external stream)."""
    if stream is None:
        return torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream))


def _on_gpu(*ts: torch.Tensor) -> None:
    for t in ts:
        if not t.is_cuda:
            raise PKVError("pkv operates on GPU tensors only")


def _dtype_code(t: torch.Tensor) -> int:
    try:
        return _DTYPE_CODE[t.dtype]
    except KeyError:
        raise PKVError(f"unsupported dtype {t.dtype}") from None


def paged_attention_workspace_size(num_seqs: int, num_heads: int, head_size: int,
                                   max_context_len: int, partition_size: int = 0) -> int:
    return int(library().pkv_paged_attention_workspace_size(num_seqs, num_heads, head_size,
                                                            max_context_len, partition_size))


def _decode_args(out, query, key_cache, value_cache, block_tables, context_lens, scale,
                 max_context_len, partition_size, workspace, stream, kv8=False):
    _on_gpu(out, query, key_cache, value_cache, block_tables, context_lens)
    B, Hq, D = query.shape
    NB, Hkv, Dx, bs, x = key_cache.shape
    dt = _dtype_code(query)
    if kv8:
        if key_cache.dtype != torch.uint8 or value_cache.dtype != torch.uint8:
            raise PKVError("an 8-bit cache holds uint8 codes")
        if query.dtype != out.dtype or query.element_size() != 2:
            raise PKVError("query and out must share one 16-bit dtype")
    elif not (query.dtype == key_cache.dtype == value_cache.dtype == out.dtype):
        raise PKVError("query, caches and out must share one dtype")
    if x * key_cache.element_size() != 16 or Dx * x != D:
        raise PKVError(f"key_cache must be [num_blocks, Hkv, D/x, bs, x] with x = 16/sizeof ({tuple(key_cache.shape)})")
    if tuple(value_cache.shape) != (NB, Hkv, D, bs):
        raise PKVError(f"value_cache must be [num_blocks, Hkv, D, bs], got {tuple(value_cache.shape)}")
    if tuple(out.shape) != (B, Hq, D):
        raise PKVError("out must have the query's shape")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise PKVError("block_tables and context_lens must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or tuple(context_lens.shape) != (B,):
        raise PKVError("block_tables must be [num_seqs, max_blocks], context_lens [num_seqs]")
    for t in (out, query, key_cache, value_cache, block_tables, context_lens):
        if not t.is_contiguous():
            raise PKVError("all decode tensors must be contiguous")
    need = paged_attention_workspace_size(B, Hq, D, max_context_len, partition_size)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=query.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    return (out.data_ptr(), query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(),
            block_tables.data_ptr(), context_lens.data_ptr(), float(scale), B, Hq, Hkv, D, bs,
            block_tables.shape[1], int(max_context_len), dt, int(partition_size), ws_ptr, ws_bytes,
            _stream(stream)), workspace


def paged_attention_decode(out, query, key_cache, value_cache, block_tables, context_lens, scale,
                           max_context_len, partition_size=0, workspace=None, stream=None):
    """out[b, h] = softmax(scale * q K_b^T) V_b over the sequence's paged tokens (both kernels)."""
    args, ws = _decode_args(out, query, key_cache, value_cache, block_tables, context_lens, scale,
                            max_context_len, partition_size, workspace, stream)
    _check(library().pkv_paged_attention_decode(*args), "pkv_paged_attention_decode")
    return out


def paged_attention_decode_noalloc(out, query, key_cache, value_cache, block_tables,
                                   context_lens, scale, max_context_len, partition_size=0,
                                   stream=None):
    """paged_attention_decode with the library's static scratch instead of a workspace (no
    device allocation anywhere in the call)."""
    need = paged_attention_workspace_size(query.shape[0], query.shape[1], query.shape[2],
                                          max_context_len, partition_size)
    if need > noalloc_scratch_bytes():
        raise PKVError(f"allocation-free decode: these sizes need {need} bytes of scratch, "
                       f"more than the {noalloc_scratch_bytes()} it holds")
    # a zero-size stand-in for the workspace keeps the checks shared without allocating
    args, _ = _decode_args(out, query, key_cache, value_cache, block_tables, context_lens, scale,
                           max_context_len, partition_size, _NO_WORKSPACE, stream)
    _check(library().pkv_paged_attention_decode_noalloc(*args[:16], args[18]),
           "pkv_paged_attention_decode_noalloc")
    return out


class _NoWorkspace:
    """Stands in for a workspace tensor: no device memory behind it."""

    def data_ptr(self):
        return None

    def numel(self):
        return 0

    def element_size(self):
        return 1


_NO_WORKSPACE = _NoWorkspace()


def noalloc_scratch_bytes() -> int:
    return int(library().pkv_paged_attention_noalloc_scratch_bytes())


def paged_attention_decode_shared(out, query, key_cache, value_cache, block_tables, context_lens,
                                  group_starts, prefix_lens, scale, max_context_len,
                                  partition_size=0, workspace=None, stream=None):
    """Decode where the sequences [group_starts[g], group_starts[g+1]) share their first
    prefix_lens[g] tokens' blocks: each shared block is read once per group."""
    _shared_call("pkv_paged_attention_decode_shared", out, query, key_cache, value_cache,
                 block_tables, context_lens, group_starts, prefix_lens, scale, max_context_len,
                 partition_size, workspace, stream)
    return out


def _shared_call(name, out, query, key_cache, value_cache, block_tables, context_lens,
                 group_starts, prefix_lens, scale, max_context_len, partition_size, workspace,
                 stream, tail=()):
    args, ws = _decode_args(out, query, key_cache, value_cache, block_tables, context_lens, scale,
                            max_context_len, partition_size, workspace, stream)
    _on_gpu(group_starts, prefix_lens)
    ng = prefix_lens.numel()
    if (group_starts.dtype != torch.int32 or prefix_lens.dtype != torch.int32
            or tuple(group_starts.shape) != (ng + 1,) or prefix_lens.dim() != 1
            or not (group_starts.is_contiguous() and prefix_lens.is_contiguous())):
        raise PKVError("group_starts must be int32 [num_groups + 1], prefix_lens int32 [num_groups]")
    args = args[:6] + (group_starts.data_ptr(), prefix_lens.data_ptr(), ng) + args[6:]
    args = args[:-1] + tuple(tail) + args[-1:]  # arguments before the stream
    _check(getattr(library(), name)(*args), name)
    return ws


def paged_attention_plan_shared(out, query, key_cache, value_cache, block_tables, context_lens,
                                group_starts, prefix_lens, scale, max_context_len,
                                partition_size=0, workspace=None, stream=None):
    """The shared-prefix work-list kernel alone; returns the workspace holding the list (for
    paged_attention_partitions_planned_shared calls with the same groups, tables and lengths)."""
    return _shared_call("pkv_paged_attention_plan_shared", out, query, key_cache, value_cache,
                        block_tables, context_lens, group_starts, prefix_lens, scale,
                        max_context_len, partition_size, workspace, stream)


def paged_attention_plan_and_cache_shared(out, query, key_cache, value_cache, block_tables,
                                          context_lens, group_starts, prefix_lens, scale,
                                          max_context_len, key, value, slot_mapping,
                                          partition_size=0, workspace=None, stream=None):
    """reshape_and_cache of the step's new tokens and the shared-prefix work-list plan in one
    launch; returns the workspace holding the list (paged_attention_partitions_planned_shared
    and paged_attention_reduce complete the step)."""
    N, NB = _cache_write_checks(key, value, key_cache, value_cache, slot_mapping)
    if key.dtype != query.dtype:
        raise PKVError("key and value must have the query's dtype")
    return _shared_call("pkv_paged_attention_plan_and_cache_shared", out, query, key_cache,
                        value_cache, block_tables, context_lens, group_starts, prefix_lens, scale,
                        max_context_len, partition_size, workspace, stream,
                        tail=(key.data_ptr(), value.data_ptr(), slot_mapping.data_ptr(), N, NB,
                              key.stride(0), value.stride(0)))


def paged_attention_partitions_planned_shared(out, query, key_cache, value_cache, block_tables,
                                              context_lens, group_starts, prefix_lens, scale,
                                              max_context_len, partition_size=0, workspace=None,
                                              stream=None):
    """The shared-prefix attention kernel alone, on the list a paged_attention_plan_shared call
    left in workspace (paged_attention_reduce completes the decode)."""
    if workspace is None:
        raise PKVError("a planned call needs the workspace its plan was written to")
    return _shared_call("pkv_paged_attention_partitions_planned_shared", out, query, key_cache,
                        value_cache, block_tables, context_lens, group_starts, prefix_lens, scale,
                        max_context_len, partition_size, workspace, stream)


def paged_attention_prefill_workspace_size(num_seqs: int, num_tokens: int, num_heads: int,
                                           num_kv_heads: int, head_size: int, max_context_len: int,
                                           partition_size: int = 0) -> int:
    return int(library().pkv_paged_attention_prefill_workspace_size(
        num_seqs, num_tokens, num_heads, num_kv_heads, head_size, max_context_len, partition_size))


def paged_attention_prefill(out, query, key_cache, value_cache, block_tables, context_lens,
                            query_start_loc, scale, max_context_len, partition_size=0,
                            workspace=None, stream=None, k_scale=None, v_scale=None,
                            code="e4m3"):
    """Multi-query (chunked prefill / mixed batch) attention: query rows
    [query_start_loc[b], query_start_loc[b+1]) of request b are the last positions of its
    context_lens[b]-token context and attend causally over its paged keys and values.
    With k_scale / v_scale the caches hold 8-bit codes (uint8): ``code`` 'e4m3' (FP8) or
    'i8' (integers -127..127)."""
    _on_gpu(out, query, key_cache, value_cache, block_tables, context_lens, query_start_loc)
    T, Hq, D = query.shape
    NB, Hkv, Dx, bs, x = key_cache.shape
    B = context_lens.numel()
    kv8 = k_scale is not None
    if kv8:
        _kv8_entry(code)
        if key_cache.dtype != torch.uint8 or value_cache.dtype != torch.uint8 or v_scale is None:
            raise PKVError("an 8-bit cache holds uint8 codes and needs k_scale and v_scale")
        if query.dtype != out.dtype or query.element_size() != 2:
            raise PKVError("query and out must share one 16-bit dtype")
    elif not (query.dtype == key_cache.dtype == value_cache.dtype == out.dtype):
        raise PKVError("query, caches and out must share one dtype")
    dt = _dtype_code(query)
    if x * key_cache.element_size() != 16 or Dx * x != D:
        raise PKVError(f"key_cache must be [num_blocks, Hkv, D/x, bs, x] with x = 16/sizeof ({tuple(key_cache.shape)})")
    if tuple(value_cache.shape) != (NB, Hkv, D, bs):
        raise PKVError(f"value_cache must be [num_blocks, Hkv, D, bs], got {tuple(value_cache.shape)}")
    if tuple(out.shape) != (T, Hq, D):
        raise PKVError("out must have the query's shape")
    if (block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32
            or query_start_loc.dtype != torch.int32):
        raise PKVError("block_tables, context_lens and query_start_loc must be int32")
    if (block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.dim() != 1
            or tuple(query_start_loc.shape) != (B + 1,)):
        raise PKVError("block_tables must be [num_seqs, max_blocks], context_lens [num_seqs], "
                       "query_start_loc [num_seqs + 1]")
    for t in (out, query, key_cache, value_cache, block_tables, context_lens, query_start_loc):
        if not t.is_contiguous():
            raise PKVError("all tensors must be contiguous")
    need = paged_attention_prefill_workspace_size(B, T, Hq, Hkv, D, max_context_len, partition_size)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=query.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    ptrs = (out.data_ptr(), query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(),
            block_tables.data_ptr(), context_lens.data_ptr(), query_start_loc.data_ptr(), float(scale))
    rest = (B, T, Hq, Hkv, D, bs, block_tables.shape[1], int(max_context_len), dt,
            int(partition_size), ws_ptr, ws_bytes, _stream(stream))
    if kv8:
        name = "pkv_paged_attention_prefill_" + _kv8_entry(code)
        _check(getattr(library(), name)(*ptrs, float(k_scale), float(v_scale), *rest), name)
    else:
        _check(library().pkv_paged_attention_prefill(*ptrs, *rest), "pkv_paged_attention_prefill")
    return out


def _kv8_entry(code: str) -> str:
    """Suffix of the C entry points for an 8-bit cache's code format."""
    try:
        return {"e4m3": "fp8", "i8": "int8"}[code]
    except KeyError:
        raise PKVError(f"8-bit cache code must be 'e4m3' or 'i8', got {code!r}") from None


def paged_attention_decode_fp8(out, query, key_cache, value_cache, block_tables, context_lens,
                               scale, k_scale, v_scale, max_context_len, partition_size=0,
                               workspace=None, stream=None, code="e4m3"):
    """Decode over an 8-bit cache: key_cache uint8 [NB, Hkv, D/16, bs, 16], value_cache uint8
    [NB, Hkv, D, bs]; key = code * k_scale, value = code * v_scale, the codes FP8 E4M3
    (``code`` 'e4m3') or integers -127..127 ('i8')."""
    name = "pkv_paged_attention_decode_" + _kv8_entry(code)
    args, ws = _decode_args(out, query, key_cache, value_cache, block_tables, context_lens, scale,
                            max_context_len, partition_size, workspace, stream, kv8=True)
    args = args[:7] + (float(k_scale), float(v_scale)) + args[7:]
    _check(getattr(library(), name)(*args), name)
    return out


def paged_attention_plan_fp8(out, query, key_cache, value_cache, block_tables, context_lens,
                             scale, k_scale, v_scale, max_context_len, partition_size=0,
                             workspace=None, stream=None, code="e4m3"):
    """The 8-bit decode's work-list kernel alone; returns the workspace holding the list (for
    paged_attention_partitions_planned_fp8 calls with the same tables, lengths and shapes)."""
    name = "pkv_paged_attention_plan_" + _kv8_entry(code)
    args, ws = _decode_args(out, query, key_cache, value_cache, block_tables, context_lens, scale,
                            max_context_len, partition_size, workspace, stream, kv8=True)
    args = args[:7] + (float(k_scale), float(v_scale)) + args[7:]
    _check(getattr(library(), name)(*args), name)
    return ws


def paged_attention_partitions_planned_fp8(out, query, key_cache, value_cache, block_tables,
                                           context_lens, scale, k_scale, v_scale, max_context_len,
                                           partition_size=0, workspace=None, stream=None,
                                           code="e4m3"):
    """The 8-bit attention kernel alone, on the list a paged_attention_plan_fp8 call left in
    workspace (paged_attention_reduce completes the decode)."""
    if workspace is None:
        raise PKVError("a planned call needs the workspace its plan was written to")
    name = "pkv_paged_attention_partitions_planned_" + _kv8_entry(code)
    args, ws = _decode_args(out, query, key_cache, value_cache, block_tables, context_lens, scale,
                            max_context_len, partition_size, workspace, stream, kv8=True)
    args = args[:7] + (float(k_scale), float(v_scale)) + args[7:]
    _check(getattr(library(), name)(*args), name)
    return ws


def paged_attention_decode_int8(out, query, key_cache, value_cache, block_tables, context_lens,
                                scale, k_scale, v_scale, max_context_len, partition_size=0,
                                workspace=None, stream=None):
    """paged_attention_decode_fp8 over INT8 codes."""
    return paged_attention_decode_fp8(out, query, key_cache, value_cache, block_tables,
                                      context_lens, scale, k_scale, v_scale, max_context_len,
                                      partition_size, workspace, stream, code="i8")


def paged_attention_partitions(out, query, key_cache, value_cache, block_tables, context_lens,
                               scale, max_context_len, partition_size=0, workspace=None,
                               stream=None):
    """Phase 1 only; returns the workspace that pkv_paged_attention_reduce must be given."""
    args, ws = _decode_args(out, query, key_cache, value_cache, block_tables, context_lens, scale,
                            max_context_len, partition_size, workspace, stream)
    _check(library().pkv_paged_attention_partitions(*args), "pkv_paged_attention_partitions")
    return ws


def paged_attention_plan(out, query, key_cache, value_cache, block_tables, context_lens, scale,
                         max_context_len, partition_size=0, workspace=None, stream=None):
    """The work-list kernel alone; returns the workspace holding the list (for
    paged_attention_partitions_planned calls with the same tables, lengths and shapes)."""
    args, ws = _decode_args(out, query, key_cache, value_cache, block_tables, context_lens, scale,
                            max_context_len, partition_size, workspace, stream)
    _check(library().pkv_paged_attention_plan(*args), "pkv_paged_attention_plan")
    return ws


def paged_attention_partitions_planned(out, query, key_cache, value_cache, block_tables,
                                       context_lens, scale, max_context_len, partition_size=0,
                                       workspace=None, stream=None):
    """The attention kernel alone, on the list a paged_attention_plan call left in workspace."""
    if workspace is None:
        raise PKVError("a planned call needs the workspace its plan was written to")
    args, ws = _decode_args(out, query, key_cache, value_cache, block_tables, context_lens, scale,
                            max_context_len, partition_size, workspace, stream)
    _check(library().pkv_paged_attention_partitions_planned(*args),
           "pkv_paged_attention_partitions_planned")
    return ws


def paged_attention_reduce(out, context_lens, max_context_len, workspace, partition_size=0,
                           stream=None):
    _on_gpu(out, context_lens)
    B, Hq, D = out.shape
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(library().pkv_paged_attention_reduce(out.data_ptr(), context_lens.data_ptr(), B, Hq, D,
                                                int(max_context_len), _dtype_code(out),
                                                int(partition_size), ws_ptr, ws_bytes,
                                                _stream(stream)),
           "pkv_paged_attention_reduce")
    return out


def _cache_write_checks(key, value, key_cache, value_cache, slot_mapping):
    _on_gpu(key, value, key_cache, value_cache, slot_mapping)
    N, Hkv, D = key.shape
    NB, Hkv2, Dx, bs, x = key_cache.shape
    if Hkv2 != Hkv or Dx * x != D or tuple(value.shape) != (N, Hkv, D):
        raise PKVError("key/value [N, Hkv, D] must match the cache layout")
    if tuple(value_cache.shape) != (NB, Hkv, D, bs):
        raise PKVError("value_cache must be [num_blocks, Hkv, D, bs]")
    if not (key.dtype == value.dtype == key_cache.dtype == value_cache.dtype):
        raise PKVError("key, value and caches must share one dtype")
    for t in (key, value):
        if t.stride(2) != 1 or t.stride(1) != D:
            raise PKVError("key/value need stride(-1) == 1 and stride(1) == head_size")
    if not (key_cache.is_contiguous() and value_cache.is_contiguous()):
        raise PKVError("caches must be contiguous")
    if slot_mapping.dtype != torch.int64 or slot_mapping.numel() != N or not slot_mapping.is_contiguous():
        raise PKVError("slot_mapping must be contiguous int64 with one entry per token")
    return N, NB


def paged_attention_plan_and_cache(out, query, key_cache, value_cache, block_tables,
                                   context_lens, scale, max_context_len, key, value,
                                   slot_mapping, partition_size=0, workspace=None, stream=None):
    """reshape_and_cache of the step's new tokens and the decode work-list plan in one launch;
    returns the workspace holding the list (paged_attention_partitions_planned and
    paged_attention_reduce complete the step)."""
    args, ws = _decode_args(out, query, key_cache, value_cache, block_tables, context_lens, scale,
                            max_context_len, partition_size, workspace, stream)
    N, NB = _cache_write_checks(key, value, key_cache, value_cache, slot_mapping)
    if key.dtype != query.dtype:
        raise PKVError("key and value must have the query's dtype")
    _check(library().pkv_paged_attention_plan_and_cache(
        *args[:18], key.data_ptr(), value.data_ptr(), slot_mapping.data_ptr(), N, NB,
        key.stride(0), value.stride(0), args[18]), "pkv_paged_attention_plan_and_cache")
    return ws


def paged_attention_plan_and_cache_fp8(out, query, key_cache, value_cache, block_tables,
                                       context_lens, scale, k_scale, v_scale, max_context_len,
                                       key, value, slot_mapping, partition_size=0,
                                       workspace=None, stream=None, code="e4m3"):
    """paged_attention_plan_and_cache over an 8-bit cache: reshape_and_cache_fp8 of the step's
    new fp16 / bf16 tokens and the work-list plan in one launch; returns the workspace holding
    the list (paged_attention_partitions_planned_fp8 and paged_attention_reduce complete the
    step)."""
    name = "pkv_paged_attention_plan_and_cache_" + _kv8_entry(code)
    args, ws = _decode_args(out, query, key_cache, value_cache, block_tables, context_lens, scale,
                            max_context_len, partition_size, workspace, stream, kv8=True)
    N, Hkv, D = key.shape
    NB = key_cache.shape[0]
    _on_gpu(key, value, slot_mapping)
    if tuple(value.shape) != (N, Hkv, D) or key.dtype != query.dtype or value.dtype != query.dtype:
        raise PKVError("key and value must be [N, Hkv, D] of the query's dtype")
    if Hkv != key_cache.shape[1] or D != key_cache.shape[2] * key_cache.shape[4]:
        raise PKVError("key/value [N, Hkv, D] must match the cache layout")
    for t in (key, value):
        if t.stride(2) != 1 or t.stride(1) != D:
            raise PKVError("key/value need stride(-1) == 1 and stride(1) == head_size")
    if slot_mapping.dtype != torch.int64 or slot_mapping.numel() != N or not slot_mapping.is_contiguous():
        raise PKVError("slot_mapping must be contiguous int64 with one entry per token")
    _check(getattr(library(), name)(
        *args[:7], float(k_scale), float(v_scale), *args[7:18], key.data_ptr(), value.data_ptr(),
        slot_mapping.data_ptr(), N, NB, key.stride(0), value.stride(0), args[18]), name)
    return ws


def reshape_and_cache(key, value, key_cache, value_cache, slot_mapping, stream=None):
    """key/value [N, Hkv, D] (token rows may be strided; heads and dims contiguous)."""
    _on_gpu(key, value, key_cache, value_cache, slot_mapping)
    N, Hkv, D = key.shape
    NB, Hkv2, Dx, bs, x = key_cache.shape
    if Hkv2 != Hkv or Dx * x != D or tuple(value.shape) != (N, Hkv, D):
        raise PKVError("key/value [N, Hkv, D] must match the cache layout")
    if tuple(value_cache.shape) != (NB, Hkv, D, bs):
        raise PKVError("value_cache must be [num_blocks, Hkv, D, bs]")
    if not (key.dtype == value.dtype == key_cache.dtype == value_cache.dtype):
        raise PKVError("key, value and caches must share one dtype")
    for t in (key, value):
        if t.stride(2) != 1 or t.stride(1) != D:
            raise PKVError("key/value need stride(-1) == 1 and stride(1) == head_size")
    if not (key_cache.is_contiguous() and value_cache.is_contiguous()):
        raise PKVError("caches must be contiguous")
    if slot_mapping.dtype != torch.int64 or slot_mapping.numel() != N or not slot_mapping.is_contiguous():
        raise PKVError("slot_mapping must be contiguous int64 with one entry per token")
    _check(library().pkv_reshape_and_cache(key.data_ptr(), value.data_ptr(), key_cache.data_ptr(),
                                           value_cache.data_ptr(), slot_mapping.data_ptr(), N, Hkv, D,
                                           bs, NB, key.stride(0), value.stride(0),
                                           _dtype_code(key), _stream(stream)),
           "pkv_reshape_and_cache")


def reshape_and_cache_fp8(key, value, key_cache, value_cache, slot_mapping, k_scale, v_scale,
                         stream=None, code="e4m3"):
    """key/value [N, Hkv, D] fp16/bf16 -> 8-bit codes in the 8-bit caches (x = 16): FP8 E4M3
    (``code`` 'e4m3') or integers -127..127 ('i8')."""
    name = "pkv_reshape_and_cache_" + _kv8_entry(code)
    _on_gpu(key, value, key_cache, value_cache, slot_mapping)
    N, Hkv, D = key.shape
    NB, Hkv2, Dx, bs, x = key_cache.shape
    if key_cache.dtype != torch.uint8 or value_cache.dtype != torch.uint8 or x != 16:
        raise PKVError("8-bit caches: uint8 [NB, Hkv, D/16, bs, 16] and [NB, Hkv, D, bs]")
    if Hkv2 != Hkv or Dx * x != D or tuple(value.shape) != (N, Hkv, D):
        raise PKVError("key/value [N, Hkv, D] must match the cache layout")
    if tuple(value_cache.shape) != (NB, Hkv, D, bs) or key.dtype != value.dtype:
        raise PKVError("value_cache must be [num_blocks, Hkv, D, bs]; key and value one dtype")
    for t in (key, value):
        if t.stride(2) != 1 or t.stride(1) != D:
            raise PKVError("key/value need stride(-1) == 1 and stride(1) == head_size")
    if not (key_cache.is_contiguous() and value_cache.is_contiguous()):
        raise PKVError("caches must be contiguous")
    if slot_mapping.dtype != torch.int64 or slot_mapping.numel() != N or not slot_mapping.is_contiguous():
        raise PKVError("slot_mapping must be contiguous int64 with one entry per token")
    _check(getattr(library(), name)(key.data_ptr(), value.data_ptr(), key_cache.data_ptr(),
                                    value_cache.data_ptr(), slot_mapping.data_ptr(), N, Hkv, D,
                                    bs, NB, key.stride(0), value.stride(0), _dtype_code(key),
                                    float(k_scale), float(v_scale), _stream(stream)), name)


def reshape_and_cache_int8(key, value, key_cache, value_cache, slot_mapping, k_scale, v_scale,
                           stream=None):
    """reshape_and_cache_fp8 writing INT8 codes."""
    return reshape_and_cache_fp8(key, value, key_cache, value_cache, slot_mapping, k_scale,
                                 v_scale, stream, code="i8")


def copy_blocks(key_caches: Sequence[torch.Tensor], value_caches: Sequence[torch.Tensor],
                block_mapping: torch.Tensor, stream=None, _ptr_buffers=None):
    """Copy whole blocks (src, dst) in every layer's key and value cache (device mapping [n, 2] int64)."""
    if len(key_caches) != len(value_caches) or not key_caches:
        raise PKVError("one key and one value cache per layer")
    ref = key_caches[0]
    _on_gpu(block_mapping, *key_caches, *value_caches)
    nb = ref.shape[0]
    block_bytes = ref[0].numel() * ref.element_size()
    for c in list(key_caches) + list(value_caches):
        if c.shape[0] != nb or c[0].numel() * c.element_size() != block_bytes or not c.is_contiguous():
            raise PKVError("all caches must be contiguous with equal block counts and block bytes")
    if block_mapping.dtype != torch.int64 or block_mapping.dim() != 2 or block_mapping.shape[1] != 2:
        raise PKVError("block_mapping must be int64 [num_pairs, 2]")
    # The pointer tables (and a contiguous copy of the mapping) are made on the launch stream, so
    # the kernel sees them written; when that is not torch's current stream, the allocator is told
    # they are in use there until the kernel has run.
    ts = _torch_stream(stream)
    with torch.cuda.stream(ts):
        if _ptr_buffers is None:
            kp = torch.tensor([c.data_ptr() for c in key_caches], dtype=torch.int64, device=ref.device)
            vp = torch.tensor([c.data_ptr() for c in value_caches], dtype=torch.int64, device=ref.device)
        else:
            kp, vp = _ptr_buffers
        bm = block_mapping.contiguous()
    if ts != torch.cuda.current_stream():
        for t in (kp, vp, bm):
            t.record_stream(ts)
    _check(library().pkv_copy_blocks(kp.data_ptr(), vp.data_ptr(), len(key_caches), bm.data_ptr(),
                                     bm.shape[0], block_bytes, nb, ts.cuda_stream),
           "pkv_copy_blocks")
    return kp, vp


def swap_blocks(src: torch.Tensor, dst: torch.Tensor, block_mapping, stream=None):
    """dst[d] = src[s] for each (s, d) pair; one side is a GPU cache, the other pinned host memory."""
    if src.is_cuda == dst.is_cuda:
        raise PKVError("swap_blocks moves between a GPU cache and a pinned host cache")
    direction = PKV_SWAP_OUT if src.is_cuda else PKV_SWAP_IN
    if src[0].numel() * src.element_size() != dst[0].numel() * dst.element_size():
        raise PKVError("block sizes differ")
    if not (src.is_contiguous() and dst.is_contiguous()):
        raise PKVError("caches must be contiguous")
    m = torch.as_tensor(block_mapping, dtype=torch.int64).cpu().contiguous()
    if m.dim() != 2 or m.shape[1] != 2:
        raise PKVError("block_mapping must be [num_pairs, 2]")
    block_bytes = src[0].numel() * src.element_size()
    _check(library().pkv_swap_blocks(dst.data_ptr(), src.data_ptr(), m.data_ptr(), m.shape[0],
                                     block_bytes, src.shape[0], dst.shape[0], direction,
                                     _stream(stream)),
           "pkv_swap_blocks")


def stream_read(src: torch.Tensor, sink: torch.Tensor, stream=None):
    """Measurement aid: read all of `src` (device, 16-byte multiple) with the decode kernels'
    streaming loads (see include/pkv.h)."""
    _on_gpu(src, sink)
    _check(library().pkv_stream_read(src.data_ptr(), src.numel() * src.element_size(),
                                     sink.data_ptr(), _stream(stream)), "pkv_stream_read")


def decode_bytes(context_lens, num_heads: int, num_kv_heads: int, head_size: int, block_size: int,
                 elem_bytes: int, kv_elem_bytes: Optional[int] = None) -> int:
    """Algorithmic HBM bytes of one decode call: every context token's K and V (all KV heads),
    q in and out, one int32 block id per block and one int32 length per sequence.  For an
    8-bit cache pass kv_elem_bytes=1 (elem_bytes is then the query's)."""
    lens = [int(v) for v in context_lens]
    kv = sum(lens) * num_kv_heads * head_size * 2 * (kv_elem_bytes or elem_bytes)
    qo = 2 * len(lens) * num_heads * head_size * elem_bytes
    ids = 4 * sum((L + block_size - 1) // block_size for L in lens)
    return kv + qo + ids + 4 * len(lens)
