"""Host block manager of the paged KV cache (ctypes over include/pkv_block_manager.h).

The manager decides which physical block holds each token; the cache operations
move the data: ``append`` gives the slot for ``reshape_and_cache`` and, when the
last block was shared, the (src, dst) pair for ``copy_blocks``; ``swap_out`` /
``swap_in`` give the (src, dst) pairs for ``swap_blocks``.  Host bookkeeping
only: no tensor and no GPU call is involved.
"""
from __future__ import annotations

import ctypes
from typing import Iterable, List, Optional, Tuple

from ._binding import PKVError, _check, library

ALLOC_OK, ALLOC_LATER, ALLOC_NEVER = 0, 1, 2
GPU, CPU = 0, 1


class BlockManager:
    """Reference-counted block tables with copy-on-write, fork and swap planning."""

    def __init__(self, block_size: int, num_gpu_blocks: int, num_cpu_blocks: int = 0,
                 watermark: float = 0.0):
        lib = library()
        handle = lib.pkv_bm_create(block_size, num_gpu_blocks, num_cpu_blocks, watermark)
        if not handle:
            raise PKVError("pkv_bm_create failed: " + lib.pkv_last_error().decode(errors="replace"))
        self._lib, self._h = lib, ctypes.c_void_p(handle)
        self.block_size = block_size

    def close(self) -> None:
        if self._h:
            self._lib.pkv_bm_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def _call(self, name: str, *args) -> int:
        rc = getattr(self._lib, name)(self._h, *args)
        if rc < 0:
            _check(rc, name)
        return rc

    def can_allocate(self, num_tokens: int) -> int:
        """ALLOC_OK, ALLOC_LATER or ALLOC_NEVER for a new sequence of num_tokens."""
        return self._call("pkv_bm_can_allocate", num_tokens)

    def allocate(self, seq_id: int, num_tokens: int) -> None:
        self._call("pkv_bm_allocate", seq_id, num_tokens)

    def fork(self, parent: int, child: int) -> None:
        self._call("pkv_bm_fork", parent, child)

    def can_append(self, num_seqs: int) -> bool:
        return self._call("pkv_bm_can_append", num_seqs) == 1

    def append(self, seq_id: int) -> Tuple[int, Optional[Tuple[int, int]]]:
        """Slot of the new token and the copy-on-write pair (or None)."""
        slot, src, dst = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        self._call("pkv_bm_append", seq_id, ctypes.byref(slot), ctypes.byref(src),
                   ctypes.byref(dst))
        return slot.value, (None if src.value < 0 else (src.value, dst.value))

    def free(self, seq_id: int) -> None:
        self._call("pkv_bm_free", seq_id)

    def _swap(self, name: str, seq_ids: Iterable[int]) -> List[Tuple[int, int]]:
        ids = list(seq_ids)
        arr = (ctypes.c_int64 * max(len(ids), 1))(*ids)
        cap = sum(len(self.block_table(s)) for s in ids)
        pairs = (ctypes.c_int64 * max(2 * cap, 2))()
        n = ctypes.c_int32()
        self._call(name, arr, len(ids), pairs, cap, ctypes.byref(n))
        return [(pairs[2 * i], pairs[2 * i + 1]) for i in range(n.value)]

    def swap_out(self, seq_ids: Iterable[int]) -> List[Tuple[int, int]]:
        """Move the sequences' blocks to the CPU pool; (gpu block, cpu block) pairs."""
        return self._swap("pkv_bm_swap_out", seq_ids)

    def swap_in(self, seq_ids: Iterable[int]) -> List[Tuple[int, int]]:
        """Move the sequences' blocks back to the GPU pool; (cpu block, gpu block) pairs."""
        return self._swap("pkv_bm_swap_in", seq_ids)

    def block_table(self, seq_id: int) -> List[int]:
        cap = -(-self.seq_len(seq_id) // self.block_size)
        buf = (ctypes.c_int32 * max(cap, 1))()
        n = ctypes.c_int32()
        self._call("pkv_bm_block_table", seq_id, buf, cap, ctypes.byref(n))
        return list(buf[:n.value])

    def seq_len(self, seq_id: int) -> int:
        return self._call("pkv_bm_seq_len", seq_id)

    def seq_device(self, seq_id: int) -> int:
        return self._call("pkv_bm_seq_device", seq_id)

    def num_free(self, device: int = GPU) -> int:
        return self._call("pkv_bm_num_free", device)

    def ref_count(self, block: int, device: int = GPU) -> int:
        return self._call("pkv_bm_ref_count", device, block)
