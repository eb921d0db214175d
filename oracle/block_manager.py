"""Plain-Python model of the paged KV cache's block bookkeeping.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Written from the
pages: the BlockSpaceManager of the AIGC interview book (section 23:
admission with a watermark, allocation of a prompt's blocks, the append step
with copy-on-write returning the (old, new) block pair, freeing), the "Vllm"
page ("Scheduler & BlockSpaceManager": swapping whole sequences between the
GPU and CPU pools, CacheEngine's swap maps), and the copy-on-write worked
example of the mlqm.cn explainer ("PagedAttention").

Readings where the pages leave a step open:
* a pool hands out its lowest free block id first (the worked example takes
  block 2, then block 3, from the free list [2, 3]);
* the watermark is int(watermark * num_gpu_blocks) blocks; admission is
  NEVER when the whole pool minus the prompt's blocks is below it, OK when the
  free blocks minus the prompt's blocks stay at or above it, else LATER;
* swapping moves the distinct blocks of the sequences in the order of first
  appearance (sequence order, then table order); a block shared inside the
  set moves once and keeps its count; a block shared with a sequence outside
  the set is refused (it cannot be in two pools).
"""
from __future__ import annotations

from typing import Dict, List, Optional, Tuple

OK, LATER, NEVER = 0, 1, 2
GPU, CPU = 0, 1


class BlockError(Exception):
    pass


class OracleBlockManager:
    def __init__(self, block_size: int, num_gpu_blocks: int, num_cpu_blocks: int = 0,
                 watermark: float = 0.0):
        self.bs = block_size
        self.total = {GPU: num_gpu_blocks, CPU: num_cpu_blocks}
        self.ref = {GPU: [0] * num_gpu_blocks, CPU: [0] * num_cpu_blocks}
        self.watermark_blocks = int(watermark * num_gpu_blocks)
        self.seqs: Dict[int, dict] = {}

    # -- pools ---------------------------------------------------------------
    def num_free(self, dev: int = GPU) -> int:
        return sum(1 for r in self.ref[dev] if r == 0)

    def _take(self, dev: int) -> int:
        for b, r in enumerate(self.ref[dev]):  # lowest free id first
            if r == 0:
                self.ref[dev][b] = 1
                return b
        raise BlockError("pool exhausted")

    def _blocks(self, n_tokens: int) -> int:
        return -(-n_tokens // self.bs)

    # -- admission and allocation (interview book, can_allocate / allocate) ---
    def can_allocate(self, n_tokens: int) -> int:
        need = self._blocks(n_tokens)
        if self.total[GPU] - need < self.watermark_blocks:
            return NEVER
        if self.num_free(GPU) - need >= self.watermark_blocks:
            return OK
        return LATER

    def allocate(self, sid: int, n_tokens: int) -> None:
        if sid in self.seqs:
            raise BlockError("sequence exists")
        if self._blocks(n_tokens) > self.num_free(GPU):
            raise BlockError("not enough free GPU blocks")
        table = [self._take(GPU) for _ in range(self._blocks(n_tokens))]
        self.seqs[sid] = {"len": n_tokens, "dev": GPU, "table": table}

    def fork(self, parent: int, child: int) -> None:
        if parent not in self.seqs or child in self.seqs:
            raise BlockError("bad fork")
        p = self.seqs[parent]
        for b in p["table"]:
            self.ref[p["dev"]][b] += 1
        self.seqs[child] = {"len": p["len"], "dev": p["dev"], "table": list(p["table"])}

    # -- decode step (interview book, can_append_slots / append_slots) --------
    def can_append(self, n_seqs: int) -> bool:
        return n_seqs <= self.num_free(GPU)

    def append(self, sid: int) -> Tuple[int, Optional[Tuple[int, int]]]:
        s = self.seqs.get(sid)
        if s is None or s["dev"] != GPU:
            raise BlockError("sequence not on the GPU")
        t = s["len"]  # position of the new token
        logical = t // self.bs
        cow = None
        if logical == len(s["table"]):  # the token opens a new logical block
            if self.num_free(GPU) == 0:
                raise BlockError("no free block")
            s["table"].append(self._take(GPU))
        else:
            last = s["table"][logical]
            if self.ref[GPU][last] > 1:  # shared: copy on write
                if self.num_free(GPU) == 0:
                    raise BlockError("no free block")
                new = self._take(GPU)
                self.ref[GPU][last] -= 1
                s["table"][logical] = new
                cow = (last, new)
        s["len"] = t + 1
        return s["table"][logical] * self.bs + t % self.bs, cow

    def free(self, sid: int) -> None:
        s = self.seqs.pop(sid)
        for b in s["table"]:
            self.ref[s["dev"]][b] -= 1

    # -- swapping ("Vllm" page, Scheduler & BlockSpaceManager) ---------------
    def _swap(self, sids: List[int], src: int, dst: int) -> List[Tuple[int, int]]:
        if len(set(sids)) != len(sids) or any(
                s not in self.seqs or self.seqs[s]["dev"] != src for s in sids):
            raise BlockError("bad swap set")
        order: List[int] = []
        inside: Dict[int, int] = {}
        for s in sids:
            for b in self.seqs[s]["table"]:
                if b not in inside:
                    order.append(b)
                    inside[b] = 0
                inside[b] += 1
        if any(inside[b] != self.ref[src][b] for b in order):
            raise BlockError("block shared outside the set")
        if len(order) > self.num_free(dst):
            raise BlockError("target pool too small")
        mapping = {}
        for b in order:
            nb = self._take(dst)
            self.ref[dst][nb] = self.ref[src][b]
            self.ref[src][b] = 0
            mapping[b] = nb
        for s in sids:
            seq = self.seqs[s]
            seq["table"] = [mapping[b] for b in seq["table"]]
            seq["dev"] = dst
        return [(b, mapping[b]) for b in order]

    def swap_out(self, sids: List[int]) -> List[Tuple[int, int]]:
        return self._swap(list(sids), GPU, CPU)

    def swap_in(self, sids: List[int]) -> List[Tuple[int, int]]:
        return self._swap(list(sids), CPU, GPU)

    # -- views -----------------------------------------------------------------
    def block_table(self, sid: int) -> List[int]:
        return list(self.seqs[sid]["table"])

    def seq_len(self, sid: int) -> int:
        return self.seqs[sid]["len"]

    def seq_device(self, sid: int) -> int:
        return self.seqs[sid]["dev"]

    def ref_count(self, block: int, dev: int = GPU) -> int:
        return self.ref[dev][block]
