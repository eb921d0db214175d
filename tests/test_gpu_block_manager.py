"""The host block manager driving the cache kernels: prompts written at the slots it
plans, forks, decode steps with copy-on-write (copy_blocks) and the new token
(reshape_and_cache), sequences swapped out to pinned host memory and back (swap_blocks,
freed device blocks poisoned and reused meanwhile).  After every step the decode over the
manager's block tables must match the fp64 oracle's attention over each sequence's own
token history, kept apart from any paging."""
import numpy as np
import pytest
import torch

import paged_kv_cache_164_amd as pkv
from gpu_cases import DEV, log, within_tolerance
from oracle import attention as OA
from workloads import draw_normal, storage_bits

pytestmark = pytest.mark.gpu

BS, HQ, HKV, D, DT = 16, 8, 2, 128, "bf16"
NG, NC = 48, 24
SCALE = D ** -0.5


class Session:
    def __init__(self, seed):
        self.seed, self.stream = seed, 0
        self.kc = torch.zeros(NG, HKV, D // 8, BS, 8, dtype=torch.bfloat16, device=DEV)
        self.vc = torch.zeros(NG, HKV, D, BS, dtype=torch.bfloat16, device=DEV)
        self.hk = torch.zeros(NC, HKV, D // 8, BS, 8, dtype=torch.bfloat16, pin_memory=True)
        self.hv = torch.zeros(NC, HKV, D, BS, dtype=torch.bfloat16, pin_memory=True)
        self.bm = pkv.BlockManager(BS, NG, NC)
        self.hist = {}  # sequence -> (K [L, Hkv, D], V [L, Hkv, D]) in float64

    def draw(self, shape):
        self.stream += 1
        return draw_normal(shape, DT, self.seed, 1000 + self.stream)

    def _write(self, slots, k, v):
        pkv.reshape_and_cache(k.to(DEV), v.to(DEV), self.kc, self.vc,
                              torch.tensor(slots, dtype=torch.int64, device=DEV))

    def add_prompt(self, sid, n):
        self.bm.allocate(sid, n)
        t = self.bm.block_table(sid)
        k, v = self.draw((n, HKV, D)), self.draw((n, HKV, D))
        self._write([t[p // BS] * BS + p % BS for p in range(n)], k, v)
        self.hist[sid] = (OA.widen(storage_bits(k), DT), OA.widen(storage_bits(v), DT))

    def fork(self, parent, child):
        self.bm.fork(parent, child)
        self.hist[child] = tuple(a.copy() for a in self.hist[parent])

    def step(self, sids):
        """One decode step of the given sequences; checks the output; returns the CoW pairs."""
        assert self.bm.can_append(len(sids))
        slots, pairs = [], []
        for s in sids:
            slot, cow = self.bm.append(s)
            slots.append(slot)
            if cow is not None:
                pairs.append(cow)
        if pairs:
            pkv.copy_blocks([self.kc], [self.vc],
                            torch.tensor(pairs, dtype=torch.int64, device=DEV))
        k, v = self.draw((len(sids), HKV, D)), self.draw((len(sids), HKV, D))
        self._write(slots, k, v)
        kb, vb = OA.widen(storage_bits(k), DT), OA.widen(storage_bits(v), DT)
        for i, s in enumerate(sids):
            K, V = self.hist[s]
            self.hist[s] = (np.concatenate([K, kb[i:i + 1]]), np.concatenate([V, vb[i:i + 1]]))
        self.check(sids)
        return pairs

    def check(self, sids):
        q = self.draw((len(sids), HQ, D))
        lens = np.array([self.bm.seq_len(s) for s in sids], dtype=np.int32)
        width = int(-(-lens.max() // BS))
        tables = np.zeros((len(sids), width), dtype=np.int32)
        for i, s in enumerate(sids):
            t = self.bm.block_table(s)
            tables[i, :len(t)] = t
        out = torch.empty(len(sids), HQ, D, dtype=torch.bfloat16, device=DEV)
        pkv.paged_attention_decode(out, q.to(DEV), self.kc, self.vc,
                                   torch.from_numpy(tables).to(DEV), torch.from_numpy(lens).to(DEV),
                                   SCALE, int(lens.max()))
        got = out.float().cpu().numpy().astype(np.float64)
        qb = OA.widen(storage_bits(q), DT)
        ref = np.empty_like(got)
        for i, s in enumerate(sids):
            K, V = self.hist[s]
            for h in range(HQ):
                kvh = h // (HQ // HKV)
                ref[i, h] = OA.dense_decode(qb[i, h], K[:, kvh], V[:, kvh], OA.as_scale(SCALE))
        ok, err, ratio = within_tolerance(got, ref, DT)
        assert ok, f"sequences {sids}: max err {err}, worst ratio {ratio}"

    def swap_out(self, sids):
        pairs = self.bm.swap_out(sids)
        pkv.swap_blocks(self.kc, self.hk, pairs)
        pkv.swap_blocks(self.vc, self.hv, pairs)
        torch.cuda.synchronize()
        gone = torch.tensor([a for a, _ in pairs], dtype=torch.int64, device=DEV)
        self.kc[gone] = float("nan")  # the freed device blocks must never be read again
        self.vc[gone] = float("nan")
        return pairs

    def swap_in(self, sids):
        pairs = self.bm.swap_in(sids)
        pkv.swap_blocks(self.hk, self.kc, pairs)
        pkv.swap_blocks(self.hv, self.vc, pairs)
        torch.cuda.synchronize()
        return pairs


@pytest.mark.parametrize("seed", [0, 1])
def test_manager_drives_cache_ops(seed):
    log(f"block manager session seed {seed}")
    s = Session(seed)
    for sid, n in ((0, 37), (1, 70), (2, 5)):
        s.add_prompt(sid, n)
    s.check([0, 1, 2])
    s.fork(0, 10)
    s.fork(0, 11)
    s.fork(1, 12)
    gpu = [0, 10, 11, 1, 12, 2]
    n_pairs = 0
    for _ in range(12):
        n_pairs += len(s.step(gpu))
    assert n_pairs >= 3  # the forked families copied their shared last blocks
    out_pairs = s.swap_out([1, 12, 2])
    assert all(s.bm.seq_device(x) == pkv.block_manager.CPU for x in (1, 12, 2))
    for _ in range(20):  # the swapped-out blocks are free and get reused here
        s.step([0, 10, 11])
    in_pairs = s.swap_in([2, 12, 1])
    assert len(out_pairs) == len(in_pairs)
    s.check(gpu)
    for _ in range(6):
        s.step(gpu)
    for x in (10, 11):
        s.bm.free(x)
    s.step([0, 1, 12, 2])
    torch.cuda.synchronize()
    log(f"seed {seed}: {n_pairs} copy-on-write pairs, {len(out_pairs)} blocks swapped")
