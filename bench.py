"""Benchmark: one decode step of paged attention on one MI355X.

A step is the whole hot path over one batch: reshape_and_cache of each sequence's newest
token into its slot and the decode work-list plan (one launch: the two are independent), then
paged decode attention (partition kernel + split-K reduce).
Inputs are seeded synthetic tensors already resident in HBM when timing starts.

Prints ONE JSON line.  `value` is the step's algorithmic bytes (every context token's K
and V for all KV heads, q in, out, block ids, lengths, plus the new tokens' K/V read and
written) divided by the step time: achieved GB/s.  `roofline` covers the dominant kernel
(phase 1: the small work-list kernel and the partition kernel it feeds), timed with HIP
events on the stream they are launched on;
`cpu_baseline` is the fp64 oracle timed on the host cores on a bounded sample.

The beam-search workload (c5) times its own step: the shared-prefix work list (it depends on
the groups, tables and lengths only), copy-on-write of each beam's partial last block
(copy_blocks), the new tokens (reshape_and_cache), the shared-prefix partition kernel on that
list, then the reduce; its bytes count each shared prompt block once (the per-sequence count
is reported beside).

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload c3]

HBM traffic of the partition kernel (the `roofline.traffic` field) comes from rocprofv3 counter
runs, scaled by the same counters read on a copy of known size:
    rocprofv3 --pmc FETCH_SIZE -- python3 bench.py --no-cpu-baseline        (then WRITE_SIZE)
    rocprofv3 --pmc FETCH_SIZE -- python3 bench.py --calibrate-copy-mib 512 (then WRITE_SIZE)
    python bench.py --derive-traffic FETCH.csv WRITE.csv CAL_FETCH.csv CAL_WRITE.csv
The last call writes profiles/partition_kernel_<workload>_traffic.json, stamped with a hash of
the kernel sources; bench.py reports the traffic only while that hash still matches.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E spec peak
# --kv: code format of an 8-bit cache, its name, and the config's kv_dtype
KV8_CODES = {"fp8": "e4m3", "int8": "i8"}
KV8_NAMES = {"fp8": "FP8 E4M3", "int8": "INT8 (-127..127)"}
KV8_DTYPES = {"fp8": "fp8_e4m3", "int8": "int8"}
WORKLOADS = {
    "c1": "tiny paged decode: batch 4, 8 heads, head 64, block 16, fp32",
    "c2": "MHA decode, 7B-like layer: batch 64, 32 heads, head 128, block 16, fp16",
    "c3": "GQA decode: batch 256, 32 q heads / 8 KV heads, head 128, block 16, bf16, lognormal lengths",
    "c4": "long-context split-K: batch 8, 64 q / 8 KV heads, head 128, block 32, bf16, 131072 tokens",
    "c5": "shared-prefix beam search: 32 prompts x 4 beams, 40 heads, head 128, block 16, fp16, "
          "2048-token shared prompts + U[1, 512] own tokens; copy-on-write + shared-prefix decode",
    "c6": "chunked prefill (multi-query paged attention): 16 requests x 1024 new tokens after "
          "U[0, 7168] cached ones, 32 q / 8 KV heads, head 128, block 16, bf16",
}
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0}  # MI355X dense matrix-core peaks
KERNEL_SOURCES = ["attention_valu.hip", "attention_gqa.hip", "work_plan.hip", "pkv_device.h",
                  "pkv_internal.h", "pkv_tile_addr.h"]
KERNEL_SOURCES_KV8 = ["attention_fp8.hip", "pkv_kv8.h", "work_plan.hip", "pkv_device.h",
                      "pkv_internal.h", "pkv_tile_addr.h"]


class _Roctx:
    """roctx ranges around the phases of a step (visible with rocprofv3 --marker-trace); no-ops
    when no roctx library is present."""

    def __init__(self):
        import ctypes
        self.lib = None
        for name in ("librocprofiler-sdk-roctx.so.1", "libroctx64.so.4", "libroctx64.so"):
            try:
                lib = ctypes.CDLL(name)
                lib.roctxRangePushA.argtypes = [ctypes.c_char_p]
                lib.roctxRangePushA.restype = ctypes.c_int
                lib.roctxRangePop.restype = ctypes.c_int
                self.lib = lib
                break
            except (OSError, AttributeError):
                continue

    def push(self, name: str) -> None:
        if self.lib is not None:
            self.lib.roctxRangePushA(name.encode())

    def pop(self) -> None:
        if self.lib is not None:
            self.lib.roctxRangePop()


ROCTX = _Roctx()


PREFILL_SOURCES = ["attention_prefill.hip", "pkv_prefill.h", "pkv_kv8.h", "pkv_device.h",
                   "pkv_internal.h"]


def kernel_source_hash(kv: str = "native", workload: str = "c3") -> str:
    h = hashlib.sha256()
    srcs = (PREFILL_SOURCES if workload == "c6"
            else KERNEL_SOURCES if kv == "native" else KERNEL_SOURCES_KV8)
    for f in srcs:
        p = os.path.join(ROOT, "paged_kv_cache_164_amd", "csrc", f)
        if os.path.exists(p):
            h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def traffic_name(workload: str, kv: str = "native") -> str:
    kind = "multi_query_kernel" if workload == "c6" else "partition_kernel"
    return f"{kind}_{workload}{'' if kv == 'native' else '_' + kv}_traffic.json"


def traffic_from_profile(workload: str, kv: str = "native"):
    """HBM bytes per launch of the partition kernel from committed rocprofv3 counter runs, or
    None when absent or taken on different kernel sources."""
    p = os.path.join(ROOT, "profiles", traffic_name(workload, kv))
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("kernel_source_hash") != kernel_source_hash(kv, workload):
        return None
    return d.get("hbm_bytes_per_launch")


PARTITION_KERNELS = ("gqa_grid_kernel", "decode_valu_kernel", "fp8_grid_kernel")
MULTI_QUERY_KERNELS = ("prefill_kernel<",)


def _counter_means(path: str):
    """Mean counter value per dispatch, by kernel name, from a rocprofv3 counter_collection.csv."""
    import csv
    acc = {}
    for r in csv.DictReader(open(path)):
        acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def derive_traffic(workload: str, fetch_csv: str, write_csv: str, cal_fetch_csv: str,
                   cal_write_csv: str, cal_mib: int, kv: str = "native") -> dict:
    """Scale FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the partition kernel by what the same
    counters read for one copy_blocks launch that moves cal_mib one-MiB blocks in each of its two
    caches (2 * cal_mib MiB read, 2 * cal_mib MiB written)."""
    known = 2 * cal_mib * 2 ** 20

    def pick(means, names):
        hits = [v for k, v in means.items() if any(n in k for n in names)]
        if len(hits) != 1:
            raise SystemExit(f"expected one matching kernel for {names}, found {len(hits)}")
        return hits[0]

    f_cal = pick(_counter_means(cal_fetch_csv), ("copy_blocks_kernel",)) * 1024
    w_cal = pick(_counter_means(cal_write_csv), ("copy_blocks_kernel",)) * 1024
    names = MULTI_QUERY_KERNELS if workload == "c6" else PARTITION_KERNELS
    f_k = pick(_counter_means(fetch_csv), names) * 1024
    w_k = pick(_counter_means(write_csv), names) * 1024
    rec = {"workload": workload if kv == "native" else f"{workload}-{kv}",
           "kernel_source_hash": kernel_source_hash(kv, workload),
           "fetch_scale": known / f_cal, "write_scale": known / w_cal,
           "fetch_bytes_raw": f_k, "write_bytes_raw": w_k,
           "hbm_bytes_per_launch": round(f_k * known / f_cal + w_k * known / w_cal)}
    out = os.path.join(ROOT, "profiles", traffic_name(workload, kv))
    with open(out, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec))
    return rec


def calibrate_copy(mib: int, repeats: int = 5) -> None:
    """copy_blocks of mib one-MiB blocks in each of two caches (reads and writes 2 * mib MiB per
    launch), for counter scaling."""
    import torch

    import paged_kv_cache_164_amd as pkv

    dev = torch.device("cuda:0")
    cache = torch.zeros((2 * mib, 2 ** 20 // 2), dtype=torch.float16, device=dev)
    other = torch.zeros((2 * mib, 2 ** 20 // 2), dtype=torch.float16, device=dev)
    mapping = torch.stack([torch.arange(mib), torch.arange(mib, 2 * mib)], dim=1).to(dev)
    for _ in range(repeats):
        pkv.copy_blocks([cache], [other], mapping)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_mib": mib, "launches": repeats}))


def cpu_baseline(case, budget_s: float = 12.0):
    """The fp64 oracle (unchanged) on the first sequences of the same workload, until the
    time budget is spent; throughput in the metric's unit (algorithmic GB/s)."""
    from threadpoolctl import threadpool_info

    import paged_kv_cache_164_amd as pkv
    from oracle import attention as OA
    from oracle import cache_ops as OC
    from workloads import storage_bits

    cfg = case.cfg
    kb, vb = storage_bits(case.key_cache).copy(), storage_bits(case.value_cache).copy()
    lens = case.context_lens.numpy()
    tables = case.block_tables.numpy()
    qbits = storage_bits(case.query)
    nk, nv = storage_bits(case.new_key), storage_bits(case.new_value)
    slots = case.slot_mapping.numpy()
    Hq, D = case.query.shape[1], case.query.shape[2]
    Hkv = case.key_cache.shape[1]
    eb = case.query.element_size()
    done, nbytes, t0 = 0, 0, time.perf_counter()
    while done < len(lens) and (time.perf_counter() - t0) < budget_s:
        b = done
        OC.reshape_and_cache(kb, vb, nk[b:b + 1], nv[b:b + 1], slots[b:b + 1])
        OA.paged_decode(qbits[b:b + 1], kb, vb, cfg.dtype, tables[b:b + 1], lens[b:b + 1], case.scale)
        nbytes += pkv.decode_bytes(lens[b:b + 1], Hq, Hkv, D, cfg.block_size, eb) + 4 * Hkv * D * eb + 8
        done += 1
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    # the same oracle on one thread, over the first sequences, for a quarter of the budget
    from threadpoolctl import threadpool_limits
    kb1, vb1 = storage_bits(case.key_cache).copy(), storage_bits(case.value_cache).copy()
    done1, nbytes1, t1 = 0, 0, time.perf_counter()
    with threadpool_limits(limits=1):
        while done1 < len(lens) and (time.perf_counter() - t1) < budget_s / 4:
            b = done1
            OC.reshape_and_cache(kb1, vb1, nk[b:b + 1], nv[b:b + 1], slots[b:b + 1])
            OA.paged_decode(qbits[b:b + 1], kb1, vb1, cfg.dtype, tables[b:b + 1], lens[b:b + 1],
                            case.scale)
            nbytes1 += pkv.decode_bytes(lens[b:b + 1], Hq, Hkv, D, cfg.block_size, eb) + 4 * Hkv * D * eb + 8
            done1 += 1
    dt1 = time.perf_counter() - t1
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"first {done} of {len(lens)} sequences ({int(lens[:done].sum())} KV tokens, "
                      f"all {Hq} query heads), {dt:.1f} s, affinity {len(os.sched_getaffinity(0))} cpus, "
                      f"{cpu_model()}",
            "single_thread_value": round(nbytes1 / dt1 / 1e9, 4),
            "single_thread_sample": f"first {done1} sequences ({int(lens[:done1].sum())} KV tokens), "
                                    f"{dt1:.1f} s, BLAS limited to 1 thread"}


def beam_setup(dev):
    """The 32 x 4 beam-search step on the GPU: each beam whose last block is partial copies it to
    a fresh block (copy-on-write), its next token is written there, and all beams decode with
    the shared-prefix kernel.  Returns (step inputs, context lengths, unique KV tokens)."""
    import torch

    from workloads import draw_normal, make_beam_case, S_COW

    bc = make_beam_case(num_prompts=32, poison=False)
    bs = bc.cfg.block_size
    B, H, D = bc.query.shape
    tables, lens = bc.block_tables.copy(), bc.context_lens.copy()
    free = list(bc.free_blocks)
    pairs, slots = [], np.full(B, -1, dtype=np.int64)
    for b in range(B):
        L = int(lens[b])
        if L % bs:
            j = (L - 1) // bs
            new = free.pop(0)
            pairs.append((int(tables[b, j]), new))
            tables[b, j] = new
            slots[b] = new * bs + L % bs
            lens[b] = L + 1
    t = dict(q=bc.query.to(dev), kc=bc.key_cache.to(dev), vc=bc.value_cache.to(dev),
             bt=torch.from_numpy(tables).to(dev), cl=torch.from_numpy(lens).to(dev),
             nk=draw_normal((B, H, D), "f16", bc.cfg.seed, S_COW).to(dev),
             nv=draw_normal((B, H, D), "f16", bc.cfg.seed, S_COW + 100).to(dev),
             slots=torch.from_numpy(slots).to(dev),
             mapping=torch.from_numpy(np.array(pairs, dtype=np.int64).reshape(-1, 2)).to(dev),
             gs=torch.arange(0, B + 1, bc.beams, dtype=torch.int32, device=dev),
             pl=torch.full((bc.num_prompts,), bc.prompt_len, dtype=torch.int32, device=dev),
             scale=bc.scale, n_pairs=len(pairs), block_bytes=H * D * bs * 2)
    unique = bc.num_prompts * bc.prompt_len + int((lens - bc.prompt_len).sum())
    return t, lens, unique


def time_steps(step, steps: int, warmup: int, graph: bool):
    """W warm-up steps; then K steps with the dominant kernel bracketed by HIP events (recorded
    on the launch stream by step(ev)), for its time alone; then the K timed steps of the whole
    step, between synchronisations and without events (an event record between two kernels
    holds the second back by ~6 us on this GPU, which is measurement, not the path): graph
    replays of one captured step when `graph`, else eager steps.  step(ev=None, st=None)
    launches on `st` when given (the capture stream), else on the stream it was set up with.
    Returns (ms per step, per-step event times in ms)."""
    import torch

    for _ in range(warmup):
        step()
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        step(events[i])
    torch.cuda.synchronize()
    k_ms = [a.elapsed_time(b) for a, b in events]
    t0 = time.perf_counter()
    for i in range(steps):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / steps
    if graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step(st=side)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(st=torch.cuda.current_stream())
        g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            g.replay()
        torch.cuda.synchronize()
        ms_step = (time.perf_counter() - t0) * 1e3 / steps
    return ms_step, k_ms


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cache_ops_cpu_baseline(budget_s: float = 3.0) -> dict:
    """The oracle's cache operations (unchanged) on the host: copy_blocks and swap_blocks over a
    512-block cache of 160 KiB blocks (128 random pairs per call), reshape_and_cache of the
    decode-step write of 256 tokens x 8 KV heads x 128 bf16 (block 16); each repeated until
    its share of the time budget is spent."""
    from oracle import cache_ops as OC

    g = np.random.default_rng(11)
    nb, pairs = 512, 128
    cache = g.integers(0, 1 << 16, size=(nb, 40, 16, 16, 8), dtype=np.uint16)
    host = np.zeros((pairs,) + cache.shape[1:], dtype=np.uint16)
    perm = g.permutation(nb)
    mapping = np.stack([perm[:pairs], perm[pairs:2 * pairs]], 1)
    out_map = np.stack([perm[:pairs], np.arange(pairs)], 1)
    block_bytes = cache[0].nbytes

    def rate(fn, share):
        n, t0 = 0, time.perf_counter()
        while n == 0 or time.perf_counter() - t0 < budget_s * share:
            fn()
            n += 1
        return n, time.perf_counter() - t0

    n, dt = rate(lambda: OC.copy_blocks([cache], mapping), 0.3)
    copy_gbs = 2 * n * pairs * block_bytes / dt / 1e9  # read + write, as for the device
    n, dt = rate(lambda: OC.swap_blocks(host, cache, out_map), 0.2)
    swap_gbs = n * pairs * block_bytes / dt / 1e9
    kc = np.zeros((nb, 8, 16, 16, 8), dtype=np.uint16)
    vc = np.zeros((nb, 8, 128, 16), dtype=np.uint16)
    key = g.integers(0, 1 << 16, size=(256, 8, 128), dtype=np.uint16)
    val = g.integers(0, 1 << 16, size=(256, 8, 128), dtype=np.uint16)
    slots = g.choice(nb * 16, 256, replace=False)
    n, dt = rate(lambda: OC.reshape_and_cache(kc, vc, key, val, slots), 0.5)
    # plain numpy copies and Python loops: one thread
    return {"kind": "oracle", "copy_blocks_GBs": round(copy_gbs, 2), "swap_GBs": round(swap_gbs, 2),
            "reshape_tokens_per_s": round(n * 256 / dt, 1), "cores": 1,
            "sample": "copy_blocks / swap_blocks: 128 random pairs of 160 KiB blocks in a 512-block "
                      "host cache; reshape_and_cache: 256 tokens x 8 KV heads x 128 (bf16 bits), "
                      f"block 16; about {budget_s:.0f} s in all"}


def auto_partition_label(elem_bytes: int, block_size: int, kv8: bool, max_context_len: int) -> str:
    """The decode entries' auto partition size (include/pkv.h), for the JSON line."""
    if elem_bytes != 2:
        return "auto: 1024"
    max_blocks = 256 if kv8 else 128
    if max_context_len >= 32768 and block_size * max_blocks >= 4096:
        return "auto: 4096"
    return "auto: 2048" if block_size * max_blocks >= 2048 else "auto: 1024"


def block_manager_session(bm, prompts: int = 32, beams: int = 4, prompt_len: int = 3000,
                          steps: int = 64, swap_every: int = 16, swap_seqs: int = 8) -> int:
    """A beam-search session on a block manager (the library's or the oracle's): each prompt
    allocated, forked into `beams` sequences, `steps` decode appends per sequence (copy-on-write
    on the first append after a fork), every `swap_every` steps `swap_seqs` sequences swapped out
    and back in, then everything freed.  Returns the number of manager calls made."""
    calls = 0
    seqs = []
    for p in range(prompts):
        sid = p * beams
        bm.allocate(sid, prompt_len)
        calls += 1
        seqs.append(sid)
        for k in range(1, beams):
            bm.fork(sid, sid + k)
            calls += 1
            seqs.append(sid + k)
    for t in range(steps):
        for sid in seqs:
            bm.append(sid)
            calls += 1
        if (t + 1) % swap_every == 0:
            group = seqs[(t * swap_seqs) % len(seqs):][:swap_seqs]
            bm.swap_out(group)
            bm.swap_in(group)
            calls += 2
    for sid in seqs:
        bm.free(sid)
        calls += 1
    return calls


def block_manager_bench(repeats: int = 5) -> None:
    """Host block manager rates: the library (C++ behind the C ABI, called through the Python
    binding) and the oracle's Python manager on the same session."""
    import paged_kv_cache_164_amd as pkv
    from oracle.block_manager import OracleBlockManager

    def run(make, n):
        best = None
        for _ in range(n):
            bm = make()
            t0 = time.perf_counter()
            calls = block_manager_session(bm)
            dt = time.perf_counter() - t0
            best = dt if best is None else min(best, dt)
            if hasattr(bm, "close"):
                bm.close()
        return calls, best

    calls, dt_lib = run(lambda: pkv.BlockManager(16, 65536, 16384), repeats)
    _, dt_or = run(lambda: OracleBlockManager(16, 65536, 16384), max(1, repeats // 2))
    print(json.dumps({
        "block_manager": "host operations per second, best of several sessions",
        "session": "32 prompts x 3000 tokens, 4 beams each (fork), 64 decode appends per beam "
                   "(copy-on-write after the fork), 8 sequences swapped out and in every 16 "
                   "steps, all freed; block 16, 65536 GPU + 16384 CPU blocks",
        "calls": calls, "library_calls_per_s": round(calls / dt_lib, 1),
        "library_session_ms": round(dt_lib * 1e3, 2),
        "cpu_baseline": {"kind": "oracle", "calls_per_s": round(calls / dt_or, 1),
                         "session_ms": round(dt_or * 1e3, 2), "cores": 1},
    }), flush=True)


def ceilings(steps: int = 20) -> None:
    """Reference rates on the running machine: the HBM read ceiling of the decode kernels' load
    type (a plain streaming read of 4 GiB), copy_blocks (device copy of whole blocks) and
    swap_blocks over the host link, both directions (pinned host memory)."""
    import torch

    import paged_kv_cache_164_amd as pkv

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    def timed(fn, n):
        fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a, b in ev:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in ev]))  # ms

    buf = torch.empty(4 << 30, dtype=torch.uint8, device=dev)
    buf.random_(0, 255)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    ms = timed(lambda: pkv.stream_read(buf, sink, stream=stream), steps)
    read_gbs = buf.numel() / (ms / 1e3) / 1e9

    def ten():
        for _ in range(10):
            pkv.stream_read(buf, sink, stream=stream)
    read10_gbs = 10 * buf.numel() / (timed(ten, 5) / 1e3) / 1e9  # back to back: no launch gaps
    del buf
    # blocks of the c5 shape: 40 heads x 128 dims x 16 tokens x 2 B = 160 KiB (keys; values alike)
    nb, pairs = 4096, 1024
    kc = torch.empty((nb, 40, 16, 16, 8), dtype=torch.float16, device=dev).normal_()
    vc = torch.empty((nb, 40, 128, 16), dtype=torch.float16, device=dev).normal_()
    g = np.random.default_rng(7)
    perm = g.permutation(nb)
    mapping = torch.from_numpy(np.stack([perm[:pairs], perm[pairs:2 * pairs]], 1).astype(np.int64)).to(dev)
    ptrs = pkv.copy_blocks([kc], [vc], mapping, stream=stream)
    block_bytes = kc[0].numel() * kc.element_size()
    ms = timed(lambda: pkv.copy_blocks([kc], [vc], mapping, stream=stream, _ptr_buffers=ptrs), steps)
    copy_gbs = 2 * 2 * pairs * block_bytes / (ms / 1e3) / 1e9  # read + write, keys and values
    # a plain contiguous device copy of the same bytes (torch's copy kernel), for comparison
    flat = kc.view(-1)
    nbytes = 2 * pairs * block_bytes  # keys and values
    n_el = nbytes // kc.element_size()
    assert 2 * n_el <= flat.numel()
    ms_dev = timed(lambda: flat[n_el:2 * n_el].copy_(flat[:n_el]), steps)
    dev_copy_gbs = 2 * nbytes / (ms_dev / 1e3) / 1e9  # read + write
    # the decode step's cache write alone: 256 tokens x 8 KV heads x 128 bf16, block 16
    rk = torch.empty((4096, 8, 16, 16, 8), dtype=torch.bfloat16, device=dev)
    rv = torch.empty((4096, 8, 128, 16), dtype=torch.bfloat16, device=dev)
    nk = torch.randn((256, 8, 128), device=dev).to(torch.bfloat16)
    nv = torch.randn((256, 8, 128), device=dev).to(torch.bfloat16)
    rs = torch.from_numpy(np.random.default_rng(5).choice(4096 * 16, 256, replace=False)).to(dev)
    ms_rc = timed(lambda: pkv.reshape_and_cache(nk, nv, rk, rv, rs, stream=stream), steps)
    del rk, rv
    host = torch.empty((pairs,) + tuple(kc.shape[1:]), dtype=kc.dtype, pin_memory=True)
    m_out = np.stack([perm[:pairs], np.arange(pairs)], 1).astype(np.int64)
    m_in = np.stack([np.arange(pairs), perm[pairs:2 * pairs]], 1).astype(np.int64)
    ms_out = timed(lambda: pkv.swap_blocks(kc, host, m_out, stream=stream), max(steps // 4, 3))
    ms_in = timed(lambda: pkv.swap_blocks(host, kc, m_in, stream=stream), max(steps // 4, 3))
    # the link itself: one contiguous copy of the same bytes each way (copy engines)
    ms_lo = timed(lambda: host.copy_(kc[:pairs], non_blocking=True), max(steps // 4, 3))
    ms_li = timed(lambda: kc[:pairs].copy_(host, non_blocking=True), max(steps // 4, 3))
    # the copy engines block by block (one asynchronous copy per scattered block)
    src_ids, dst_ids = [int(v) for v in perm[:pairs]], [int(v) for v in perm[pairs:2 * pairs]]

    def per_block_out():
        for i, s in enumerate(src_ids):
            host[i].copy_(kc[s], non_blocking=True)

    def per_block_in():
        for i, d in enumerate(dst_ids):
            kc[d].copy_(host[i], non_blocking=True)
    ms_bo = timed(per_block_out, max(steps // 4, 3))
    ms_bi = timed(per_block_in, max(steps // 4, 3))
    gbs = lambda ms: round(pairs * block_bytes / (ms / 1e3) / 1e9, 2)  # noqa: E731
    print(json.dumps({
        "ceilings": "reference rates on this GPU",
        "stream_read_GBs": round(read_gbs, 1), "stream_read_frac_of_8TBs": round(read_gbs / HBM_PEAK_GBS, 4),
        "stream_read_back_to_back_GBs": round(read10_gbs, 1), "stream_read_bytes": 4 << 30,
        "copy_blocks_GBs": round(copy_gbs, 1), "copy_blocks_pairs": pairs, "block_bytes": block_bytes,
        "device_contiguous_copy_GBs": round(dev_copy_gbs, 1),
        "reshape_and_cache_256x8x128_us": round(ms_rc * 1e3, 2),
        "reshape_and_cache_tokens_per_s": round(256 / (ms_rc / 1e3), 1),
        "swap_out_GBs": gbs(ms_out), "swap_in_GBs": gbs(ms_in), "swap_bytes": pairs * block_bytes,
        "host_link_contiguous_out_GBs": gbs(ms_lo), "host_link_contiguous_in_GBs": gbs(ms_li),
        "copy_engine_per_block_out_GBs": gbs(ms_bo), "copy_engine_per_block_in_GBs": gbs(ms_bi),
        "cpu_baseline": cache_ops_cpu_baseline(),
    }), flush=True)


def prefill_cpu_baseline(case, budget_s: float = 12.0):
    """The fp64 oracle (unchanged) on the first rows of the chunked-prefill workload, row by
    row until the time budget is spent; throughput in TFLOP/s of useful attention flops."""
    from threadpoolctl import threadpool_info

    from oracle import cache_ops as OC
    from oracle import prefill as OP
    from workloads import storage_bits

    kb, vb = storage_bits(case.key_cache).copy(), storage_bits(case.value_cache).copy()
    OC.reshape_and_cache(kb, vb, storage_bits(case.new_key), storage_bits(case.new_value),
                         case.slot_mapping)
    qb = storage_bits(case.query)
    Hq, D = case.query.shape[1], case.query.shape[2]
    qsl, lens = case.query_start_loc, case.context_lens
    n0, L0 = int(qsl[1] - qsl[0]), int(lens[0])
    done, t0 = 0, time.perf_counter()
    while done < n0 and (time.perf_counter() - t0) < budget_s:
        rows = list(range(done, min(done + 8, n0)))
        OP.chunked_prefill(qb, kb, vb, case.cfg.dtype, case.block_tables, lens, qsl, case.scale,
                           [(r, h) for r in rows for h in range(Hq)])
        done = rows[-1] + 1
    dt = time.perf_counter() - t0
    # rows 0..done-1 of request 0 sit at positions L0 - n0 .. and see L0 - n0 + 1 .. keys
    pairs = sum(L0 - n0 + 1 + i for i in range(done))
    flops = 4 * D * Hq * pairs
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"first {done} of {case.num_tokens} query rows (request 0, all {Hq} heads), "
                      f"{dt:.1f} s, affinity {len(os.sched_getaffinity(0))} cpus, {cpu_model()}"}


def run_prefill(args) -> int:
    """Chunked-prefill step: reshape_and_cache of every new token, then multi-query attention."""
    import torch

    import paged_kv_cache_164_amd as pkv
    from oracle.prefill import attention_flops
    from workloads import draw_prefill_requests, make_prefill_case, with_8bit_cache

    t_gen = time.perf_counter()
    dev = torch.device("cuda:0")
    P = args.partition
    case = make_prefill_case(draw_prefill_requests(), poison=False)
    kv8 = args.kv != "native"
    code = KV8_CODES.get(args.kv)
    if kv8:
        case = with_8bit_cache(case, code)
    q = case.query.to(dev)
    kc, vc = case.key_cache.to(dev), case.value_cache.to(dev)
    bt = torch.from_numpy(case.block_tables).to(dev)
    cl = torch.from_numpy(case.context_lens).to(dev)
    qsl = torch.from_numpy(case.query_start_loc).to(dev)
    nk, nv = case.new_key.to(dev), case.new_value.to(dev)
    slots = torch.from_numpy(case.slot_mapping).to(dev)
    print(f"# generated {args.workload} in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)
    out = torch.empty_like(q)
    T, Hq, D = q.shape
    Hkv, bs = kc.shape[1], kc.shape[3]
    B, lmax = len(case.context_lens), case.max_context_len
    need = pkv.paged_attention_prefill_workspace_size(B, T, Hq, Hkv, D, lmax, P)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(ev=None, st=None):
        st = stream if st is None else st
        ROCTX.push("step")
        ROCTX.push("reshape_and_cache")
        if kv8:
            pkv.reshape_and_cache_fp8(nk, nv, kc, vc, slots, case.k_scale, case.v_scale, stream=st,
                                      code=code)
        else:
            pkv.reshape_and_cache(nk, nv, kc, vc, slots, stream=st)
        ROCTX.pop()
        if ev is not None:
            ev[0].record(st)
        ROCTX.push("multi-query attention")
        pkv.paged_attention_prefill(out, q, kc, vc, bt, cl, qsl, case.scale, lmax, P, ws,
                                    stream=st, k_scale=case.k_scale if kv8 else None,
                                    v_scale=case.v_scale if kv8 else None, code=code or "e4m3")
        if ev is not None:
            ev[1].record(st)
        ROCTX.pop()
        ROCTX.pop()

    ms_step, k_ms = time_steps(step, args.steps, args.warmup, args.graph)
    k_avg = float(np.mean(k_ms))
    flops = attention_flops(case.context_lens, case.query_start_loc, Hq, D)
    dt = {torch.float16: "f16", torch.bfloat16: "bf16"}[q.dtype]
    peak = MFMA_PEAK_TFLOPS[dt]
    tflops = flops / (ms_step / 1e3) / 1e12
    k_tflops = flops / (k_avg / 1e3) / 1e12
    rec = {
        "metric": "multi-query paged attention achieved TFLOP/s (useful causal flops), 1 GPU",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt,
        "data": "synthetic",
        "config": {"workload": f"{args.workload}{'-' + args.kv if kv8 else ''}: {WORKLOADS[args.workload]}"
                               + (f"; KV cache as {KV8_NAMES[args.kv]} codes with per-cache scales" if kv8 else ""),
                   "num_seqs": B,
                   "num_tokens": T, "num_heads": Hq, "num_kv_heads": Hkv, "head_size": D,
                   "block_size": bs, "partition_size": P or "auto: 8192",
                   "kv_tokens": int(case.context_lens.sum()), "max_context_len": lmax,
                   "attention_flops": flops, "timing": "graph replay" if args.graph else "eager"},
        "query_tokens_per_s": round(T / (ms_step / 1e3), 1),
        "roofline": {"bound": "mfma", "achieved": round(k_tflops, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(k_tflops / peak, 4),
                     "traffic": traffic_from_profile(args.workload, args.kv),
                     "kernel": "multi-query attention: plan + attention kernel",
                     "kernel_ms": round(k_avg, 5), "kernel_ms_median": round(float(np.median(k_ms)), 5),
                     "kernel_ms_p10_p90":
                         [round(float(np.percentile(k_ms, 10)), 5), round(float(np.percentile(k_ms, 90)), 5)],
                     "algorithmic_flops_per_launch": flops},
    }
    if kv8:
        rec["config"]["kv_dtype"] = KV8_DTYPES[args.kv]
    if not args.no_cpu_baseline and not kv8:
        rec["cpu_baseline"] = prefill_cpu_baseline(case)
    print(json.dumps(rec), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the matrix-core-bound chunked-prefill kernel speeds up over the first ~30 ms of a run
    # (launch times fall by ~20% over its first 25 launches, then hold); 50 warm-up steps cover it
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="c3", choices=sorted(WORKLOADS))
    ap.add_argument("--partition", type=int, default=0)
    ap.add_argument("--kv", default="native", choices=["native", "fp8", "int8"],
                    help="fp8 / int8: the same workload over an 8-bit KV cache (FP8 E4M3 or "
                         "INT8 codes with per-cache scales)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of the step captured in a HIP graph instead of eager steps")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0)
    ap.add_argument("--derive-traffic", nargs=4, metavar="CSV")
    ap.add_argument("--calibration-mib", type=int, default=512)
    ap.add_argument("--block-manager", action="store_true",
                    help="print host block-manager rates (library and oracle) instead")
    ap.add_argument("--ceilings", action="store_true",
                    help="print reference rates (streaming read, block copy, host-link swap) instead")
    args = ap.parse_args()
    if args.derive_traffic:
        derive_traffic(args.workload, *args.derive_traffic, args.calibration_mib, args.kv)
        return 0
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the decode path has no multi-GPU mode "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        return 2

    if args.ceilings:
        ceilings()
        return 0
    if args.block_manager:
        block_manager_bench()
        return 0
    if args.calibrate_copy_mib:
        calibrate_copy(args.calibrate_copy_mib)
        return 0

    if args.workload == "c6":
        return run_prefill(args)

    import torch

    import paged_kv_cache_164_amd as pkv
    from workloads import make_decode_case, with_8bit_cache

    t_gen = time.perf_counter()
    dev = torch.device("cuda:0")
    P = args.partition
    beam = args.workload == "c5"
    kv8 = args.kv != "native"
    code = KV8_CODES.get(args.kv)
    if kv8 and (beam or args.workload == "c1"):
        print("--kv fp8 / int8 apply to the 16-bit workloads c2, c3, c4, c6", file=sys.stderr)
        return 2
    if beam:
        t, lens_np, unique_tokens = beam_setup(dev)
        q, kc, vc, bt, cl = t["q"], t["kc"], t["vc"], t["bt"], t["cl"]
        nk, nv, slots, scale = t["nk"], t["nv"], t["slots"], t["scale"]
        lmax = int(lens_np.max())
        case = None
    else:
        case = make_decode_case(args.workload)
        if kv8:
            case = with_8bit_cache(case, code)
        q = case.query.to(dev)
        kc, vc = case.key_cache.to(dev), case.value_cache.to(dev)
        bt, cl = case.block_tables.to(dev), case.context_lens.to(dev)
        nk, nv, slots = case.new_key.to(dev), case.new_value.to(dev), case.slot_mapping.to(dev)
        scale, lmax = case.scale, case.max_context_len
    print(f"# generated {args.workload} in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)
    out = torch.empty_like(q)
    B, Hq, D = q.shape
    Hkv, bs = kc.shape[1], kc.shape[3]
    eb = q.element_size()
    need = pkv.paged_attention_workspace_size(B, Hq, D, lmax, P)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)

    stream = torch.cuda.current_stream()
    ptrs = pkv.copy_blocks([kc], [vc], t["mapping"]) if beam else None

    def step(ev=None, st=None):
        st = stream if st is None else st
        ROCTX.push("step")
        # the work list depends on tables, lengths (and groups) only: one launch builds it and
        # writes the new tokens
        if beam:
            # copy-on-write first: new tokens land in the copied blocks.  Device pointer table
            # made once, outside any graph capture.
            ROCTX.push("copy_blocks")
            pkv.copy_blocks([kc], [vc], t["mapping"], stream=st, _ptr_buffers=ptrs)
            ROCTX.pop()
            ROCTX.push("plan and reshape_and_cache")
            pkv.paged_attention_plan_and_cache_shared(out, q, kc, vc, bt, cl, t["gs"], t["pl"],
                                                      scale, lmax, nk, nv, slots, P, ws, stream=st)
            ROCTX.pop()
        elif kv8:
            ROCTX.push("plan and reshape_and_cache")
            pkv.paged_attention_plan_and_cache_fp8(out, q, kc, vc, bt, cl, scale, case.k_scale,
                                                   case.v_scale, lmax, nk, nv, slots, P, ws,
                                                   stream=st, code=code)
            ROCTX.pop()
        else:
            # the plan and the new tokens' cache write are independent: one launch
            ROCTX.push("plan and reshape_and_cache")
            pkv.paged_attention_plan_and_cache(out, q, kc, vc, bt, cl, scale, lmax, nk, nv, slots,
                                               P, ws, stream=st)
            ROCTX.pop()
        if ev is not None:
            ev[0].record(st)
        ROCTX.push("partition kernel")
        if kv8:
            pkv.paged_attention_partitions_planned_fp8(out, q, kc, vc, bt, cl, scale, case.k_scale,
                                                       case.v_scale, lmax, P, ws, stream=st,
                                                       code=code)
        elif beam:
            pkv.paged_attention_partitions_planned_shared(out, q, kc, vc, bt, cl, t["gs"], t["pl"],
                                                          scale, lmax, P, ws, stream=st)
        else:
            pkv.paged_attention_partitions_planned(out, q, kc, vc, bt, cl, scale, lmax, P, ws,
                                                   stream=st)
        if ev is not None:
            ev[1].record(st)
        ROCTX.pop()
        ROCTX.push("reduce")
        pkv.paged_attention_reduce(out, cl, lmax, ws, P, stream=st)
        ROCTX.pop()
        ROCTX.pop()

    ms_step, k_ms = time_steps(step, args.steps, args.warmup, args.graph)
    k_avg = float(np.mean(k_ms))

    lens = lens_np if beam else case.context_lens.numpy()
    kvb = 1 if kv8 else eb
    dec_bytes = pkv.decode_bytes(lens, Hq, Hkv, D, bs, eb, kvb)
    logical_dec_bytes = dec_bytes
    if beam:
        # HBM holds each shared prompt block once and the shared-prefix kernel reads it once:
        # the algorithmic bytes count the unique KV tokens (per-sequence counts are given beside)
        dec_bytes -= (int(lens.sum()) - unique_tokens) * Hkv * D * 2 * kvb
    n_new = int((slots >= 0).sum().item())
    write_bytes = 2 * n_new * Hkv * D * (eb + kvb) + 8 * B  # new K/V read, codes written
    if beam:  # copy-on-write: each pair reads and writes one key block and one value block
        write_bytes += 2 * 2 * t["n_pairs"] * t["block_bytes"] + 16 * t["n_pairs"]
    step_bytes = dec_bytes + write_bytes
    gbs = step_bytes / (ms_step / 1e3) / 1e9
    kernel_gbs = dec_bytes / (k_avg / 1e3) / 1e9
    traffic = None if beam else traffic_from_profile(args.workload, args.kv)
    rec = {
        "metric": "paged decode attention achieved HBM GB/s (% of peak) and KV-tokens/s, 1 GPU",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}[q.dtype],
        "data": "synthetic",
        "config": {"workload": f"{args.workload}{'-' + args.kv if kv8 else ''}: {WORKLOADS[args.workload]}"
                               + (f"; KV cache as {KV8_NAMES[args.kv]} codes with per-cache scales" if kv8 else ""),
                   "num_seqs": B,
                   "num_heads": Hq, "num_kv_heads": Hkv, "head_size": D, "block_size": bs,
                   "partition_size": P or auto_partition_label(eb, bs, kv8, lmax),
                   "kv_tokens": int(lens.sum()), "max_context_len": lmax,
                   "step_bytes": step_bytes, "timing": "graph replay" if args.graph else "eager"},
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "kv_tokens_per_s": round(float(lens.sum()) / (ms_step / 1e3), 1),
        "roofline": {"bound": "hbm", "achieved": round(kernel_gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(kernel_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": ("shared-prefix partition kernel (its work list planned before the timed region)" if beam
                                else "8-bit cache partition kernel (its work list planned before the timed region)" if kv8
                                else "partition kernel (its work list planned before the timed region)"),
                     "kernel_ms": round(k_avg, 5), "kernel_ms_median": round(float(np.median(k_ms)), 5),
                     "kernel_ms_p10_p90":
                         [round(float(np.percentile(k_ms, 10)), 5), round(float(np.percentile(k_ms, 90)), 5)],
                     "algorithmic_bytes_per_launch": dec_bytes},
    }
    if kv8:
        rec["config"]["kv_dtype"] = KV8_DTYPES[args.kv]
    if beam:
        # per-sequence (logical) bytes: every sequence's attention over all of its tokens
        rec["config"]["unique_kv_tokens"] = unique_tokens
        rec["logical_decode_bytes"] = logical_dec_bytes
        rec["logical_decode_GBs"] = round(logical_dec_bytes / (k_avg / 1e3) / 1e9, 2)
    if not args.no_cpu_baseline and not beam and not kv8:
        rec["cpu_baseline"] = cpu_baseline(case)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
