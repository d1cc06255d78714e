"""Benchmark of the paged decode path on one MI355X.

A step is one pass of the whole path over one synthetic decode batch: copy-on-write block
copies (shared-prefix batch only), the cache write of one new token per sequence, the
per-partition attention kernel and the partition merge. Inputs are resident in HBM before the
timed region; three independently drawn input sets rotate so that repeated steps are not
served from the 256 MB Infinity Cache.

Per decode workload, two timed passes of K steps each: an eager pass with HIP events around
every kernel (the attention kernel's average duration gives ``roofline``), then the timed region
proper, where the whole step is captured once per input set in a HIP graph and replayed K times
(``--eager`` skips the graph pass and reports the eager step time instead). The headline
workload (``--config``, the OPT-13B-shape batch) gives the top-level fields; the other decode
workloads (``--also``: GQA, long-context, shared-prefix, tiny) are measured in the same run and
reported under ``workloads`` with the same fields.

Prints one JSON line. ``value`` is KV bytes read per step / step time (GB/s, whole step);
``roofline`` reports the attention kernel alone (HIP events on its stream) against the 8 TB/s
HBM peak (for batches that share blocks, against the bytes of the distinct blocks);
``hbm_copy_gbps`` is a plain 1 GiB device copy on the same GPU (``frac_of_copy`` = value /
that); ``cpu_baseline`` times the CPU oracle on every host core (at most 16 worker processes)
over the whole batch, with the one-thread figure on a bounded sample beside it.

``prefill`` (default: the GQA prompt workload) times pa_prefill on a prefill batch and reports
it against the 16-bit matrix-core peak, with its own CPU-oracle sample.

    python bench.py [--steps K] [--warmup W] [--config NAME] [--also NAMES] [--partition P]
                    [--eager] [--prefill NAMES] [--prefill-only]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
# the attention stage's kernels: the decode kernel, and the share plan (shared-prefix batches)
KERNEL_SOURCES = ["paged_kv_cache_384_amd/csrc/pa_attention.h",
                  "paged_kv_cache_384_amd/csrc/pa_device.h",
                  "paged_kv_cache_384_amd/csrc/pa_reduce.hip"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str):
    """HBM bytes per attention launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"pa_decode_attention_{workload}_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    src = re.search(r"kernel_source_hash:\s*([0-9a-f]+)", text)
    val = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not src or not val or src.group(1) != kernel_source_hash():
        return None
    return float(val.group(1))


def host_storage(t):
    """Host numpy copy of a tensor's stored elements (bf16 as raw uint16 bits)."""
    import numpy as np
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def cpu_baseline(batch, host, budget_s: float):
    """The CPU oracle, single-threaded, on as many whole sequences as fit in ``budget_s``."""
    from threadpoolctl import threadpool_limits

    import oracle
    cfg = batch.cfg
    kw = dict(dtype=cfg.dtype, num_kv_heads=cfg.num_kv_heads, block_size=cfg.block_size,
              head_dim=cfg.head_dim)
    done, kv = 0, 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=1):
        for s in range(cfg.num_seqs):
            oracle.paged_decode_ref(host["query"], host["k_pool"], host["v_pool"],
                                    batch.block_tables, batch.context_lens, cfg.scale,
                                    seqs=[s], **kw)
            done += 1
            kv += int(batch.context_lens[s]) * cfg.num_kv_heads * cfg.head_dim * 2 * cfg.esz
            if time.perf_counter() - t0 > budget_s:
                break
    dt = time.perf_counter() - t0
    return {"value": round(kv / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} of {cfg.num_seqs} sequences (all {cfg.num_q_heads} query heads), "
                      f"{kv / 1e6:.1f} MB of KV in {dt:.1f} s, numpy float64, 1 thread",
            "seconds": round(dt, 2), "tokens_per_s": round(done / dt, 3)}


# ---- the oracle on every host core: spawned worker processes over shared memory ----------
# The workers are fresh interpreters (they never touch the GPU); the pools, query and tables are
# copied once into shared memory, each worker maps them and runs the oracle on groups of whole
# sequences with one BLAS thread.

_WORKER = {}


def _oracle_worker_init(spec):
    import numpy as np
    from multiprocessing import shared_memory
    from threadpoolctl import threadpool_limits
    _WORKER["limits"] = threadpool_limits(limits=1)
    _WORKER["shm"] = []
    arrays = {}
    for name, (shm_name, shape, dtype) in spec["arrays"].items():
        # attaching registers the name with the parent's resource tracker again (the spawned
        # workers share it), which is harmless: the parent unlinks the segments once at the end
        shm = shared_memory.SharedMemory(name=shm_name)
        _WORKER["shm"].append(shm)
        arrays[name] = np.ndarray(shape, dtype=dtype, buffer=shm.buf)
    _WORKER["arrays"] = arrays
    _WORKER["meta"] = spec["meta"]


def _oracle_worker_run(seqs):
    import oracle
    a, m = _WORKER["arrays"], _WORKER["meta"]
    t0 = time.perf_counter()
    if seqs:
        oracle.paged_decode_ref(a["query"], a["k_pool"], a["v_pool"], a["block_tables"],
                                a["context_lens"], m["scale"], seqs=seqs, dtype=m["dtype"],
                                num_kv_heads=m["num_kv_heads"], block_size=m["block_size"],
                                head_dim=m["head_dim"])
    return time.perf_counter() - t0


def host_workers() -> int:
    """Host cores this process may use, at most 16 (the host share of one GPU)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def cpu_baseline_all_cores(batch, host, workers: int):
    """The CPU oracle over the whole batch on ``workers`` processes (one BLAS thread each), timed
    from the moment the sequence groups are handed out (workers started and inputs in shared
    memory already) to the last result."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor
    from multiprocessing import shared_memory

    import numpy as np
    cfg = batch.cfg
    arrays = {"query": host["query"], "k_pool": host["k_pool"], "v_pool": host["v_pool"],
              "block_tables": batch.block_tables, "context_lens": batch.context_lens}
    segs, spec = [], {"arrays": {}, "meta": dict(scale=float(cfg.scale), dtype=cfg.dtype,
                                                 num_kv_heads=cfg.num_kv_heads,
                                                 block_size=cfg.block_size,
                                                 head_dim=cfg.head_dim)}
    try:
        for name, arr in arrays.items():
            arr = np.ascontiguousarray(arr)
            shm = shared_memory.SharedMemory(create=True, size=max(arr.nbytes, 1))
            segs.append(shm)
            np.ndarray(arr.shape, dtype=arr.dtype, buffer=shm.buf)[...] = arr
            spec["arrays"][name] = (shm.name, arr.shape, arr.dtype.str)
        # groups of whole sequences of similar total length, heaviest first
        lens = batch.context_lens.astype(np.int64)
        order = np.argsort(-lens, kind="stable")
        n_groups = min(cfg.num_seqs, 4 * workers)
        groups = [[] for _ in range(n_groups)]
        load = np.zeros(n_groups, np.int64)
        for s in order.tolist():
            g = int(np.argmin(load))
            groups[g].append(s)
            load[g] += lens[s] + 1
        groups.sort(key=lambda g: -sum(int(lens[s]) for s in g))
        # a worker that dies makes the pool raise (BrokenProcessPool) instead of restarting it
        with ProcessPoolExecutor(workers, mp_context=mp.get_context("spawn"),
                                 initializer=_oracle_worker_init, initargs=(spec,)) as pool:
            list(pool.map(_oracle_worker_run, [[]] * workers))   # workers up and mapped
            t0 = time.perf_counter()
            busy = list(pool.map(_oracle_worker_run, groups))
            dt = time.perf_counter() - t0
    finally:
        for shm in segs:
            shm.close()
            shm.unlink()
    kv = batch.kv_bytes()
    return {"value": round(kv / dt / 1e9, 4), "unit": "GB/s", "cores": workers, "kind": "oracle",
            "sample": f"all {cfg.num_seqs} sequences (all {cfg.num_q_heads} query heads), "
                      f"{kv / 1e6:.1f} MB of KV in {dt:.2f} s, numpy float64, {workers} worker "
                      f"processes of one thread each (cores from sched_getaffinity, at most 16)",
            "seconds": round(dt, 3), "cpu_seconds": round(float(sum(busy)), 2),
            "tokens_per_s": round(cfg.num_seqs / dt, 3)}


def paging_overhead(args, cfg, batch, sets, outs, ws, part, shared, stream):
    """Whole pa_decode calls (attention + merge), HIP events on the launch stream, K calls each:
    paged over the batch as drawn (shuffled placement), paged over a contiguously laid out copy
    (identity tables), and the contiguous twin over that copy (no table at all)."""
    import numpy as np
    import torch

    import paged_kv_cache_384_amd as pa
    from paged_kv_cache_384_amd import workloads as wl
    if shared:
        return {"skipped": "sequences share blocks; a contiguous layout cannot hold the batch"}
    dev = sets[0]["query"].device
    cb = wl.build_batch(wl.config(cfg.name, placement="contiguous"))
    csets = [wl.make_values(cb, device=dev, seed=10 + k, poison_nan=False)
             for k in range(len(sets))]
    bt = torch.from_numpy(batch.block_tables).to(dev)
    cbt = torch.from_numpy(cb.block_tables).to(dev)
    ctx = torch.from_numpy(batch.context_lens).to(dev)
    W = cb.max_blocks_per_seq
    mx = batch.max_context_len

    def paged(k):
        v = sets[k % len(sets)]
        pa.pa_decode(outs[k % len(outs)], v["query"], v["k_pool"], v["v_pool"], bt, ctx,
                     cfg.scale, mx, part, ws)

    def paged_identity(k):
        v = csets[k % len(csets)]
        pa.pa_decode(outs[k % len(outs)], v["query"], v["k_pool"], v["v_pool"], cbt, ctx,
                     cfg.scale, mx, part, ws)

    def twin(k):
        v = csets[k % len(csets)]
        pa.pa_decode_contiguous(outs[k % len(outs)], v["query"], v["k_pool"], v["v_pool"], ctx,
                                cfg.scale, mx, W, part, ws)

    res = {}
    for name, fn in (("paged_shuffled_us", paged), ("paged_identity_us", paged_identity),
                     ("contiguous_us", twin)):
        for k in range(args.warmup):
            fn(k)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        torch.cuda.synchronize()
        for k in range(args.steps):
            evs[k][0].record(stream)
            fn(k)
            evs[k][1].record(stream)
        torch.cuda.synchronize()
        res[name] = round(float(np.mean([a.elapsed_time(b) * 1e3 for a, b in evs])), 2)
    c = res["contiguous_us"]
    res["slowdown_shuffled"] = round(res["paged_shuffled_us"] / c - 1.0, 4)
    res["slowdown_identity"] = round(res["paged_identity_us"] / c - 1.0, 4)
    print(f"[bench] paging overhead: paged (shuffled) {res['paged_shuffled_us']} us, paged "
          f"(identity tables) {res['paged_identity_us']} us, contiguous twin {c} us",
          file=sys.stderr, flush=True)
    del csets
    return res


def swap_rate(cfg, batch, v, stream, reps=5):
    """Every block of the first half of the sequences swapped out to a pinned host pool and back
    into the same GPU blocks (pa_swap_blocks, copy engines over the host link), HIP events on
    the stream; GB/s counts key and value bytes once per direction."""
    import numpy as np
    import torch

    import paged_kv_cache_384_amd as pa
    B = cfg.block_size
    rows = []
    for s_ in range(cfg.num_seqs // 2):
        nb = -(-int(batch.context_lens[s_]) // B)
        rows.extend(batch.block_tables[s_, :nb].tolist())
    gpu_ids = np.array(rows, np.int32)
    n = len(gpu_ids)
    host_shape = (n,) + tuple(v["k_pool"].shape[1:])
    hk = torch.empty(host_shape, dtype=v["k_pool"].dtype, pin_memory=True)
    hv = torch.empty(host_shape, dtype=v["k_pool"].dtype, pin_memory=True)
    out_pairs = np.stack([gpu_ids, np.arange(n, dtype=np.int32)], 1)
    in_pairs = out_pairs[:, ::-1].copy()
    block_bytes = v["k_pool"][0].numel() * v["k_pool"].element_size()
    nbytes = 2 * n * block_bytes
    res = {"blocks": n, "bytes_per_direction": nbytes}
    for name, args_ in (("out", (hk, hv, v["k_pool"], v["v_pool"], out_pairs)),
                        ("in", (v["k_pool"], v["v_pool"], hk, hv, in_pairs))):
        pa.pa_swap_blocks(*args_, head_dim=cfg.head_dim)
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            pa.pa_swap_blocks(*args_, head_dim=cfg.head_dim)
        b.record(stream)
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / reps
        res[f"{name}_us"] = round(us, 1)
        res[f"{name}_gbps"] = round(nbytes / (us * 1e-6) / 1e9, 2)
    print(f"[bench] swap {n} blocks ({nbytes / 1e6:.1f} MB each way): out {res['out_gbps']} GB/s, "
          f"in {res['in_gbps']} GB/s", file=sys.stderr, flush=True)
    return res


def copy_bandwidth(dev, reps=5):
    """A plain 1 GiB device-to-device copy (read + written bytes / time, HIP events): the
    achievable HBM bandwidth the attention kernel is also compared against."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    b = torch.empty(n, dtype=torch.uint8, device=dev)
    a.fill_(1)
    b.copy_(a)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    s = e0.elapsed_time(e1) * 1e-3 / reps
    del a, b
    torch.cuda.empty_cache()
    return round(2 * n / s / 1e9, 1)


def copy_calibration(dev):
    """Three plain 1 GiB device-to-device copies: the reference for HBM byte counters."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    b = torch.empty(n, dtype=torch.uint8, device=dev)
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(f"[bench] copy calibration: 3 x {n} byte device copies", file=sys.stderr)


MFMA_PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0}  # dense 16-bit matrix-core peak


def prefill_cpu_baseline(batch, v, budget_s: float):
    """The CPU oracle's prefill, single-threaded, on query rows of the longest sequence (4 at a
    time, from its last query down) until ``budget_s`` is spent; flop counted as in the GPU
    figure (4·d per seen token per query head)."""
    from threadpoolctl import threadpool_limits

    import oracle
    cfg = batch.cfg
    kw = dict(dtype=cfg.dtype, num_kv_heads=cfg.num_kv_heads, block_size=cfg.block_size,
              head_dim=cfg.head_dim)
    host = {k: host_storage(v[k]) for k in ("query", "k_pool", "v_pool")}
    s = int(batch.query_lens.argmax())
    n, q = int(batch.context_lens[s]), int(batch.query_lens[s])
    done_rows, flops = 0, 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=1):
        for hi in range(q, 0, -4):
            rows = list(range(max(0, hi - 4), hi))
            oracle.paged_prefill_ref(host["query"], host["k_pool"], host["v_pool"],
                                     batch.block_tables, batch.query_start, batch.context_lens,
                                     cfg.scale, seqs=[s], rows={s: rows}, **kw)
            done_rows += len(rows)
            flops += sum(4 * cfg.head_dim * cfg.num_q_heads * (n - q + j + 1) for j in rows)
            if time.perf_counter() - t0 > budget_s:
                break
    dt = time.perf_counter() - t0
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "sample": f"the last {done_rows} queries of the longest sequence ({n} tokens), all "
                      f"{cfg.num_q_heads} query heads, in {dt:.1f} s, numpy float64, 1 thread"}


def prefill_rate(name, steps, warmup, stream, cpu_budget=0.0, **overrides):
    """pa_prefill on a prefill workload: the new tokens' cache write, then the causal attention
    of every new token, K calls each with HIP events on the launch stream. The attention is two
    dense products per key/value tile on the matrix cores, so its roofline is the 16-bit MFMA
    peak, with the flops counted from the causal definition (no masked or padded work).
    ``overrides`` replace workload fields (block_size, placement)."""
    import numpy as np
    import torch

    import paged_kv_cache_384_amd as pa
    from paged_kv_cache_384_amd import workloads as wl
    cfg = wl.config(name, **overrides)
    batch = wl.build_batch(cfg)
    dev = torch.device("cuda:0")
    v = wl.make_values(batch, device=dev, seed=0, poison_nan=False)
    bt = torch.from_numpy(batch.block_tables).to(dev)
    ctx = torch.from_numpy(batch.context_lens).to(dev)
    qs = torch.from_numpy(batch.query_start).to(dev)
    tseq = torch.from_numpy(batch.token_seq).to(dev)
    tpos = torch.from_numpy(batch.token_pos).to(dev)
    out = torch.empty_like(v["query"])

    def write():
        pa.pa_reshape_and_cache(v["k_pool"], v["v_pool"], v["key"], v["value"], bt, tseq, tpos)

    def attend():
        pa.pa_prefill(out, v["query"], v["k_pool"], v["v_pool"], bt, qs, ctx, cfg.scale,
                      batch.max_query_len, batch.max_context_len)

    for _ in range(max(1, warmup)):
        write()
        attend()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for e in ev:
        e[0].record(stream)
        write()
        e[1].record(stream)
        attend()
        e[2].record(stream)
    torch.cuda.synchronize()
    w_us = float(np.mean([e[0].elapsed_time(e[1]) * 1e3 for e in ev]))
    a_list = [e[1].elapsed_time(e[2]) * 1e3 for e in ev]
    a_us = float(np.mean(a_list))
    flops = batch.attention_flops()
    tf = flops / (a_us * 1e-6) / 1e12
    peak = MFMA_PEAK_TFLOPS[cfg.dtype]
    new_tokens = int(batch.query_lens.sum())
    print(f"[bench] prefill {name}: attention {a_us:.1f} us (p10 {np.percentile(a_list, 10):.1f}, "
          f"p90 {np.percentile(a_list, 90):.1f}) = {tf:.1f} TFLOP/s ({tf / peak:.3f} of peak), "
          f"cache write {w_us:.1f} us", file=sys.stderr, flush=True)
    cpu = prefill_cpu_baseline(batch, v, cpu_budget) if cpu_budget > 0 else None
    return {"workload": name, "description": cfg.description, "dtype": cfg.dtype,
            "block_size": cfg.block_size, "placement": cfg.placement,
            "new_tokens": new_tokens, "context_tokens": int(batch.context_lens.sum()),
            "attention_us": round(a_us, 2), "cache_write_us": round(w_us, 2),
            "tokens_per_s": round(new_tokens / ((a_us + w_us) * 1e-6), 1),
            "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": peak,
                         "unit": "TFLOP/s", "frac": round(tf / peak, 4), "traffic": None,
                         "kernel": "prefill_kernel", "avg_us": round(a_us, 2),
                         "flops_per_launch": flops},
            "cpu_baseline": cpu}


def tile_read_reference(sets, nbytes, tile_bytes, steps, stream):
    """pa_measure_tile_read over as many K+V bytes as ``nbytes``: whole tiles of the workload's
    own pools in a seeded random order, rotating over the input sets like the decode steps, HIP
    events on the stream. What plain reads of the decode access pattern reach at this size."""
    import numpy as np
    import torch

    import paged_kv_cache_384_amd as pa
    pool = sets[0]["k_pool"]
    total = pool.numel() * pool.element_size() // tile_bytes
    n = min(total, max(1, round(nbytes / (2 * tile_bytes))))
    order = np.random.default_rng(1234).permutation(total)[:n].astype(np.int32)
    tiles = torch.from_numpy(order).to(pool.device)
    sink = torch.empty((n + 31) // 32, dtype=torch.int32, device=pool.device)

    def once(k):
        v = sets[k % len(sets)]
        pa.pa_measure_tile_read(v["k_pool"], v["v_pool"], tiles, tile_bytes, sink)

    for k in range(3):
        once(k)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for k in range(steps):
        ev[k][0].record(stream)
        once(k)
        ev[k][1].record(stream)
    torch.cuda.synchronize()
    us = float(np.mean([a.elapsed_time(b) * 1e3 for a, b in ev]))
    read = 2 * n * tile_bytes
    gbps = read / (us * 1e-6) / 1e9
    return {"tiles": n, "tile_bytes": tile_bytes, "bytes": read, "us": round(us, 2),
            "gbps": round(gbps, 1), "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4)}


def decode_rate(name, args, dev, stream, *, part_override=-1, block_size=0, cpu=True,
                paging=False, swap=False, kv_head_shards=1):
    """One decode workload: K eager steps with HIP events around every kernel, then K
    graph-replayed steps, the CPU oracle (one thread on a bounded sample, and every host core on
    the whole batch), and the optional paging-overhead and swap measurements. Returns the
    workload's figures (the headline line is built from the first workload's)."""
    import numpy as np
    import torch

    import paged_kv_cache_384_amd as pa
    from paged_kv_cache_384_amd import workloads as wl
    cfg = wl.CONFIGS[name]
    if block_size and block_size != cfg.block_size:
        cfg = wl.config(name, block_size=block_size, num_blocks=0)
    if kv_head_shards > 1:
        # one GPU's share when the KV heads (and their query heads) are split over that many
        # GPUs: the same sequences, tables and block count, 1/shards of every block's heads
        if cfg.num_kv_heads % kv_head_shards:
            raise SystemExit(f"{name}: {cfg.num_kv_heads} KV heads do not split {kv_head_shards} ways")
        from dataclasses import replace
        cfg = replace(cfg, name=f"{cfg.name}_kvshard{kv_head_shards}",
                      num_q_heads=cfg.num_q_heads // kv_head_shards,
                      num_kv_heads=cfg.num_kv_heads // kv_head_shards,
                      description=f"{cfg.description}; one GPU's share of its KV heads split "
                                  f"{kv_head_shards} ways")
    part = cfg.partition_size if part_override < 0 else part_override
    batch = wl.build_batch(cfg)
    print(f"[bench] {cfg.name}: {cfg.description}", file=sys.stderr, flush=True)

    sets = [wl.make_values(batch, device=dev, seed=k, poison_nan=False) for k in range(args.sets)]
    bt = torch.from_numpy(batch.block_tables).to(dev)
    ctx = torch.from_numpy(batch.context_lens).to(dev)
    tseq = torch.from_numpy(batch.token_seq).to(dev)
    tpos = torch.from_numpy(batch.token_pos).to(dev)
    pairs = torch.from_numpy(batch.copy_pairs.reshape(-1)).to(dev)
    outs = [torch.empty_like(v["query"]) for v in sets]
    # tables that share physical blocks (shared prompts) are read through the caches, and
    # partitions that consecutive sequences share are computed once
    shared = batch.shares_blocks
    ws_bytes = pa.pa_decode_workspace_bytes(sets[0]["k_pool"], cfg.num_seqs, cfg.num_q_heads,
                                            cfg.head_dim, batch.max_context_len, part,
                                            shared_blocks=shared)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    kv_bytes = batch.kv_bytes()
    n_pairs = batch.copy_pairs.shape[0]

    def step(k, ev=None):
        v = sets[k % len(sets)]
        if ev is not None:
            ev[0].record(stream)
        if n_pairs:
            pa.pa_copy_blocks(v["k_pool"], v["v_pool"], pairs, head_dim=cfg.head_dim)
        pa.pa_reshape_and_cache(v["k_pool"], v["v_pool"], v["key"], v["value"], bt, tseq, tpos)
        if ev is not None:
            ev[1].record(stream)
        pa.pa_decode_attention(outs[k % len(sets)], v["query"], v["k_pool"], v["v_pool"], bt, ctx,
                               cfg.scale, batch.max_context_len, part, ws, shared_blocks=shared)
        if ev is not None:
            ev[2].record(stream)
        pa.pa_decode_reduce(outs[k % len(sets)], v["query"], v["k_pool"], v["v_pool"], bt, ctx,
                            cfg.scale, batch.max_context_len, part, ws, shared_blocks=shared)
        if ev is not None:
            ev[3].record(stream)

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()

    # pass 1, eager: K whole steps with HIP events on the launch stream around every kernel, for
    # the per-kernel durations (the attention kernel's average gives the roofline figure)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start.record(stream)
    for k in range(args.steps):
        step(k, evs[k])
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_step_eager = t_start.elapsed_time(t_end) / args.steps
    cache_us = [e[0].elapsed_time(e[1]) * 1e3 for e in evs]
    attn_us = [e[1].elapsed_time(e[2]) * 1e3 for e in evs]
    red_us = [e[2].elapsed_time(e[3]) * 1e3 for e in evs]
    attn_avg = float(np.mean(attn_us))
    # with one partition per context pa_decode_reduce launches nothing: its events then time only
    # the gap between two launches, which is not part of pa_decode
    red_avg = float(np.mean(red_us)) if ws_bytes > 0 else 0.0
    print(f"[bench] {cfg.name}: {args.steps} eager steps {ms_step_eager * 1e3:.1f} us/step; "
          f"attention {attn_avg:.1f} us (p10 {np.percentile(attn_us, 10):.1f}, p90 "
          f"{np.percentile(attn_us, 90):.1f}), reduce {red_avg:.1f} us, cache write "
          f"{np.mean(cache_us):.1f} us", file=sys.stderr, flush=True)

    # pass 2, the timed region: the whole step captured once per input set in a HIP graph (the
    # library allocates nothing and every launch goes to torch's current stream, which is the
    # capture stream), then K replays between two events, synchronised on both sides
    ms_step = ms_step_eager
    if not args.eager:
        graphs = []
        for k in range(len(sets)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(k)
            graphs.append(g)
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()
        g_start = torch.cuda.Event(enable_timing=True)
        g_end = torch.cuda.Event(enable_timing=True)
        g_start.record()
        for k in range(args.steps):
            graphs[k % len(graphs)].replay()
        g_end.record()
        torch.cuda.synchronize()
        ms_step = g_start.elapsed_time(g_end) / args.steps
        del graphs
        print(f"[bench] {cfg.name}: {args.steps} graph-replayed steps {ms_step * 1e3:.1f} "
              "us/step", file=sys.stderr, flush=True)

    unique = batch.unique_kv_bytes()
    # the bytes the attention must bring from HBM: every context token's K and V, counted once
    # per distinct (block, slot) when sequences share blocks
    algo_bytes = unique if shared else kv_bytes
    achieved = algo_bytes / (attn_avg * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": recorded_traffic(cfg.name),
                "kernel": "decode_attention_kernel", "avg_us": round(attn_avg, 2),
                "bytes_per_launch": algo_bytes}
    ref = None
    if kv_bytes >= (64 << 20):  # a latency case below that
        tile_bytes = cfg.block_size * cfg.head_dim * cfg.esz
        ref = tile_read_reference(sets, algo_bytes, tile_bytes, args.steps, stream)
        roofline["reference_gbps"] = ref["gbps"]
        roofline["frac_of_reference"] = round(achieved / ref["gbps"], 4)
        print(f"[bench] {cfg.name}: random-tile read of {ref['bytes'] / 1e9:.3f} GB: "
              f"{ref['us']:.1f} us = {ref['gbps']:.0f} GB/s; attention at "
              f"{roofline['frac_of_reference']:.3f} of it", file=sys.stderr, flush=True)
    decode_us = attn_avg + red_avg
    step_algo_gbps = algo_bytes / (ms_step * 1e-3) / 1e9
    decode_algo_gbps = algo_bytes / (decode_us * 1e-6) / 1e9
    res = {
        "workload": cfg.name, "description": cfg.description, "dtype": cfg.dtype,
        "config": {"workload": cfg.name, "num_seqs": cfg.num_seqs,
                   "num_q_heads": cfg.num_q_heads, "num_kv_heads": cfg.num_kv_heads,
                   "head_dim": cfg.head_dim, "block_size": cfg.block_size,
                   "context_lens": list(cfg.ctx), "num_blocks": batch.num_blocks,
                   "partition_size": part, "max_context_len": batch.max_context_len,
                   "kv_bytes_per_step": kv_bytes, "accumulate": "f32",
                   "copy_pairs": int(n_pairs), "shared_blocks": bool(shared),
                   "blocks_distinct": batch.block_counts()[0],
                   "blocks_if_unshared": batch.block_counts()[1]},
        "step_us": round(ms_step * 1e3, 2),
        "step_us_eager": round(ms_step_eager * 1e3, 2),
        "step_gbps": round(kv_bytes / (ms_step * 1e-3) / 1e9, 1),
        "step_frac_of_peak": round(step_algo_gbps / HBM_PEAK_GBPS, 4),
        "tokens_per_s": round(cfg.num_seqs / (ms_step * 1e-3), 1),
        "kernel_us": {"cache_write_and_copies": round(float(np.mean(cache_us)), 2),
                      "attention": round(attn_avg, 2), "partition_reduce": round(red_avg, 2),
                      "pa_decode": round(decode_us, 2)},
        "pa_decode_gbps": round(kv_bytes / (decode_us * 1e-6) / 1e9, 1),
        "pa_decode_frac_of_peak": round(decode_algo_gbps / HBM_PEAK_GBPS, 4),
        # GB/s fields count every context token's K and V (the metric's KV-read bytes); the
        # fractions of peak count the bytes that must come from HBM (distinct blocks when
        # sequences share them)
        "frac_basis": "unique_kv_bytes" if shared else "kv_bytes",
        "tokens_per_s_attention_only": round(cfg.num_seqs / (decode_us * 1e-6), 1),
        "roofline": roofline,
        "tile_read_reference": ref,
    }
    if shared:
        res["logical_kv_bytes"] = kv_bytes
        res["unique_kv_bytes"] = unique
        res["attention_logical_gbps"] = round(kv_bytes / (attn_avg * 1e-6) / 1e9, 1)
    if swap:
        res["swap"] = swap_rate(cfg, batch, sets[0], stream)
    if paging:
        res["paging_overhead"] = paging_overhead(args, cfg, batch, sets, outs, ws, part, shared,
                                                 stream)
    if cpu:
        host = {n: host_storage(sets[0][n]) for n in ("query", "k_pool", "v_pool")}
        del sets, outs, ws
        torch.cuda.empty_cache()
        one = cpu_baseline(batch, host, args.cpu_budget)
        allc = cpu_baseline_all_cores(batch, host, host_workers())
        allc["one_core"] = one
        res["cpu_baseline"] = allc
        print(f"[bench] {cfg.name}: oracle {allc['value']} GB/s on {allc['cores']} cores, "
              f"{one['value']} GB/s on one", file=sys.stderr, flush=True)
        del host
    else:
        res["cpu_baseline"] = None
        del sets, outs, ws
        torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="opt13b_fp16", help="the headline decode workload")
    ap.add_argument("--also", default="gqa_bf16,long_bf16,cow_fp16,tiny_fp32",
                    help="comma-separated decode workloads measured in the same run and reported "
                         "under 'workloads' (empty for none)")
    ap.add_argument("--partition", type=int, default=-1,
                    help="partition size in tokens for the headline workload; -1 = the "
                         "workload's own setting")
    ap.add_argument("--sets", type=int, default=3, help="rotating input sets")
    ap.add_argument("--kv-head-shards", type=int, default=1,
                    help="time one GPU's share of the --config batch when its KV heads are split "
                         "this many ways (tensor parallelism over heads); the one-GPU run "
                         "measures that share at its real shape")
    ap.add_argument("--block-size", type=int, default=0,
                    help="run the headline workload at this block size (8, 16 or 32) instead of "
                         "its own; the pool is then sized for the blocks in use (1.25x)")
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of the one-thread oracle sample per workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="time the eager launches only (no HIP-graph replay of the step)")
    ap.add_argument("--paging-overhead", action="store_true",
                    help="also time pa_decode against its contiguous twin (no block table) on a "
                         "contiguously laid out copy of the headline batch")
    ap.add_argument("--swap", action="store_true",
                    help="also time swapping every block of half the sequences out to pinned "
                         "host memory and back (pa_swap_blocks)")
    ap.add_argument("--prefill", default="prefill_bf16",
                    help="comma-separated prefill workloads to time as well (pa_prefill), e.g. "
                         "prefill_bf16,chunked_fp16; empty for none")
    ap.add_argument("--prefill-only", action="store_true",
                    help="time only the --prefill workloads and print their JSON (--block-size "
                         "and --placement then apply to them)")
    ap.add_argument("--placement", default="", choices=["", "shuffled", "contiguous"],
                    help="with --prefill-only: physical block placement of the prefill batch")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path has no multi-GPU mode)", file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    prefill_names = [n for n in args.prefill.split(",") if n]
    if args.prefill_only:
        budget = 0.0 if args.no_cpu_baseline else 5.0
        over = {}
        if args.block_size:
            over.update(block_size=args.block_size, num_blocks=0)
        if args.placement:
            over.update(placement=args.placement)
        res = [prefill_rate(n, args.steps, args.warmup, stream, budget, **over)
               for n in prefill_names]
        if args.copy_calibration:
            copy_calibration(dev)
        print(json.dumps({"prefill": res}), flush=True)
        return

    cpu = not args.no_cpu_baseline
    head = decode_rate(args.config, args, dev, stream, part_override=args.partition,
                       block_size=args.block_size, cpu=cpu, paging=args.paging_overhead,
                       swap=args.swap, kv_head_shards=args.kv_head_shards)
    if args.copy_calibration:
        copy_calibration(dev)
    others = [decode_rate(n, args, dev, stream, cpu=cpu)
              for n in args.also.split(",") if n and n != args.config]
    prefill = [prefill_rate(n, args.steps, args.warmup, stream, 5.0 if cpu else 0.0)
               for n in prefill_names]
    copy_gbps = copy_bandwidth(dev)

    value = head["step_gbps"]
    line = {
        "metric": "pa_decode KV-read HBM GB/s (fraction of MI355X peak) + decode tokens/s",
        "value": value,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["step_us"] / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic",
        "config": head["config"],
        "frac_of_peak": head["step_frac_of_peak"],
        "tokens_per_s": head["tokens_per_s"],
        "tokens_per_s_attention_only": head["tokens_per_s_attention_only"],
        "pa_decode_gbps": head["pa_decode_gbps"],
        "pa_decode_frac_of_peak": head["pa_decode_frac_of_peak"],
        "hbm_copy_gbps": copy_gbps,
        "frac_of_copy": round(value / copy_gbps, 4),
        "launch": "eager" if args.eager else "hip_graph",
        "ms_per_step_eager": round(head["step_us_eager"] / 1e3, 5),
        "kernel_us": head["kernel_us"],
        "roofline": head["roofline"],
        "cpu_baseline": head["cpu_baseline"],
    }
    for key in ("paging_overhead", "swap"):
        if key in head:
            line[key] = head[key]
    if others:
        line["workloads"] = others
    if prefill:
        line["prefill"] = prefill
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
