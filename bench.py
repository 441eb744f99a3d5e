"""Benchmark of one paged decode step on one MI355X.

A step is the whole hot path for one batch: the append of every request's
new K/V and paged decode attention (pkv_decode_step: the partition kernel,
which also performs the append, + split-K combine) for one layer (or every
layer of the ``shared_prefix`` workload).  Inputs are
seeded synthetic draws resident in HBM before the timed region.  To keep the
256 MB last-level cache from serving repeated reads, single-layer workloads
rotate over ``--rotate`` copies of the KV pools (same tables, different
buffers); the 32-layer workload rotates by itself.

Prints ONE JSON line on stdout (diagnostics go to stderr).  ``value`` is the
achieved algorithmic GB/s of the whole step, over exactly K timed steps
between two synchronizations, timed by a HIP event pair on the stream around
them (the host's wall clock over the same region is in
``config.wall_us_per_step_per_layer``); ``roofline`` reports the
partition kernel alone, timed with HIP events on the stream it runs on;
``cpu_baseline`` times the float64 CPU oracle on a bounded sample of the
same workload, on one core and (``all_cores``) on every allowed core;
``also_measured`` holds the step and kernel figures of the other target
workloads (``--also``, by default the 32K-context batch) from the same run.
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

METRIC = "paged GQA decode attn: achieved HBM GB/s (% of peak) + µs/step per layer"
PEAK_GBS = 8000.0   # MI355X HBM3E, vendor figure
KERNEL_SOURCES = ["decode_mfma.hip", "mfma_tiles.h", "decode_generic.hip", "pkv_device.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "paged_kv_cache_105_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, partition: int):
    """HBM bytes per launch of the partition kernel from the committed
    rocprofv3 counter summary, if it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"pmc_decode_{workload}.md")
    if not os.path.exists(path):
        return None
    m = re.search(r"```json\n(.*?)\n```", open(path).read(), re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("kernel_source_digest") != kernel_source_digest():
        return None
    if rec.get("partition_tokens") != partition:
        return None
    return rec.get("hbm_bytes_per_launch")


def gather_reference(w, pools, stream, steps, waves=(512, 1024)):
    """Achieved bandwidth of a compute-free read of exactly the K/V tiles one
    attention step reads (libpkv_bench.so), timed like the partition kernel,
    the best over the grid sizes in ``waves`` (two waves per CU and one per
    SIMD; 2,048 waves read 1-2% slower than 1,024 on MI355X)."""
    import ctypes as C

    import numpy as np
    import torch

    lib = C.CDLL(os.path.join(ROOT, "paged_kv_cache_105_amd", "libpkv_bench.so"))
    lib.pkvb_gather_read.restype = C.c_int
    lib.pkvb_gather_read.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int64, C.c_int32,
                                     C.c_int32, C.c_void_p, C.c_void_p]
    tile = w.block_size * w.d_h * (2 if w.kv_dtype == "bf16" else 1)
    table = w.block_table.cpu().numpy().astype(np.int64)
    lens = w.context_lens.cpu().numpy()
    offs = []
    for b in range(w.B):
        nb = -(-int(lens[b]) // w.block_size)
        blk = table[b, :nb]
        for h in range(w.H_KV):
            offs.append((blk * w.H_KV + h) * tile)
    offs = torch.from_numpy(np.concatenate(offs)).to(pools[0][0][0].device)
    sink = torch.empty(max(waves) * 64 * 4, dtype=torch.int32, device=offs.device)
    R = len(pools)
    nbytes = 2 * offs.numel() * tile
    best = 0.0
    for W in waves:
        def run(i):
            kc, vc = pools[i % R][0]
            rc = lib.pkvb_gather_read(kc.data_ptr(), vc.data_ptr(), offs.data_ptr(),
                                      offs.numel(), tile, W, sink.data_ptr(), stream.cuda_stream)
            assert rc == 0, rc
        for i in range(3):
            run(i)
        ms = []
        for rep in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for i in range(steps):
                run(i)
            e1.record(stream)
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1) / steps)
        ms.sort()
        gbs = nbytes / (ms[1] * 1e-3) / 1e9
        log(f"compute-free gather, {W} waves: {gbs:.1f} GB/s")
        best = max(best, gbs)
    return round(best, 1)


def host_prefix_identity(block_size: int, prompt_tokens: int = 32768, reps: int = 20):
    """Host cost of prefix reuse for one long prompt: chained block identities
    (the library's SHA-256), a full match against a pool that holds them as
    idle cached blocks (each block leaves the free queue) and the release that
    puts them back.  For scale, the same chain through Python's hashlib
    (OpenSSL) is timed too."""
    import ctypes as C

    import numpy as np

    import paged_kv_cache_105_amd as pkv
    rng = np.random.default_rng(11)
    toks = rng.integers(0, 128_000, prompt_tokens).astype(np.int32)
    h0 = pkv.prefix_root(b"bench;bf16")
    nblk = prompt_tokens // block_size
    t0 = time.perf_counter()
    for _ in range(reps):
        hs = pkv.block_hashes(h0, toks, block_size)
    hash_us = (time.perf_counter() - t0) * 1e6 / reps
    pool = pkv.BlockPool(4 * nblk, block_size)
    row = (C.c_int32 * nblk)()
    n = 0
    for _ in range(nblk):
        n, _, _ = pool.prepare_append(row, n, n * block_size)
    pool.cache_blocks(row, n, nblk * block_size, hs)
    pool.release(row, n)
    t0 = time.perf_counter()
    for _ in range(reps):
        hit = pool.match_prefix(hs, row)
        pool.release(row, hit)
    match_us = (time.perf_counter() - t0) * 1e6 / reps
    if hit != nblk:
        raise RuntimeError(f"prefix match found {hit} of {nblk} blocks")
    raw = toks.astype("<i4").tobytes()
    step = 4 * block_size
    t0 = time.perf_counter()
    h = h0
    for j in range(nblk):
        h = hashlib.sha256(h + raw[j * step:(j + 1) * step]).digest()
    openssl_us = (time.perf_counter() - t0) * 1e6
    if h != hs[-32:]:
        raise RuntimeError("library block identities differ from hashlib's")
    return {"prompt_tokens": prompt_tokens, "blocks": nblk,
            "hash_us": round(hash_us, 1), "hash_blocks_per_s": round(nblk / hash_us * 1e6),
            "match_and_release_us": round(match_us, 1),
            "hashlib_chain_us": round(openssl_us, 1)}


def swap_measurement(w, pool, k_scale, v_scale, stream, dev, reps: int = 5):
    """Swap one layer of a 32,768-token request (2,048 blocks of 16) to
    pinned host memory and back with the library's gather/scatter kernel,
    next to the runtime's DMA copy of the same bytes; and the time these
    rates give for the 4 GiB of all 32 layers, against the page's floors of
    that transfer at 50 and 10 GB/s."""
    import torch

    import paged_kv_cache_105_amd as pkv
    n = min(2048, w.num_blocks)
    kc, vc = pool
    blk, rec = pkv.swap_record_bytes(pkv.dtype_code(kc), w.H_KV, w.d_h, w.block_size)
    ids = torch.arange(n, dtype=torch.int32, device=dev)
    host = torch.empty(n * rec, dtype=torch.uint8, pin_memory=True)
    staged = torch.empty(n * rec, dtype=torch.uint8, device=dev)
    moved = n * 2 * blk + (n * 8 * w.H_KV if w.kv_dtype == "fp8_e4m3" else 0)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    out_ms = timed(lambda: pkv.swap_out(kc, vc, ids, host, k_scale, v_scale, stream=stream))
    in_ms = timed(lambda: pkv.swap_in(kc, vc, ids, host, k_scale, v_scale, stream=stream))
    d2h_ms = timed(lambda: host.copy_(staged, non_blocking=True))
    h2d_ms = timed(lambda: staged.copy_(host, non_blocking=True))
    gbs = lambda nbytes, ms: round(nbytes / (ms * 1e-3) / 1e9, 2)
    full = 32 * moved          # all 32 layers of the request
    res = {"blocks": n, "bytes_per_layer": moved,
           "swap_out_gbs": gbs(moved, out_ms), "swap_in_gbs": gbs(moved, in_ms),
           "dma_d2h_gbs": gbs(n * rec, d2h_ms), "dma_h2d_gbs": gbs(n * rec, h2d_ms),
           "all_layers_bytes": full,
           "all_layers_out_s": round(32 * out_ms * 1e-3, 4),
           "all_layers_in_s": round(32 * in_ms * 1e-3, 4),
           "page_floor_s_at_50GBps": round(full / 50e9, 4),
           "page_floor_s_at_10GBps": round(full / 10e9, 4)}
    log(f"swap of {n} blocks ({moved} B per layer): out {res['swap_out_gbs']} GB/s, in "
        f"{res['swap_in_gbs']} GB/s; DMA copy {res['dma_d2h_gbs']} / {res['dma_h2d_gbs']} GB/s")
    return res


# ---- CPU oracle baselines ---------------------------------------------------
#
# They run before this process touches the GPU: the all-cores figure forks
# worker processes, which is only safe while no device has been opened.  The
# inputs are drawn on the host with the same recipe (lengths and block tables
# are identical; values come from the host generator).

_CPU_DATA = None


def _cpu_workload(name: str):
    import numpy as np

    from paged_kv_cache_105_amd.workloads import as_numpy, make_workload
    w = make_workload(name, layers=1) if name == "shared_prefix" else make_workload(name)
    d = dict(q=as_numpy(w.q[0]), kn=as_numpy(w.k_new[0]), vn=as_numpy(w.v_new[0]),
             kc=as_numpy(w.k_cache[0]).copy(), vc=as_numpy(w.v_cache[0]).copy(),
             table=as_numpy(w.block_table), lens=as_numpy(w.context_lens),
             ks=as_numpy(w.k_scale[0]) if w.k_scale else None,
             vs=as_numpy(w.v_scale[0]) if w.v_scale else None)
    np.ones((2, 2)) @ np.ones((2, 2))   # load BLAS, so that its thread limit applies
    return w, d


def _attend_request(w, d, b):
    from oracle import paged
    from paged_kv_cache_105_amd import metrics
    paged.attend(d["q"], w.q_dtype, d["kc"], d["vc"], w.kv_dtype, d["table"], d["lens"],
                 w.block_size, w.softmax_scale, d["ks"], d["vs"], requests=[b])
    return metrics.attention_bytes([int(d["lens"][b])], w.H_Q, w.H_KV, w.d_h, w.block_size,
                                   w.kv_dtype, w.q_dtype)["total"]


def _cpu_worker(args):
    """One worker of the all-cores run: its share of the requests (b = k,
    k + n, ...), over and over, until the deadline; BLAS on one thread."""
    k, n, deadline = args
    from threadpoolctl import threadpool_limits
    w, d = _CPU_DATA
    nbytes, reqs = 0, 0
    with threadpool_limits(limits=1):
        while time.time() < deadline:
            for b in range(k, w.B, n):
                nbytes += _attend_request(w, d, b)
                reqs += 1
                if time.time() >= deadline:
                    break
    return nbytes, reqs


def cpu_baselines(name: str, budget_1: float, budget_n: float):
    """The oracle as it stands, on a bounded sample of the workload:
    one core (BLAS pinned to one thread): whole decode steps -- the append of
    the batch, then attention request by request -- until ~budget_1 s;
    all allowed cores: one process per core, each attending its share of the
    requests with BLAS on one thread, for ~budget_n s of wall time (the
    append is serial and tiny, so the sample is attention only)."""
    import multiprocessing as mp

    from threadpoolctl import threadpool_limits

    from oracle import paged
    from paged_kv_cache_105_amd import metrics
    global _CPU_DATA
    t_gen = time.perf_counter()
    w, d = _cpu_workload(name)
    log(f"cpu baseline inputs drawn on the host in {time.perf_counter() - t_gen:.1f} s")

    nbytes, passes, reqs = 0, 0, 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < budget_1:
            paged.append(d["kc"], d["vc"], w.kv_dtype, d["kn"], d["vn"], w.q_dtype, d["table"],
                         d["lens"], w.block_size, d["ks"], d["vs"], inplace=True)
            nbytes += metrics.append_bytes(w.B, w.H_KV, w.d_h, w.kv_dtype, w.q_dtype)
            for b in range(w.B):
                nbytes += _attend_request(w, d, b)
                reqs += 1
                if time.perf_counter() - t0 > budget_1:
                    break
            passes += 1
        dt = time.perf_counter() - t0
    one = {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": f"one layer of {name}: {passes} decode step(s) (append of all {w.B} "
                     f"requests, attention of {reqs} request-steps), float64 numpy, BLAS "
                     f"pinned to 1 thread, {dt:.1f} s"}

    allowed = len(os.sched_getaffinity(0))
    # the box's share of host cores (OMP_NUM_THREADS there) caps the workers
    cap = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    n = min(allowed, cap) if cap > 0 else allowed
    _CPU_DATA = (w, d)
    deadline = time.time() + budget_n
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(n) as pool:
        res = pool.map(_cpu_worker, [(k, n, deadline) for k in range(n)])
    dt = time.perf_counter() - t0
    _CPU_DATA = None
    nb = sum(r[0] for r in res)
    rq = sum(r[1] for r in res)
    alln = {"value": round(nb / dt / 1e9, 4), "unit": "GB/s", "cores": n,
            "cores_allowed": allowed, "kind": "oracle",
            "sample": f"one layer of {name}: attention of {rq} request-steps by {n} worker "
                      f"processes (one per core, requests dealt round robin), float64 numpy, "
                      f"BLAS on 1 thread each, {dt:.1f} s wall"}
    log(f"cpu oracle, 1 core: {one['value']} GB/s; {n} cores: {alln['value']} GB/s")
    return one, alln


PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, vendor figure
CHUNK_METRIC = "paged chunk attention: achieved TFLOP/s (% of bf16 MFMA peak) + us/step"


def chunk_flops(lens, qstart, H_Q, d_h) -> float:
    """Algorithmic FLOPs of chunk attention: each new token at position p
    multiplies its query by p + 1 keys and mixes p + 1 values, for every
    query head (2 d_h each)."""
    total = 0
    for b in range(len(lens)):
        n_new, ctx = qstart[b + 1] - qstart[b], lens[b]
        first = ctx - n_new
        # sum over positions first .. ctx - 1 of (p + 1)
        total += (first + 1 + ctx) * n_new // 2
    return 4.0 * d_h * H_Q * total


def chunk_cpu_baseline(name: str, budget_s: float):
    """The oracle's chunk step (append + attention) on one request of the
    same workload, in FLOP/s of chunk attention, on one core."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import paged
    from paged_kv_cache_105_amd.workloads import as_numpy, make_workload
    w = make_workload(name, B=1)
    lens, qs = w.context_lens.tolist(), w.query_start.tolist()
    flops = chunk_flops(lens, qs, w.H_Q, w.d_h)
    d = [as_numpy(t[0]) for t in (w.q, w.k_new, w.v_new, w.k_cache, w.v_cache)]
    np.ones((2, 2)) @ np.ones((2, 2))   # load BLAS, so that its thread limit applies
    runs, t0 = 0, time.perf_counter()
    with threadpool_limits(limits=1):
        while True:
            paged.chunk_step(d[0], w.q_dtype, d[1], d[2], d[3], d[4], w.kv_dtype,
                             as_numpy(w.block_table), np.asarray(lens), np.asarray(qs),
                             w.block_size, w.softmax_scale)
            runs += 1
            if time.perf_counter() - t0 >= budget_s or runs >= 50:
                break
    el = time.perf_counter() - t0
    return {"value": round(flops * runs / el / 1e12, 6), "unit": "TFLOP/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{runs} oracle chunk steps of one request ({qs[1]} new tokens at context "
                      f"{lens[0]}, {w.H_Q} query heads) in {el:.1f} s; float64 numpy, BLAS "
                      f"limited to one thread"}


def chunk_main(args, w, dev):
    """Chunk workloads: one step = chunk append + chunk attention."""
    import torch

    import paged_kv_cache_105_amd as pkv
    pkv.set_decode_variant(args.variant)
    lens, qs = w.context_lens.cpu().tolist(), w.query_start.cpu().tolist()
    R = max(1, min(args.rotate, 2))
    pools = [(w.k_cache[0], w.v_cache[0])] + [(w.k_cache[0].clone(), w.v_cache[0].clone())
                                              for _ in range(R - 1)]
    out = torch.empty((w.total_q, w.H_Q, w.d_h), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    ks = w.k_scale[0] if w.k_scale else None
    vs = w.v_scale[0] if w.v_scale else None

    def attend(r):
        kc, vc = pools[r]
        pkv.paged_chunk_attention(out, w.q[0], kc, vc, w.block_table, w.context_lens,
                                  w.query_start, w.max_q_len, w.max_context_len,
                                  w.softmax_scale, ks, vs, stream=stream)

    def step(r):
        kc, vc = pools[r]
        pkv.kv_append_chunk(w.k_new[0], w.v_new[0], kc, vc, w.block_table, w.context_lens,
                            w.query_start, ks, vs, stream=stream)
        attend(r)

    for i in range(args.warmup):
        step(i % R)
    ms_per_step, wall_ms_per_step = timed_steps(step, args.steps, R, stream)
    kern_ms = []
    n_kern = max(args.steps, 10)
    for rep in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(n_kern):
            attend(i % R)
        e1.record(stream)
        torch.cuda.synchronize()
        kern_ms.append(e0.elapsed_time(e1) / n_kern)
    kern_ms.sort()
    kern_avg_ms = kern_ms[len(kern_ms) // 2]
    flops = chunk_flops(lens, qs, w.H_Q, w.d_h)
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (kern_avg_ms * 1e-3) / 1e12
    kernel = ("chunk_generic_kernel" if args.variant == 1 or w.d_h != 128 or w.block_size != 16
              or w.q_dtype != "bf16" else "chunk_mfma_kernel")
    log(f"chunk step {ms_per_step * 1e3:.1f} us; attention kernel avg {kern_avg_ms * 1e3:.1f} us "
        f"(batches: {', '.join(f'{x * 1e3:.1f}' for x in kern_ms)}); {flops / 1e9:.1f} GFLOP; "
        f"kernel {achieved:.1f} TFLOP/s = {100 * achieved / PEAK_BF16_TFLOPS:.1f}% of peak")
    cpu = None
    if not args.no_cpu_baseline:
        cpu = chunk_cpu_baseline(args.workload, args.cpu_budget)
        log(f"cpu baseline: {cpu}")
    res = {
        "metric": CHUNK_METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "B": w.B, "H_Q": w.H_Q, "H_KV": w.H_KV,
                   "d_h": w.d_h, "block_size": w.block_size, "kv_dtype": w.kv_dtype,
                   "q_dtype": w.q_dtype, "new_tokens": w.total_q,
                   "max_context": w.max_context_len, "shared_blocks": w.shared_blocks,
                   "pool_copies": R, "us_per_step": round(ms_per_step * 1e3, 2),
                   "step_timing": "HIP event pair on the stream around the K timed steps",
                   "wall_us_per_step": round(wall_ms_per_step * 1e3, 2)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": None, "kernel": kernel,
                     "algorithmic_flops_per_launch": flops,
                     "avg_launch_us": round(kern_avg_ms * 1e3, 3)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


def timed_steps(step, steps, R, stream):
    """Run exactly ``steps`` steps (step(i) for pool copy i % R) between two
    synchronizations; returns (ms per step from a HIP event pair on
    ``stream`` around them, ms per step by the host's wall clock over the
    same region)."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        step(i % R)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    return e0.elapsed_time(e1) / steps, wall


def decode_measure(args, name, dev, full=True):
    """Measure one decode workload: the step (append + attention + combine)
    over exactly args.steps steps (HIP events on the stream, and the host's
    wall clock beside them), and the partition kernel alone by HIP events
    around back-to-back launches on its stream.  With ``full``,
    also the reference bandwidths of plain kernels on this machine, the
    compute-free gather of the same tiles, and the optional block-copy and
    calibration measurements.  Returns (record, workload, pools)."""
    import torch

    import paged_kv_cache_105_amd as pkv
    from paged_kv_cache_105_amd import metrics
    from paged_kv_cache_105_amd.workloads import make_workload

    t_gen = time.perf_counter()
    w = make_workload(name, device=dev)
    lens = w.context_lens.cpu().tolist()
    log(f"workload {name}: B={w.B} H_Q={w.H_Q} H_KV={w.H_KV} d_h={w.d_h} "
        f"bs={w.block_size} kv={w.kv_dtype} layers={w.layers} blocks={w.num_blocks} "
        f"max_len={w.max_context_len} (generated in {time.perf_counter() - t_gen:.1f} s)")

    # pools per (rotation, layer)
    R = max(1, args.rotate) if w.layers == 1 else 1
    pools = []
    for r in range(R):
        pools.append([(w.k_cache[L] if r == 0 else w.k_cache[L].clone(),
                       w.v_cache[L] if r == 0 else w.v_cache[L].clone()) for L in range(w.layers)])
    pkv.set_decode_variant(args.variant)  # the plan depends on the variant
    pt, parts, ws_bytes = pkv.decode_plan(w.B, w.H_Q, w.H_KV, w.d_h, w.block_size,
                                          w.max_context_len, args.partition,
                                          pkv.dtype_code(w.q[0]), pkv.dtype_code(w.k_cache[0]))
    # requests that share prefix blocks: the cascade step reads them once
    cascade = w.shared_blocks > 0 and not args.no_cascade and args.variant in (0, 2)
    if cascade:
        splits, cws = pkv.cascade_plan(w.B, w.H_Q, w.H_KV, w.d_h, w.block_size,
                                       w.max_context_len, w.shared_blocks,
                                       pkv.dtype_code(w.q[0]), pkv.dtype_code(w.k_cache[0]))
        ws_bytes = max(ws_bytes, cws)
        log(f"cascade over {w.shared_blocks} shared blocks, {splits} prefix splits")
    work = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    out = torch.empty((w.B, w.H_Q, w.d_h), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    ks = w.k_scale or [None] * w.layers
    vs = w.v_scale or [None] * w.layers

    def step(r):
        # append + attention (+ combine): the append runs inside the attention
        # launch where the MFMA kernels apply
        for L in range(w.layers):
            kc, vc = pools[r][L]
            if cascade:
                pkv.decode_step_cascade(w.k_new[L], w.v_new[L], out, w.q[L], kc, vc,
                                        w.block_table, w.context_lens, w.max_context_len,
                                        w.softmax_scale, w.shared_blocks, ks[L], vs[L],
                                        workspace=work, stream=stream)
            else:
                pkv.decode_step(w.k_new[L], w.v_new[L], out, w.q[L], kc, vc, w.block_table,
                                w.context_lens, w.max_context_len, w.softmax_scale, ks[L],
                                vs[L], partition_tokens=pt, workspace=work, stream=stream)

    for i in range(args.warmup):
        step(i % R)
    torch.cuda.synchronize()

    # timed region 1: exactly K steps between two synchronizations, timed by
    # one HIP event pair on the step's stream around them (the time the GPU
    # spends on the K steps).  The host's wall clock over the same region is
    # reported beside it: it also holds the GPU's start from idle and the
    # final synchronization's wake-up, a fixed ~0.1 ms that weighs on short
    # runs (20 steps: ~7 us per step).
    ms_per_step, wall_ms_per_step = timed_steps(step, args.steps, R, stream)

    # timed region 3 (reported beside the headline, not used for it): the
    # spread of single steps, one HIP event recorded between consecutive
    # steps on the step's stream, so each interval also holds one event
    # record
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(args.steps):
        step(i % R)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = sorted(ev[i].elapsed_time(ev[i + 1]) * 1e3 / w.layers for i in range(args.steps))
    pick = lambda f: per[min(len(per) - 1, int(round(f * (len(per) - 1))))]
    step_dist = {"p10": round(pick(0.1), 2), "p50": round(pick(0.5), 2),
                 "p90": round(pick(0.9), 2), "unit": "us per layer",
                 "method": f"{args.steps} single steps between HIP events on the stream"}

    # timed region 2: the partition kernel alone, launched back to back over
    # the rotating pool copies, one HIP event pair on its stream around the
    # whole batch (per-launch event pairs would add the dispatch latency of
    # each launch to its time); at least 100 launches per batch, so the
    # start of a batch from an idle GPU weighs little
    kern_ms = []
    n_kern = max(args.steps, 100)
    for rep in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(n_kern):
            for L in range(w.layers):
                kc, vc = pools[i % R][L]
                if cascade:
                    pkv.cascade_partitions(out, w.q[L], kc, vc, w.block_table, w.context_lens,
                                           w.max_context_len, w.softmax_scale, w.shared_blocks,
                                           ks[L], vs[L], workspace=work, stream=stream)
                else:
                    pkv.decode_partitions(out, w.q[L], kc, vc, w.block_table, w.context_lens,
                                          w.max_context_len, w.softmax_scale, ks[L], vs[L],
                                          partition_tokens=pt, workspace=work, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        kern_ms.append(e0.elapsed_time(e1) / (n_kern * w.layers))
    kern_ms.sort()
    kern_avg_ms = kern_ms[len(kern_ms) // 2]

    att = metrics.attention_bytes(lens, w.H_Q, w.H_KV, w.d_h, w.block_size, w.kv_dtype,
                                  w.q_dtype)
    logical_bytes = att["total"]
    if cascade:
        # the shared prefix is read once per layer for the whole batch
        att = metrics.cascade_attention_bytes(lens, w.shared_blocks, w.H_Q, w.H_KV, w.d_h,
                                              w.block_size, w.kv_dtype, w.q_dtype)
    app = metrics.append_bytes(w.B, w.H_KV, w.d_h, w.kv_dtype, w.q_dtype)
    step_bytes = w.layers * (att["total"] + app)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = att["total"] / (kern_avg_ms * 1e-3) / 1e9
    traffic = measured_traffic(name, pt)
    log(f"partition={pt} parts={parts} workspace={ws_bytes} B; step {ms_per_step * 1e3:.1f} us "
        f"({ms_per_step * 1e3 / w.layers:.1f} us/layer) = {value:.0f} GB/s = "
        f"{100 * value / PEAK_GBS:.1f}% of peak; partition kernel avg "
        f"{kern_avg_ms * 1e3:.1f} us (batches: {', '.join(f'{x * 1e3:.1f}' for x in kern_ms)}); "
        f"KV bytes/layer {att['kv']}; kernel {achieved:.0f} GB/s = "
        f"{100 * achieved / PEAK_GBS:.1f}% of peak; single steps p10/p50/p90 "
        f"{step_dist['p10']}/{step_dist['p50']}/{step_dist['p90']} us/layer")
    kernel = {0: "decode_mfma_flat_kernel", 1: "decode_generic_kernel",
              2: "decode_mfma_flat_kernel", 3: "decode_mfma_kernel"}[args.variant]
    if cascade:
        kernel = "decode_mfma_flat_kernel (cascade: prefix and private waves)"
    rec = {"value": round(value, 2), "ms_per_step": round(ms_per_step, 5),
           "config": {"workload": name, "B": w.B, "H_Q": w.H_Q, "H_KV": w.H_KV,
                      "d_h": w.d_h, "block_size": w.block_size, "kv_dtype": w.kv_dtype,
                      "q_dtype": w.q_dtype, "layers": w.layers, "partition_tokens": pt,
                      "partitions_max": parts, "pool_copies": R,
                      "cascade_shared_blocks": w.shared_blocks if cascade else 0,
                      "bytes_counted": "unique (shared prefix once per layer)" if cascade
                      else "every request's positions",
                      "logical_bytes_per_layer": logical_bytes,
                      "mean_context": round(sum(lens) / len(lens), 1),
                      "us_per_step_per_layer": round(ms_per_step * 1e3 / w.layers, 2),
                      "pct_of_peak_step": round(100 * value / PEAK_GBS, 2),
                      "step_timing": "HIP event pair on the stream around the K timed steps",
                      "wall_us_per_step_per_layer": round(wall_ms_per_step * 1e3 / w.layers, 2),
                      "step_us_per_layer_spread": step_dist},
           "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_GBS,
                        "unit": "GB/s", "frac": round(achieved / PEAK_GBS, 4),
                        "traffic": traffic, "kernel": kernel,
                        "algorithmic_bytes_per_launch": att["total"],
                        "avg_launch_us": round(kern_avg_ms * 1e3, 3)},
           "dtype": w.kv_dtype}
    if not full:
        return rec, w, pools

    # reference bandwidths of plain torch kernels on this machine (context for the
    # % of peak): a 1 GiB device-to-device copy and a 2 GiB read-only sum
    ref = {}
    x = torch.empty(2 ** 30 // 2, dtype=torch.bfloat16, device=dev).fill_(1.0)
    y = torch.empty_like(x[: 2 ** 29 // 2])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for kind in ("copy", "read"):
        for rep in range(4):
            e0.record(stream)
            if kind == "copy":
                y.copy_(x[: y.numel()])
            else:
                x.sum(dtype=torch.float32)
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
        nbytes = 2 * y.numel() * 2 if kind == "copy" else x.numel() * 2
        ref[f"{kind}_gbs"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    del x, y
    log(f"reference torch kernels: {ref}")

    ref["gather_gbs"] = gather_reference(w, pools, stream, max(args.steps, 100))
    log(f"compute-free gather of the same tiles: {ref['gather_gbs']} GB/s "
        f"(partition kernel at {100 * achieved / ref['gather_gbs']:.1f}% of it)")

    if args.copy_blocks > 0:
        n = min(args.copy_blocks, w.num_blocks // 2)
        gen = torch.Generator(device="cpu")
        gen.manual_seed(11)
        ids = torch.randperm(w.num_blocks, generator=gen)[:2 * n].to(torch.int32)
        pairs = torch.stack([ids[:n], ids[n:]], dim=1).contiguous().to(dev)
        for i in range(3):
            kc, vc = pools[i % R][0]
            pkv.copy_blocks(kc, vc, pairs, ks[0], vs[0], stream=stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(args.steps):
            kc, vc = pools[i % R][0]
            pkv.copy_blocks(kc, vc, pairs, ks[0], vs[0], stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        cms = e0.elapsed_time(e1) / args.steps
        blk = w.H_KV * w.block_size * w.d_h * metrics.DTYPE_BYTES[w.kv_dtype]
        ref["copy_blocks_gbs"] = round(2 * 2 * n * blk / (cms * 1e-3) / 1e9, 1)
        ref["copy_blocks_us"] = round(cms * 1e3, 2)
        log(f"copy_blocks: {n} pairs x {blk} B x (K, V) in {cms * 1e3:.1f} us = "
            f"{ref['copy_blocks_gbs']} GB/s read+write")

    if args.calibrate_copy > 0:
        src = torch.ones(args.calibrate_copy * 2 ** 20 // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: {args.calibrate_copy} MiB read + written, 5 launches")

    rec["config"]["reference_gbs"] = ref
    rec["config"]["pct_of_gather_reference"] = round(100 * achieved / ref["gather_gbs"], 1)
    return rec, w, pools


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama8b")
    ap.add_argument("--also", default="long32k",
                    help="comma-separated decode workloads measured in the same run as "
                         "sub-records (step and kernel figures); empty for none")
    ap.add_argument("--partition", type=int, default=0, help="positions per partition, 0 = default")
    ap.add_argument("--rest", type=float, default=5.0,
                    help="seconds the GPU idles before each --also workload is measured")
    ap.add_argument("--rotate", type=int, default=4, help="KV pool copies for cold-cache timing")
    ap.add_argument("--variant", type=int, default=0, help="0 auto, 1 generic, 2 mfma")
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of the one-core oracle sample")
    ap.add_argument("--cpu-budget-all", type=float, default=6.0,
                    help="wall seconds of the all-cores oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-blocks", type=int, default=0, metavar="N",
                    help="also time pkv_copy_blocks on N random disjoint block pairs")
    ap.add_argument("--no-cascade", action="store_true",
                    help="plain decode steps even where requests share prefix blocks")
    ap.add_argument("--no-swap", action="store_true",
                    help="skip the swap-to-host measurement")
    ap.add_argument("--no-host", action="store_true",
                    help="skip the host prefix-identity measurement")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="after the bench, copy a MIB-sized buffer 5 times (plain copy kernel "
                         "of known size, to scale HBM counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        log(f"bench.py: measures one GPU only (the decode path is not sharded); --gpus {args.gpus} is not supported")
        sys.exit(2)

    from paged_kv_cache_105_amd.workloads import CONFIGS
    chunk = CONFIGS[args.workload].get("lens") in ("fixed_after", "prefix_chunk")

    # the CPU oracle first: its all-cores run forks, before any device use
    cpu = None
    if not args.no_cpu_baseline and not chunk:
        one, alln = cpu_baselines(args.workload, args.cpu_budget, args.cpu_budget_all)
        cpu = dict(one)
        cpu["all_cores"] = alln

    import torch

    import paged_kv_cache_105_amd as pkv
    from paged_kv_cache_105_amd.workloads import make_workload

    pkv.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if chunk:
        w = make_workload(args.workload, device=dev)
        log(f"workload {args.workload}: B={w.B} H_Q={w.H_Q} H_KV={w.H_KV} d_h={w.d_h} "
            f"bs={w.block_size} kv={w.kv_dtype} new tokens={w.total_q}")
        chunk_main(args, w, dev)
        return

    rec, w, pools = decode_measure(args, args.workload, dev, full=True)
    stream = torch.cuda.current_stream()
    ks = w.k_scale or [None] * w.layers
    vs = w.v_scale or [None] * w.layers
    swap = swap_measurement(w, pools[0][0], ks[0], vs[0], stream, dev) if not args.no_swap \
        else None
    del w, pools
    torch.cuda.empty_cache()

    # the other target workloads, measured in the same run.  Each starts from
    # the rested state the first one starts from: after ~10 s of
    # full-bandwidth load the chip runs ~4% slower for a few seconds (a
    # workload measured right after another reads 168-169 us instead of
    # 161.5-162 us on the 32K batch, whichever order), so the GPU idles
    # args.rest seconds first, outside every timed region.
    also = {}
    for name in [x for x in args.also.split(",") if x and x != args.workload]:
        torch.cuda.synchronize()
        time.sleep(max(args.rest, 0.0))
        sub, w2, p2 = decode_measure(args, name, dev, full=False)
        also[name] = {"us_per_step_per_layer": sub["config"]["us_per_step_per_layer"],
                      "step_gbs": sub["value"],
                      "pct_of_peak_step": sub["config"]["pct_of_peak_step"],
                      "step_us_per_layer_spread": sub["config"]["step_us_per_layer_spread"],
                      "kernel_us": sub["roofline"]["avg_launch_us"],
                      "kernel_gbs": sub["roofline"]["achieved"],
                      "kernel_frac": sub["roofline"]["frac"],
                      "traffic": sub["roofline"]["traffic"],
                      "algorithmic_bytes_per_launch":
                          sub["roofline"]["algorithmic_bytes_per_launch"],
                      "config": {k: sub["config"][k] for k in
                                 ("B", "H_Q", "H_KV", "d_h", "block_size", "kv_dtype",
                                  "mean_context", "pool_copies")}}
        del w2, p2
        torch.cuda.empty_cache()

    res = {
        "metric": METRIC,
        "value": rec["value"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": rec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": rec["dtype"],
        "data": "synthetic",
        "config": rec["config"],
        "roofline": rec["roofline"],
        "cpu_baseline": cpu,
        "also_measured": also,
        "host_prefix_identity": None if args.no_host else host_prefix_identity(16),
        "swap_32k_request_layer": swap,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
