"""Benchmark: paged decode attention on one MI355X.

One step = one decode step of the whole batch of one layer: kv_append of every
sequence's new token, then paged_decode (partition kernel + reduce kernel),
with the pool, tables, queries and new K/V already resident in device memory.
The host-side allocator work of a step (reserve one slot per sequence and
rebuild the block tables) is timed separately on the CPU and reported beside.

Prints one JSON line.  value = algorithmic KV bytes read per step / step time,
in GB/s (every live K and V element once per sequence).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload mha7b]
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

import workloads as wl  # noqa: E402

HBM_PEAK_GBS = 8000.0
METRIC = "paged decode KV GB/s (% of HBM peak) and decode tokens/s per layer, 1 MI355X"
# sources of each measured kernel (a stored traffic figure is valid while they are unchanged)
KERNEL_SOURCES = {
    "paged_decode_partition": ["paged_kv_cache_152_amd/csrc/decode.hip", "paged_kv_cache_152_amd/csrc/append.hip"],
    "paged_prefill": ["paged_kv_cache_152_amd/csrc/prefill.hip"],
}


def kernel_hash(kernel: str = "paged_decode_partition") -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def traffic_for(workload: str, kernel: str, partition_tokens: int, key: str = "bytes_per_launch"):
    """HBM bytes per launch (`key`: the dominant kernel's, or "call_bytes" for
    every kernel of one library call) from the committed rocprofv3 counter
    summary, if it was taken on the current kernel sources at the same
    partition size; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_hash") != kernel_hash(kernel) or t.get("partition_tokens") != partition_tokens:
        return None
    return t.get(key)


COPY_PROBE_BYTES = 2 << 30     # copy_probe_gbs: bytes read (and written) by each pkv_copy launch
CALL_KERNELS = {"paged_decode_partition": ["paged_decode_plan", "paged_decode_partition", "paged_decode_reduce"],
                "paged_prefill": ["paged_prefill"]}


def _pmc_mean_kib(run_dir: str, counter: str) -> dict:
    """Mean value of `counter` per dispatch, per kernel name, from a rocprofv3
    --pmc run's counter_collection CSV (values summed over a dispatch's rows)."""
    import csv
    import glob
    per = {}
    for path in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                key = (r["Kernel_Name"], r["Dispatch_Id"])
                per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    sums, counts = {}, {}
    for (name, _), v in per.items():
        sums[name] = sums.get(name, 0.0) + v
        counts[name] = counts.get(name, 0) + 1
    return {name: sums[name] / counts[name] for name in sums}


def _match(table: dict, short: str) -> float:
    hits = [v for name, v in table.items() if short in name and (short != "paged_decode_partition" or "plan" not in name)]
    if not hits:
        raise SystemExit(f"no dispatches of {short} in the counter run")
    return float(np.mean(hits))


def traffic_summary(args) -> None:
    """--traffic-from FETCH_DIR WRITE_DIR: turn two rocprofv3 counter runs of
    this script on --workload (FETCH_SIZE, then WRITE_SIZE, each its own run)
    into profiles/traffic_<kernel>_<workload>.json.  Each counter is scaled by
    what it reads for pkv_copy in the same run (the copy probe moves
    COPY_PROBE_BYTES each way per launch)."""
    fetch_dir, write_dir = args.traffic_from
    fetch, write = _pmc_mean_kib(fetch_dir, "FETCH_SIZE"), _pmc_mean_kib(write_dir, "WRITE_SIZE")
    kib = COPY_PROBE_BYTES / 1024
    fscale, wscale = kib / _match(fetch, "pkv_copy"), kib / _match(write, "pkv_copy")
    prefill = args.workload.startswith("prefill")
    kernel = "paged_prefill" if prefill else "paged_decode_partition"
    if prefill:
        w = wl.make_prefill(args.workload)
        algo, P = w.kv_bytes(), 0
    else:
        w = wl.make(args.workload)
        algo = w.kv_bytes_per_step()
        import paged_kv_cache_152_amd as pkv
        hp = pkv.KVPool(8, w.H_kv, w.D, w.kv_dtype, host_only=True)
        if args.partition:
            hp.set_partition(args.partition)
        P = hp.partition_tokens(w.B, w.H_q, w.max_len())
        hp.close()
    per_kernel = {}
    for k in CALL_KERNELS[kernel]:
        try:
            f, wr = _match(fetch, k) * 1024 * fscale, _match(write, k) * 1024 * wscale
        except SystemExit:
            continue                               # a kernel this call did not launch (one partition)
        per_kernel[k] = {"fetch_bytes": round(f), "write_bytes": round(wr)}
    main = per_kernel[kernel]
    call = sum(v["fetch_bytes"] + v["write_bytes"] for v in per_kernel.values())
    out = {"kernel": kernel, "workload": args.workload, "kernel_hash": kernel_hash(kernel), "partition_tokens": P,
           "bytes_per_launch": main["fetch_bytes"] + main["write_bytes"], "call_bytes": call,
           "per_kernel": per_kernel, "algorithmic_bytes_per_launch": algo,
           "traffic_over_algorithmic": round((main["fetch_bytes"] + main["write_bytes"]) / algo, 5),
           "call_traffic_over_algorithmic": round(call / algo, 5),
           "fetch_scale": round(fscale, 5), "write_scale": round(wscale, 5),
           "calibration": f"pkv_copy of {COPY_PROBE_BYTES >> 30} GiB in the same runs: FETCH_SIZE "
                          f"{_match(fetch, 'pkv_copy'):.1f} KiB, WRITE_SIZE {_match(write, 'pkv_copy'):.1f} KiB per launch",
           "commands": [f"rocprofv3 --pmc {c} --output-format csv -d {d} -o run -- python -u bench.py "
                        f"--workload {args.workload} --steps 5 --warmup 2 --no-cpu-baseline"
                        + ("" if prefill else " --no-companion")
                        for c, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir))]}
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{args.workload}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(path, json.dumps({k: out[k] for k in ("bytes_per_launch", "call_bytes", "traffic_over_algorithmic")}))


def host_alloc_us(w: wl.Workload, reps: int = 20) -> float:
    """CPU cost of one decode step's bookkeeping (reserve 1 slot per sequence,
    rebuild the block tables) on a metadata-only pool of the same shape."""
    import paged_kv_cache_152_amd as pkv
    pool = pkv.KVPool(w.num_blocks + w.B * (reps + 1), w.H_kv, w.D, w.kv_dtype, host_only=True)
    seqs = [pool.seq_create() for _ in range(w.B)]
    for s, n in zip(seqs, w.lens):
        pool.seq_reserve(s, int(n) - 1)
    mb = w.max_blocks_per_seq() + reps
    t0 = time.perf_counter()
    for _ in range(reps):
        pool.batch_reserve(seqs)
        pool.block_tables(seqs, mb)
    dt = (time.perf_counter() - t0) / reps
    pool.close()
    return dt * 1e6


def per_step_us(torch, prep, out, ws, stream, n: int, mode: str) -> dict:
    """p10 / p50 / p90 of single steps, each between its own event pair on the
    library's stream.  Between steps, outside the events:
      warm         nothing (the steps run back to back);
      cold         a 1 GiB scratch buffer is written and then read, so the
                   256 MB last-level cache (MALL) holds none of the previous
                   step's K/V and no dirty lines;
      after_write  the 1 GiB write alone: the step then also competes with the
                   write-back of the dirty lines the fill left in the caches."""
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda") if mode != "warm" else None
    evs = []
    for i in range(n):
        if mode != "warm":
            scratch.fill_(i & 0xFF)
        if mode == "cold":
            scratch.sum(dtype=torch.int64)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        prep.step(out=out, workspace=ws)
        b.record(stream)
        evs.append((a, b))
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
    del scratch
    return {k: round(float(np.percentile(us, q)), 2) for k, q in (("p10", 10), ("p50", 50), ("p90", 90))}


def copy_probe_gbs(nbytes: int = 2 << 30, reps: int = 10) -> float:
    """Practical HBM rate of a plain device copy (pkv_copy, 16-byte loads and
    stores): (bytes read + bytes written) / time, median of `reps` copies."""
    import torch
    import paged_kv_cache_152_amd as pkv
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    pkv.copy(dst, src)
    times = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        pkv.copy(dst, src)
        b.record()
        b.synchronize()
        times.append(a.elapsed_time(b) * 1e-3)
    del src, dst
    return 2 * nbytes / float(np.median(times)) / 1e9


def read_probe_gbs(nbytes: int = 2 << 30, reps: int = 10, fill: str = "normal_f16") -> dict:
    """HBM read rate of pkv_read_probe (16-byte loads, four or, gathered, eight
    4 KiB loads in flight per workgroup, two workgroups per CU), plain and with
    the nontemporal hint:
    bytes read / time, median of `reps` passes each (one event pair per pass).
    "plain" / "nontemporal" read the buffer in address order; "gather_4KiB" and
    "gather_32KiB" read it in chunks of that size in a seeded random order, as
    the decode kernels read their tiles (one KV head's 16-token tile of a
    128-dim 16-bit cache is 4 KiB; one block of eight such heads is 32 KiB).
    The rate depends on the bytes read, so `fill` picks them: "normal_f16"
    (seeded N(0,1) half floats, what the fp16 decode workloads cache),
    "uniform_u8" (seeded uniform random bytes) or "constant" (every byte 0x01)."""
    import torch
    import paged_kv_cache_152_amd as pkv
    g = torch.Generator(device="cuda").manual_seed(1)
    if fill == "normal_f16":
        src = torch.randn(nbytes // 2, dtype=torch.float16, device="cuda", generator=g).view(torch.uint8)
    elif fill == "uniform_u8":
        src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=g)
    elif fill == "constant":
        src = torch.full((nbytes,), 1, dtype=torch.uint8, device="cuda")
    else:
        raise ValueError(f"unknown fill {fill!r}")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    orders = {c: torch.from_numpy(np.random.default_rng(c).permutation(nbytes // c).astype(np.int32)).cuda()
              for c in (4096, 32768)}
    cases = [("plain", False, None), ("nontemporal", True, None)]
    for c in (4096, 32768):
        cases += [(f"gather_{c // 1024}KiB_plain", False, c), (f"gather_{c // 1024}KiB_nontemporal", True, c)]
    out = {}
    for name, nt, chunk in cases:
        kw = {} if chunk is None else {"order": orders[chunk], "chunk_bytes": chunk}
        pkv.read_probe(src, sink, nt, **kw)
        times = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            pkv.read_probe(src, sink, nt, **kw)
            b.record()
            b.synchronize()
            times.append(a.elapsed_time(b) * 1e-3)
        out[name] = round(nbytes / float(np.median(times)) / 1e9, 1)
    del src, sink, orders
    return out


def cpu_baseline(w: wl.Workload, budget_s: float = 15.0):
    """The fp64 oracle on a bounded sample of the same workload, timed on the host.

    The oracle spreads (sequence, KV head) pairs over its threads, so each call
    gets enough sequences to give every thread at least two pairs."""
    import oracle
    from tests.oracle_ref import fp8_codes, int8_values
    order = np.random.default_rng(0).permutation(w.B)
    threads = oracle.num_threads()
    group = max(1, min(w.B, -(-2 * threads // w.H_kv)))
    scales = w.fp8_scales()
    kw = dict(k_scale=scales[0], v_scale=scales[1]) if scales else {}
    q_all = w.q()
    lens = w.step_lens()
    # one seeded group of sequences, generated once (not timed), decoded repeatedly
    seqs = [int(b) for b in order[:group]]
    Ks, Vs, offs, ns, off = [], [], [], [], 0
    kv_code = oracle.F64 if w.kv_dtype == wl.INT8 else w.kv_dtype
    for b in seqs:
        n = int(lens[b])
        if w.kv_dtype == wl.INT8:            # the values the pool's codes stand for
            K, V = int8_values(w, b, n)
        else:
            K, V = w.kv(b)
            K, V = K[:n], V[:n]
        if w.kv_dtype == wl.E4M3:
            K, V = fp8_codes(K, scales[0]), fp8_codes(V, scales[1])
        Ks.append(K)
        Vs.append(V)
        offs.append(off)
        ns.append(n)
        off += n
    K, V = np.concatenate(Ks), np.concatenate(Vs)
    q = q_all[seqs]
    done_time, calls = 0.0, 0
    while done_time < budget_s:
        t0 = time.perf_counter()
        oracle.decode_attention(q, w.q_dtype, K, V, kv_code, offs, ns, w.scale, **kw)
        done_time += time.perf_counter() - t0
        calls += 1
    done_bytes = calls * w.kv_bytes(ns)
    return {"value": round(done_bytes / done_time / 1e9, 4), "unit": "GB/s",
            "cores": min(threads, group * w.H_kv), "kind": "oracle",
            "sample": f"fp64 oracle, {calls} calls each decoding the same {group} of the {w.B} sequences "
                      f"(seeded choice, {sum(ns)} context tokens; {done_bytes / 2**30:.2f} GiB of KV in "
                      f"{done_time:.1f} s of CPU time); KV GB/s at the same algorithmic bytes as value"}


PREFILL_METRIC = "paged chunked-prefill attention TFLOP/s (algorithmic, causal), 1 MI355X"
MFMA_BF16_PEAK_TFLOPS = 2500.0


def bench_prefill(args):
    """Multi-query attention over the paged cache: one step = kv_append of every
    sequence's chunk + paged_prefill of the chunk (queries attend causally to the
    cached tokens and to the chunk).  value = algorithmic flops / step time."""
    w = wl.make_prefill(args.workload)
    result = measure_prefill(w, args)
    # the plain copy kernel whose FETCH_SIZE / WRITE_SIZE calibrate the traffic counters of a run
    result["copy_probe_GBps"] = round(copy_probe_gbs(), 1)
    result["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline_prefill(w, args.cpu_budget)
    print(json.dumps(result), flush=True)


def measure_prefill(w, args) -> dict:
    """Fill a pool with prefill workload w, time K steps (after W warm-ups), then
    the same K steps again with per-kernel events.  Returns the bench record
    without the copy probe and the CPU baseline."""
    import torch
    import harness
    import paged_kv_cache_152_amd as pkv

    log(f"[bench] workload {w.name}: B={w.B} H_q={w.H_q} H_kv={w.H_kv} D={w.D} "
        f"cached={w.cached} chunk={w.chunk} blocks={w.num_blocks}")
    order = np.random.default_rng(w.seed).permutation(w.num_blocks)
    pool = pkv.KVPool(w.num_blocks, w.H_kv, w.D, w.kv_dtype, free_order=order)
    if args.partition:
        pool.set_partition(args.partition)
    scales = w.fp8_scales()
    if scales is not None:
        pool.set_fp8_scales(*scales)
    seqs, cs, kc, vc = [], [], [], []
    for bi in range(w.B):
        K, V = w.kv(bi)
        s = pool.seq_create()
        seqs.append(s)
        slots = pool.seq_reserve(s, w.n)
        pool.append(torch.from_numpy(slots[: w.cached]).cuda(), harness.to_device(K[: w.cached], w.src_dtype),
                    harness.to_device(V[: w.cached], w.src_dtype))
        cs.append(slots[w.cached:])
        kc.append(K[w.cached:])
        vc.append(V[w.cached:])
    slots_d = torch.from_numpy(np.concatenate(cs)).cuda()
    k_d = harness.to_device(np.concatenate(kc), w.src_dtype)
    v_d = harness.to_device(np.concatenate(vc), w.src_dtype)
    q = harness.to_device(w.q(), w.src_dtype)
    out = torch.empty_like(q)
    q_start = torch.arange(0, (w.B + 1) * w.chunk, w.chunk, dtype=torch.int32, device="cuda")
    tables, lens = pool.block_tables(seqs, -(-w.n // wl.BLOCK))
    tables, lens = torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda()

    def step():
        pool.append(slots_d, k_d, v_d)
        pool.prefill(q, q_start, tables, lens, w.chunk, w.scale, causal=w.causal, out=out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_step = ev0.elapsed_time(ev1) / args.steps
    pool.profile_enable(True)
    pool.profile_read()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    stats = pool.profile_read()
    pool.profile_enable(False)
    pool.close()
    kern = {k: {"launches": v["launches"], "timed": v["launches"] - v["dropped"],
                "avg_us": round(v["total_ms"] / max(1, v["launches"] - v["dropped"]) * 1e3, 3)}
            for k, v in stats.items()}
    flops = w.flops()
    pre_us = kern["paged_prefill"]["avg_us"]
    achieved = flops / (pre_us * 1e-6) / 1e12
    log(f"[bench] {ms_step * 1e3:.1f} us/step, paged_prefill {pre_us:.1f} us = {achieved:.1f} TFLOP/s")
    result = {
        "metric": PREFILL_METRIC,
        "value": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.DTYPE_NAMES[w.kv_dtype],
        "data": "synthetic (seeded N(0,1) K/V and q; block tables from a seeded permutation of the pool)",
        "config": {"workload": w.name, "batch": w.B, "q_heads": w.H_q, "kv_heads": w.H_kv, "head_dim": w.D,
                   "block_size": wl.BLOCK, "kv_dtype": wl.DTYPE_NAMES[w.kv_dtype], "cached_tokens": w.cached,
                   "chunk_tokens": w.chunk, "causal": w.causal, "layers": 1},
        "flops_per_step": flops,
        "prefill_tokens_per_s_per_layer": round(w.B * w.chunk / (ms_step * 1e-3), 1),
        "kernels_us": kern,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": traffic_for(w.name, "paged_prefill", 0), "kernel": "paged_prefill",
                     "algorithmic_flops_per_launch": flops,
                     "timing": "a HIP event pair per launch on the library's stream, recorded by the kernel's own "
                               "start and end (hipExtLaunchKernel), over a second pass of the same K steps"},
        "kernel_hash": kernel_hash("paged_prefill"),
    }
    return result


def cpu_baseline_prefill(w, budget_s: float = 15.0):
    """The fp64 oracle's prefill attention on a bounded sample: the last 64 query
    rows of a chunk, per sequence, over 2 sequences per call."""
    import oracle
    from tests.oracle_ref import fp8_codes
    rows, group = 64, 2
    Ks, Vs, qs = [], [], []
    qall = w.q()
    scales = w.fp8_scales()
    kw = dict(k_scale=scales[0], v_scale=scales[1]) if scales is not None else {}
    for bi in range(group):
        K, V = w.kv(bi)
        if scales is not None:                 # the codes the pool holds
            K, V = fp8_codes(K, scales[0]), fp8_codes(V, scales[1])
        Ks.append(K)
        Vs.append(V)
        qs.append(qall[(bi + 1) * w.chunk - rows:(bi + 1) * w.chunk])
    K, V, q = np.concatenate(Ks), np.concatenate(Vs), np.concatenate(qs)
    q_start = np.arange(0, (group + 1) * rows, rows, dtype=np.int64)
    off = np.arange(group, dtype=np.int64) * w.n
    lens = np.full(group, w.n, np.int32)
    visible = sum(w.n - rows + i + 1 for i in range(rows)) if w.causal else rows * w.n
    flops_call = group * w.H_q * visible * 4 * w.D
    done, calls = 0.0, 0
    while done < budget_s:
        t0 = time.perf_counter()
        oracle.prefill_attention(q, w.src_dtype, q_start, K, V, w.kv_dtype, off, lens, w.scale, causal=w.causal, **kw)
        done += time.perf_counter() - t0
        calls += 1
    return {"value": round(calls * flops_call / done / 1e12, 6), "unit": "TFLOP/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"fp64 oracle, {calls} calls each attending the last {rows} chunk rows of {group} of the "
                      f"{w.B} sequences over their {w.n}-token contexts ({done:.1f} s of CPU time); TFLOP/s at "
                      f"the same algorithmic flops per row as value"}


SWAP_METRIC = "sequence swap-out + swap-in GB/s (host <-> HBM, pinned), 1 MI355X"


def bench_swap(args):
    """Swap one long sequence out to pinned host memory and back, K times.
    value = bytes moved (out + in) / time of the pair.  Each call is
    synchronous, so host wall time brackets it."""
    import torch
    import harness
    import paged_kv_cache_152_amd as pkv
    H_kv, D, n = 8, 128, 32768                       # one Llama-3-8B-shaped layer, 32K context, bf16
    nb = -(-n // wl.BLOCK)
    pool = pkv.KVPool(nb + 8, H_kv, D, pkv.BF16, free_order=np.random.default_rng(8).permutation(nb + 8))
    s = pool.seq_create()
    slots = torch.from_numpy(pool.seq_reserve(s, n)).cuda()
    kv = torch.randn(n, H_kv, D, device="cuda").to(torch.bfloat16)
    pool.append(slots, kv, kv)
    torch.cuda.synchronize()
    nbytes = pool.swap_bytes(s)
    host = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    for _ in range(args.warmup):
        pool.swap_out(s, host)
        pool.swap_in(s, host)
    t_out = t_in = 0.0
    for _ in range(args.steps):
        t0 = time.perf_counter()
        pool.swap_out(s, host)
        t1 = time.perf_counter()
        pool.swap_in(s, host)
        t2 = time.perf_counter()
        t_out += t1 - t0
        t_in += t2 - t1
    pool.close()
    step = (t_out + t_in) / args.steps
    result = {"metric": SWAP_METRIC, "value": round(2 * nbytes / step / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
              "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step * 1e3, 4),
              "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
              "data": "synthetic (random bf16 K/V)",
              "config": {"workload": "swap", "kv_heads": H_kv, "head_dim": D, "tokens": n, "bytes_each_way": nbytes},
              "swap_out_GBps": round(nbytes * args.steps / t_out / 1e9, 2),
              "swap_in_GBps": round(nbytes * args.steps / t_in / 1e9, 2),
              "roofline": None, "cpu_baseline": None}
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100,
                    help="untimed steps first; the FP8 and INT8 workloads need about 40 and 90 to reach steady state")
    ap.add_argument("--workload", default="mha7b", choices=["tiny", "mha7b", "gqa8b", "mixed", "fp8", "int8", "prefill8b", "prefill8b_fp8", "swap"])
    ap.add_argument("--partition", type=int, default=0, help="partition tokens (0 = library default)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-companion", action="store_true",
                    help="mha7b: skip the gqa8b and prefill8b figures that are otherwise measured in the same run")
    ap.add_argument("--probes-only", action="store_true",
                    help="time only the copy probe and the streaming-read probe (2 GiB, three fills) and print them")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the workload's traffic summary from two rocprofv3 counter runs, then exit (no GPU)")
    args = ap.parse_args()
    if args.traffic_from:
        return traffic_summary(args)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this library has no multi-GPU path "
              "(each GPU would own its own pool and sequences); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.probes_only:
        reads = {f: read_probe_gbs(fill=f) for f in ("normal_f16", "uniform_u8", "constant")}
        print(json.dumps({"copy_probe_GBps": round(copy_probe_gbs(), 1), "read_probe_GBps": reads}), flush=True)
        return
    if args.workload.startswith("prefill"):
        return bench_prefill(args)
    if args.workload == "swap":
        return bench_swap(args)

    w = wl.make(args.workload)
    result = measure_decode(w, args)
    if args.workload == "mha7b" and not args.no_companion:
        # the second target shape, measured in the same run (no CPU leg, no copy probe)
        g = measure_decode(wl.make("gqa8b"), args, spread=False)
        result["companion"] = {"gqa8b": {k: g[k] for k in (
            "value", "unit", "ms_per_step", "pct_of_hbm_peak", "decode_tokens_per_s_per_layer", "kv_bytes_per_step",
            "decode_only_us", "kernels_us", "roofline", "partition_kernel", "config")}}
        log(f"[bench] gqa8b: {g['ms_per_step'] * 1e3:.1f} us/step, paged_decode {g['decode_only_us']:.1f} us "
            f"= {100 * g['roofline']['frac']:.1f}% of 8 TB/s")
        # chunked prefill on the GQA shape, the matrix-core kernel (no CPU leg)
        pf = measure_prefill(wl.make_prefill("prefill8b"), args)
        result["companion"]["prefill8b"] = {k: pf[k] for k in (
            "metric", "value", "unit", "ms_per_step", "flops_per_step", "kernels_us", "roofline", "config")}
    result["copy_probe_GBps"] = round(copy_probe_gbs(), 1)
    log(f"[bench] plain copy kernel: {result['copy_probe_GBps']} GB/s (read + write)")
    result["read_probe_GBps"] = read_probe_gbs()
    log(f"[bench] read probe (GB/s): {result['read_probe_GBps']}")
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample")
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


def measure_decode(w: wl.Workload, args, spread: bool = True) -> dict:
    """Fill a pool with workload w, time K decode steps (after W warm-ups), then
    the same K steps again with per-kernel events.  Returns the bench record
    without the copy probe and the CPU baseline."""
    import torch
    import harness

    log(f"[bench] workload {w.name}: B={w.B} H_q={w.H_q} H_kv={w.H_kv} D={w.D} "
        f"kv={wl.DTYPE_NAMES[w.kv_dtype]} blocks={w.num_blocks} tokens={int(w.lens.sum())}")
    t0 = time.time()
    prep = harness.prepare(w, partition_tokens=args.partition)
    torch.cuda.synchronize()
    log(f"[bench] pool filled in {time.time() - t0:.1f} s")
    pool = prep.pool
    out = torch.empty_like(prep.q)
    ws_bytes = pool.workspace_bytes(w.B, w.H_q, prep.max_len)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")
    P = pool.partition_tokens(w.B, w.H_q, prep.max_len)

    for _ in range(args.warmup):
        prep.step(out=out, workspace=ws)
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({args.warmup} steps), timing {args.steps} steps")

    # Timed region: K steps bracketed by two events on the library's stream.
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        prep.step(out=out, workspace=ws)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = ev0.elapsed_time(ev1) / args.steps
    log(f"[bench] {ms_step * 1e3:.1f} us/step (wall {wall / args.steps * 1e6:.1f} us/step)")
    # Per-kernel durations: the same K steps again, each kernel recording an
    # event pair at its own start and end.  Kept out of the pass that gives
    # value all the same, so that nothing but the steps runs in that region.
    pool.profile_enable(True)
    pool.profile_read()
    torch.cuda.synchronize()
    for _ in range(args.steps):
        prep.step(out=out, workspace=ws)
    torch.cuda.synchronize()
    stats = pool.profile_read()
    pool.profile_enable(False)
    graph = graph_steps(torch, prep, out, ws, stream, args.steps, w.kv_bytes_per_step())
    step_dist = None
    if spread:
        step_dist = {m: per_step_us(torch, prep, out, ws, stream, args.steps, m) for m in ("warm", "cold", "after_write")}
        log("[bench] per-step p10/p50/p90 (us): " +
            ", ".join(f"{m} {d['p10']}/{d['p50']}/{d['p90']}" for m, d in step_dist.items()))

    kv_bytes = w.kv_bytes_per_step()
    kern = {k: {"launches": v["launches"], "timed": v["launches"] - v["dropped"],
                "avg_us": round(v["total_ms"] / max(1, v["launches"] - v["dropped"]) * 1e3, 3)}
            for k, v in stats.items()}
    part_us = kern.get("paged_decode_partition", {}).get("avg_us")
    red_us = kern.get("paged_decode_reduce", {}).get("avg_us", 0.0)
    plan_us = kern.get("paged_decode_plan", {}).get("avg_us", 0.0)
    decode_us = (part_us or 0) + (red_us or 0) + plan_us
    achieved = kv_bytes / (decode_us * 1e-6) / 1e9 if decode_us else None
    part_gbs = kv_bytes / (part_us * 1e-6) / 1e9 if part_us else None
    traffic = traffic_for(w.name, "paged_decode_partition", P)
    call_traffic = traffic_for(w.name, "paged_decode_partition", P, "call_bytes")
    result = {
        "metric": METRIC,
        "value": round(kv_bytes / (ms_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.DTYPE_NAMES[w.kv_dtype],
        "data": "synthetic (seeded N(0,1) K/V and q; block tables from a seeded permutation of the pool)",
        "config": {"workload": w.name, "batch": w.B, "q_heads": w.H_q, "kv_heads": w.H_kv, "head_dim": w.D,
                   "block_size": wl.BLOCK, "kv_dtype": wl.DTYPE_NAMES[w.kv_dtype],
                   "q_dtype": wl.DTYPE_NAMES[w.q_dtype], "context_min": int(w.step_lens().min()),
                   "context_max": int(w.step_lens().max()), "context_tokens": int(w.step_lens().sum()),
                   "pool_blocks": w.num_blocks, "partition_tokens": P, "layers": 1},
        "decode_tokens_per_s_per_layer": round(w.B / (ms_step * 1e-3), 1),
        "kv_bytes_per_step": kv_bytes,
        "pct_of_hbm_peak": round(100 * kv_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
        "kernels_us": kern,
        "decode_only_us": round(decode_us, 3),
        "step_us": step_dist,
        "host_alloc_us_per_step": round(host_alloc_us(w), 2) if spread else None,
        # paged_decode as a whole: the plan, partition and reduce kernels of one
        # call, each timed by its own kernel-recorded event pair, summed
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2) if achieved else None, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4) if achieved else None,
                     "traffic": call_traffic, "kernel": "paged_decode (plan + partition + reduce)",
                     "algorithmic_bytes_per_launch": kv_bytes,
                     "timing": "a HIP event pair per kernel on the library's stream, recorded by the kernel's own "
                               "start and end (hipExtLaunchKernel), over a second pass of the same K steps; the "
                               "call's kernels summed"},
        # the partition kernel alone (the one that streams the K/V bytes)
        "partition_kernel": {"kernel": "paged_decode_partition", "avg_us": part_us,
                             "achieved": round(part_gbs, 2) if part_gbs else None,
                             "frac": round(part_gbs / HBM_PEAK_GBS, 4) if part_gbs else None,
                             "traffic": traffic},
        "kernel_hash": kernel_hash(),
        "graph": graph,
    }
    pool.close()
    return result


def graph_steps(torch, prep, out, ws, stream, n: int, kv_bytes: int):
    """The same step captured once into a HIP graph (through torch) and replayed
    n times between two events: the per-step figure without host launch cost.
    Reported beside value, which stays the eagerly launched step."""
    try:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            prep.step(out=out, workspace=ws)
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / n
        del g
        log(f"[bench] graph replay: {ms * 1e3:.1f} us/step")
        return {"ms_per_step": round(ms, 5), "value": round(kv_bytes / (ms * 1e-3) / 1e9, 2),
                "how": "one step (kv_append + paged_decode) captured with torch.cuda.graph, replayed back to back"}
    except Exception as e:                      # capture refused: report, do not fail the bench
        log(f"[bench] graph capture failed: {e}")
        return None


if __name__ == "__main__":
    main()
