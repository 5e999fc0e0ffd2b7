"""Benchmark: one context-parallel rank's ring-attention forward on one MI355X.

A step is one whole pass of the path: cp_attn_rank_forward for the last rank
of the 128K-token example split over 4 ranks (S=131072, N=4, L=32768, rank 3,
causal, B=1, H=32, d=128, bf16): ring schedule, simulated ring receives of
blocks 2, 1, 0 into the two workspace slots on a second stream (double
buffered), four attention kernels (diagonal block first) and the fused
finalise.  Inputs are resident in HBM before timing starts.

Prints ONE JSON line.  The metric is causal-adjusted attention TFLOP/s:
4 d B H x (visible query/key pairs) flops per step.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk (the published 2.5 PF)
PEAK_FP8_TFLOPS = 5033.2      # MI355X dense FP8 MFMA: twice the bf16 rate (the published 5.0 PF)
PEAK_HBM_GBS = 8000.0
COPY_KERNEL = "__amd_rocclr_copyBuffer"
STREAM_KERNEL = "lds_stream_kernel"     # the global->LDS read of cp_attn_measure_lds_stream
STREAM_MIB = 256
_BLK = 32768 * 32 * 128                 # elements of one K or V block of the 128K example
# Per profiled kernel: its name in the traces, the sources it is compiled
# from, the committed PMC summary, the bytes of one ring-receive copy of the
# same run (the counters' calibration) and the command the runs profile.
KERNELS = {
    # the bf16 kernel's two forms (<128, false>: V row-major, the rank's own
    # block; <128, true>: V in the tiles the ring receive writes) share the prefix
    "bf16": dict(name="attn_block_bf16_kernel<128", srcs=("attn_mfma.hip", "gfx950_util.h", "kernels.h"),
                 json="attn_block_bf16__causal_128k_last_rank.traffic.json", copy_bytes=2 * _BLK,
                 cmd="python3 bench.py --steps 1 --warmup 0 --no-cpu-baseline --no-secondary --calibration-read-mib 256"),
    "fp8": dict(name="attn_block_fp8_kernel<128", srcs=("attn_fp8.hip", "gfx950_util.h", "kernels.h"),
                json="attn_block_fp8__causal_128k_last_rank.traffic.json", copy_bytes=_BLK,
                cmd="python3 bench.py --fp8-only --steps 1 --warmup 0 --calibration-read-mib 256"),
}
TRAFFIC_JSON = os.path.join(ROOT, "profiles", KERNELS["bf16"]["json"])


def kernel_device_text(path: str) -> bytes:
    """The part of a kernel source that is device code: a .hip file up to its
    first host launcher (`hipError_t launch_`), a header whole.  Launcher
    changes that leave the kernel, its grid and its arguments as they were do
    not invalidate a traffic measurement."""
    with open(path, "rb") as f:
        text = f.read()
    if path.endswith(".hip"):
        cut = text.find(b"\nhipError_t launch_")
        if cut >= 0:
            text = text[:cut]
    return text


def kernel_sha256(which: str = "bf16") -> str:
    """SHA-256 over the device code a forward block kernel is compiled from."""
    h = hashlib.sha256()
    for f in KERNELS[which]["srcs"]:
        h.update(kernel_device_text(os.path.join(ROOT, "context_ring_attention_cp_amd", "csrc", f)))
    return h.hexdigest()


def _pmc_rows(d: str, counter: str):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    rows = []
    for f in files:
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter:
                rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    return sorted(rows)


def summarize_pmc(fetch_dir: str, write_dir: str, which: str = "bf16", out: str = None) -> dict:
    """HBM traffic of an attention kernel from a FETCH_SIZE run and a
    WRITE_SIZE run (KiB per dispatch) of its one-step bench command.  Each
    counter is scaled by what it reads for the ring-receive copy kernels of
    the same run, which move one K or V block each.  Written to the kernel's
    committed summary under profiles/ unless `out` names another file."""
    kern = KERNELS[which]
    copy_bytes, attn_kernel = kern["copy_bytes"], kern["name"]
    res = {}
    for name, d, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        rows = _pmc_rows(d, counter)
        cal = [v for _, k, v in rows if COPY_KERNEL in k and abs(v * 1024 - copy_bytes) < 0.6 * copy_bytes]
        att = [v for _, k, v in rows if attn_kernel in k]
        stream = [v for _, k, v in rows if STREAM_KERNEL in k]
        if not cal or not att:
            raise SystemExit(f"{counter}: calibration copies {len(cal)}, attention dispatches {len(att)}")
        copy_factor = copy_bytes / (sum(cal) / len(cal) * 1024)
        res[name] = {"counter": counter, "kib_per_dispatch": att, "copy_kib": sum(cal) / len(cal),
                     "copy_factor": copy_factor}
        if name == "fetch" and stream:
            # bytes read through the same global->LDS fetch as the attention kernel's tiles
            res[name]["stream_kib"] = stream[-1]
            res[name]["stream_factor"] = (STREAM_MIB << 20) / (stream[-1] * 1024)
            res[name]["factor"] = res[name]["stream_factor"]
            res[name]["calibration"] = f"{STREAM_KERNEL}: global_load_lds_dwordx4 over {STREAM_MIB} MiB"
        else:
            res[name]["factor"] = copy_factor
            res[name]["calibration"] = f"ring-receive copies ({COPY_KERNEL}) of {copy_bytes} bytes"
    n = min(len(res["fetch"]["kib_per_dispatch"]), len(res["write"]["kib_per_dispatch"]))
    per = [res["fetch"]["kib_per_dispatch"][i] * 1024 * res["fetch"]["factor"]
           + res["write"]["kib_per_dispatch"][i] * 1024 * res["write"]["factor"] for i in range(n)]
    summary = {"kernel": attn_kernel, "kernel_source_sha256": kernel_sha256(which), "dispatches": n,
               "traffic_bytes_per_dispatch": per, "traffic_bytes_mean": sum(per) / n,
               "fetch": res["fetch"], "write": res["write"], "calibration_copy_bytes": copy_bytes,
               "command": "rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) --output-format csv -d <dir> -o <name> -- "
                          + kern["cmd"]}
    with open(out or os.path.join(ROOT, "profiles", kern["json"]), "w") as f:
        json.dump(summary, f, indent=1)
    return summary


def measured_traffic(which: str = "bf16"):
    """Mean HBM bytes per attention dispatch from the committed PMC summary,
    or None if it was taken on a different kernel source."""
    try:
        with open(os.path.join(ROOT, "profiles", KERNELS[which]["json"])) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != kernel_sha256(which):
        return None
    return t["traffic_bytes_mean"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the brief timing of the other workloads")
    ap.add_argument("--cpu-rows", type=int, default=4096,
                    help="query rows of one head timed on the CPU oracle")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the traffic summary from two rocprofv3 --pmc runs and exit (no GPU)")
    ap.add_argument("--pmc-kernel", choices=sorted(KERNELS), default="bf16",
                    help="the kernel --summarize-pmc summarises")
    ap.add_argument("--fp8-only", action="store_true",
                    help="time only the FP8 (e4m3) forward of the 128K last-rank shard and print its JSON")
    ap.add_argument("--calibration-read-mib", type=int, default=0,
                    help="after the timed steps, read this many MiB once through the global->LDS fetch "
                         "(the HBM counter calibration of a --pmc run)")
    ap.add_argument("--only", choices=SECONDARY, default=None,
                    help="time only this secondary workload and print its JSON (for a profiler run)")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def attn_flops(spec, pairs: int) -> float:
    """Causal-adjusted forward flops: 4 d per visible (query, key) pair (2 d
    for QK^T, 2 d for PV) of each batch element and head; `pairs` is the
    per-(batch, head) count of cp_attn_visible_pairs."""
    return 4.0 * spec.d * spec.B * spec.H * pairs


def cpu_baseline(spec, q, k, v, rows_n: int):
    """The fp64 oracle, as it is, on a bounded sample of the same workload:
    `rows_n` evenly spaced query rows of head 0, against all keys."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # noqa: BLE001
        blas_threads = 1
    L = spec.L
    rows = np.linspace(0, L - 1, rows_n).astype(np.int64)
    t0 = time.perf_counter()
    oracle.rank_attention(q, k, v, spec.rank, spec.N, spec.mask, spec.cu_seqlens, rows=rows, heads=[0])
    dt = time.perf_counter() - t0
    p = spec.rank * L + rows
    pairs = int(np.sum(p + 1)) if spec.mask == "causal" else int(rows_n * spec.S)
    flops = 4.0 * spec.d * pairs          # one head, one batch element: the sample
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": f"{rows_n} evenly spaced query rows of head 0 of {spec.H} ({pairs} visible pairs, "
                      f"{dt:.1f} s wall, fp64 numpy, materialised score rows)",
            "host_cpus": len(os.sched_getaffinity(0))}


def oracle_timing(seed: int, rows_n: int = 1024) -> dict:
    """The fp64 oracle, as it is, timed on every workload: the tiny fp32 ring
    whole (all 4 ranks), and for the others `rows_n` evenly spaced query rows
    of the benchmarked rank against all its keys, on a one-head draw of the
    same shapes (the oracle's cost per head does not depend on the values).
    Reports the BLAS library and its threads, the sample's wall time and
    rate on the causal-adjusted count, and the whole config's time
    extrapolated from that rate (labelled as such)."""
    import oracle
    from harness.inputs import ShardSpec, make_inputs, standard_configs
    blas = {}
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if info:
            blas = {"library": info[0].get("internal_api"), "version": info[0].get("version"),
                    "threads": info[0].get("num_threads"), "path": os.path.basename(info[0].get("filepath", ""))}
    except Exception:  # noqa: BLE001
        pass
    res = {"blas": blas, "host_cpus": len(os.sched_getaffinity(0)), "configs": {}}
    for cfg, full in standard_configs(seed).items():
        spec1 = ShardSpec(S=full.S, N=full.N, H=1, d=full.d, dtype=full.dtype, mask=full.mask, rank=full.rank,
                          B=full.B, cfg_id=full.cfg_id, q_scale=full.q_scale, cu_seqlens=full.cu_seqlens)
        ranks = list(range(full.N)) if cfg == 1 else [full.rank]
        inp = make_inputs(spec1, seed, ranks=ranks)
        blocks = oracle.ring_schedule(full.N, full.rank, full.L, full.mask, full.cu_seqlens)
        t0 = time.perf_counter()
        pairs = 0
        for r in ranks:
            rows = (np.arange(full.L, dtype=np.int64) if cfg == 1
                    else np.linspace(0, full.L - 1, min(rows_n, full.L)).astype(np.int64))
            kb = {j: inp["k"][j] for j in range(full.N)} if cfg == 1 else {j: inp["k"][j] for j in blocks}
            vb = {j: inp["v"][j] for j in range(full.N)} if cfg == 1 else {j: inp["v"][j] for j in blocks}
            oracle.rank_attention(inp["q"][r], kb, vb, r, full.N, full.mask, full.cu_seqlens, rows=rows, heads=[0])
            p = r * full.L + rows
            if full.mask == "none":
                pairs += len(rows) * full.S
            else:
                first = 0 if full.mask == "causal" else oracle.doc_start(p, full.cu_seqlens)
                pairs += int(np.sum(p - first + 1))
        dt = time.perf_counter() - t0
        rate = 4.0 * full.d * pairs / dt
        total_pairs = sum(oracle.visible_pairs(full.N, full.L, r, full.mask, full.cu_seqlens) for r in ranks)
        res["configs"][f"cfg{cfg}"] = {
            "workload": full.name,
            "sample": ("all rows of the 4 ranks, one head of 2" if cfg == 1 else
                       f"{len(rows)} evenly spaced rows of rank {full.rank}, one head of {full.H}"),
            "sample_s": round(dt, 3), "gflops": round(rate / 1e9, 2),
            "full_config_s_extrapolated": round(4.0 * full.d * total_pairs * full.H * full.B / rate, 1)}
    return res


def calibration_read(cp, mib: int, stream) -> None:
    """Read `mib` MiB once through the global->LDS fetch (cp_attn_measure_lds_stream):
    the HBM byte counters of a --pmc run are calibrated on this kernel."""
    if not mib:
        return
    import torch
    buf = torch.ones(mib << 18, device="cuda")     # MiB of float32
    torch.cuda.synchronize()
    cp.cp_attn_measure_lds_stream(buf, stream=stream)
    torch.cuda.synchronize()
    del buf


def _timed(fn, stream, warmup: int, reps: int) -> float:
    """Mean milliseconds of fn() over `reps` runs on `stream` (HIP events).
    The inputs were made on the default stream, and the caching allocator
    reuses memory in that stream's order only: everything queued so far must
    finish before `stream` touches any of it."""
    import torch
    torch.cuda.synchronize()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def _timed_flushed(fn, stream, warmup: int, reps: int, flush) -> dict:
    """Per-iteration HIP-event times of fn() on `stream`, each iteration
    preceded (outside its events) by a read of the 512 MiB `flush` buffer on
    the same stream, which evicts the L2 and the 256 MB Infinity Cache, so that
    inputs that would fit there are read from HBM as in a real ring step.  A
    read leaves clean lines behind (a write would leave the timed kernel to
    write back up to the whole cache).  Returns the median and the mean in ms."""
    import torch
    torch.cuda.synchronize()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    sink = torch.zeros(2, device="cuda")
    ev = []
    for i in range(reps):
        with torch.cuda.stream(stream):
            sink[i % 2] = flush.sum()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        ev.append((e0, e1))
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in ev)
    return {"median": float(np.median(t)), "mean": float(np.mean(t))}


def _timed_rotating(fn, stream, warmup: int, reps: int) -> dict:
    """Per-iteration HIP-event times of fn(i) on `stream`, back to back, where
    fn(i) works on input set i mod (number of sets): with the sets together
    more than twice the 256 MB Infinity Cache, each iteration reads inputs
    that earlier iterations have evicted, as a ring step reads a freshly
    received block, and no other kernel runs between iterations.  Returns
    the median, mean, min and max in ms."""
    import torch
    torch.cuda.synchronize()
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    ev = []
    for i in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn(i)
        e1.record(stream)
        ev.append((e0, e1))
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in ev)
    return {"median": float(np.median(t)), "mean": float(np.mean(t)), "min": t[0], "max": t[-1]}


# Cold-input sets: enough copies of a workload's inputs to span twice the
# 256 MB Infinity Cache.
MALL_BYTES = 256 << 20


def _n_sets(set_bytes: int) -> int:
    return max(2, -(-2 * MALL_BYTES // set_bytes) + 1)


SECONDARY = ("cfg2", "cfg5", "cfg4", "ulysses", "fp8")
# Untimed calls before timing a workload of about a millisecond: its first few
# dozen calls run up to 10 % slower than the steady state (the kernels' own
# durations do not change; the time between dependent launches does).
SHORT_WARMUP = 30


def secondary(seed: int, reps: int = 5, only=None, streams=None):
    """The other workloads of the path, timed briefly: the causal 32K
    last-rank shard, the packed-document shard (rank_forward, ring prefetch),
    the bidirectional 64K merge stress case (8 PARTIAL_LSE launches, then one
    merge in a shuffled order; the merge is reported against HBM), one rank's
    share of all-to-all (Ulysses) context parallelism at 128K and the FP8
    forward.  The inputs of the 32K shard would stay in the caches, so it and
    the merge stress case are timed over rotating copies of their inputs,
    each evicted before reuse (medians), with the medians of calls each after
    a cache-flushing read reported beside them.  `only` names one of
    SECONDARY to run alone (for a profiler run).  `streams`: the (compute,
    copy) stream pair to use; a process keeps its streams on few hardware
    queues, and two more streams beside the headline's can land the copy
    stream on the compute stream's queue, which serialises the receives with
    the kernels they should overlap."""
    import torch

    import context_ring_attention_cp_amd as cp
    from harness.inputs import standard_configs

    out = {}
    cfgs = standard_configs(seed)
    cs, xs = streams if streams is not None else (torch.cuda.Stream(), torch.cuda.Stream())
    for name in SECONDARY:
        if only is not None and name != only:
            continue
        if name in ("cfg2", "cfg5"):
            out[name] = _sec_ring(cp, cfgs[int(name[3])], seed, cs, xs, reps)
        elif name == "cfg4":
            out[name] = _sec_merge(cp, cfgs[4], seed, cs)
        elif name == "ulysses":
            out[name] = _sec_ulysses(cp, cfgs[3], seed, cs, reps)
        else:
            out[name] = fp8_forward(cp, cfgs[3], seed, cs, xs, reps)
        torch.cuda.empty_cache()
    return out


def _dev_bf16(x):
    import torch

    from harness.inputs import bf16_bits
    return torch.from_numpy(np.ascontiguousarray(bf16_bits(x)).view(np.int16)).view(torch.bfloat16).to("cuda")


def _sec_ring(cp, spec, seed, cs, xs, reps):
    """A rank forward with ring prefetch: the causal 32K last-rank shard (its
    inputs would stay in the caches, so it is timed over rotating copies of
    its inputs that are evicted before reuse: median of 40 back-to-back
    calls; the median of 10 calls each after a 512 MiB cache-flushing read is
    reported beside it) or the packed-document shard (mean of reps; its
    inputs exceed the caches)."""
    import torch

    from harness.inputs import TENSOR_K, TENSOR_Q, TENSOR_V, draw_shard
    cu_dev = None if spec.cu_seqlens is None else torch.from_numpy(spec.cu_seqlens).to("cuda")
    desc = cp.Desc(spec.B, spec.H, spec.d, spec.N, spec.L, spec.rank, "bf16", spec.mask,
                   cu_seqlens=spec.cu_seqlens, cu_seqlens_dev=cu_dev)
    sched = cp.cp_attn_ring_schedule(desc, cp.CP_RING_PREFETCH)
    q = _dev_bf16(draw_shard(spec, seed, TENSOR_Q, spec.rank))
    kb = [_dev_bf16(draw_shard(spec, seed, TENSOR_K, j)) if j in sched else None for j in range(spec.N)]
    vb = [_dev_bf16(draw_shard(spec, seed, TENSOR_V, j)) if j in sched else None for j in range(spec.N)]
    o = torch.empty((1, spec.L, spec.H, spec.d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((1, spec.H, spec.L), device="cuda")
    ws = cp.alloc_workspace(desc)
    sets = [(q, kb, vb)]

    def run(i=0):
        qq, kk, vv = sets[i % len(sets)]
        cp.cp_attn_rank_forward(desc, qq, kk, vv, o, None, None, lse, workspace=ws, compute_stream=cs,
                                copy_stream=xs, flags=cp.CP_RING_PREFETCH)

    fl = attn_flops(spec, cp.cp_attn_visible_pairs(desc))
    extra = {}
    if spec.S <= 32768:
        set_bytes = sum(t.numel() * t.element_size() for t in [q] + [t for t in kb + vb if t is not None])
        for _ in range(_n_sets(set_bytes) - 1):
            sets.append((q.clone(), [None if t is None else t.clone() for t in kb],
                         [None if t is None else t.clone() for t in vb]))
        t = _timed_rotating(run, cs, SHORT_WARMUP, 40)
        ms = t["median"]
        flush = torch.ones(128 << 20, device="cuda")     # 512 MiB
        tf = _timed_flushed(run, cs, SHORT_WARMUP, 10, flush)
        del flush
        extra = {"ms_mean": round(t["mean"], 4), "ms_min_max": [round(t["min"], 4), round(t["max"], 4)],
                 "timing": f"median of 40 back-to-back calls over {len(sets)} rotating copies of the inputs "
                           f"({len(sets)} x {set_bytes / 2**20:.0f} MiB, each evicted from the caches before reuse)",
                 "ms_flushed": round(tf["median"], 4),
                 "tflops_flushed": round(fl / (tf["median"] * 1e-3) / 1e12, 2)}
    else:
        ms = _timed(run, cs, SHORT_WARMUP, reps)
    # per-launch attention kernel and receive times: medians of 10 profiled
    # calls with the receives beside the kernels (prefetch) and after them on
    # the compute stream (serial), which shows what the overlap costs the
    # kernels that share the compute units with the copies
    def per_launch(flags):
        ks, rs = [], []
        for _ in range(10):
            prof = cp.Profiler(len(sched))
            cp.cp_attn_rank_forward(desc, q, kb, vb, o, None, None, lse, workspace=ws, compute_stream=cs,
                                    copy_stream=xs, flags=flags, profiler=prof)
            ks.append(prof.read())
            rs.append(prof.read_copies())
            prof.close()
        med = lambda col: round(float(np.median(col)), 4)
        return ([med([k[i] for k in ks]) for i in range(len(ks[0]))],
                [med([r[i] for r in rs]) for i in range(len(rs[0]))])
    kms, rms = per_launch(cp.CP_RING_PREFETCH)
    kms_serial, rms_serial = per_launch(0)
    del sets
    return {"workload": spec.name, "blocks": sched, "ms": round(ms, 4),
            "tflops": round(fl / (ms * 1e-3) / 1e12, 2),
            "pct_of_peak": round(100.0 * fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
            "kernel_ms": kms, "receive_ms": rms,
            "kernel_ms_serial": kms_serial, "receive_ms_serial": rms_serial, **extra}


def _sec_merge(cp, spec, seed, cs):
    """Bidirectional 64K over 8 ranks, rank 5, Q x 3: eight PARTIAL_LSE
    launches, then one merge in a seeded shuffled order.  Timed over two
    rotating copies of the inputs and of the partials (each set larger than
    the 256 MB Infinity Cache): partials median of 10, merge median of 40; the
    medians with a 512 MiB cache-flushing read before each call are reported
    beside them."""
    import torch

    from harness.inputs import TENSOR_K, TENSOR_Q, TENSOR_V, draw_shard, shuffled_order
    desc = cp.Desc(spec.B, spec.H, spec.d, spec.N, spec.L, spec.rank, "bf16", spec.mask)
    q = _dev_bf16(draw_shard(spec, seed, TENSOR_Q, spec.rank))
    kb = [_dev_bf16(draw_shard(spec, seed, TENSOR_K, j)) for j in range(spec.N)]
    vb = [_dev_bf16(draw_shard(spec, seed, TENSOR_V, j)) for j in range(spec.N)]
    big, vec = (1, spec.L, spec.H, spec.d), (1, spec.H, spec.L)
    ins = [(q, kb, vb), (q.clone(), [t.clone() for t in kb], [t.clone() for t in vb])]
    parts = [([torch.empty(big, device="cuda") for _ in range(spec.N)],
              [torch.empty(vec, device="cuda") for _ in range(spec.N)]) for _ in range(2)]
    o = torch.empty(big, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(vec, device="cuda")
    order = shuffled_order(seed, 4, spec.N)

    def partials(i=0):
        qq, kk, vv = ins[i % 2]
        op, lp = parts[i % 2]
        with torch.cuda.stream(cs):
            for j in range(spec.N):
                cp.cp_attn_block_partial(desc, j, cp.CP_MODE_PARTIAL_LSE, qq, kk[j], vv[j], o_part=op[j],
                                         lse_part=lp[j], stream=cs)

    def merge(i=0):
        op, lp = parts[i % 2]
        cp.cp_attn_merge_lse(desc, op, lp, order, o, lse, stream=cs)

    tp = _timed_rotating(partials, cs, 2, 10)
    tm = _timed_rotating(merge, cs, SHORT_WARMUP, 40)
    flush = torch.ones(128 << 20, device="cuda")
    tpf = _timed_flushed(partials, cs, 1, 10, flush)
    tmf = _timed_flushed(merge, cs, SHORT_WARMUP, 10, flush)
    del flush
    ms_p, ms_m = tp["median"], tm["median"]
    fl = attn_flops(spec, cp.cp_attn_visible_pairs(desc))
    rows = spec.L * spec.H
    merge_bytes = spec.N * rows * (spec.d * 4 + 4) + rows * (spec.d * 2 + 4)
    gbs = lambda ms: merge_bytes / (ms * 1e-3) / 1e9      # noqa: E731
    res = {"workload": spec.name, "order": order,
           "timing": "medians over two rotating copies of the inputs and partials (partials 10 calls, merge 40)",
           "partials_ms_mean": round(tp["mean"], 4), "merge_ms_mean": round(tm["mean"], 4),
           "partials_ms": round(ms_p, 4),
           "partials_tflops": round(fl / (ms_p * 1e-3) / 1e12, 2), "merge_ms": round(ms_m, 4),
           "merge_algorithmic_bytes": merge_bytes,
           "merge_gbs": round(gbs(ms_m), 1),
           "merge_frac_of_hbm": round(gbs(ms_m) / PEAK_HBM_GBS, 4),
           "partials_ms_flushed": round(tpf["median"], 4), "merge_ms_flushed": round(tmf["median"], 4),
           "merge_gbs_flushed": round(gbs(tmf["median"]), 1)}
    del ins, parts
    return res


def _sec_ulysses(cp, spec, seed, cs, reps):
    """All-to-all (Ulysses) share of the 128K example: rank 3 of 4 runs the
    whole sequence (S = 131072) on its 8 of 32 heads; the two all-to-alls are
    the regrouping copies.  Seeded N(0, 1) inputs drawn on the device."""
    import torch
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed + 303)
    shape = (spec.B, spec.L, spec.H, spec.d)
    qs, ks, vs = ([torch.randn(shape, generator=gen, device="cuda").to(torch.bfloat16) for _ in range(spec.N)]
                  for _ in range(3))
    os_ = [torch.empty(shape, dtype=torch.bfloat16, device="cuda") for _ in range(spec.N)]
    desc = cp.Desc(spec.B, spec.H, spec.d, spec.N, spec.L, spec.rank, "bf16", "causal")
    ws = cp.alloc_ulysses_workspace(desc)
    hn = spec.H // spec.N
    lse = torch.empty((spec.B, hn, spec.S), device="cuda")
    ms = _timed(lambda: cp.cp_attn_ulysses_forward(desc, qs, ks, vs, os_, None, None, lse, workspace=ws, stream=cs),
                cs, 2, reps)
    fl = 4.0 * spec.d * hn * spec.B * spec.S * (spec.S + 1) / 2
    regroup = 8 * spec.B * spec.S * hn * spec.d * 2      # Q, K, V gathered and O scattered, each read + written
    return {"workload": "all-to-all (Ulysses) share of the 128K example: rank 3 of 4, 8 of 32 heads "
                        "over S=131072, causal, bf16; the two all-to-alls simulated by regrouping copies",
            "ms": round(ms, 4), "tflops": round(fl / (ms * 1e-3) / 1e12, 2), "regroup_bytes": regroup}


def fp8_forward(cp, spec, seed: int, cs, xs, reps: int) -> dict:
    """The causal 128K last-rank shard with e4m3 inputs: Q and the K/V blocks
    quantised once on the device (per-(batch, head) scales), then the FP8 ring
    forward with prefetch.  Seeded N(0, 1) inputs drawn on the device.  The
    kernel rate is the algorithmic flops over the summed launch durations
    (HIP events around each block launch), against the dense FP8 MFMA peak."""
    import torch
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed + 404)
    shape = (spec.B, spec.L, spec.H, spec.d)
    desc = cp.Desc(spec.B, spec.H, spec.d, spec.N, spec.L, spec.rank, "bf16", "causal")
    qd1 = cp.Desc(spec.B, spec.H, spec.d, 1, spec.L, 0, "bf16", "none")
    codes, scales = [], []
    x = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    for i in range(1 + 2 * spec.N):          # the query (with the softmax's base-2 factor), then K and V blocks
        x.copy_(torch.randn(shape, generator=gen, device="cuda"))
        c = torch.empty(shape, dtype=torch.uint8, device="cuda")
        sc = torch.empty((spec.B, spec.H), device="cuda")
        cp.cp_attn_quantize_fp8(qd1, x, c, sc, role=cp.CP_FP8_QUERY if i == 0 else cp.CP_FP8_KV)
        codes.append(c)
        scales.append(sc)
    ms_q = _timed(lambda: cp.cp_attn_quantize_fp8(qd1, x, codes[-1], scales[-1], stream=cs), cs, 2, reps)
    del x
    qc, qs = codes[0], scales[0]
    kc, ks = codes[1:1 + spec.N], scales[1:1 + spec.N]
    vc, vs = codes[1 + spec.N:], scales[1 + spec.N:]
    o = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((spec.B, spec.H, spec.L), device="cuda")
    ws = cp.alloc_workspace(desc)
    sched = cp.cp_attn_ring_schedule(desc, cp.CP_RING_PREFETCH)
    prof = cp.Profiler(len(sched) * reps)

    def run(p=None):
        cp.cp_attn_rank_forward_fp8(desc, qc, qs, kc, ks, vc, vs, o, None, None, lse, workspace=ws,
                                    compute_stream=cs, copy_stream=xs, flags=cp.CP_RING_PREFETCH, profiler=p)

    for _ in range(2):
        run()
    torch.cuda.synchronize()
    prof.reset()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(cs)
    for _ in range(reps):
        run(prof)
    e1.record(cs)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    kms = prof.read()
    prof.close()
    assert torch.isfinite(o.float()).all(), "non-finite FP8 output"
    fl = attn_flops(spec, cp.cp_attn_visible_pairs(desc))
    k_tf = fl * reps / (sum(kms) * 1e-3) / 1e12
    res = {"workload": "causal last-rank shard of the 128K example with e4m3 Q/K/V (per-(batch, head) power-of-two "
                       "scales), "
                       "bf16 output: S=131072 N=4 L=32768 rank=3 B=1 H=32 d=128, ring prefetch",
           "blocks": sched, "ms": round(ms, 4), "tflops": round(fl / (ms * 1e-3) / 1e12, 2),
           "kernel_mean_ms": round(sum(kms) / max(1, len(kms)), 4), "kernel_tflops": round(k_tf, 2),
           "frac_of_fp8_peak": round(k_tf / PEAK_FP8_TFLOPS, 4), "fp8_peak": PEAK_FP8_TFLOPS,
           "traffic_bytes_per_launch": measured_traffic("fp8"),
           "quantize_ms_per_block": round(ms_q, 4),
           "quantize_gbs": round(spec.B * spec.L * spec.H * spec.d * 3 / (ms_q * 1e-3) / 1e9, 1),
           "ring_bytes_copied": spec.B * spec.L * spec.H * spec.d * 2 * (len(sched) - 1)}
    del codes, scales, o, lse, ws
    return res


def backward(spec, seed, desc, qd, kd, vd, out, lse, pairs, stream, reps: int = 3) -> dict:
    """cp_attn_rank_backward of the benchmarked shard (delta, then the dQ and
    dK/dV kernels per visible block), with the forward's out and lse and a
    seeded dO.  tflops counts the algorithmic 10 d flops per visible pair (the
    five products S, dP, dV, dK, dQ); the kernels execute 14 d (S and dP are
    computed by both kernels), reported as mfma_tflops."""
    import torch

    import context_ring_attention_cp_amd as cp
    from harness.inputs import bf16_bits, draw_grad

    big, vec = (spec.B, spec.L, spec.H, spec.d), (spec.B, spec.H, spec.L)
    do = torch.from_numpy(np.ascontiguousarray(bf16_bits(draw_grad(spec, seed, spec.rank))).view(np.int16))
    do = do.view(torch.bfloat16).to("cuda")
    delta = torch.empty(vec, device="cuda")
    dq = torch.empty(big, device="cuda")
    dk = [torch.empty(big, device="cuda") for _ in range(spec.N)]
    dv = [torch.empty(big, device="cuda") for _ in range(spec.N)]
    ms = _timed(lambda: cp.cp_attn_rank_backward(desc, qd, kd, vd, out, do, lse, delta, dq, dk, dv, stream=stream),
                stream, 1, reps)
    assert torch.isfinite(dq).all(), "non-finite dq"
    fl = 10.0 * spec.d * spec.B * spec.H * pairs
    res = {"workload": "backward of the benchmarked shard (rank_backward: delta, dQ and dK/dV kernels per block)",
           "ms": round(ms, 4), "tflops": round(fl / (ms * 1e-3) / 1e12, 2),
           "pct_of_peak": round(100.0 * fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
           "mfma_tflops": round(1.4 * fl / (ms * 1e-3) / 1e12, 2), "flops_counted": fl}
    del do, delta, dq, dk, dv
    return res


def main():
    args = parse()
    if args.summarize_pmc:
        print(json.dumps(summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.pmc_kernel)))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import context_ring_attention_cp_amd as cp
    from harness.inputs import TENSOR_K, TENSOR_Q, TENSOR_V, bf16_bits, draw_shard, standard_configs

    cp.lib()
    if args.only:
        print(json.dumps(secondary(args.seed, max(args.steps, 1), only=args.only)[args.only]), flush=True)
        return
    if args.fp8_only:
        cs, xs = torch.cuda.Stream(), torch.cuda.Stream()
        print(json.dumps(fp8_forward(cp, standard_configs(args.seed)[3], args.seed, cs, xs, max(args.steps, 1))),
              flush=True)
        calibration_read(cp, args.calibration_read_mib, cs)
        return
    spec = standard_configs(args.seed)[3]
    N, L, H, d, r = spec.N, spec.L, spec.H, spec.d, spec.rank
    log(f"[bench] generating inputs for {spec.name}")
    q = draw_shard(spec, args.seed, TENSOR_Q, r)
    k = {j: draw_shard(spec, args.seed, TENSOR_K, j) for j in range(N)}
    v = {j: draw_shard(spec, args.seed, TENSOR_V, j) for j in range(N)}

    def dev(x):
        return torch.from_numpy(np.ascontiguousarray(bf16_bits(x)).view(np.int16)).view(torch.bfloat16).to("cuda")

    qd = dev(q)
    kd = [dev(k[j]) for j in range(N)]
    vd = [dev(v[j]) for j in range(N)]
    desc = cp.Desc(spec.B, H, d, N, L, r, "bf16", "causal")
    out = torch.empty((spec.B, L, H, d), dtype=torch.bfloat16, device="cuda")
    m = torch.empty((spec.B, H, L), device="cuda")
    lsum = torch.empty_like(m)
    lse = torch.empty_like(m)
    ws = cp.alloc_workspace(desc)
    cs, xs = torch.cuda.Stream(), torch.cuda.Stream()
    sched = cp.cp_attn_ring_schedule(desc, cp.CP_RING_PREFETCH)
    prof = cp.Profiler(len(sched) * max(args.steps, 1))
    pairs = cp.cp_attn_visible_pairs(desc)
    flops = attn_flops(spec, pairs)
    torch.cuda.synchronize()

    def step(p=None):
        cp.cp_attn_rank_forward(desc, qd, kd, vd, out, m, lsum, lse, workspace=ws, compute_stream=cs,
                                copy_stream=xs, flags=cp.CP_RING_PREFETCH, profiler=p)

    log(f"[bench] warmup {args.warmup} steps, schedule {sched}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    prof.reset()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(cs)
    for i in range(args.steps):
        step(prof)
        marks[i].record(cs)
    e1.record(cs)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = e0.elapsed_time(e1) / args.steps
    step_ms = [e0.elapsed_time(marks[0])] + [marks[i - 1].elapsed_time(marks[i]) for i in range(1, args.steps)]
    kernel_ms = prof.read()
    copy_ms = prof.read_copies()
    assert torch.isfinite(out.float()).all(), "non-finite output"
    value = flops / (ms_step * 1e-3) / 1e12

    # dominant kernel: the attention block kernel; achieved = algorithmic flops
    # of its launches / their summed duration (= mean flops per launch / mean duration)
    k_sum = sum(kernel_ms)
    achieved = flops * args.steps / (k_sum * 1e-3) / 1e12
    per_step = [kernel_ms[i:i + len(sched)] for i in range(0, len(kernel_ms), len(sched))]
    traffic = measured_traffic()
    blk_bytes = spec.B * L * H * d * 2
    res = {
        "metric": "causal-adjusted attention TFLOP/s per rank shard; % of MI355X bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_median": round(float(np.median(step_ms)), 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "causal last-rank shard of the 128K example: S=131072 N=4 L=32768 rank=3 "
                               "B=1 H=32 d=128 bf16, simulated ring with double-buffered prefetch",
                   "S": spec.S, "N": N, "L": L, "rank": r, "B": spec.B, "H": H, "d": d, "mask": "causal",
                   "seed": args.seed},
        "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic},
        "flops_per_step": flops,
        "kernel_ms_per_step": [round(x, 4) for x in per_step[-1]] if per_step else [],
        "kernel_mean_ms": round(k_sum / max(1, len(kernel_ms)), 4),
        "ring_bytes_copied_per_step": 2 * blk_bytes * (len(sched) - 1),
        # the simulated communication of each step (K copy + V re-layout on
        # the copy stream, HIP events on that stream) against its computation
        "comm": {"receive_ms_per_step": round(sum(copy_ms) / max(1, args.steps), 4),
                 "receive_ms_each": [round(x, 4) for x in copy_ms[-(len(sched) - 1):]] if copy_ms else [],
                 "attention_ms_per_step": round(k_sum / max(1, args.steps), 4),
                 "comm_over_compute": round(sum(copy_ms) / k_sum, 4) if k_sum > 0 else None,
                 "exposed_ms_per_step": round(ms_step - k_sum / max(1, args.steps), 4),
                 "receive_gbs": round(2 * 2 * blk_bytes * len(copy_ms) / (sum(copy_ms) * 1e-3) / 1e9, 1)
                 if copy_ms else None},
        "ring_traffic_formula_bytes": 2 * (2 * spec.B * spec.S * H * d * 2 // N) * (N - 1),
        "wall_s_timed": round(wall, 3),
    }
    prof.close()
    calibration_read(cp, args.calibration_read_mib, cs)
    del m, lsum, ws
    if not args.no_secondary:
        log("[bench] backward of the same shard")
        res["backward"] = backward(spec, args.seed, desc, qd, kd, vd, out, lse, pairs, cs)
    del qd, kd, vd, out, lse
    if not args.no_secondary:
        log("[bench] secondary workloads")
        res["secondary"] = secondary(args.seed, streams=(cs, xs))
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline: oracle on {args.cpu_rows} rows of head 0")
        res["cpu_baseline"] = cpu_baseline(spec, q, k, v, args.cpu_rows)
        log("[bench] oracle timing of every workload")
        res["cpu_baseline"]["per_config"] = oracle_timing(args.seed)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
