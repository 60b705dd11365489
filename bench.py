#!/usr/bin/env python3
"""Benchmark: busBW of the N-rank ring all-reduce on one MI355X.

One step is one ring all-reduce (reduce-scatter stages then all-gather stages,
every channel and chunk) of the headline workload: 8 simulated ranks, 64 MiB
of fp32 per rank drawn N(0,1), 8 channels, 512 KiB chunks, sum. The inputs are
resident in HBM before the timed region starts. Prints ONE JSON line on
stdout; details go to stderr.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                  [--no-cpu-baseline] [--no-check]

busBW = algBW * 2(N-1)/N with algBW = bytes per rank / time per step
(the ring cost model's nSteps/nRanks factor, "NCCL" book, ch. 5, ring.cc).
The roofline entry divides the algorithmic HBM bytes of one launch,
(6N-4) * S for the all-reduce, by the average launch duration measured with
HIP events on the launch stream, against the 8 TB/s HBM3E peak.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "busBW GB/s of N-rank ring all-reduce on 1 MI355X; % of HBM peak"
_CSRC = os.path.join(ROOT, "ring_all_reduce_allreduce_amd", "csrc")
# Sources of the kernel that dominates each collective's workloads: a counter
# record under profiles/ is used only while these files are unchanged.
KERNEL_SOURCES = [os.path.join(_CSRC, f) for f in ("ring_bulk.hip", "ringsim_device.h", "ring_plan.h",
                                                   "ringsim_internal.h")]
COPY_KERNEL_SOURCES = [os.path.join(_CSRC, f) for f in ("copy.hip", "ringsim_internal.h")]

# Named single-GPU workloads. "ar8x64" is the headline; the others exist for
# exploration and print the same JSON fields.
WORKLOADS = {
    "ar4x4k": dict(coll="allreduce", nranks=4, count=1024, dtype="float32", nchannels=1,
                   chunk_bytes=524_288, synth_workload=1, op="sum", proto="bulk", graph_calls=100,
                   desc="ring all-reduce sum, 4 simulated ranks x 1024 fp32 (integers in [-8, 8]), 1 channel, "
                        "bulk protocol (latency-bound: report us per call)"),
    "ar8x64": dict(coll="allreduce", nranks=8, count=16_777_216, dtype="float32", nchannels=8,
                   chunk_bytes=524_288, synth_workload=2, op="sum",
                   desc="ring all-reduce sum, 8 simulated ranks x 64 MiB fp32 (16,777,216 elems, N(0,1)), "
                        "8 channels, 512 KiB chunks"),
    "ar8x25bf16": dict(coll="allreduce", nranks=8, count=13_107_200, dtype="bfloat16", nchannels=16,
                       chunk_bytes=524_288, synth_workload=3, op="sum", buckets=40,
                       desc="DDP bucket ring all-reduce sum, 8 simulated ranks x 25 MiB bf16 "
                            "(13,107,200 elems, N(0,1e-3)), 16 channels, 40 distinct buckets (each drawn on the "
                            "device with a seed of its own) back to back on one stream (one bucket per step)"),
    "ar16x256i32": dict(coll="allreduce", nranks=16, count=67_108_864, dtype="int32", nchannels=16,
                        chunk_bytes=524_288, synth_workload=4, op="sum",
                        desc="ring all-reduce sum, 16 simulated ranks x 256 MiB int32, 16 channels"),
    "rs8x128bf16": dict(coll="reduce_scatter", nranks=8, count=67_108_864, dtype="bfloat16", nchannels=8,
                        chunk_bytes=524_288, synth_workload=5, op="sum",
                        desc="ring reduce-scatter sum, 8 simulated ranks x 128 MiB bf16 in, 16 MiB out"),
    "ag8x128bf16": dict(coll="all_gather", nranks=8, count=67_108_864, dtype="bfloat16", nchannels=8,
                        chunk_bytes=524_288, synth_workload=5, op="sum",
                        desc="ring all-gather, 8 simulated ranks x 16 MiB bf16 in, 128 MiB out"),
    "a2a8x32bf16": dict(coll="alltoall", nranks=8, count=16_777_216, dtype="bfloat16", nchannels=1,
                        chunk_bytes=524_288, synth_workload=5, op="sum", buffer_sets=4,
                        desc="all-to-all, 8 simulated ranks x 8 chunks of 512x4096 bf16 (32 MiB per rank); "
                             "4 buffer sets in turn, so that no step finds its input in the Infinity Cache"),
}
DTYPE_TAG = {"float32": "f32", "bfloat16": "bf16", "int32": "i32", "int64": "i64"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash(coll: str = "allreduce") -> str:
    h = hashlib.sha256()
    for p in COPY_KERNEL_SOURCES if coll == "alltoall" else KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(coll: str, n: int, s: int) -> int:
    """HBM bytes the ring method moves in one launch, summed over ranks; S is
    the full per-rank buffer (all-reduce buffer, reduce-scatter input,
    all-gather output, all-to-all buffer). All-reduce: every rank reads S,
    writes S and writes then reads 2(N-1)/N * S of FIFO slots; reduce-scatter
    and all-gather: (3N-1)/N * S per rank; all-to-all: 2S per rank."""
    if n == 1:
        return 2 * s
    if coll == "allreduce":
        return (6 * n - 4) * s
    if coll in ("reduce_scatter", "all_gather"):
        return (3 * n - 1) * s
    return 2 * n * s


def bus_factor(coll: str, n: int) -> float:
    if n == 1:
        return 1.0
    return 2.0 * (n - 1) / n if coll == "allreduce" else (n - 1) / n


def load_traffic(name: str, src_hash: str):
    """Counter-measured bytes per launch between the L2 and the memory side
    (HBM and Infinity Cache alike), if a summary for this workload and this
    exact kernel source is committed under profiles/: the record's fields."""
    p = os.path.join(ROOT, "profiles", f"traffic_{name}.txt")
    if not os.path.exists(p):
        return None
    t = {}
    with open(p) as f:
        for line in f:
            if ":" in line:
                k, v = line.split(":", 1)
                t[k.strip()] = v.strip()
    if t.get("kernel_source_hash") != src_hash:
        return None
    return t


def make_inputs(w: dict):
    import numpy as np
    import synth

    n, dtype = w["nranks"], w["dtype"]
    if w["coll"] == "alltoall":
        return synth.a2a_inputs(nranks=n)
    if w["coll"] == "all_gather":
        return synth.rank_inputs(w["synth_workload"], n, w["count"] // n, dtype, "normal", 1.0, bucket=2)
    if w["coll"] == "reduce_scatter":
        return synth.rank_inputs(w["synth_workload"], n, w["count"], dtype, "normal", 1.0)
    if w["synth_workload"] == 4:
        return synth.rank_inputs(4, n, w["count"], dtype, "int", lo=-(1 << 20), hi=(1 << 20))
    if w.get("buckets", 1) > 1:
        # DDP buckets are drawn on the device (40 x 200 MiB would take minutes
        # on the host); bucket 0 comes back for the oracle.
        import torch

        return [t.view(torch.int16).cpu().numpy().view(np.uint16) if dtype == "bfloat16" else t.cpu().numpy()
                for t in ddp_bucket(w, 0)]
    xs = synth.workload_inputs(w["synth_workload"])
    assert xs[0].shape[0] == w["count"] and len(xs) == n
    _ = np
    return xs


def ddp_bucket(w: dict, b: int):
    """Device buffers of DDP bucket b: N(0, 1e-3) bf16 from torch's seeded
    device generator, seed = 1,000,000 x workload + 1,000 x bucket + rank."""
    import synth

    return synth.device_inputs(w["synth_workload"], w["nranks"], w["count"], w["dtype"], "normal", 1e-3, bucket=b)


def oracle_call(w: dict, xs):
    import oracle

    if w["coll"] == "allreduce":
        return oracle.ring_allreduce(xs, w["op"], w["dtype"], nchannels=w["nchannels"], chunk_bytes=w["chunk_bytes"])
    if w["coll"] == "reduce_scatter":
        return oracle.ring_reduce_scatter(xs, w["op"], w["dtype"], nchannels=w["nchannels"],
                                          chunk_bytes=w["chunk_bytes"])
    if w["coll"] == "all_gather":
        return oracle.ring_all_gather(xs, w["dtype"], nchannels=w["nchannels"], chunk_bytes=w["chunk_bytes"])
    return oracle.alltoall(xs, w["dtype"])


def cpu_model() -> str:
    """The host CPU's model name from /proc/cpuinfo ("unknown" elsewhere)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w: dict, xs, per_rank_bytes: int, budget_s: float = 10.0):
    """The oracle, as it stands, timed on this host on the same workload:
    whole calls, repeated until about `budget_s` seconds of CPU work (at
    least three calls), median per call. Returns the baseline record and the
    oracle's result, against which the GPU result is then checked."""
    import numpy as np  # noqa: F401

    times = []
    t_start = time.perf_counter()
    c_start = time.process_time()
    result = None
    while len(times) < 3 or time.perf_counter() - t_start < budget_s:
        t0 = time.perf_counter()
        result = oracle_call(w, xs)
        times.append(time.perf_counter() - t0)
    # Threads actually busy: process CPU time over wall time.
    busy = (time.process_time() - c_start) / max(time.perf_counter() - t_start, 1e-9)
    t = statistics.median(times)
    n = w["nranks"]
    busbw = per_rank_bytes / t * bus_factor(w["coll"], n) / 1e9
    return {
        "value": round(busbw, 4),
        "unit": "GB/s",
        "cores": max(1, round(busy)),
        "kind": "oracle",
        "sample": f"the full workload ({w['desc']}), NumPy ring replay on one thread, median of {len(times)} "
                  f"whole calls ({sum(times):.1f} s, CPU time / wall time {busy:.2f}), {t * 1e3:.3f} ms per call; host has "
                  f"{len(os.sched_getaffinity(0))} cores available ({cpu_model()})",
    }, result


def mixed_copy_gbs(stream_bytes: int, resident_bytes: int, trials: int = 7) -> float:
    """Plain copies with an all-reduce's byte mix, run concurrently on two
    streams (bytes moved / time, median of `trials`): one copy of
    `stream_bytes` from HBM (the user buffers' reads and writes), and
    back-to-back copies between two 64 MiB buffers that the Infinity Cache
    holds, moving `resident_bytes` in all (the FIFO slots' writes and
    reads). The ceiling for the kernel's traffic on this part, with no ring,
    no flow control and no arithmetic."""
    import torch

    big_a = torch.empty(stream_bytes // 2, dtype=torch.uint8, device="cuda")
    big_b = torch.empty_like(big_a)
    sm = [torch.empty(64 << 20, dtype=torch.uint8, device="cuda") for _ in range(2)]
    k = max(1, round(resident_bytes / (128 << 20)))
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    cur = torch.cuda.current_stream()
    big_b.copy_(big_a)
    torch.cuda.synchronize()
    rates = []
    for _ in range(trials):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        d1, d2 = torch.cuda.Event(), torch.cuda.Event()
        e0.record(cur)
        s1.wait_event(e0)
        s2.wait_event(e0)
        with torch.cuda.stream(s1):
            big_b.copy_(big_a)
            d1.record(s1)
        with torch.cuda.stream(s2):
            for i in range(k):
                sm[(i + 1) % 2].copy_(sm[i % 2])
            d2.record(s2)
        cur.wait_event(d1)
        cur.wait_event(d2)
        e1.record(cur)
        torch.cuda.synchronize()
        rates.append((2 * big_a.numel() + k * 2 * (64 << 20)) / (e0.elapsed_time(e1) / 1e3) / 1e9)
    del big_a, big_b, sm
    return statistics.median(rates)


def d2d_copy_gbs(nbytes: int = 1 << 30, reps: int = 10, trials: int = 5) -> float:
    """Device-to-device copy (read + write bytes / time, median of `trials`
    batches of `reps` copies) as the achievable-bandwidth context of this GPU:
    1 GiB streams from HBM; 64 MiB (source and destination both fit in the
    256 MB Infinity Cache) is the ceiling for traffic that the cache serves,
    as the FIFO slots are."""
    import torch

    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    rates = []
    for _ in range(trials):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        rates.append(2 * nbytes / (e0.elapsed_time(e1) / 1e3 / reps) / 1e9)
    del a, b
    return statistics.median(rates)


def copy_calibration(args) -> int:
    """Known-size reference for the byte counters: the copy kernel moving
    1 GiB (reads 1 GiB, writes 1 GiB) per launch."""
    import torch

    import ring_all_reduce_allreduce_amd as rs

    nbytes = 1 << 30
    src = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda:0").fill_(7)
    dst = torch.empty_like(src)
    comm = rs.comm_init(1, 1, "bulk")
    for _ in range(args.warmup):
        rs.alltoall(comm, [src], [dst])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        rs.alltoall(comm, [src], [dst])
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / 1e3 / args.steps
    ok = bool(torch.equal(src, dst))
    rs.comm_destroy(comm)
    print(json.dumps({"metric": "copy kernel HBM bandwidth (read+write)", "value": round(2 * nbytes / t / 1e9, 1),
                      "unit": "GB/s", "bytes_read_per_launch": nbytes, "bytes_written_per_launch": nbytes,
                      "launch_avg_us": round(t * 1e6, 2), "copy_ok": ok}), flush=True)
    return 0 if ok else 1


def size_sweep(args) -> int:
    """Latency / bandwidth of an int32 collective across message sizes
    (default: all-reduce, 16 ranks, 16 channels); AUTO picks the algorithm,
    protocol and line workgroups per size with the library's cost model, and
    each line reports what it ran. Sizes are bytes per rank: the all-reduce
    buffer, the reduce-scatter input, the all-gather output. Each size is
    checked on sampled elements against the plain definition: for int32 the
    wrapping sum and the maximum do not depend on the fold order, and an
    all-gather output is its inputs."""
    import numpy as np
    import torch

    import ring_all_reduce_allreduce_amd as rs
    import synth

    coll = args.sweep_coll
    n = args.sweep_ranks
    comms = {c: rs.comm_init(n, c, args.proto, workgroups_per_channel=args.wpc or None, algo=args.algo,
                             line_workgroups_per_channel=args.line_wpc or None)
             for c in sorted({args.sweep_channels, args.sweep_small_channels or args.sweep_channels})}
    size = 8
    k = 0
    while size < max(args.sweep_min_bytes, 4 if coll == "allreduce" else 4 * n):
        size *= 2
        k += 1
    while size <= args.sweep_max_bytes:
        # below 64 KiB per rank the small-message channel count
        nch = (args.sweep_small_channels or args.sweep_channels) if size < 65536 else args.sweep_channels
        comm = comms[nch]
        total = size // 4                                   # elements per rank of the sized buffer
        part = total if coll == "allreduce" else total // n  # the other buffer of RS / AG
        nin = part if coll == "all_gather" else total
        send = synth.device_inputs(4, n, nin, "int32", "int", lo=-(1 << 20), hi=1 << 20, bucket=k)
        recv = [torch.empty(total if coll != "reduce_scatter" else part, dtype=torch.int32, device="cuda")
                for _ in range(n)]

        def call():
            if coll == "allreduce":
                rs.allreduce(comm, send, recv, op=args.sweep_op)
            elif coll == "reduce_scatter":
                rs.reduce_scatter(comm, send, recv, op=args.sweep_op)
            else:
                rs.all_gather(comm, send, recv)

        for _ in range(args.warmup):
            call()
        torch.cuda.synchronize()
        # Sampled parity: element columns of every rank's input, reduced by
        # definition (wrapping int32 sum, or maximum) or gathered, against the
        # same elements of one rank's output.
        r = k % n
        m = part if coll != "all_gather" else nin
        idx = np.unique(np.linspace(0, m - 1, min(m, 4096)).astype(np.int64))
        tidx = torch.from_numpy(idx).cuda()
        if coll == "all_gather":
            want = np.concatenate([t[tidx].cpu().numpy() for t in send])
            got = np.concatenate([recv[r][b * part + tidx].cpu().numpy() for b in range(n)])
        else:
            off = r * part if coll == "reduce_scatter" else 0
            cols = np.stack([t[off + tidx].cpu().numpy() for t in send])
            want = cols.max(axis=0) if args.sweep_op == "max" else cols.sum(axis=0, dtype=np.int32)
            got = recv[r][tidx].cpu().numpy()
        ok = bool(np.array_equal(got, want))
        steps = args.steps if size < (64 << 20) else max(5, args.steps // 4)
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        torch.cuda.synchronize()
        torch.cuda._sleep(2_000_000)
        for i in range(steps):
            starts[i].record()
            call()
            ends[i].record()
        torch.cuda.synchronize()
        t = statistics.median([a.elapsed_time(b) / 1e3 for a, b in zip(starts, ends)])
        info = rs.comm_query(comm)
        algo = {1: "ring", 2: "tree"}.get(info["last_algo"], "?") if coll == "allreduce" else "ring"
        proto = "wide" if algo == "tree" else {1: "bulk", 2: "flag", 3: "wide"}.get(info["last_proto"], "?")
        busbw = size / t * bus_factor(coll, n) / 1e9
        byts = algorithmic_bytes(coll, n, size)
        print(json.dumps({"coll": coll, "nranks": n, "nchannels": nch, "op": args.sweep_op, "bytes_per_rank": size,
                          "algo": algo, "proto": proto,
                          "wpc": 0 if algo == "tree" else info["last_workgroups_per_channel"],
                          "tree_channels": info["last_tree_channels"],
                          "us": round(t * 1e6, 2), "busbw_gbs": round(busbw, 3),
                          "alg_frac": round(byts / t / 1e9 / HBM_PEAK_GBS, 4), "sampled_parity": ok}), flush=True)
        if not ok:
            return 1
        del send, recv
        size *= 2
        k += 1
    for c in comms.values():
        rs.comm_destroy(c)
    return 0


def graph_timing(call, calls: int, stream, launches: int = 20) -> dict:
    """Captures `calls` back-to-back calls into one HIP graph (torch.cuda.CUDAGraph)
    and times `launches` launches of it with one HIP event pair each, on the
    launch stream: microseconds per call with no host work between calls."""
    import torch

    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for _ in range(calls):
            call()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(launches)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(launches)]
    torch.cuda._sleep(2_000_000)
    for a, b in zip(starts, ends):
        a.record(stream)
        g.replay()
        b.record(stream)
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) * 1e3 / calls for a, b in zip(starts, ends))
    return {"calls": calls, "launches": launches, "us_per_call": round(statistics.median(per), 3),
            "us_per_call_min": round(per[0], 3)}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="ar8x64", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-check", action="store_true")
    ap.add_argument("--wpc", type=int, default=0, help="workgroups per channel (0 = library default)")
    ap.add_argument("--line-wpc", type=int, default=0,
                    help="most workgroups per channel of a FLAG/WIDE launch: 1, 2, 4, 8 (0 = per call)")
    ap.add_argument("--slot-bytes", type=int, default=0)
    ap.add_argument("--nslots", type=int, default=0)
    ap.add_argument("--sweep", action="store_true",
                    help="message-size sweep instead (16 ranks, int32, 8 B .. 256 MiB per rank, 16 channels, "
                         "auto protocol): one JSON line per size")
    ap.add_argument("--sweep-min-bytes", type=int, default=8)
    ap.add_argument("--sweep-max-bytes", type=int, default=256 << 20)
    ap.add_argument("--sweep-ranks", type=int, default=16)
    ap.add_argument("--sweep-channels", type=int, default=16)
    ap.add_argument("--sweep-small-channels", type=int, default=1,
                    help="channels below 64 KiB per rank (0 = --sweep-channels)")
    ap.add_argument("--sweep-op", default="sum", choices=["sum", "max"])
    ap.add_argument("--sweep-coll", default="allreduce", choices=["allreduce", "reduce_scatter", "all_gather"])
    ap.add_argument("--proto", default="auto", choices=["auto", "bulk", "flag", "wide"])
    ap.add_argument("--algo", default="auto", choices=["auto", "ring", "tree"],
                    help="all-reduce algorithm for --sweep (auto: the library's choice)")
    ap.add_argument("--graph-calls", type=int, default=-1,
                    help="also time K back-to-back calls captured in one HIP graph (0 = off; default: the "
                         "workload's own setting, 100 calls for ar4x4k, else off)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="time the library's copy kernel on 1 GiB (a one-rank all-to-all) instead; used to "
                         "scale the HBM byte counters")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: ringsim simulates all ranks on ONE GPU; run it with --gpus 1 "
              "(rings across GPUs over xGMI are not implemented)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import ring_all_reduce_allreduce_amd as rs

    if args.copy_calibration:
        return copy_calibration(args)
    if args.sweep:
        return size_sweep(args)

    w = WORKLOADS[args.workload]
    n, dtype, coll = w["nranks"], w["dtype"], w["coll"]
    esize = rs.ELEM_SIZE[dtype]
    tdt = {"float32": torch.float32, "bfloat16": torch.bfloat16, "int32": torch.int32, "int64": torch.int64}[dtype]
    dev = torch.device("cuda:0")

    log(f"[bench] workload {args.workload}: {w['desc']}")
    xs = make_inputs(w)

    def upload(x):
        if dtype == "bfloat16":
            return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(x).to(dev)

    nbuckets = w.get("buckets", 1)
    send = None if coll == "allreduce" and nbuckets > 1 else [upload(x) for x in xs]
    if coll == "allreduce" and nbuckets > 1:
        # Distinct buckets back to back, each with seeded inputs of its own
        # (drawn on the device) and a receive buffer set of its own.
        sends = [ddp_bucket(w, b) for b in range(nbuckets)]
        send = sends[0]
        recvs = [[torch.empty_like(send[0]) for _ in range(n)] for _ in range(nbuckets)]
        per_rank_bytes = w["count"] * esize
        bucket = [0]

        def call():
            b = bucket[0] % nbuckets
            bucket[0] += 1
            rs.allreduce(comm, sends[b], recvs[b], op=w["op"])

        recv = recvs[0]
    elif coll == "allreduce":
        recv = [torch.empty_like(s) for s in send]
        per_rank_bytes = w["count"] * esize
        call = lambda: rs.allreduce(comm, send, recv, op=w["op"])  # noqa: E731
    elif coll == "reduce_scatter":
        recv = [torch.empty(w["count"] // n, dtype=tdt, device=dev) for _ in range(n)]
        per_rank_bytes = w["count"] * esize
        call = lambda: rs.reduce_scatter(comm, send, recv, op=w["op"])  # noqa: E731
    elif coll == "all_gather":
        recv = [torch.empty(w["count"], dtype=tdt, device=dev) for _ in range(n)]
        per_rank_bytes = w["count"] * esize
        call = lambda: rs.all_gather(comm, send, recv)  # noqa: E731
    else:
        # Distinct buffer sets in turn (1 GiB of inputs for 4 sets): a step
        # never reads what the previous step left in the 256 MB cache.
        nsets = w.get("buffer_sets", 1)
        sends = [send] + [[t.clone() for t in send] for _ in range(nsets - 1)]
        recvs = [[torch.empty_like(t) for t in send] for _ in range(nsets)]
        recv = recvs[0]
        per_rank_bytes = xs[0].shape[0] * esize
        step = [0]

        def call():
            b = step[0] % nsets
            step[0] += 1
            rs.alltoall(comm, sends[b], recvs[b])

    comm = rs.comm_init(n, w["nchannels"], w.get("proto", "auto"), chunk_bytes=w["chunk_bytes"],
                        workgroups_per_channel=args.wpc or None, slot_bytes=args.slot_bytes or None,
                        nslots=args.nslots or None)
    info = rs.comm_query(comm)
    log(f"[bench] comm {json.dumps(info)}")

    stream = torch.cuda.current_stream()
    for _ in range(max(args.warmup, 1) if nbuckets > 1 or w.get("buffer_sets", 1) > 1 else args.warmup):
        call()
    torch.cuda.synchronize()
    if rs.get_async_error(comm) != rs.SUCCESS:
        log("[bench] warmup left the communicator in error state")
        return 1

    # Timed region: K steps, per-launch HIP events on the launch stream. A
    # short device sleep goes first so that every timed launch is already
    # queued when the one before it ends: event intervals then hold device
    # time only, not the host's launch latency.
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    torch.cuda._sleep(2_000_000)
    t0 = time.perf_counter()
    for k in range(args.steps):
        starts[k].record(stream)
        call()
        ends[k].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if rs.get_async_error(comm) != rs.SUCCESS:
        log("[bench] timed region left the communicator in error state")
        return 1
    per = [s.elapsed_time(e) / 1e3 for s, e in zip(starts, ends)]
    t_med = statistics.median(per)
    t_avg = sum(per) / len(per)
    t_p95 = sorted(per)[min(len(per) - 1, int(0.95 * len(per)))]
    cv = statistics.pstdev(per) / t_avg if len(per) > 1 else 0.0
    ms_per_step = wall / args.steps * 1e3

    algbw = per_rank_bytes / t_med / 1e9
    busbw = algbw * bus_factor(coll, n)
    bytes_alg = algorithmic_bytes(coll, n, per_rank_bytes)
    achieved = bytes_alg / t_avg / 1e9
    compulsory = 2 * n * per_rank_bytes if coll in ("allreduce", "alltoall") else (n + 1) * per_rank_bytes
    src_hash = kernel_source_hash(coll)
    traffic = load_traffic(args.workload, src_hash)
    d2d = d2d_copy_gbs()
    cache_copy = d2d_copy_gbs(64 << 20, reps=50)
    mixed = mixed_copy_gbs(compulsory, bytes_alg - compulsory) if coll == "allreduce" else None
    log(f"[bench] per-launch median {t_med * 1e6:.1f} us, avg {t_avg * 1e6:.1f} us, p95 {t_p95 * 1e6:.1f} us, "
        f"CV {cv * 100:.2f}%  algBW {algbw:.1f} GB/s busBW {busbw:.1f} GB/s  "
        f"alg-bytes rate {achieved:.0f} GB/s ({achieved / HBM_PEAK_GBS * 100:.1f}% of peak)  "
        f"compulsory rate {compulsory / t_avg / 1e9:.0f} GB/s  D2D copy {d2d:.0f} GB/s "
        f"(cache-resident {cache_copy:.0f} GB/s" + (f", this byte mix {mixed:.0f} GB/s)" if mixed else ")"))

    # Back-to-back buckets: one event pair around all of them (no host
    # synchronization in between), three times from bucket 0.
    back_to_back = None
    if coll == "allreduce" and nbuckets > 1:
        runs = []
        for _ in range(3):
            bucket[0] = 0
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            torch.cuda._sleep(2_000_000)
            a.record(stream)
            for _ in range(nbuckets):
                call()
            b.record(stream)
            torch.cuda.synchronize()
            runs.append(a.elapsed_time(b) * 1e3 / nbuckets)
        if rs.get_async_error(comm) != rs.SUCCESS:
            log("[bench] back-to-back buckets left the communicator in error state")
            return 1
        back_to_back = {"calls": nbuckets, "us_per_call": round(statistics.median(runs), 2),
                        "busbw_gbs": round(per_rank_bytes / (statistics.median(runs) * 1e-6) / 1e9
                                           * bus_factor(coll, n), 2)}
        log(f"[bench] {nbuckets} buckets back to back: {back_to_back['us_per_call']:.1f} us per bucket")

    graph = None
    gk = args.graph_calls if args.graph_calls >= 0 else w.get("graph_calls", 0)
    if gk > 0:
        graph = graph_timing(call, gk, stream)
        if rs.get_async_error(comm) != rs.SUCCESS:
            log("[bench] graph launches left the communicator in error state")
            return 1
        log(f"[bench] graph of {gk} calls: {graph['us_per_call']:.2f} us per call")

    # The CPU oracle, timed (the cpu_baseline leg); the GPU result of the
    # last launch (timed, back to back or from the graph; every launch of a
    # buffer set computes the same values) is then checked against its
    # result bit for bit.
    cpu = None
    check = "not checked (the oracle runs only in the cpu_baseline leg)"
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle ...")
        cpu, want = cpu_baseline(w, xs, per_rank_bytes)
        log(f"[bench] cpu baseline {cpu}")
        if not args.no_check:
            ok = True
            for r in range(n):
                got = recv[r].view(torch.int16).cpu().numpy().view(np.uint16) if dtype == "bfloat16" else recv[r].cpu().numpy()
                ok &= bool(np.array_equal(got.view(np.uint8), np.asarray(want[r]).view(np.uint8)))
            check = "bit-exact vs oracle" if ok else "MISMATCH vs oracle"
            log(f"[bench] parity: {check}")
            if not ok:
                return 1

    kernel_name = {"allreduce": "ring_bulk_kernel (all-reduce)", "reduce_scatter": "ring_bulk_kernel (reduce-scatter)",
                   "all_gather": "ring_bulk_kernel (all-gather)", "alltoall": "copy_kernel (all-to-all)"}[coll]
    out = {
        "metric": METRIC,
        "value": round(busbw, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_TAG[dtype],
        "data": "synthetic",
        "config": {
            "workload": w["desc"],
            "collective": coll,
            "simulated_ranks": n,
            "bytes_per_rank": per_rank_bytes,
            "nchannels": w["nchannels"],
            "chunk_bytes": w["chunk_bytes"],
            "buckets": nbuckets,
            "buffer_sets": w.get("buffer_sets", 1),
            # the count the timed calls took (a bulk call with short stages
            # takes fewer than the communicator holds)
            "workgroups_per_channel": rs.comm_query(comm)["last_workgroups_per_channel"],
            "proto": {1: "bulk", 2: "flag", 3: "wide"}.get(rs.comm_query(comm)["last_proto"], "?"),
            "parallelism": "1 GPU, simulated ranks",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": kernel_name,
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": int(traffic["bytes_per_launch"]) if traffic else None,
            "bytes_per_launch": bytes_alg,
            "launch_avg_us": round(t_avg * 1e6, 2),
            # What the bytes are: `achieved` counts the method's algorithmic
            # bytes, `traffic` the counted bytes between the L2 and the memory
            # side. Both include the FIFO slots, which the 256 MB Infinity
            # Cache serves (they are rewritten before HBM sees them), so `frac`
            # is the byte model's rate against the HBM peak, not HBM's own
            # utilisation. The user buffers (2N x S, or (N+1) x S for
            # reduce-scatter / all-gather) must cross HBM: `frac_compulsory`
            # is that rate, a lower bound of HBM's utilisation.
            "bytes_counted_at": "L2 to memory side (HBM and Infinity Cache together)",
            "frac_compulsory": round(compulsory / t_avg / 1e9 / HBM_PEAK_GBS, 4),
            "dram_request_bytes": int(traffic["dram_request_bytes"]) if traffic and "dram_request_bytes" in traffic
            else None,
        },
        "cpu_baseline": cpu,
        "extra": {
            "algbw_gbs": round(algbw, 2),
            "busbw_gbs": round(busbw, 2),
            "t_median_us": round(t_med * 1e6, 2),
            "t_p95_us": round(t_p95 * 1e6, 2),
            "cv": round(cv, 4),
            "cv_above_5pct": cv > 0.05,
            "frac_compulsory": round(compulsory / t_avg / 1e9 / HBM_PEAK_GBS, 4),
            "d2d_copy_gbs": round(d2d, 1),
            "cache_resident_copy_gbs": round(cache_copy, 1),
            "mixed_copy_gbs": round(mixed, 1) if mixed else None,
            "parity": check,
            "kernel_source_hash": src_hash,
            "graph": graph,
            "back_to_back": back_to_back,
        },
    }
    rs.comm_destroy(comm)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
