"""The named workloads at full size on the MI355X, in the launch configuration
bench.py times, compared with the oracle on every element: whole calls where
the oracle replays them in seconds, column blocks of all ranks where the
result does not depend on the fold order (int32 sums and maxima), whole
blocks for the reduce-scatter (the oracle's reduce to the block's rank);
properties that hold at any size are checked too (all ranks agree; blocks
land where the definition says)."""
import numpy as np
import pytest

import oracle
import ring_all_reduce_allreduce_amd as rs
import synth
from tests import _gpu as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    rs.lib()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _bits(t):
    import torch

    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def _all_ranks_equal(recv):
    import torch

    return all(torch.equal(_bits(t), _bits(recv[0])) for t in recv[1:])


def test_workload3_ddp_buckets_back_to_back():
    """40 distinct bucket all-reduces (8 ranks x 25 MiB bf16, 16 channels,
    seeded inputs of their own drawn on the device) enqueued back to back on
    one stream, checked after one synchronisation: every bucket on one rank
    against the oracle, element by element, and all ranks against each
    other."""
    import torch

    w = synth.WORKLOADS[3]
    n, count, nch = w["nranks"], w["n"], w["nchannels"]
    sends = [synth.device_inputs(3, n, count, "bfloat16", "normal", 1e-3, bucket=b) for b in range(w["buckets"])]
    comm = rs.comm_init(n, nch, "auto")
    try:
        recvs = []
        for b, send in enumerate(sends):
            recv = [torch.empty(count, dtype=torch.bfloat16, device="cuda:0") for _ in range(n)]
            rs.allreduce(comm, send, recv)
            recvs.append(recv)
        G.say(f"{len(sends)} ddp buckets enqueued")
        G.sync()
        G.check_comm_ok(comm)
        for b in range(w["buckets"]):
            assert _all_ranks_equal(recvs[b]), f"bucket {b}: ranks disagree"
            xs = [G.to_host(t, "bfloat16") for t in sends[b]]
            want = oracle.ring_allreduce(xs, "sum", "bfloat16", nchannels=nch)
            got = G.to_host(recvs[b][b % n], "bfloat16")
            mm = G.first_mismatch(got, want[b % n], "bfloat16")
            assert mm is None, f"bucket {b}: {mm}"
            if b % 10 == 0:
                G.say(f"ddp bucket {b} matches the oracle")
                exact = np.sum(np.stack([oracle.bf16_to_f64(x) for x in xs]), axis=0)
                g64 = oracle.bf16_to_f64(got)
                assert np.linalg.norm(g64 - exact) / np.linalg.norm(exact) <= 8e-3
    finally:
        rs.comm_destroy(comm)


@pytest.mark.parametrize("choice", ["threshold", "auto"])
@pytest.mark.parametrize("op", ["sum", "max"])
def test_workload4_size_sweep(op, choice):
    """16 ranks, int32 in [-2^20, 2^20], 8 B .. 256 MiB per rank; one channel
    below 64 KiB, 16 channels from 64 KiB up (the sweep's channel choice).
    "threshold": the ring, flag-packed below 64 KiB and bulk above (the
    sweep's own fixed threshold); "auto": whatever algorithm, protocol and
    workgroups the cost model takes (the tree, FLAG, WIDE or BULK). Integer
    sums and maxima do not depend on the fold order, so both equal the ring
    oracle."""
    import torch

    n = 16
    cfg = dict(flag_threshold_bytes=65536, algo="ring") if choice == "threshold" else {}
    comms = {1: rs.comm_init(n, 1, "auto", **cfg), 16: rs.comm_init(n, 16, "auto", **cfg)}
    try:
        for k, size in enumerate(synth.WORKLOADS[4]["sizes_bytes"]):
            count = size // 4
            nch = 1 if size < 65536 else 16
            comm = comms[nch]
            want_proto = 2 if size < 65536 else 1
            G.say(f"sweep {choice} op={op} bytes/rank={size}")
            if size <= (4 << 20):
                xs = synth.rank_inputs(4, n, count, "int32", "int", lo=-(1 << 20), hi=1 << 20, bucket=k)
                send = [G.to_device(x, "int32") for x in xs]
            else:
                send = synth.device_inputs(4, n, count, "int32", "int", lo=-(1 << 20), hi=1 << 20, bucket=k)
                xs = None
            recv = [torch.empty(count, dtype=torch.int32, device="cuda:0") for _ in range(n)]
            rs.allreduce(comm, send, recv, op=op)
            G.sync()
            G.check_comm_ok(comm)
            if choice == "threshold":
                assert rs.comm_query(comm)["last_proto"] == want_proto, f"size {size}"
            assert _all_ranks_equal(recv), f"size {size}: ranks disagree"
            if xs is not None:
                want = oracle.ring_allreduce(xs, op, "int32", nchannels=nch)
                got = G.to_host(recv[k % n], "int32")
                assert G.first_mismatch(got, want[0], "int32") is None, f"size {size}"
            else:
                # Every element, in column blocks of all ranks: an int32 sum
                # (wrapping) or maximum does not depend on the fold order, so
                # the oracle's ring over one block of columns gives exactly
                # those columns of the result.
                blk = 1 << 22
                for lo in range(0, count, blk):
                    hi = min(count, lo + blk)
                    cols = [G.to_host(t[lo:hi], "int32") for t in send]
                    want = oracle.ring_allreduce(cols, op, "int32", nchannels=1)[0]
                    got = G.to_host(recv[k % n][lo:hi], "int32")
                    assert G.first_mismatch(got, want, "int32") is None, f"size {size} columns {lo}:{hi}"
            del send, recv
    finally:
        for c in comms.values():
            rs.comm_destroy(c)


def test_workload5_reduce_scatter_then_all_gather():
    """8 ranks: reduce-scatter of 128 MiB bf16 per rank (16 MiB shards), then
    all-gather of the shards back to 128 MiB, 8 channels."""
    import torch

    n, count, nch = 8, 67_108_864, 8
    rc = count // n
    send = synth.device_inputs(5, n, count, "bfloat16", "normal", 1.0)
    shard = [torch.empty(rc, dtype=torch.bfloat16, device="cuda:0") for _ in range(n)]
    full = [torch.empty(count, dtype=torch.bfloat16, device="cuda:0") for _ in range(n)]
    comm = rs.comm_init(n, nch, "auto")
    try:
        G.say("reduce_scatter 8 x 128 MiB bf16")
        rs.reduce_scatter(comm, send, shard)
        G.say("all_gather 8 x 16 MiB bf16")
        rs.all_gather(comm, shard, full)
        G.sync()
        G.check_comm_ok(comm)
        # reduce-scatter: block b folded b+1, ..., b -- the oracle's reduce to
        # root b -- on every element of every shard
        for b in range(n):
            cols = [G.to_host(t[b * rc:(b + 1) * rc], "bfloat16") for t in send]
            want = oracle.reduce(cols, b, "sum", "bfloat16")
            mm = G.first_mismatch(G.to_host(shard[b], "bfloat16"), want, "bfloat16")
            assert mm is None, f"block {b}: {mm}"
        # all-gather: block b of every output is shard b, on every element
        for r in range(n):
            for b in range(n):
                assert torch.equal(full[r][b * rc:(b + 1) * rc].view(torch.int16), shard[b].view(torch.int16)), (r, b)
    finally:
        rs.comm_destroy(comm)


def test_workload5_alltoall_full():
    """8 ranks x 8 chunks of 512 x 4096 bf16: chunk j of rank i -> slot i of rank j."""
    import torch

    n = 8
    xs = synth.a2a_inputs(nranks=n)
    send = [G.to_device(x, "bfloat16") for x in xs]
    recv = [torch.empty_like(s) for s in send]
    comm = rs.comm_init(n, 1, "auto")
    try:
        G.say("alltoall 8 x 32 MiB bf16")
        rs.alltoall(comm, send, recv)
        G.sync()
        G.check_comm_ok(comm)
        want = oracle.alltoall(xs, "bfloat16")
        for r in range(n):
            assert np.array_equal(G.to_host(recv[r], "bfloat16"), want[r]), r
    finally:
        rs.comm_destroy(comm)
