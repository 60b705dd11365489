"""The named workloads at full size on the MI355X, in the launch configuration
bench.py times. Where the oracle can replay the whole call in seconds it does;
otherwise the oracle computes sampled elements one by one (the ring fold of
those elements across ranks) and properties that hold at any size are checked
on every element (all ranks agree; blocks land where the definition says)."""
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


def _sample_idx(n, k, seed):
    rng = np.random.default_rng(seed)
    idx = np.unique(np.concatenate([rng.integers(0, n, k), [0, n - 1], np.arange(min(n, 64))]))
    return idx


def _host_at(t, idx, dtype):
    import torch

    sel = t.index_select(0, torch.from_numpy(idx).to(t.device))
    return G.to_host(sel, dtype)


def _bits(t):
    import torch

    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def _all_ranks_equal(recv):
    import torch

    return all(torch.equal(_bits(t), _bits(recv[0])) for t in recv[1:])


def test_workload3_ddp_buckets_back_to_back():
    """40 bucket all-reduces (8 ranks x 25 MiB bf16, 16 channels) enqueued
    back to back on one stream, checked after one synchronisation."""
    import torch

    w = synth.WORKLOADS[3]
    n, count, nch = w["nranks"], w["n"], w["nchannels"]
    base = [synth.rank_inputs(3, n, count, "bfloat16", "normal", 1e-3, bucket=b) for b in range(5)]
    base_dev = [[G.to_device(x, "bfloat16") for x in bb] for bb in base]
    comm = rs.comm_init(n, nch, "auto")
    try:
        recvs = []
        for b in range(w["buckets"]):
            bb, src = synth.ddp_bucket_ranks(b, n)
            send = [base_dev[bb][src[r]] for r in range(n)]
            recv = [torch.empty(count, dtype=torch.bfloat16, device="cuda:0") for _ in range(n)]
            G.say(f"ddp bucket {b} base {bb} ranks {src}")
            rs.allreduce(comm, send, recv)
            recvs.append(recv)
        G.sync()
        G.check_comm_ok(comm)
        for b in range(w["buckets"]):
            assert _all_ranks_equal(recvs[b]), f"bucket {b}: ranks disagree"
        for b in (0, 17, 39):
            bb, src = synth.ddp_bucket_ranks(b, n)
            xs = [base[bb][src[r]] for r in range(n)]
            want = oracle.ring_allreduce(xs, "sum", "bfloat16", nchannels=nch)
            got = G.to_host(recvs[b][b % n], "bfloat16")
            mm = G.first_mismatch(got, want[b % n], "bfloat16")
            assert mm is None, f"bucket {b}: {mm}"
            exact = np.sum(np.stack([oracle.bf16_to_f64(x) for x in xs]), axis=0)
            g64 = oracle.bf16_to_f64(got)
            assert np.linalg.norm(g64 - exact) / np.linalg.norm(exact) <= 8e-3
    finally:
        rs.comm_destroy(comm)


@pytest.mark.parametrize("choice", ["threshold", "auto"])
@pytest.mark.parametrize("op", ["sum", "max"])
def test_workload4_size_sweep(op, choice):
    """16 ranks, int32 in [-2^20, 2^20], 8 B .. 256 MiB per rank, 16 channels.
    "threshold": the ring, flag-packed below 64 KiB and bulk above (the
    sweep's own fixed threshold); "auto": whatever algorithm, protocol and
    workgroups the cost model takes (the tree, FLAG, WIDE or BULK). Integer
    sums and maxima do not depend on the fold order, so both equal the ring
    oracle."""
    import torch

    n, nch = 16, 16
    if choice == "threshold":
        comm = rs.comm_init(n, nch, "auto", flag_threshold_bytes=65536, algo="ring")
    else:
        comm = rs.comm_init(n, nch, "auto")
    try:
        for k, size in enumerate(synth.WORKLOADS[4]["sizes_bytes"]):
            count = size // 4
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
                idx = _sample_idx(count, 50_000, k)
                cols = [_host_at(t, idx, "int32") for t in send]
                want = oracle.ring_allreduce(cols, op, "int32", nchannels=1)[0]
                got = _host_at(recv[k % n], idx, "int32")
                assert np.array_equal(got, want), f"size {size}"
            del send, recv
    finally:
        rs.comm_destroy(comm)


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
        # reduce-scatter: block b folded b+1, ..., b -- the oracle's reduce to root b
        for b in range(n):
            idx = _sample_idx(rc, 20_000, 100 + b)
            cols = [_host_at(t, idx + b * rc, "bfloat16") for t in send]
            want = oracle.reduce(cols, b, "sum", "bfloat16")
            got = _host_at(shard[b], idx, "bfloat16")
            assert np.array_equal(got, want), f"block {b}"
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
