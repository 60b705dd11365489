"""A collective overlapped with compute (MI355X only).

Data-parallel training all-reduces gradient buckets on a stream of their own
while the backward pass keeps computing ("AI Systems Performance Engineering
(3)", Overlapping Communication and Computation; "NCCL 专家课程 29": the
collective runs on its own stream). Here one stream runs a chain of bf16
matrix products (~20 ms) while a second stream all-reduces four 25 MiB bf16
buckets of 8 ranks. Every workgroup of a ring launch spins on its
neighbours, so a launch whose workgroups cannot all find a compute unit
waits for the products to free some: the test checks that both sides finish,
that the communicator reports no error and that a bucket is bit-exact
against the oracle, and prints each side's time alone and overlapped."""
import pytest

import oracle
import ring_all_reduce_allreduce_amd as rs
import synth
from tests import _gpu as G

pytestmark = pytest.mark.gpu

N, COUNT, NCH, BUCKETS = 8, 13_107_200, 16, 4
WORKLOAD = 3  # the DDP bucket workload's seed space


def _timed(stream, fn):
    import torch

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record()
        fn()
        e1.record()
    return e0, e1


def test_bucket_allreduce_overlapped_with_matmuls():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    comp, comm_stream = torch.cuda.Stream(), torch.cuda.Stream()
    a = torch.randn(4096, 4096, device="cuda:0").to(torch.bfloat16).contiguous()
    b = torch.randn(4096, 4096, device="cuda:0").to(torch.bfloat16).contiguous()
    outs = [torch.empty(4096, 4096, device="cuda:0", dtype=torch.bfloat16) for _ in range(2)]
    buckets = [synth.device_inputs(WORKLOAD, N, COUNT, "bfloat16", "normal", scale=1e-3, bucket=k)
               for k in range(BUCKETS)]
    recvs = [[torch.empty_like(t) for t in bk] for bk in buckets]
    comm = rs.comm_init(N, NCH, "auto")
    try:
        def products(reps):
            for i in range(reps):
                torch.mm(a, b, out=outs[i % 2])

        def allreduces():
            for bk, rv in zip(buckets, recvs):
                rs.allreduce(comm, bk, rv, stream=comm_stream)

        # size the product chain to about 20 ms, warm both sides up
        products(4)
        allreduces()
        torch.cuda.synchronize()
        e0, e1 = _timed(comp, lambda: products(20))
        torch.cuda.synchronize()
        reps = max(20, int(20 * 20.0 / max(e0.elapsed_time(e1), 1e-3)))
        G.say(f"overlap: {reps} bf16 products of 4096^2 against {BUCKETS} buckets of {N} x 25 MiB")
        c0, c1 = _timed(comp, lambda: products(reps))
        torch.cuda.synchronize()
        r0, r1 = _timed(comm_stream, allreduces)
        torch.cuda.synchronize()
        alone = (c0.elapsed_time(c1), r0.elapsed_time(r1))
        # overlapped: the products start first, the buckets follow at once
        c0, c1 = _timed(comp, lambda: products(reps))
        r0, r1 = _timed(comm_stream, allreduces)
        torch.cuda.synchronize()
        both = (c0.elapsed_time(c1), r0.elapsed_time(r1))
        G.check_comm_ok(comm)
        G.say(f"alone: products {alone[0]:.2f} ms, all-reduces {alone[1]:.3f} ms; overlapped: products "
              f"{both[0]:.2f} ms, all-reduces {both[1]:.3f} ms (from their own launch to their end)")
        # the last bucket of the overlapped run, against the oracle
        xs = [G.to_host(t, "bfloat16") for t in buckets[-1]]
        want = oracle.ring_allreduce(xs, "sum", "bfloat16", nchannels=NCH)
        for r in (0, N - 1):
            mm = G.first_mismatch(G.to_host(recvs[-1][r], "bfloat16"), want[r], "bfloat16")
            assert mm is None, f"rank {r}: first mismatch {mm}"
        assert both[0] < 20 * alone[0] and both[1] < 1000.0, (alone, both)
    finally:
        rs.comm_destroy(comm)
