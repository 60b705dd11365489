"""HIP graph capture of collective calls (MI355X only).

A sequence of calls that covers every kernel family (FLAG, WIDE and BULK
ring all-reduces, the double-tree all-reduce, reduce-scatter, all-gather and
all-to-all) is captured once into a torch.cuda.CUDAGraph, which is a hipGraph
on ROCm, and launched several times. Between launches the host writes fresh
seeded inputs into the captured send buffers, refills the receive buffers
with a byte pattern and runs a direct call on the same communicator, with a
device synchronization after each step; every launch and every direct call
is compared bit for bit with the oracle on its own inputs. The library's
calls enqueue kernel launches only and each kernel takes its FIFO positions
from the persistent counters, so captured and direct calls interleave
freely."""
import numpy as np
import pytest

import oracle
import ring_all_reduce_allreduce_amd as rs
from tests import _gpu as G

pytestmark = pytest.mark.gpu

N, NCH = 8, 8
BULK, FLAG, WIDE = 1, 2, 3
RING, TREE = 1, 2

# (collective, dtype, elements per send buffer, op, expected all-reduce (algo, proto))
CASES = [
    ("allreduce", "float32", 1000, "sum", (RING, FLAG)),
    ("allreduce", "float32", 1 << 16, "sum", (RING, WIDE)),
    ("allreduce", "float32", 1 << 21, "sum", (RING, BULK)),
    ("allreduce", "int32", 4096, "max", (TREE, None)),
    ("reduce_scatter", "bfloat16", N * 3000, "sum", (None, None)),
    ("all_gather", "bfloat16", 3000, None, (None, None)),
    ("alltoall", "float32", N * 500, None, (None, None)),
]


@pytest.fixture(scope="module", autouse=True)
def _device():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    rs.lib()
    yield
    torch.cuda.synchronize()


def _inputs(dtype, count, seed):
    rng = np.random.default_rng(seed)
    if dtype == "int32":
        return [rng.integers(-(1 << 20), 1 << 20, count, endpoint=True).astype(np.int32) for _ in range(N)]
    f = [(rng.standard_normal(count) * np.exp2(rng.integers(-4, 12, count))).astype(np.float32) for _ in range(N)]
    if dtype == "bfloat16":
        import synth

        return [synth.f32_to_bf16_bits(x) for x in f]
    return f


def _out_count(coll, m):
    return {"allreduce": m, "reduce_scatter": m // N, "all_gather": m * N, "alltoall": m}[coll]


def _want(coll, dtype, op, xs):
    if coll == "allreduce" and dtype == "int32":
        return oracle.tree_allreduce(xs, op, dtype)
    if coll == "allreduce":
        return oracle.ring_allreduce(xs, op, dtype, nchannels=NCH)
    if coll == "reduce_scatter":
        return oracle.ring_reduce_scatter(xs, op, dtype, nchannels=NCH)
    if coll == "all_gather":
        return oracle.ring_all_gather(xs, dtype, nchannels=NCH)
    return oracle.alltoall(xs, dtype)


def _call(comm, coll, op, send, recv):
    if coll == "allreduce":
        rs.allreduce(comm, send, recv, op=op)
    elif coll == "reduce_scatter":
        rs.reduce_scatter(comm, send, recv, op=op)
    elif coll == "all_gather":
        rs.all_gather(comm, send, recv)
    else:
        rs.alltoall(comm, send, recv, count=send[0].numel() // N)


def _load(bufs, xs, dtype):
    for t, x in zip(bufs, xs):
        t.copy_(G.to_device(x, dtype))


def _check(recv, want, dtype, what):
    for r in range(N):
        got = G.to_host(recv[r], dtype)
        assert G.first_mismatch(got, want[r], dtype) is None, (what, r, G.first_mismatch(got, want[r], dtype))


def test_graph_launches_match_the_oracle_between_direct_calls():
    import torch

    comm = rs.comm_init(N, NCH, "auto")
    try:
        bufs = []
        for coll, dtype, m, op, _ in CASES:
            send = [G.empty_like_rank(m, dtype, 0) for _ in range(N)]
            recv = [G.empty_like_rank(_out_count(coll, m), dtype) for _ in range(N)]
            bufs.append((send, recv))
        G.sync()
        graph = torch.cuda.CUDAGraph()
        G.say(f"capture {len(CASES)} calls, N={N} C={NCH}")
        with torch.cuda.graph(graph):
            for (coll, dtype, m, op, (algo, proto)), (send, recv) in zip(CASES, bufs):
                _call(comm, coll, op, send, recv)
                info = rs.comm_query(comm)
                if algo is not None:
                    assert info["last_algo"] == algo, (coll, dtype, m, info["last_algo"])
                if proto is not None:
                    assert info["last_proto"] == proto, (coll, dtype, m, info["last_proto"])
        G.sync()
        for launch in range(3):
            # fresh inputs in the captured buffers, patterned outputs
            wants = []
            for k, ((coll, dtype, m, op, _), (send, recv)) in enumerate(zip(CASES, bufs)):
                xs = _inputs(dtype, m, 9000 + 100 * launch + k)
                _load(send, xs, dtype)
                for t in recv:
                    t.view(torch.uint8).fill_(0x7F)
                wants.append(_want(coll, dtype, op, xs))
            G.sync()
            G.say(f"graph launch {launch}")
            graph.replay()
            G.sync()
            G.check_comm_ok(comm)
            for (coll, dtype, m, op, _), (send, recv), want in zip(CASES, bufs, wants):
                _check(recv, want, dtype, f"launch {launch}: {coll} {dtype} x{m}")
            # a direct call between launches moves the same counters on
            coll, dtype, m, op, _ = CASES[launch % 3]
            xs = _inputs(dtype, m, 7000 + launch)
            send = [G.to_device(x, dtype) for x in xs]
            recv = [G.empty_like_rank(m, dtype) for _ in range(N)]
            G.say(f"direct call after launch {launch}: {coll} {dtype} x{m}")
            _call(comm, coll, op, send, recv)
            G.sync()
            G.check_comm_ok(comm)
            _check(recv, _want(coll, dtype, op, xs), dtype, f"direct after launch {launch}")
    finally:
        rs.comm_destroy(comm)


def test_async_error_during_capture_leaves_the_capture_intact():
    """Querying the communicator while its stream is captured reports the
    known errors only; the capture still completes and launches correctly."""
    import torch

    comm = rs.comm_init(N, NCH, "auto")
    try:
        dtype, m = "float32", 4096
        send = [G.empty_like_rank(m, dtype, 0) for _ in range(N)]
        recv = [G.empty_like_rank(m, dtype) for _ in range(N)]
        G.sync()
        graph = torch.cuda.CUDAGraph()
        G.say("capture with an async-error query inside")
        with torch.cuda.graph(graph):
            rs.allreduce(comm, send, recv, op="sum")
            assert rs.get_async_error(comm) == rs.SUCCESS
        G.sync()
        xs = _inputs(dtype, m, 4242)
        _load(send, xs, dtype)
        G.sync()
        graph.replay()
        G.sync()
        G.check_comm_ok(comm)
        _check(recv, oracle.ring_allreduce(xs, "sum", dtype, nchannels=NCH), dtype, "captured with query")
    finally:
        rs.comm_destroy(comm)
