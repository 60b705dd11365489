"""The allocation-free all-reduce (MI355X only): its result equals the
communicator all-reduce's bit for bit on the same inputs (same partition,
same fold order), on two calls in a row, the second with a smaller input;
shapes beyond the scratch limit are refused before anything is launched."""
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


def _inputs(n, count, dtype, seed):
    rng = np.random.default_rng(seed)
    if dtype == "int32":
        return [rng.integers(-(1 << 20), 1 << 20, count, endpoint=True).astype(np.int32) for _ in range(n)]
    f = [rng.standard_normal(count).astype(np.float32) for _ in range(n)]
    return [synth.f32_to_bf16_bits(x) for x in f] if dtype == "bfloat16" else f


def _comm_allreduce(xs, dtype, op, nchannels):
    """The existing entry point: a communicator's ring all-reduce."""
    n, count = len(xs), xs[0].shape[0]
    comm = rs.comm_init(n, nchannels, "bulk", algo="ring")
    try:
        send = [G.to_device(x, dtype) for x in xs]
        recv = [G.empty_like_rank(count, dtype) for _ in range(n)]
        rs.allreduce(comm, send, recv, op=op)
        G.sync()
        G.check_comm_ok(comm)
        return [G.to_host(t, dtype) for t in recv]
    finally:
        rs.comm_destroy(comm)


def _noalloc_allreduce(xs, dtype, op, nchannels):
    n, count = len(xs), xs[0].shape[0]
    send = [G.to_device(x, dtype) for x in xs]
    recv = [G.empty_like_rank(count, dtype, fill_bits=0x5A) for _ in range(n)]
    rs.allreduce_noalloc(n, nchannels, send, recv, op=op)
    G.sync()
    return [G.to_host(t, dtype) for t in recv]


def _assert_same(got, want, dtype, what):
    for r, (g, w) in enumerate(zip(got, want)):
        mm = G.first_mismatch(g, w, dtype)
        assert mm is None, f"{what}: rank {r} first mismatch at {mm}"


# (dtype, op, first call (ranks, channels, count), second, smaller call)
CASES = [
    ("float32", "sum", (8, 8, 4_194_307), (8, 4, 70_001)),
    ("bfloat16", "sum", (8, 16, 2_621_451), (4, 2, 1_027)),
    ("int32", "max", (16, 8, 1_048_583), (3, 1, 17)),
]


@pytest.mark.parametrize("dtype,op,first,second", CASES, ids=[c[0] for c in CASES])
def test_noalloc_equals_comm_allreduce_twice(dtype, op, first, second):
    for k, (n, nch, count) in enumerate((first, second)):
        G.say(f"allreduce_noalloc call {k} N={n} C={nch} count={count} dtype={dtype} op={op}")
        xs = _inputs(n, count, dtype, seed=7000 + 10 * k + n)
        got = _noalloc_allreduce(xs, dtype, op, nch)
        want = _comm_allreduce(xs, dtype, op, nch)
        _assert_same(got, want, dtype, f"call {k} N={n} C={nch} count={count}")


def test_noalloc_matches_oracle_small():
    xs = _inputs(5, 3001, "float32", seed=7100)
    G.say("allreduce_noalloc N=5 C=2 count=3001 float32 vs oracle")
    got = _noalloc_allreduce(xs, "float32", "sum", 2)
    want = oracle.ring_allreduce(xs, "sum", "float32", nchannels=2)
    _assert_same(got, want, "float32", "vs oracle")


def test_noalloc_refuses_shapes_beyond_its_scratch():
    import torch

    send = [torch.zeros(64, dtype=torch.float32, device="cuda:0") for _ in range(16)]
    recv = [torch.empty_like(t) for t in send]
    with pytest.raises(rs.RingsimError) as e:
        rs.allreduce_noalloc(16, 16, send, recv)  # 256 ring pipelines > 128
    assert e.value.name == "INVALID_ARGUMENT"
    # count == 0 is a no-op, and a single rank is a plain copy
    rs.allreduce_noalloc(16, 8, send, recv, count=0)
    rs.allreduce_noalloc(1, 1, send[:1], recv[:1])
    G.sync()
    assert torch.equal(recv[0], send[0])
