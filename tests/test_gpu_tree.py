"""Parity of the HIP double-binary-tree all-reduce with the CPU oracle
(MI355X only). Every case runs the library through its C ABI and compares
each rank's result bit for bit with ``oracle.tree_allreduce`` on the same
seeded inputs."""
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


def _inputs(n, count, dtype, seed, op="sum"):
    rng = np.random.default_rng(seed)
    if dtype in ("int32", "int64"):
        lo, hi = (-3, 3) if op == "prod" else (-(1 << 20), 1 << 20)
        return [rng.integers(lo, hi, count, endpoint=True).astype(oracle.STORAGE[dtype]) for _ in range(n)]
    if op == "prod":
        f = [(1.0 + 0.01 * rng.standard_normal(count)).astype(np.float32) for _ in range(n)]
    else:
        # mixed magnitudes, so that a different fold order shows in the bits
        f = [(rng.standard_normal(count) * np.exp2(rng.integers(-4, 20, count))).astype(np.float32) for _ in range(n)]
    return [synth.f32_to_bf16_bits(x) for x in f] if dtype == "bfloat16" else f


def _run(comm, xs, dtype, op, inplace=False, offset=0):
    n, count = len(xs), xs[0].shape[0]
    if offset:
        # element-aligned but not 16-byte aligned buffers
        e = oracle.ELEM_SIZE[dtype]
        k = offset // e
        send = []
        for x in xs:
            big = G.to_device(np.concatenate([np.zeros(k, dtype=x.dtype), x]), dtype)
            send.append(big[k:])
        recv = send if inplace else [G.empty_like_rank(count + k, dtype)[k:] for _ in range(n)]
    else:
        send = [G.to_device(x, dtype) for x in xs]
        recv = send if inplace else [G.empty_like_rank(count, dtype) for _ in range(n)]
    rs.allreduce(comm, send, recv, op=op)
    G.sync()
    G.check_comm_ok(comm)
    return [G.to_host(t, dtype) for t in recv]


def _assert_tree(got, xs, dtype, op, what):
    want = oracle.tree_allreduce(xs, op, dtype)
    for r in range(len(xs)):
        mm = G.first_mismatch(got[r], want[r], dtype)
        assert mm is None, f"{what}: rank {r} first mismatch {mm}"


@pytest.mark.parametrize("dtype", ["float32", "bfloat16", "int32", "int64"])
def test_tree_matrix(dtype):
    for n in (2, 3, 5, 8, 16):
        comm = rs.comm_init(n, 4, "auto", algo="tree")
        try:
            for count in (1, 5, 17, 1027, 40_003):
                ops = ("sum", "max", "min", "prod") if n in (3, 8) else ("sum",)
                for op in ops:
                    xs = _inputs(n, count, dtype, 7 * n + count, op)
                    G.say(f"tree N={n} count={count} dtype={dtype} op={op}")
                    got = _run(comm, xs, dtype, op)
                    assert rs.comm_query(comm)["last_algo"] == 2
                    _assert_tree(got, xs, dtype, op, f"N={n} count={count} {op}")
        finally:
            rs.comm_destroy(comm)


@pytest.mark.parametrize("dtype", ["float32", "int32"])
def test_tree_maximum_ranks(dtype):
    """RINGSIM_MAX_RANKS (64) ranks: trees of depth 6 in which every rank is
    a leaf of exactly one of the two trees, one or two tree channels per
    call (64 ranks x 4 workgroups already fill the device once)."""
    n = rs.MAX_RANKS
    comm = rs.comm_init(n, 4, "auto", algo="tree")
    try:
        for count in (1, 1027, 40_003):
            xs = _inputs(n, count, dtype, 3000 + count)
            G.say(f"tree N={n} count={count} dtype={dtype}")
            got = _run(comm, xs, dtype, "sum")
            assert rs.comm_query(comm)["last_algo"] == 2
            _assert_tree(got, xs, dtype, "sum", f"N={n} count={count}")
    finally:
        rs.comm_destroy(comm)


def test_tree_many_slices_flow_control():
    """4 MiB per rank over 8 tree channels (two per ring channel): 86 steps
    of 3 KiB per channel, five times the FIFO depth, so every producer waits
    on its consumer's head."""
    n, count = 8, 1 << 20
    comm = rs.comm_init(n, 4, "auto", algo="tree")
    try:
        assert rs.comm_query(comm)["tree_channels"] == 8
        for dtype in ("float32", "int32"):
            xs = _inputs(n, count, dtype, 99)
            G.say(f"tree flow control N={n} count={count} dtype={dtype}")
            got = _run(comm, xs, dtype, "sum")
            _assert_tree(got, xs, dtype, "sum", dtype)
    finally:
        rs.comm_destroy(comm)


def test_tree_inplace_unaligned_and_mixed_with_ring():
    """In-place and 4-byte-offset buffers, then ring and tree calls
    alternating on one communicator (separate FIFOs, persistent counters)."""
    n = 6
    comm = rs.comm_init(n, 2, "auto", algo="tree")
    ring = rs.comm_init(n, 2, "auto", algo="ring")
    try:
        for count, inplace, offset in ((3001, True, 0), (3001, False, 4), (257, True, 4)):
            xs = _inputs(n, count, "float32", count + offset)
            G.say(f"tree N={n} count={count} inplace={inplace} offset={offset}")
            got = _run(comm, xs, "float32", "sum", inplace=inplace, offset=offset)
            _assert_tree(got, xs, "float32", "sum", f"inplace={inplace} offset={offset}")
        for k in range(6):
            count = 500 + 977 * k
            xs = _inputs(n, count, "float32", 1000 + k)
            G.say(f"alternate k={k} count={count}")
            got_t = _run(comm, xs, "float32", "sum")
            _assert_tree(got_t, xs, "float32", "sum", f"tree k={k}")
            got_r = _run(ring, xs, "float32", "sum")
            want_r = oracle.ring_allreduce(xs, "sum", "float32", nchannels=2)
            for r in range(n):
                assert G.first_mismatch(got_r[r], want_r[r], "float32") is None, (k, r)
    finally:
        rs.comm_destroy(comm)
        rs.comm_destroy(ring)


def test_auto_takes_the_tree_only_where_order_cannot_show():
    """AUTO at 16 ranks: tiny int32 sums and fp32 maxima go to the tree (both
    are order-free), tiny fp32 sums stay on the ring, and every result equals
    the order-independent reference or the ring oracle."""
    n, nch = 16, 16
    comm = rs.comm_init(n, nch, "auto")
    try:
        for count in (2, 1000, 4096):
            xi = _inputs(n, count, "int32", count)
            G.say(f"auto int32 sum count={count}")
            got = _run(comm, xi, "int32", "sum")
            assert rs.comm_query(comm)["last_algo"] == 2
            want = np.sum(np.stack(xi).astype(np.int64), axis=0).astype(np.int32)
            assert all(np.array_equal(g, want) for g in got)
            xf = _inputs(n, count, "float32", count + 1)
            G.say(f"auto fp32 max count={count}")
            got = _run(comm, xf, "float32", "max")
            assert rs.comm_query(comm)["last_algo"] == 2
            want = np.max(np.stack(xf), axis=0)
            assert all(G.bits_equal(g, want, "float32") for g in got)
            G.say(f"auto fp32 sum count={count}")
            got = _run(comm, xf, "float32", "sum")
            assert rs.comm_query(comm)["last_algo"] == 1
            want = oracle.ring_allreduce(xf, "sum", "float32", nchannels=nch)
            assert all(G.first_mismatch(g, w, "float32") is None for g, w in zip(got, want))
    finally:
        rs.comm_destroy(comm)


def test_tree_degenerate_shapes():
    import torch

    # one rank: a local copy; zero elements: a no-op
    comm = rs.comm_init(1, 1, "auto", algo="tree")
    try:
        x = _inputs(1, 100, "float32", 1)
        got = _run(comm, x, "float32", "sum")
        assert G.bits_equal(got[0], x[0], "float32")
    finally:
        rs.comm_destroy(comm)
    comm = rs.comm_init(4, 2, "auto", algo="tree")
    try:
        bufs = [torch.zeros(4, device="cuda:0") for _ in range(4)]
        rs.allreduce(comm, bufs, bufs, count=0)
        G.sync()
        G.check_comm_ok(comm)
        # a count that leaves tree 1 empty (h = count) and one that leaves
        # most channels empty
        for count in (3, 4, 9):
            xs = _inputs(4, count, "float32", 50 + count)
            got = _run(comm, xs, "float32", "sum")
            _assert_tree(got, xs, "float32", "sum", f"count={count}")
    finally:
        rs.comm_destroy(comm)


@pytest.mark.parametrize("dtype", ["int32", "bfloat16", "int64"])
def test_tree_channel_and_slice_boundaries(dtype):
    """A channel carries its share of a tree's half in steps of one WIDE line
    per thread: 3 KiB of payload (2 KiB for int64). Tree 0 takes the larger
    half; a half of exactly one step takes one channel and one 16-byte
    vector more takes two; a half of exactly eight steps fills the eight
    tree channels (two per ring channel) with one step each and one vector
    more gives the first channel a second, short step. Every case must be
    whole and bit-exact."""
    e = {"int32": 4, "bfloat16": 2, "int64": 8}[dtype]
    step_bytes = 256 * (8 if e == 8 else 12)
    n = 8
    comm = rs.comm_init(n, 4, "auto", algo="tree")
    try:
        for steps, channels in ((1, (1, 2)), (8, (8, 8))):
            for extra, want_channels in zip((0, 16 // e), channels):
                count = 2 * (steps * step_bytes // e + extra)
                xs = _inputs(n, count, dtype, 1600 + count)
                G.say(f"tree boundary {dtype} count={count}")
                got = _run(comm, xs, dtype, "sum")
                assert rs.comm_query(comm)["last_tree_channels"] == want_channels
                _assert_tree(got, xs, dtype, "sum", f"tree boundary count={count}")
    finally:
        rs.comm_destroy(comm)
