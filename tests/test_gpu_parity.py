"""Parity of the HIP ring collectives with the CPU oracle (MI355X only).

Every case runs the library through its C ABI on seeded synthetic inputs and
compares the device result element by element with the oracle's replay of
the same ring order: bit-exact for every dtype (the oracle rounds each hop
exactly as the ring does), plus the fp64 error bounds for floating point.
"""
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


def _inputs(n, count, dtype, seed, kind="normal"):
    rng = np.random.default_rng(seed)
    if dtype in ("int32", "int64"):
        info = np.iinfo(np.int32 if dtype == "int32" else np.int64)
        lo, hi = (-(1 << 20), 1 << 20) if kind == "normal" else (info.min, info.max)
        return [rng.integers(lo, hi, count, endpoint=True).astype(oracle.STORAGE[dtype]) for _ in range(n)]
    f = [rng.standard_normal(count).astype(np.float32) for _ in range(n)]
    if dtype == "bfloat16":
        return [synth.f32_to_bf16_bits(x) for x in f]
    return f


def _run_allreduce(xs, dtype, op, nchannels, proto, chunk_bytes=None, inplace=False, **cfg):
    n = len(xs)
    count = xs[0].shape[0]
    G.say(f"allreduce N={n} count={count} dtype={dtype} op={op} C={nchannels} proto={proto} "
          f"chunk={chunk_bytes} inplace={inplace} cfg={cfg}")
    comm = rs.comm_init(n, nchannels, proto, chunk_bytes=chunk_bytes, **cfg)
    try:
        send = [G.to_device(x, dtype) for x in xs]
        recv = send if inplace else [G.empty_like_rank(count, dtype) for _ in range(n)]
        rs.allreduce(comm, send, recv, op=op)
        G.sync()
        G.check_comm_ok(comm)
        return [G.to_host(t, dtype) for t in recv]
    finally:
        rs.comm_destroy(comm)


def _assert_same(got, want, dtype, what):
    for r, (g, w) in enumerate(zip(got, want)):
        mm = G.first_mismatch(g, w, dtype)
        assert mm is None, f"{what}: rank {r} first mismatch at {mm}"


def test_workload1_exact():
    xs = synth.workload_inputs(1)
    got = _run_allreduce(xs, "float32", "sum", 1, "bulk")
    want = oracle.ring_allreduce(xs, "sum", "float32", nchannels=1)
    _assert_same(got, want, "float32", "workload 1")
    exact = np.sum(np.stack(xs).astype(np.int64), axis=0).astype(np.float32)
    assert np.array_equal(got[0], exact)


@pytest.mark.parametrize("proto", ["bulk", "flag", "wide"])
@pytest.mark.parametrize("dtype", ["float32", "bfloat16", "int32", "int64"])
def test_allreduce_matrix(proto, dtype):
    seed = 100
    for n in (2, 3, 8):
        for count, nch, chunk in ((1, 1, 4096), (1000, 3, 4096), (100_003, 3, 4096), (70_001, 2, 524_288)):
            ops = ("sum", "max") if n != 3 else ("sum", "min", "prod")
            for op in ops:
                seed += 1
                xs = _inputs(n, count, dtype, seed)
                got = _run_allreduce(xs, dtype, op, nch, proto, chunk_bytes=chunk)
                want = oracle.ring_allreduce(xs, op, dtype, nchannels=nch, chunk_bytes=chunk)
                _assert_same(got, want, dtype, f"N={n} count={count} C={nch} op={op}")


@pytest.mark.parametrize("proto", ["bulk", "flag", "wide"])
def test_allreduce_inplace_and_unaligned(proto):
    import torch

    n, count, dtype = 4, 50_001, "float32"
    xs = _inputs(n, count, dtype, 7)
    want = oracle.ring_allreduce(xs, "sum", dtype, nchannels=2, chunk_bytes=8192)
    got = _run_allreduce(xs, dtype, "sum", 2, proto, chunk_bytes=8192, inplace=True)
    _assert_same(got, want, dtype, "in place")
    # buffers offset by one element: element-wise path
    G.say(f"allreduce unaligned proto={proto}")
    comm = rs.comm_init(n, 2, proto, chunk_bytes=8192)
    try:
        base_s = [torch.zeros(count + 1, dtype=torch.float32, device="cuda:0") for _ in range(n)]
        base_r = [torch.zeros(count + 1, dtype=torch.float32, device="cuda:0") for _ in range(n)]
        for b, x in zip(base_s, xs):
            b[1:].copy_(torch.from_numpy(x))
        rs.allreduce(comm, [b[1:] for b in base_s], [b[1:] for b in base_r])
        G.sync()
        G.check_comm_ok(comm)
        _assert_same([b[1:].cpu().numpy() for b in base_r], want, dtype, "unaligned")
    finally:
        rs.comm_destroy(comm)


@pytest.mark.parametrize("proto", ["bulk", "flag", "wide"])
@pytest.mark.parametrize("dtype", ["float32", "bfloat16", "int64"])
def test_reduce_scatter(proto, dtype):
    for n, rc, nch in ((2, 5000, 1), (5, 33_333, 3), (8, 65_536, 4)):
        xs = _inputs(n, n * rc, dtype, 300 + n)
        G.say(f"reduce_scatter N={n} recvcount={rc} dtype={dtype} C={nch} proto={proto}")
        comm = rs.comm_init(n, nch, proto, chunk_bytes=16384)
        try:
            send = [G.to_device(x, dtype) for x in xs]
            recv = [G.empty_like_rank(rc, dtype) for _ in range(n)]
            rs.reduce_scatter(comm, send, recv, op="sum")
            G.sync()
            G.check_comm_ok(comm)
            got = [G.to_host(t, dtype) for t in recv]
        finally:
            rs.comm_destroy(comm)
        want = oracle.ring_reduce_scatter(xs, "sum", dtype, nchannels=nch, chunk_bytes=16384)
        _assert_same(got, want, dtype, f"reduce_scatter N={n}")


@pytest.mark.parametrize("proto", ["bulk", "flag", "wide"])
def test_all_gather(proto):
    for n, sc, nch, dtype in ((2, 777, 1, "bfloat16"), (6, 40_000, 3, "int32"), (8, 131_072, 8, "float32")):
        xs = _inputs(n, sc, dtype, 400 + n)
        G.say(f"all_gather N={n} sendcount={sc} dtype={dtype} C={nch} proto={proto}")
        comm = rs.comm_init(n, nch, proto, chunk_bytes=32768)
        try:
            send = [G.to_device(x, dtype) for x in xs]
            recv = [G.empty_like_rank(n * sc, dtype) for _ in range(n)]
            rs.all_gather(comm, send, recv)
            G.sync()
            G.check_comm_ok(comm)
            got = [G.to_host(t, dtype) for t in recv]
        finally:
            rs.comm_destroy(comm)
        want = oracle.ring_all_gather(xs, dtype, nchannels=nch, chunk_bytes=32768)
        _assert_same(got, want, dtype, f"all_gather N={n}")


def test_alltoall():
    """Blocks of every alignment: whole 16-byte vectors, 8-, 4- and 2-byte
    units (block sizes that are no multiple of 16 bytes), and buffers that
    start off a 16-byte boundary (shift = elements of offset)."""
    for n, cnt, dtype, shift in ((1, 100, "float32", 0), (3, 1001, "bfloat16", 0), (8, 65_536, "bfloat16", 0),
                                 (4, 3, "int64", 0), (5, 1001, "float32", 0), (2, 7, "int32", 0),
                                 (4, 4096, "bfloat16", 1), (3, 2048, "float32", 3)):
        xs = _inputs(n, n * cnt, dtype, 500 + n + shift)
        G.say(f"alltoall N={n} count={cnt} dtype={dtype} shift={shift}")
        comm = rs.comm_init(n, 1, "auto")
        try:
            send = [G.to_device(np.concatenate([np.zeros(shift, x.dtype), x]), dtype)[shift:] for x in xs]
            recv = [G.empty_like_rank(n * cnt + shift, dtype)[shift:] for _ in range(n)]
            rs.alltoall(comm, send, recv)
            G.sync()
            G.check_comm_ok(comm)
            got = [G.to_host(t, dtype) for t in recv]
        finally:
            rs.comm_destroy(comm)
        _assert_same(got, oracle.alltoall(xs, dtype), dtype, f"alltoall N={n}")


def test_degenerate_shapes():
    # one rank: local copy; zero count: no-op; 16 ranks x 2 elements: most chunks empty
    for n, count, nch, proto in ((1, 1000, 1, "bulk"), (16, 2, 16, "bulk"), (16, 2, 16, "flag"),
                                 (16, 5, 1, "bulk"), (7, 13, 4, "flag"), (16, 2, 16, "wide"), (7, 13, 4, "wide"),
                                 (5, 1, 3, "wide")):
        xs = _inputs(n, count, "int32", 600 + n + count)
        got = _run_allreduce(xs, "int32", "sum", nch, proto)
        want = oracle.ring_allreduce(xs, "sum", "int32", nchannels=nch)
        _assert_same(got, want, "int32", f"degenerate N={n} count={count}")
    comm = rs.comm_init(4, 2, "auto")
    try:
        import torch

        t = [torch.zeros(0, device="cuda:0") for _ in range(4)]
        rs.allreduce(comm, t, t, count=0)
        G.sync()
        G.check_comm_ok(comm)
    finally:
        rs.comm_destroy(comm)


@pytest.mark.parametrize("proto", ["bulk", "flag", "wide"])
def test_maximum_ranks_and_channels(proto):
    """The limits of the ABI: RINGSIM_MAX_RANKS (64) ranks over 4 channels,
    and RINGSIM_MAX_CHANNELS (64) channels over 4 ranks, with ragged counts
    that span several loops per channel."""
    for n, nch, count in ((rs.MAX_RANKS, 4, 64 * 4 * 300 + 37), (4, rs.MAX_CHANNELS, 64 * 4 * 300 + 5)):
        xs = _inputs(n, count, "float32", 900 + n)
        got = _run_allreduce(xs, "float32", "sum", nch, proto, chunk_bytes=1024)
        want = oracle.ring_allreduce(xs, "sum", "float32", nchannels=nch, chunk_bytes=1024)
        _assert_same(got, want, "float32", f"limits N={n} C={nch} proto={proto}")


def test_back_to_back_calls_one_stream():
    # many collectives of different shapes and both protocols on one stream:
    # the FIFO counters carry over from call to call
    n, dtype = 8, "float32"
    comm = rs.comm_init(n, 4, "auto", chunk_bytes=16384)
    try:
        cases = []
        for k in range(24):
            count = [10, 3000, 20_000, 250_000][k % 4] + k
            xs = _inputs(n, count, dtype, 700 + k)
            send = [G.to_device(x, dtype) for x in xs]
            recv = [G.empty_like_rank(count, dtype) for _ in range(n)]
            G.say(f"back-to-back call {k} count={count}")
            rs.allreduce(comm, send, recv)
            cases.append((xs, recv, count))
        G.sync()
        G.check_comm_ok(comm)
        for xs, recv, count in cases:
            proto_chunk = 16384
            want = oracle.ring_allreduce(xs, "sum", dtype, nchannels=4, chunk_bytes=proto_chunk)
            _assert_same([G.to_host(t, dtype) for t in recv], want, dtype, f"back-to-back count={count}")
    finally:
        rs.comm_destroy(comm)


def test_workload2_full_size():
    w = synth.WORKLOADS[2]
    xs = synth.workload_inputs(2)
    got = _run_allreduce(xs, "float32", "sum", w["nchannels"], "bulk", chunk_bytes=w["chunk_bytes"])
    want = oracle.ring_allreduce(xs, "sum", "float32", nchannels=w["nchannels"], chunk_bytes=w["chunk_bytes"])
    _assert_same(got, want, "float32", "workload 2")
    st = np.stack(xs).astype(np.float64)
    err = np.abs(got[3].astype(np.float64) - st.sum(axis=0))
    assert np.all(err <= 1e-6 * np.abs(st).sum(axis=0))


def _random_float_bits(rng, count, dtype, exp_lo, exp_hi):
    """Finite values with random sign, mantissa and biased exponent in
    [exp_lo, exp_hi]; exponent 0 gives subnormals and signed zeros."""
    if dtype == "float32":
        mant = rng.integers(0, 1 << 23, count, dtype=np.uint64)
        exp = rng.integers(exp_lo, exp_hi + 1, count, dtype=np.uint64)
        sign = rng.integers(0, 2, count, dtype=np.uint64)
        bits = (sign << 31) | (exp << 23) | mant
        bits[::97] = 0                      # +0
        bits[1::97] = 1 << 31               # -0
        return bits.astype(np.uint32).view(np.float32)
    mant = rng.integers(0, 1 << 7, count, dtype=np.uint32)
    exp = rng.integers(exp_lo, exp_hi + 1, count, dtype=np.uint32)
    sign = rng.integers(0, 2, count, dtype=np.uint32)
    bits = (sign << 15) | (exp << 7) | mant
    bits[::97] = 0
    bits[1::97] = 1 << 15
    return bits.astype(np.uint16)


@pytest.mark.parametrize("proto", ["bulk", "flag", "wide"])
@pytest.mark.parametrize("dtype", ["float32", "bfloat16"])
def test_allreduce_random_bit_patterns(proto, dtype):
    """Subnormals, signed zeros, ties and wide exponent ranges: every hop must
    round exactly like the oracle (no flush to zero, no fused operations)."""
    rng = np.random.default_rng(2024)
    n, count, nch = 5, 20_011, 3
    for op, (lo, hi) in (("sum", (0, 200)), ("max", (0, 254)), ("min", (0, 254)), ("prod", (120, 134)),
                         ("sum", (0, 3))):
        xs = [_random_float_bits(rng, count, dtype, lo, hi) for _ in range(n)]
        got = _run_allreduce(xs, dtype, op, nch, proto, chunk_bytes=16384)
        want = oracle.ring_allreduce(xs, op, dtype, nchannels=nch, chunk_bytes=16384)
        _assert_same(got, want, dtype, f"{dtype} {op} exponents {lo}..{hi}")


@pytest.mark.parametrize("n,nch", [(16, 16), (8, 8), (4, 4)])
def test_auto_protocol_choice_does_not_change_results(n, nch):
    """Around the cost model's crossovers AUTO switches between protocols;
    every protocol walks the same 512 KiB chunks, so the bits equal the
    oracle's either way."""
    comm = rs.comm_init(n, nch, "auto")
    seen = set()
    try:
        for k, nbytes in enumerate((16 << 10, 64 << 10, 256 << 10, 512 << 10, 1 << 20, 2 << 20)):
            count = nbytes // 4 + 3  # ragged tail
            xs = _inputs(n, count, "float32", 1000 + k)
            G.say(f"auto N={n} C={nch} bytes/rank={nbytes}")
            send = [G.to_device(x, "float32") for x in xs]
            recv = [G.empty_like_rank(count, "float32") for _ in range(n)]
            rs.allreduce(comm, send, recv)
            G.sync()
            G.check_comm_ok(comm)
            seen.add(rs.comm_query(comm)["last_proto"])
            want = oracle.ring_allreduce(xs, "sum", "float32", nchannels=nch, chunk_bytes=524_288)
            _assert_same([G.to_host(t, "float32") for t in recv], want, "float32", f"auto {nbytes} B/rank")
    finally:
        rs.comm_destroy(comm)
    assert len(seen) >= 2, f"expected more than one protocol across the sizes, saw {seen}"


@pytest.mark.parametrize("dtype", ["float32", "bfloat16", "int64"])
def test_protocols_agree_across_groups_and_loops(dtype):
    """The line protocols walk every loop in groups of 8 slot steps; with the
    full 512 KiB chunk a stage holds several groups, and two loops (the
    second ragged) follow. All three protocols must give the oracle's bits
    for the same chunk."""
    n, nch, chunk = 4, 2, 524_288
    e = {"float32": 4, "bfloat16": 2, "int64": 8}[dtype]
    count = (2 * n * chunk + 3 * chunk // 2) // e + 5  # two full loops per channel pair, a ragged third
    xs = _inputs(n, count, dtype, 1200 + e)
    want = oracle.ring_allreduce(xs, "sum", dtype, nchannels=nch, chunk_bytes=chunk)
    for proto in ("bulk", "flag", "wide"):
        got = _run_allreduce(xs, dtype, "sum", nch, proto, chunk_bytes=chunk)
        _assert_same(got, want, dtype, f"{proto} {dtype} multi-group")


@pytest.mark.parametrize("proto", ["flag", "wide"])
@pytest.mark.parametrize("dtype", ["float32", "bfloat16", "int64"])
def test_line_kernel_variant_boundary(proto, dtype):
    """The host runs the alternating-halves kernel when no unit of the launch
    holds more than 128 lines, the one-line-per-thread kernel up to 256
    lines (2 KiB of FLAG payload, 3 KiB of WIDE payload, 2 KiB for int64
    lines) and the several-lines kernel above. Units of exactly each limit
    and one 16-byte vector more take different kernels; all must be whole and
    bit-exact, for the all-reduce, reduce-scatter and all-gather. One
    workgroup per channel, so that the unit is the step."""
    e = {"float32": 4, "bfloat16": 2, "int64": 8}[dtype]
    line_payload = 12 if proto == "wide" and dtype != "int64" else 8
    n = 4
    for lines, extra in ((128, 0), (128, 16 // e), (256, 0), (256, 16 // e)):
        unit = lines * line_payload // e + extra
        count = n * unit  # one tail loop per channel: chunk = unit
        xs = _inputs(n, count, dtype, 1300 + unit)
        got = _run_allreduce(xs, dtype, "sum", 1, proto, line_workgroups_per_channel=1)
        want = oracle.ring_allreduce(xs, "sum", dtype, nchannels=1)
        _assert_same(got, want, dtype, f"allreduce {proto} unit={unit}")
        # reduce-scatter / all-gather: one unit per loop of each block
        for coll in ("reduce_scatter", "all_gather"):
            comm = rs.comm_init(n, 1, proto, chunk_bytes=unit * e, line_workgroups_per_channel=1)
            try:
                if coll == "reduce_scatter":
                    src = _inputs(n, n * unit, dtype, 1400 + unit)
                    send = [G.to_device(x, dtype) for x in src]
                    recv = [G.empty_like_rank(unit, dtype) for _ in range(n)]
                    G.say(f"reduce_scatter {proto} {dtype} unit={unit}")
                    rs.reduce_scatter(comm, send, recv, op="sum")
                    want = oracle.ring_reduce_scatter(src, "sum", dtype, nchannels=1, chunk_bytes=unit * e)
                else:
                    src = _inputs(n, unit, dtype, 1500 + unit)
                    send = [G.to_device(x, dtype) for x in src]
                    recv = [G.empty_like_rank(n * unit, dtype) for _ in range(n)]
                    G.say(f"all_gather {proto} {dtype} unit={unit}")
                    rs.all_gather(comm, send, recv)
                    want = oracle.ring_all_gather(src, dtype, nchannels=1, chunk_bytes=unit * e)
                G.sync()
                G.check_comm_ok(comm)
                _assert_same([G.to_host(t, dtype) for t in recv], want, dtype, f"{coll} {proto} unit={unit}")
            finally:
                rs.comm_destroy(comm)


def _run_coll(coll, xs, dtype, nch, proto, chunk_bytes, **cfg):
    n = len(xs)
    comm = rs.comm_init(n, nch, proto, chunk_bytes=chunk_bytes, **cfg)
    try:
        send = [G.to_device(x, dtype) for x in xs]
        m = xs[0].shape[0]
        out = {"allreduce": m, "reduce_scatter": m // n, "all_gather": m * n}[coll]
        recv = [G.empty_like_rank(out, dtype) for _ in range(n)]
        G.say(f"{coll} N={n} in={m} dtype={dtype} C={nch} proto={proto} chunk={chunk_bytes} cfg={cfg}")
        if coll == "allreduce":
            rs.allreduce(comm, send, recv, op="sum")
        elif coll == "reduce_scatter":
            rs.reduce_scatter(comm, send, recv, op="sum")
        else:
            rs.all_gather(comm, send, recv)
        G.sync()
        G.check_comm_ok(comm)
        return [G.to_host(t, dtype) for t in recv], rs.comm_query(comm)
    finally:
        rs.comm_destroy(comm)


@pytest.mark.parametrize("proto", ["flag", "wide"])
@pytest.mark.parametrize("dtype", ["float32", "bfloat16", "int64"])
def test_line_workgroups_per_channel(proto, dtype):
    """A line launch may split every unit over 1, 2, 4 or 8 workgroups per
    (rank, channel), each with its own FIFO slots and counters. The split
    changes which workgroup moves an element, never the chunk it belongs to,
    so every count gives the oracle's bits: two full loops and a ragged third
    per channel, units of several step groups, for all three collectives."""
    n, nch, chunk = 5, 2, 262_144
    e = {"float32": 4, "bfloat16": 2, "int64": 8}[dtype]
    per_channel = 2 * n * chunk + 300 * 1024 + 48
    count = (nch * per_channel) // e - 3
    xs = _inputs(n, count, dtype, 1600 + e)
    want = oracle.ring_allreduce(xs, "sum", dtype, nchannels=nch, chunk_bytes=chunk)
    for lw in (1, 2, 4, 8):
        got, info = _run_coll("allreduce", xs, dtype, nch, proto, chunk, line_workgroups_per_channel=lw, algo="ring")
        assert info["last_workgroups_per_channel"] == lw
        _assert_same(got, want, dtype, f"allreduce {proto} line wpc {lw}")
    rc = (3 * chunk + 20_000) // e + 1  # three loops per block, the last ragged
    src = _inputs(n, n * rc, dtype, 1700 + e)
    want_rs = oracle.ring_reduce_scatter(src, "sum", dtype, nchannels=nch, chunk_bytes=chunk)
    sc = (chunk + 5000) // e + 3
    src_ag = _inputs(n, sc, dtype, 1800 + e)
    want_ag = oracle.ring_all_gather(src_ag, dtype, nchannels=nch, chunk_bytes=chunk)
    for lw in (2, 8):
        got, _ = _run_coll("reduce_scatter", src, dtype, nch, proto, chunk, line_workgroups_per_channel=lw)
        _assert_same(got, want_rs, dtype, f"reduce_scatter {proto} line wpc {lw}")
        got, _ = _run_coll("all_gather", src_ag, dtype, nch, proto, chunk, line_workgroups_per_channel=lw)
        _assert_same(got, want_ag, dtype, f"all_gather {proto} line wpc {lw}")


@pytest.mark.parametrize("proto", ["flag", "wide"])
def test_line_workgroup_counts_switch_on_one_comm(proto):
    """Consecutive calls of one communicator take different workgroup counts
    per channel (each count has a FIFO array of its own, and a line's flag is
    a step of the one pipeline that owns that array part, so no line left by
    an earlier call can match). The cost model splits a stage of 1, 2, 4 and
    16 lines per (rank, channel) over 1, 2, 4 and 8 workgroups (fewer lines
    per step is faster, ties go to fewer workgroups). Two rounds through the
    sizes, then larger messages, fresh data every call, every result
    checked."""
    n, nch, dtype = 8, 4, "float32"
    payload = 12 if proto == "wide" else 8
    comm = rs.comm_init(n, nch, proto)
    try:
        cases = []
        sizes = [(lines * payload * n * nch) // 4 for lines in (1, 2, 4, 16)] * 2
        sizes += [(lines * payload * n * nch) // 4 - 5 for lines in (100, 300, 900, 3000)]
        for k, count in enumerate(sizes):
            xs = _inputs(n, count, dtype, 1900 + k)
            send = [G.to_device(x, dtype) for x in xs]
            recv = [G.empty_like_rank(count, dtype) for _ in range(n)]
            G.say(f"switch {proto} call {k} count={count}")
            rs.allreduce(comm, send, recv)
            G.sync()
            G.check_comm_ok(comm)
            cases.append((xs, recv, count, rs.comm_query(comm)["last_workgroups_per_channel"]))
        assert [c[3] for c in cases[:8]] == [1, 2, 4, 8] * 2
        for xs, recv, count, lw in cases:
            want = oracle.ring_allreduce(xs, "sum", dtype, nchannels=nch)
            _assert_same([G.to_host(t, dtype) for t in recv], want, dtype, f"switch count={count} wpc={lw}")
    finally:
        rs.comm_destroy(comm)


def test_bulk_workgroup_counts_switch_on_one_comm():
    """Bulk calls of one communicator take as many workgroups per channel as
    their stages need (about one per 4 KiB of a channel's stage, at least
    two, all of them for long stages): small, large and middle calls, a
    reduce-scatter and an all-gather, in turn on one communicator, so that a
    launch with more pipelines finds the counters that launches with fewer
    left untouched. Fresh data every call, every result checked."""
    n, nch, dtype = 8, 8, "float32"
    comm = rs.comm_init(n, nch, "bulk")
    try:
        top = rs.comm_query(comm)["workgroups_per_channel"]
        cases = []
        for k, (coll, count) in enumerate([("allreduce", 1024), ("allreduce", (4 << 20) // 4 - 5),
                                          ("allreduce", (1 << 20) // 4 + 3), ("allreduce", 16383),
                                          ("reduce_scatter", 2048), ("all_gather", 3001),
                                          ("allreduce", 1024), ("allreduce", (4 << 20) // 4 - 5)]):
            m = count * n if coll == "reduce_scatter" else count
            xs = _inputs(n, m, dtype, 2100 + k)
            send = [G.to_device(x, dtype) for x in xs]
            out = {"allreduce": m, "reduce_scatter": count, "all_gather": count * n}[coll]
            recv = [G.empty_like_rank(out, dtype) for _ in range(n)]
            G.say(f"bulk switch call {k}: {coll} count={count}")
            if coll == "allreduce":
                rs.allreduce(comm, send, recv)
            elif coll == "reduce_scatter":
                rs.reduce_scatter(comm, send, recv)
            else:
                rs.all_gather(comm, send, recv)
            G.sync()
            G.check_comm_ok(comm)
            cases.append((coll, xs, recv, count, rs.comm_query(comm)["last_workgroups_per_channel"]))
        ws = [c[4] for c in cases]
        assert ws[0] == ws[3] == ws[4] == ws[5] == ws[6] == min(2, top), ws
        assert ws[1] == ws[7] == top, ws
        assert min(2, top) <= ws[2] <= top, ws
        for coll, xs, recv, count, w in cases:
            if coll == "allreduce":
                want = oracle.ring_allreduce(xs, "sum", dtype, nchannels=nch)
            elif coll == "reduce_scatter":
                want = oracle.ring_reduce_scatter(xs, "sum", dtype, nchannels=nch)
            else:
                want = oracle.ring_all_gather(xs, dtype, nchannels=nch)
            _assert_same([G.to_host(t, dtype) for t in recv], want, dtype, f"bulk switch {coll} count={count} wpc={w}")
    finally:
        rs.comm_destroy(comm)


@pytest.mark.parametrize("n,nch,wpc,chunk,dtype", [(4, 1, 1, 524_288, "float32"), (8, 2, 2, 1 << 20, "int64"),
                                                   (3, 1, 1, 524_288, "bfloat16")])
def test_bulk_long_stages_in_groups(n, nch, wpc, chunk, dtype):
    """A stage longer than half the configured FIFO depth (one workgroup per
    channel moving a whole 512 KiB or 1 MiB chunk: 16 or 32 slot steps)
    makes the communicator deepen its FIFOs; all-reduce calls with such
    stages run in groups of 4 steps over the first 8 slots instead, and
    reduce-scatter, all-gather and short calls on the same communicator use
    the deepened FIFOs. Several loops and a ragged tail, every result
    against the oracle."""
    comm = rs.comm_init(n, nch, "bulk", chunk_bytes=chunk, workgroups_per_channel=wpc)
    try:
        info = rs.comm_query(comm)
        assert info["nslots"] > 8, info
        e = {"float32": 4, "bfloat16": 2, "int64": 8}[dtype]
        per_channel = 2 * n * chunk + chunk // 2 + 48
        big = (nch * per_channel) // e + 3
        cases = [("allreduce", big, 4), ("reduce_scatter", (2 * chunk + 4096) // e + 1, 0),
                 ("allreduce", 1000, 0), ("all_gather", (chunk + 4096) // e + 5, 0), ("allreduce", big - 7, 4)]
        for k, (coll, count, want_group) in enumerate(cases):
            m = count * n if coll == "reduce_scatter" else count
            xs = _inputs(n, m, dtype, 2300 + k)
            send = [G.to_device(x, dtype) for x in xs]
            out = {"allreduce": m, "reduce_scatter": count, "all_gather": count * n}[coll]
            recv = [G.empty_like_rank(out, dtype) for _ in range(n)]
            G.say(f"long stages N={n} C={nch} wpc={wpc} chunk={chunk} {dtype} call {k}: {coll} count={count}")
            if coll == "allreduce":
                rs.allreduce(comm, send, recv)
            elif coll == "reduce_scatter":
                rs.reduce_scatter(comm, send, recv)
            else:
                rs.all_gather(comm, send, recv)
            G.sync()
            G.check_comm_ok(comm)
            assert rs.comm_query(comm)["last_group_steps"] == want_group, (coll, count)
            if coll == "allreduce":
                want = oracle.ring_allreduce(xs, "sum", dtype, nchannels=nch, chunk_bytes=chunk)
            elif coll == "reduce_scatter":
                want = oracle.ring_reduce_scatter(xs, "sum", dtype, nchannels=nch, chunk_bytes=chunk)
            else:
                want = oracle.ring_all_gather(xs, dtype, nchannels=nch, chunk_bytes=chunk)
            _assert_same([G.to_host(t, dtype) for t in recv], want, dtype, f"{coll} count={count}")
    finally:
        rs.comm_destroy(comm)
