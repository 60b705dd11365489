"""Pins of the CPU oracle against values the pages and the mathematics fix.

None of these checks re-types the oracle's own formulas: each compares it with
a golden file derived by hand from a cited passage, a library special case
(NumPy integer sums, torch's float32->bfloat16 cast), exact rational
arithmetic on tiny inputs, a closed form, or an identity between collectives.
"""
import itertools
import os

import numpy as np
import pytest

import oracle
from oracle import ring as R
from tests import _exact as X
from tests.conftest import GOLDEN


def _golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


def _rand_inputs(rng, n, count, dtype, kind="normal"):
    if dtype == "float32":
        if kind == "int":
            return [rng.integers(-8, 9, count).astype(np.float32) for _ in range(n)]
        return [rng.standard_normal(count, dtype=np.float32) for _ in range(n)]
    if dtype == "bfloat16":
        f = [rng.standard_normal(count, dtype=np.float32) for _ in range(n)]
        return [R.f64_to_bf16(v.astype(np.float64)) for v in f]
    info = np.iinfo(R.STORAGE[dtype])
    if kind == "wide":
        return [rng.integers(info.min, info.max, count, dtype=R.STORAGE[dtype], endpoint=True) for _ in range(n)]
    return [rng.integers(-1000, 1001, count).astype(R.STORAGE[dtype]) for _ in range(n)]


# ---------------------------------------------------------------- golden files

def test_allgather_slice_table_rank0():
    rows = _golden_rows("allgather_rank0_4ranks.txt")
    want = [(int(s), int(r)) for _, s, r in rows]
    assert oracle.all_gather_slice_schedule(0, 4) == want
    # the replay itself moves blocks in that order
    trace = []
    xs = [np.full(4, 10 * b, dtype=np.int32) for b in range(4)]
    out = oracle.ring_all_gather(xs, dtype="int32", trace=trace)
    sends = [b for (kind, j, r, b) in sorted(trace) if kind == "send" and r == 0]
    recvs = [b for (kind, j, r, b) in sorted(trace) if kind == "recv" and r == 0]
    assert list(zip(sends, recvs)) == want
    for r in range(4):
        assert np.array_equal(out[r], np.concatenate(xs))


def test_fold_order_adversarial_fp32():
    rows = _golden_rows("fold_order_fp32.txt")
    by_seed = {int(s): float(v) for s, v in rows}
    v = [np.float32(2.0 ** 24), np.float32(1.0), np.float32(-(2.0 ** 24)), np.float32(1.0)]
    n, count = 4, 16
    xs = [np.zeros(count, dtype=np.float32) for _ in range(n)]
    for k in range(4):
        for t in range(4):
            xs[(k + t) % n][4 * k: 4 * k + 4] = v[t]
    out = oracle.ring_allreduce(xs, "sum", "float32", nchannels=1, chunk_bytes=1 << 20)
    for r in range(n):
        assert np.all(out[r] == np.float32(by_seed[1])), out[r]
    # the exact-arithmetic fold agrees for every start offset in the file
    vals = [X.to_scalar_list(x, "float32") for x in xs]
    for s, want in by_seed.items():
        acc = vals[s % n][0]
        for t in range(1, n):
            acc = X.hop(acc, vals[(s + t) % n][0], "sum", "float32")
        assert np.uint32(acc).view(np.float32) == np.float32(want)


def test_walkthrough_4ranks():
    rows = _golden_rows("allreduce_walkthrough_4ranks.txt")
    meta = {r[0]: int(r[1]) for r in rows if not r[0].isdigit()}
    want = np.array([float(r[1]) for r in rows if r[0].isdigit()], dtype=np.float32)
    n, count = meta["nranks"], meta["count"]
    xs = [np.array([100 * r + i for i in range(count)], dtype=np.float32) for r in range(n)]
    trace = []
    stats = R.Stats([0] * n, [0] * n)
    out = oracle.ring_allreduce(xs, "sum", "float32", nchannels=1, chunk_bytes=1 << 20, stats=stats, trace=trace)
    for r in range(n):
        assert np.array_equal(out[r], want)
    assert len({j for (_, _, j, _, _) in trace}) == meta["stages"]
    assert stats.sends == [meta["sends_per_rank"]] * n
    assert oracle.allreduce_fifo_steps_per_loop(n) == meta["sends_per_rank"]
    # after the reduce-scatter half (stage N-1) rank r holds chunk r
    finals = {r: k for (_, _, j, r, k) in trace if j == n - 1}
    assert finals == {r: r for r in range(n)}


def test_bf16_round_cases():
    for op, a, b, want in _golden_rows("bf16_round_cases.txt"):
        a16 = np.array([int(a, 16)], dtype=np.uint16)
        b16 = np.array([int(b, 16)], dtype=np.uint16)
        got = int(oracle.combine(a16, b16, op, "bfloat16")[0])
        assert got == int(want, 16), (op, a, b, hex(got), want)
        # operand order does not matter for any of the ops
        got2 = int(oracle.combine(b16, a16, op, "bfloat16")[0])
        assert got2 == int(want, 16)
        # and the exact rational reference agrees with the hand values
        assert X.hop(int(a, 16), int(b, 16), op, "bfloat16") == int(want, 16)


def test_fp32_signed_zero_max_min():
    pz = np.array([0.0], dtype=np.float32)
    nz = np.array([-0.0], dtype=np.float32)
    assert not np.signbit(oracle.combine(pz, nz, "max", "float32")[0])
    assert not np.signbit(oracle.combine(nz, pz, "max", "float32")[0])
    assert np.signbit(oracle.combine(pz, nz, "min", "float32")[0])
    assert np.signbit(oracle.combine(nz, nz, "max", "float32")[0])


# --------------------------------------------------- library / exact arithmetic

def test_bf16_rounding_matches_torch_cast():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(7)
    with np.errstate(over="ignore"):  # the largest draws become infinities, kept on purpose
        f = np.concatenate([
            rng.standard_normal(200_000).astype(np.float32),
            (rng.standard_normal(50_000) * 1e-38).astype(np.float32),   # subnormal range
            (rng.standard_normal(50_000) * 1e38).astype(np.float32),
            # exact ties: a bf16 value plus half of its ulp
            ((np.arange(1, 20_001, dtype=np.float32) * 2 + 1) * np.float32(2.0 ** -8)).astype(np.float32),
        ])
    ours = R.f64_to_bf16(f.astype(np.float64))
    theirs = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)


@pytest.mark.parametrize("op", ["sum", "prod", "max", "min"])
@pytest.mark.parametrize("dtype", ["float32", "bfloat16"])
def test_hop_matches_exact_rounding(op, dtype):
    rng = np.random.default_rng(11)
    n = 3000
    a = rng.standard_normal(n).astype(np.float32) * np.float32(4.0) ** rng.integers(-20, 20, n).astype(np.float32)
    b = rng.standard_normal(n).astype(np.float32) * np.float32(4.0) ** rng.integers(-20, 20, n).astype(np.float32)
    a[:50] = -b[:50]          # exact cancellations
    a[50:60] = 0.0
    b[55:65] = -0.0
    if dtype == "bfloat16":
        a = R.f64_to_bf16(a.astype(np.float64))
        b = R.f64_to_bf16(b.astype(np.float64))
    got = X.to_scalar_list(oracle.combine(a, b, op, dtype), dtype)
    la = X.to_scalar_list(a, dtype)
    lb = X.to_scalar_list(b, dtype)
    want = [X.hop(x, y, op, dtype) for x, y in zip(la, lb)]
    assert got == want


@pytest.mark.parametrize("dtype", ["int32", "int64"])
@pytest.mark.parametrize("op", ["sum", "max", "min", "prod"])
def test_int_allreduce_is_elementwise_reduction(dtype, op):
    rng = np.random.default_rng(3)
    n, count = 5, 1000
    xs = _rand_inputs(rng, n, count, dtype, "wide")
    out = oracle.ring_allreduce(xs, op, dtype, nchannels=3, chunk_bytes=64)
    stack = np.stack(xs).astype(object)  # Python ints: no overflow
    if op == "sum":
        want = stack.sum(axis=0)
    elif op == "prod":
        want = np.prod(stack, axis=0)
    elif op == "max":
        want = stack.max(axis=0)
    else:
        want = stack.min(axis=0)
    bits = 32 if dtype == "int32" else 64
    want = np.array([((int(v) + (1 << (bits - 1))) % (1 << bits)) - (1 << (bits - 1)) for v in want],
                    dtype=R.STORAGE[dtype])
    for r in range(n):
        assert np.array_equal(out[r], want)


def _bruteforce_cases():
    cases = []
    for n in (1, 2, 3, 4, 5):
        for count in (0, 1, 3, 7, 8, 17, 40):
            for c in (1, 2, 3):
                for chunk_bytes in (16, 32, 64):
                    cases.append((n, count, c, chunk_bytes))
    return cases


@pytest.mark.parametrize("dtype,op", [("float32", "sum"), ("bfloat16", "sum"), ("int32", "sum"),
                                      ("int64", "max"), ("float32", "max"), ("bfloat16", "prod")])
def test_allreduce_bruteforce_tiny(dtype, op):
    rng = np.random.default_rng(5)
    align = 16 // R.ELEM_SIZE[dtype]
    for n, count, c, chunk_bytes in _bruteforce_cases():
        xs = _rand_inputs(rng, n, count, dtype)
        out = oracle.ring_allreduce(xs, op, dtype, nchannels=c, chunk_bytes=chunk_bytes)
        vals = [X.to_scalar_list(x, dtype) for x in xs]
        want = X.brute_allreduce(vals, op, dtype, c, chunk_bytes // R.ELEM_SIZE[dtype], align)
        for r in range(n):
            assert X.to_scalar_list(out[r], dtype) == want, (n, count, c, chunk_bytes, r)


def test_chunk_ids_match_closed_form():
    for n, count, c, chunk_bytes in itertools.product((2, 3, 8, 16), (1, 5, 33, 100, 1000), (1, 3, 8), (16, 48, 512)):
        for dtype in ("float32", "bfloat16", "int64"):
            e = R.ELEM_SIZE[dtype]
            ids = oracle.allreduce_chunk_of(count, n, c, chunk_bytes, dtype)
            want = [X.ar_chunk_id(i, count, n, c, chunk_bytes // e, 16 // e) for i in range(count)]
            assert ids.tolist() == want


@pytest.mark.parametrize("dtype,op", [("float32", "sum"), ("bfloat16", "sum"), ("int32", "max")])
def test_reduce_scatter_bruteforce_tiny(dtype, op):
    rng = np.random.default_rng(9)
    for n in (1, 2, 3, 5):
        for rc in (0, 1, 5, 8, 13):
            for c in (1, 2):
                xs = _rand_inputs(rng, n, n * rc, dtype)
                out = oracle.ring_reduce_scatter(xs, op, dtype, nchannels=c, chunk_bytes=16)
                vals = [X.to_scalar_list(x, dtype) for x in xs]
                for r in range(n):
                    want = X.brute_reduce_block(vals, r, rc, op, dtype) if n > 1 else vals[0]
                    assert X.to_scalar_list(out[r], dtype) == want


def test_all_gather_and_alltoall_definitions():
    rng = np.random.default_rng(1)
    for n in (1, 2, 3, 8):
        for cnt in (0, 1, 9, 64):
            xs = [rng.integers(-99, 99, cnt).astype(np.int32) for _ in range(n)]
            ag = oracle.ring_all_gather(xs, dtype="int32", nchannels=2, chunk_bytes=16)
            for r in range(n):
                for b in range(n):
                    assert np.array_equal(ag[r][b * cnt:(b + 1) * cnt], xs[b])
            ys = [rng.integers(-99, 99, n * cnt).astype(np.int32) for _ in range(n)]
            a2a = oracle.alltoall(ys, dtype="int32")
            for i in range(n):
                for j in range(n):
                    assert np.array_equal(a2a[j][i * cnt:(i + 1) * cnt], ys[i][j * cnt:(j + 1) * cnt])
            # the transpose applied twice is the identity
            back = oracle.alltoall(a2a, dtype="int32")
            for r in range(n):
                assert np.array_equal(back[r], ys[r])


# ---------------------------------------------------------------- identities

@pytest.mark.parametrize("dtype", ["int32", "int64"])
def test_allreduce_equals_rs_then_ag_and_reduce_then_bcast_integers(dtype):
    rng = np.random.default_rng(21)
    for n in (2, 3, 4, 7):
        for rc in (1, 4, 31):
            xs = _rand_inputs(rng, n, n * rc, dtype, "wide")
            ar = oracle.ring_allreduce(xs, "sum", dtype, nchannels=2, chunk_bytes=32)
            rs = oracle.ring_reduce_scatter(xs, "sum", dtype, nchannels=3, chunk_bytes=16)
            ag = oracle.ring_all_gather(rs, dtype=dtype, nchannels=1, chunk_bytes=48)
            root = n // 2
            red = oracle.reduce(xs, root, "sum", dtype)
            bc = oracle.broadcast(red, n)
            for r in range(n):
                assert np.array_equal(ar[r], ag[r])
                assert np.array_equal(ar[r], bc[r])


def test_allreduce_equals_rs_then_ag_bitwise_fp_when_partitions_coincide():
    # one channel, one loop and blocks that are whole 16-byte multiples: the
    # all-reduce chunk k is exactly block k, so both fold in the same order
    rng = np.random.default_rng(4)
    for dtype in ("float32", "bfloat16"):
        for n in (2, 3, 8):
            a = 16 // R.ELEM_SIZE[dtype]
            count = n * a * 5
            xs = _rand_inputs(rng, n, count, dtype)
            ar = oracle.ring_allreduce(xs, "sum", dtype, nchannels=1, chunk_bytes=1 << 20)
            rs = oracle.ring_reduce_scatter(xs, "sum", dtype, nchannels=1, chunk_bytes=1 << 20)
            ag = oracle.ring_all_gather(rs, dtype=dtype, nchannels=1, chunk_bytes=1 << 20)
            for r in range(n):
                assert np.array_equal(ar[r], ag[r])
            # reduce to root k folds like chunk k of the ring
            for k in range(n):
                red = oracle.reduce(xs, k, "sum", dtype)
                seg = slice(k * count // n, (k + 1) * count // n)
                assert np.array_equal(ar[0][seg], red[seg])


# ------------------------------------------------------------ traffic model

def test_fifo_traffic_invariants():
    n = 8
    for dtype in ("float32", "bfloat16"):
        e = R.ELEM_SIZE[dtype]
        count = n * 16 * 4
        s = count * e
        xs = [np.zeros(count, dtype=R.STORAGE[dtype]) for _ in range(n)]
        st = R.Stats([0] * n, [0] * n)
        oracle.ring_allreduce(xs, "sum", dtype, nchannels=1, chunk_bytes=1 << 20, stats=st)
        # each rank receives 2(N-1)/N of the buffer over the 2(N-1) stages
        assert st.recv_bytes == [2 * (n - 1) * s // n] * n
        assert st.sends == [2 * (n - 1)] * n
        st = R.Stats([0] * n, [0] * n)
        oracle.ring_reduce_scatter(xs, "sum", dtype, nchannels=1, chunk_bytes=1 << 20, stats=st)
        # ring reduce-scatter: B(n-1)/n bytes reach each rank over n-1 hops
        assert st.recv_bytes == [(n - 1) * s // n] * n
        assert st.sends == [n - 1] * n
        st = R.Stats([0] * n, [0] * n)
        oracle.ring_all_gather([x[: count // n] for x in xs], dtype=dtype, chunk_bytes=1 << 20, stats=st)
        assert st.recv_bytes == [(n - 1) * s // n] * n


def test_algorithmic_bytes_model():
    s = 64 << 20
    assert oracle.algorithmic_bytes("allreduce", 8, s) == 44 * s
    assert oracle.algorithmic_bytes("allreduce", 16, s, "flag") == 152 * s
    assert oracle.algorithmic_bytes("reduce_scatter", 8, s) == 23 * s
    assert oracle.algorithmic_bytes("all_gather", 8, s) == 23 * s
    assert oracle.algorithmic_bytes("alltoall", 8, s) == 16 * s


# ------------------------------------------------------------ special cases

def test_special_cases():
    xs = [np.zeros(0, dtype=np.float32) for _ in range(3)]
    out = oracle.ring_allreduce(xs, "sum", "float32", nchannels=4)
    assert all(o.shape == (0,) for o in out)
    x1 = [np.arange(10, dtype=np.float32)]
    assert np.array_equal(oracle.ring_allreduce(x1, "sum", "float32")[0], x1[0])
    # 16 ranks, 2 elements: most chunks and channels are empty
    xs = [np.array([r, -r], dtype=np.int32) for r in range(16)]
    out = oracle.ring_allreduce(xs, "sum", "int32", nchannels=16)
    assert all(np.array_equal(o, [120, -120]) for o in out)


def test_workload1_closed_form():
    from synth import workload_inputs
    xs = workload_inputs(1)
    assert all(np.all(np.abs(x) <= 8) and np.all(x == np.round(x)) for x in xs)
    out = oracle.ring_allreduce(xs, "sum", "float32", nchannels=1)
    want = np.sum(np.stack(xs).astype(np.int64), axis=0).astype(np.float32)
    for o in out:
        assert np.array_equal(o, want)


# ------------------------------------------------------------ error bounds

def test_fp32_within_recursive_summation_bound():
    rng = np.random.default_rng(8)
    n, count = 16, 50_000
    xs = [rng.standard_normal(count, dtype=np.float32) for _ in range(n)]
    out = oracle.ring_allreduce(xs, "sum", "float32", nchannels=3, chunk_bytes=4096)
    st = np.stack(xs).astype(np.float64)
    exact = st.sum(axis=0)
    absum = np.abs(st).sum(axis=0)
    err = np.abs(out[0].astype(np.float64) - exact)
    u = 2.0 ** -24
    gamma = (n - 1) * u / (1 - (n - 1) * u)
    assert np.all(err <= gamma * absum)
    assert np.all(err <= 1e-6 * absum)


def test_bf16_within_tolerance():
    rng = np.random.default_rng(12)
    n, count = 8, 50_000
    xs = [R.f64_to_bf16(rng.standard_normal(count) * 1e-3) for _ in range(n)]
    out = oracle.ring_allreduce(xs, "sum", "bfloat16", nchannels=2, chunk_bytes=2048)
    st = np.stack([R.bf16_to_f64(x) for x in xs])
    exact = st.sum(axis=0)
    got = R.bf16_to_f64(out[0])
    assert np.linalg.norm(got - exact) / np.linalg.norm(exact) <= 8e-3
    u = 2.0 ** -8
    gamma = (n - 1) * u / (1 - (n - 1) * u)
    assert np.all(np.abs(got - exact) <= gamma * np.abs(st).sum(axis=0) + 1e-300)
