"""Plain CPU oracle for ring collectives over N simulated ranks.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything under
``oracle/``. The library in ``ring_all_reduce_allreduce_amd`` never imports
it, and the two share no code: no kernels, headers, helpers, tables or
constants. The only thing both sides consume is the seeded input generator in
``synth``, which holds no collective arithmetic.

The oracle is deliberately slow and literal. It replays the ring schedule
stage by stage with an explicit FIFO object per receiving rank, moving whole
chunks as NumPy arrays, and rounds every hop to the buffer's data type.

Sources (page title, section):
  [NB 2.2]  "NCCL" book (aireadcode.com), ch. 2, s. 2.2 "channel": each channel
            owns count/nChannels elements and runs the ring independently.
  [NB 2.3]  same book, s. 2.3 "algorithm": RingARAlgorithm::getNextSendAddr
            (loop/chunk sizes, tail chunk rule, chunk id per stage) and the
            4-rank ring walkthrough; nStepsPerLoop = 2(nRanks-1)chunkSteps.
  [NB 2.4]  same book, s. 2.4 "protocol": FIFO head/tail counters.
  [NB enq]  same book, enqueue chapter, "taskAppend": count == 0 is a no-op,
            a single rank is a local copy.
  [L17]     "NCCL 专家课程 17: Bootstrap 与 Communicator 初始化状态机",
            section "Bootstrap Ring 与 AllGather": ring all-gather slice order
            and the rank-0 table for 4 ranks.
  [AISPE]   "AI Systems Performance Engineering (3)", collectives table:
            definitions of reduce, all-reduce, all-gather, reduce-scatter,
            broadcast and all-to-all; "In-Network SHARP Aggregation": a ring
            reduce-scatter delivers B(n-1)/n bytes to each rank.

Readings taken where the pages are silent or disagree:
  R1  chunk k is seeded by rank k+1 and finished by rank k. This follows the
      chunk-id formula of [NB 2.3]; the walkthrough's prose disagrees with it
      and with itself.
  R2  channel c covers [c*per, min((c+1)*per, count)) with
      per = alignUp(ceil(count/C), 16/e); trailing channels may be empty.
  R3  inside a channel, a loop spans N*chunk elements; a loop with fewer
      elements left uses chunk = alignUp(ceil(rem/N), 16/e) [NB 2.3].
  R4  reduce-scatter and all-gather split each rank block into channels and
      loops of ``chunk`` elements; loop l of every block moves together.
  R5  every hop rounds to the buffer type: fp32 in IEEE RNE with subnormals;
      bf16 as the correctly rounded (RNE) result of the exact operation.
  R6  max/min follow IEEE 754-2019 maximum/minimum on zeros (-0 < +0);
      inputs are finite. Integers wrap in two's complement; max/min signed.

Parity status: every public function here is pinned by ``tests/test_oracle_*``
against hand-derived golden values, closed forms, library special cases or a
brute-force exact-arithmetic fold. Nothing is "parity unpinned".
"""
from __future__ import annotations

from collections import deque
from dataclasses import dataclass, field

import numpy as np

DTYPES = ("int32", "int64", "float32", "bfloat16")
OPS = ("sum", "prod", "max", "min")
ELEM_SIZE = {"int32": 4, "int64": 8, "float32": 4, "bfloat16": 2}
STORAGE = {"int32": np.int32, "int64": np.int64, "float32": np.float32, "bfloat16": np.uint16}
DEFAULT_CHUNK_BYTES = 524_288


# --------------------------------------------------------------------------
# Element arithmetic (one hop)
# --------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64 (exact: bf16 is the top half of fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bfloat16, nearest-even, returning bit patterns.

    First to float32 (NumPy, IEEE RNE with subnormals), then the low 16 bits of
    the float32 pattern are dropped with round-half-even. Rounding twice is
    harmless here: for a sum or product of two bf16 values, float64 holds
    53 >= 2*24+2 bits and float32 holds 24 >= 2*8+2 bits, so each step keeps
    the correctly rounded result (Figueroa's double-rounding condition).
    Finite inputs only; values past the bf16 range round to infinity.
    """
    with np.errstate(over="ignore"):
        f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32)
    upper = u >> np.uint32(16)
    lower = u & np.uint32(0xFFFF)
    half = np.uint32(0x8000)
    up = (lower > half) | ((lower == half) & ((upper & np.uint32(1)) == np.uint32(1)))
    return (upper + up.astype(np.uint32)).astype(np.uint16)


def _select_max(a, b, a_bits, b_bits, is_max: bool, sign_and: bool):
    """Pick the larger (or smaller) operand; on equal values combine the bit
    patterns so that -0 and +0 resolve as IEEE 754-2019 maximum/minimum."""
    if is_max:
        pick_a = a > b
        pick_b = b > a
    else:
        pick_a = a < b
        pick_b = b < a
    tie = (a_bits & b_bits) if sign_and else (a_bits | b_bits)
    return np.where(pick_a, a_bits, np.where(pick_b, b_bits, tie))


def combine(acc: np.ndarray, local: np.ndarray, op: str, dtype: str) -> np.ndarray:
    """One ring hop: ``op(acc, local)`` rounded to ``dtype`` (readings R5, R6)."""
    if op not in OPS:
        raise ValueError(op)
    if dtype == "bfloat16":
        a = bf16_to_f64(acc)
        b = bf16_to_f64(local)
        if op == "sum":
            return f64_to_bf16(a + b)
        if op == "prod":
            return f64_to_bf16(a * b)
        ab = np.asarray(acc, dtype=np.uint16)
        bb = np.asarray(local, dtype=np.uint16)
        return _select_max(a, b, ab, bb, op == "max", op == "max").astype(np.uint16)
    if dtype == "float32":
        a = np.asarray(acc, dtype=np.float32)
        b = np.asarray(local, dtype=np.float32)
        if op == "sum":
            return np.add(a, b, dtype=np.float32)
        if op == "prod":
            return np.multiply(a, b, dtype=np.float32)
        ab = a.view(np.uint32)
        bb = b.view(np.uint32)
        return _select_max(a, b, ab, bb, op == "max", op == "max").astype(np.uint32).view(np.float32)
    if dtype in ("int32", "int64"):
        t = STORAGE[dtype]
        a = np.asarray(acc, dtype=t)
        b = np.asarray(local, dtype=t)
        with np.errstate(over="ignore"):
            if op == "sum":
                return np.add(a, b, dtype=t)
            if op == "prod":
                return np.multiply(a, b, dtype=t)
        return (np.maximum(a, b) if op == "max" else np.minimum(a, b)).astype(t)
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# Partition (readings R2-R4)
# --------------------------------------------------------------------------

def div_up(x: int, y: int) -> int:
    return -(-x // y)


def align_up(x: int, a: int) -> int:
    return div_up(x, a) * a


def elems_per_16b(dtype: str) -> int:
    return 16 // ELEM_SIZE[dtype]


def channel_ranges(count: int, nchannels: int, align: int) -> list[tuple[int, int]]:
    """[NB 2.2] each channel takes its own slice of count/nChannels elements.
    Reading R2: the slice length is rounded up to 16 bytes, so the last
    channels may be short or empty."""
    per = align_up(div_up(count, nchannels), align) if count > 0 else 0
    out = []
    for c in range(nchannels):
        lo = min(c * per, count)
        hi = min(lo + per, count)
        out.append((lo, hi))
    return out


def allreduce_loop_chunks(length: int, nranks: int, chunk: int, align: int) -> list[list[tuple[int, int]]]:
    """Chunk ranges of every loop of one channel, relative to the channel start.

    [NB 2.3] getNextSendAddr: a loop spans nRanks*chunkSize; when fewer
    elements remain than one loop, the chunk becomes
    alignUp(divUp(remaining, nRanks), 16/elemSize); chunk k starts at
    k*chunk inside the loop and is cut at the channel end (may be empty).
    """
    loop = nranks * chunk
    loops = []
    off = 0
    while off < length:
        rem = length - off
        cur = chunk if rem >= loop else align_up(div_up(rem, nranks), align)
        loops.append([(off + min(k * cur, rem), off + min((k + 1) * cur, rem)) for k in range(nranks)])
        off += loop
    return loops


def block_loop_ranges(length: int, chunk: int) -> list[tuple[int, int]]:
    """Reading R4: reduce-scatter / all-gather walk each rank block's channel
    slice in loops of ``chunk`` elements."""
    return [(off, min(off + chunk, length)) for off in range(0, length, chunk)]


def allreduce_chunk_of(count: int, nranks: int, nchannels: int, chunk_bytes: int, dtype: str) -> np.ndarray:
    """Chunk id (0..N-1) of every element under readings R2/R3."""
    a = elems_per_16b(dtype)
    chunk = chunk_bytes // ELEM_SIZE[dtype]
    ids = np.full(count, -1, dtype=np.int64)
    for clo, chi in channel_ranges(count, nchannels, a):
        for ks in allreduce_loop_chunks(chi - clo, nranks, chunk, a):
            for k, (lo, hi) in enumerate(ks):
                ids[clo + lo: clo + hi] = k
    return ids


# --------------------------------------------------------------------------
# FIFO between neighbouring ranks
# --------------------------------------------------------------------------

@dataclass
class Fifo:
    """Slots travelling from rank r-1 into rank r within one channel.

    ``tail`` counts slots produced, ``head`` slots consumed, as the step
    counters of [NB 2.4]; ``bytes`` counts payload bytes that passed through.
    """

    slots: deque = field(default_factory=deque)
    tail: int = 0
    head: int = 0
    bytes: int = 0

    def send(self, data: np.ndarray) -> None:
        self.slots.append(data)
        self.tail += 1
        self.bytes += data.nbytes

    def recv(self) -> np.ndarray:
        self.head += 1
        return self.slots.popleft()


@dataclass
class Stats:
    """Per-rank FIFO traffic of one collective call."""

    sends: list
    recv_bytes: list


def _new_stats(n: int) -> Stats:
    return Stats([0] * n, [0] * n)


def _check_inputs(inputs, dtype):
    if dtype not in DTYPES:
        raise ValueError(dtype)
    arrs = [np.ascontiguousarray(x, dtype=STORAGE[dtype]) for x in inputs]
    if len(arrs) < 1:
        raise ValueError("need at least one rank")
    n = arrs[0].shape[0]
    if any(a.ndim != 1 or a.shape[0] != n for a in arrs):
        raise ValueError("every rank needs a 1-D buffer of the same length")
    return arrs


# --------------------------------------------------------------------------
# Collectives
# --------------------------------------------------------------------------

def ring_allreduce(inputs, op: str = "sum", dtype: str = "float32", nchannels: int = 1,
                   chunk_bytes: int = DEFAULT_CHUNK_BYTES, stats: Stats | None = None,
                   trace: list | None = None) -> list[np.ndarray]:
    """Ring all-reduce = reduce-scatter stages then all-gather stages.

    [NB 2.3] at stage j (0 .. 2N-2) rank r handles chunk (r + N - 1 - j) mod N.
    Stage 0 sends the rank's own chunk; stages 1..N-1 add the incoming partial
    to the local chunk (stage N-1 completes chunk r on rank r); stages N-1..2N-2
    store the finished chunk; every stage but the last forwards to rank r+1.
    One rank is a plain copy [NB enq]. ``trace`` (optional) collects
    (channel, loop, stage, rank, chunk) for every stage of every rank.
    """
    xs = _check_inputs(inputs, dtype)
    nr = len(xs)
    count = xs[0].shape[0]
    if chunk_bytes <= 0 or chunk_bytes % 16:
        raise ValueError("chunk_bytes must be a positive multiple of 16")
    if nr == 1:
        return [xs[0].copy()]
    a = elems_per_16b(dtype)
    chunk = chunk_bytes // ELEM_SIZE[dtype]
    out = [np.zeros_like(x) for x in xs]
    for clo, chi in channel_ranges(count, nchannels, a):
        for li, ks in enumerate(allreduce_loop_chunks(chi - clo, nr, chunk, a)):
            fifos = [Fifo() for _ in range(nr)]
            for j in range(2 * nr - 1):
                outgoing = []
                for r in range(nr):
                    k = (r + nr - 1 - j) % nr
                    if trace is not None:
                        trace.append((clo, li, j, r, k))
                    seg = slice(clo + ks[k][0], clo + ks[k][1])
                    if j == 0:
                        data = xs[r][seg].copy()
                    else:
                        data = fifos[r].recv()
                        if j <= nr - 1:
                            data = combine(data, xs[r][seg], op, dtype)
                        if j >= nr - 1:
                            out[r][seg] = data
                    if j <= 2 * nr - 3:
                        outgoing.append(((r + 1) % nr, data))
                for dst, data in outgoing:
                    fifos[dst].send(data)
            if stats is not None:
                for r in range(nr):
                    stats.sends[(r - 1) % nr] += fifos[r].tail
                    stats.recv_bytes[r] += fifos[r].bytes
            assert all(f.head == f.tail for f in fifos)
    return out


def ring_reduce_scatter(inputs, op: str = "sum", dtype: str = "float32", nchannels: int = 1,
                        chunk_bytes: int = DEFAULT_CHUNK_BYTES, stats: Stats | None = None) -> list[np.ndarray]:
    """Ring reduce-scatter: rank r ends with the reduction of block r.

    [AISPE] the reduction result is split so that each rank keeps one chunk.
    Same stage rule as the all-reduce's first half: at stage j (0 .. N-1) rank
    r handles block (r + N - 1 - j) mod N, so block b is folded in the order
    b+1, b+2, ..., b and completes on rank b.
    """
    xs = _check_inputs(inputs, dtype)
    nr = len(xs)
    total = xs[0].shape[0]
    if total % nr:
        raise ValueError("each send buffer must hold N equal blocks")
    rc = total // nr
    if nr == 1:
        return [xs[0].copy()]
    a = elems_per_16b(dtype)
    chunk = chunk_bytes // ELEM_SIZE[dtype]
    out = [np.zeros(rc, dtype=STORAGE[dtype]) for _ in range(nr)]
    for clo, chi in channel_ranges(rc, nchannels, a):
        for lo, hi in block_loop_ranges(chi - clo, chunk):
            fifos = [Fifo() for _ in range(nr)]
            for j in range(nr):
                outgoing = []
                for r in range(nr):
                    b = (r + nr - 1 - j) % nr
                    seg = slice(b * rc + clo + lo, b * rc + clo + hi)
                    if j == 0:
                        data = xs[r][seg].copy()
                    else:
                        data = combine(fifos[r].recv(), xs[r][seg], op, dtype)
                    if j == nr - 1:
                        out[r][clo + lo: clo + hi] = data
                    else:
                        outgoing.append(((r + 1) % nr, data))
                for dst, data in outgoing:
                    fifos[dst].send(data)
            if stats is not None:
                for r in range(nr):
                    stats.sends[(r - 1) % nr] += fifos[r].tail
                    stats.recv_bytes[r] += fifos[r].bytes
    return out


def ring_all_gather(inputs, dtype: str = "float32", nchannels: int = 1,
                    chunk_bytes: int = DEFAULT_CHUNK_BYTES, stats: Stats | None = None,
                    trace: list | None = None) -> list[np.ndarray]:
    """Ring all-gather: block b of every output is rank b's input.

    [L17] in round i rank r sends slice (r - i) mod N and receives slice
    (r - i - 1) mod N from rank r-1; here round i is stage i, where stage 0
    also copies the rank's own block into its output. ``trace`` (optional)
    collects ("send"|"recv", stage, rank, block) events.
    """
    xs = _check_inputs(inputs, dtype)
    nr = len(xs)
    sc = xs[0].shape[0]
    out = [np.zeros(nr * sc, dtype=STORAGE[dtype]) for _ in range(nr)]
    if nr == 1:
        out[0][:] = xs[0]
        return out
    a = elems_per_16b(dtype)
    chunk = chunk_bytes // ELEM_SIZE[dtype]
    for clo, chi in channel_ranges(sc, nchannels, a):
        for lo, hi in block_loop_ranges(chi - clo, chunk):
            fifos = [Fifo() for _ in range(nr)]
            for j in range(nr):
                outgoing = []
                for r in range(nr):
                    b = (r - j) % nr
                    data = xs[r][clo + lo: clo + hi].copy() if j == 0 else fifos[r].recv()
                    if trace is not None and j > 0:
                        trace.append(("recv", j, r, b))
                    out[r][b * sc + clo + lo: b * sc + clo + hi] = data
                    if j < nr - 1:
                        if trace is not None:
                            trace.append(("send", j, r, b))
                        outgoing.append(((r + 1) % nr, data))
                for dst, data in outgoing:
                    fifos[dst].send(data)
            if stats is not None:
                for r in range(nr):
                    stats.sends[(r - 1) % nr] += fifos[r].tail
                    stats.recv_bytes[r] += fifos[r].bytes
    return out


def all_gather_slice_schedule(rank: int, nranks: int) -> list[tuple[int, int]]:
    """(send slice, receive slice) of ``rank`` in each of the N-1 rounds [L17]."""
    return [((rank - i) % nranks, (rank - i - 1) % nranks) for i in range(nranks - 1)]


def alltoall(inputs, dtype: str = "float32") -> list[np.ndarray]:
    """[AISPE] all-to-all: chunk j of rank i goes to rank j (a block transpose),
    landing in slot i of rank j's output."""
    xs = _check_inputs(inputs, dtype)
    nr = len(xs)
    total = xs[0].shape[0]
    if total % nr:
        raise ValueError("each send buffer must hold N equal chunks")
    c = total // nr
    out = [np.zeros_like(x) for x in xs]
    for i in range(nr):
        for j in range(nr):
            out[j][i * c:(i + 1) * c] = xs[i][j * c:(j + 1) * c]
    return out


def reduce(inputs, root: int, op: str = "sum", dtype: str = "float32") -> np.ndarray:
    """[AISPE] reduce to ``root``. The fold runs along the ring ending at the
    root: root+1, root+2, ..., root (hop-by-hop rounding, reading R5)."""
    xs = _check_inputs(inputs, dtype)
    nr = len(xs)
    acc = xs[(root + 1) % nr].copy()
    for t in range(2, nr + 1):
        acc = combine(acc, xs[(root + t) % nr], op, dtype)
    return acc


def broadcast(buf, nranks: int) -> list[np.ndarray]:
    """[AISPE] broadcast: the root's buffer is copied to every rank."""
    return [np.array(buf, copy=True) for _ in range(nranks)]


# --------------------------------------------------------------------------
# Traffic model used by the measurements
# --------------------------------------------------------------------------

def allreduce_fifo_steps_per_loop(nranks: int) -> int:
    """[NB 2.3] nStepsPerLoop = 2(nRanks-1)*chunkSteps; at chunk granularity
    (chunkSteps = 1) each rank sends 2(N-1) slots per loop."""
    return 2 * (nranks - 1)


def algorithmic_bytes(coll: str, nranks: int, nbytes: int, proto: str = "bulk") -> int:
    """HBM bytes the ring method moves for one call, summed over all ranks.

    ``nbytes`` is S: the all-reduce buffer per rank, the reduce-scatter input
    per rank, the all-gather output per rank, the all-to-all buffer per rank.
    Per rank: the all-reduce reads S and writes S of user data and writes and
    reads 2(N-1)/N * S of FIFO data ((6N-4)/N * S per rank); reduce-scatter
    and all-gather move (3N-1)/N * S; the flag-packed protocol doubles the
    FIFO bytes. All-to-all (direct copy) reads and writes S.
    """
    n, s = nranks, nbytes
    if n == 1:
        return 2 * s
    fifo_mult = 2 if proto == "flag" else 1
    if coll == "allreduce":
        return 2 * n * s + fifo_mult * 4 * (n - 1) * s
    if coll in ("reduce_scatter", "all_gather"):
        # user data: N*S on the full-size side plus S in total on the shard side
        return (n + 1) * s + fifo_mult * 2 * (n - 1) * s
    if coll == "alltoall":
        return 2 * n * s
    raise ValueError(coll)
