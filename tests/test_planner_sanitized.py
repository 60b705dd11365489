"""The library's planning headers (ring_plan.h, tree_plan.h, ring_model.h)
built into a host driver with AddressSanitizer and UndefinedBehaviorSanitizer
(g++, CPU only): over many shapes the partition equals the oracle's own, the
double-tree links equal the oracle's, the cost model stays finite and
positive, a bulk call's workgroup count keeps its rules, and the sanitizers
report nothing."""
import itertools
import os
import shutil
import subprocess

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ is not installed")
    exe = str(tmp_path_factory.mktemp("planner") / "planner_check")
    subprocess.run([gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", "-Wall", "-Werror", os.path.join(HERE, "planner_check.cpp"), "-o", exe],
                   check=True)
    return exe


def _run(exe, commands):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    out = subprocess.run([exe], input="\n".join(commands) + "\n", capture_output=True, text=True, env=env, timeout=300)
    assert out.returncode == 0, out.stderr[-3000:]
    assert "runtime error" not in out.stderr and "Sanitizer" not in out.stderr, out.stderr[-3000:]
    blocks, cur = [], []
    for line in out.stdout.splitlines():
        if line == "end":
            blocks.append(cur)
            cur = []
        else:
            cur.append(line)
    return blocks


def _oracle_rows(coll, count, n, c, chunk_bytes, esize):
    dtype = {2: "bfloat16", 4: "float32", 8: "int64"}[esize]
    a = 16 // esize
    chunk = chunk_bytes // esize
    rows = []
    for ci, (lo, hi) in enumerate(oracle.channel_ranges(count, c, a)):
        if coll == 0:
            for l, ks in enumerate(oracle.allreduce_loop_chunks(hi - lo, n, chunk, a)):
                for k, (b, e) in enumerate(ks):
                    rows.append(f"{ci} {l} {k} {lo + b} {lo + e}")
        else:
            for l, (b, e) in enumerate(oracle.block_loop_ranges(hi - lo, chunk)):
                rows.append(f"{ci} {l} -1 {lo + b} {lo + e}")
    _ = dtype
    return rows


def test_partition_under_sanitizers_equals_the_oracle(driver):
    cases = [c for c in itertools.product((0, 1), (0, 1, 7, 100, 4097, 65_536, 1_000_003), (1, 2, 3, 8, 16, 64),
                                          (1, 2, 5, 16, 64), (16, 4096, 524_288), (2, 4, 8))
             if c[1] // max(1, c[4] // 16) <= 20_000]
    blocks = _run(driver, [f"plan {c} {n} {r} {ch} {cb} {e}" for c, n, r, ch, cb, e in cases])
    assert len(blocks) == len(cases)
    for (coll, count, n, ch, cb, e), rows in zip(cases, blocks):
        assert "bad split" not in rows and "bad chunk id" not in rows, (coll, count, n, ch, cb, e)
        assert rows == _oracle_rows(coll, count, n, ch, cb, e), (coll, count, n, ch, cb, e)


def test_tree_shapes_under_sanitizers_equal_the_oracle(driver):
    blocks = _run(driver, [f"tree {n}" for n in range(1, 65)])
    for n, lines in zip(range(1, 65), blocks):
        assert lines[-1].startswith("depth ") and int(lines[-1].split()[1]) >= 0
        for line in lines[:-1]:
            t, r, p, k0, k1 = map(int, line.split())
            want = oracle.dtree(n, r)[t]
            assert (p, k0, k1) == tuple(want), (n, t, r)


def test_cost_model_under_sanitizers_is_finite(driver):
    shapes = list(itertools.product((1, 2, 4, 8, 16, 64), (1, 8, 64), (8, 4096, 1 << 20, 1 << 28)))
    blocks = _run(driver, [f"model {n} {c} {b}" for n, c, b in shapes])
    for shape, lines in zip(shapes, blocks):
        for line in lines:
            v = float(line.split()[-1])
            assert v > 0 and v < 1e9, (shape, line)


def _longest_unit_bytes(coll, count, n, ch, chunk_bytes, esize):
    """Longest chunk of channel 0's first loop, from the oracle's partition."""
    a = 16 // esize
    lo, hi = oracle.channel_ranges(count, ch, a)[0]
    if hi <= lo:
        return 0
    if coll == 0:
        ks = oracle.allreduce_loop_chunks(hi - lo, n, chunk_bytes // esize, a)[0]
        return max(e - b for b, e in ks) * esize
    b, e = oracle.block_loop_ranges(hi - lo, chunk_bytes // esize)[0]
    return (e - b) * esize


def test_bulk_workgroups_per_call_keep_their_rules(driver):
    """A bulk call takes the communicator's workgroup count, or fewer when its
    stages are short: at least two, about one per 4 KiB of a channel's stage,
    channels x workgroups a multiple of 8, and one workgroup's stage within
    half of its FIFO; long stages take the full count. The stage length it
    starts from is the longest chunk of the oracle's partition, rounded up to
    whole 16-byte vectors (a bound: the library sizes channel 0 before
    clamping it to a tiny count)."""
    cases = []
    for coll, count, n, ch, esize in itertools.product((0, 1), (1, 1000, 4096, 65_536, 262_144, 1 << 20, 1 << 22),
                                                       (2, 4, 8, 16, 64), (1, 3, 8, 16), (2, 4, 8)):
        if n * ch > 512:
            continue
        wpc_max = max(1, min(16, 2 * 256 // (n * ch)))
        for slot in (4096, 32768):
            # the communicator's FIFO depth: 8 slots, more when one
            # workgroup's stage at the full count needs them
            stage = -(-(-(-524_288 // wpc_max)) // 16) * 16
            nslots = max(8, 2 * -(-stage // slot))
            cases.append((coll, count, n, ch, 524_288, esize, wpc_max, slot, nslots))
    blocks = _run(driver, [f"bulkw {' '.join(map(str, c))}" for c in cases])
    assert len(blocks) == len(cases)
    for c, lines in zip(cases, blocks):
        coll, count, n, ch, cb, esize, wpc_max, slot, nslots = c
        w, unit, unit1 = map(int, lines[0].split())
        longest = _longest_unit_bytes(coll, count, n, ch, cb, esize)
        assert longest <= unit1 < longest + 16, c
        assert 1 <= w <= wpc_max, c
        need = -(-unit1 // 4096)
        if w < wpc_max:
            assert w >= 2 and (ch * w) % 8 == 0, c
            assert w >= need, c
            assert 2 * -(-unit // slot) <= nslots, c
        if need >= wpc_max:
            assert w == wpc_max, c
    anchors = {(0, 1024, 4, 1, 4): 8, (0, 1024, 8, 8, 4): 2, (0, 1 << 20, 8, 8, 4): 8, (0, 1024, 16, 16, 4): 2}
    for (coll, count, n, ch, esize), want in anchors.items():
        wpc_max = max(1, min(16, 2 * 256 // (n * ch)))
        lines = _run(driver, [f"bulkw {coll} {count} {n} {ch} 524288 {esize} {wpc_max} 32768 8"])[0]
        assert int(lines[0].split()[0]) == want, (coll, count, n, ch, esize)
