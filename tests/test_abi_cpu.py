"""Host-side checks of libringsim that need no GPU: the shared library loads,
exports every function include/ringsim.h declares, plans exactly the ranges
the oracle's independent partition gives, and follows the error conventions
for bad arguments and bad handles."""
import ctypes
import itertools
import os
import subprocess

import pytest

import oracle
import ring_all_reduce_allreduce_amd as rs


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(rs.LIB_PATH):
        from ring_all_reduce_allreduce_amd import build

        build.build()
    return rs.lib()


def test_exports_every_declared_function(L):
    declared = rs.header_exports()
    assert len(declared) >= 13
    out = subprocess.run(["nm", "-D", "--defined-only", rs.LIB_PATH], check=True, capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    missing = [f for f in declared if f not in exported]
    assert not missing, missing
    for f in declared:
        assert hasattr(L, f)


def _header_struct_fields(name):
    import re

    with open(rs.HEADER_PATH) as f:
        text = f.read()
    body = re.search(r"typedef struct \{((?:(?!typedef struct).)*?)\}\s*" + name + ";", text, re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    return [(m.group(1), m.group(2)) for m in re.finditer(r"^\s*([a-z_0-9]+)\s+([a-z_0-9]+);", body, re.M)]


def test_binding_mirrors_the_header():
    """The ctypes structures list the header's fields in order, with C types
    of the same size, and the binding's limits equal the header's macros."""
    import re

    sizes = {"int": ctypes.sizeof(ctypes.c_int), "size_t": ctypes.sizeof(ctypes.c_size_t),
             "uint64_t": 8, "double": 8}
    for cname, pycls in (("ringsim_config_t", rs.Config), ("ringsim_comm_info_t", rs.CommInfo)):
        fields = _header_struct_fields(cname)
        assert [f for _, f in fields] == [f for f, _ in pycls._fields_], cname
        for (ctype, f), (_, pytype) in zip(fields, pycls._fields_):
            assert sizes[ctype] == ctypes.sizeof(pytype), (cname, f)
    with open(rs.HEADER_PATH) as f:
        text = f.read()
    macros = dict(re.findall(r"#define RINGSIM_(MAX_[A-Z_]+) (\d+)", text))
    assert int(macros["MAX_RANKS"]) == rs.MAX_RANKS
    assert int(macros["MAX_CHANNELS"]) == rs.MAX_CHANNELS
    assert int(macros["MAX_WORKGROUPS_PER_CHANNEL"]) == rs.MAX_WORKGROUPS_PER_CHANNEL


def test_tree_model_workgroups_per_cu(L):
    """The tree's cost model, as measured at 16 ranks on 256 CUs: a second
    tree workgroup per compute unit (8 channels instead of 4) loses while
    each channel holds a few steps (64 KiB per rank) and wins once every
    channel pipelines many (512 KiB and up)."""
    assert rs.debug_tree_model(16, 4, 64 << 10) < rs.debug_tree_model(16, 8, 64 << 10)
    for size in (512 << 10, 1 << 20, 4 << 20):
        assert rs.debug_tree_model(16, 8, size) < rs.debug_tree_model(16, 4, size)


def test_error_strings(L):
    for code in (0, 1, 2, 3, 4, 5, 7, 8):
        assert rs.error_string(code)
    assert rs.error_string(5) == "invalid usage"


def _oracle_rows(coll, count, n, c, chunk_bytes, dtype):
    a = 16 // oracle.ELEM_SIZE[dtype]
    chunk = chunk_bytes // oracle.ELEM_SIZE[dtype]
    rows = []
    for ci, (lo, hi) in enumerate(oracle.channel_ranges(count, c, a)):
        if coll == "allreduce":
            for l, ks in enumerate(oracle.allreduce_loop_chunks(hi - lo, n, chunk, a)):
                for k, (b, e) in enumerate(ks):
                    rows.append((ci, l, k, lo + b, lo + e))
        else:
            for l, (b, e) in enumerate(oracle.block_loop_ranges(hi - lo, chunk)):
                rows.append((ci, l, -1, lo + b, lo + e))
    return rows


@pytest.mark.parametrize("coll", ["allreduce", "reduce_scatter", "all_gather"])
def test_plan_matches_oracle_partition(L, coll):
    cases = itertools.product((1, 2, 3, 8, 16), (0, 1, 7, 100, 4097, 1 << 16, 3_000_001), (1, 2, 5, 16),
                              (16, 4096, 524_288), ("float32", "bfloat16", "int64"))
    for n, count, c, cb, dt in cases:
        if count // max(1, cb // 16) > 20_000:  # keep the Python side quick
            continue
        assert rs.debug_plan(coll, count, n, c, cb, dt) == _oracle_rows(coll, count, n, c, cb, dt), \
            (coll, n, count, c, cb, dt)


def test_plan_workload_shapes(L):
    # 8 ranks, 64 MiB fp32, 8 channels, 512 KiB chunks: 2 full loops per channel
    rows = rs.debug_plan("allreduce", 16_777_216, 8, 8, 524_288, "float32")
    assert len(rows) == 8 * 2 * 8
    assert all(e - b == 131_072 for (_, _, _, b, e) in rows)
    # 8 ranks, 25 MiB bf16, 16 channels: one short loop, chunk 102,400
    rows = rs.debug_plan("allreduce", 13_107_200, 8, 16, 524_288, "bfloat16")
    assert len(rows) == 16 * 8
    assert all(e - b == 102_400 for (_, _, _, b, e) in rows)


def test_invalid_arguments_fail_before_touching_a_device(L):
    h = ctypes.c_void_p(12345)
    for nr, nc, p in ((0, 1, 0), (65, 1, 0), (4, 0, 0), (4, 65, 0), (4, 1, 4), (4, 1, -1)):
        assert L.ringsim_comm_init(ctypes.byref(h), nr, nc, p) == 4
        assert h.value == 12345  # untouched on error
    assert L.ringsim_comm_init(None, 4, 1, 0) == 4
    cfg = rs.Config()
    cfg.chunk_bytes = 24  # not a multiple of 16
    assert L.ringsim_comm_init_config(ctypes.byref(h), 4, 1, 0, ctypes.byref(cfg)) == 4
    cfg = rs.Config()
    cfg.slot_bytes = 1000
    assert L.ringsim_comm_init_config(ctypes.byref(h), 4, 1, 0, ctypes.byref(cfg)) == 4
    for lw in (-1, 3, 6, 16):  # line workgroups per channel: 0 (per call), 1, 2, 4 or 8
        cfg = rs.Config()
        cfg.line_workgroups_per_channel = lw
        assert L.ringsim_comm_init_config(ctypes.byref(h), 4, 1, 0, ctypes.byref(cfg)) == 4
        assert h.value == 12345
    n = ctypes.c_size_t()
    assert L.ringsim_debug_plan(0, 10, 4, 1, 24, 2, None, 0, ctypes.byref(n)) == 4
    assert L.ringsim_debug_plan(0, 10, 4, 1, 16, 9, None, 0, ctypes.byref(n)) == 4
    assert L.ringsim_debug_plan(7, 10, 4, 1, 16, 2, None, 0, ctypes.byref(n)) == 4


def test_bad_handles_are_invalid_usage(L):
    bogus = ctypes.c_void_p(0xdeadbeef)
    arr = (ctypes.c_void_p * 4)()
    assert L.ringsim_comm_destroy(None) == 5
    assert L.ringsim_comm_destroy(bogus) == 5
    assert L.ringsim_allreduce(bogus, arr, arr, 16, 2, 0, None) == 5
    assert L.ringsim_reduce_scatter(bogus, arr, arr, 16, 2, 0, None) == 5
    assert L.ringsim_all_gather(bogus, arr, arr, 16, 2, None) == 5
    assert L.ringsim_alltoall(bogus, arr, arr, 16, 2, None) == 5
    assert L.ringsim_abort(bogus) == 5
    err = ctypes.c_int()
    assert L.ringsim_get_async_error(bogus, ctypes.byref(err)) == 5
    info = rs.CommInfo()
    assert L.ringsim_comm_query(bogus, ctypes.byref(info)) == 5


def test_config_defaults(L):
    cfg = rs.config_default()
    assert cfg.chunk_bytes == 524_288
    assert cfg.nslots == 8
    assert cfg.slot_bytes == 32_768
    assert cfg.flag_threshold_bytes == 0  # 0: AUTO uses the cost model
    assert cfg.line_workgroups_per_channel == 0  # 0: chosen per call


def test_cost_model_shape(L):
    """The model behind AUTO: flag-packed wins for tiny messages and bulk for
    large ones, each protocol's time grows with size and with the hop count
    2(N-1), and the wide lines (12 payload bytes per 16 against 8) need fewer
    steps than the flag lines once the steps, not the hops, dominate."""
    for n, c in ((4, 4), (8, 8), (16, 16)):
        tiny = rs.debug_model("allreduce", n, c, 8)
        big = rs.debug_model("allreduce", n, c, 256 << 20)
        assert tiny["flag_us"] < tiny["bulk_us"]
        assert big["bulk_us"] < big["wide_us"] < big["flag_us"]
        prev = None
        for k in range(3, 29):
            m = rs.debug_model("allreduce", n, c, 1 << k)
            # the wide lines carry 12 payload bytes per 16 against the flag lines' 8:
            # once the steps dominate they win
            if k >= 24:
                assert m["wide_us"] < m["flag_us"]
            if prev:
                assert all(m[p] >= prev[p] for p in ("bulk_us", "flag_us", "wide_us"))
            prev = m
    # more ranks: more hops, higher latency floor
    assert rs.debug_model("allreduce", 16, 16, 8)["flag_us"] > rs.debug_model("allreduce", 8, 16, 8)["flag_us"]
    # reduce-scatter has half the hops of the all-reduce
    ar = rs.debug_model("allreduce", 8, 8, 8)
    rsm = rs.debug_model("reduce_scatter", 8, 8, 8)
    assert rsm["bulk_us"] < ar["bulk_us"]
    # the line protocols' lead over bulk grows with the ring: measured on MI355X
    # (C = N, best line protocol and workgroup count against bulk) the crossover is
    # ~1 MiB at 4x4, ~4 MiB at 8x8 and 4-8 MiB at 16x16
    def crossover(n, c):
        for k in range(3, 30):
            m = rs.debug_model("allreduce", n, c, 1 << k)
            if m["bulk_us"] <= min(m["flag_us"], m["wide_us"]):
                return 1 << k
        return 1 << 30
    x4, x8, x16 = crossover(4, 4), crossover(8, 8), crossover(16, 16)
    assert x4 < x8 <= x16
    assert (256 << 10) <= x4 <= (2 << 20) and (1 << 20) <= x8 <= (8 << 20) and (2 << 20) <= x16 <= (16 << 20)


def test_library_tree_matches_oracle_tree(L):
    """The kernels' tree links (built in C++ from the same page) equal the
    oracle's for every rank count the library accepts."""
    for n in range(1, 65):
        for r in range(n):
            assert rs.debug_tree(n, r) == oracle.dtree(n, r), (n, r)


def test_tree_debug_arguments(L):
    out = (ctypes.c_int * 6)()
    assert L.ringsim_debug_tree(0, 0, out) == 4
    assert L.ringsim_debug_tree(4, 4, out) == 4
    assert L.ringsim_debug_tree(65, 0, out) == 4
    assert L.ringsim_debug_tree(4, 0, None) == 4
    us = ctypes.c_double()
    assert L.ringsim_debug_tree_model(4, 0, 16, ctypes.byref(us)) == 4
    assert L.ringsim_debug_tree_model(4, 1, 16, None) == 4
    h = ctypes.c_void_p(12345)
    cfg = rs.Config()
    cfg.algo = 3
    assert L.ringsim_comm_init_config(ctypes.byref(h), 4, 1, 0, ctypes.byref(cfg)) == 4
    assert h.value == 12345


def test_tree_config_default(L):
    assert rs.config_default().algo == 0  # AUTO


def test_tree_model_shape(L):
    """2 log2(N) hops against the ring's 2(N-1): the tree is predicted faster
    for tiny messages at 8 and 16 ranks, slower for large ones, and its
    latency floor grows with the tree depth, not with N."""
    for n, c in ((8, 8), (16, 16)):
        ring = rs.debug_model("allreduce", n, c, 8)
        assert rs.debug_tree_model(n, 1, 8) < min(ring["flag_us"], ring["bulk_us"])
        big = rs.debug_model("allreduce", n, c, 256 << 20)
        assert rs.debug_tree_model(n, c, 256 << 20) > big["bulk_us"]
    assert rs.debug_tree_model(16, 1, 8) - rs.debug_tree_model(8, 1, 8) < \
        rs.debug_model("allreduce", 16, 16, 8)["flag_us"] - rs.debug_model("allreduce", 8, 16, 8)["flag_us"]


# Names by which the header cites the four pages the library follows.
PAGE_MARKERS = ('"NCCL" book', "NCCL 专家课程 17", "NCCL 专家课程 29", "AI Systems Performance Engineering (3)")


def _declared_with_comments():
    """(function name, the comment block right above its declaration) for
    every function include/ringsim.h declares."""
    import re

    with open(rs.HEADER_PATH) as f:
        text = f.read()
    out = []
    for m in re.finditer(r"^(?:ringsim_result_t|const char\*)\s+(ringsim_[a-z_]+)\s*\(", text, re.M):
        before = text[: m.start()].rstrip()
        assert before.endswith("*/"), f"{m.group(1)} has no comment block above it"
        out.append((m.group(1), before[before.rindex("/*"):]))
    return out


def test_every_export_cites_the_page_that_defines_it():
    """Each declared call names, in the comment right above it, the page (and
    its section) that defines what the call does; the allocation-free entry
    point instead names the callers it serves."""
    decls = _declared_with_comments()
    assert {n for n, _ in decls} == set(rs.header_exports())
    for name, comment in decls:
        if name.endswith("_noalloc"):
            assert "cannot allocate" in comment, name
            continue
        assert any(p in comment for p in PAGE_MARKERS), f"{name}: no page cited in {comment!r}"


def _split_part(n, parts, w, align):
    sub = -(-(-(-n // parts)) // align) * align
    lo = min(w * sub, n)
    return min(lo + sub, n) - lo


def _exact_line_steps(coll, nranks, nchannels, chunk_bytes, count, dtype, payload, wpc):
    """Steps of the busiest FIFO of a ring line launch, walked from the
    library's partition: each sending stage moves its workgroup's part of the
    stage's unit in ceil(part / slice) steps."""
    esize = rs.ELEM_SIZE[dtype]
    align = 16 // esize
    slice_elems = 1024 * payload // esize
    rows = rs.debug_plan(coll, count, nranks, nchannels, chunk_bytes, dtype)
    loops = {}
    for ch, lp, k, lo, hi in rows:
        loops.setdefault((ch, lp), {})[k] = hi - lo
    best = 0
    sends = range(2 * nranks - 2) if coll == "allreduce" else range(nranks - 1)
    for ch in range(nchannels):
        for w in range(wpc):
            for r in range(nranks):
                steps = 0
                for (c2, lp), chunks in loops.items():
                    if c2 != ch:
                        continue
                    for j in sends:
                        m = chunks[(r + nranks - 1 - j) % nranks] if coll == "allreduce" else chunks[-1]
                        part = _split_part(m, wpc, w, align)
                        steps += -(-part // slice_elems)
                best = max(best, steps)
    return best


@pytest.mark.parametrize("coll", ["allreduce", "reduce_scatter", "all_gather"])
def test_flag_step_bound_covers_every_fifo(L, coll):
    """The flag-span bookkeeping's per-call bound is never below the steps the
    busiest FIFO of the launch really moves (any workgroup split), nor far
    above it; the tree's bound covers its half of the buffer in 3 KiB (int64:
    2 KiB) steps."""
    cases = [(4, 1, 4096, 3, "float32"), (16, 16, 524288, 1 << 20, "int32"), (8, 8, 524288, 5_000_003, "bfloat16"),
             (3, 2, 65536, 100_003, "int64"), (16, 1, 524288, 1 << 22, "float32"), (2, 4, 16, 999, "int32")]
    for n, nch, chunk, count, dtype in cases:
        for proto, payload in (("flag", 8), ("wide", 8 if dtype == "int64" else 12)):
            bound = rs.debug_flag_steps(coll, "ring", n, nch, chunk, count, dtype, proto)
            exact = max(_exact_line_steps(coll, n, nch, chunk, count, dtype, payload, w) for w in (1, 2, 4, 8))
            assert exact <= bound, (coll, n, nch, chunk, count, dtype, proto, exact, bound)
            assert bound <= 4 * exact + 4 * n + 64, (coll, n, nch, chunk, count, dtype, proto, exact, bound)
    if coll == "allreduce":
        for count, dtype in ((1, "int32"), (1000, "float32"), (1 << 20, "bfloat16"), (777_777, "int64")):
            esize = rs.ELEM_SIZE[dtype]
            half = -(-(-(-count // 2)) // (16 // esize)) * (16 // esize)
            per_step = 256 * (8 if esize == 8 else 12)
            assert rs.debug_flag_steps("allreduce", "tree", 8, 8, 524288, count, dtype) >= -(-half * esize // per_step)


def test_roctx_ranges_load_on_request(L):
    """RINGSIM_ROCTX=1 makes the library load a roctx library at its first
    call (here a comm init refused before any device work) and say so at
    INFO level; without it the library looks for none."""
    code = ("import ctypes, ring_all_reduce_allreduce_amd as rs\n"
            "h = ctypes.c_void_p()\n"
            "assert rs.lib().ringsim_comm_init(ctypes.byref(h), 0, 1, 0) == 4\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for flag in ("1", "0"):
        env = dict(os.environ, RINGSIM_ROCTX=flag, RINGSIM_DEBUG="INFO", PYTHONPATH=root)
        out = subprocess.run(["python3", "-c", code], capture_output=True, text=True, env=env, cwd=root, timeout=300)
        assert out.returncode == 0, out.stderr[-2000:]
        assert ("roctx ranges on" in out.stderr) == (flag == "1"), (flag, out.stderr[-2000:])
        assert "no roctx library" not in out.stderr, out.stderr[-2000:]
