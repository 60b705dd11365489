"""Pins of the double-binary-tree oracle (``oracle/tree.py``).

The tree shapes are checked against tables derived by hand from the bit rules
of the "NCCL" book's ch. 4 (and its worked example), plus invariants every
double binary tree must satisfy; the fold order against hand-computed
float32 folds; the values against NumPy's integer reductions, exact-rational
brute force and the recursive-summation bound.
"""
import math
import os

import numpy as np
import pytest

from oracle import ring as R
from oracle import tree as T
from tests import _exact as X
from tests.conftest import GOLDEN


def _rows(name):
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                out.append(line.split())
    return out


def _tables():
    tab = {}
    for n, r, t, p, c0, c1 in _rows("dtree_tables.txt"):
        tab[(int(n), int(r), int(t))] = (int(p), int(c0), int(c1))
    return tab


def test_dtree_golden_tables():
    tab = _tables()
    assert len(tab) == 2 * (4 + 5 + 6 + 8)
    for (n, r, t), want in tab.items():
        assert T.dtree(n, r)[t] == want, (n, r, t)


def test_page_worked_example_rank1_of_8():
    # "NCCL" book, ch. 4: rank 1 of 8 has parent 2 and is a leaf.
    assert T.btree(8, 1) == (2, -1, -1)


@pytest.mark.parametrize("n", range(1, 65))
def test_double_tree_invariants(n):
    depth_bound = max(0, math.ceil(math.log2(n))) if n > 1 else 0
    interior = []
    for t in (0, 1):
        links = [T.dtree(n, r)[t] for r in range(n)]
        roots = [r for r in range(n) if links[r][0] < 0]
        assert len(roots) == 1
        root = roots[0]
        assert root == (0 if t == 0 else (n - 1 if n % 2 == 0 else 1 % n))
        kids_of = {r: [c for c in links[r][1:] if c >= 0] for r in range(n)}
        for r in range(n):
            assert len(set(kids_of[r])) == len(kids_of[r])
            for c in kids_of[r]:
                assert 0 <= c < n and links[c][0] == r
            if r != root:
                assert r in kids_of[links[r][0]]
        # spanning, acyclic, shallow
        seen, frontier, depth = {root}, [root], 0
        while frontier:
            nxt = [c for r in frontier for c in kids_of[r]]
            assert not (set(nxt) & seen)
            seen |= set(nxt)
            if nxt:
                depth += 1
            frontier = nxt
        assert seen == set(range(n))
        assert depth <= depth_bound, (n, t, depth)
        # the root has one child (second slot), as in ncclGetBtree
        if n > 1:
            assert links[root][1] == -1 or t == 1 and n % 2 == 1
        interior.append({r for r in range(n) if kids_of[r]})
    if n % 2 == 0 and n > 1:
        # mirror: tree 0's interior ranks are the even ones, tree 1's the odd
        # ones, so every rank forwards in exactly one tree
        assert interior[0] == set(range(0, n, 2))
        assert interior[1] == set(range(1, n, 2))


@pytest.mark.parametrize("row", _rows("tree_fold_fp32.txt"), ids=lambda r: f"{r[0]}{r[1]}")
def test_tree_fold_golden(row):
    pat, count, h, v0, v1 = row[0], int(row[1]), int(row[2]), float(row[3]), float(row[4])
    big = float(1 << 24)
    values = {"A": [5.0, 1.0, big, -big], "B": [-big, big, 1.0, 3.0]}[pat]
    xs = [np.full(count, v, dtype=np.float32) for v in values]
    assert T.tree_split(count, "float32") == h
    out = T.tree_allreduce(xs, "sum", "float32")
    want = np.array([v0] * h + [v1] * (count - h), dtype=np.float32)
    for r in range(4):
        assert np.array_equal(out[r], want), (pat, count, r, out[r])


def _wrap_reduce(stack, op, dtype):
    if op == "sum":
        return np.sum(stack.astype(np.int64), axis=0).astype(R.STORAGE[dtype])
    if op == "prod":
        return np.prod(stack.astype(np.int64), axis=0).astype(R.STORAGE[dtype])
    return (np.max if op == "max" else np.min)(stack, axis=0)


@pytest.mark.parametrize("dtype", ["int32", "int64"])
@pytest.mark.parametrize("op", ["sum", "prod", "max", "min"])
@pytest.mark.parametrize("n", [1, 2, 3, 5, 8, 13, 16])
def test_tree_integers_equal_numpy(dtype, op, n):
    rng = np.random.default_rng(1000 * n + len(op))
    info = np.iinfo(R.STORAGE[dtype])
    count = 77
    xs = [rng.integers(info.min, info.max, count, dtype=R.STORAGE[dtype], endpoint=True) for _ in range(n)]
    out = T.tree_allreduce(xs, op, dtype)
    want = _wrap_reduce(np.stack(xs), op, dtype)
    for r in range(n):
        assert np.array_equal(out[r], want), r


@pytest.mark.parametrize("op", ["max", "min"])
@pytest.mark.parametrize("dtype", ["float32", "bfloat16"])
def test_tree_float_max_min_are_order_free(op, dtype):
    """max/min are order-free (signed zeros included), so the tree must agree
    with the ring oracle bit for bit."""
    rng = np.random.default_rng(7)
    n, count = 11, 203
    f = [rng.standard_normal(count).astype(np.float32) for _ in range(n)]
    for x in f:
        x[::7] = 0.0
        x[::11] = -0.0
    xs = f if dtype == "float32" else [R.f64_to_bf16(x.astype(np.float64)) for x in f]
    t = T.tree_allreduce(xs, op, dtype)
    g = R.ring_allreduce(xs, op, dtype, nchannels=3)
    for r in range(n):
        assert np.array_equal(t[r].view(np.uint32 if dtype == "float32" else np.uint16),
                              g[r].view(np.uint32 if dtype == "float32" else np.uint16))


def _brute_tree(vals, links, h, op, dtype):
    """Per-element fold from the hand-derived link table: own value, then the
    first child's subtree, then the second's (reading T1)."""
    n = len(vals)
    count = len(vals[0])

    def fold(r, e, t):
        acc = vals[r][e]
        for c in links[(n, r, t)][1:]:
            if c >= 0:
                acc = X.hop(acc, fold(c, e, t), op, dtype)
        return acc

    res = []
    for e in range(count):
        t = 0 if e < h else 1
        root = [r for r in range(n) if links[(n, r, t)][0] < 0][0]
        res.append(fold(root, e, t))
    return res


@pytest.mark.parametrize("dtype", ["float32", "bfloat16", "int32"])
@pytest.mark.parametrize("op", ["sum", "prod", "max", "min"])
@pytest.mark.parametrize("n", [4, 5, 6, 8])
def test_tree_brute_force_exact(dtype, op, n):
    tab = _tables()
    rng = np.random.default_rng(31 * n + 3 * len(op) + len(dtype))
    for count in (0, 1, 3, 4, 5, 8, 9, 17, 24, 33):
        if dtype == "int32":
            xs = [rng.integers(-50, 51, count).astype(np.int32) for _ in range(n)]
        else:
            # mixed magnitudes so that the fold order changes roundings
            hi = 4 if op == "prod" else 25  # products of 8 values must stay finite
            f = [(rng.standard_normal(count) * np.exp2(rng.integers(-3, hi, count))).astype(np.float32)
                 for _ in range(n)]
            xs = f if dtype == "float32" else [R.f64_to_bf16(x.astype(np.float64)) for x in f]
        out = T.tree_allreduce(xs, op, dtype)
        vals = [X.to_scalar_list(x, dtype) for x in xs]
        h = T.tree_split(count, dtype)
        want = _brute_tree(vals, tab, h, op, dtype)
        for r in range(n):
            assert X.to_scalar_list(out[r], dtype) == want, (count, r)


def test_tree_fifo_traffic_equals_ring():
    """Each tree moves its half once up and once down every edge: 2(N-1)S
    bytes of FIFO writes in all, the same as the ring's 2(N-1)/N S per rank."""
    rng = np.random.default_rng(3)
    for n, count in ((2, 64), (5, 1000), (8, 4096), (16, 333)):
        xs = [rng.integers(-5, 6, count).astype(np.int32) for _ in range(n)]
        st = {}
        T.tree_allreduce(xs, "sum", "int32", stats=st)
        rs = R._new_stats(n)
        R.ring_allreduce(xs, "sum", "int32", stats=rs)
        total = sum(st["up_bytes"]) + sum(st["down_bytes"])
        assert total == sum(rs.recv_bytes) == 2 * (n - 1) * count * 4


@pytest.mark.parametrize("dtype,tol", [("float32", 1e-6), ("bfloat16", None)])
def test_tree_error_bound(dtype, tol):
    rng = np.random.default_rng(11)
    n, count = 16, 20_000
    f = [rng.standard_normal(count).astype(np.float32) for _ in range(n)]
    xs = f if dtype == "float32" else [R.f64_to_bf16(x.astype(np.float64)) for x in f]
    x64 = np.stack([x.astype(np.float64) if dtype == "float32" else R.bf16_to_f64(x) for x in xs])
    exact = x64.sum(axis=0)
    mag = np.abs(x64).sum(axis=0)
    y = T.tree_allreduce(xs, "sum", dtype)[0]
    y64 = y.astype(np.float64) if dtype == "float32" else R.bf16_to_f64(y)
    if dtype == "float32":
        assert np.all(np.abs(y64 - exact) <= tol * mag)
    else:
        u = 2.0 ** -8
        gamma = (n - 1) * u / (1 - (n - 1) * u)
        assert np.all(np.abs(y64 - exact) <= gamma * mag)
        assert np.linalg.norm(y64 - exact) / np.linalg.norm(exact) <= 8e-3
