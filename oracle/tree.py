"""Plain CPU oracle for the double-binary-tree all-reduce.

TEST INFRASTRUCTURE, under the same rule as ``oracle/ring.py``: only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it, and it shares no code with the library.

Sources (page title, section):
  [NB 4]   "NCCL" book (aireadcode.com), ch. 4 (topology to algorithm),
           ``ncclGetBtree``: a rank's parent and two children follow from its
           lowest set bit; rank 0 is the root and has one child. The worked
           example gives rank 1 of 8 the parent 2 and no children.
           ``ncclGetDtree``: the second tree mirrors the first
           (rank r plays N-1-r) for an even rank count and shifts it by one
           (rank r plays r-1) for an odd one. The two trees run at once, one
           on the first half of the data and one on the second.
  [NB 5]   same book, ch. 5 (tuning), tree.cc: the tree serves the all-reduce
           only, as a reduce up the tree followed by a broadcast down it.

The tree rule, restated. Let ``bit`` be the lowest set bit of the rank; for
rank 0 it is the smallest power of two >= N.
  * Rank 0 is the root: no parent; its only child is bit/2 (when N > 1),
    held in the second child slot.
  * Any other rank r: the parent is r with ``bit`` cleared and 2*bit set, or,
    when that is >= N, r with ``bit`` cleared. The first child is r - bit/2
    (none when bit == 1). The second child is r + b for the largest b among
    bit/2, bit/4, ..., 1 with r + b < N (none when bit == 1 or no b fits).

Readings taken where the pages are silent:
  T1  Fold order at a node: its own data first, then the partial result of
      its first child, then that of its second child, rounding to the buffer
      type after every operation (reading R5 of ``oracle/ring.py``). The
      root's partial is the result, which every rank receives unchanged.
  T2  Child order in the second tree: the first tree's child slots are
      carried through the relabelling (mirror: N-1-c; shift: c+1 mod N).
  T3  "Half of the data": tree 0 takes elements [0, h) and tree 1 [h, count)
      with h = min(count, alignUp(ceil(count/2), 16/e)), so that tree 1
      starts on a 16-byte boundary like every channel of the ring (R2).
  T4  Channels, slices and pipelining split each tree's range further but
      never change which tree folds an element, so results do not depend on
      them; the oracle folds each tree's range whole.

Parity status: pinned by ``tests/test_oracle_tree.py`` (hand-derived tree
tables and fold values in ``tests/golden/``, spanning-tree and double-tree
invariants for every N up to 64, integer and max/min equality with NumPy's
reductions, exact-rational brute force on small inputs, the error bound).
"""
from __future__ import annotations

import numpy as np

from .ring import ELEM_SIZE, _check_inputs, align_up, combine, div_up, elems_per_16b


def btree(nranks: int, rank: int) -> tuple[int, int, int]:
    """[NB 4] (parent, first child, second child) of ``rank``; -1 = none."""
    if not 0 <= rank < nranks:
        raise ValueError("rank out of range")
    bit = 1
    while bit < nranks and not (rank & bit):
        bit <<= 1
    half = bit >> 1
    if rank == 0:
        return -1, -1, (half if nranks > 1 else -1)
    parent = (rank & ~bit) | (bit << 1)
    if parent >= nranks:
        parent = rank & ~bit
    first = rank - half if half else -1
    second = -1
    b = half
    while b:
        if rank + b < nranks:
            second = rank + b
            break
        b >>= 1
    return parent, first, second


def dtree(nranks: int, rank: int) -> tuple[tuple[int, int, int], tuple[int, int, int]]:
    """[NB 4] both trees of the double binary tree for ``rank``:
    ((parent, child0, child1) in tree 0, the same in tree 1)."""
    t0 = btree(nranks, rank)
    if nranks % 2 == 0:
        role = nranks - 1 - rank

        def back(x):
            return -1 if x < 0 else nranks - 1 - x
    else:
        role = (rank - 1) % nranks

        def back(x):
            return -1 if x < 0 else (x + 1) % nranks
    p, c0, c1 = btree(nranks, role)
    return t0, (back(p), back(c0), back(c1))


def tree_root(nranks: int, tree: int) -> int:
    for r in range(nranks):
        if dtree(nranks, r)[tree][0] < 0:
            return r
    raise AssertionError("no root")


def tree_split(count: int, dtype: str) -> int:
    """Reading T3: first element of tree 1's half."""
    return min(count, align_up(div_up(count, 2), elems_per_16b(dtype)))


def tree_allreduce(inputs, op: str = "sum", dtype: str = "float32", stats: dict | None = None) -> list[np.ndarray]:
    """Double-binary-tree all-reduce [NB 4, NB 5]: in each tree, every rank
    sends its partial result up to its parent once all of its children's
    partials have arrived (reading T1 for the fold order); the root's partial
    is the reduction, and it travels back down, each rank storing it and
    passing it on to its children.

    ``stats`` (optional) receives per-rank FIFO bytes sent up and down.
    """
    xs = _check_inputs(inputs, dtype)
    nr = len(xs)
    count = xs[0].shape[0]
    if nr == 1:
        return [xs[0].copy()]
    e = ELEM_SIZE[dtype]
    h = tree_split(count, dtype)
    out = [np.zeros_like(x) for x in xs]
    if stats is not None:
        stats.setdefault("up_bytes", [0] * nr)
        stats.setdefault("down_bytes", [0] * nr)
    for t, (lo, hi) in enumerate(((0, h), (h, count))):
        if hi <= lo:
            continue
        links = [dtree(nr, r)[t] for r in range(nr)]
        root = [r for r in range(nr) if links[r][0] < 0]
        assert len(root) == 1
        # Up: a rank is ready once every child has delivered. Messages are
        # kept per (child -> parent) edge.
        up_msg: dict[int, np.ndarray] = {}
        partial: dict[int, np.ndarray] = {}
        pending = set(range(nr))
        while pending:
            progressed = False
            for r in sorted(pending):
                kids = [c for c in links[r][1:] if c >= 0]
                if all(c in up_msg for c in kids):
                    acc = xs[r][lo:hi].copy()
                    for c in kids:
                        acc = combine(acc, up_msg.pop(c), op, dtype)
                    partial[r] = acc
                    if links[r][0] >= 0:
                        up_msg[r] = acc
                        if stats is not None:
                            stats["up_bytes"][r] += (hi - lo) * e
                    pending.discard(r)
                    progressed = True
            assert progressed, "tree has a cycle"
        assert not up_msg
        # Down: the root's result is passed parent -> child unchanged.
        frontier = [root[0]]
        out[root[0]][lo:hi] = partial[root[0]]
        while frontier:
            nxt = []
            for r in frontier:
                for c in links[r][1:]:
                    if c >= 0:
                        out[c][lo:hi] = out[r][lo:hi]
                        if stats is not None:
                            stats["down_bytes"][r] += (hi - lo) * e
                        nxt.append(c)
            frontier = nxt
    return out
