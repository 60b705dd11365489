"""CPU oracle for the ring collectives and the double-binary-tree
all-reduce (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. See ``oracle/ring.py`` and
``oracle/tree.py`` for the sources they follow and the readings they take.
"""
from .ring import (  # noqa: F401
    DTYPES,
    OPS,
    ELEM_SIZE,
    STORAGE,
    DEFAULT_CHUNK_BYTES,
    Stats,
    algorithmic_bytes,
    all_gather_slice_schedule,
    allreduce_chunk_of,
    allreduce_fifo_steps_per_loop,
    allreduce_loop_chunks,
    alltoall,
    bf16_to_f64,
    block_loop_ranges,
    broadcast,
    channel_ranges,
    combine,
    f64_to_bf16,
    reduce,
    ring_all_gather,
    ring_allreduce,
    ring_reduce_scatter,
)
from .tree import btree, dtree, tree_allreduce, tree_root, tree_split  # noqa: F401,E402
