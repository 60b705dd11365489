"""CPU oracle for the ring collectives (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. See ``oracle/ring.py`` for the sources
it follows and the readings it takes.
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
