"""ringsim: ring collectives over N simulated ranks in one MI355X's HBM.

A thin ctypes binding over ``libringsim.so`` (C ABI in ``include/ringsim.h``).
It only marshals arguments: every step of a collective runs in the library's
HIP kernels. PyTorch provides device memory and streams.

Functions carry the C names without the ``ringsim_`` prefix:

    comm = comm_init(nranks, nchannels, proto="auto", **config)
    allreduce(comm, sendbufs, recvbufs, count=None, op="sum", stream=None)
    allreduce_noalloc(nranks, nchannels, sendbufs, recvbufs, count=None, op="sum", stream=None)
    reduce_scatter(comm, sendbufs, recvbufs, recvcount=None, op="sum", stream=None)
    all_gather(comm, sendbufs, recvbufs, sendcount=None, stream=None)
    alltoall(comm, sendbufs, recvbufs, count=None, stream=None)
    get_async_error(comm); abort(comm); comm_query(comm); comm_destroy(comm)
    debug_plan(coll, count, nranks, nchannels, chunk_bytes, dtype)
    debug_model(coll, nranks, nchannels, bytes_per_rank)
    debug_tree(nranks, rank); debug_tree_model(nranks, tree_channels, bytes_per_rank)
    debug_flag_steps(coll, algo, nranks, nchannels, chunk_bytes, count, dtype, proto)

``sendbufs``/``recvbufs`` are lists (one per simulated rank) of CUDA/HIP
tensors of one dtype, or of raw device addresses (ints; then ``dtype`` and the
count must be given). Every call is asynchronous on ``stream`` (default: the
current torch stream) and raises :class:`RingsimError` on a non-success code.

The library is loaded on first use. ``torch`` is imported before it so that
libringsim binds to the HIP runtime torch already loaded (both carry the same
soname); a missing library raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os
from typing import Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libringsim.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "ringsim.h")

SUCCESS = 0
RESULT_NAMES = {
    0: "SUCCESS",
    1: "UNHANDLED_DEVICE_ERROR",
    2: "SYSTEM_ERROR",
    3: "INTERNAL_ERROR",
    4: "INVALID_ARGUMENT",
    5: "INVALID_USAGE",
    7: "IN_PROGRESS",
    8: "ABORTED",
}
DTYPES = {"int32": 0, "int64": 1, "float32": 2, "bfloat16": 3}
ELEM_SIZE = {"int32": 4, "int64": 8, "float32": 4, "bfloat16": 2}
OPS = {"sum": 0, "prod": 1, "max": 2, "min": 3}
PROTOS = {"auto": 0, "bulk": 1, "flag": 2, "wide": 3}
ALGOS = {"auto": 0, "ring": 1, "tree": 2}
COLLS = {"allreduce": 0, "reduce_scatter": 1, "all_gather": 2, "alltoall": 3}
# Limits of the ABI (the RINGSIM_MAX_* macros of the header).
MAX_RANKS = 64
MAX_CHANNELS = 64
MAX_WORKGROUPS_PER_CHANNEL = 16


class RingsimError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        self.name = RESULT_NAMES.get(code, str(code))
        super().__init__(f"{what}: {self.name} ({code})")


class Config(ctypes.Structure):
    _fields_ = [
        ("chunk_bytes", ctypes.c_size_t),
        ("workgroups_per_channel", ctypes.c_int),
        ("slot_bytes", ctypes.c_size_t),
        ("nslots", ctypes.c_int),
        ("timeout_ms", ctypes.c_int),
        ("flag_threshold_bytes", ctypes.c_size_t),
        ("algo", ctypes.c_int),
        ("line_workgroups_per_channel", ctypes.c_int),
    ]


class CommInfo(ctypes.Structure):
    _fields_ = [
        ("nranks", ctypes.c_int),
        ("nchannels", ctypes.c_int),
        ("proto", ctypes.c_int),
        ("workgroups_per_channel", ctypes.c_int),
        ("nslots", ctypes.c_int),
        ("device", ctypes.c_int),
        ("chunk_bytes", ctypes.c_size_t),
        ("slot_bytes", ctypes.c_size_t),
        ("flag_threshold_bytes", ctypes.c_size_t),
        ("fifo_bytes", ctypes.c_size_t),
        ("flag_fifo_bytes", ctypes.c_size_t),
        ("max_resident_workgroups", ctypes.c_int),
        ("compute_units", ctypes.c_int),
        ("calls", ctypes.c_uint64),
        ("last_proto", ctypes.c_int),
        ("algo", ctypes.c_int),
        ("tree_channels", ctypes.c_int),
        ("tree_fifo_bytes", ctypes.c_size_t),
        ("last_algo", ctypes.c_int),
        ("line_max_workgroups_per_channel", ctypes.c_int),
        ("last_workgroups_per_channel", ctypes.c_int),
        ("last_tree_channels", ctypes.c_int),
        ("line_fifo_resets", ctypes.c_uint64),
        ("tree_fifo_resets", ctypes.c_uint64),
        ("last_group_steps", ctypes.c_int),
    ]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


_lib = None
_c_ptrs = ctypes.POINTER(ctypes.c_void_p)


def lib() -> ctypes.CDLL:
    """The loaded library (loads it on first call)."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  -- bind to torch's HIP runtime first

    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m ring_all_reduce_allreduce_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i, sz, res = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_int
    sig = {
        "ringsim_config_default": (res, [ctypes.POINTER(Config)]),
        "ringsim_comm_init": (res, [ctypes.POINTER(vp), i, i, i]),
        "ringsim_comm_init_config": (res, [ctypes.POINTER(vp), i, i, i, ctypes.POINTER(Config)]),
        "ringsim_comm_destroy": (res, [vp]),
        "ringsim_comm_query": (res, [vp, ctypes.POINTER(CommInfo)]),
        "ringsim_allreduce": (res, [vp, _c_ptrs, _c_ptrs, sz, i, i, vp]),
        "ringsim_reduce_scatter": (res, [vp, _c_ptrs, _c_ptrs, sz, i, i, vp]),
        "ringsim_all_gather": (res, [vp, _c_ptrs, _c_ptrs, sz, i, vp]),
        "ringsim_alltoall": (res, [vp, _c_ptrs, _c_ptrs, sz, i, vp]),
        "ringsim_get_async_error": (res, [vp, ctypes.POINTER(res)]),
        "ringsim_abort": (res, [vp]),
        "ringsim_get_error_string": (ctypes.c_char_p, [res]),
        "ringsim_debug_plan": (res, [i, sz, i, i, sz, i, ctypes.POINTER(ctypes.c_int64), sz, ctypes.POINTER(sz)]),
        "ringsim_debug_model": (res, [i, i, i, sz, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double),
                                        ctypes.POINTER(ctypes.c_double)]),
        "ringsim_debug_tree": (res, [i, i, ctypes.POINTER(ctypes.c_int)]),
        "ringsim_debug_tree_model": (res, [i, i, sz, ctypes.POINTER(ctypes.c_double)]),
        "ringsim_allreduce_noalloc": (res, [i, i, _c_ptrs, _c_ptrs, sz, i, i, vp]),
        "ringsim_debug_flag_steps": (res, [i, i, i, i, sz, sz, i, i, ctypes.POINTER(ctypes.c_uint64)]),
    }
    for name, (rt, args) in sig.items():
        f = getattr(L, name)
        f.restype = rt
        f.argtypes = args
    _lib = L
    return L


def _check(code: int, what: str) -> None:
    if code != SUCCESS:
        raise RingsimError(code, what)


def error_string(code: int) -> str:
    return lib().ringsim_get_error_string(code).decode()


class Comm:
    """A communicator handle (owns the library object until destroyed)."""

    def __init__(self, handle: int, nranks: int):
        self.handle = handle
        self.nranks = nranks

    @property
    def _as_parameter_(self):
        return ctypes.c_void_p(self.handle)

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        if self.handle:
            comm_destroy(self)


def config_default() -> Config:
    cfg = Config()
    _check(lib().ringsim_config_default(ctypes.byref(cfg)), "ringsim_config_default")
    return cfg


def comm_init(nranks: int, nchannels: int, proto: str | int = "auto", **config) -> Comm:
    """Creates a communicator. Keyword tunables: chunk_bytes,
    workgroups_per_channel, slot_bytes, nslots, timeout_ms,
    flag_threshold_bytes, algo ("auto", "ring", "tree"; 0 or absent = library
    default), line_workgroups_per_channel (1, 2, 4 or 8; 0 = per call)."""
    p = PROTOS[proto] if isinstance(proto, str) else int(proto)
    if isinstance(config.get("algo"), str):
        config["algo"] = ALGOS[config["algo"]]
    h = ctypes.c_void_p()
    if config:
        cfg = Config()
        for k, v in config.items():
            if v is not None:
                setattr(cfg, k, int(v))
        code = lib().ringsim_comm_init_config(ctypes.byref(h), nranks, nchannels, p, ctypes.byref(cfg))
    else:
        code = lib().ringsim_comm_init(ctypes.byref(h), nranks, nchannels, p)
    _check(code, "ringsim_comm_init")
    return Comm(h.value, nranks)


def comm_destroy(comm: Comm) -> None:
    h = comm.handle
    comm.handle = 0
    _check(lib().ringsim_comm_destroy(ctypes.c_void_p(h)), "ringsim_comm_destroy")


def comm_query(comm: Comm) -> dict:
    info = CommInfo()
    _check(lib().ringsim_comm_query(comm, ctypes.byref(info)), "ringsim_comm_query")
    return info.as_dict()


_TORCH_DTYPES: dict | None = None


def _dtype_name(t) -> str:
    global _TORCH_DTYPES
    if _TORCH_DTYPES is None:
        import torch

        _TORCH_DTYPES = {torch.int32: "int32", torch.int64: "int64", torch.float32: "float32",
                         torch.bfloat16: "bfloat16"}
    name = _TORCH_DTYPES.get(t.dtype)
    if name is None:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return name


def _ptr_array(bufs: Sequence) -> ctypes.Array:
    return (ctypes.c_void_p * len(bufs))(*[b if isinstance(b, int) else b.data_ptr() for b in bufs])


def _marshal(comm: Comm, sendbufs, recvbufs, dtype, send_need=None, recv_need=None):
    """Pointer arrays and the dtype code. Tensor buffers must be contiguous
    device tensors of one dtype (the given one, if any) holding at least
    `send_need` / `recv_need` elements; raw addresses are taken as they are."""
    if len(sendbufs) != comm.nranks or len(recvbufs) != comm.nranks:
        raise ValueError(f"need {comm.nranks} send and receive buffers")
    tensors = [b for b in list(sendbufs) + list(recvbufs) if not isinstance(b, int)]
    if dtype is None:
        if isinstance(sendbufs[0], int):
            raise ValueError("dtype is required with raw pointers")
        dtype = _dtype_name(sendbufs[0])
    code = DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
    for b in tensors:
        if DTYPES.get(_dtype_name(b)) != code:
            raise TypeError("all buffers must share the call's dtype")
        if not b.is_cuda:
            raise ValueError("buffers must be device tensors")
        if not b.is_contiguous():
            raise ValueError("buffers must be contiguous")
    for bufs, need in ((sendbufs, send_need), (recvbufs, recv_need)):
        if need is not None:
            for b in bufs:
                if not isinstance(b, int) and b.numel() < need:
                    raise ValueError(f"a buffer holds {b.numel()} elements, the call needs {need}")
    return _ptr_array(sendbufs), _ptr_array(recvbufs), code


def _current_stream() -> int:
    """The current HIP stream of the current device, as an integer handle."""
    import torch

    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return raw(torch.cuda.current_device())
    return torch.cuda.current_stream().cuda_stream


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        return ctypes.c_void_p(_current_stream())
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _numel(b) -> int:
    if isinstance(b, int):
        raise ValueError("a count is required with raw pointers")
    return b.numel()


def allreduce(comm: Comm, sendbufs, recvbufs, count: int | None = None, op: str | int = "sum",
              stream=None, dtype=None) -> None:
    n = _numel(sendbufs[0]) if count is None else count
    s, r, dt = _marshal(comm, sendbufs, recvbufs, dtype, n, n)
    o = OPS[op] if isinstance(op, str) else int(op)
    _check(lib().ringsim_allreduce(comm, s, r, n, dt, o, _stream(stream)), "ringsim_allreduce")


def allreduce_noalloc(nranks: int, nchannels: int, sendbufs, recvbufs, count: int | None = None,
                      op: str | int = "sum", stream=None, dtype=None) -> None:
    """The allocation-free all-reduce: the ring all-reduce of a communicator
    with ``nranks`` ranks and ``nchannels`` channels, run on the library's
    per-GPU scratch array instead of a communicator's memory."""
    n = _numel(sendbufs[0]) if count is None else count
    s, r, dt = _marshal(Comm(0, nranks), sendbufs, recvbufs, dtype, n, n)
    o = OPS[op] if isinstance(op, str) else int(op)
    _check(lib().ringsim_allreduce_noalloc(nranks, nchannels, s, r, n, dt, o, _stream(stream)),
           "ringsim_allreduce_noalloc")


def reduce_scatter(comm: Comm, sendbufs, recvbufs, recvcount: int | None = None, op: str | int = "sum",
                   stream=None, dtype=None) -> None:
    n = _numel(recvbufs[0]) if recvcount is None else recvcount
    s, r, dt = _marshal(comm, sendbufs, recvbufs, dtype, n * comm.nranks, n)
    o = OPS[op] if isinstance(op, str) else int(op)
    _check(lib().ringsim_reduce_scatter(comm, s, r, n, dt, o, _stream(stream)), "ringsim_reduce_scatter")


def all_gather(comm: Comm, sendbufs, recvbufs, sendcount: int | None = None, stream=None, dtype=None) -> None:
    n = _numel(sendbufs[0]) if sendcount is None else sendcount
    s, r, dt = _marshal(comm, sendbufs, recvbufs, dtype, n, n * comm.nranks)
    _check(lib().ringsim_all_gather(comm, s, r, n, dt, _stream(stream)), "ringsim_all_gather")


def alltoall(comm: Comm, sendbufs, recvbufs, count: int | None = None, stream=None, dtype=None) -> None:
    n = _numel(sendbufs[0]) // comm.nranks if count is None else count
    s, r, dt = _marshal(comm, sendbufs, recvbufs, dtype, n * comm.nranks, n * comm.nranks)
    _check(lib().ringsim_alltoall(comm, s, r, n, dt, _stream(stream)), "ringsim_alltoall")


def get_async_error(comm: Comm) -> int:
    out = ctypes.c_int(-1)
    _check(lib().ringsim_get_async_error(comm, ctypes.byref(out)), "ringsim_get_async_error")
    return out.value


def abort(comm: Comm) -> None:
    _check(lib().ringsim_abort(comm), "ringsim_abort")


def debug_model(coll: str | int, nranks: int, nchannels: int, bytes_per_rank: int) -> dict:
    """Predicted microseconds per protocol (host-only cost model behind AUTO)."""
    c = COLLS[coll] if isinstance(coll, str) else int(coll)
    b, f, w = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    _check(lib().ringsim_debug_model(c, nranks, nchannels, bytes_per_rank, ctypes.byref(b), ctypes.byref(f),
                                     ctypes.byref(w)),
           "ringsim_debug_model")
    return {"bulk_us": b.value, "flag_us": f.value, "wide_us": w.value}


def debug_tree(nranks: int, rank: int) -> tuple[tuple[int, int, int], tuple[int, int, int]]:
    """((parent, child0, child1) in tree 0, the same in tree 1) of ``rank``;
    host-only."""
    out = (ctypes.c_int * 6)()
    _check(lib().ringsim_debug_tree(nranks, rank, out), "ringsim_debug_tree")
    v = list(out)
    return tuple(v[:3]), tuple(v[3:])


def debug_tree_model(nranks: int, tree_channels: int, bytes_per_rank: int) -> float:
    """Predicted microseconds of a tree all-reduce; host-only."""
    us = ctypes.c_double()
    _check(lib().ringsim_debug_tree_model(nranks, tree_channels, bytes_per_rank, ctypes.byref(us)),
           "ringsim_debug_tree_model")
    return us.value


def debug_flag_steps(coll: str | int, algo: str | int, nranks: int, nchannels: int, chunk_bytes: int, count: int,
                     dtype: str | int, proto: str | int = "flag") -> int:
    """Upper bound of the steps one FIFO moves in a line (or tree) call, as
    the flag-span bookkeeping counts it; host-only."""
    c = COLLS[coll] if isinstance(coll, str) else int(coll)
    a = ALGOS[algo] if isinstance(algo, str) else int(algo)
    d = DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
    p = PROTOS[proto] if isinstance(proto, str) else int(proto)
    out = ctypes.c_uint64(0)
    _check(lib().ringsim_debug_flag_steps(c, a, nranks, nchannels, chunk_bytes, count, d, p, ctypes.byref(out)),
           "ringsim_debug_flag_steps")
    return out.value


def debug_plan(coll: str | int, count: int, nranks: int, nchannels: int, chunk_bytes: int, dtype: str | int):
    """Rows (channel, loop, chunk, begin, end) of the partition the kernels
    walk; host-only, needs no device."""
    c = COLLS[coll] if isinstance(coll, str) else int(coll)
    d = DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
    n = ctypes.c_size_t(0)
    _check(lib().ringsim_debug_plan(c, count, nranks, nchannels, chunk_bytes, d, None, 0, ctypes.byref(n)),
           "ringsim_debug_plan")
    rows = (ctypes.c_int64 * (5 * max(n.value, 1)))()
    _check(lib().ringsim_debug_plan(c, count, nranks, nchannels, chunk_bytes, d, rows, n.value, ctypes.byref(n)),
           "ringsim_debug_plan")
    flat = list(rows)[: 5 * n.value]
    return [tuple(flat[5 * k: 5 * k + 5]) for k in range(n.value)]


def header_exports() -> list[str]:
    """Function names declared in include/ringsim.h."""
    import re

    with open(HEADER_PATH) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(ringsim_[a-z_]+)\s*\(", text)))
