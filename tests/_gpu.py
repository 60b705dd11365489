"""Helpers for the GPU tests: host <-> device copies of per-rank buffers and
one-call wrappers around the C ABI. Device results are always compared with
values the CPU oracle computed from the same host inputs."""
from __future__ import annotations

import sys

import numpy as np

import ring_all_reduce_allreduce_amd as rs


def torch_dtype(dtype: str):
    import torch

    return {"int32": torch.int32, "int64": torch.int64, "float32": torch.float32,
            "bfloat16": torch.bfloat16}[dtype]


def to_device(x: np.ndarray, dtype: str):
    import torch

    if dtype == "bfloat16":
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint16).view(np.int16))
        return t.to("cuda:0").view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0")


def to_host(t, dtype: str) -> np.ndarray:
    import torch

    if dtype == "bfloat16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def empty_like_rank(n: int, dtype: str, fill_bits: int = 0x7F):
    """A device buffer filled with a byte pattern, so that unwritten elements show."""
    import torch

    e = {"int32": 4, "int64": 8, "float32": 4, "bfloat16": 2}[dtype]
    raw = torch.full((n * e,), fill_bits, dtype=torch.uint8, device="cuda:0")
    return raw.view(torch_dtype(dtype))


def say(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def bits_equal(a: np.ndarray, b: np.ndarray, dtype: str) -> bool:
    if dtype == "float32":
        return np.array_equal(np.asarray(a, np.float32).view(np.uint32), np.asarray(b, np.float32).view(np.uint32))
    return np.array_equal(a, b)


def first_mismatch(a: np.ndarray, b: np.ndarray, dtype: str):
    if dtype == "float32":
        a = np.asarray(a, np.float32).view(np.uint32)
        b = np.asarray(b, np.float32).view(np.uint32)
    idx = np.nonzero(a != b)[0]
    if idx.size == 0:
        return None
    i = int(idx[0])
    return i, a[i], b[i], int(idx.size)


def sync():
    import torch

    torch.cuda.synchronize()


def check_comm_ok(comm) -> None:
    err = rs.get_async_error(comm)
    assert err == rs.SUCCESS, rs.RESULT_NAMES.get(err, err)
