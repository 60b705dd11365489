"""Seeded synthetic inputs for the ring collectives.

This module is shared by the GPU-side tests, the oracle-side tests and the
benchmark. It draws random numbers and casts them to the storage type; it
contains none of the collective arithmetic (no reduction, no ring order).

Every generator uses NumPy ``Generator(PCG64(seed))`` with
``seed = 1_000_000 * workload + 1_000 * bucket + rank``, so that each rank's
buffer is reproducible on its own. Host arrays are plain NumPy arrays; bfloat16
data is carried as ``uint16`` bit patterns, produced from float32 draws by
round-to-nearest-even through ``torch`` (CPU).

Workloads (shapes follow the pages' use cases; no benchmark data is copied):
  1  nccl-tests-style correctness AllReduce: 4 ranks x 1024 fp32, integers in
     [-8, 8] (inclusive) stored as fp32 so every sum is exact.
  2  large AllReduce: 8 ranks x 16,777,216 fp32 (64 MiB) ~ N(0, 1).
  3  DDP gradient bucket: 8 ranks x 13,107,200 bf16 (25 MiB) ~ N(0, 1e-3),
     40 distinct buckets (bucket b drawn with seed ... + 1,000 b; at full size
     on the device, see device_inputs).
  4  message-size sweep: 16 ranks, int32 uniform in [-2^20, 2^20] (inclusive).
  5  FSDP / MoE: reduce-scatter of 8 ranks x 67,108,864 bf16 (128 MiB) ~ N(0,1);
     all-to-all of 8 chunks x 512 tokens x 4096 bf16 uniform in [-1, 1).
"""
from __future__ import annotations

import numpy as np

STORAGE = {
    "int32": np.int32,
    "int64": np.int64,
    "float32": np.float32,
    "bfloat16": np.uint16,
}
ELEM_SIZE = {"int32": 4, "int64": 8, "float32": 4, "bfloat16": 2}


def seed_for(workload: int, rank: int, bucket: int = 0) -> int:
    return 1_000_000 * workload + 1_000 * bucket + rank


def rng_for(workload: int, rank: int, bucket: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed_for(workload, rank, bucket)))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest-even) and return the bits."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def draw(rng: np.random.Generator, n: int, dtype: str, dist: str, scale: float = 1.0,
         lo: int = 0, hi: int = 0) -> np.ndarray:
    """Draw ``n`` values of ``dtype`` from a named distribution.

    dist: "normal" (mean 0, std ``scale``), "uniform" (float in [-scale, scale)),
    "int" (integers in [lo, hi], inclusive).
    """
    if dist == "int":
        v = rng.integers(lo, hi + 1, size=n, dtype=np.int64)
        if dtype == "bfloat16":
            return f32_to_bf16_bits(v.astype(np.float32))
        return v.astype(STORAGE[dtype])
    if dist == "normal":
        v = rng.standard_normal(n, dtype=np.float32)
        if scale != 1.0:
            v = (v * np.float32(scale)).astype(np.float32)
    elif dist == "uniform":
        v = (rng.random(n, dtype=np.float32) * np.float32(2.0) - np.float32(1.0)) * np.float32(scale)
        v = v.astype(np.float32)
    else:
        raise ValueError(dist)
    if dtype == "bfloat16":
        return f32_to_bf16_bits(v)
    if dtype in ("int32", "int64"):
        raise ValueError("integer dtypes need dist='int'")
    return v.astype(STORAGE[dtype])


def rank_inputs(workload: int, nranks: int, n: int, dtype: str, dist: str, scale: float = 1.0,
                lo: int = 0, hi: int = 0, bucket: int = 0) -> list[np.ndarray]:
    """One seeded buffer of ``n`` elements per rank."""
    return [draw(rng_for(workload, r, bucket), n, dtype, dist, scale, lo, hi) for r in range(nranks)]


# Named workloads --------------------------------------------------------------

WORKLOADS = {
    1: dict(coll="allreduce", nranks=4, n=1024, dtype="float32", dist="int", lo=-8, hi=8,
            nchannels=1, op="sum", proto="bulk"),
    2: dict(coll="allreduce", nranks=8, n=16_777_216, dtype="float32", dist="normal", scale=1.0,
            nchannels=8, op="sum", chunk_bytes=524_288, proto="bulk"),
    3: dict(coll="allreduce", nranks=8, n=13_107_200, dtype="bfloat16", dist="normal", scale=1e-3,
            nchannels=16, op="sum", buckets=40, proto="bulk"),
    4: dict(coll="allreduce", nranks=16, dtype="int32", dist="int", lo=-(1 << 20), hi=(1 << 20),
            ops=("sum", "max"), sizes_bytes=[8 << k for k in range(26)]),
    5: dict(coll="rs_ag_a2a", nranks=8, n_rs=67_108_864, dtype="bfloat16", dist="normal", scale=1.0,
            nchannels=8, a2a_chunk=(512, 4096), a2a_dist="uniform"),
}


def workload_inputs(workload: int, n: int | None = None, bucket: int = 0, nranks: int | None = None,
                    dtype: str | None = None) -> list[np.ndarray]:
    """Inputs of a named workload, optionally at a reduced element count."""
    w = WORKLOADS[workload]
    nr = nranks if nranks is not None else w["nranks"]
    dt = dtype if dtype is not None else w["dtype"]
    if n is None:
        n = w.get("n", w.get("n_rs"))
    return rank_inputs(workload, nr, n, dt, w["dist"], w.get("scale", 1.0), w.get("lo", 0),
                       w.get("hi", 0), bucket)


def a2a_inputs(nranks: int = 8, tokens: int = 512, hidden: int = 4096, dtype: str = "bfloat16",
               workload: int = 5, bucket: int = 1) -> list[np.ndarray]:
    """All-to-all buffers: each rank holds ``nranks`` chunks of tokens x hidden."""
    n = nranks * tokens * hidden
    return rank_inputs(workload, nranks, n, dtype, "uniform", 1.0, bucket=bucket)


# Device-side generators for the full-size workloads --------------------------
# Host generation of gigabytes of draws takes minutes; these use torch's seeded
# device RNG instead (same seed formula). Tests copy the sampled elements they
# check back to the host and give those to the oracle.

def device_inputs(workload: int, nranks: int, n: int, dtype: str, dist: str, scale: float = 1.0,
                  lo: int = 0, hi: int = 0, bucket: int = 0, device: str = "cuda:0"):
    """One seeded device buffer of ``n`` elements per rank (torch tensors)."""
    import torch

    tdt = {"int32": torch.int32, "int64": torch.int64, "float32": torch.float32,
           "bfloat16": torch.bfloat16}[dtype]
    out = []
    for r in range(nranks):
        g = torch.Generator(device=device)
        g.manual_seed(seed_for(workload, r, bucket))
        if dist == "int":
            t = torch.randint(lo, hi + 1, (n,), generator=g, device=device, dtype=torch.int64)
            out.append(t.to(tdt))
        elif dist == "normal":
            t = torch.randn(n, generator=g, device=device, dtype=torch.float32) * scale
            out.append(t.to(tdt))
        elif dist == "uniform":
            t = (torch.rand(n, generator=g, device=device, dtype=torch.float32) * 2.0 - 1.0) * scale
            out.append(t.to(tdt))
        else:
            raise ValueError(dist)
    return out
