"""Soak of the WIDE line format (MI355X only).

WIDE lines (the ring's WIDE protocol and every tree step) carry 12 payload
bytes and their flag in one 16-byte line, written and read as one 128-bit
access: a consumer that saw the flag takes the payload of the same access.
That relies on the line never being delivered torn. Here a few hundred calls
with fresh seeded inputs run through both users of the format at the sizes
where they run by default, each compared element by element with the
oracle; the test stops at the first mismatch and reports how many lines
moved before it."""
import numpy as np
import pytest

import oracle
import ring_all_reduce_allreduce_amd as rs
import synth
from tests import _gpu as G

pytestmark = pytest.mark.gpu

SOAK_WORKLOAD = 90  # seed space of this test's inputs


@pytest.fixture(scope="module", autouse=True)
def _device():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    rs.lib()
    yield
    torch.cuda.synchronize()


# (name, ranks, channels, comm config, byte range per rank, calls)
CONFIGS = [
    ("wide ring 16x16 w1", 16, 16, dict(proto="wide", algo="ring", line_workgroups_per_channel=1),
     (1 << 20, 2 << 20), 100),
    ("wide ring 8x8 w4", 8, 8, dict(proto="wide", algo="ring", line_workgroups_per_channel=4),
     (1 << 20, 2 << 20), 100),
    ("tree 16x16", 16, 16, dict(proto="auto", algo="tree"), (64 << 10, 1 << 20), 100),
]


@pytest.mark.parametrize("name,n,nch,cfg,span,calls", CONFIGS, ids=[c[0] for c in CONFIGS])
def test_wide_lines_soak(name, n, nch, cfg, span, calls):
    import torch

    proto = cfg.pop("proto")
    comm = rs.comm_init(n, nch, proto, **cfg)
    rng = np.random.default_rng(4242 + n * 100 + nch)
    lines = 0
    try:
        for k in range(calls):
            dtype = "int32" if k % 2 == 0 else "float32"
            count = int(rng.integers(span[0] // 4, span[1] // 4 + 1))
            if k % 25 == 0:
                G.say(f"{name}: call {k} count {count} {dtype}")
            if dtype == "int32":
                send = synth.device_inputs(SOAK_WORKLOAD, n, count, dtype, "int", lo=-(1 << 20), hi=1 << 20, bucket=k)
            else:
                send = synth.device_inputs(SOAK_WORKLOAD, n, count, dtype, "normal", bucket=k)
            recv = [torch.empty_like(t) for t in send]
            rs.allreduce(comm, send, recv)
            xs = [t.cpu().numpy() for t in send]
            G.sync()
            G.check_comm_ok(comm)
            if cfg.get("algo") == "tree":
                want = oracle.tree_allreduce(xs, "sum", dtype)
            else:
                want = oracle.ring_allreduce(xs, "sum", dtype, nchannels=nch)
            for r in range(n):
                mm = G.first_mismatch(recv[r].cpu().numpy(), want[r], dtype)
                assert mm is None, f"{name}: call {k} ({count} {dtype}) rank {r} first mismatch {mm} after {lines} lines"
            # every rank forwards 2(N-1)/N of its buffer, 12 payload bytes per line
            lines += 2 * (n - 1) * count * 4 // 12
            del send, recv
        info = rs.comm_query(comm)
        assert info["last_algo"] == (2 if cfg.get("algo") == "tree" else 1)
        if cfg.get("algo") != "tree":
            assert info["last_proto"] == 3  # WIDE
        G.say(f"{name}: {calls} calls, about {lines / 1e6:.1f} M WIDE lines, no mismatch")
    finally:
        rs.comm_destroy(comm)
