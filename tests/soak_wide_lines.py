"""Long soak of the WIDE line format, outside the pytest suite (MI355X only).

Usage: python tests/soak_wide_lines.py [seconds]   (default 480)

Runs the WIDE ring (16 ranks x 16 channels, one workgroup per channel; 8 x 8
with four) and the double-binary tree (16 x 16) in turn, 1-2 MiB and
64 KiB-1 MiB per rank, with fresh int32 inputs every call, and compares every
rank's result with the column sums of its inputs (an int32 sum does not
depend on the fold order). A torn 16-byte line would hand its consumer a
stale payload under a current flag and change a sum. Stops at the first
mismatch or asynchronous error; prints progress every 20 s and the lines
moved at the end. tests/test_gpu_line_soak.py is the short version that the
GPU suite runs against the oracle."""
import os
import sys
import time

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import torch  # noqa: E402
import ring_all_reduce_allreduce_amd as rs  # noqa: E402

CONFIGS = [
    ("wide ring 16x16 w1", 16, 16, dict(proto="wide", algo="ring", line_workgroups_per_channel=1), (1 << 20, 2 << 20)),
    ("wide ring 8x8 w4", 8, 8, dict(proto="wide", algo="ring", line_workgroups_per_channel=4), (1 << 20, 2 << 20)),
    ("tree 16x16", 16, 16, dict(proto="auto", algo="tree"), (64 << 10, 1 << 20)),
]


def main(budget: float) -> int:
    g = torch.Generator(device="cuda")
    g.manual_seed(20261202)
    t0 = time.time()
    last = t0
    tot_lines = {c[0]: 0 for c in CONFIGS}
    tot_calls = {c[0]: 0 for c in CONFIGS}
    comms = {}
    for name, n, nch, cfg, span in CONFIGS:
        c = dict(cfg)
        proto = c.pop("proto")
        comms[name] = rs.comm_init(n, nch, proto, **c)
    k = 0
    while time.time() - t0 < budget:
        name, n, nch, cfg, span = CONFIGS[k % 3]
        comm = comms[name]
        count = int(torch.randint(span[0] // 4, span[1] // 4 + 1, (1,), generator=g, device="cuda").item())
        pad = (count + 3) // 4 * 4  # rows start on 16-byte boundaries
        base = torch.randint(-(1 << 20), 1 << 20, (n, pad), generator=g, device="cuda", dtype=torch.int32)
        send = [base[r, :count] for r in range(n)]
        recv = torch.empty((n, pad), dtype=torch.int32, device="cuda")
        rs.allreduce(comm, send, [recv[r, :count] for r in range(n)])
        want = base[:, :count].sum(0, dtype=torch.int64).to(torch.int32)
        bad = (recv[:, :count] != want.unsqueeze(0))
        if bool(bad.any()):
            r, i = [int(x) for x in bad.nonzero()[0]]
            print(f"MISMATCH {name} call {tot_calls[name]} count {count} rank {r} index {i}: got {int(recv[r, i])} want {int(want[i])}", flush=True)
            return 1
        err = rs.get_async_error(comm)
        if err != rs.SUCCESS:
            print(f"ASYNC ERROR {name}: {rs.RESULT_NAMES.get(err, err)}", flush=True)
            return 1
        tot_calls[name] += 1
        per_line = 12
        if name.startswith("tree"):
            tot_lines[name] += 2 * n * count * 4 // per_line  # up and down the trees, every rank once each way
        else:
            tot_lines[name] += 2 * (n - 1) * count * 4 // per_line
        k += 1
        now = time.time()
        if now - last > 20:
            last = now
            print(f"[soak] {now - t0:6.0f} s " + "; ".join(f"{a}: {tot_calls[a]} calls, {tot_lines[a] / 1e9:.2f} G lines" for a in tot_calls), flush=True)
    for c in comms.values():
        rs.comm_destroy(c)
    print("[soak] done, no mismatch: " + "; ".join(f"{a}: {tot_calls[a]} calls, {tot_lines[a] / 1e9:.2f} G lines" for a in tot_calls), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main(float(sys.argv[1]) if len(sys.argv) > 1 else 480.0))
