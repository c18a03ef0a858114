"""The exchange floor of the persistent recurrences against their measured
step times, as a short text table for profiles/.

    python -m layer_lstm_amd.exchange_floor [--workloads A,B,...] [--out FILE]

For each workload: the forward recurrence's per-step exchange alone
(lstm_probe_exchange: flags, ring copy, ring stores, no arithmetic) in the
workload's own layout and with its batch groups spread over the XCDs, next
to the forward and backward recurrences' measured time per step (HIP
events around their launches, lstm_timing_*).  A recurrence step can not be
faster than the floor of its layout; what it spends above the floor is its
product, its gate math and its memory traffic.
"""
from __future__ import annotations

import argparse
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from layer_lstm_amd import synth  # noqa: E402

DEFAULT = ("f32_T64_B32_I256_H256", "bf16_T128_B64_I512_H1024", "bf16_T512_B16_I1024_H2048",
           "bf16_T256_B256_I1024_H1024")


def measure(name, reps=3, steps=5):
    import numpy as np
    import torch
    from layer_lstm_amd import lstm

    w = synth.WORKLOADS[name]
    code = {"f32": lstm.F32, "bf16": lstm.BF16, "f16": lstm.F16}[w.dtype]
    m = lstm.Lstm(w.T, w.B, w.I, w.H, code)
    plan = lstm.query_plan(m.shape)
    floor = [min(lstm.probe_exchange(m.shape, m.workspace, layout) for _ in range(reps)) for layout in (0, 1)]
    inp = synth.workload_inputs(name)
    td = lstm.torch_dtype(code)
    d = {k: None if inp[k] is None else torch.from_numpy(np.asarray(inp[k], dtype=np.float32)).cuda().to(td)
         for k in ("x", "W", "b", "h0", "c0", "dy", "dhT", "dcT")}

    def step():
        m.forward(d["x"], d["W"], d["b"], d["h0"], d["c0"])
        m.backward(d["dy"], d["dhT"], d["dcT"], d["x"], d["W"], d["h0"], d["c0"])

    step()
    m.check()
    lstm.timing_enable(True)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    kt = lstm.timing_read()
    lstm.timing_enable(False)
    m.check()
    per = {k: kt[k][0] / kt[k][1] * 1e3 / w.T for k in ("forward_recurrence", "backward_recurrence")}
    return plan, floor, per


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--workloads", default=",".join(DEFAULT))
    ap.add_argument("--out", default=None)
    args = ap.parse_args()
    lines = ["Exchange floor of the persistent recurrences (one MI355X)", "",
             "command: python -m layer_lstm_amd.exchange_floor " + " ".join(sys.argv[1:]), "",
             "us per step; floor = the forward's exchange alone (lstm_probe_exchange), in the",
             "workload's layout and spread over the XCDs; fwd / bwd = the recurrences' measured step", "",
             f"{'workload':30s} {'layout':22s} {'floor':>7s} {'spread':>7s} {'fwd':>7s} {'bwd':>7s}"]
    for name in args.workloads.split(","):
        plan, floor, per = measure(name)
        lay = f"{plan['groups']}x{plan['units_groups']} {'xcd-local' if plan['xcd_local'] else 'spread'}"
        lines.append(f"{name:30s} {lay:22s} {floor[0]:7.2f} {floor[1]:7.2f} "
                     f"{per['forward_recurrence']:7.2f} {per['backward_recurrence']:7.2f}")
        print(lines[-1], flush=True)
    text = "\n".join(lines) + "\n"
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    print(text)


if __name__ == "__main__":
    main()
