"""Step-phase breakdown of the persistent recurrences of one workload.

    python -m layer_lstm_amd.phases WORKLOAD [--out FILE]

Runs one forward + backward of the workload (seeded synthetic inputs, on
cuda:0) with the library's step stamps on (lstm_stamps_set: thread 0 of
work-groups 0..7 records the 100 MHz s_memrealtime clock at six points of
every step) and prints, per pass, the median duration of a step and of each
phase, and the share of the step spent waiting for other work-groups (the
exchange wait -- the per-step barrier of the method) against the share spent
computing.  Needs a GPU.
"""
from __future__ import annotations

import argparse
import sys

import numpy as np

FWD_PHASES = ("exchange wait (h flags)", "h load (tagged: +P, record)", "product",
              "P, record + k-part reduction", "gate math + publish")
# backward: the MFMA kernel (column partition, bf16 and most fp32 shapes) and
# the VALU kernel (fp32 batch groups of 4 rows, the fp32 workloads here)
BWD_PHASES_MFMA = ("exchange wait (dG flags)", "dG loads + product", "wave reduction", "gate deltas + publish",
                   "operand prefetch issue")
BWD_PHASES_VALU = ("exchange wait + dh gather", "gate deltas + barrier", "partial product + publish",
                   "operand prefetch issue", "barrier")


def measure(name: str):
    import torch
    from layer_lstm_amd import lstm, synth

    w = synth.WORKLOADS[name]
    inp = synth.workload_inputs(name)
    td = torch.float32 if w.dtype == "f32" else torch.bfloat16
    d = {k: (None if inp[k] is None else torch.from_numpy(np.asarray(inp[k], np.float32)).cuda().to(td))
         for k in ("x", "W", "b", "h0", "c0", "dy", "dhT", "dcT")}
    m = lstm.Lstm(w.T, w.B, w.I, w.H, lstm.F32 if w.dtype == "f32" else lstm.BF16)
    npt = lstm.STAMP_POINTS
    buf = torch.zeros(2 * lstm.STAMP_WGS * w.T * npt, dtype=torch.int64, device="cuda")
    for it in range(3):  # two warm-up passes, then one stamped
        lstm.stamps_set(buf if it == 2 else None, w.T)
        m.forward(d["x"], d["W"], d["b"], d["h0"], d["c0"])
        m.backward(d["dy"], d["dhT"], d["dcT"], d["x"], d["W"], d["h0"], d["c0"])
        m.check()
        torch.cuda.synchronize()
    lstm.stamps_set(None, 0)
    return w, buf.cpu().numpy().reshape(2, lstm.STAMP_WGS, w.T, npt).astype(np.float64) * 0.01  # us


def summarize(name, w, s):
    lines = [f"workload {name} (T={w.T} B={w.B} I={w.I} H={w.H} {w.dtype}); microseconds, medians over "
             f"steps 1..T-1 of the stamped work-groups"]
    bwd = BWD_PHASES_VALU if w.dtype == "f32" else BWD_PHASES_MFMA
    for p, (pname, names) in enumerate((("forward", FWD_PHASES), ("backward", bwd))):
        a = s[p]
        valid = [g for g in range(a.shape[0]) if a[g, 0, 0] > 0]
        a = a[valid]
        steps = np.diff(a[:, :, 0], axis=1)
        ph = np.diff(a, axis=2)[:, 1:, :]
        step = float(np.median(steps))
        lines.append(f"{pname}: step {step:.2f} us (work-groups {valid})")
        for i, n in enumerate(names):
            v = float(np.median(ph[:, :, i]))
            lines.append(f"   {n:28s} {v:7.2f} us  {100 * v / step:5.1f} %")
        wait = float(np.median(ph[:, :, 0]))
        lines.append(f"   waiting on other work-groups (first phase): {100 * wait / step:.1f} % of the step")
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("workload")
    ap.add_argument("--out")
    a = ap.parse_args()
    w, s = measure(a.workload)
    text = summarize(a.workload, w, s)
    print(text, flush=True)
    if a.out:
        with open(a.out, "w") as f:
            f.write(f"# step phases of the recurrent kernels\n\ncommand:\n\n    python -m layer_lstm_amd.phases "
                    f"{a.workload} --out {a.out}\n\n{text}\n")


if __name__ == "__main__":
    sys.exit(main())
