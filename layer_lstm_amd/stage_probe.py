"""The parts of a pipelined bf16 product stage against the matrix cores'
peak, as a short text table for profiles/.

    python -m layer_lstm_amd.stage_probe [--iters N] [--reps R] [--out FILE]

Runs lstm_probe_mfma_stage (include/lstm.h) for each combination of a
stage's parts -- fragment reads from LDS (before the products, or for the
next iteration ahead of them), the work-group barrier, the direct-to-LDS
loads -- around 32 bf16 MFMAs per wave and iteration, 8 waves per compute
unit as the products run, and prints the best of --reps runs as a fraction
of the dense bf16 peak.  The last rows are the products' own measured
fractions (HIP events, lstm_timing_*) on the largest workload, for
comparison.  Needs a GPU.
"""
from __future__ import annotations

import argparse
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

ROWS = (
    ("MFMAs alone", 0),
    ("+ fragment reads before the products", 1),
    ("+ fragment reads for the next iteration", 2),
    ("+ barrier", 4),
    ("+ direct-to-LDS loads (L2-resident buffer)", 8),
    ("+ reads before + barrier", 1 | 4),
    ("+ reads ahead + barrier", 2 | 4),
    ("+ reads before + loads", 1 | 8),
    ("+ barrier + loads", 4 | 8),
    ("+ reads before + barrier + loads (the products' stage)", 1 | 4 | 8),
    ("+ reads ahead + barrier + loads", 2 | 4 | 8),
)


def product_fractions(name="bf16_T256_B256_I1024_H1024", steps=5):
    """Fraction of the bf16 peak of the three products on a workload, from
    the library's HIP-event timings (split-K sums included)."""
    import numpy as np
    import torch
    from layer_lstm_amd import lstm, synth

    w = synth.WORKLOADS[name]
    inp = synth.workload_inputs(name)
    d = {k: (None if inp[k] is None else torch.from_numpy(np.asarray(inp[k], np.float32)).cuda().to(torch.bfloat16))
         for k in ("x", "W", "b", "h0", "c0", "dy", "dhT", "dcT")}
    m = lstm.Lstm(w.T, w.B, w.I, w.H, lstm.BF16)
    for _ in range(2):
        m.forward(d["x"], d["W"], d["b"], d["h0"], d["c0"])
        m.backward(d["dy"], d["dhT"], d["dcT"], d["x"], d["W"], d["h0"], d["c0"])
    torch.cuda.synchronize()
    lstm.timing_enable(True)
    for _ in range(steps):
        m.forward(d["x"], d["W"], d["b"], d["h0"], d["c0"])
        m.backward(d["dy"], d["dhT"], d["dcT"], d["x"], d["W"], d["h0"], d["c0"])
    torch.cuda.synchronize()
    t = lstm.timing_read()
    lstm.timing_enable(False)
    TB, H, I = w.T * w.B, w.H, w.I
    flops = {"input_projection": 8.0 * TB * H * I, "dW_product": 8.0 * TB * H * (H + I), "dx_product": 8.0 * TB * H * I}
    out = {}
    for k, f in flops.items():
        ms, n = t[k]
        if n:
            out[k] = f / (ms * 1e-3 / n) / 2516.6e12
    return name, out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--iters", type=int, default=4000)
    ap.add_argument("--reps", type=int, default=3)
    ap.add_argument("--out", default=None)
    a = ap.parse_args()
    import torch
    from layer_lstm_amd import lstm

    torch.cuda.set_device(0)
    scratch = torch.empty(lstm.PROBE_SCRATCH_BYTES, dtype=torch.uint8, device="cuda")
    lines = ["# the parts of a pipelined bf16 product stage against the MFMA peak", "", "command:", "",
             "    python -m layer_lstm_amd.stage_probe" + (f" --out {a.out}" if a.out else ""), "",
             f"lstm_probe_mfma_stage: one work-group of 8 waves per compute unit, {a.iters} iterations of 32",
             "v_mfma_f32_16x16x32_bf16 per wave (operands in registers) plus the parts named; best of "
             f"{a.reps} runs;", "fraction of the dense bf16 peak (2516.6 TFLOP/s for 256 compute units)", ""]
    for label, parts in ROWS:
        best = max(lstm.probe_mfma_stage(parts, scratch, a.iters) for _ in range(a.reps))
        lines.append(f"{label:58s} {best:6.3f}")
        print(lines[-1], flush=True)
    name, fr = product_fractions()
    lines += ["", f"the products themselves on {name} (lstm_timing_*, split-K sums included):"]
    for k, v in fr.items():
        lines.append(f"{k:58s} {v:6.3f}")
    text = "\n".join(lines) + "\n"
    if a.out:
        with open(a.out, "w") as f:
            f.write(text)
    print(text, end="")


if __name__ == "__main__":
    main()
