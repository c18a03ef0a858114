"""The three products of a step against the vendor library on the same
shapes, as a short text table for profiles/.

    python -m layer_lstm_amd.blas_reference [--workloads A,B,...] [--out FILE]

For each bf16 workload: the launch time of this library's input
projection, dW and dx (HIP events around their launches, lstm_timing_*),
next to torch.matmul (hipBLASLt on ROCm) on operands of the same shapes and
storage type -- x[TB,I] @ W_x^T, dG[TB,4H] @ W_x, dG^T[4H,TB] @ Z[TB,H+I] --
each with its fraction of the bf16 matrix-core peak.  The library products
differ from the plain ones in their epilogues (the input projection writes
fp32 P with the bias added, twice the output bytes of a bf16 result; dW
writes its rows back in gate-block order), so the table is a reference
point for the attainable rate on these shapes, not a like-for-like race.
"""
from __future__ import annotations

import argparse
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from layer_lstm_amd import synth  # noqa: E402

PEAK_BF16 = 2516.6  # dense bf16 MFMA TFLOP/s of one MI355X
DEFAULT = ("bf16_T128_B64_I512_H1024", "bf16_T512_B16_I1024_H2048", "bf16_T256_B256_I1024_H1024")


def _time(fn, reps):
    import torch
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps * 1e3  # us


def measure(name, reps=20):
    import numpy as np
    import torch
    from layer_lstm_amd import lstm

    w = synth.WORKLOADS[name]
    assert w.dtype == "bf16", name
    TB, H, I = w.T * w.B, w.H, w.I
    flops = {"input_projection": 2.0 * TB * 4 * H * I, "dx_product": 2.0 * TB * 4 * H * I,
             "dW_product": 2.0 * TB * 4 * H * (H + I)}

    # this library: one step for the record, then `reps` timed steps
    m = lstm.Lstm(w.T, w.B, w.I, w.H, lstm.BF16)
    inp = synth.workload_inputs(name)
    d = {k: None if inp[k] is None else torch.from_numpy(np.asarray(inp[k], dtype=np.float32)).cuda().to(
        torch.bfloat16) for k in ("x", "W", "b", "h0", "c0", "dy", "dhT", "dcT")}

    def step():
        m.forward(d["x"], d["W"], d["b"], d["h0"], d["c0"])
        m.backward(d["dy"], d["dhT"], d["dcT"], d["x"], d["W"], d["h0"], d["c0"])

    step()
    torch.cuda.synchronize()
    m.check()
    lstm.timing_enable(True)
    for _ in range(reps):
        step()
    torch.cuda.synchronize()
    kt = lstm.timing_read()
    lstm.timing_enable(False)
    m.check()
    ours = {k: kt[k][0] / kt[k][1] * 1e3 for k in flops}

    # the library GEMM on operands of the same shapes (contiguous, bf16 out)
    g = torch.Generator(device="cuda").manual_seed(0)
    x = torch.randn(TB, I, device="cuda", dtype=torch.bfloat16, generator=g)
    WxT = torch.randn(I, 4 * H, device="cuda", dtype=torch.bfloat16, generator=g)
    Wx = WxT.t().contiguous()
    dG = torch.randn(TB, 4 * H, device="cuda", dtype=torch.bfloat16, generator=g)
    dGT = dG.t().contiguous()
    Z = torch.randn(TB, H + I, device="cuda", dtype=torch.bfloat16, generator=g)
    blas = {"input_projection": _time(lambda: torch.matmul(x, WxT), reps),
            "dx_product": _time(lambda: torch.matmul(dG, Wx), reps),
            "dW_product": _time(lambda: torch.matmul(dGT, Z), reps)}
    return {k: (ours[k], blas[k], flops[k]) for k in flops}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--workloads", default=",".join(DEFAULT))
    ap.add_argument("--reps", type=int, default=20)
    ap.add_argument("--out", default=None)
    args = ap.parse_args(argv)
    out_rel = os.path.relpath(os.path.abspath(args.out), ROOT) if args.out else None
    cmd = "python -m layer_lstm_amd.blas_reference" + (f" --out {out_rel}" if out_rel else "")
    lines = ["The step's products against torch.matmul (hipBLASLt) on the same shapes, one MI355X", "",
             f"command: {cmd}", "",
             "us per launch (HIP events, mean of the timed launches); fraction of the 2.5166 PFLOP/s bf16 peak.",
             "library: input projection x[TB,I] W_x^T with bias into fp32 P; dx dG[TB,4H] W_x into bf16; dW",
             "dG^T[4H,TB] Z[TB,H+I] into bf16 (gate-block rows).  torch.matmul: the same products into bf16.", "",
             f"{'workload':28s} {'product':18s} {'this library':>18s} {'torch.matmul':>18s}"]
    for name in args.workloads.split(","):
        res = measure(name, args.reps)
        for k, (us_o, us_b, fl) in res.items():
            fo, fb = fl / us_o / 1e6 / PEAK_BF16, fl / us_b / 1e6 / PEAK_BF16
            lines.append(f"{name:28s} {k:18s} {us_o:9.1f} us {fo:5.1%} {us_b:9.1f} us {fb:5.1%}")
        print(lines[-3], lines[-2], lines[-1], sep="\n", flush=True)
    text = "\n".join(lines) + "\n"
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    print(text, flush=True)


if __name__ == "__main__":
    main()
