#!/usr/bin/env python3
"""Benchmark of the single-layer LSTM forward + BPTT on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--reverse]
                    [--gate-order ifjo|ijfo] [--two-bias] [--bidirectional] [--lengths none|ragged]

The default workload is the largest one that fits one GPU,
bf16_T256_B256_I1024_H1024 (T=256, B=256, I=1024, H=1024, bf16 storage with
fp32 accumulation); --workload picks another of layer_lstm_amd/synth.py.
One step = lstm_fwd_train + lstm_bwd on one batch of seeded synthetic input
(every kernel of the path: input projection, forward recurrence, backward
recurrence, dW, dx, db).  Inputs, weights and outputs are resident in HBM
before the timed region starts.  Prints one JSON line with the metric
(sequences/s; effective TFLOP/s = 24*T*B*H*(H+I) per step / time, and its
fraction of the MFMA peak of the storage type), a roofline record of the
kernel that takes the most time, and the fp64 CPU oracle timed on the host
on a bounded sample of the same workload.  --reverse runs the reverse
direction of time (lstm_shape.flags = LSTM_REVERSE), --gate-order ijfo the
other gate order of W's row blocks (LSTM_GATES_IJFO), --two-bias two bias
vectors (LSTM_TWO_BIAS; the second one the first reversed), --bidirectional
both directions of time (LSTM_BIDIRECTIONAL; effective FLOPs counted for both),
--lengths ragged seeded sequence lengths (seq_length; the FLOPs counted are
those of the full T steps, which the products still run), on the same
workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from layer_lstm_amd import synth  # noqa: E402

METRIC = "LSTM fwd+bwd sequences/s and effective TFLOP/s (fraction of MFMA peak)"
PEAK_TFLOPS = {"f32": 157.3, "bf16": 2516.6, "f16": 2516.6}  # MI355X dense matrix peaks
VALU_TFLOPS = 157.3  # MI355X fp32 vector peak (256 CUs x 2.4 GHz)
HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def step_work(w, kind, layers=1, directions=1):
    """Algorithmic FLOPs of one step's launches of `kind` (all of them:
    every layer of a stack, both directions of a bidirectional layer)."""
    T, B, I, H = w.T, w.B, w.I, w.H
    TB = T * B
    ins = I + (layers - 1) * H  # the layers' input sizes, summed
    if kind in ("input_projection", "dx_product"):
        return directions * 2.0 * TB * 4 * H * ins
    if kind in ("forward_recurrence", "backward_recurrence"):
        return directions * layers * 2.0 * TB * 4 * H * H
    if kind == "dW_product":
        return directions * 2.0 * TB * 4 * H * (layers * H + ins)
    return 0.0


def kernel_work(w, kind, plan=None, launches_per_step=1.0, layers=1, directions=1):
    """Algorithmic work of one launch of `kind`: (amount, unit, bound) --
    the step's work over its launches.  A recurrence whose product runs on
    the vector ALUs (plan from lstm_query_plan) is bound by "alu"
    arithmetic, else by the matrix cores."""
    work = step_work(w, kind, layers, directions) / max(launches_per_step, 1e-9)
    if kind in ("forward_recurrence", "backward_recurrence"):
        key = "fwd_valu" if kind == "forward_recurrence" else "bwd_valu"
        return work, "flop", "alu" if plan and plan[key] else "mfma"
    if kind in ("input_projection", "dW_product", "dx_product"):
        return work, "flop", "mfma"
    return 0.0, "byte", "hbm"


def traffic_for(workload, kind):
    """HBM bytes per launch from the committed rocprofv3 counter runs, or
    None when there are none for this kernel or its source has changed."""
    from layer_lstm_amd import profile_summary
    try:
        rec = json.load(open(TRAFFIC_FILE))[workload][kind]
    except (OSError, KeyError, ValueError):
        return None
    if kind not in profile_summary.KINDS or rec.get("source_sha") != profile_summary.source_sha(
            profile_summary.KINDS[kind][0]):
        return None
    return rec.get("bytes_per_launch")


def copy_calibration(mib):
    """A plain device copy of `mib` MiB (three times), for scaling the
    rocprofv3 FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.arange(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    assert torch.equal(dst[-4:], src[-4:])
    print(json.dumps({"copy_bytes": n * 4, "launches": 3}), flush=True)


def cpu_model():
    """Model name of the host CPU (/proc/cpuinfo), or None."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, inp, budget_s, reverse=False, gate_order="ifjo", two_bias=False, bidirectional=False):
    """Time the fp64 oracle (as it stands) on a bounded sample of the same
    workload: whole sequences (batch rows), as many as fit in about
    `budget_s` seconds by a one-row probe; when the whole batch takes less,
    the full fwd+bwd is repeated until about `budget_s` seconds have run."""
    from oracle import oracle

    def rows(n):
        sub = dict(inp, B=n, reverse=reverse, gate_order=gate_order, two_bias=two_bias, bidirectional=bidirectional)
        for k in ("x", "dy"):
            sub[k] = inp[k][:, :n]
        for k in ("h0", "c0", "dhT", "dcT"):
            sub[k] = None if inp[k] is None else (inp[k][:, :n] if bidirectional else inp[k][:n])
        if inp.get("lengths") is not None:
            sub["lengths"] = inp["lengths"][:n]
        return sub

    t0 = time.perf_counter()
    oracle.fwd_bwd(rows(1))
    t1 = time.perf_counter() - t0
    n = int(max(1, min(w.B, budget_s / max(t1, 1e-6))))
    sub = rows(n)
    passes, dt = 0, 0.0
    t0 = time.perf_counter()
    while passes == 0 or (n == w.B and dt < budget_s):
        oracle.fwd_bwd(sub)
        passes += 1
        dt = time.perf_counter() - t0
    return {"value": passes * n / dt, "unit": "sequences/s", "cores": oracle.num_threads(), "kind": "oracle",
            "cpu_model": cpu_model(), "logical_cpus": os.cpu_count(),
            "gflops": round(passes * n * w.flops / w.B / dt / 1e9, 3),
            "sample": f"{passes} x {n} of {w.B} sequences (batch rows) of {w.name}, fwd+bwd in fp64, "
                      f"{dt:.2f} s wall"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=synth.HEADLINE, choices=sorted(synth.WORKLOADS))
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--reverse", action="store_true", help="the reverse direction of time")
    ap.add_argument("--gate-order", default="ifjo", choices=("ifjo", "ijfo"), help="row-block order of W, b, dW, db")
    ap.add_argument("--two-bias", action="store_true", help="two bias vectors (b_ih, b_hh)")
    ap.add_argument("--bidirectional", action="store_true",
                    help="both directions of time (the second direction's tensors seeded with seed 1)")
    ap.add_argument("--layers", type=int, default=1,
                    help="a stack of this many layers (lstm_stack_*: the wavefront schedule), layers >= 1 of input "
                         "size H seeded with seeds 1, 2, ...")
    ap.add_argument("--chunks", type=int, default=0, help="chunks of time of the stack's wavefront (0: default; "
                                                          "1: the layers one after the other)")
    ap.add_argument("--lengths", default="none", choices=("none", "ragged"),
                    help="sequence lengths: none, or ragged (seeded, uniform over 1..T)")
    ap.add_argument("--copy-calibration", type=int, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (for scaling rocprofv3 byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: there is no multi-GPU path (sequences are "
              "independent, so several GPUs would each take a share of the batch with "
              "one all-reduce of dW and db); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    import numpy as np
    import torch
    from layer_lstm_amd import lstm

    w = synth.WORKLOADS[args.workload]
    inp = synth.workload_inputs(w.name)
    if args.bidirectional:
        other = synth.workload_inputs(w.name, seed=1)
        inp["dy"] = np.concatenate([inp["dy"], other["dy"]], axis=2)
        for k in ("W", "b", "h0", "c0", "dhT", "dcT"):
            inp[k] = None if inp[k] is None else np.stack([inp[k], other[k]])
    if args.two_bias:
        inp["b"] = np.stack([inp["b"], inp["b"][..., ::-1].copy()], axis=-2)
    if args.lengths == "ragged":
        inp["lengths"] = np.random.default_rng([0, 8]).integers(1, w.T + 1, size=w.B).astype(np.int32)
    code = {"f32": lstm.F32, "bf16": lstm.BF16, "f16": lstm.F16}[w.dtype]
    td = lstm.torch_dtype(code)
    dev = torch.device("cuda:0")

    def put(a):
        return None if a is None else torch.from_numpy(np.asarray(a, dtype=np.float32)).to(dev).to(td)

    d = {k: put(inp[k]) for k in ("x", "W", "b", "h0", "c0", "dy", "dhT", "dcT")}
    lens = None if inp.get("lengths") is None else torch.from_numpy(inp["lengths"]).to(dev)
    if args.layers > 1:
        # a stack: layer 0 on the workload's inputs, layers l >= 1 (input size
        # H) on inputs seeded with seed l; W back to back, b and the states
        # with a leading layer axis
        Ws, bs, st = [inp["W"]], [inp["b"]], {k: [inp[k]] for k in ("h0", "c0", "dhT", "dcT")}
        for ll in range(1, args.layers):
            o = synth.make_inputs(w.T, w.B, w.H, w.H, w.dtype, seed=ll, dist=w.dist)
            Ws.append(o["W"])
            bs.append(o["b"])
            for k in st:
                st[k].append(o[k])
        d["W"] = put(np.concatenate([a.reshape(-1) for a in Ws]))
        d["b"] = put(np.stack(bs))
        for k in st:
            d[k] = None if st[k][0] is None else put(np.stack(st[k]))
        m = lstm.Stack(w.T, w.B, w.I, w.H, args.layers, code, chunks=args.chunks, gate_order=args.gate_order,
                       two_bias=args.two_bias)

        def step():
            m.forward(d["x"], d["W"], d["b"], d["h0"], d["c0"])
            m.backward(d["dy"], d["dhT"], d["dcT"], d["x"], d["W"], d["h0"], d["c0"])
    else:
        m = lstm.Lstm(w.T, w.B, w.I, w.H, code, reverse=args.reverse, gate_order=args.gate_order,
                      two_bias=args.two_bias, bidirectional=args.bidirectional)

        def step():
            m.forward(d["x"], d["W"], d["b"], d["h0"], d["c0"], seq_length=lens)
            m.backward(d["dy"], d["dhT"], d["dcT"], d["x"], d["W"], d["h0"], d["c0"], seq_length=lens)

    log(f"workload {w.name}{' (reverse)' if args.reverse else ''}: warmup {args.warmup}, steps {args.steps}")
    for _ in range(args.warmup):
        step()
    m.check()
    torch.cuda.synchronize()

    # timed region: events on the stream every kernel is launched on
    stream = torch.cuda.current_stream()
    lstm.timing_enable(False)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    m.check()

    # per-kernel HIP-event timing over a second pass of the same steps
    lstm.timing_enable(True)
    torch.cuda.synchronize()
    e2, e3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e2.record(stream)
    for _ in range(args.steps):
        step()
    e3.record(stream)
    torch.cuda.synchronize()
    ms_timed = e2.elapsed_time(e3) / args.steps
    kt = lstm.timing_read()
    lstm.timing_enable(False)
    log(f"step {ms * 1e3:.1f} us (with per-kernel events {ms_timed * 1e3:.1f} us)")
    for k, (tot, n) in kt.items():
        if n:
            log(f"  {k:22s} {tot / n * 1e3:10.1f} us/launch  x{n // args.steps}/step")

    kinds = [k for k in kt if kt[k][1] > 0 and k != "state_copy"]
    dom = max(kinds, key=lambda k: kt[k][0])
    tot, n = kt[dom]
    avg_s = tot / n / 1e3
    plan = lstm.query_plan(lstm.make_shape(w.T, w.B, w.I, w.H, code, bidirectional=args.bidirectional))
    nd = 2 if args.bidirectional else 1
    work, unit, bound = kernel_work(w, dom, plan, n / args.steps, args.layers, nd)
    if unit == "flop":
        achieved = work / avg_s / 1e12
        peak, runit = (VALU_TFLOPS if bound == "alu" else PEAK_TFLOPS[w.dtype]), "TFLOP/s"
    else:
        achieved = work / avg_s / 1e9
        peak, runit = HBM_GBS, "GB/s"
    roofline = {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": runit,
                "frac": round(achieved / peak, 5),
                # (the counter runs are of the forward direction, default gate order, one bias)
                "traffic": None if (args.reverse or args.gate_order != "ifjo" or args.two_bias or
                                    args.bidirectional or args.lengths != "none" or args.layers > 1)
                else traffic_for(w.name, dom),
                "kernel": dom, "avg_launch_us": round(avg_s * 1e6, 2)}

    # each batched product against the MFMA peak of the storage type: its
    # algorithmic FLOPs per launch over its average launch time (the dW
    # launch includes its split-K sum and the db sum)
    gemm_frac = {}
    for kind in ("input_projection", "dW_product", "dx_product"):
        tot_k, n_k = kt.get(kind, (0.0, 0))
        if n_k:
            fl = kernel_work(w, kind, plan, n_k / args.steps, args.layers, nd)[0]
            gemm_frac[kind] = {"us": round(tot_k / n_k * 1e3, 2),
                               "frac": round(fl / (tot_k / n_k / 1e3) / 1e12 / PEAK_TFLOPS[w.dtype], 4)}
    rec_us = {k: round(kt[k][0] / kt[k][1] * 1e3, 2) for k in ("forward_recurrence", "backward_recurrence")
              if kt.get(k, (0, 0))[1]}

    flops = w.flops * (2 if args.bidirectional else 1)
    if args.layers > 1:  # layers >= 1 take input size H
        flops += (args.layers - 1) * 24.0 * w.T * w.B * w.H * 2 * w.H
    value = w.B / (ms / 1e3)
    eff_tflops = flops / (ms / 1e3) / 1e12
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "sequences/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded; see layer_lstm_amd/synth.py)",
        "config": {"workload": w.name, "T": w.T, "B": w.B, "I": w.I, "H": w.H, "storage": w.dtype,
                   "direction": "reverse" if args.reverse else "forward", "gate_order": args.gate_order,
                   "biases": 2 if args.two_bias else 1,
                   "bidirectional": args.bidirectional, "lengths": args.lengths,
                   "layers": args.layers, "chunks": args.chunks,
                   "parallelism": "single GPU"},
        "effective_tflops": round(eff_tflops, 3),
        "fraction_of_peak": round(eff_tflops / PEAK_TFLOPS[w.dtype], 5),
        "roofline": roofline,
        "gemm_fraction_of_peak": gemm_frac,
        "recurrence_us": rec_us,
        "recurrence_plan": plan,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline and args.layers == 1:
        log("timing the CPU oracle ...")
        out["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_budget, args.reverse, args.gate_order, args.two_bias,
                                           args.bidirectional)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
