"""Shared helpers of the GPU parity tests: move the seeded stored inputs to
the device, run the HIP path through the C-ABI binding, and compare with the
fp64 oracle by relative L2 norm per output tensor."""
import numpy as np

# Relative L2 bounds per storage type: fp32 1e-5 and bf16 (fp32 accumulation)
# 2e-2 as stated for the method; fp16 takes bf16's bound scaled by the ratio
# of the two unit roundoffs (2^-11 / 2^-8), since the error comes from
# rounding the stored operands (inputs, gates, gate deltas, h) to the
# storage type.
TOL = {"f32": 1e-5, "bf16": 2e-2, "f16": 2.5e-3}
OUTPUTS = ("y", "hT", "cT", "dx", "dW", "db", "dh0", "dc0")
# Bound of the per-row check (row_errors), five times the whole-tensor
# tolerance: a row is a small sample (a db value sums T*B terms, a dW row
# H+I columns), so its rounding error spreads wider than the whole tensor's
# (bf16 rows reach 2-4e-2 where the tensors sit at 5e-3), while a corrupted,
# stale or unwritten row is off by about its own size (a ratio near 1).
ROW_TOL = {"f32": 5e-5, "bf16": 1e-1, "f16": 1.25e-2}


def rel_l2(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((got - ref).ravel())
    return num / den if den > 0 else num


def to_dev(a, dtype, torch):
    if a is None:
        return None
    td = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dtype]
    # stored values are exactly representable in the storage type
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda").to(td)


def to_host(t):
    return t.float().cpu().numpy().astype(np.float64)


def run_gpu(inp, lstm, torch, want_db=True, stream=None, poison=False):
    """Forward + backward on the GPU; returns fp64 host copies of the 8
    outputs.  poison: fill every output buffer with NaN first, so that an
    output the library fails to write shows up."""
    T, B, I, H, dt = inp["T"], inp["B"], inp["I"], inp["H"], inp["dtype"]
    code = {"f32": lstm.F32, "bf16": lstm.BF16, "f16": lstm.F16}[dt]
    m = lstm.Lstm(T, B, I, H, code, reverse=bool(inp.get("reverse", False)),
                  gate_order=inp.get("gate_order", "ifjo"), two_bias=bool(inp.get("two_bias", False)),
                  bidirectional=bool(inp.get("bidirectional", False)))
    if poison:
        for k in OUTPUTS:
            getattr(m, k).fill_(float("nan"))
    d = {k: to_dev(inp.get(k), dt, torch) for k in ("x", "W", "b", "h0", "c0", "dy", "dhT", "dcT")}
    lens = inp.get("lengths")
    d["len"] = None if lens is None else torch.tensor(np.asarray(lens), dtype=torch.int32, device="cuda")
    m.forward(d["x"], d["W"], d["b"], d["h0"], d["c0"], stream=stream, seq_length=d["len"])
    m.backward(d["dy"], d["dhT"], d["dcT"], d["x"], d["W"], d["h0"], d["c0"], want_db=want_db, stream=stream,
               seq_length=d["len"])
    m.check(stream)
    torch.cuda.synchronize()
    out = dict(y=to_host(m.y), hT=to_host(m.hT), cT=to_host(m.cT), dx=to_host(m.dx), dW=to_host(m.dW),
               db=to_host(m.db), dh0=to_host(m.dh0), dc0=to_host(m.dc0))
    return out, m, d


def compare(out, ref, dtype, keys=OUTPUTS, tol=None):
    tol = TOL[dtype] if tol is None else tol
    errs = {k: rel_l2(out[k], ref[k]) for k in keys}
    bad = {k: v for k, v in errs.items() if not (v <= tol)}
    return errs, bad


def row_errors(got, ref, row_dims):
    """Per-row relative error: rows are the slices over the trailing
    dimensions after the first `row_dims` (a (t, b) row of y or dx, a batch
    row of hT, a gate row of dW; row_dims = 0: one value per row).  Each
    row's L2 error is divided by the larger of its own L2 norm and the RMS
    row norm of the reference, so that a row whose reference is small is
    not held to a relative bound it cannot meet, while a corrupted or stale
    row (an error as large as a typical row) stands out.  Returns the array
    of ratios."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if row_dims == 0:
        got, ref = got.reshape(-1, 1), ref.reshape(-1, 1)
    else:
        n = int(np.prod(ref.shape[:row_dims]))
        got, ref = got.reshape(n, -1), ref.reshape(n, -1)
    err = np.linalg.norm(got - ref, axis=1)
    nrm = np.linalg.norm(ref, axis=1)
    rms = np.sqrt(np.mean(nrm * nrm)) if nrm.size else 0.0
    den = np.maximum(nrm, rms)
    return np.where(den > 0, err / np.where(den > 0, den, 1.0), err)


def compare_rows(out, ref, tol, keys=OUTPUTS):
    """Worst per-row error of each output (row_errors) and the outputs over
    `tol`.  Rows: (t, b) rows of y and dx, batch rows of the [B, H] states,
    gate rows of dW (per direction where there are two), single values of
    db."""
    worst = {}
    for k in keys:
        rd = 0 if k == "db" else np.ndim(ref[k]) - 1
        r = row_errors(out[k], ref[k], rd)
        worst[k] = float(r.max()) if r.size else 0.0
    bad = {k: v for k, v in worst.items() if not (v <= tol)}
    return worst, bad
