"""Shared helpers of the GPU parity tests: move the seeded stored inputs to
the device, run the HIP path through the C-ABI binding, and compare with the
fp64 oracle by relative L2 norm per output tensor."""
import numpy as np

TOL = {"f32": 1e-5, "bf16": 2e-2}
OUTPUTS = ("y", "hT", "cT", "dx", "dW", "db", "dh0", "dc0")


def rel_l2(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((got - ref).ravel())
    return num / den if den > 0 else num


def to_dev(a, dtype, torch):
    if a is None:
        return None
    td = torch.float32 if dtype == "f32" else torch.bfloat16
    # stored values are exactly representable in the storage type
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda").to(td)


def to_host(t):
    return t.float().cpu().numpy().astype(np.float64)


def run_gpu(inp, lstm, torch, want_db=True, stream=None):
    """Forward + backward on the GPU; returns fp64 host copies of the 8 outputs."""
    T, B, I, H, dt = inp["T"], inp["B"], inp["I"], inp["H"], inp["dtype"]
    code = lstm.F32 if dt == "f32" else lstm.BF16
    m = lstm.Lstm(T, B, I, H, code, reverse=bool(inp.get("reverse", False)),
                  gate_order=inp.get("gate_order", "ifjo"), two_bias=bool(inp.get("two_bias", False)))
    d = {k: to_dev(inp.get(k), dt, torch) for k in ("x", "W", "b", "h0", "c0", "dy", "dhT", "dcT")}
    m.forward(d["x"], d["W"], d["b"], d["h0"], d["c0"], stream=stream)
    m.backward(d["dy"], d["dhT"], d["dcT"], d["x"], d["W"], d["h0"], d["c0"], want_db=want_db, stream=stream)
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
