"""GPU parity of stacked layers (lstm_stack_*: the MXNet page's "Stack
Multiple RNN Cells", the CMU page's LSTM with num_layers) against the fp64
oracle's composition of one-layer passes, through the wavefront schedule
(chunks of time, the layers of a wave in one persistent launch where a
layout for cus / L exists, else one after the other) and with one chunk
(the layers strictly one after the other).  Every output whole (relative
L2) and row by row; output buffers NaN-poisoned first."""
import numpy as np
import pytest

from layer_lstm_amd import synth
from oracle import oracle
from parity_util import ROW_TOL, TOL, compare, compare_rows, rel_l2, to_dev, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

ALL = dict(W=("u", 0.3), b=("u", 0.3), x=("n", 1.0), h0=("n", 0.5), c0=("n", 0.5), dy=("n", 1.0),
           dhT=("n", 1.0), dcT=("n", 1.0))


@pytest.fixture(scope="module")
def lstm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from layer_lstm_amd import lstm as mod
    return mod


def stacked_inputs(L, T, B, I, H, dt, seed, dist=None, two_bias=False):
    """The layers' inputs; W, b ~ U(+-0.3) below H = 512, else the
    workloads' U(+-1/sqrt(H)) (at large H the wider range makes the
    recurrence chaotic: rounding grows over the steps on any side)."""
    if dist is None:
        k = 0.3 if H < 512 else 1.0 / np.sqrt(H)
        dist = dict(ALL, W=("u", k), b=("u", k))
    first = synth.make_inputs(T, B, I, H, dt, seed=seed, dist=dist)
    inp = dict(first, layers=L, W=[first["W"]], b=[first["b"]])
    for k in ("h0", "c0", "dhT", "dcT"):
        inp[k] = [first[k]]
    for ll in range(1, L):
        nxt = synth.make_inputs(T, B, H, H, dt, seed=seed + 100 * ll, dist=dist)
        inp["W"].append(nxt["W"])
        inp["b"].append(nxt["b"])
        for k in ("h0", "c0", "dhT", "dcT"):
            inp[k].append(nxt[k])
    inp["b"] = np.stack(inp["b"])
    if two_bias:
        rng = np.random.default_rng(seed + 7)
        inp["b"] = np.stack([inp["b"], synth.round_to_storage(rng.uniform(-0.3, 0.3, inp["b"].shape), dt)], axis=1)
        inp["two_bias"] = True
    for k in ("h0", "c0", "dhT", "dcT"):
        inp[k] = None if inp[k][0] is None else np.stack(inp[k])  # absent in the distribution: NULL
    return inp


def oracle_stacked(inp):
    """The oracle's stack on the layers' inputs: two biases enter as their
    sum (each half then receives db), and the "ijfo" order relabels the row
    blocks of every layer's W and b (and of dW, db back)."""
    sub = dict(inp, two_bias=False, gate_order="ifjo")
    if inp.get("two_bias"):
        sub["b"] = inp["b"][:, 0] + inp["b"][:, 1]
    order = inp.get("gate_order", "ifjo")
    rows = oracle.ifjo_rows(inp["H"], order) if order != "ifjo" else None
    if rows is not None:
        sub["W"] = [w[rows] for w in sub["W"]]
        sub["b"] = sub["b"][:, rows]
    ref = oracle.fwd_bwd(sub)
    if rows is not None:
        ref["dW"] = [w[rows] for w in ref["dW"]]
        ref["db"] = ref["db"][:, rows]
    if inp.get("two_bias"):
        ref["db"] = np.stack([ref["db"], ref["db"]], axis=1)
    ref["dW"] = np.concatenate([w.reshape(-1) for w in ref["dW"]])
    return ref


def run_stack(lstm, inp, chunks):
    T, B, I, H, dt, L = inp["T"], inp["B"], inp["I"], inp["H"], inp["dtype"], inp["layers"]
    code = {"f32": lstm.F32, "bf16": lstm.BF16, "f16": lstm.F16}[dt]
    m = lstm.Stack(T, B, I, H, L, code, chunks=chunks, gate_order=inp.get("gate_order", "ifjo"),
                   two_bias=bool(inp.get("two_bias")))
    for k in ("y", "hT", "cT", "dx", "dW", "db", "dh0", "dc0"):
        getattr(m, k).fill_(float("nan"))
    Wflat = np.concatenate([w.reshape(-1) for w in inp["W"]])
    d = {k: to_dev(inp.get(k), dt, torch) for k in ("x", "b", "h0", "c0", "dy", "dhT", "dcT")}
    d["W"] = to_dev(Wflat, dt, torch)
    m.forward(d["x"], d["W"], d["b"], d["h0"], d["c0"])
    m.backward(d["dy"], d["dhT"], d["dcT"], d["x"], d["W"], d["h0"], d["c0"])
    m.check()
    torch.cuda.synchronize()
    out = {k: to_host(getattr(m, k)) for k in ("y", "hT", "cT", "dx", "dW", "db", "dh0", "dc0")}
    return out, m


def check(inp, out, tol=None):
    dt = inp["dtype"]
    ref = oracle_stacked(inp)
    errs, bad = compare(out, ref, dt, tol=tol)
    worst, bad_rows = compare_rows({k: v for k, v in out.items() if k != "dW"}, ref, ROW_TOL[dt],
                                   keys=("y", "hT", "cT", "dx", "db", "dh0", "dc0"))
    print("rel-L2:", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    print("worst row:", {k: f"{v:.2e}" for k, v in worst.items()}, flush=True)
    assert not bad, bad
    assert not bad_rows, bad_rows


@pytest.mark.parametrize("dt,L,T,B,I,H,chunks", [
    ("f32", 2, 8, 4, 16, 32, 1),      # one chunk: the layers one after the other
    ("f32", 2, 8, 4, 16, 32, 3),      # chunks of 3, 3, 2 steps
    ("f32", 2, 300, 4, 16, 32, 0),    # default chunks: two of 150 steps
    ("f32", 3, 20, 32, 64, 256, 5),   # the VALU recurrences; waves of 1, 2, 3 layers
    ("bf16", 2, 12, 60, 32, 512, 4),  # MFMA recurrences, XCD-local
    ("bf16", 4, 9, 19, 40, 72, 5),    # four layers in one launch
    ("f16", 2, 10, 40, 64, 1024, 5),
    ("bf16", 3, 7, 5, 0, 48, 7),      # no input features, one step per chunk
])
def test_stacked_layers(lstm, dt, L, T, B, I, H, chunks):
    inp = stacked_inputs(L, T, B, I, H, dt, seed=141)
    code = {"f32": lstm.F32, "bf16": lstm.BF16, "f16": lstm.F16}[dt]
    nb, conc = lstm.stack_query(lstm.make_shape(T, B, I, H, code), L, chunks)
    print(f"case: stack {dt} L={L} T={T} B={B} I={I} H={H} chunks={chunks} concurrent={conc}", flush=True)
    out, _ = run_stack(lstm, inp, chunks)
    check(inp, out)


def test_stacked_flags(lstm):
    """The "ijfo" gate order and two biases through the stack."""
    inp = stacked_inputs(2, 6, 60, 32, 512, "bf16", seed=143, two_bias=True)
    inp["gate_order"] = "ijfo"
    print("case: stack, ijfo, two biases", flush=True)
    out, _ = run_stack(lstm, inp, 3)
    check(inp, out)


def test_wavefront_equals_layer_by_layer(lstm):
    """The wavefront schedule (chunks, concurrent layers) gives what one
    chunk (the layers strictly one after the other) gives, within the
    tolerance, and the stack's repeated backward gives the same bits."""
    inp = stacked_inputs(2, 16, 60, 32, 512, "bf16", seed=145)
    a, m = run_stack(lstm, inp, 4)
    b, _ = run_stack(lstm, inp, 1)
    for k in a:
        assert rel_l2(a[k], b[k]) <= TOL["bf16"], k
    Wflat = np.concatenate([w.reshape(-1) for w in inp["W"]])
    d = {k: to_dev(inp.get(k), "bf16", torch) for k in ("x", "h0", "c0", "dy", "dhT", "dcT")}
    m.backward(d["dy"], d["dhT"], d["dcT"], d["x"], to_dev(Wflat, "bf16", torch), d["h0"], d["c0"])
    m.check()
    torch.cuda.synchronize()
    for k in ("dx", "dW", "db", "dh0", "dc0"):
        assert np.array_equal(to_host(getattr(m, k)), a[k]), k


def test_stacked_workload_size(lstm):
    """Two layers at T=128 B=64 I=512 H=1024 (bf16) in four chunks, against
    the oracle on the whole batch."""
    w = synth.WORKLOADS["bf16_T128_B64_I512_H1024"]
    inp = stacked_inputs(2, w.T, w.B, w.I, w.H, "bf16", seed=0, dist=w.dist)
    nb, conc = lstm.stack_query(lstm.make_shape(w.T, w.B, w.I, w.H, lstm.BF16), 2, 4)
    print(f"case: stack of 2 at {w.name}, concurrent={conc}", flush=True)
    out, _ = run_stack(lstm, inp, 4)
    check(inp, out)
