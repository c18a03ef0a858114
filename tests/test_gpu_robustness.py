"""Failure paths of the persistent recurrences, forced from the host
(lstm_debug_inject) so that every kernel still exits normally:

 * a time-out recorded at a chosen step (as if a per-step wait had run past
   its bound) is reported by lstm_check_workspace as LSTM_ERR_TIMEOUT, is
   sticky until it is reported, and the next call on the same workspace is
   correct again;
 * a work-group that takes the role of another XCD's (as on a device that
   dealt work-groups to its XCDs otherwise than the XCD-local layout
   assumes) is detected by the role claims and reported as
   LSTM_ERR_PLACEMENT; later plans use the spread layout, and calls are
   correct.
"""
import numpy as np
import pytest

from layer_lstm_amd import synth
from oracle import oracle
from parity_util import compare, to_dev, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

ALL = dict(W=("u", 0.3), b=("u", 0.3), x=("n", 1.0), h0=("n", 0.5), c0=("n", 0.5), dy=("n", 1.0),
           dhT=("n", 1.0), dcT=("n", 1.0))


@pytest.fixture(scope="module")
def lstm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from layer_lstm_amd import lstm as mod
    yield mod
    mod.debug_inject(mod.DEBUG_FAIL_STEP, -1)
    mod.debug_inject(mod.DEBUG_MISPLACE, 0)
    mod.debug_inject(mod.DEBUG_XCD_LOCAL, 1)


def run(lstm, inp, m=None):
    dt = inp["dtype"]
    code = {"f32": lstm.F32, "bf16": lstm.BF16, "f16": lstm.F16}[dt]
    if m is None:
        m = lstm.Lstm(inp["T"], inp["B"], inp["I"], inp["H"], code)
    d = {k: to_dev(inp.get(k), dt, torch) for k in ("x", "W", "b", "h0", "c0", "dy", "dhT", "dcT")}
    m.forward(d["x"], d["W"], d["b"], d["h0"], d["c0"])
    m.backward(d["dy"], d["dhT"], d["dcT"], d["x"], d["W"], d["h0"], d["c0"])
    rc = lstm.check_workspace(m.workspace)
    out = {k: to_host(getattr(m, k)) for k in ("y", "hT", "cT", "dx", "dW", "db", "dh0", "dc0")}
    return rc, out, m


# the VALU recurrences (fp32, 4-row groups) and the MFMA ones (bf16)
@pytest.mark.parametrize("dt,T,B,I,H", [("f32", 12, 32, 64, 256), ("bf16", 12, 60, 32, 512)])
def test_forced_timeout_is_reported_and_recovers(lstm, dt, T, B, I, H):
    inp = synth.make_inputs(T, B, I, H, dt, seed=121, dist=ALL)
    print(f"case: forced time-out {dt} T={T} B={B} I={I} H={H}", flush=True)
    try:
        lstm.debug_inject(lstm.DEBUG_FAIL_STEP, 5)
        rc, _, m = run(lstm, inp)
    finally:
        lstm.debug_inject(lstm.DEBUG_FAIL_STEP, -1)
    assert rc == -9, rc
    # reported once, then cleared
    assert lstm.check_workspace(m.workspace) == 0
    rc, out, _ = run(lstm, inp, m)
    assert rc == 0, rc
    errs, bad = compare(out, oracle.fwd_bwd(inp), dt)
    assert not bad, bad


def test_misplaced_work_group_is_detected_and_spread_layout_taken(lstm):
    dt, T, B, I, H = "bf16", 6, 60, 32, 512
    shape = lstm.make_shape(T, B, I, H, lstm.BF16)
    if not lstm.query_plan(shape)["xcd_local"]:
        pytest.skip("this shape is not laid out XCD-local on this device")
    inp = synth.make_inputs(T, B, I, H, dt, seed=123, dist=ALL)
    print("case: misplaced work-group", flush=True)
    try:
        lstm.debug_inject(lstm.DEBUG_MISPLACE, 1)
        rc, _, _ = run(lstm, inp)
        lstm.debug_inject(lstm.DEBUG_MISPLACE, 0)
        assert rc == -12, rc
        # later plans on this device avoid the XCD-local layout, and are right
        assert lstm.query_plan(shape)["xcd_local"] == 0
        rc, out, _ = run(lstm, inp)
        assert rc == 0, rc
        errs, bad = compare(out, oracle.fwd_bwd(inp), dt)
        assert not bad, bad
    finally:
        lstm.debug_inject(lstm.DEBUG_MISPLACE, 0)
        lstm.debug_inject(lstm.DEBUG_XCD_LOCAL, 1)
    assert lstm.query_plan(shape)["xcd_local"] == 1


def test_exchange_probe_runs_in_both_layouts(lstm):
    """lstm_probe_exchange (the forward's exchange alone) completes without a
    time-out in the workload layouts and spread, and a step of it costs less
    than a step of the real forward recurrence."""
    for name in ("f32_T64_B32_I256_H256", "bf16_T256_B256_I1024_H1024"):
        w = synth.WORKLOADS[name]
        code = lstm.F32 if w.dtype == "f32" else lstm.BF16
        m = lstm.Lstm(w.T, w.B, w.I, w.H, code)
        us = [lstm.probe_exchange(m.shape, m.workspace, layout) for layout in (0, 1)]
        print(name, "floor us/step", us, flush=True)
        assert all(0 < u < 50 for u in us)


def test_mfma_stage_probe(lstm):
    """lstm_probe_mfma_stage runs every combination of a product stage's
    parts and reports a fraction of the bf16 peak in (0, 1.1]; it rejects
    both read orders at once and a scratch buffer that is too small."""
    scratch = torch.empty(lstm.PROBE_SCRATCH_BYTES, dtype=torch.uint8, device="cuda")
    fr = {}
    for parts in (0, 1, 2, 4, 8, 5, 6, 9, 10, 12, 13, 14):
        fr[parts] = lstm.probe_mfma_stage(parts, scratch, 200)
    print("stage probe fractions", {k: round(v, 3) for k, v in fr.items()}, flush=True)
    assert all(0.0 < v <= 1.1 for v in fr.values())
    with pytest.raises(lstm.LstmError) as e:
        lstm.probe_mfma_stage(lstm.PROBE_READS | lstm.PROBE_READS_AHEAD, scratch, 10)
    assert e.value.code == -2
    with pytest.raises(lstm.LstmError) as e:
        lstm.probe_mfma_stage(0, scratch[: lstm.PROBE_SCRATCH_BYTES // 2], 10)
    assert e.value.code == -5


def test_status_word_of_empty_calls_and_unfilled_workspaces(lstm):
    """A forward with T = 0 or B = 0 (no recurrence runs) still defines the
    workspace's status word, so checking it after such a call reports OK
    whatever the memory held before; a word holding bits no call writes (a
    workspace no forward pass has filled) reports ERR_STATE and leaves the
    layout choice alone.  (A stale word used to read as a placement error
    and switch the device to the spread layout.)"""
    probe = lstm.make_shape(6, 60, 32, 512, lstm.BF16)
    local = lstm.query_plan(probe)["xcd_local"]
    for T, B in ((0, 4), (3, 0)):
        m = lstm.Lstm(T, B, 8, 16, lstm.F32)
        m.workspace.fill_(0xFF)
        x = torch.zeros((T, B, 8), device="cuda")
        W = torch.zeros((64, 24), device="cuda")
        h0 = torch.zeros((B, 16), device="cuda")
        m.forward(x, W, None, h0, h0)
        m.check()  # raises on anything but OK
    m = lstm.Lstm(3, 4, 8, 16, lstm.F32)
    m.workspace.fill_(0xFF)
    torch.cuda.synchronize()
    assert lstm.check_workspace(m.workspace) == -13
    assert lstm.query_plan(probe)["xcd_local"] == local
    stack = lstm.Stack(0, 4, 8, 16, 2, lstm.F32)
    stack.workspace.fill_(0xFF)
    h = torch.zeros((2, 4, 16), device="cuda")
    stack.forward(torch.zeros((0, 4, 8), device="cuda"), torch.zeros(stack.w_elems, device="cuda"), None, h, h)
    stack.check()
