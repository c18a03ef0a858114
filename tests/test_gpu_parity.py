"""GPU parity of the HIP path (through the C-ABI) against the fp64 oracle.

Tolerance (relative L2 per output tensor, over the whole tensor): 1e-5 for
fp32 storage, 2e-2 for bf16 storage with fp32 accumulation.  Inputs are the
seeded synthetic tensors of layer_lstm_amd.synth; the oracle consumes the
same stored values.

 * the two fp32 workloads (T=8 B=4 I=16 H=32; T=64 B=32 I=256 H=256): every
   output element against the oracle;
 * ragged shapes that span several tiles with partial tails, odd sizes,
   I = 0, missing optional tensors, T = 0 and B = 0;
 * the three bf16 workloads at full size in the benchmark's launch
   configuration: every output against the oracle on the whole batch (run in
   chunks of batch rows, which are independent in both passes), whole and
   row by row -- the largest on the first and last row of each batch group
   (with masked cotangents for dW, db) unless LSTM_FULL_PARITY=1 asks for its
   whole batch too; linearity of the backward in its cotangents; run-to-run
   determinism of the largest;
 * besides the whole-tensor relative L2, every comparison checks each row
   (a (t, b) row, a batch row of a state, a gate row of dW) against the
   larger of its own norm and the RMS row norm (parity_util.row_errors);
 * output buffers are filled with NaN before each call, so an output left
   unwritten fails;
 * shapes whose input projection takes the persistent form: fp32 (sampled
   rows and masked dW/db, as above) and bf16 with a partial last row tile;
 * the reverse direction of time against the oracle through every kernel
   variant, and against the forward direction on time-flipped inputs;
 * the "ijfo" gate order against the oracle, and against the default order
   on relabelled weights;
 * two biases (b_ih, b_hh) against the oracle, and against their sum as one
   bias;
 * every flag at once at full size (T=128 B=64 I=512 H=1024), sampled rows.
"""
import os

import numpy as np
import pytest

from layer_lstm_amd import synth
from oracle import oracle
from parity_util import ROW_TOL, TOL, compare, compare_rows, rel_l2, run_gpu, to_dev, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def lstm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from layer_lstm_amd import lstm as mod
    return mod


def say(*a):
    print(*a, flush=True)


def full_check(inp, lstm, tol=None):
    code = {"f32": lstm.F32, "bf16": lstm.BF16, "f16": lstm.F16}[inp["dtype"]]
    say("plan:", lstm.query_plan(lstm.make_shape(inp["T"], inp["B"], inp["I"], inp["H"], code)))
    ref = oracle.fwd_bwd(inp)
    out, _, _ = run_gpu(inp, lstm, torch, poison=True)
    errs, bad = compare(out, ref, inp["dtype"], tol=tol)
    worst, bad_rows = compare_rows(out, ref, ROW_TOL[inp["dtype"]] if tol is None else 5 * tol)
    say("rel-L2:", {k: f"{v:.2e}" for k, v in errs.items()})
    say("worst row:", {k: f"{v:.2e}" for k, v in worst.items()})
    assert not bad, bad
    assert not bad_rows, bad_rows
    return errs


# Layouts of the persistent recurrences on one MI355X (256 CUs in 8 XCDs):
# (rows per group, units per group, waves, XCD-local, forward VALU, backward
# VALU), and the input projection's output tiles per work-group (> 1: the
# persistent form; 256 x 256 bf16 tiles, 32-deep stages)
# (rows, units, waves, XCD-local, VALU forward, VALU backward), input
# projection tiles per work-group, tagged forward exchange (the spread
# layout's 16-bit form)
PLANS = {
    "f32_T8_B4_I16_H32": ((4, 8, 4, 0, 1, 1), 1, 0),
    "f32_T64_B32_I256_H256": ((4, 8, 4, 1, 1, 1), 1, 0),
    "bf16_T128_B64_I512_H1024": ((8, 32, 8, 1, 0, 0), 2, 0),     # 32 x 16 tiles
    "bf16_T512_B16_I1024_H2048": ((8, 16, 8, 0, 0, 0), 4, 1),    # 32 x 32 tiles
    "bf16_T256_B256_I1024_H1024": ((32, 32, 8, 1, 0, 0), 16, 0), # 256 x 16 tiles
}


@pytest.mark.parametrize("name", list(PLANS))
def test_workload_plans(lstm, name):
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("layouts are stated for 256 CUs")
    w = synth.WORKLOADS[name]
    code = lstm.F32 if w.dtype == "f32" else lstm.BF16
    p = lstm.query_plan(lstm.make_shape(w.T, w.B, w.I, w.H, code))
    say(name, p)
    got = (p["rows_per_group"], p["units_per_group"], p["waves"], p["xcd_local"], p["fwd_valu"], p["bwd_valu"])
    assert got == PLANS[name][0]
    assert p["inproj_tiles_per_wg"] == PLANS[name][1]
    assert p["fwd_tagged"] == PLANS[name][2]
    assert p["grid"] == p["groups"] * p["units_groups"] <= 256


def test_small_workload(lstm):
    say("case: f32_T8_B4_I16_H32")
    full_check(synth.workload_inputs("f32_T8_B4_I16_H32"), lstm)


def test_headline_workload(lstm):
    say("case: f32_T64_B32_I256_H256")
    full_check(synth.workload_inputs("f32_T64_B32_I256_H256"), lstm)


ALL = dict(W=("u", 0.3), b=("u", 0.3), x=("n", 1.0), h0=("n", 0.5), c0=("n", 0.5), dy=("n", 1.0),
           dhT=("n", 1.0), dcT=("n", 1.0))


@pytest.mark.parametrize("dt,T,B,I,H", [
    ("f32", 5, 20, 72, 96),     # ragged batch and hidden tiles
    ("f32", 3, 17, 13, 40),     # input size not a multiple of the vector width
    ("f32", 1, 1, 1, 1),
    ("f32", 6, 3, 0, 8),        # no input features
    ("f32", 4, 40, 130, 200),   # several batch groups
    ("bf16", 4, 19, 40, 72),
    ("bf16", 8, 32, 40, 72),    # dW through the LDS path, the h / x border inside a swizzle group
    ("bf16", 4, 64, 64, 96),
    ("f32", 32, 32, 40, 72),    # the same for fp32 (T*B >= 1024)
    ("bf16", 3, 5, 7, 33),      # odd hidden size
    ("bf16", 2, 33, 24, 130),
    # rows of whole kilobytes (the forward's direct-to-LDS path, P and the
    # record staged in LDS), with a last batch group that is not full
    ("bf16", 3, 5, 24, 512),    # 4-row groups: P of a step is half a wave-load
    ("f32", 3, 100, 16, 256),   # fp32 through the MFMA forward, 8-row groups
    ("bf16", 2, 100, 64, 512),  # 8-row groups, 32 units, 8 waves
    ("bf16", 3, 60, 32, 512),   # 8 batch groups (one per XCD)
])
def test_ragged_shapes(lstm, dt, T, B, I, H):
    say(f"case: ragged {dt} T={T} B={B} I={I} H={H}")
    inp = synth.make_inputs(T, B, I, H, dt, seed=21, dist=ALL)
    full_check(inp, lstm)


def test_optional_inputs_absent(lstm):
    """b, h0, c0, dhT, dcT all NULL: zero bias, zero initial state, zero
    final-state cotangents (and db still computed)."""
    say("case: optional inputs absent")
    dist = dict(ALL, b=("z",), h0=("z",), c0=("z",), dhT=("z",), dcT=("z",))
    inp = synth.make_inputs(6, 9, 24, 48, "f32", seed=22, dist=dist)
    full_check(inp, lstm)


@pytest.mark.parametrize("T,B,two", [(0, 4, False), (3, 0, False), (0, 4, True), (3, 0, True)])
def test_empty(lstm, T, B, two):
    """T = 0 or B = 0: the final states are the initial ones, the state
    gradients the final-state cotangents, dW and db zero -- both halves of
    db with two biases, whatever the output buffer held before."""
    say(f"case: empty T={T} B={B} two_bias={two}")
    inp = two_bias_inputs("f32", T, B, 8, 16, 23) if two else synth.make_inputs(T, B, 8, 16, "f32", seed=23, dist=ALL)
    ref = oracle.fwd_bwd(inp)
    out, _, _ = run_gpu(inp, lstm, torch, poison=True)
    for k in ("hT", "cT", "dh0", "dc0", "dW", "db"):
        np.testing.assert_array_equal(out[k], ref[k], err_msg=k)


def test_nondefault_stream_and_repeat_backward(lstm):
    """Launches follow the given stream; the backward does not consume the
    forward record, so a second backward gives identical results."""
    say("case: side stream, repeated backward")
    inp = synth.make_inputs(7, 18, 40, 64, "f32", seed=24, dist=ALL)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out, m, d = run_gpu(inp, lstm, torch, stream=s)
        m.backward(d["dy"], d["dhT"], d["dcT"], d["x"], d["W"], d["h0"], d["c0"], stream=s)
    s.synchronize()
    for k, t in (("dx", m.dx), ("dW", m.dW), ("db", m.db), ("dh0", m.dh0), ("dc0", m.dc0)):
        np.testing.assert_array_equal(to_host(t), out[k], err_msg=k)
    ref = oracle.fwd_bwd(inp)
    errs, bad = compare(out, ref, "f32")
    assert not bad, bad


def test_segment_composition_gpu(lstm):
    """Forward over T1 then T2 steps from the returned state equals the
    forward over T1+T2 steps (within the fp32 tolerance)."""
    say("case: segment composition")
    T1, T2 = 4, 5
    inp = synth.make_inputs(T1 + T2, 12, 20, 40, "f32", seed=25, dist=ALL)
    full, _, _ = run_gpu(inp, lstm, torch)
    s1 = dict(inp, T=T1, x=inp["x"][:T1], dy=inp["dy"][:T1])
    o1, _, _ = run_gpu(s1, lstm, torch)
    s2 = dict(inp, T=T2, x=inp["x"][T1:], dy=inp["dy"][T1:], h0=o1["hT"], c0=o1["cT"])
    o2, _, _ = run_gpu(s2, lstm, torch)
    assert rel_l2(np.concatenate([o1["y"], o2["y"]]), full["y"]) <= TOL["f32"]
    assert rel_l2(o2["cT"], full["cT"]) <= TOL["f32"]


# ---------------------------------------------------------------------------
# bf16 workloads at full size, in the benchmark's launch configuration,
# against the oracle on the whole batch.  Rows of the batch are independent in
# both passes, so the oracle runs on chunks of batch rows (each a few tens of
# seconds of fp64 on the host cores, with a progress line after each): the
# per-row outputs (y, hT, cT, dx, dh0, dc0) are the chunks' own, and dW, db are
# the sums of the chunks' (summed in fp64, in chunk order -- the same sums over
# (t, b) as one call, grouped by rows).  Every output is compared whole
# (relative L2) and row by row (row_errors: a corrupted or stale row of any
# batch group, time step or gate fails).
#
# The largest workload (T=256 B=256 I=1024 H=1024) takes about six minutes of
# oracle time on the whole batch; by default it is compared on the first and
# last batch row of each of its eight batch groups (one per XCD: every
# work-group role of the XCD-local layout), with dW and db from cotangents
# that are zero outside those rows (every other row's gate deltas are then
# exactly zero); LSTM_FULL_PARITY=1 compares its whole batch as well.
FULL_CHUNK = {
    "bf16_T128_B64_I512_H1024": 32,
    "bf16_T512_B16_I1024_H2048": 4,
    "bf16_T256_B256_I1024_H1024": 16,
}
LARGEST = "bf16_T256_B256_I1024_H1024"
FULL_PARITY = os.environ.get("LSTM_FULL_PARITY") == "1"


def rows_of(inp, rows):
    sub = dict(inp, B=len(rows))
    for k in ("x", "dy"):
        sub[k] = inp[k][:, rows]
    for k in ("h0", "c0", "dhT", "dcT"):
        sub[k] = None if inp[k] is None else inp[k][rows]
    return sub


def oracle_by_chunks(inp, chunk, progress):
    """The oracle on the whole batch, run on chunks of `chunk` batch rows."""
    B = inp["B"]
    parts = []
    for b0 in range(0, B, chunk):
        rows = list(range(b0, min(B, b0 + chunk)))
        parts.append(oracle.fwd_bwd(rows_of(inp, rows)))
        progress(f"  oracle rows [{b0}, {rows[-1] + 1}) of {B} done")
    ref = {k: np.concatenate([p[k] for p in parts], axis=1) for k in ("y", "dx")}
    ref.update({k: np.concatenate([p[k] for p in parts], axis=0) for k in ("hT", "cT", "dh0", "dc0")})
    for k in ("dW", "db"):
        acc = np.zeros_like(parts[0][k])
        for p in parts:
            acc = acc + p[k]
        ref[k] = acc
    return ref


@pytest.fixture
def progress(capsys):
    """Print a line to the terminal at once (long oracle runs stay visible)."""
    def emit(msg):
        with capsys.disabled():
            print(msg, flush=True)
    return emit


@pytest.fixture(scope="module")
def big_runs(lstm):
    """One full-size GPU forward+backward per bf16 workload, kept for the
    checks below."""
    res = {}
    for name in FULL_CHUNK:
        say("case: full-size", name)
        inp = synth.workload_inputs(name)
        out, m, d = run_gpu(inp, lstm, torch, poison=True)
        res[name] = (inp, out, m, d)
    return res


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", list(FULL_CHUNK))
def test_bf16_workload_full_batch(lstm, big_runs, name, progress):
    if name == LARGEST and not FULL_PARITY:
        pytest.skip("about six minutes of fp64 oracle on the host; LSTM_FULL_PARITY=1 runs it "
                    "(test_bf16_largest_workload_every_group covers every batch group by default)")
    inp, out, _, _ = big_runs[name]
    progress(f"case: full batch {name}")
    ref = oracle_by_chunks(inp, FULL_CHUNK[name], progress)
    errs, bad = compare(out, ref, "bf16")
    worst, bad_rows = compare_rows(out, ref, ROW_TOL["bf16"])
    progress("  rel-L2: " + str({k: f"{v:.2e}" for k, v in errs.items()}))
    progress("  worst row: " + str({k: f"{v:.2e}" for k, v in worst.items()}))
    assert not bad, bad
    assert not bad_rows, bad_rows


def check_every_group(lstm, inp, out, m, d, progress):
    """The first and last batch row of each batch group of the recurrences'
    layout against the oracle on those rows (whole and row by row), and dW,
    db from a second backward on `m` whose cotangents are zero outside those
    rows (every other row's gate deltas are then exactly zero)."""
    dt = inp["dtype"]
    code = {"f32": lstm.F32, "bf16": lstm.BF16, "f16": lstm.F16}[dt]
    nb = lstm.query_plan(lstm.make_shape(inp["T"], inp["B"], inp["I"], inp["H"], code))["rows_per_group"]
    rows = sorted({r for g0 in range(0, inp["B"], nb) for r in (g0, min(inp["B"], g0 + nb) - 1)})
    progress(f"  rows {rows}")
    ref = oracle.fwd_bwd(rows_of(inp, rows))
    keys = ("y", "hT", "cT", "dx", "dh0", "dc0")
    got = dict(y=out["y"][:, rows], hT=out["hT"][rows], cT=out["cT"][rows], dx=out["dx"][:, rows],
               dh0=out["dh0"][rows], dc0=out["dc0"][rows])
    errs, bad = compare(got, ref, dt, keys=keys)
    worst, bad_rows = compare_rows(got, ref, ROW_TOL[dt], keys=keys)
    progress("  rel-L2: " + str({k: f"{v:.2e}" for k, v in errs.items()}))
    progress("  worst row: " + str({k: f"{v:.2e}" for k, v in worst.items()}))
    assert not bad and not bad_rows, (bad, bad_rows)
    mask = np.zeros(inp["B"])
    mask[rows] = 1.0
    masked = dict(inp, dy=inp["dy"] * mask[None, :, None])
    for k in ("dhT", "dcT"):
        masked[k] = None if inp[k] is None else inp[k] * mask[:, None]
    dm = {k: to_dev(masked[k], dt, torch) for k in ("dy", "dhT", "dcT")}
    m.forward(d["x"], d["W"], d["b"], d["h0"], d["c0"])
    m.backward(dm["dy"], dm["dhT"], dm["dcT"], d["x"], d["W"], d["h0"], d["c0"])
    m.check()
    torch.cuda.synchronize()
    refm = oracle.fwd_bwd(rows_of(masked, rows))
    gotm = {"dW": to_host(m.dW), "db": to_host(m.db)}
    errs, bad = compare(gotm, refm, dt, keys=("dW", "db"))
    worst, bad_rows = compare_rows(gotm, refm, ROW_TOL[dt], keys=("dW", "db"))
    progress("  masked dW/db rel-L2: " + str({k: f"{v:.2e}" for k, v in errs.items()}) +
             " worst row: " + str({k: f"{v:.2e}" for k, v in worst.items()}))
    assert not bad and not bad_rows, (bad, bad_rows)


def test_bf16_largest_workload_every_group(lstm, big_runs, progress):
    """T=256 B=256 I=1024 H=1024 at full size: the first and last batch row
    of each of the eight 32-row batch groups, and the masked dW, db
    (check_every_group)."""
    inp, out, m, d = big_runs[LARGEST]
    progress(f"case: every batch group of {LARGEST}")
    check_every_group(lstm, inp, out, m, d, progress)


def test_bf16_determinism_full_size(lstm, big_runs):
    """A second forward+backward of the largest workload (T=256 B=256
    I=1024 H=1024) on fresh buffers gives the same bits: no float atomics,
    fixed summation orders in every kernel."""
    name = "bf16_T256_B256_I1024_H1024"
    inp, out, _, _ = big_runs[name]
    say("case: full-size determinism", name)
    again, _, _ = run_gpu(inp, lstm, torch, poison=True)
    for k in out:
        np.testing.assert_array_equal(again[k], out[k], err_msg=k)


def test_bf16_backward_linearity_full_size(lstm, big_runs):
    """bwd(g1 + g2) = bwd(g1) + bwd(g2) over the cotangents, at full size
    (T=128 B=64 I=512 H=1024)."""
    name = "bf16_T128_B64_I512_H1024"
    inp, _, m, d = big_runs[name]
    say("case: linearity", name)
    rng = np.random.default_rng(99)
    g2 = synth.round_to_storage(rng.normal(0, 1, inp["dy"].shape), "bf16")
    m.forward(d["x"], d["W"], d["b"], d["h0"], d["c0"])
    outs = []
    for dy in (inp["dy"], g2, inp["dy"] + g2):
        m.backward(to_dev(dy, "bf16", torch), None, None, d["x"], d["W"], d["h0"], d["c0"])
        torch.cuda.synchronize()
        outs.append({k: to_host(getattr(m, k)) for k in ("dx", "dW", "db", "dh0", "dc0")})
    for k in outs[0]:
        e = rel_l2(outs[2][k], outs[0][k] + outs[1][k])
        assert e <= TOL["bf16"], (k, e)


def test_f32_persistent_input_projection(lstm):
    """fp32 through the persistent input projection (128 x 128 tiles, 16-deep
    stages: 32 x 16 tiles, two per work-group on 256 CUs): sampled batch rows
    of every output, and dW/db from cotangents zero outside those rows,
    against the oracle on the rows alone."""
    T, B, I, H = 16, 256, 1024, 512
    shape = lstm.make_shape(T, B, I, H, lstm.F32)
    p = lstm.query_plan(shape)
    say("case: f32 persistent input projection", p)
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert p["inproj_tiles_per_wg"] == 2
    inp = synth.make_inputs(T, B, I, H, "f32", seed=23, dist=ALL)
    rows = [0, 97, 255]
    out, m, d = run_gpu(inp, lstm, torch)
    ref = oracle.fwd_bwd(rows_of(inp, rows))
    got = dict(y=out["y"][:, rows], hT=out["hT"][rows], cT=out["cT"][rows], dx=out["dx"][:, rows],
               dh0=out["dh0"][rows], dc0=out["dc0"][rows])
    errs, bad = compare(got, ref, "f32", keys=tuple(got))
    say("rel-L2:", {k: f"{v:.2e}" for k, v in errs.items()})
    assert not bad, bad
    mask = np.zeros(B)
    mask[rows] = 1.0
    masked = dict(inp)
    masked["dy"] = inp["dy"] * mask[None, :, None]
    for k in ("dhT", "dcT"):
        masked[k] = None if inp[k] is None else inp[k] * mask[:, None]
    dm = {k: to_dev(masked[k], "f32", torch) for k in ("dy", "dhT", "dcT")}
    m.forward(d["x"], d["W"], d["b"], d["h0"], d["c0"])
    m.backward(dm["dy"], dm["dhT"], dm["dcT"], d["x"], d["W"], d["h0"], d["c0"])
    m.check()
    torch.cuda.synchronize()
    refm = oracle.fwd_bwd(rows_of(masked, rows))
    errs = {"dW": rel_l2(to_host(m.dW), refm["dW"]), "db": rel_l2(to_host(m.db), refm["db"])}
    say("rel-L2:", errs)
    assert errs["dW"] <= TOL["f32"] and errs["db"] <= TOL["f32"], errs


def test_persistent_input_projection_ragged_rows(lstm):
    """bf16 through the persistent input projection with a partial last row
    tile: T*B = 131070 = 511 full 256-row tiles + 254 rows, one column tile
    (4H = 256), two tiles per work-group on 256 CUs.  Sampled batch rows
    against the oracle on those rows; at t = T-1, rows b >= 3 lie in the
    partial tile."""
    T, B, I, H = 510, 257, 128, 64
    p = lstm.query_plan(lstm.make_shape(T, B, I, H, lstm.BF16))
    say("case: bf16 persistent input projection, ragged rows", p)
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert p["inproj_tiles_per_wg"] == 2
    inp = synth.make_inputs(T, B, I, H, "bf16", seed=29, dist=ALL)
    rows = [0, 128, 256]
    out, _, _ = run_gpu(inp, lstm, torch)
    ref = oracle.fwd_bwd(rows_of(inp, rows))
    got = dict(y=out["y"][:, rows], hT=out["hT"][rows], cT=out["cT"][rows], dx=out["dx"][:, rows],
               dh0=out["dh0"][rows], dc0=out["dc0"][rows])
    errs, bad = compare(got, ref, "bf16", keys=tuple(got))
    say("rel-L2:", {k: f"{v:.2e}" for k, v in errs.items()})
    assert not bad, bad
    last = dict(y=out["y"][T - 1, rows[1:]])
    errs, bad = compare(last, dict(y=ref["y"][T - 1, 1:]), "bf16", keys=("y",))
    say("rel-L2 (last step, partial tile):", errs)
    assert not bad, bad


# The reverse direction (flags = LSTM_REVERSE) through every kernel variant:
# fp32 VALU recurrences with the register-staged and the pipelined products,
# the fp32 MFMA forward, and the bf16 MFMA recurrences with and without the
# forward's direct-to-LDS path.
@pytest.mark.parametrize("dt,T,B,I,H", [
    ("f32", 8, 4, 16, 32),
    ("f32", 64, 32, 256, 256),
    ("f32", 3, 100, 16, 256),
    ("bf16", 4, 19, 40, 72),
    ("bf16", 3, 60, 32, 512),
    ("bf16", 5, 40, 64, 1024),
])
def test_reverse_direction(lstm, dt, T, B, I, H):
    say(f"case: reverse {dt} T={T} B={B} I={I} H={H}")
    inp = synth.make_inputs(T, B, I, H, dt, seed=37, dist=ALL)
    inp["reverse"] = True
    full_check(inp, lstm)


@pytest.mark.parametrize("dt,T,B,I,H", [("f32", 64, 32, 256, 256), ("bf16", 3, 60, 32, 512)])
def test_reverse_is_forward_on_flipped_time_gpu(lstm, dt, T, B, I, H):
    """On the GPU, the reverse direction equals the forward direction on
    time-flipped x and dy: the same arithmetic on the same values, so every
    output but dW and db (whose sums over t run in another order) matches
    bit for bit."""
    say(f"case: reverse vs flipped forward {dt} T={T} B={B} I={I} H={H}")
    inp = synth.make_inputs(T, B, I, H, dt, seed=41, dist=ALL)
    rev, _, _ = run_gpu(dict(inp, reverse=True), lstm, torch)
    fwd, _, _ = run_gpu(dict(inp, x=inp["x"][::-1].copy(), dy=inp["dy"][::-1].copy()), lstm, torch)
    for k in ("y", "dx"):
        assert np.array_equal(rev[k], fwd[k][::-1]), k
    for k in ("hT", "cT", "dh0", "dc0"):
        assert np.array_equal(rev[k], fwd[k]), k
    for k in ("dW", "db"):
        e = rel_l2(rev[k], fwd[k])
        assert e <= TOL[dt], (k, e)


# The "ijfo" gate order (flags = LSTM_GATES_IJFO) through the register-staged
# and direct-to-LDS products and both recurrence forms; once with the
# reverse direction as well.
@pytest.mark.parametrize("dt,T,B,I,H,rev", [
    ("f32", 8, 4, 16, 32, False),
    ("f32", 64, 32, 256, 256, False),
    ("bf16", 4, 19, 40, 72, False),
    ("bf16", 3, 60, 32, 512, True),
])
def test_gate_order_ijfo(lstm, dt, T, B, I, H, rev):
    say(f"case: ijfo {dt} T={T} B={B} I={I} H={H} reverse={rev}")
    inp = synth.make_inputs(T, B, I, H, dt, seed=43, dist=ALL)
    inp["gate_order"] = "ijfo"
    inp["reverse"] = rev
    full_check(inp, lstm)


@pytest.mark.parametrize("dt,T,B,I,H", [("f32", 16, 256, 1024, 512), ("bf16", 3, 60, 32, 512)])
def test_gate_order_is_a_relabelling_gpu(lstm, dt, T, B, I, H):
    """On the GPU, the "ijfo" order on relabelled W and b equals the default
    order bit for bit (dW and db relabelled back): the same arithmetic.  The
    fp32 shape takes the persistent input projection."""
    say(f"case: ijfo relabelling {dt} T={T} B={B} I={I} H={H}")
    inp = synth.make_inputs(T, B, I, H, dt, seed=47, dist=ALL)
    rows = oracle.ifjo_rows(H, "ijfo")
    a, _, _ = run_gpu(inp, lstm, torch)
    c, _, _ = run_gpu(dict(inp, W=inp["W"][rows], b=inp["b"][rows], gate_order="ijfo"), lstm, torch)
    for k in ("y", "hT", "cT", "dx", "dh0", "dc0"):
        assert np.array_equal(c[k], a[k]), k
    assert np.array_equal(c["dW"], a["dW"][rows]) and np.array_equal(c["db"], a["db"][rows])


def two_bias_inputs(dt, T, B, I, H, seed):
    inp = synth.make_inputs(T, B, I, H, dt, seed=seed, dist=ALL)
    rng = np.random.default_rng(seed + 1)
    b_hh = synth.round_to_storage(rng.uniform(-0.3, 0.3, 4 * H), dt)
    return dict(inp, b=np.stack([inp["b"], b_hh]), two_bias=True)


# Two biases (flags = LSTM_TWO_BIAS) through the register-staged, the
# pipelined and the persistent input projection; once with every flag.
@pytest.mark.parametrize("dt,T,B,I,H,rev,order", [
    ("f32", 8, 4, 16, 32, False, "ifjo"),
    ("f32", 64, 32, 256, 256, False, "ifjo"),
    ("bf16", 4, 19, 40, 72, False, "ifjo"),
    ("bf16", 3, 60, 32, 512, True, "ijfo"),
])
def test_two_biases(lstm, dt, T, B, I, H, rev, order):
    say(f"case: two biases {dt} T={T} B={B} I={I} H={H} reverse={rev} order={order}")
    inp = two_bias_inputs(dt, T, B, I, H, 59)
    inp.update(reverse=rev, gate_order=order)
    full_check(inp, lstm)


def test_two_biases_are_their_sum_gpu(lstm):
    """fp32: two biases give bit for bit what their fp32 sum gives as one
    bias (the kernel adds them in fp32 before the product's sum), with db
    in both halves.  The shape takes the persistent input projection."""
    T, B, I, H = 16, 256, 1024, 512
    say(f"case: two biases vs their sum f32 T={T} B={B} I={I} H={H}")
    two = two_bias_inputs("f32", T, B, I, H, 61)
    one = dict(two, two_bias=False, b=(two["b"][0].astype(np.float32) + two["b"][1].astype(np.float32)))
    a, _, _ = run_gpu(two, lstm, torch)
    c, _, _ = run_gpu(one, lstm, torch)
    for k in ("y", "hT", "cT", "dx", "dW", "dh0", "dc0"):
        assert np.array_equal(a[k], c[k]), k
    assert np.array_equal(a["db"][0], c["db"]) and np.array_equal(a["db"][1], c["db"])


def test_all_flags_full_size_sampled_rows(lstm):
    """bf16_T128_B64_I512_H1024 at full size, in the benchmark's launch
    configuration, with every flag: the reverse direction, the "ijfo" gate
    order and two biases.  Sampled batch rows of every per-row output
    against the oracle on those rows."""
    name = "bf16_T128_B64_I512_H1024"
    w = synth.WORKLOADS[name]
    say("case: full size, all flags", name)
    inp = synth.workload_inputs(name)
    rng = np.random.default_rng(67)
    b_hh = synth.round_to_storage(rng.uniform(-0.03, 0.03, 4 * w.H), "bf16")
    inp = dict(inp, b=np.stack([inp["b"], b_hh]), two_bias=True, reverse=True, gate_order="ijfo")
    out, _, _ = run_gpu(inp, lstm, torch)
    rows = [1, 40]
    ref = oracle.fwd_bwd(rows_of(inp, rows))
    got = dict(y=out["y"][:, rows], hT=out["hT"][rows], cT=out["cT"][rows], dx=out["dx"][:, rows],
               dh0=out["dh0"][rows], dc0=out["dc0"][rows])
    errs, bad = compare(got, ref, "bf16", keys=tuple(got))
    say("rel-L2:", {k: f"{v:.2e}" for k, v in errs.items()})
    assert not bad, bad


def test_determinism(lstm):
    say("case: determinism")
    inp = synth.workload_inputs("f32_T64_B32_I256_H256")
    a, _, _ = run_gpu(inp, lstm, torch)
    b, _, _ = run_gpu(inp, lstm, torch)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)


def test_abi_errors_leave_outputs_untouched(lstm):
    say("case: ABI errors")
    m = lstm.Lstm(4, 8, 16, 32, lstm.F32)
    x = torch.randn(4, 8, 16, device="cuda")
    W = torch.randn(128, 48, device="cuda")
    m.y.fill_(7.0)
    # workspace too small
    rc = lstm.fwd_train(m.shape, x, W, None, None, None, m.y, m.hT, m.cT, m.workspace, m.ws_bytes - 256,
                        check=False)
    assert rc == -5
    # misaligned output
    rc = lstm.fwd_train(m.shape, x, W, None, None, None, m.y.data_ptr() + 2, m.hT, m.cT, m.workspace,
                        m.ws_bytes, check=False)
    assert rc == -4
    # missing required pointer
    rc = lstm.fwd_train(m.shape, None, W, None, None, None, m.y, m.hT, m.cT, m.workspace, m.ws_bytes,
                        check=False)
    assert rc == -1
    rc = lstm.bwd(m.shape, None, None, None, x, W, None, None, m.y, m.workspace, m.dx, m.dW, None, m.dh0,
                  m.dc0, check=False)
    assert rc == -1
    torch.cuda.synchronize()
    assert bool((m.y == 7.0).all())
    # unsupported size
    big = lstm.make_shape(2, 2, 2, 4096, lstm.F32)
    import ctypes
    n = ctypes.c_size_t(0)
    assert lstm.lib().lstm_query(ctypes.byref(big), ctypes.byref(n)) == -6


def test_two_streams_concurrent(lstm):
    """Two calls issued on two streams without synchronisation in between
    (each recurrence a grid of up to one work-group per CU): the library
    orders the persistent launches, both complete without a time-out and
    both match the oracle."""
    say("case: two streams")
    inps = [synth.make_inputs(9, 32, 256, 256, "f32", seed=71 + i, dist=ALL) for i in range(2)]
    refs = [oracle.fwd_bwd(inp) for inp in inps]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    runs = []
    for inp, s in zip(inps, streams):
        m = lstm.Lstm(inp["T"], inp["B"], inp["I"], inp["H"], lstm.F32)
        with torch.cuda.stream(s):
            d = {k: to_dev(inp.get(k), "f32", torch) for k in ("x", "W", "b", "h0", "c0", "dy", "dhT", "dcT")}
        runs.append((m, d, s))
    torch.cuda.synchronize()
    for m, d, s in runs:
        m.forward(d["x"], d["W"], d["b"], d["h0"], d["c0"], stream=s)
    for m, d, s in runs:
        m.backward(d["dy"], d["dhT"], d["dcT"], d["x"], d["W"], d["h0"], d["c0"], stream=s)
    for (m, d, s), ref in zip(runs, refs):
        m.check(s)
        out = {k: to_host(getattr(m, k)) for k in ("y", "hT", "cT", "dx", "dW", "db", "dh0", "dc0")}
        errs, bad = compare(out, ref, "f32")
        assert not bad, bad


# ---------------------------------------------------------------------------
# fp16 storage (LSTM_F16: the FLOAT16 of the operator page's dtype column)
# through every kernel variant on ragged shapes, and at the three 16-bit
# workload shapes at full size, against the oracle on the same fp16-rounded
# inputs within the fp16 bound (parity_util.TOL).

@pytest.mark.parametrize("T,B,I,H,rev", [
    (4, 19, 40, 72, False),
    (3, 5, 7, 33, False),      # odd hidden size
    (3, 5, 24, 512, False),    # 4-row groups, the forward's direct-to-LDS path
    (2, 100, 64, 512, True),   # 8-row groups, 32 units, 8 waves; reverse
    (3, 60, 32, 512, False),   # 8 batch groups (one per XCD)
    (5, 40, 64, 1024, False),
])
def test_f16_ragged_shapes(lstm, T, B, I, H, rev):
    say(f"case: f16 T={T} B={B} I={I} H={H} reverse={rev}")
    inp = dict(synth.make_inputs(T, B, I, H, "f16", seed=83, dist=ALL), reverse=rev)
    full_check(inp, lstm)


def test_f16_all_flags(lstm):
    """fp16 with the "ijfo" gate order and two biases."""
    say("case: f16 ijfo, two biases")
    inp = two_bias_inputs("f16", 3, 60, 32, 512, 85)
    inp.update(gate_order="ijfo")
    full_check(inp, lstm)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["f16_T128_B64_I512_H1024", "f16_T512_B16_I1024_H2048",
                                  "f16_T256_B256_I1024_H1024"])
def test_f16_workload_every_group(lstm, name, progress):
    """The 16-bit workload shapes in fp16 at full size, in the benchmark's
    launch configuration: every batch group's first and last row and the
    masked dW, db against the oracle (check_every_group)."""
    progress(f"case: fp16 full size {name}")
    inp = synth.workload_inputs(name)
    out, m, d = run_gpu(inp, lstm, torch, poison=True)
    for k, v in out.items():
        assert np.all(np.isfinite(v)), k
    check_every_group(lstm, inp, out, m, d, progress)


# ---------------------------------------------------------------------------
# The bidirectional layer (LSTM_BIDIRECTIONAL: the num_directions = 2 layout
# of the PyTorch recurrent-layer page) and sequence lengths (the seq_length
# mask of the operator page's parameter table, per-sequence form), against
# the oracle's composition of its forward and reverse passes and its masked
# blend.

def contracting(H):
    """ALL with W, b ~ U(+-1/sqrt(H)), the workloads' range.  ALL's 0.3 at
    H = 1024 makes the recurrence chaotic (a gain of about 0.3*sqrt(H/3) per
    step), so that over a hundred steps the rounding of the stored values
    grows into errors of whole percent on both sides alike; long sequences at
    large H take this range instead."""
    k = 1.0 / np.sqrt(H)
    return dict(ALL, W=("u", k), b=("u", k))


def bidir_gpu_inputs(dt, T, B, I, H, seed, dist=ALL):
    if dist is None:
        dist = contracting(H)
    a = synth.make_inputs(T, B, I, H, dt, seed=seed, dist=dist)
    c = synth.make_inputs(T, B, I, H, dt, seed=seed + 1000, dist=dist)
    inp = dict(a, bidirectional=True, dy=np.concatenate([a["dy"], c["dy"]], axis=2))
    for k in ("W", "b", "h0", "c0", "dhT", "dcT"):
        inp[k] = None if a[k] is None else np.stack([a[k], c[k]])
    return inp


# fp32 VALU recurrences (4-row groups), the fp32 MFMA forward, 16-bit MFMA
# recurrences with and without the forward's direct-to-LDS path and the
# XCD-local layout; the T=64 B=32 I=256 H=256 and T=128 B=64 I=512 H=1024
# workload shapes; a ragged one.
@pytest.mark.parametrize("dt,T,B,I,H", [
    ("f32", 8, 4, 16, 32),
    ("f32", 64, 32, 256, 256),
    ("f32", 3, 100, 16, 256),
    ("bf16", 4, 19, 40, 72),
    ("bf16", 3, 60, 32, 512),
    ("f16", 5, 40, 64, 1024),
    ("bf16", 128, 64, 512, 1024),
])
def test_bidirectional(lstm, dt, T, B, I, H):
    inp = bidir_gpu_inputs(dt, T, B, I, H, seed=101, dist=ALL if T * H <= 8192 else None)
    code = {"f32": lstm.F32, "bf16": lstm.BF16, "f16": lstm.F16}[dt]
    p = lstm.query_plan(lstm.make_shape(T, B, I, H, code, bidirectional=True))
    say(f"case: bidirectional {dt} T={T} B={B} I={I} H={H}, plan {p}")
    full_check(inp, lstm)


def test_bidirectional_all_flags(lstm):
    """Both directions with the "ijfo" gate order and two biases."""
    inp = bidir_gpu_inputs("bf16", 3, 60, 32, 512, seed=103)
    rng = np.random.default_rng(104)
    inp["b"] = np.stack([inp["b"], synth.round_to_storage(rng.uniform(-0.3, 0.3, (2, 2048)), "bf16")], axis=1)
    inp.update(two_bias=True, gate_order="ijfo")
    say("case: bidirectional, ijfo, two biases")
    full_check(inp, lstm)


def test_bidirectional_is_two_directions_gpu(lstm):
    """On the GPU the bidirectional layer gives what the forward direction
    and the reverse direction give as two one-direction calls, within the
    tolerance (dx: their sum).  Not bit for bit: the concurrent launch lays
    each direction out for half the compute units, so its sums over units
    and gate rows group differently."""
    dt, T, B, I, H = "bf16", 3, 60, 32, 512
    inp = bidir_gpu_inputs(dt, T, B, I, H, seed=105)
    both, _, _ = run_gpu(inp, lstm, torch)
    outs = []
    for dd in range(2):
        one = dict(inp, bidirectional=False, reverse=bool(dd), W=inp["W"][dd], b=inp["b"][dd],
                   dy=inp["dy"][:, :, dd * H:(dd + 1) * H].copy())
        for k in ("h0", "c0", "dhT", "dcT"):
            one[k] = inp[k][dd]
        outs.append(run_gpu(one, lstm, torch)[0])
    assert rel_l2(both["y"], np.concatenate([outs[0]["y"], outs[1]["y"]], axis=2)) <= TOL[dt]
    for k in ("hT", "cT", "dW", "db", "dh0", "dc0"):
        assert rel_l2(both[k], np.stack([outs[0][k], outs[1][k]])) <= TOL[dt], k
    assert rel_l2(both["dx"], outs[0]["dx"] + outs[1]["dx"]) <= TOL[dt]


LENGTHS_DIST = dict(ALL)


def ragged_lengths(T, B, seed):
    """Lengths covering the edges: full (T), longer than T, empty (0),
    negative, one step, and the rest spread over [1, T]."""
    rng = np.random.default_rng(seed)
    L = rng.integers(1, T + 1, size=B)
    edges = [T, T + 3, 0, -2, 1]
    L[:min(B, len(edges))] = edges[:min(B, len(edges))]
    return L.astype(np.int32)


@pytest.mark.parametrize("dt,T,B,I,H,rev", [
    ("f32", 8, 4, 16, 32, False),
    ("f32", 8, 4, 16, 32, True),
    ("f32", 64, 32, 256, 256, False),
    ("f32", 3, 100, 16, 256, True),
    ("bf16", 6, 19, 40, 72, False),
    ("bf16", 5, 60, 32, 512, True),
    ("f16", 7, 40, 64, 1024, False),
])
def test_sequence_lengths(lstm, dt, T, B, I, H, rev):
    inp = synth.make_inputs(T, B, I, H, dt, seed=107, dist=ALL)
    inp.update(lengths=ragged_lengths(T, B, 108), reverse=rev)
    say(f"case: lengths {dt} T={T} B={B} I={I} H={H} reverse={rev} lengths[:8]={inp['lengths'][:8]}")
    full_check(inp, lstm)


def test_sequence_lengths_bidirectional(lstm):
    inp = bidir_gpu_inputs("bf16", 6, 60, 32, 512, seed=109)
    inp["lengths"] = ragged_lengths(6, 60, 110)
    say("case: lengths, bidirectional")
    full_check(inp, lstm)


def test_sequence_lengths_full_size(lstm, progress):
    """T=128 B=64 I=512 H=1024 (bf16) at full size with ragged lengths,
    every output against the oracle on the whole batch."""
    name = "bf16_T128_B64_I512_H1024"
    inp = synth.workload_inputs(name)
    inp["lengths"] = ragged_lengths(inp["T"], inp["B"], 111)
    progress(f"case: lengths at full size {name}")
    out, _, _ = run_gpu(inp, lstm, torch, poison=True)
    ref = oracle.fwd_bwd(inp)
    errs, bad = compare(out, ref, "bf16")
    worst, bad_rows = compare_rows(out, ref, ROW_TOL["bf16"])
    progress("  rel-L2: " + str({k: f"{v:.2e}" for k, v in errs.items()}))
    progress("  worst row: " + str({k: f"{v:.2e}" for k, v in worst.items()}))
    assert not bad and not bad_rows, (bad, bad_rows)


def test_full_lengths_are_the_plain_path_gpu(lstm):
    """Every length >= T gives the same bits as no lengths at all."""
    inp = synth.make_inputs(5, 60, 32, 512, "bf16", seed=113, dist=ALL)
    a, _, _ = run_gpu(inp, lstm, torch)
    b, _, _ = run_gpu(dict(inp, lengths=np.full(60, 5, np.int32)), lstm, torch)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("dt,T,B,I,H,rev,lengths", [
    ("bf16", 6, 16, 64, 2048, False, False),   # the T=512 B=16 layout, short
    ("bf16", 5, 13, 40, 2048, False, False),   # a last batch group that is not full
    ("f16", 5, 16, 32, 2048, True, False),     # fp16, reverse direction
    ("bf16", 7, 16, 24, 2048, False, True),    # sequence lengths (held states travel as words too)
    ("bf16", 9, 9, 16, 1536, True, True),      # H not a power of two, both
])
def test_tagged_exchange(lstm, dt, T, B, I, H, rev, lengths):
    """The forward recurrence's tagged-word exchange (spread layout, 16-bit
    storage): h_t as words of two values and the step, polled in place."""
    code = {"bf16": lstm.BF16, "f16": lstm.F16}[dt]
    p = lstm.query_plan(lstm.make_shape(T, B, I, H, code, reverse=rev))
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("layouts are stated for 256 CUs")
    assert p["fwd_tagged"] == 1, p
    inp = synth.make_inputs(T, B, I, H, dt, seed=131, dist=contracting(H))
    inp["reverse"] = rev
    if lengths:
        inp["lengths"] = ragged_lengths(T, B, 132)
    say(f"case: tagged exchange {dt} T={T} B={B} I={I} H={H} reverse={rev} lengths={lengths} plan={p}")
    full_check(inp, lstm)
