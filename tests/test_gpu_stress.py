"""Randomised shapes at the edges of the envelope (-m gpu).

Seeded draws of storage type, T, B, I, H (odd, non-power-of-two and
maximal hidden sizes, no input features, one step, batches that leave a
group ragged) and of every flag (reverse direction, "ijfo", two biases,
bidirectional, sequence lengths).  Each case runs forward + backward twice:
the two runs must agree bit for bit (the step exchange and every fixed-order
sum leave no room for scheduling to change a result), and the first must
match the fp64 oracle within the storage type's bound, whole tensor and row
by row.  The draw lands on every recurrence form the plan can pick (VALU
and MFMA, XCD-local and spread, flags and tagged words) without naming
them; each case prints its plan.
"""
import numpy as np
import pytest
import torch

from layer_lstm_amd import synth
from oracle import oracle
from parity_util import OUTPUTS, ROW_TOL, compare, compare_rows, run_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lstm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from layer_lstm_amd import lstm as mod
    return mod


ALL = dict(W=("u", 0.3), b=("u", 0.3), x=("n", 1.0), h0=("n", 0.5), c0=("n", 0.5), dy=("n", 1.0),
           dhT=("n", 1.0), dcT=("n", 1.0))
H_CHOICES = (1, 7, 32, 48, 72, 96, 130, 256, 512, 768, 1024, 1536, 2048)
B_CHOICES = (1, 3, 4, 5, 16, 17, 31, 32, 33, 60, 64, 96, 128)
I_CHOICES = (0, 1, 16, 40, 64, 200)
MAX_WORK = 3e8  # T * B * directions * 4H * (H + I): a second or two of oracle time


def inside_envelope(dt, B, H):
    """The shapes lstm_query accepts on 256 CUs (include/lstm.h): fp32 up to
    H = 512 at any batch here, H = 1024 up to B = 8; 16-bit storage up to
    H = 1024 at any batch here, H = 2048 up to B = 32."""
    if dt == "f32":
        return H <= 512 or (H <= 1024 and B <= 8)
    return H <= 1024 or (H <= 2048 and B <= 32)


def draw_cases(n=16, seed=2026):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        dt = str(rng.choice(["f32", "bf16", "f16"]))
        H = int(rng.choice(H_CHOICES))
        B = int(rng.choice(B_CHOICES))
        I = int(rng.choice(I_CHOICES))
        T = 1 if rng.random() < 0.1 else int(rng.integers(2, 24))
        bidir = bool(rng.random() < 0.2)
        rev = (not bidir) and bool(rng.random() < 0.35)
        ijfo = bool(rng.random() < 0.3)
        two = (not bidir) and bool(rng.random() < 0.3)
        lengths = bool(rng.random() < 0.3)
        dirs = 2 if bidir else 1
        while T * B * dirs * 4 * H * (H + I) > MAX_WORK and B > 1:
            B = max(1, B // 2)
        if T * B * dirs * 4 * H * (H + I) > MAX_WORK or not inside_envelope(dt, B, H):
            continue
        cases.append((len(cases), dt, T, B, I, H, rev, ijfo, two, bidir, lengths))
    return cases


def make_case(dt, T, B, I, H, rev, ijfo, two, bidir, lengths, seed):
    # U(+-1/sqrt(H)) from H = 64 up: the wider U(+-0.3) makes the recurrence
    # chaotic there over a few dozen steps (rounding grows alike on both sides)
    dist = ALL if H < 64 else dict(ALL, W=("u", 1.0 / np.sqrt(H)), b=("u", 1.0 / np.sqrt(H)))
    a = synth.make_inputs(T, B, I, H, dt, seed=seed, dist=dist)
    inp = dict(a)
    if bidir:
        c = synth.make_inputs(T, B, I, H, dt, seed=seed + 1000, dist=dist)
        inp = dict(a, bidirectional=True, dy=np.concatenate([a["dy"], c["dy"]], axis=2))
        for k in ("W", "b", "h0", "c0", "dhT", "dcT"):
            inp[k] = None if a[k] is None else np.stack([a[k], c[k]])
    if two:
        rng = np.random.default_rng(seed + 1)
        b_hh = synth.round_to_storage(rng.uniform(-0.3, 0.3, 4 * H), dt)
        inp["b"] = np.stack([inp["b"], b_hh])
        inp["two_bias"] = True
    inp["reverse"] = rev
    inp["gate_order"] = "ijfo" if ijfo else "ifjo"
    if lengths:
        rng = np.random.default_rng(seed + 2)
        L = rng.integers(0, T + 2, size=B)
        L[0] = T
        inp["lengths"] = L.astype(np.int32)
    return inp


# The envelope's edges, next to the draw: the largest hidden size of each
# storage type at its largest batch, one step of one row of one unit, and a
# wide batch.
EDGES = [
    (100, "bf16", 4, 32, 16, 2048, False, False, False, False, False),
    (101, "f16", 3, 32, 0, 2048, True, True, False, False, True),
    (102, "f32", 3, 8, 40, 1024, False, False, True, False, False),
    (103, "f32", 4, 64, 24, 512, True, False, False, False, True),
    (104, "bf16", 1, 1, 0, 1, False, False, False, False, False),
    (105, "f16", 2, 256, 8, 64, False, True, True, False, False),
]


@pytest.mark.parametrize("case", draw_cases() + EDGES, ids=lambda c: f"case{c[0]}")
def test_random_shape(lstm, case):
    i, dt, T, B, I, H, rev, ijfo, two, bidir, lengths = case
    code = {"f32": lstm.F32, "bf16": lstm.BF16, "f16": lstm.F16}[dt]
    plan = lstm.query_plan(lstm.make_shape(T, B, I, H, code, reverse=rev, gate_order="ijfo" if ijfo else "ifjo",
                                           two_bias=two, bidirectional=bidir))
    print(f"case{i}: {dt} T={T} B={B} I={I} H={H} reverse={rev} ijfo={ijfo} two_bias={two} "
          f"bidirectional={bidir} lengths={lengths} plan={plan}", flush=True)
    inp = make_case(dt, T, B, I, H, rev, ijfo, two, bidir, lengths, seed=500 + i)
    first, _, _ = run_gpu(inp, lstm, torch, poison=True)
    again, _, _ = run_gpu(inp, lstm, torch, poison=True)
    for k in OUTPUTS:
        np.testing.assert_array_equal(first[k], again[k], err_msg=f"{k} differs between two runs")
    ref = oracle.fwd_bwd(inp)
    errs, bad = compare(first, ref, dt)
    worst, bad_rows = compare_rows(first, ref, ROW_TOL[dt])
    print("  rel-L2:", {k: f"{v:.1e}" for k, v in errs.items()}, flush=True)
    assert not bad, bad
    assert not bad_rows, bad_rows
