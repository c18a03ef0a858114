"""The hand-checkable scalar case of the Darknet LSTM walkthrough (B=I=H=1,
two steps, simple weights; zero and non-zero initial state).

tests/golden/scalar_T2.json holds the oracle's values (written by
tests/golden/make_golden.py).  Here they are checked against a by-hand
scalar evaluation with Python's math module -- one named variable per
quantity of the "SingleLayerLstmGrad" page's forward table and backward
steps, no arrays -- and against the oracle as it stands now.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import oracle

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "scalar_T2.json")


def s(u):
    return 1.0 / (1.0 + math.exp(-u))


def by_hand(W, b, x, h0, c0, dy, dhT, dcT):
    (wih, wix), (wfh, wfx), (wgh, wgx), (woh, wox) = W
    bi, bf, bg, bo = b
    # step 0
    i0 = s(wih * h0 + wix * x[0] + bi)
    f0 = s(wfh * h0 + wfx * x[0] + bf)
    g0 = math.tanh(wgh * h0 + wgx * x[0] + bg)
    o0 = s(woh * h0 + wox * x[0] + bo)
    c0n = f0 * c0 + i0 * g0
    h0n = o0 * math.tanh(c0n)
    # step 1
    i1 = s(wih * h0n + wix * x[1] + bi)
    f1 = s(wfh * h0n + wfx * x[1] + bf)
    g1 = math.tanh(wgh * h0n + wgx * x[1] + bg)
    o1 = s(woh * h0n + wox * x[1] + bo)
    c1n = f1 * c0n + i1 * g1
    h1n = o1 * math.tanh(c1n)
    # backward, step 1
    dh1 = dy[1] + dhT
    dc1 = dh1 * o1 * (1 - math.tanh(c1n) ** 2) + dcT
    do1 = dh1 * math.tanh(c1n) * o1 * (1 - o1)
    dg1 = dc1 * i1 * (1 - g1 ** 2)
    di1 = dc1 * g1 * i1 * (1 - i1)
    df1 = dc1 * c0n * f1 * (1 - f1)
    dhn = wih * di1 + wfh * df1 + wgh * dg1 + woh * do1      # to h_0
    dx1 = wix * di1 + wfx * df1 + wgx * dg1 + wox * do1
    dcn = dc1 * f1
    # backward, step 0
    dh0_ = dy[0] + dhn
    dc0_ = dh0_ * o0 * (1 - math.tanh(c0n) ** 2) + dcn
    do0 = dh0_ * math.tanh(c0n) * o0 * (1 - o0)
    dg0 = dc0_ * i0 * (1 - g0 ** 2)
    di0 = dc0_ * g0 * i0 * (1 - i0)
    df0 = dc0_ * c0 * f0 * (1 - f0)
    dh_init = wih * di0 + wfh * df0 + wgh * dg0 + woh * do0
    dx0 = wix * di0 + wfx * df0 + wgx * dg0 + wox * do0
    dc_init = dc0_ * f0
    d1 = (di1, df1, dg1, do1)
    d0 = (di0, df0, dg0, do0)
    dW = [[d1[r] * h0n + d0[r] * h0, d1[r] * x[1] + d0[r] * x[0]] for r in range(4)]
    db = [d1[r] + d0[r] for r in range(4)]
    return dict(y=[h0n, h1n], hT=h1n, cT=c1n, cell=[c0n, c1n],
                gates=[[i0, f0, g0, o0], [i1, f1, g1, o1]],
                dx=[dx0, dx1], dW=dW, db=db, dh0=dh_init, dc0=dc_init)


@pytest.mark.parametrize("case", ["zero_state", "nonzero_state"])
def test_scalar_case(case):
    g = json.load(open(GOLD))
    inp, rec = g["inputs"], g["cases"][case]
    hand = by_hand(inp["W"], inp["b"], [inp["x"][0][0][0], inp["x"][1][0][0]],
                   rec["h0"][0][0], rec["c0"][0][0], [inp["dy"][0][0][0], inp["dy"][1][0][0]],
                   inp["dhT"][0][0], inp["dcT"][0][0])
    stored = dict(y=np.ravel(rec["y"]), hT=rec["hT"][0][0], cT=rec["cT"][0][0],
                  cell=np.ravel(rec["cell"]), gates=np.array(rec["gates"]).reshape(2, 4),
                  dx=np.ravel(rec["dx"]), dW=np.array(rec["dW"]), db=np.array(rec["db"]),
                  dh0=rec["dh0"][0][0], dc0=rec["dc0"][0][0])
    for k, v in hand.items():
        np.testing.assert_allclose(stored[k], v, rtol=1e-14, atol=1e-16, err_msg=k)
    # the oracle as it stands reproduces the stored values
    a = {k: np.array(v, dtype=np.float64) for k, v in inp.items()}
    h0, c0 = np.array(rec["h0"]), np.array(rec["c0"])
    fw = oracle.fwd(a["x"], a["W"], a["b"], h0, c0)
    bw = oracle.bwd(a["x"], a["W"], h0, c0, fw, a["dy"], a["dhT"], a["dcT"])
    np.testing.assert_array_equal(fw["y"].ravel(), stored["y"])
    np.testing.assert_array_equal(bw["dW"], stored["dW"])
    np.testing.assert_array_equal(bw["dx"].ravel(), stored["dx"])


def test_nonzero_state_changes_first_step():
    """The initial state enters step 0 (no leakage check would be possible
    otherwise): the two cases differ in y_0."""
    g = json.load(open(GOLD))
    assert g["cases"]["zero_state"]["y"][0] != g["cases"]["nonzero_state"]["y"][0]
