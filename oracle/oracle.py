"""ctypes wrapper around the fp64 CPU oracle (``lstm_oracle.c``).

TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the CPU-baseline
leg of ``bench.py`` are the only callers.  Nothing here imports the HIP
library or its Python binding, and the HIP path never imports this module.

The oracle follows the forward table and the backward recursion of the
"SingleLayerLstmGrad" operator page (Ascend CANN ops-nn); see the header of
``lstm_oracle.c`` for the conventions (gate order i,f,g,o in W's row blocks,
columns [h | x], time-major tensors, the forget factor applied once in the
cell carry).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lstm_oracle.c")
_LIB = os.path.join(_HERE, "liblstm_oracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-std=c99", "-shared", "-fPIC",
                               "-Wall", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _bind(path):
    lib = ctypes.CDLL(path)
    L, P = ctypes.c_long, ctypes.c_void_p
    lib.oracle_lstm_fwd.argtypes = [L, L, L, L, ctypes.c_int] + [P] * 10
    lib.oracle_lstm_fwd.restype = ctypes.c_int
    lib.oracle_lstm_bwd.argtypes = [L, L, L, L, ctypes.c_int] + [P] * 18
    lib.oracle_lstm_bwd.restype = ctypes.c_int
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    return lib


def _load():
    global _lib
    if _lib is None:
        build()
        _lib = _bind(_LIB)
    return _lib


def use_library(path):
    """Point this module at another build of the oracle source (the mutation
    test builds deliberately broken copies); returns the previous handle so
    that the caller can restore it with ``restore_library``."""
    global _lib
    prev = _load()
    _lib = _bind(path)
    return prev


def restore_library(handle):
    global _lib
    _lib = handle


def num_threads() -> int:
    return _load().oracle_num_threads()


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def _f64(a, shape=None):
    if a is None:
        return None
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    if shape is not None and a.shape != tuple(shape):
        raise ValueError(f"expected shape {tuple(shape)}, got {a.shape}")
    return a


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def fwd(x, W, b=None, h0=None, c0=None, reverse=False, mask=None):
    """Forward pass.  Returns dict(y, hT, cT, gates, cell) as fp64 arrays.

    x [T,B,I], W [4H,H+I], b [4H] or None, h0/c0 [B,H] or None (zero state).
    gates is [T,B,4H] (activated i,f,g,o blocks), cell is c_t, [T,B,H].
    reverse: the steps run from t = T-1 down to 0 (the operator's reverse
    direction); tensors keep their time-major layout.
    mask: [T,B,H] or None, the seq_length mask matrix (see lstm_oracle.c:
    the state is blended with the step's new values, m = 0 keeps it).
    """
    x = _f64(x)
    T, B, I = x.shape
    H = W.shape[0] // 4
    W = _f64(W, (4 * H, H + I))
    b = _f64(b, (4 * H,))
    h0 = _f64(h0, (B, H))
    c0 = _f64(c0, (B, H))
    mask = _f64(mask, (T, B, H))
    y = np.empty((T, B, H))
    hT = np.empty((B, H))
    cT = np.empty((B, H))
    gates = np.empty((T, B, 4 * H))
    cell = np.empty((T, B, H))
    rc = _load().oracle_lstm_fwd(T, B, I, H, int(bool(reverse)), _p(x), _p(W), _p(b), _p(h0), _p(c0), _p(mask),
                                 _p(y), _p(hT), _p(cT), _p(gates), _p(cell))
    if rc != 0:
        raise RuntimeError(f"oracle_lstm_fwd failed ({rc})")
    return dict(y=y, hT=hT, cT=cT, gates=gates, cell=cell)


def bwd(x, W, h0, c0, fw, dy, dhT=None, dcT=None, want_debug=False, reverse=False, mask=None):
    """Backward pass from the forward record ``fw`` (the dict ``fwd`` returns,
    with the same ``reverse`` and ``mask``).

    Returns dict(dx, dW, db, dh0, dc0) and, with want_debug, also dgates
    [T,B,4H] (gate deltas) and dcell [T,B,H] (cell gradient per step).
    """
    x = _f64(x)
    T, B, I = x.shape
    H = W.shape[0] // 4
    W = _f64(W, (4 * H, H + I))
    h0 = _f64(h0, (B, H))
    c0 = _f64(c0, (B, H))
    dy = _f64(dy, (T, B, H))
    dhT = _f64(dhT, (B, H))
    dcT = _f64(dcT, (B, H))
    mask = _f64(mask, (T, B, H))
    y, gates, cell = (_f64(fw[k]) for k in ("y", "gates", "cell"))
    dx = np.empty((T, B, I))
    dW = np.empty((4 * H, H + I))
    db = np.empty((4 * H,))
    dh0 = np.empty((B, H))
    dc0 = np.empty((B, H))
    dgates = np.empty((T, B, 4 * H)) if want_debug else None
    dcell = np.empty((T, B, H)) if want_debug else None
    rc = _load().oracle_lstm_bwd(T, B, I, H, int(bool(reverse)), _p(x), _p(W), _p(h0), _p(c0), _p(mask),
                                 _p(y), _p(gates), _p(cell), _p(dy), _p(dhT), _p(dcT),
                                 _p(dx), _p(dW), _p(db), _p(dh0), _p(dc0),
                                 _p(dgates), _p(dcell))
    if rc != 0:
        raise RuntimeError(f"oracle_lstm_bwd failed ({rc})")
    out = dict(dx=dx, dW=dW, db=db, dh0=dh0, dc0=dc0)
    if want_debug:
        out.update(dgates=dgates, dcell=dcell)
    return out


def ifjo_rows(H: int, gate_order: str):
    """Row index map from the i, f, g, o block order to `gate_order`'s: W in
    the "ijfo" order (blocks i, g, f, o) is W_ifjo[ifjo_rows(H, "ijfo")].  The
    two orders are the values of the gate_order attribute of the
    SingleLayerLstmGrad page (参数说明); the map is its own inverse."""
    blocks = {"ifjo": (0, 1, 2, 3), "ijfo": (0, 2, 1, 3)}[gate_order]
    return np.concatenate([np.arange(H) + g * H for g in blocks])


def length_mask(lengths, T, H):
    """The seq_length mask matrix [T,B,H] of per-sequence lengths: 1 at the
    steps t < lengths[b] of sequence b, 0 past its end (lengths outside
    [0, T] are taken as the nearest end of that range)."""
    L = np.clip(np.asarray(lengths, dtype=np.int64), 0, T)
    m = (np.arange(T)[:, None] < L[None, :]).astype(np.float64)
    return np.repeat(m[:, :, None], H, axis=2)


def fwd_bwd(inp: dict) -> dict:
    """Run forward then backward on an input dict with keys
    x, W, b, h0, c0, dy, dhT, dcT (values may be None where optional) and
    optionally reverse (default False), gate_order ("ifjo", the oracle's
    own order, or "ijfo": W, b, dW and db with their row blocks relabelled),
    two_bias (b and db [2][4H]), mask ([T,B,H], the seq_length mask matrix)
    or lengths ([B], turned into that mask by length_mask), and
    bidirectional (see below)."""
    if inp.get("layers"):
        return stacked_fwd_bwd(inp)
    if inp.get("bidirectional"):
        # Two directions of one layer: direction 0 runs forward in time and
        # direction 1 in reverse, each with its own W, b and initial state
        # ([2][...] of the one-direction shapes), on the same x; the output
        # at time t is the two directions' h_t side by side ([T,B,2H]) and
        # the final states are [2][B][H] -- the num_directions layout of the
        # PyTorch recurrent-layer page.  dy [T,B,2H] splits the same way;
        # dx is the sum of the two directions' input gradients (x feeds
        # both).
        H = inp["W"].shape[1] // 4
        outs = []
        for d in range(2):
            sub = dict(inp, bidirectional=False, reverse=bool(d), W=inp["W"][d],
                       b=None if inp.get("b") is None else inp["b"][d],
                       dy=inp["dy"][:, :, d * H:(d + 1) * H])
            for k in ("h0", "c0", "dhT", "dcT"):
                sub[k] = None if inp.get(k) is None else inp[k][d]
            outs.append(fwd_bwd(sub))
        out = {"y": np.concatenate([outs[0]["y"], outs[1]["y"]], axis=2), "dx": outs[0]["dx"] + outs[1]["dx"]}
        for k in ("hT", "cT", "dW", "db", "dh0", "dc0"):
            out[k] = np.stack([outs[0][k], outs[1][k]])
        return out
    if inp.get("lengths") is not None and inp.get("mask") is None:
        x = inp["x"]
        return fwd_bwd(dict(inp, lengths=None, mask=length_mask(inp["lengths"], x.shape[0], inp["W"].shape[0] // 4)))
    if inp.get("two_bias"):
        # b = [b_ih; b_hh] enter the pre-activation as their sum (bias_ih and
        # bias_hh of the CMU 10-414 HW4 page's LSTMCell); both receive the one
        # bias gradient
        b2 = inp["b"]
        out = fwd_bwd(dict(inp, two_bias=False, b=None if b2 is None else b2[0] + b2[1]))
        out["db"] = np.stack([out["db"], out["db"]])
        return out
    order = inp.get("gate_order", "ifjo")
    if order != "ifjo":
        H = inp["W"].shape[0] // 4
        rows = ifjo_rows(H, order)
        sub = dict(inp, gate_order="ifjo", W=inp["W"][rows], b=None if inp.get("b") is None else inp["b"][rows])
        out = fwd_bwd(sub)
        out["dW"] = out["dW"][rows]
        out["db"] = out["db"][rows]
        return out
    rev = bool(inp.get("reverse", False))
    mask = inp.get("mask")
    fw = fwd(inp["x"], inp["W"], inp.get("b"), inp.get("h0"), inp.get("c0"), reverse=rev, mask=mask)
    bw = bwd(inp["x"], inp["W"], inp.get("h0"), inp.get("c0"), fw, inp["dy"],
             inp.get("dhT"), inp.get("dcT"), reverse=rev, mask=mask)
    out = {k: fw[k] for k in ("y", "hT", "cT")}
    out.update(bw)
    return out


def stacked_fwd_bwd(inp: dict) -> dict:
    """A stack of inp["layers"] = L one-direction layers (the MXNet page's
    "Stack Multiple RNN Cells": the output sequence of a layer is the input
    sequence of the next, each layer with its own initial state; the CMU
    10-414 page's LSTM module with num_layers: h0, c0 and h_n, c_n of shape
    [num_layers, B, H], the output the last layer's).

    W is the list of the L weight matrices (layer 0 [4H, H+I], the others
    [4H, 2H]), b the list of the L biases or None; h0, c0, dhT, dcT are
    [L][B][H] or None; x [T,B,I]; dy [T,B,H] is the cotangent of the last
    layer's output.  The backward runs the layers from the last to the
    first; the input gradient of layer l is the output cotangent of layer
    l - 1 (only the last layer's output is the stack's output).  Returns y
    (the last layer's), hT, cT, dh0, dc0 as [L][B][H], dx, and dW, db as
    lists of the L layers' gradients."""
    L = int(inp["layers"])
    x = inp["x"]
    layer_in, fws, subs = x, [], []
    for ll in range(L):
        sub = dict(inp, layers=None, x=layer_in, W=inp["W"][ll], b=None if inp.get("b") is None else inp["b"][ll])
        for k in ("h0", "c0", "dhT", "dcT"):
            sub[k] = None if inp.get(k) is None else inp[k][ll]
        fw = fwd(sub["x"], sub["W"], sub["b"], sub["h0"], sub["c0"])
        fws.append(fw)
        subs.append(sub)
        layer_in = fw["y"]
    out = {"y": fws[-1]["y"], "hT": np.stack([f["hT"] for f in fws]), "cT": np.stack([f["cT"] for f in fws])}
    dy = inp["dy"]
    bws = [None] * L
    for ll in range(L - 1, -1, -1):
        sub = subs[ll]
        bws[ll] = bwd(sub["x"], sub["W"], sub["h0"], sub["c0"], fws[ll], dy, sub["dhT"], sub["dcT"])
        dy = bws[ll]["dx"]
    out["dx"] = bws[0]["dx"]
    out["dW"] = [b["dW"] for b in bws]
    out["db"] = np.stack([b["db"] for b in bws])
    out["dh0"] = np.stack([b["dh0"] for b in bws])
    out["dc0"] = np.stack([b["dc0"] for b in bws])
    return out
