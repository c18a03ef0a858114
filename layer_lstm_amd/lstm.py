"""Thin ctypes binding of liblstm.so (include/lstm.h).

Argument marshalling only: every step of the forward and backward pass runs
in the library's HIP kernels.  torch is used for device memory and streams
(it is imported before the library so that both share one HIP runtime).
There is no fallback: if liblstm.so is missing or cannot be loaded, importing
this module raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblstm.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python -m layer_lstm_amd.build`")
_lib = ctypes.CDLL(LIB_PATH)

# --- constants restated from include/lstm.h ---------------------------------
ABI_VERSION = 3
REVERSE = 1  # lstm_shape.flags: the reverse direction of time
GATES_IJFO = 2  # lstm_shape.flags: W/b/dW/db row blocks in the gate order i, g, f, o
TWO_BIAS = 4  # lstm_shape.flags: b and db are [2][4H] (b_ih, b_hh)
BIDIRECTIONAL = 8  # lstm_shape.flags: both directions of time, outputs side by side
GATE_I, GATE_F, GATE_G, GATE_O = 0, 1, 2, 3
F32, BF16, F16 = 0, 1, 2
OK = 0
STATUS = {0: "OK", -1: "ERR_NULL", -2: "ERR_DIMS", -3: "ERR_DTYPE", -4: "ERR_ALIGN",
          -5: "ERR_WORKSPACE", -6: "ERR_UNSUPPORTED", -7: "ERR_COOP", -8: "ERR_LAUNCH",
          -9: "ERR_TIMEOUT", -10: "ERR_DEVICE", -11: "ERR_SCRATCH", -12: "ERR_PLACEMENT",
          -13: "ERR_STATE"}
DEBUG_FAIL_STEP, DEBUG_MISPLACE, DEBUG_XCD_LOCAL = 1, 2, 3  # lstm_debug_inject
PROBE_READS, PROBE_READS_AHEAD, PROBE_BARRIER, PROBE_DMA = 1, 2, 4, 8  # lstm_probe_mfma_stage
PROBE_SCRATCH_BYTES = 1 << 20  # LSTM_PROBE_SCRATCH_BYTES
SCRATCH_BYTES = 64 << 20  # LSTM_SCRATCH_BYTES
EXPORTS = ("lstm_abi_version", "lstm_status_string", "lstm_query", "lstm_query_plan", "lstm_fwd_train",
           "lstm_fwd_train_scratch", "lstm_bwd", "lstm_check_workspace", "lstm_timing_enable", "lstm_timing_read",
           "lstm_stamps_set", "lstm_probe_exchange", "lstm_probe_mfma_stage", "lstm_debug_inject", "lstm_stack_query",
           "lstm_stack_fwd_train", "lstm_stack_bwd")
STAMP_WGS, STAMP_POINTS = 8, 6
KERNEL_KINDS = ("input_projection", "forward_recurrence", "backward_recurrence", "dW_product",
                "dx_product", "direction_copy", "state_copy")


class Shape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("B", ctypes.c_int64), ("I", ctypes.c_int64),
                ("H", ctypes.c_int64), ("dtype", ctypes.c_int32), ("flags", ctypes.c_int32)]


class PlanInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("rows_per_group", "units_per_group", "groups", "units_groups",
                                               "grid", "waves", "xcd_local", "fwd_valu", "bwd_valu",
                                               "inproj_tiles_per_wg", "directions_concurrent", "fwd_tagged")] + \
               [("reserved", ctypes.c_int32 * 4)]


_P = ctypes.c_void_p
_lib.lstm_abi_version.restype = ctypes.c_int
_lib.lstm_status_string.restype = ctypes.c_char_p
_lib.lstm_status_string.argtypes = [ctypes.c_int]
_lib.lstm_query.restype = ctypes.c_int
_lib.lstm_query.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(ctypes.c_size_t)]
_lib.lstm_query_plan.restype = ctypes.c_int
_lib.lstm_query_plan.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(PlanInfo)]
_lib.lstm_fwd_train.restype = ctypes.c_int
_lib.lstm_fwd_train.argtypes = [ctypes.POINTER(Shape)] + [_P] * 9 + [_P, ctypes.c_size_t, _P]
_lib.lstm_fwd_train_scratch.restype = ctypes.c_int
_lib.lstm_fwd_train_scratch.argtypes = [ctypes.POINTER(Shape)] + [_P] * 9 + [_P]
_lib.lstm_bwd.restype = ctypes.c_int
_lib.lstm_bwd.argtypes = [ctypes.POINTER(Shape)] + [_P] * 9 + [_P, ctypes.c_size_t] + [_P] * 5 + [_P]
_lib.lstm_check_workspace.restype = ctypes.c_int
_lib.lstm_check_workspace.argtypes = [_P, ctypes.c_size_t, _P]
_lib.lstm_timing_enable.restype = ctypes.c_int
_lib.lstm_timing_enable.argtypes = [ctypes.c_int]
_lib.lstm_timing_read.restype = ctypes.c_int
_lib.lstm_timing_read.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
_lib.lstm_probe_exchange.restype = ctypes.c_int
_lib.lstm_probe_exchange.argtypes = [ctypes.POINTER(Shape), ctypes.c_int, _P, ctypes.c_size_t,
                                     ctypes.POINTER(ctypes.c_double), _P]
_lib.lstm_probe_mfma_stage.restype = ctypes.c_int
_lib.lstm_probe_mfma_stage.argtypes = [ctypes.c_int, ctypes.c_int64, _P, ctypes.c_size_t,
                                       ctypes.POINTER(ctypes.c_double), _P]
_lib.lstm_stack_query.restype = ctypes.c_int
_lib.lstm_stack_query.argtypes = [ctypes.POINTER(Shape), ctypes.c_int64, ctypes.c_int64,
                                  ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_int32)]
_lib.lstm_stack_fwd_train.restype = ctypes.c_int
_lib.lstm_stack_fwd_train.argtypes = [ctypes.POINTER(Shape), ctypes.c_int64, ctypes.c_int64] + [_P] * 8 + \
    [_P, ctypes.c_size_t, _P]
_lib.lstm_stack_bwd.restype = ctypes.c_int
_lib.lstm_stack_bwd.argtypes = [ctypes.POINTER(Shape), ctypes.c_int64, ctypes.c_int64] + [_P] * 8 + \
    [_P, ctypes.c_size_t] + [_P] * 5 + [_P]
_lib.lstm_debug_inject.restype = ctypes.c_int
_lib.lstm_debug_inject.argtypes = [ctypes.c_int, ctypes.c_int64]
_lib.lstm_stamps_set.restype = ctypes.c_int
_lib.lstm_stamps_set.argtypes = [_P, ctypes.c_size_t, ctypes.c_int64]


class LstmError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        msg = _lib.lstm_status_string(code).decode()
        super().__init__(f"{where}: {STATUS.get(code, code)} ({msg})")


def lib():
    return _lib


def abi_version() -> int:
    return _lib.lstm_abi_version()


def status_string(code: int) -> str:
    return _lib.lstm_status_string(code).decode()


def torch_dtype(dtype: int):
    return {F32: torch.float32, BF16: torch.bfloat16, F16: torch.float16}[dtype]


def make_shape(T, B, I, H, dtype, reverse=False, gate_order="ifjo", two_bias=False, bidirectional=False) -> Shape:
    if gate_order not in ("ifjo", "ijfo"):
        raise ValueError(f"gate_order {gate_order!r}: 'ifjo' or 'ijfo'")
    flags = (REVERSE if reverse else 0) | (GATES_IJFO if gate_order == "ijfo" else 0) | \
        (TWO_BIAS if two_bias else 0) | (BIDIRECTIONAL if bidirectional else 0)
    return Shape(int(T), int(B), int(I), int(H), int(dtype), flags)


def query(shape: Shape) -> int:
    n = ctypes.c_size_t(0)
    rc = _lib.lstm_query(ctypes.byref(shape), ctypes.byref(n))
    if rc != OK:
        raise LstmError(rc, "lstm_query")
    return n.value


def query_plan(shape: Shape) -> dict:
    """Layout of the persistent recurrences for `shape` (lstm_query_plan)."""
    info = PlanInfo()
    rc = _lib.lstm_query_plan(ctypes.byref(shape), ctypes.byref(info))
    if rc != OK:
        raise LstmError(rc, "lstm_query_plan")
    return {n: getattr(info, n) for n, _ in PlanInfo._fields_ if n != "reserved"}


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr() if t.numel() > 0 else None


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def fwd_train(shape, x, W, b, h0, c0, y, hT, cT, workspace, ws_bytes=None, stream=None, check=True,
              seq_length=None):
    """lstm_fwd_train on torch tensors (None = NULL; seq_length: int32 [B]
    device tensor of sequence lengths).  Returns the status."""
    if ws_bytes is None:
        ws_bytes = workspace.numel() * workspace.element_size()
    rc = _lib.lstm_fwd_train(ctypes.byref(shape), _ptr(x), _ptr(W), _ptr(b), _ptr(h0), _ptr(c0),
                             _ptr(seq_length), _ptr(y), _ptr(hT), _ptr(cT), _ptr(workspace), ws_bytes,
                             _stream(stream))
    if check and rc != OK:
        raise LstmError(rc, "lstm_fwd_train")
    return rc


def fwd_train_scratch(shape, x, W, b, h0, c0, y, hT, cT, stream=None, check=True, seq_length=None):
    """lstm_fwd_train_scratch on torch tensors (None = NULL): the forward
    pass with the library's own device array as the workspace.  Returns the
    status."""
    rc = _lib.lstm_fwd_train_scratch(ctypes.byref(shape), _ptr(x), _ptr(W), _ptr(b), _ptr(h0), _ptr(c0),
                                     _ptr(seq_length), _ptr(y), _ptr(hT), _ptr(cT), _stream(stream))
    if check and rc != OK:
        raise LstmError(rc, "lstm_fwd_train_scratch")
    return rc


def bwd(shape, dy, dhT, dcT, x, W, h0, c0, y, workspace, dx, dW, db, dh0, dc0, ws_bytes=None,
        stream=None, check=True, seq_length=None):
    """lstm_bwd on torch tensors (None = NULL).  Returns the status."""
    if ws_bytes is None:
        ws_bytes = workspace.numel() * workspace.element_size()
    rc = _lib.lstm_bwd(ctypes.byref(shape), _ptr(dy), _ptr(dhT), _ptr(dcT), _ptr(x), _ptr(W),
                       _ptr(h0), _ptr(c0), _ptr(seq_length), _ptr(y), _ptr(workspace), ws_bytes, _ptr(dx),
                       _ptr(dW), _ptr(db), _ptr(dh0), _ptr(dc0), _stream(stream))
    if check and rc != OK:
        raise LstmError(rc, "lstm_bwd")
    return rc


def check_workspace(workspace, stream=None) -> int:
    return _lib.lstm_check_workspace(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                     _stream(stream))


def timing_enable(on: bool) -> None:
    _lib.lstm_timing_enable(1 if on else 0)


def timing_read() -> dict:
    """{kind name: (total ms, launches)} of the per-kernel event timing."""
    out = {}
    for k, name in enumerate(KERNEL_KINDS):
        ms, n = ctypes.c_double(0), ctypes.c_int64(0)
        rc = _lib.lstm_timing_read(k, ctypes.byref(ms), ctypes.byref(n))
        if rc != OK:
            raise LstmError(rc, "lstm_timing_read")
        out[name] = (ms.value, n.value)
    return out


def probe_exchange(shape: Shape, workspace, layout: int = 0, stream=None) -> float:
    """lstm_probe_exchange: microseconds per step of the forward
    recurrence's exchange alone (layout 0: the plan's own; 1: spread over
    the XCDs)."""
    us = ctypes.c_double(0)
    rc = _lib.lstm_probe_exchange(ctypes.byref(shape), int(layout), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), ctypes.byref(us), _stream(stream))
    if rc != OK:
        raise LstmError(rc, "lstm_probe_exchange")
    return us.value


def probe_mfma_stage(parts: int, scratch, iters: int = 4000, stream=None) -> float:
    """lstm_probe_mfma_stage: fraction of the bf16 dense peak of 32 MFMAs
    per wave and iteration with the stage parts `parts` (PROBE_* bits);
    scratch: device memory of at least PROBE_SCRATCH_BYTES."""
    frac = ctypes.c_double(0)
    rc = _lib.lstm_probe_mfma_stage(int(parts), int(iters), _ptr(scratch), scratch.numel() * scratch.element_size(),
                                    ctypes.byref(frac), _stream(stream))
    if rc != OK:
        raise LstmError(rc, "lstm_probe_mfma_stage")
    return frac.value


def debug_inject(what: int, value: int) -> None:
    """lstm_debug_inject: the test hooks of the failure paths."""
    rc = _lib.lstm_debug_inject(int(what), int(value))
    if rc != OK:
        raise LstmError(rc, "lstm_debug_inject")


def stamps_set(buf, T) -> None:
    """Point the recurrent kernels' phase stamps at a device tensor of at
    least 2*8*T*6 int64 values (None disables)."""
    if buf is None:
        _lib.lstm_stamps_set(None, 0, 0)
        return
    rc = _lib.lstm_stamps_set(_ptr(buf), buf.numel() * buf.element_size(), int(T))
    if rc != OK:
        raise LstmError(rc, "lstm_stamps_set")


class Lstm:
    """One problem shape with its workspace and output buffers on the current
    device.  ``forward``/``backward`` take device tensors and return device
    tensors; nothing is synchronised."""

    def __init__(self, T, B, I, H, dtype=F32, device="cuda", reverse=False, gate_order="ifjo", two_bias=False,
                 bidirectional=False):
        self.shape = make_shape(T, B, I, H, dtype, reverse, gate_order, two_bias, bidirectional)
        self.T, self.B, self.I, self.H, self.dtype = T, B, I, H, dtype
        self.tdtype = torch_dtype(dtype)
        self.ws_bytes = query(self.shape)
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        dev, td = device, self.tdtype
        nd = (2,) if bidirectional else ()
        self.y = torch.empty((T, B, 2 * H if bidirectional else H), dtype=td, device=dev)
        self.hT = torch.empty(nd + (B, H), dtype=td, device=dev)
        self.cT = torch.empty(nd + (B, H), dtype=td, device=dev)
        self.dx = torch.empty((T, B, I), dtype=td, device=dev)
        self.dW = torch.empty(nd + (4 * H, H + I), dtype=td, device=dev)
        self.db = torch.empty(nd + ((2, 4 * H) if two_bias else (4 * H,)), dtype=td, device=dev)
        self.dh0 = torch.empty(nd + (B, H), dtype=td, device=dev)
        self.dc0 = torch.empty(nd + (B, H), dtype=td, device=dev)

    def forward(self, x, W, b=None, h0=None, c0=None, stream=None, seq_length=None):
        fwd_train(self.shape, x, W, b, h0, c0, self.y, self.hT, self.cT, self.workspace,
                  self.ws_bytes, stream, seq_length=seq_length)
        return self.y, self.hT, self.cT

    def backward(self, dy, dhT, dcT, x, W, h0=None, c0=None, want_db=True, stream=None, seq_length=None):
        bwd(self.shape, dy, dhT, dcT, x, W, h0, c0, self.y, self.workspace, self.dx, self.dW,
            self.db if want_db else None, self.dh0, self.dc0, self.ws_bytes, stream, seq_length=seq_length)
        return self.dx, self.dW, self.db, self.dh0, self.dc0

    def check(self, stream=None):
        rc = check_workspace(self.workspace, stream)
        if rc != OK:
            raise LstmError(rc, "lstm_check_workspace")


def stack_query(shape: Shape, layers: int, chunks: int = 0):
    """lstm_stack_query: (workspace bytes, the most layers whose
    recurrences share one launch; 1: one after the other)."""
    n, conc = ctypes.c_size_t(0), ctypes.c_int32(0)
    rc = _lib.lstm_stack_query(ctypes.byref(shape), int(layers), int(chunks), ctypes.byref(n), ctypes.byref(conc))
    if rc != OK:
        raise LstmError(rc, "lstm_stack_query")
    return n.value, conc.value


class Stack:
    """An L-layer stack (lstm_stack_*) of one problem shape with its
    workspace and output buffers on the current device.  W is the layers'
    weights back to back (layer 0 [4H][H+I], the others [4H][2H]); b, h0, c0,
    dhT, dcT have a leading layer axis."""

    def __init__(self, T, B, I, H, layers, dtype=F32, chunks=0, device="cuda", gate_order="ifjo", two_bias=False):
        self.shape = make_shape(T, B, I, H, dtype, False, gate_order, two_bias)
        self.T, self.B, self.I, self.H, self.L, self.chunks = T, B, I, H, layers, chunks
        self.tdtype = torch_dtype(dtype)
        self.ws_bytes, self.concurrent = stack_query(self.shape, layers, chunks)
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        dev, td, L = device, self.tdtype, layers
        self.w_elems = 4 * H * (H + I) + (L - 1) * 4 * H * 2 * H
        self.y = torch.empty((T, B, H), dtype=td, device=dev)
        self.hT = torch.empty((L, B, H), dtype=td, device=dev)
        self.cT = torch.empty((L, B, H), dtype=td, device=dev)
        self.dx = torch.empty((T, B, I), dtype=td, device=dev)
        self.dW = torch.empty((self.w_elems,), dtype=td, device=dev)
        self.db = torch.empty((L, 2, 4 * H) if two_bias else (L, 4 * H), dtype=td, device=dev)
        self.dh0 = torch.empty((L, B, H), dtype=td, device=dev)
        self.dc0 = torch.empty((L, B, H), dtype=td, device=dev)

    def forward(self, x, W, b=None, h0=None, c0=None, stream=None):
        rc = _lib.lstm_stack_fwd_train(ctypes.byref(self.shape), self.L, self.chunks, _ptr(x), _ptr(W), _ptr(b),
                                       _ptr(h0), _ptr(c0), _ptr(self.y), _ptr(self.hT), _ptr(self.cT),
                                       _ptr(self.workspace), self.ws_bytes, _stream(stream))
        if rc != OK:
            raise LstmError(rc, "lstm_stack_fwd_train")
        return self.y, self.hT, self.cT

    def backward(self, dy, dhT, dcT, x, W, h0=None, c0=None, want_db=True, stream=None):
        rc = _lib.lstm_stack_bwd(ctypes.byref(self.shape), self.L, self.chunks, _ptr(dy), _ptr(dhT), _ptr(dcT),
                                 _ptr(x), _ptr(W), _ptr(h0), _ptr(c0), _ptr(self.y), _ptr(self.workspace),
                                 self.ws_bytes, _ptr(self.dx), _ptr(self.dW), _ptr(self.db if want_db else None),
                                 _ptr(self.dh0), _ptr(self.dc0), _stream(stream))
        if rc != OK:
            raise LstmError(rc, "lstm_stack_bwd")
        return self.dx, self.dW, self.db, self.dh0, self.dc0

    def check(self, stream=None):
        rc = check_workspace(self.workspace, stream)
        if rc != OK:
            raise LstmError(rc, "lstm_check_workspace")
