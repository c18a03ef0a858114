"""Host-side checks of the C-ABI library (no GPU needed): it loads, exports
every function include/lstm.h declares, and its constants agree with the
header and with the oracle's conventions; argument errors that need no
device are reported with the documented codes."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lstm.h")


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(lstm_\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def header_enum(name):
    src = open(HEADER).read()
    m = re.search(rf"\b{name}\s*=\s*(-?\d+)", src) or re.search(rf"#define\s+{name}\s+(-?\d+)", src)
    return int(m.group(1))


@pytest.fixture(scope="module")
def lstm():
    from layer_lstm_amd import lstm as mod
    return mod


def test_library_exports_every_declared_function(lstm):
    names = header_functions()
    assert set(names) == set(lstm.EXPORTS), names
    for n in names:
        assert hasattr(lstm.lib(), n), f"liblstm.so does not export {n}"


def test_constants_match_header(lstm):
    assert lstm.abi_version() == header_enum("LSTM_ABI_VERSION") == lstm.ABI_VERSION
    for g, v in (("LSTM_GATE_I", 0), ("LSTM_GATE_F", 1), ("LSTM_GATE_G", 2), ("LSTM_GATE_O", 3)):
        assert header_enum(g) == v
    assert header_enum("LSTM_F32") == lstm.F32 and header_enum("LSTM_BF16") == lstm.BF16
    assert header_enum("LSTM_F16") == lstm.F16
    assert header_enum("LSTM_REVERSE") == lstm.REVERSE
    assert header_enum("LSTM_GATES_IJFO") == lstm.GATES_IJFO
    assert header_enum("LSTM_TWO_BIAS") == lstm.TWO_BIAS
    assert header_enum("LSTM_BIDIRECTIONAL") == lstm.BIDIRECTIONAL
    for code, name in lstm.STATUS.items():
        if code != 0:
            assert header_enum("LSTM_" + name) == code


def test_gate_order_matches_oracle_convention(lstm):
    """The oracle restates the gate order i,f,g,o and the [h | x] column
    order in its own source (it includes nothing of the library); the two
    must agree."""
    src = open(os.path.join(ROOT, "oracle", "lstm_oracle.c")).read()
    assert "order i, f, g, o" in src
    assert "columns\n *     [0,H) multiply h_{t-1} and [H,H+I) multiply x_t" in src
    assert (lstm.GATE_I, lstm.GATE_F, lstm.GATE_G, lstm.GATE_O) == (0, 1, 2, 3)


def test_status_strings(lstm):
    for code in list(lstm.STATUS) + [12345]:
        s = lstm.status_string(code)
        assert isinstance(s, str) and s


@pytest.mark.parametrize("T,B,I,H,code", [(-1, 1, 1, 1, -2), (1, -1, 1, 1, -2), (1, 1, -1, 1, -2),
                                          (1, 1, 1, 0, -2)])
def test_query_rejects_bad_dims(lstm, T, B, I, H, code):
    n = ctypes.c_size_t(777)
    s = lstm.make_shape(T, B, I, H, 0)
    assert lstm.lib().lstm_query(ctypes.byref(s), ctypes.byref(n)) == code
    assert n.value == 777  # untouched on error


def test_query_rejects_bad_dtype_and_nulls(lstm):
    n = ctypes.c_size_t(0)
    s = lstm.make_shape(2, 2, 2, 2, 7)
    assert lstm.lib().lstm_query(ctypes.byref(s), ctypes.byref(n)) == -3
    assert lstm.lib().lstm_query(None, ctypes.byref(n)) == -1
    s = lstm.make_shape(2, 2, 2, 2, 0)
    assert lstm.lib().lstm_query(ctypes.byref(s), None) == -1
    info = lstm.PlanInfo()
    assert lstm.lib().lstm_query_plan(None, ctypes.byref(info)) == -1
    assert lstm.lib().lstm_query_plan(ctypes.byref(s), None) == -1
    assert lstm.lib().lstm_query_plan(ctypes.byref(lstm.make_shape(2, 2, 2, 2, 7)), ctypes.byref(info)) == -3
    assert lstm.lib().lstm_query_plan(ctypes.byref(lstm.make_shape(2, -1, 2, 2, 0)), ctypes.byref(info)) == -2
    assert info.grid == 0  # untouched on error
    s = lstm.make_shape(2, 2, 2, 2, 0)
    s.flags = 16  # an unknown flag
    assert lstm.lib().lstm_query(ctypes.byref(s), ctypes.byref(n)) == -3
    assert lstm.lib().lstm_query_plan(ctypes.byref(s), ctypes.byref(info)) == -3
    assert lstm.lib().lstm_fwd_train(None, *([None] * 10), 0, None) == -1
    assert lstm.lib().lstm_bwd(None, *([None] * 10), 0, *([None] * 6)) == -1


def test_scratch_entry_point_host_checks(lstm):
    """lstm_fwd_train_scratch: the array size stated in the header matches
    the binding's, and a NULL shape is refused before any device work."""
    src = open(HEADER).read()
    m = re.search(r"#define\s+LSTM_SCRATCH_BYTES\s+\((\d+)u\s*<<\s*(\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == lstm.SCRATCH_BYTES
    assert header_enum("LSTM_ERR_SCRATCH") == -11
    assert lstm.lib().lstm_fwd_train_scratch(None, *([None] * 9), None) == -1


def test_reverse_and_bidirectional_flags_exclude_each_other(lstm):
    n = ctypes.c_size_t(0)
    s = lstm.make_shape(2, 2, 2, 2, 0, reverse=True, bidirectional=True)
    assert lstm.lib().lstm_query(ctypes.byref(s), ctypes.byref(n)) == -3


def test_debug_inject_host_checks(lstm):
    """The test hooks: an unknown kind is refused; the step hook is a host
    setting (no device needed) and is turned off again."""
    assert lstm.lib().lstm_debug_inject(99, 0) == -2
    assert lstm.lib().lstm_debug_inject(lstm.DEBUG_FAIL_STEP, 3) == 0
    assert lstm.lib().lstm_debug_inject(lstm.DEBUG_FAIL_STEP, -1) == 0
    assert header_enum("LSTM_ERR_PLACEMENT") == -12
    assert header_enum("LSTM_ERR_STATE") == -13
    assert header_enum("LSTM_DEBUG_FAIL_STEP") == lstm.DEBUG_FAIL_STEP
    assert header_enum("LSTM_DEBUG_MISPLACE") == lstm.DEBUG_MISPLACE
    assert header_enum("LSTM_DEBUG_XCD_LOCAL") == lstm.DEBUG_XCD_LOCAL


def test_stack_query_host_checks(lstm):
    """lstm_stack_query refuses a bad layer count, an unknown or unsupported
    flag, and NULLs before any device work."""
    n, c = ctypes.c_size_t(5), ctypes.c_int32(0)
    s = lstm.make_shape(4, 2, 3, 8, 0)
    assert lstm.lib().lstm_stack_query(None, 2, 0, ctypes.byref(n), ctypes.byref(c)) == -1
    assert lstm.lib().lstm_stack_query(ctypes.byref(s), 0, 0, ctypes.byref(n), ctypes.byref(c)) == -2
    assert lstm.lib().lstm_stack_query(ctypes.byref(s), 9, 0, ctypes.byref(n), ctypes.byref(c)) == -2
    r = lstm.make_shape(4, 2, 3, 8, 0, reverse=True)
    assert lstm.lib().lstm_stack_query(ctypes.byref(r), 2, 0, ctypes.byref(n), ctypes.byref(c)) == -3
    assert n.value == 5
