"""lstm_fwd_train_scratch -- the forward pass with the library's own device
array as its workspace, for callers that cannot allocate device memory --
against lstm_fwd_train with a caller-owned workspace, through the C ABI.

Two calls in a row on the same device array, the second with a smaller
shape (and another storage type), each compared bit for bit with the
workspace entry point on the same inputs and against the fp64 oracle within
the storage type's tolerance; a shape whose workspace exceeds the array is
refused with LSTM_ERR_SCRATCH and leaves the outputs untouched."""
import numpy as np
import pytest

from layer_lstm_amd import synth
from oracle import oracle
from parity_util import TOL, rel_l2, to_dev, to_host

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


def forward_both(lstm, inp):
    T, B, I, H, dt = inp["T"], inp["B"], inp["I"], inp["H"], inp["dtype"]
    code = lstm.F32 if dt == "f32" else lstm.BF16
    shape = lstm.make_shape(T, B, I, H, code)
    assert lstm.query(shape) <= lstm.SCRATCH_BYTES
    d = {k: to_dev(inp.get(k), dt, torch) for k in ("x", "W", "b", "h0", "c0")}
    ref = lstm.Lstm(T, B, I, H, code)
    ref.forward(d["x"], d["W"], d["b"], d["h0"], d["c0"])
    ref.check()
    td = ref.tdtype
    y = torch.full((T, B, H), float("nan"), dtype=td, device="cuda")
    hT = torch.full((B, H), float("nan"), dtype=td, device="cuda")
    cT = torch.full((B, H), float("nan"), dtype=td, device="cuda")
    lstm.fwd_train_scratch(shape, d["x"], d["W"], d["b"], d["h0"], d["c0"], y, hT, cT)
    torch.cuda.synchronize()
    return dict(y=to_host(y), hT=to_host(hT), cT=to_host(cT)), dict(y=to_host(ref.y), hT=to_host(ref.hT),
                                                                    cT=to_host(ref.cT))


def test_scratch_forward_two_calls(lstm):
    cases = [synth.workload_inputs("f32_T64_B32_I256_H256"),
             synth.make_inputs(5, 19, 40, 72, "bf16", seed=81, dist=ALL)]
    for inp in cases:
        print(f"case: scratch forward {inp['dtype']} T={inp['T']} B={inp['B']} I={inp['I']} H={inp['H']}",
              flush=True)
        got, want = forward_both(lstm, inp)
        ora = oracle.fwd(inp["x"], inp["W"], inp["b"], inp["h0"], inp["c0"])
        for k in ("y", "hT", "cT"):
            np.testing.assert_array_equal(got[k], want[k], err_msg=k)
            assert rel_l2(got[k], ora[k]) <= TOL[inp["dtype"]], k


def test_scratch_forward_refuses_large_shape(lstm):
    w = synth.WORKLOADS["bf16_T128_B64_I512_H1024"]
    shape = lstm.make_shape(w.T, w.B, w.I, w.H, lstm.BF16)
    assert lstm.query(shape) > lstm.SCRATCH_BYTES
    x = torch.zeros((w.T, w.B, w.I), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((4 * w.H, w.H + w.I), dtype=torch.bfloat16, device="cuda")
    y = torch.full((w.T, w.B, w.H), 7.0, dtype=torch.bfloat16, device="cuda")
    hT = torch.full((w.B, w.H), 7.0, dtype=torch.bfloat16, device="cuda")
    cT = torch.full((w.B, w.H), 7.0, dtype=torch.bfloat16, device="cuda")
    rc = lstm.fwd_train_scratch(shape, x, W, None, None, None, y, hT, cT, check=False)
    assert rc == -11, rc
    torch.cuda.synchronize()
    assert bool((y == 7.0).all()) and bool((hT == 7.0).all()) and bool((cT == 7.0).all())
