"""Pins of the fp64 CPU oracle against facts that do not come from the oracle.

Each test names what it pins and the passage of the "SingleLayerLstmGrad"
operator page (Ascend CANN ops-nn) -- or the mathematics -- that fixes the
expected value.  All of these run on the CPU.

 * central finite differences of the loss (the Darknet walkthrough's gradient
   check recipe) pin every backward output against the forward;
 * the zero-weight closed forms and the T=1 closed form pin the forward
   recursion and one backward step;
 * the forget-gate product law of "LSTM梯度流动特性" pins the cell carry and the
   reading that f enters it once;
 * segment composition and linearity pin the carry-in / carry-out contract;
 * the reverse direction (the page's direction attribute, "参数说明") equals
   the forward direction on time-flipped inputs, and passes finite
   differences of its own loss;
 * PyTorch's CPU nn.LSTM in fp64 with autograd is an independent library
   implementation of the same cell (gate order i,f,g,o and the two weight
   blocks are its documented layout) -- licensed by the MXNet page's remark
   that autodiff of the unrolled graph is equivalent to BPTT.
"""
import math

import numpy as np
import pytest

from oracle import oracle
from layer_lstm_amd import synth


def sig(u):
    return 1.0 / (1.0 + np.exp(-u))


def loss(inp, fw):
    """L = sum_t <dy_t, h_t> + <dhT, h_{T-1}> + <dcT, c_{T-1}>: the scalar
    whose gradient the backward computes (dy, dhT, dcT are its cotangents)."""
    L = float(np.sum(inp["dy"] * fw["y"]))
    if inp.get("dhT") is not None:
        L += float(np.sum(inp["dhT"] * fw["hT"]))
    if inp.get("dcT") is not None:
        L += float(np.sum(inp["dcT"] * fw["cT"]))
    return L


def run_loss(inp):
    b = inp.get("b")
    if inp.get("two_bias") and b is not None:
        b = b[0] + b[1]  # bias_ih + bias_hh of the CMU page's LSTMCell, entering as their sum
    fw = oracle.fwd(inp["x"], inp["W"], b, inp.get("h0"), inp.get("c0"),
                    reverse=bool(inp.get("reverse", False)))
    return loss(inp, fw)


def full_inputs(T, B, I, H, seed=0, scale_w=None):
    """Inputs with every optional tensor present (so FD can perturb it)."""
    k = 1.0 / math.sqrt(H) if scale_w is None else scale_w
    dist = dict(W=("u", k), b=("u", k), x=("n", 1.0), h0=("n", 0.5), c0=("n", 0.5),
                dy=("n", 1.0), dhT=("n", 1.0), dcT=("n", 1.0))
    return synth.make_inputs(T, B, I, H, "f32", seed, dist)


GRAD_OF = dict(x="dx", W="dW", b="db", h0="dh0", c0="dc0")


def fd_check(inp, eps_rel=1e-6, tol=1e-7):
    g = oracle.fwd_bwd(inp)
    worst = 0.0
    for p, gname in GRAD_OF.items():
        base = inp[p]
        flat = base.reshape(-1)
        gflat = g[gname].reshape(-1)
        for idx in range(flat.size):
            th = flat[idx]
            eps = eps_rel * max(1.0, abs(th))
            flat[idx] = th + eps
            lp = run_loss(inp)
            flat[idx] = th - eps
            lm = run_loss(inp)
            flat[idx] = th
            fd = (lp - lm) / (2 * eps)
            err = abs(fd - gflat[idx]) / (1.0 + abs(gflat[idx]))
            worst = max(worst, err)
            assert err <= tol, f"{p}[{idx}] FD {fd!r} vs analytic {gflat[idx]!r}"
    return worst


@pytest.fixture(autouse=True, scope="module")
def _single_thread():
    prev = oracle.num_threads()
    oracle.set_threads(1)
    yield
    oracle.set_threads(prev)


@pytest.mark.parametrize("T", [1, 2, 3])
@pytest.mark.parametrize("B", [1, 2])
@pytest.mark.parametrize("I", [1, 3])
@pytest.mark.parametrize("H", [1, 2, 4])
def test_fd_tiny(T, B, I, H):
    inp = full_inputs(T, B, I, H, seed=T * 100 + B * 10 + I + H * 1000, scale_w=0.9)
    fd_check(inp)


@pytest.mark.parametrize("T,B,I,H", [(3, 2, 3, 2), (4, 1, 2, 3)])
def test_fd_tiny_reverse(T, B, I, H):
    """Finite differences of the loss in the reverse direction: every
    gradient, including dh0 and dc0 of the state that enters at t = T-1."""
    inp = full_inputs(T, B, I, H, seed=31 + T + 10 * H, scale_w=0.9)
    inp["reverse"] = True
    fd_check(inp)


def test_reverse_direction_is_the_forward_on_flipped_time():
    """The reverse direction runs the same cell from t = T-1 down to 0; on
    time-flipped x and dy that is the forward direction, so y and dx flip
    back and every other output agrees.  The two runs take different step
    orders and index the previous step differently."""
    inp = full_inputs(5, 3, 4, 6, seed=7)
    rev = oracle.fwd_bwd(dict(inp, reverse=True))
    fwd = oracle.fwd_bwd(dict(inp, x=inp["x"][::-1].copy(), dy=inp["dy"][::-1].copy()))
    for k in ("y", "dx"):
        np.testing.assert_allclose(rev[k], fwd[k][::-1], rtol=1e-12, atol=1e-13)
    for k in ("hT", "cT", "dW", "db", "dh0", "dc0"):
        np.testing.assert_allclose(rev[k], fwd[k], rtol=1e-12, atol=1e-13)
    # and it is not the forward direction on the unflipped inputs
    same = oracle.fwd_bwd(inp)
    assert np.max(np.abs(same["y"] - rev["y"])) > 1e-3


def test_fd_two_biases():
    """Finite differences with two biases b = [b_ih; b_hh]: each half of db
    against the loss's change with its own bias."""
    inp = full_inputs(3, 2, 3, 2, seed=53, scale_w=0.9)
    inp["b"] = np.stack([inp["b"], np.linspace(-0.3, 0.4, inp["b"].size)])
    inp["two_bias"] = True
    fd_check(inp)


def test_gate_order_relabelling():
    """The gate_order attribute ("参数说明": "ifjo" or "ijfo") only relabels
    the row blocks of W, b, dW and db: the map is its own inverse, and with
    equal f and g blocks of W and b the two orders give the same forward
    values and input gradients, and dW / db with those blocks exchanged
    (the forget and candidate gates still differ, so do their deltas)."""
    H = 3
    rows = oracle.ifjo_rows(H, "ijfo")
    assert np.array_equal(rows[rows], np.arange(4 * H))
    assert np.array_equal(oracle.ifjo_rows(H, "ifjo"), np.arange(4 * H))
    inp = full_inputs(3, 2, 2, H, seed=5)
    W, b = inp["W"].copy(), inp["b"].copy()
    W[2 * H:3 * H] = W[H:2 * H]
    b[2 * H:3 * H] = b[H:2 * H]
    a = oracle.fwd_bwd(dict(inp, W=W, b=b))
    c = oracle.fwd_bwd(dict(inp, W=W, b=b, gate_order="ijfo"))
    for k in ("y", "hT", "cT", "dx", "dh0", "dc0"):
        np.testing.assert_allclose(c[k], a[k], rtol=0, atol=0)
    np.testing.assert_allclose(c["dW"], a["dW"][rows], rtol=0, atol=0)
    np.testing.assert_allclose(c["db"], a["db"][rows], rtol=0, atol=0)
    assert np.max(np.abs(a["dW"][H:2 * H] - a["dW"][2 * H:3 * H])) > 1e-6


def test_fd_small_workload_shape():
    """Every element of x, W, b, h0, c0 at the smallest workload's shape
    (T=8, B=4, I=16, H=32; 7040 scalars)."""
    inp = full_inputs(8, 4, 16, 32, seed=7)
    fd_check(inp)


def test_directional_fd_headline_shape():
    """Directional derivative along a random direction over all inputs at
    T=64, B=32, I=256, H=256."""
    oracle.set_threads(0)
    inp = full_inputs(64, 32, 256, 256, seed=3)
    g = oracle.fwd_bwd(inp)
    rng = np.random.default_rng(11)
    dirs = {p: rng.standard_normal(inp[p].shape) for p in GRAD_OF}
    nrm = math.sqrt(sum(float(np.sum(v * v)) for v in dirs.values()))
    # directional derivative <grad L, v> from the backward
    dd = sum(float(np.sum(g[GRAD_OF[p]] * dirs[p])) for p in GRAD_OF) / nrm
    eps = 1e-4
    def shifted(s):
        j = dict(inp)
        for p in GRAD_OF:
            j[p] = inp[p] + s * eps * dirs[p] / nrm
        return run_loss(j)
    fd = (shifted(1) - shifted(-1)) / (2 * eps)
    assert abs(fd - dd) <= 1e-7 * max(1.0, abs(dd)), (fd, dd)


def test_zero_weights_closed_form():
    """W=0, b=0: i=f=o=1/2 and g=0, so c_t = c0 / 2^(t+1) and
    h_t = tanh(c_t)/2 (forward table with constant gates)."""
    T, B, I, H = 6, 3, 5, 4
    inp = full_inputs(T, B, I, H, seed=5)
    W = np.zeros((4 * H, H + I))
    fw = oracle.fwd(inp["x"], W, np.zeros(4 * H), inp["h0"], inp["c0"])
    for t in range(T):
        c = inp["c0"] / 2.0 ** (t + 1)
        np.testing.assert_allclose(fw["cell"][t], c, rtol=1e-15, atol=0)
        np.testing.assert_allclose(fw["y"][t], 0.5 * np.tanh(c), rtol=1e-15, atol=1e-300)


def test_zero_weights_bias_geometric_series():
    """W=0, b!=0: the gates are constant, so the cell recursion
    c_t = f c_{t-1} + i g is a geometric series:
    c_t = f^(t+1) c0 + i g (1 - f^(t+1)) / (1 - f)."""
    T, B, I, H = 9, 2, 3, 5
    inp = full_inputs(T, B, I, H, seed=6)
    rng = np.random.default_rng(1)
    b = rng.uniform(-2, 2, 4 * H)
    fw = oracle.fwd(inp["x"], np.zeros((4 * H, H + I)), b, inp["h0"], inp["c0"])
    i, f, g, o = sig(b[:H]), sig(b[H:2 * H]), np.tanh(b[2 * H:3 * H]), sig(b[3 * H:])
    for t in range(T):
        c = f ** (t + 1) * inp["c0"] + i * g * (1 - f ** (t + 1)) / (1 - f)
        np.testing.assert_allclose(fw["cell"][t], c, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(fw["y"][t], o * np.tanh(c), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(fw["gates"][:, :, H:2 * H], np.broadcast_to(f, (T, B, H)), rtol=1e-15)


def test_forget_product_law():
    """"LSTM梯度流动特性": with no recurrent weights and no gradient reaching
    any h, the cell gradient flows back only through the forget gates, so
    dc0 = dcT * prod_t f_t (elementwise) and dh0 = 0.  The forget gates are
    computed here straight from x and W's input block.  Applying f twice per
    step in the cell carry would give prod f^2 and fail this."""
    T, B, I, H = 7, 3, 4, 5
    inp = full_inputs(T, B, I, H, seed=8, scale_w=1.5)
    inp["W"][:, :H] = 0.0
    inp["dy"] = np.zeros_like(inp["dy"])
    inp["dhT"] = np.zeros_like(inp["dhT"])
    g = oracle.fwd_bwd(inp)
    Wf_x = inp["W"][H:2 * H, H:]
    prod = np.ones((B, H))
    for t in range(T):
        prod = prod * sig(inp["x"][t] @ Wf_x.T + inp["b"][H:2 * H])
    np.testing.assert_allclose(g["dc0"], inp["dcT"] * prod, rtol=1e-13, atol=0)
    assert np.all(g["dh0"] == 0.0)
    assert np.all(g["dx"][:, :, :] != 0.0)  # input gradients flow through f


def test_dc0_is_first_cell_delta_times_f0():
    """Step 5 ("传播到前一时刻"): the carry handed to t-1 is delta-c_t . f_t, so
    the initial-cell gradient is delta-c_0 . f_0."""
    inp = full_inputs(5, 3, 4, 6, seed=9)
    fw = oracle.fwd(inp["x"], inp["W"], inp["b"], inp["h0"], inp["c0"])
    bw = oracle.bwd(inp["x"], inp["W"], inp["h0"], inp["c0"], fw, inp["dy"], inp["dhT"],
                    inp["dcT"], want_debug=True)
    H = 6
    np.testing.assert_array_equal(bw["dc0"], bw["dcell"][0] * fw["gates"][0][:, H:2 * H])


def test_t1_closed_form():
    """One step written out without loops: gates from a = W[h0;x0] + b, the
    cell and hidden update, then the backward step and all parameter
    gradients of a single time step."""
    T, B, I, H = 1, 3, 4, 5
    inp = full_inputs(T, B, I, H, seed=10)
    W, b, x0, h0, c0 = inp["W"], inp["b"], inp["x"][0], inp["h0"], inp["c0"]
    z = np.concatenate([h0, x0], axis=1)  # [B, H+I]
    a = z @ W.T + b
    i, f, g, o = sig(a[:, :H]), sig(a[:, H:2 * H]), np.tanh(a[:, 2 * H:3 * H]), sig(a[:, 3 * H:])
    c1 = f * c0 + i * g
    h1 = o * np.tanh(c1)
    dh = inp["dy"][0] + inp["dhT"]
    dc = dh * o * (1 - np.tanh(c1) ** 2) + inp["dcT"]
    dG = np.concatenate([dc * g * i * (1 - i), dc * c0 * f * (1 - f), dc * i * (1 - g ** 2),
                         dh * np.tanh(c1) * o * (1 - o)], axis=1)
    out = oracle.fwd_bwd(inp)
    r = dict(y=h1[None], hT=h1, cT=c1, dW=dG.T @ z, db=dG.sum(0), dx=(dG @ W[:, H:])[None],
             dh0=dG @ W[:, :H], dc0=dc * f)
    for k, v in r.items():
        np.testing.assert_allclose(out[k], v, rtol=1e-13, atol=1e-15, err_msg=k)


def test_segment_composition():
    """Running T1 steps, then T2 steps from the returned state, equals
    running T1+T2 steps (the Darknet walkthrough: state is carried only
    within one stream); and the backward of the second segment, its
    dh0/dc0 fed as dhT/dcT of the first, equals the full backward, with dW
    and db the sum of the two segments'."""
    T1, T2, B, I, H = 3, 4, 2, 3, 4
    inp = full_inputs(T1 + T2, B, I, H, seed=12)
    full = oracle.fwd_bwd(inp)
    s1 = dict(inp, x=inp["x"][:T1], dy=inp["dy"][:T1])
    fw1 = oracle.fwd(s1["x"], inp["W"], inp["b"], inp["h0"], inp["c0"])
    s2 = dict(inp, x=inp["x"][T1:], dy=inp["dy"][T1:], h0=fw1["hT"], c0=fw1["cT"])
    g2 = oracle.fwd_bwd(s2)
    s1.update(dhT=g2["dh0"], dcT=g2["dc0"])
    g1 = oracle.fwd_bwd(s1)
    rt = dict(rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(np.concatenate([g1["y"], g2["y"]]), full["y"], **rt)
    np.testing.assert_allclose(g2["hT"], full["hT"], **rt)
    np.testing.assert_allclose(g2["cT"], full["cT"], **rt)
    np.testing.assert_allclose(np.concatenate([g1["dx"], g2["dx"]]), full["dx"], **rt)
    np.testing.assert_allclose(g1["dh0"], full["dh0"], **rt)
    np.testing.assert_allclose(g1["dc0"], full["dc0"], **rt)
    np.testing.assert_allclose(g1["dW"] + g2["dW"], full["dW"], **rt)
    np.testing.assert_allclose(g1["db"] + g2["db"], full["db"], **rt)


def test_backward_linear_in_cotangents():
    """The backward is a vector-Jacobian product: linear in (dy, dhT, dcT)."""
    T, B, I, H = 4, 3, 5, 6
    a = full_inputs(T, B, I, H, seed=13)
    b_ = full_inputs(T, B, I, H, seed=14)
    al, be = 0.75, -1.5
    mix = dict(a, dy=al * a["dy"] + be * b_["dy"], dhT=al * a["dhT"] + be * b_["dhT"],
               dcT=al * a["dcT"] + be * b_["dcT"])
    gb = oracle.fwd_bwd(dict(a, dy=b_["dy"], dhT=b_["dhT"], dcT=b_["dcT"]))
    ga = oracle.fwd_bwd(a)
    gm = oracle.fwd_bwd(mix)
    for k in ("dx", "dW", "db", "dh0", "dc0"):
        np.testing.assert_allclose(gm[k], al * ga[k] + be * gb[k], rtol=1e-12, atol=1e-13, err_msg=k)


def test_empty_sequence():
    """T=0: no step runs; the final state is the initial state and the
    backward hands dhT/dcT straight to dh0/dc0 with zero parameter
    gradients."""
    inp = full_inputs(0, 2, 3, 4, seed=15)
    out = oracle.fwd_bwd(inp)
    np.testing.assert_array_equal(out["hT"], inp["h0"])
    np.testing.assert_array_equal(out["cT"], inp["c0"])
    np.testing.assert_array_equal(out["dh0"], inp["dhT"])
    np.testing.assert_array_equal(out["dc0"], inp["dcT"])
    assert np.all(out["dW"] == 0) and np.all(out["db"] == 0) and out["dx"].size == 0


def torch_lstm_reference(inp, b_ih, b_hh):
    """torch.nn.LSTM (CPU, fp64) with weight_hh = W[:, :H], weight_ih =
    W[:, H:] and the given biases; outputs and autograd gradients of the
    loss L = sum_t <dy_t, h_t> + <dhT, h_{T-1}> + <dcT, c_{T-1}>."""
    torch = pytest.importorskip("torch")
    T, B, I, H = inp["T"], inp["B"], inp["I"], inp["H"]
    m = torch.nn.LSTM(I, H, num_layers=1, bias=True, batch_first=False).double()
    with torch.no_grad():
        m.weight_hh_l0.copy_(torch.from_numpy(inp["W"][:, :H]))
        m.weight_ih_l0.copy_(torch.from_numpy(inp["W"][:, H:]))
        m.bias_ih_l0.copy_(torch.from_numpy(b_ih))
        m.bias_hh_l0.copy_(torch.from_numpy(b_hh))
    x = torch.from_numpy(inp["x"]).requires_grad_(True)
    h0 = torch.from_numpy(inp["h0"])[None].clone().requires_grad_(True)
    c0 = torch.from_numpy(inp["c0"])[None].clone().requires_grad_(True)
    y, (hn, cn) = m(x, (h0, c0))
    L = (y * torch.from_numpy(inp["dy"])).sum() + (hn[0] * torch.from_numpy(inp["dhT"])).sum() \
        + (cn[0] * torch.from_numpy(inp["dcT"])).sum()
    L.backward()
    return dict(y=y.detach().numpy(), hT=hn[0].detach().numpy(), cT=cn[0].detach().numpy(),
                dx=x.grad.numpy(), dh0=h0.grad[0].numpy(), dc0=c0.grad[0].numpy(),
                dW=np.concatenate([m.weight_hh_l0.grad.numpy(), m.weight_ih_l0.grad.numpy()], axis=1),
                db_ih=m.bias_ih_l0.grad.numpy(), db_hh=m.bias_hh_l0.grad.numpy())


@pytest.mark.parametrize("T,B,I,H", [(5, 3, 4, 6), (8, 4, 16, 32), (3, 1, 1, 1)])
def test_against_torch_nn_lstm_fp64(T, B, I, H):
    """Independent library implementation: torch.nn.LSTM on the CPU in fp64
    with weight_hh = W[:, :H], weight_ih = W[:, H:], bias_ih = b,
    bias_hh = 0; gradients by autograd of the same scalar loss."""
    inp = full_inputs(T, B, I, H, seed=16)
    ref = torch_lstm_reference(inp, inp["b"], np.zeros_like(inp["b"]))
    ref["db"] = ref.pop("db_ih")
    ref.pop("db_hh")
    out = oracle.fwd_bwd(inp)
    for k, v in ref.items():
        np.testing.assert_allclose(out[k], v, rtol=1e-11, atol=1e-13, err_msg=k)


@pytest.mark.parametrize("T,B,I,H", [(5, 3, 4, 6), (6, 2, 7, 5)])
def test_two_biases_against_torch_nn_lstm_fp64(T, B, I, H):
    """The two-bias path (b = [b_ih; b_hh], both nonzero) against
    torch.nn.LSTM's bias_ih_l0 / bias_hh_l0: every output, and db[0], db[1]
    against the two bias gradients autograd returns."""
    inp = full_inputs(T, B, I, H, seed=17)
    rng = np.random.default_rng(171)
    b_hh = synth.round_to_storage(rng.uniform(-0.4, 0.4, 4 * H), "f32")
    ref = torch_lstm_reference(inp, inp["b"], b_hh)
    out = oracle.fwd_bwd(dict(inp, b=np.stack([inp["b"], b_hh]), two_bias=True))
    for k in ("y", "hT", "cT", "dx", "dh0", "dc0", "dW"):
        np.testing.assert_allclose(out[k], ref[k], rtol=1e-11, atol=1e-13, err_msg=k)
    np.testing.assert_allclose(out["db"][0], ref["db_ih"], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(out["db"][1], ref["db_hh"], rtol=1e-11, atol=1e-13)


# ---------------------------------------------------------------------------
# seq_length mask (the parameter table's mask matrix [T, Batch, hidden_size]
# for the actual sequence lengths) and the bidirectional layer (two
# directions, outputs side by side: the num_directions layout of the
# PyTorch recurrent-layer page)

def outputs_loss(inp, out):
    """The scalar whose gradient the backward computes, from the forward
    outputs in `out`: sum <dy, y> + <dhT, hT> + <dcT, cT> (any layout)."""
    L = float(np.sum(inp["dy"] * out["y"]))
    for c, k in (("dhT", "hT"), ("dcT", "cT")):
        if inp.get(c) is not None:
            L += float(np.sum(inp[c] * out[k]))
    return L


def fd_check_general(inp, params=("x", "W", "b", "h0", "c0"), eps_rel=1e-6, tol=1e-7):
    """Central differences of outputs_loss against the backward, every
    element of every parameter, through oracle.fwd_bwd (any flags)."""
    g = oracle.fwd_bwd(inp)
    for p in params:
        flat = inp[p].reshape(-1)
        gflat = g[GRAD_OF[p]].reshape(-1)
        for idx in range(flat.size):
            th = flat[idx]
            eps = eps_rel * max(1.0, abs(th))
            flat[idx] = th + eps
            lp = outputs_loss(inp, oracle.fwd_bwd(inp))
            flat[idx] = th - eps
            lm = outputs_loss(inp, oracle.fwd_bwd(inp))
            flat[idx] = th
            fd = (lp - lm) / (2 * eps)
            err = abs(fd - gflat[idx]) / (1.0 + abs(gflat[idx]))
            assert err <= tol, f"{p}[{idx}] FD {fd!r} vs analytic {gflat[idx]!r}"


@pytest.mark.parametrize("T,B,I,H,rev", [(3, 2, 2, 3, False), (3, 2, 2, 3, True), (4, 3, 1, 2, False)])
def test_fd_mask(T, B, I, H, rev):
    """Finite differences through the mask's blend, with mask values
    anywhere in [0, 1] (not only 0 and 1), in both directions: the backward
    is the exact gradient of the blended forward."""
    inp = full_inputs(T, B, I, H, seed=91)
    rng = np.random.default_rng(92)
    mask = rng.uniform(0, 1, (T, B, H))
    mask[rng.uniform(0, 1, (T, B, H)) < 0.3] = 0.0
    mask[rng.uniform(0, 1, (T, B, H)) < 0.3] = 1.0
    fd_check_general(dict(inp, mask=mask, reverse=rev))


def test_mask_of_ones_is_the_plain_cell():
    """A mask of ones gives the unmasked result bit for bit (m = 1 is the
    page's cell), in both directions."""
    for rev in (False, True):
        inp = dict(full_inputs(5, 3, 4, 6, seed=93), reverse=rev)
        a = oracle.fwd_bwd(inp)
        b = oracle.fwd_bwd(dict(inp, mask=np.ones((5, 3, 6))))
        for k in a:
            np.testing.assert_array_equal(a[k], b[k], err_msg=k)


@pytest.mark.parametrize("rev", [False, True])
def test_mask_is_truncation(rev):
    """Lengths L_b (a 0/1 mask of whole steps): sequence b gives what the
    unmasked cell gives on its first L_b steps alone -- y at those steps, the
    final state (hT, cT), dh0, dc0, dx at those steps, and its share of dW,
    db -- and the padded outputs (t >= L_b) repeat the state they hold: the
    last state in the forward direction, h0 in the reverse one (whose steps
    past the end come first), with dx zero there.  In the reverse direction
    the truncated sequence runs from t = L_b - 1 down to 0.  dy, dhT and dcT
    are nonzero everywhere: the cotangent of a padded output reaches the
    state it repeats (the final state, or h0 in reverse)."""
    T, B, I, H = 6, 4, 3, 5
    inp = dict(full_inputs(T, B, I, H, seed=94), reverse=rev)
    lengths = [6, 3, 0, 1]
    out = oracle.fwd_bwd(dict(inp, lengths=lengths))
    dW, db = np.zeros_like(out["dW"]), np.zeros_like(out["db"])
    for b, L in enumerate(lengths):
        one = {k: (None if inp[k] is None else inp[k][b:b + 1]) for k in ("h0", "c0", "dhT", "dcT")}
        pad_dy = inp["dy"][L:, b:b + 1].sum(axis=0)
        dhT = one["dhT"] if rev else one["dhT"] + pad_dy
        sub = dict(inp, B=1, T=L, x=inp["x"][:L, b:b + 1], dy=inp["dy"][:L, b:b + 1], dhT=dhT, **{
            k: one[k] for k in ("h0", "c0", "dcT")})
        ref = oracle.fwd_bwd(sub)
        if rev:
            ref["dh0"] = ref["dh0"] + pad_dy
        np.testing.assert_allclose(out["y"][:L, b], ref["y"][:, 0], rtol=1e-13, atol=1e-15)
        held = inp["h0"][b] if rev else ref["hT"][0]
        np.testing.assert_allclose(out["y"][L:, b], np.broadcast_to(held, (T - L, H)), rtol=1e-13, atol=1e-15)
        for k in ("hT", "cT", "dh0", "dc0"):
            np.testing.assert_allclose(out[k][b], ref[k][0], rtol=1e-12, atol=1e-14, err_msg=f"{k} b={b}")
        np.testing.assert_allclose(out["dx"][:L, b], ref["dx"][:, 0], rtol=1e-12, atol=1e-14)
        assert np.all(out["dx"][L:, b] == 0.0)
        dW += ref["dW"]
        db += ref["db"]
    np.testing.assert_allclose(out["dW"], dW, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(out["db"], db, rtol=1e-12, atol=1e-13)


def bidir_inputs(T, B, I, H, seed):
    """Inputs of a bidirectional layer: W, b, h0, c0, dhT, dcT with a
    leading direction axis, dy [T,B,2H]."""
    a = full_inputs(T, B, I, H, seed=seed)
    c = full_inputs(T, B, I, H, seed=seed + 1000)
    inp = dict(a, bidirectional=True, dy=np.concatenate([a["dy"], c["dy"]], axis=2))
    for k in ("W", "b", "h0", "c0", "dhT", "dcT"):
        inp[k] = np.stack([a[k], c[k]])
    return inp


@pytest.mark.parametrize("T,B,I,H", [(3, 2, 2, 3), (2, 1, 3, 2)])
def test_fd_bidirectional(T, B, I, H):
    """Finite differences of the two-direction loss: dx collects both
    directions' input gradients, and each direction's dW, db, dh0, dc0 are
    its own."""
    fd_check_general(bidir_inputs(T, B, I, H, seed=95))


def test_fd_bidirectional_masked():
    """Finite differences with a length mask under both directions."""
    inp = bidir_inputs(4, 3, 2, 3, seed=96)
    fd_check_general(dict(inp, lengths=[4, 2, 0]))


def torch_bidir_reference(inp, lengths=None):
    """torch.nn.LSTM(bidirectional=True) on the CPU in fp64, direction d's
    weights from W[d] ([W_h | W_x] columns), b[d] as bias_ih and a zero
    bias_hh; with lengths, through a packed sequence (outputs past a
    sequence's end come back as zeros, h_n / c_n are the states at each
    sequence's last step).  Returns outputs and autograd gradients of
    outputs_loss."""
    torch = pytest.importorskip("torch")
    T, B, I, H = inp["T"], inp["B"], inp["I"], inp["H"]
    m = torch.nn.LSTM(I, H, num_layers=1, bias=True, batch_first=False, bidirectional=True).double()
    with torch.no_grad():
        for d, sfx in enumerate(("", "_reverse")):
            getattr(m, "weight_hh_l0" + sfx).copy_(torch.from_numpy(inp["W"][d][:, :H]))
            getattr(m, "weight_ih_l0" + sfx).copy_(torch.from_numpy(inp["W"][d][:, H:]))
            getattr(m, "bias_ih_l0" + sfx).copy_(torch.from_numpy(inp["b"][d]))
            getattr(m, "bias_hh_l0" + sfx).zero_()
    x = torch.from_numpy(inp["x"]).requires_grad_(True)
    h0 = torch.from_numpy(inp["h0"]).clone().requires_grad_(True)
    c0 = torch.from_numpy(inp["c0"]).clone().requires_grad_(True)
    if lengths is None:
        y, (hn, cn) = m(x, (h0, c0))
    else:
        packed = torch.nn.utils.rnn.pack_padded_sequence(x, torch.tensor(lengths), enforce_sorted=False)
        yp, (hn, cn) = m(packed, (h0, c0))
        y, _ = torch.nn.utils.rnn.pad_packed_sequence(yp, total_length=T)
    L = (y * torch.from_numpy(inp["dy"])).sum() + (hn * torch.from_numpy(inp["dhT"])).sum() \
        + (cn * torch.from_numpy(inp["dcT"])).sum()
    L.backward()
    grads = lambda name: np.stack([getattr(m, name + sfx).grad.numpy() for sfx in ("", "_reverse")])
    return dict(y=y.detach().numpy(), hT=hn.detach().numpy(), cT=cn.detach().numpy(), dx=x.grad.numpy(),
                dh0=h0.grad.numpy(), dc0=c0.grad.numpy(),
                dW=np.concatenate([grads("weight_hh_l0"), grads("weight_ih_l0")], axis=2), db=grads("bias_ih_l0"))


def test_bidirectional_against_torch_nn_lstm_fp64():
    """The two-direction layer against torch.nn.LSTM(bidirectional=True):
    every output and gradient (this also pins the reverse direction against
    an independent implementation)."""
    inp = bidir_inputs(5, 3, 4, 6, seed=97)
    ref = torch_bidir_reference(inp)
    out = oracle.fwd_bwd(inp)
    for k, v in ref.items():
        np.testing.assert_allclose(out[k], v, rtol=1e-11, atol=1e-13, err_msg=k)


def test_masked_bidirectional_against_torch_packed_sequence():
    """Lengths under both directions against torch's packed sequences.
    torch returns zeros past each sequence's end where this reading repeats
    the state, so the comparison takes the outputs at valid steps, the
    final states, and the gradients with dy zero past each end (then the
    two readings have the same loss)."""
    T = 6
    inp = bidir_inputs(T, 4, 3, 5, seed=98)
    lengths = [6, 2, 4, 1]
    valid = (np.arange(T)[:, None] < np.array(lengths)[None, :]).astype(np.float64)
    inp["dy"] = inp["dy"] * valid[:, :, None]
    ref = torch_bidir_reference(inp, lengths)
    out = oracle.fwd_bwd(dict(inp, lengths=lengths))
    np.testing.assert_allclose(out["y"] * valid[:, :, None], ref["y"], rtol=1e-11, atol=1e-13)
    for k in ("hT", "cT", "dx", "dh0", "dc0", "dW", "db"):
        np.testing.assert_allclose(out[k], ref[k], rtol=1e-11, atol=1e-13, err_msg=k)


# ---------------------------------------------------------------------------
# Stacked layers (the MXNet page's "Stack Multiple RNN Cells"; the CMU page's
# LSTM module with num_layers)

def stacked_inputs(L, T, B, I, H, seed):
    """Inputs of an L-layer stack: layer 0 sees x [T,B,I], the others the
    layer below's output (input size H)."""
    first = full_inputs(T, B, I, H, seed=seed)
    inp = dict(first, layers=L, W=[first["W"]], b=[first["b"]])
    for k in ("h0", "c0", "dhT", "dcT"):
        inp[k] = [first[k]]
    for ll in range(1, L):
        nxt = full_inputs(T, B, H, H, seed=seed + 100 * ll)
        inp["W"].append(nxt["W"])
        inp["b"].append(nxt["b"])
        for k in ("h0", "c0", "dhT", "dcT"):
            inp[k].append(nxt[k])
    inp["b"] = np.stack(inp["b"])
    for k in ("h0", "c0", "dhT", "dcT"):
        inp[k] = np.stack(inp[k])
    return inp


def test_fd_stacked():
    """Finite differences of the stack's loss (the last layer's outputs, and
    every layer's final state) with respect to x, every layer's W, b, h0,
    c0: the input gradient of a layer is the output cotangent of the layer
    below."""
    inp = stacked_inputs(3, 3, 2, 2, 2, seed=131)
    g = oracle.fwd_bwd(inp)
    params = [("x", None), ("b", None), ("h0", None), ("c0", None)] + [("W", ll) for ll in range(3)]
    for p, ll in params:
        base = inp[p] if ll is None else inp[p][ll]
        grad = g[GRAD_OF[p]] if ll is None else g["dW"][ll]
        flat, gflat = base.reshape(-1), np.asarray(grad).reshape(-1)
        for idx in range(flat.size):
            th = flat[idx]
            eps = 1e-6 * max(1.0, abs(th))
            flat[idx] = th + eps
            lp = outputs_loss(inp, oracle.fwd_bwd(inp))
            flat[idx] = th - eps
            lm = outputs_loss(inp, oracle.fwd_bwd(inp))
            flat[idx] = th
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - gflat[idx]) <= 1e-7 * (1.0 + abs(gflat[idx])), (p, ll, idx, fd, gflat[idx])


def test_stacked_against_torch_nn_lstm_fp64():
    """A 3-layer stack against torch.nn.LSTM(num_layers=3) in fp64: every
    output and every layer's gradients (bias_hh zero)."""
    torch = pytest.importorskip("torch")
    L, T, B, I, H = 3, 5, 3, 4, 6
    inp = stacked_inputs(L, T, B, I, H, seed=133)
    m = torch.nn.LSTM(I, H, num_layers=L, bias=True, batch_first=False).double()
    with torch.no_grad():
        for ll in range(L):
            getattr(m, f"weight_hh_l{ll}").copy_(torch.from_numpy(inp["W"][ll][:, :H]))
            getattr(m, f"weight_ih_l{ll}").copy_(torch.from_numpy(inp["W"][ll][:, H:]))
            getattr(m, f"bias_ih_l{ll}").copy_(torch.from_numpy(inp["b"][ll]))
            getattr(m, f"bias_hh_l{ll}").zero_()
    x = torch.from_numpy(inp["x"]).requires_grad_(True)
    h0 = torch.from_numpy(inp["h0"]).clone().requires_grad_(True)
    c0 = torch.from_numpy(inp["c0"]).clone().requires_grad_(True)
    y, (hn, cn) = m(x, (h0, c0))
    loss_t = (y * torch.from_numpy(inp["dy"])).sum() + (hn * torch.from_numpy(inp["dhT"])).sum() \
        + (cn * torch.from_numpy(inp["dcT"])).sum()
    loss_t.backward()
    out = oracle.fwd_bwd(inp)
    ref = dict(y=y.detach().numpy(), hT=hn.detach().numpy(), cT=cn.detach().numpy(), dx=x.grad.numpy(),
               dh0=h0.grad.numpy(), dc0=c0.grad.numpy(),
               db=np.stack([getattr(m, f"bias_ih_l{ll}").grad.numpy() for ll in range(L)]))
    for k, v in ref.items():
        np.testing.assert_allclose(out[k], v, rtol=1e-11, atol=1e-13, err_msg=k)
    for ll in range(L):
        dW = np.concatenate([getattr(m, f"weight_hh_l{ll}").grad.numpy(), getattr(m, f"weight_ih_l{ll}").grad.numpy()],
                            axis=1)
        np.testing.assert_allclose(out["dW"][ll], dW, rtol=1e-11, atol=1e-13, err_msg=f"dW[{ll}]")


def test_one_layer_stack_is_the_layer():
    """A stack of one layer is the one-layer oracle bit for bit."""
    inp = stacked_inputs(1, 4, 3, 5, 6, seed=135)
    a = oracle.fwd_bwd(inp)
    plain = dict(inp, layers=None, W=inp["W"][0], b=inp["b"][0])
    for k in ("h0", "c0", "dhT", "dcT"):
        plain[k] = inp[k][0]
    b = oracle.fwd_bwd(plain)
    for k in ("y", "dx"):
        np.testing.assert_array_equal(a[k], b[k])
    for k in ("hT", "cT", "db", "dh0", "dc0"):
        np.testing.assert_array_equal(a[k][0], b[k])
    np.testing.assert_array_equal(a["dW"][0], b["dW"])
