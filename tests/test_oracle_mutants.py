"""The oracle's pins have teeth: plausible mistakes planted in a copy of the
oracle source (compiled on the CPU into a temporary library) must each fail
at least one pin.  The mistakes are the ones a reading of the
"SingleLayerLstmGrad" page's equations can plausibly produce: the forget
factor applied twice in the cell carry, a dropped carry, a wrong sign in a
gate derivative, swapped gate blocks, the [x | h] column order, the cell
value of the wrong step in the forget-gate delta, the wrong step's hidden
state in the parameter gradient, the input block used for delta-h, and
three ways of getting the seq_length mask's blend wrong.""" 
import os
import subprocess
import tempfile

import pytest

from oracle import oracle
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "lstm_oracle.c")

MUTANTS = {
    "forget_twice": ("const double dc = dhn * og * (1.0 - tc * tc) + m * dcc[bb * H + j];",
                     "const double dc = dhn * og * (1.0 - tc * tc) + m * dcc[bb * H + j] * fg;"),
    "carry_dropped": ("const double dc = dhn * og * (1.0 - tc * tc) + m * dcc[bb * H + j];",
                      "const double dc = dhn * og * (1.0 - tc * tc);"),
    "sign_output_gate": ("const double d_o = dhn * tc * og * (1.0 - og);",
                         "const double d_o = dhn * tc * og * (og - 1.0);"),
    "gates_if_swapped": ("const double ig = sigm(ab[j]);          /* input gate      */\n"
                         "        const double fg = sigm(ab[H + j]);      /* forget gate     */",
                         "const double ig = sigm(ab[H + j]);\n        const double fg = sigm(ab[j]);"),
    "columns_x_first": ("for (long k = 0; k < H; ++k) s += wr[k] * hp[bb * H + k];\n"
                        "      for (long k = 0; k < I; ++k) s += wr[H + k] * xt[bb * I + k];",
                        "for (long k = 0; k < H; ++k) s += wr[I + k] * hp[bb * H + k];\n"
                        "      for (long k = 0; k < I; ++k) s += wr[k] * xt[bb * I + k];"),
    "forget_delta_uses_c_t": ("const double d_f = dc * cprev * fg * (1.0 - fg);",
                              "const double d_f = dc * c * fg * (1.0 - fg);"),
    "dW_uses_h_t": ("const double* hprev = t > 0 ? y + ((t - 1) * B + bb) * H : (h0 ? h0 + bb * H : NULL);",
                    "const double* hprev = y + (t * B + bb) * H;"),
    # seq_length mask: the state not kept where the mask is 0 (the new
    # value scaled down instead), the state's own gradient not passed on,
    # and the cell carry's (1-m) part dropped
    "mask_state_not_kept": ("const double c = m * cn + (1.0 - m) * cp[bb * H + j];",
                            "const double c = m * cn;"),
    "mask_carry_not_passed": ("dhp[bb * H + j] = (1.0 - m) * dh;",
                              "dhp[bb * H + j] = 0.0;"),
    "mask_cell_carry_dropped": ("dcc[bb * H + j] = (1.0 - m) * dcc[bb * H + j] + dc * fg;",
                                "dcc[bb * H + j] = dc * fg;"),
    # delta-h read from the wrong block of delta-z (column k+I instead of k)
    "dh_from_input_block": ("for (long r = 0; r < G4; ++r) s += W[r * Z + k] * g[r];",
                            "for (long r = 0; r < G4; ++r) s += W[r * Z + ((k < H) ? (k + I) % Z : k)] * g[r];"),
}


def battery():
    """Run a compact set of pins; return the names of those that failed."""
    failed = []
    checks = [
        ("fd_tiny", lambda: pins.test_fd_tiny(3, 2, 3, 2)),
        ("fd_tiny_sq", lambda: pins.test_fd_tiny(2, 2, 3, 4)),
        ("zero_weights", pins.test_zero_weights_closed_form),
        ("geometric", pins.test_zero_weights_bias_geometric_series),
        ("forget_product", pins.test_forget_product_law),
        ("t1_closed_form", pins.test_t1_closed_form),
        ("torch", lambda: pins.test_against_torch_nn_lstm_fp64(5, 3, 4, 6)),
        ("fd_mask", lambda: pins.test_fd_mask(3, 2, 2, 3, False)),
        ("mask_truncation", lambda: pins.test_mask_is_truncation(False)),
    ]
    for name, fn in checks:
        try:
            fn()
        except AssertionError:
            failed.append(name)
    return failed


def test_unmutated_source_passes_battery():
    assert battery() == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mpath = tmp_path / "mutant.c"
    mpath.write_text(src.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-shared", "-fPIC", str(mpath), "-o", str(so), "-lm"])
    prev = oracle.use_library(str(so))
    try:
        failed = battery()
    finally:
        oracle.restore_library(prev)
    assert failed, f"planted mistake {name} passed every pin"
