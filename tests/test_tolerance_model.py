"""The bar used by the bf16 parity checks of tiny-d_ff shapes
(parity_util.emulated_tol), checked on the CPU.

With d_ff of 8 to 88 the layer's outputs are heavy-tailed, and rounding the
hidden activation H = silu(G) U to bf16 (the dtype the layer stores it in)
moves the largest output elements by more than 2e-2 of the RMS on its own.
For such shapes the GPU must come within 1.25 times the error of an emulation
that rounds the oracle's exact H correctly and finishes in fp64.  Pinned here:
the emulation rounds each H element by at most half a bf16 ulp, i.e. the
unit roundoff u = 2^-8 relative (its effect on Y stays inside the worst-case
u |H| |W_down|^T), the shapes that get the exception really do miss the plain
bar under correct rounding alone, and the bar is not vacuous: a dropped
hidden unit, or twice the emulation's rounding error, fails it."""

import numpy as np
import pytest

import oracle as O
from mixture_experts_layer_wavefront_amd import workloads as W

from parity_util import (BF16_TOL, bf16_err, bf16_rne, emulated_tol,
                         y_with_rounded_h)

TK, ST = W.TOPK_THEN_SOFTMAX, W.SOFTMAX_THEN_TOPK
# the shapes of the seeded sweep whose emulation misses the plain bar, and
# one more with d_ff = 24
SHAPES = {
    "dff24": W.Workload("dff24", 205, 144, 62, 7, 24, W.BF16, ST, 0.0, 0.0, 1015),
    "sweep23": W.Workload("sweep23", 477, 16, 59, 8, 8, W.BF16, TK, 0.0, 1.2, 1023),
    "sweep29": W.Workload("sweep29", 626, 8, 19, 2, 8, W.BF16, TK, 0.0, 0.0, 1029),
    "sweep_tall5": W.Workload("sweep_tall5", 5148, 160, 6, 1, 88, W.BF16, TK, 0.0, 0.0,
                              2005),
}


def _layer(wl):
    h = W.make_host(wl)
    o = O.moe_forward(h["X"], h["W_r"], h["bias"], h["W_gate"], h["W_up"], h["W_down"],
                      wl.top_k, None, wl.gating)
    return h, o


def test_bf16_rne_is_round_to_nearest_even():
    # values between two bf16 neighbours of 1 (spacing 2^-7): below, at and
    # above the midpoint; ties go to the even mantissa
    x = np.array([1 + 2.0 ** -9, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -20,
                  -(1 + 2.0 ** -8), 3.0])
    r = bf16_rne(x)
    np.testing.assert_array_equal(r, [1.0, 1.0, 1 + 2.0 ** -6, 1 + 2.0 ** -7,
                                      -1.0, 3.0])


def test_emulation_rounds_h_by_at_most_half_an_ulp():
    wl = SHAPES["dff24"]
    h, o = _layer(wl)
    Yr = y_with_rounded_h(o["X_perm"], o["offsets"], h["W_gate"], h["W_up"], h["W_down"])
    bound = np.zeros_like(Yr)
    for e in range(wl.E):
        lo, hi = int(o["offsets"][e]), int(o["offsets"][e + 1])
        if hi > lo:
            A = o["X_perm"][lo:hi]
            H = O.silu(A @ h["W_gate"][e].astype(np.float64).T) * \
                (A @ h["W_up"][e].astype(np.float64).T)
            bound[lo:hi] = 2.0 ** -8 * (np.abs(H) @ np.abs(h["W_down"][e]).astype(np.float64).T)
    d = np.abs(Yr - o["Y_perm"])
    assert np.all(d <= bound * (1 + 1e-9) + 1e-18)
    assert d.max() > 0


@pytest.mark.parametrize("name", list(SHAPES))
def test_exception_shapes_miss_the_plain_bar_and_the_bar_is_not_vacuous(name):
    wl = SHAPES[name]
    h, o = _layer(wl)
    Yr = y_with_rounded_h(o["X_perm"], o["offsets"], h["W_gate"], h["W_up"], h["W_down"])
    Y = o["Y_perm"]
    out_r = O.combine(Yr, o["dest"], o["w"], wl.T)
    e_y, e_out = bf16_err(Yr, Y), bf16_err(out_r, o["out"])
    # correct rounding of H alone misses the plain bar (Y_perm or the output)
    assert max(e_y, e_out) > BF16_TOL
    # the emulation itself passes its own bar
    assert e_y <= emulated_tol(e_y) and e_out <= emulated_tol(e_out)
    # twice the rounding error of the emulation fails it
    assert bf16_err(Y + 2 * (Yr - Y), Y) > emulated_tol(e_y)
    # a dropped hidden unit fails it
    Wd = np.array(h["W_down"], np.float64)
    Wd[:, :, 3 % wl.d_ff] = 0.0
    Yd = y_with_rounded_h(o["X_perm"], o["offsets"], h["W_gate"], h["W_up"], Wd)
    assert bf16_err(Yd, Y) > emulated_tol(e_y)
