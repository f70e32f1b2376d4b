"""GPU parity of the training path (moe_forward_train + moe_backward) with the
CPU oracle's backward: both GEMM tile sizes, N and K tails that are not
multiples of 64, capacity with fully dropped tokens, unused experts, both
gating orders and top-1.

Tolerance (derived from the arithmetic).  The kernels round to bf16
(unit roundoff u = 2^-8) at fixed points: the saved G, U and H, dY = w dout,
dG and dU; sums accumulate in fp32.  ``_error_sigma`` models each rounding
as an independent relative error uniform in [-u, u] and propagates its
variance to first order through the oracle's own fp64 intermediates (the
probabilistic form of the forward-error analysis of a product, where
errors of independent terms add in quadrature); every element of every
gradient must satisfy |g - o| <= 6 sigma + 1e-5 rms(o) (the second term
covers fp32 accumulation).  The same model applied to a CPU simulation of
the rounding points gives at most 3.7 sigma on the shapes below.  Over each
tensor, rms(g - o) / rms(o) <= 1e-2 as well.  One exception: the router-bias
gradient dbias[e] = sum_t dl[t, e] sums terms of both signs, and where those
cancel (rms(dbias) <= 0.1 rms of the sums of the terms' magnitudes, as with
three experts) its exact values are small against the rounding noise of the
terms; for it rms(g - o) <= 2 rms(sigma) is required instead.  Exact checks: zero
gradients of unused experts and of fully dropped tokens, zero router
gradient at top-1 with the softmax of the selected logit, the training
forward's output equal to moe_forward's bit for bit, two backward runs
bit-identical."""

import numpy as np
import pytest
import torch

import oracle as O
from mixture_experts_layer_wavefront_amd import binding as B
from mixture_experts_layer_wavefront_amd import workloads as W

from parity_util import problem_of, to_device

pytestmark = pytest.mark.gpu

TK, ST = W.TOPK_THEN_SOFTMAX, W.SOFTMAX_THEN_TOPK
WL = W.Workload
CASES = {
    # 256-row tiles (128 rows per expert, weights streamed), N tail 448
    "mix_bwd": WL("mix_bwd", 512, 512, 8, 2, 448, W.BF16, TK, 0.0, 0.0, 61),
    # 600 rows per expert: several M-tiles per expert, weight reuse in L2
    "rows600_bwd": WL("rows600_bwd", 1200, 256, 4, 2, 320, W.BF16, TK, 0.0, 0.0, 62),
    # few rows per expert (32-row tiles), unused experts
    "decode_bwd": WL("decode_bwd", 24, 512, 64, 8, 320, W.BF16, TK, 0.0, 0.0, 63),
    # softmax over all experts, then top-k
    "ds_bwd": WL("ds_bwd", 300, 256, 64, 8, 128, W.BF16, ST, 0.0, 0.0, 64),
    # capacity with Zipf skew: dropped copies and fully dropped tokens
    "cap_bwd": WL("cap_bwd", 1000, 128, 16, 2, 64, W.BF16, TK, 0.3, 1.2, 65),
    # top-1 with the softmax of the selected logit: no router gradient
    "top1_bwd": WL("top1_bwd", 256, 128, 4, 1, 192, W.BF16, TK, 0.0, 0.0, 66),
    # d_model and d_ff not multiples of 64 (K and N tails everywhere)
    "ragged_bwd": WL("ragged_bwd", 200, 264, 8, 2, 328, W.BF16, ST, 0.0, 0.8, 67),
    # the training forward's down projection split in two K halves
    "split_bwd": WL("split_bwd", 600, 520, 4, 2, 2080, W.BF16, TK, 0.0, 0.0, 68),
}


BWD_RMS_TOL = 1e-2   # rms(g - o) / rms(o)
U_BF16 = 2.0 ** -8   # bf16 unit roundoff
Z_MAX = 6.0          # |g - o| <= Z_MAX sigma (+ the fp32 floor) for every element
FP32_FLOOR = 1e-5    # fp32 accumulation, relative to rms(o)


def _f64(t):
    return t.detach().double().cpu().numpy()


def _rms_err(g, o):
    r = np.sqrt(np.mean(np.square(o)))
    return float(np.sqrt(np.mean(np.square(g - o))) / (r if r > 0 else 1.0))


def _silu_dd(z):
    """Second derivative of silu: s (1 - s) (2 + z (1 - 2 s)), s = sigmoid."""
    s = 1.0 / (1.0 + np.exp(-z))
    return s * (1.0 - s) * (2.0 + z * (1.0 - 2.0 * s))


def _error_sigma(host, dout, k, cf, gating, idx):
    """Standard deviation of |GPU - oracle| for every gradient element: each
    bf16 rounding point of the kernels (module docstring) contributes an
    independent relative error of variance u^2 / 3 (uniform in [-u, u]),
    propagated to first order through the oracle's own fp64 intermediates:
    a product C = A B whose factors carry error variances vA, vB gets
    vC = vA (B o B) + (A o A) vB (o: elementwise square)."""
    v3 = U_BF16 ** 2 / 3.0
    X = np.asarray(host["X"], np.float64)
    W_r = np.asarray(host["W_r"], np.float64)
    T, d = X.shape
    E = W_r.shape[0]
    logits = O.router_logits(host["X"], host["W_r"], host["bias"])
    w = O.gate_weights(logits, idx, gating)
    a = O.assign(idx, E, O.capacity(T, k, E, cf))
    off, dest = a["offsets"], a["dest"]
    row_tok = a["row_token"]
    row_slot = np.zeros(int(off[E]), np.int64)
    for t in range(T):
        for j in range(k):
            if dest[t, j] >= 0:
                row_slot[dest[t, j]] = j
    X2 = X[row_tok] ** 2
    var = {n: np.zeros(np.shape(host[m]), np.float64)
           for n, m in (("dW_gate", "W_gate"), ("dW_up", "W_up"), ("dW_down", "W_down"))}
    N = int(off[E])
    v_dA = np.zeros((N, d))
    v_Y = np.zeros((N, d))
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        Wg2 = np.asarray(host["W_gate"][e], np.float64) ** 2
        Wu2 = np.asarray(host["W_up"][e], np.float64) ** 2
        Wd = np.asarray(host["W_down"][e], np.float64)
        Wd2 = Wd ** 2
        A = X[row_tok[lo:hi]]
        G = A @ np.asarray(host["W_gate"][e], np.float64).T
        U = A @ np.asarray(host["W_up"][e], np.float64).T
        sG, s1, s2 = O.silu(G), O.silu_grad(G), _silu_dd(G)
        H = sG * U
        vG, vU, vH = v3 * G ** 2, v3 * U ** 2, v3 * H ** 2
        dY = w[row_tok[lo:hi], row_slot[lo:hi]][:, None] * dout[row_tok[lo:hi]]
        vdY = v3 * dY ** 2
        dH = dY @ Wd
        vdH = vdY @ Wd2
        dG, dU = dH * U * s1, dH * sG
        vdG = v3 * dG ** 2 + (U * s1) ** 2 * vdH + (dH * s1) ** 2 * vU + (dH * U * s2) ** 2 * vG
        vdU = v3 * dU ** 2 + sG ** 2 * vdH + (dH * s1) ** 2 * vG
        var["dW_down"][e] = vdY.T @ H ** 2 + (dY ** 2).T @ vH
        var["dW_gate"][e] = vdG.T @ X2[lo:hi]
        var["dW_up"][e] = vdU.T @ X2[lo:hi]
        v_dA[lo:hi] = vdG @ Wg2 + vdU @ Wu2
        v_Y[lo:hi] = vH @ Wd2.T
    # router: dw = <dout, Y>, dl_j = w_j (dw_j - sum_i w_i dw_i)
    v_dw = np.zeros((T, k))
    v_dX = np.zeros((T, d))
    for t in range(T):
        for j in range(k):
            r = dest[t, j]
            if r >= 0:
                v_dw[t, j] = dout[t] ** 2 @ v_Y[r]
                v_dX[t] += v_dA[r]
    v_dl = np.zeros((T, k))
    for j in range(k):
        for i in range(k):
            v_dl[:, j] += (w[:, j] * ((i == j) - w[:, i])) ** 2 * v_dw[:, i]
    v_full = np.zeros((T, E))
    for t in range(T):
        for j in range(k):
            v_full[t, idx[t, j]] += v_dl[t, j]
    var["dX"] = v_dX + v_full @ W_r ** 2
    var["dW_r"] = v_full.T @ X ** 2
    var["dbias"] = v_full.sum(axis=0)
    return {n: np.sqrt(v) for n, v in var.items()}


CANCEL_MAX = 0.1     # dbias: rms(exact) / rms(sum of |terms|) at which it cancels


def _dbias_cancellation(o):
    """rms of the exact router-bias gradient over the rms of the sums of its
    terms' magnitudes (dbias[e] = sum_t dl[t, e]): near 1 without
    cancellation, near 0 when the terms cancel."""
    mag = np.abs(o["dl"]).sum(axis=0)
    return float(np.sqrt(np.mean(o["dbias"] ** 2)) /
                 max(np.sqrt(np.mean(mag ** 2)), 1e-300))


def check_gradients(name, wl, g, o, sigma):
    """Every gradient element within Z_MAX sigma of the oracle (plus the fp32
    floor), rms error <= BWD_RMS_TOL (a cancelling dbias: at most twice the
    rms of sigma), unused experts exactly zero, and no router gradient at
    top-1 with the softmax of the selected logit."""
    kept = np.diff(o["offsets"]) > 0
    exact_router = wl.top_k == 1 and wl.gating == TK
    ratio, rms_errs, rms_sig = {}, {}, {}
    for key in ("dX", "dW_r", "dbias", "dW_gate", "dW_up", "dW_down"):
        if g.get(key) is None:
            continue
        got = _f64(g[key])
        if key in ("dW_r", "dbias") and exact_router:
            assert np.all(got == 0), f"{key}: top-1 gives no router gradient"
            continue
        if key in ("dW_gate", "dW_up", "dW_down"):
            assert np.all(got[~kept] == 0), f"{key}: unused experts must get zero"
        floor = FP32_FLOOR * np.sqrt(np.mean(o[key] ** 2))
        ratio[key] = float(np.max(np.abs(got - o[key]) / (sigma[key] + floor + 1e-300)))
        rms_errs[key] = _rms_err(got, o[key])
        rms_sig[key] = float(np.sqrt(np.mean(np.square(got - o[key]))) /
                             max(np.sqrt(np.mean(np.square(sigma[key] + floor))), 1e-300))
        del got
    print(f"[backward] {name}: max |g - o| / sigma " +
          ", ".join(f"{k} {v:.2f}" for k, v in ratio.items()), flush=True)
    print(f"[backward] {name}: rms(g - o) / rms(o) " +
          ", ".join(f"{k} {v:.2e}" for k, v in rms_errs.items()) +
          f"; unused experts {int((~kept).sum())}", flush=True)
    cancel = _dbias_cancellation(o) if "dbias" in ratio else None
    for key in ratio:
        assert ratio[key] <= Z_MAX, f"{key}: error {ratio[key]:.2f} sigma"
        if key == "dbias" and cancel <= CANCEL_MAX and rms_errs[key] > BWD_RMS_TOL:
            print(f"[backward] {name}: dbias cancels ({cancel:.3f}): rms error "
                  f"{rms_sig[key]:.2f} rms sigma", flush=True)
            assert rms_sig[key] <= 2.0, \
                f"{key}: rms {rms_errs[key]:.3e} ({rms_sig[key]:.2f} rms sigma)"
        else:
            assert rms_errs[key] <= BWD_RMS_TOL, \
                f"{key}: rms {rms_errs[key]:.3e} ({rms_sig[key]:.2f} rms sigma)"


@pytest.mark.parametrize("name", list(CASES))
def test_backward_layer(name):
    wl = CASES[name]
    print(f"[backward] {name} T={wl.T} d={wl.d_model} E={wl.E} k={wl.top_k} "
          f"d_ff={wl.d_ff} cf={wl.capacity_factor}", flush=True)
    host = W.make_host(wl)
    dev = to_device(host, wl)
    dout_h = W.make_dout(wl)
    dout = torch.from_numpy(dout_h).to("cuda")
    p = problem_of(wl)
    args = (dev["X"], dev["W_r"], dev["bias"], dev["W_gate"], dev["W_up"], dev["W_down"])
    out, state = B.moe_forward_train(p, *args)
    ref_out = B.moe_forward(p, *args)
    idx, _ = B.moe_route(p, dev["X"], dev["W_r"], dev["bias"])
    g = B.moe_backward(p, dev["X"], dev["W_r"], dev["W_gate"], dev["W_up"],
                       dev["W_down"], state, dout)
    g2 = B.moe_backward(p, dev["X"], dev["W_r"], dev["W_gate"], dev["W_up"],
                        dev["W_down"], state, dout)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out), "training forward differs from moe_forward"
    for key in g:
        assert torch.equal(g[key], g2[key]), f"{key}: two runs differ"

    cf = float(np.float32(wl.capacity_factor))
    o = O.moe_backward(host["X"], host["W_r"], host["bias"], host["W_gate"],
                       host["W_up"], host["W_down"], dout_h, wl.top_k,
                       cf if cf > 0 else None, wl.gating, idx=idx.cpu().numpy())
    sigma = _error_sigma(host, dout_h, wl.top_k, cf if cf > 0 else None, wl.gating,
                         idx.cpu().numpy())
    check_gradients(name, wl, g, o, sigma)
    gone = np.all(o["dest"] < 0, axis=1)
    if name == "cap_bwd":
        assert gone.any()
    assert torch.all(g["dX"][torch.from_numpy(gone).to("cuda")] == 0)
