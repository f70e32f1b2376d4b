"""GPU parity of the training path at the full Mixtral-shaped size (T=4096,
d_model=4096, E=8, top-2, d_ff=14336), in the launch configuration the
benchmark's training step uses: moe_forward_train then moe_backward, every
gradient element against the CPU oracle's fp64 backward (the whole layer;
a few seconds of fp64 BLAS on the host), with the tolerance of the scaled
backward tests (propagated bf16 rounding, see test_gpu_backward)."""

import time

import numpy as np
import pytest
import torch

import oracle as O
from mixture_experts_layer_wavefront_amd import binding as B
from mixture_experts_layer_wavefront_amd import workloads as W

from parity_util import problem_of
from test_gpu_backward import _error_sigma, check_gradients

pytestmark = pytest.mark.gpu


def test_backward_mixtral_fullsize():
    wl = W.WORKLOADS["mixtral"]
    t0 = time.time()
    print(f"[backward-full] {wl.name} T={wl.T} d={wl.d_model} E={wl.E} k={wl.top_k} "
          f"d_ff={wl.d_ff}", flush=True)
    dev = W.make_device(wl, "cuda")
    p = problem_of(wl)
    dout_h = W.make_dout(wl)
    dout = torch.from_numpy(dout_h).to("cuda")
    args = (dev["X"], dev["W_r"], dev["bias"], dev["W_gate"], dev["W_up"], dev["W_down"])
    out, state = B.moe_forward_train(p, *args)
    g = B.moe_backward(p, dev["X"], dev["W_r"], dev["W_gate"], dev["W_up"],
                       dev["W_down"], state, dout, with_dbias=dev["bias"] is not None)
    idx, _ = B.moe_route(p, dev["X"], dev["W_r"], dev["bias"])
    torch.cuda.synchronize()
    print(f"[backward-full] GPU done ({time.time() - t0:.1f} s)", flush=True)
    X, (W_r, bias) = W.make_x(wl), W.make_router(wl)
    host = dict(X=X, W_r=W_r, bias=bias)
    for key in ("W_gate", "W_up", "W_down"):
        host[key] = dev[key].float().cpu().numpy()
    del dev, out, state
    o = O.moe_backward(host["X"], host["W_r"], host["bias"], host["W_gate"],
                       host["W_up"], host["W_down"], dout_h, wl.top_k, None, wl.gating,
                       idx=idx.cpu().numpy())
    print(f"[backward-full] oracle done ({time.time() - t0:.1f} s)", flush=True)
    sigma = _error_sigma(host, dout_h, wl.top_k, None, wl.gating, idx.cpu().numpy())
    print(f"[backward-full] error model done ({time.time() - t0:.1f} s)", flush=True)
    check_gradients(wl.name, wl, g, o, sigma)
    print(f"[backward-full] compared ({time.time() - t0:.1f} s)", flush=True)
