"""GPU router statistics (moe_route_stats / moe_forward_stats) against the
oracle's router_stats: every router path (few-token K-split, matrix-core
logits, the fp32 layer), both gating orders, expert counts for every
selection-kernel width.  Routing itself is bit-identical to moe_route's."""

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
    "few_tokens": WL("few_tokens_st", 40, 512, 64, 8, 64, W.BF16, TK, 0.0, 0.0, 71),
    "mfma_E128": WL("mfma_E128_st", 700, 256, 128, 8, 64, W.BF16, TK, 0.0, 1.2, 72),
    "mfma_E256_st": WL("mfma_E256_st", 300, 128, 256, 8, 64, W.BF16, ST, 0.0, 0.0, 73),
    "mfma_E8": WL("mfma_E8_st", 1030, 128, 8, 2, 64, W.BF16, TK, 0.0, 0.0, 74),
    # more than 64 x 4 tokens: the two-level sum of the per-workgroup rows
    "rows_2level": WL("rows_2level_st", 4100, 64, 32, 4, 64, W.BF16, TK, 0.0, 1.2, 76),
    "fp32": W.WORKLOADS["tiny"].replace(name="tiny_st", seed=75),
}


@pytest.mark.parametrize("name", list(CASES))
def test_router_stats(name):
    wl = CASES[name]
    print(f"[stats] {name} T={wl.T} d={wl.d_model} E={wl.E} k={wl.top_k}", flush=True)
    host = W.make_host(wl)
    dev = to_device(host, wl)
    p = problem_of(wl)
    idx0, w0 = B.moe_route(p, dev["X"], dev["W_r"], dev["bias"])
    idx, w, rs = B.moe_route_stats(p, dev["X"], dev["W_r"], dev["bias"])
    args = (dev["X"], dev["W_r"], dev["bias"], dev["W_gate"], dev["W_up"], dev["W_down"])
    out0 = B.moe_forward(p, *args)
    out, rs2 = B.moe_forward_stats(p, *args)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx0) and torch.equal(w, w0)
    assert torch.equal(out, out0)
    assert torch.equal(rs, rs2)
    rs = rs.double().cpu().numpy()
    E = wl.E
    # the oracle's statistics of the GPU's selection, from the oracle's logits
    logits = O.router_logits(host["X"], host["W_r"], host["bias"])
    o = O.router_stats(logits, idx.cpu().numpy(), w.cpu().numpy())
    np.testing.assert_allclose(rs[:E], o["importance"], rtol=1e-5, atol=1e-5)
    np.testing.assert_allclose(rs[E:2 * E], o["mean_prob"], rtol=1e-4, atol=1e-7)
    np.testing.assert_allclose(rs[2 * E], o["aux_loss"], rtol=1e-4)
    np.testing.assert_allclose(rs[2 * E + 1], o["z_loss"], rtol=1e-5)
    assert abs(rs[:E].sum() - wl.T) <= 1e-4 * wl.T
    assert abs(rs[E:2 * E].sum() - 1.0) <= 1e-4
    print(f"[stats] {name}: aux {rs[2 * E]:.6f} (oracle {o['aux_loss']:.6f}), "
          f"z {rs[2 * E + 1]:.6f} (oracle {o['z_loss']:.6f})", flush=True)
