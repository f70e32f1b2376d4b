"""Parity of the shared-expert, router-statistics and FP8-weight variants at
the workloads' full sizes, in the configurations the benchmark times them
(``--shared-dff``, ``--router-stats``, ``--fp8``):

  * router statistics of every workload against the oracle's statistics of
    the GPU's selection (all tokens);
  * the shared expert: its part of the output (layer minus routed layer, both
    on the GPU) on every token of sampled rows against the oracle's dense
    SwiGLU FFN, and the whole layer on sampled tokens;
  * FP8 weights: bit-identical to the bf16 layer on the decoded weights (the
    per-expert scales are powers of two and the accumulation order is the
    same), and sampled tokens against the oracle on the decoded weights.
"""

import numpy as np
import pytest
import torch

import oracle as O
from mixture_experts_layer_wavefront_amd import binding as B
from mixture_experts_layer_wavefront_amd import workloads as W

from parity_util import host_f64, out_err, out_tol, problem_of

pytestmark = pytest.mark.gpu


def _sample_tokens(T, n, seed=0):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, T - 1], rng.choice(T, n, replace=False)]))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_router_stats_full_size(name):
    wl = W.WORKLOADS[name]
    print(f"[next-full] router stats {name}", flush=True)
    X, (W_r, bias) = W.make_x(wl), W.make_router(wl)
    tdt = torch.bfloat16 if wl.dtype == W.BF16 else torch.float32
    Xd = torch.from_numpy(X).to("cuda").to(tdt)
    Wr_d = torch.from_numpy(W_r).to("cuda")
    b_d = None if bias is None else torch.from_numpy(bias).to("cuda")
    p = problem_of(wl)
    idx0, w0 = B.moe_route(p, Xd, Wr_d, b_d)
    idx, w, rs = B.moe_route_stats(p, Xd, Wr_d, b_d)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx0) and torch.equal(w, w0)
    rs = rs.double().cpu().numpy()
    E = wl.E
    o = O.router_stats(O.router_logits(X, W_r, bias), idx.cpu().numpy(), w.cpu().numpy())
    np.testing.assert_allclose(rs[:E], o["importance"], rtol=1e-5, atol=1e-5 * wl.T / E)
    np.testing.assert_allclose(rs[E:2 * E], o["mean_prob"], rtol=1e-4, atol=1e-7)
    np.testing.assert_allclose(rs[2 * E], o["aux_loss"], rtol=1e-4)
    np.testing.assert_allclose(rs[2 * E + 1], o["z_loss"], rtol=1e-5)
    print(f"[next-full] {name}: aux {rs[2 * E]:.6f} (oracle {o['aux_loss']:.6f}), "
          f"z {rs[2 * E + 1]:.6f} (oracle {o['z_loss']:.6f})", flush=True)


SHARED = {"deepseekv3": 2048, "qwen3_decode": 768}


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", list(SHARED))
def test_shared_expert_full_size(name):
    wl, sdff = W.WORKLOADS[name], SHARED[name]
    print(f"[next-full] shared expert {name} shared_d_ff={sdff}", flush=True)
    dev = W.make_device(wl, "cuda")
    S = W.make_shared_device(wl, sdff, "cuda")
    p = problem_of(wl)
    args = (dev["X"], dev["W_r"], dev["bias"], dev["W_gate"], dev["W_up"], dev["W_down"])
    out = B.moe_forward_shared(p, sdff, *args, *S)
    out_serial = B.moe_forward_shared(p, sdff, *args, *S, side_stream=None)
    routed = B.moe_forward(p, *args)
    idx, w = B.moe_route(p, dev["X"], dev["W_r"], dev["bias"])
    torch.cuda.synchronize()
    assert torch.equal(out, out_serial), "side stream changes the result"
    toks = _sample_tokens(wl.T, min(wl.T - 2, 24))
    Xs = host_f64(dev["X"][torch.from_numpy(toks).to("cuda")])
    Sh = [host_f64(t) for t in S]
    sh_o = O.shared_expert_ffn(Xs, *Sh)
    sh_g = host_f64(out)[toks] - host_f64(routed)[toks]
    err = out_err(wl, sh_g, sh_o)
    print(f"[next-full] {name}: shared part err {err:.3e} on {len(toks)} tokens", flush=True)
    assert err <= out_tol(wl)
    # the whole layer on the sampled tokens: routed part from the oracle on
    # the GPU's selection and assignment of all tokens, plus the shared FFN
    X = host_f64(dev["X"])
    W_r = dev["W_r"].cpu().numpy()
    bias = None if dev["bias"] is None else dev["bias"].cpu().numpy()
    g_idx = idx.cpu().numpy()
    wo = O.gate_weights(O.router_logits(X, W_r, bias), g_idx, wl.gating)
    a = O.assign(g_idx, wl.E, None)
    fetch = lambda e: tuple(host_f64(dev[k][e]) for k in ("W_gate", "W_up", "W_down"))  # noqa: E731
    o_out = O.moe_forward_tokens(toks, X, g_idx, wo, a["dest"], fetch, wl.d_model) + sh_o
    err = out_err(wl, host_f64(out)[toks], o_out)
    print(f"[next-full] {name}: layer err {err:.3e}", flush=True)
    assert err <= out_tol(wl)


FP8 = ("qwen3_decode", "deepseekv3", "mixtral")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", FP8)
def test_fp8_full_size(name):
    wl = W.WORKLOADS[name]
    print(f"[next-full] fp8 {name}", flush=True)
    d8 = W.make_device_fp8(wl, "cuda")
    sc = d8["scales"]
    Wb = []
    for j, q in enumerate(("Q_gate", "Q_up", "Q_down")):
        t = torch.empty(d8[q].shape, dtype=torch.bfloat16, device="cuda")
        for e in range(wl.E):
            t[e] = (d8[q][e].view(torch.float8_e4m3fn).to(torch.float32) * sc[e, j]).to(
                torch.bfloat16)
        Wb.append(t)
    p8 = B.problem(wl.T, wl.d_model, wl.E, wl.top_k, wl.d_ff, wl.capacity_factor,
                   "bf16", wl.gating, "f32", w_dtype="fp8")
    pb = problem_of(wl)
    base = (d8["X"], d8["W_r"], d8["bias"])
    out8 = B.moe_forward_scaled(p8, *base, d8["Q_gate"], d8["Q_up"], d8["Q_down"], sc)
    outb = B.moe_forward(pb, *base, *Wb)
    idx, w = B.moe_route(pb, *base)
    torch.cuda.synchronize()
    assert torch.equal(out8, outb), "FP8 and decoded-bf16 layer differ"
    # sampled tokens against the oracle on the decoded weights
    X = host_f64(d8["X"])
    W_r = d8["W_r"].cpu().numpy()
    bias = None if d8["bias"] is None else d8["bias"].cpu().numpy()
    g_idx = idx.cpu().numpy()
    wo = O.gate_weights(O.router_logits(X, W_r, bias), g_idx, wl.gating)
    a = O.assign(g_idx, wl.E, None)
    sch = sc.double().cpu().numpy()

    def fetch(e):
        return tuple(O.dequant_expert_weights(d8[q][e:e + 1].cpu().numpy(), sch[e:e + 1, j])[0]
                     for j, q in enumerate(("Q_gate", "Q_up", "Q_down")))
    toks = _sample_tokens(wl.T, min(wl.T - 2, 6))
    o_out = O.moe_forward_tokens(toks, X, g_idx, wo, a["dest"], fetch, wl.d_model)
    err = out_err(wl, host_f64(out8)[toks], o_out)
    print(f"[next-full] {name}: fp8 layer err {err:.3e} on {len(toks)} tokens", flush=True)
    assert err <= out_tol(wl)
