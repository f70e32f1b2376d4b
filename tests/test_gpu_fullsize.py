"""Parity at the workloads' full sizes, through moe_forward with a single
workspace exactly as the benchmark launches it.

  * routing (ids bit-exact, near ties excluded; gate weights to 1e-4) and the
    permute (counts, offsets, drops, dest rows, inverse map: bit-exact,
    against the oracle's assignment of the GPU's ids) on ALL tokens;
  * X_perm is a bit-exact row gather of X (all rows, on the device);
  * expert FFN rows, the combine and the whole layer on sampled tokens the
    oracle computes one at a time;
  * two runs are bit-identical.
"""

import numpy as np
import pytest
import torch

import oracle as O
from mixture_experts_layer_wavefront_amd import binding as B
from mixture_experts_layer_wavefront_amd import workloads as W

from parity_util import (bf16_err, check_permute, check_routing, fp32_err,
                         host_f64, oracle_capacity, out_err, out_tol,
                         problem_of)

pytestmark = pytest.mark.gpu

SAMPLES = {"tiny": 16, "mixtral": 4, "gptoss": 6, "deepseekv3": 3,
           "qwen3_cap": 12, "qwen3_decode": 32}


def _expert_fetch(dev, e):
    return tuple(host_f64(dev[k][e]) for k in ("W_gate", "W_up", "W_down"))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_full_size(name):
    wl = W.WORKLOADS[name]
    print(f"[full] {name}: generating inputs on the device", flush=True)
    dev = W.make_device(wl, "cuda")
    p = problem_of(wl)
    C = oracle_capacity(wl)
    ws = torch.empty(B.workspace_bytes(p), dtype=torch.uint8, device="cuda")
    stats = torch.empty(2 * wl.E + 2, dtype=torch.int32, device="cuda")
    args = (dev["X"], dev["W_r"], dev["bias"], dev["W_gate"], dev["W_up"],
            dev["W_down"])
    out = B.moe_forward(p, *args, stats=stats, workspace=ws)
    out2 = B.moe_forward(p, *args, workspace=ws)
    # the stages, through their own entry points
    idx, w = B.moe_route(p, dev["X"], dev["W_r"], dev["bias"])
    perm = B.moe_permute(p, dev["X"], idx)
    N = int(perm["offsets"][-1].item())
    assert torch.equal(perm["X_perm"][:N],
                       dev["X"][perm["row_token"][:N].long()])
    Y = B.moe_grouped_ffn(p, perm["X_perm"], perm["offsets"], dev["W_gate"],
                          dev["W_up"], dev["W_down"])
    out_s = B.moe_combine(p, Y, perm["dest_row"], w)
    torch.cuda.synchronize()
    assert torch.equal(out, out2), "two runs differ"
    assert torch.equal(out, out_s), "forward != stage-by-stage"
    print(f"[full] {name}: N={N} kept copies; checking routing", flush=True)

    X = host_f64(dev["X"])
    W_r = dev["W_r"].cpu().numpy()
    bias = None if dev["bias"] is None else dev["bias"].cpu().numpy()
    o_idx, o_w, near, logits = O.route(X, W_r, bias, wl.top_k, wl.gating)
    g_idx = idx.cpu().numpy()
    n_near, differ = check_routing(g_idx, w.cpu().numpy(), o_idx, o_w, near,
                                   logits)
    a = check_permute(perm, g_idx, wl.E, C, wl.T, wl.top_k)
    s = stats.cpu().numpy()
    np.testing.assert_array_equal(s[:wl.E], a["counts"])
    np.testing.assert_array_equal(s[wl.E:2 * wl.E + 1], a["offsets"])
    assert s[-1] == a["dropped"]
    print(f"[full] {name}: routing and permute exact (near ties {n_near}, "
          f"dropped {a['dropped']}, max/mean load "
          f"{a['counts'].max() / a['counts'].mean():.2f})", flush=True)

    # sampled tokens (non-near-tie), spread over the batch
    rng = np.random.default_rng(0)
    cand = np.flatnonzero(~near)
    ns = min(SAMPLES[name], len(cand))
    toks = np.unique(np.concatenate([cand[[0, -1]],
                                     rng.choice(cand, ns, replace=False)]))[:ns]
    o_a = O.assign(o_idx, wl.E, C)
    Yg = Y.cpu().numpy()
    # expert rows on the GPU's own rows: Y_perm[r] vs the oracle FFN of X_perm[r]
    rows_by_e = {}
    for t in toks:
        for j in range(wl.top_k):
            r = a["dest"][t, j]
            if r >= 0:
                rows_by_e.setdefault(int(g_idx[t, j]), []).append(int(r))
    Xp = perm["X_perm"]
    y_g, y_o = [], []
    for e in sorted(rows_by_e)[:6]:
        Wg, Wu, Wd = _expert_fetch(dev, e)
        rr = rows_by_e[e]
        y_o.append(O.expert_ffn(host_f64(Xp[rr]), Wg, Wu, Wd))
        y_g.append(Yg[rr])
    if y_o:
        err = out_err(wl, np.concatenate(y_g), np.concatenate(y_o))
        print(f"[full] {name}: expert FFN rows err {err:.3e}", flush=True)
        assert err <= out_tol(wl)
    # combine, on the GPU's Y / dest rows / weights (fp32 output: tight)
    oc = O.combine(Yg, a["dest"][toks], w.cpu().numpy()[toks], len(toks))
    assert fp32_err(host_f64(out)[toks], oc) <= 1e-5
    # the whole layer, oracle routing and assignment throughout
    o_out = O.moe_forward_tokens(toks, X, o_idx, o_w, o_a["dest"],
                                 lambda e: _expert_fetch(dev, e), wl.d_model)
    g_out = host_f64(out)[toks]
    empty = np.all(o_a["dest"][toks] < 0, axis=1)
    assert np.all(g_out[empty] == 0.0)
    if differ:
        same = np.all((o_a["dest"][toks] >= 0) == (a["dest"][toks] >= 0), axis=1)
    else:
        same = np.ones(len(toks), dtype=bool)
    m = ~empty & same
    if m.any():
        err = out_err(wl, g_out[m], o_out[m])
        print(f"[full] {name}: layer output err {err:.3e} over {int(m.sum())} "
              f"sampled tokens ({int(empty.sum())} fully dropped)", flush=True)
        assert err <= out_tol(wl)
