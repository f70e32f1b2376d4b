"""GPU parity of the FP8-weight layer (moe_grouped_ffn_scaled /
moe_forward_scaled): against the oracle on the decoded weights, and bit for
bit against the bf16 path given the same weights decoded to bf16 (the
per-expert scales are powers of two, so decoding and scaling are exact and
the two paths add the same fp32 products in the same order)."""

import numpy as np
import pytest
import torch

import oracle as O
from mixture_experts_layer_wavefront_amd import binding as B
from mixture_experts_layer_wavefront_amd import workloads as W

from parity_util import (host_f64, oracle_capacity, out_err, out_tol, problem_of,
                         run_stages)

pytestmark = pytest.mark.gpu

TK, ST = W.TOPK_THEN_SOFTMAX, W.SOFTMAX_THEN_TOPK
WL = W.Workload
CASES = {
    # 32-row tiles (decode-like)
    "decode_f8": WL("decode_f8", 24, 512, 64, 8, 320, W.BF16, TK, 0.0, 0.0, 91),
    # 256-row tiles, N tail (448 = 3.5 x 128)
    "mixtral_f8": WL("mixtral_f8", 512, 512, 8, 2, 448, W.BF16, TK, 0.0, 0.0, 92),
    # K tails (336, 208 not multiples of 64), Zipf skew
    "gptoss_f8": WL("gptoss_f8", 1000, 336, 32, 4, 208, W.BF16, TK, 0.0, 1.2, 93),
    # ~128 rows per expert: one tile per expert, weights streamed
    "deepseek_f8": WL("deepseek_f8", 512, 256, 16, 4, 128, W.BF16, ST, 0.0, 0.0, 94),
    # capacity with drops
    "cap_f8": WL("cap_f8", 700, 128, 16, 4, 96, W.BF16, TK, 0.5, 1.2, 95),
    # ~300 rows per expert: several 128-row tiles share each weight tile
    "rows300_f8": WL("rows300_f8", 1200, 256, 4, 1, 128, W.BF16, TK, 0.0, 0.0, 96),
    # ~600 rows per expert: 256-row tiles
    "rows600_f8": WL("rows600_f8", 2400, 256, 4, 1, 128, W.BF16, TK, 0.0, 0.0, 97),
    # the down projection split in two K halves (256-row and 128-row tiles)
    "split_f8": WL("split_f8", 2400, 528, 4, 1, 2080, W.BF16, TK, 0.0, 0.0, 98),
    "split128_f8": WL("split128_f8", 800, 528, 4, 1, 2080, W.BF16, TK, 0.0, 0.0, 99),
}


def _decoded_bf16(Q, scales_col):
    v = Q.view(torch.float8_e4m3fn).to(torch.float32) * scales_col.view(-1, 1, 1)
    return v.to(torch.bfloat16)


@pytest.mark.parametrize("name", list(CASES))
def test_fp8_layer(name):
    wl = CASES[name]
    print(f"[fp8] {name} T={wl.T} d={wl.d_model} E={wl.E} k={wl.top_k} d_ff={wl.d_ff}",
          flush=True)
    h = W.make_host_fp8(wl)
    dev = {k: torch.from_numpy(v).to("cuda") if v is not None else None
           for k, v in h.items()}
    dev["X"] = dev["X"].to(torch.bfloat16)
    p8 = B.problem(wl.T, wl.d_model, wl.E, wl.top_k, wl.d_ff, wl.capacity_factor,
                   "bf16", wl.gating, "f32", w_dtype="fp8")
    pb = problem_of(wl)
    sc = dev["scales"]
    Wb = [_decoded_bf16(dev[q], sc[:, j]) for j, q in enumerate(("Q_gate", "Q_up", "Q_down"))]
    base = (dev["X"], dev["W_r"], dev["bias"])
    out8 = B.moe_forward_scaled(p8, *base, dev["Q_gate"], dev["Q_up"], dev["Q_down"], sc)
    outb = B.moe_forward(pb, *base, *Wb)
    # the stage on the GPU's own permutation
    idx, w = B.moe_route(pb, *base)
    perm = B.moe_permute(pb, dev["X"], idx)
    Y8 = B.moe_grouped_ffn_scaled(p8, perm["X_perm"], perm["offsets"], dev["Q_gate"],
                                  dev["Q_up"], dev["Q_down"], sc)
    Yb = B.moe_grouped_ffn(pb, perm["X_perm"], perm["offsets"], *Wb)
    torch.cuda.synchronize()
    N = int(perm["offsets"][-1])
    assert torch.equal(Y8[:N], Yb[:N]), "FP8 and decoded-bf16 grouped FFN differ"
    assert torch.equal(out8, outb), "FP8 and decoded-bf16 layer differ"

    # against the oracle on the decoded weights
    offs = perm["offsets"].cpu().numpy()
    sch = h["scales"].astype(np.float64)
    Yo = O.grouped_ffn(host_f64(perm["X_perm"][:N]), offs,
                       O.dequant_expert_weights(h["Q_gate"], sch[:, 0]),
                       O.dequant_expert_weights(h["Q_up"], sch[:, 1]),
                       O.dequant_expert_weights(h["Q_down"], sch[:, 2]))
    assert out_err(wl, Y8[:N].cpu().numpy(), Yo) <= out_tol(wl)
    C = oracle_capacity(wl)
    o = O.moe_forward_fp8(h["X"], h["W_r"], h["bias"], h["Q_gate"], h["Q_up"],
                          h["Q_down"], h["scales"], wl.top_k,
                          None if C is None else float(np.float32(wl.capacity_factor)),
                          wl.gating)
    keep = ~o["near_tie"]
    g = host_f64(out8)
    empty = np.all(o["dest"] < 0, axis=1) & keep
    assert np.all(g[empty] == 0.0)
    keep &= ~empty
    err = out_err(wl, g[keep], o["out"][keep])
    print(f"[fp8] {name}: out err {err:.3e} over {int(keep.sum())} rows", flush=True)
    assert err <= out_tol(wl)
