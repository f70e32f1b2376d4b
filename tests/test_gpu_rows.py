"""GPU checks of the grouped FFN that reads its input rows from X through the
permute's row map (moe_grouped_ffn_rows, and moe_forward's bf16 path): the
permute without its row copy publishes the same counts, offsets, dest rows
and row map as with it, and the grouped FFN on the gathered rows equals the
one on X_perm bit for bit (the same rows reach the same kernels; only the
address of each row differs), rows past the kept ones untouched.  The cases
cover every tile kind of the bf16 and FP8 GEMMs: 32-row tiles (few rows per
expert), 160-row tiles, 256-row tiles, tall tiles with merged remainders,
K and N tails, capacity drops and the split down projection."""

import pytest
import torch

from mixture_experts_layer_wavefront_amd import binding as B
from mixture_experts_layer_wavefront_amd import workloads as W

from parity_util import problem_of, to_device

pytestmark = pytest.mark.gpu

TK, ST = W.TOPK_THEN_SOFTMAX, W.SOFTMAX_THEN_TOPK
WL = W.Workload
CASES = {
    "rows32": WL("rows32", 40, 512, 64, 8, 320, W.BF16, TK, 0.0, 0.0, 61),
    "rows160": WL("rows160", 600, 328, 8, 2, 200, W.BF16, ST, 0.0, 0.0, 62),
    "rows256": WL("rows256", 1000, 264, 8, 2, 448, W.BF16, TK, 0.0, 0.8, 63),
    "tall": WL("tall", 2300, 320, 8, 2, 192, W.BF16, TK, 0.0, 0.0, 64),
    "cap_drops": WL("cap_drops", 2048, 256, 32, 8, 192, W.BF16, TK, 1.25, 1.2, 65),
    "split_down": WL("split_down", 600, 520, 4, 2, 2080, W.BF16, TK, 0.0, 0.8, 66),
    "e256": WL("e256", 300, 136, 256, 8, 64, W.BF16, ST, 0.0, 1.2, 67),
}
CASES_F8 = {
    "f8_rows32": WL("f8_rows32", 24, 512, 64, 8, 320, W.BF16, TK, 0.0, 0.0, 71),
    "f8_rows128": WL("f8_rows128", 512, 336, 16, 4, 208, W.BF16, ST, 0.0, 0.0, 72),
    "f8_rows300": WL("f8_rows300", 1200, 256, 4, 1, 128, W.BF16, TK, 0.0, 0.0, 73),
    "f8_tall": WL("f8_tall", 2400, 320, 4, 1, 448, W.BF16, TK, 0.0, 0.0, 74),
    "f8_cap": WL("f8_cap", 700, 128, 16, 4, 96, W.BF16, TK, 0.5, 1.2, 75),
}


def _maps_agree(a, b, N):
    for key in ("counts", "offsets", "dropped", "dest_row"):
        assert torch.equal(a[key], b[key]), key
    assert torch.equal(a["row_token"][:N], b["row_token"][:N]), "row_token"


@pytest.mark.parametrize("name", list(CASES))
def test_rows_equal_x_perm(name):
    wl = CASES[name]
    print(f"[rows] {name} T={wl.T} d={wl.d_model} E={wl.E} k={wl.top_k} d_ff={wl.d_ff}",
          flush=True)
    dev = to_device(W.make_host(wl), wl)
    p = problem_of(wl)
    idx, w = B.moe_route(p, dev["X"], dev["W_r"], dev["bias"])
    perm = B.moe_permute(p, dev["X"], idx)
    maps = B.moe_permute(p, dev["X"], idx, copy_rows=False)
    assert maps["X_perm"] is None
    torch.cuda.synchronize()
    N = int(perm["offsets"][-1])
    _maps_agree(perm, maps, N)
    R = B.rows_bound(p)
    Y = B.moe_grouped_ffn(p, perm["X_perm"], perm["offsets"], dev["W_gate"], dev["W_up"],
                          dev["W_down"])
    Yr = torch.full((max(R, 1), wl.d_model), 7.0, dtype=torch.float32, device="cuda")
    B.moe_grouped_ffn_rows(p, dev["X"], maps["row_token"], maps["offsets"], dev["W_gate"],
                           dev["W_up"], dev["W_down"], Yr)
    torch.cuda.synchronize()
    print(f"[rows] {name}: {N} rows of {R}", flush=True)
    assert torch.equal(Yr[:N], Y[:N]), "gathered rows and X_perm differ"
    assert torch.all(Yr[N:] == 7.0), "rows past the kept ones were written"


@pytest.mark.parametrize("name", list(CASES_F8))
def test_rows_equal_x_perm_fp8(name):
    wl = CASES_F8[name]
    print(f"[rows] {name} T={wl.T} d={wl.d_model} E={wl.E} k={wl.top_k} d_ff={wl.d_ff}",
          flush=True)
    h = W.make_host_fp8(wl)
    dev = {k: torch.from_numpy(v).to("cuda") if v is not None else None
           for k, v in h.items()}
    dev["X"] = dev["X"].to(torch.bfloat16)
    p8 = B.problem(wl.T, wl.d_model, wl.E, wl.top_k, wl.d_ff, wl.capacity_factor,
                   "bf16", wl.gating, "f32", w_dtype="fp8")
    pb = problem_of(wl)
    q = (dev["Q_gate"], dev["Q_up"], dev["Q_down"])
    idx, w = B.moe_route(pb, dev["X"], dev["W_r"], dev["bias"])
    perm = B.moe_permute(pb, dev["X"], idx)
    maps = B.moe_permute(pb, dev["X"], idx, copy_rows=False)
    torch.cuda.synchronize()
    N = int(perm["offsets"][-1])
    _maps_agree(perm, maps, N)
    Y = B.moe_grouped_ffn_scaled(p8, perm["X_perm"], perm["offsets"], *q, dev["scales"])
    Yr = B.moe_grouped_ffn_rows(p8, dev["X"], maps["row_token"], maps["offsets"], *q,
                                w_scales=dev["scales"])
    torch.cuda.synchronize()
    print(f"[rows] {name}: {N} rows", flush=True)
    assert torch.equal(Yr[:N], Y[:N]), "gathered rows and X_perm differ (FP8 weights)"
