"""moe_forward inside a captured HIP graph: the library allocates, frees,
clears and synchronises nothing, so a caller can capture a whole layer call
(inputs, weights, output and workspace preallocated) and replay it.  Each
replay, with eager work and host synchronisations between replays, must
equal the eager call bit for bit (the layer is deterministic)."""

import pytest
import torch

from mixture_experts_layer_wavefront_amd import binding as B
from mixture_experts_layer_wavefront_amd import workloads as W

from parity_util import problem_of

pytestmark = pytest.mark.gpu

WL = W.Workload
CASES = {
    "decode": W.WORKLOADS["qwen3_decode"],
    "mixtral_s": WL("mixtral_s", 512, 512, 8, 2, 448, W.BF16, W.TOPK_THEN_SOFTMAX, 0.0, 0.0, 12),
    "cap_skew": WL("cap_skew", 600, 256, 16, 4, 192, W.BF16, W.TOPK_THEN_SOFTMAX, 0.8, 1.2, 81),
    "tall": WL("tall_g", 1100, 264, 8, 2, 200, W.BF16, W.SOFTMAX_THEN_TOPK, 0.0, 0.0, 82),
    # 64 experts, 300 rows each on average with Zipf skew: the two classes of
    # experts on the library's side stream, forked and joined inside the graph
    "two_class": WL("two_class_g", 4800, 256, 64, 4, 192, W.BF16, W.TOPK_THEN_SOFTMAX, 0.0,
                    1.2, 83),
}


@pytest.mark.parametrize("name", list(CASES))
def test_forward_graph_replays(name):
    wl = CASES[name]
    print(f"[graph] {name} T={wl.T} d={wl.d_model} E={wl.E} k={wl.top_k} d_ff={wl.d_ff}",
          flush=True)
    dev = W.make_device(wl, "cuda")
    p = problem_of(wl)
    args = (dev["X"], dev["W_r"], dev["bias"], dev["W_gate"], dev["W_up"], dev["W_down"])
    ws = torch.empty(B.workspace_bytes(p), dtype=torch.uint8, device="cuda")
    out = torch.empty((wl.T, wl.d_model), dtype=torch.float32, device="cuda")
    stats = torch.empty(2 * wl.E + 2, dtype=torch.int32, device="cuda")
    ref = B.moe_forward(p, *args)
    ref_stats = torch.empty_like(stats)
    B.moe_forward(p, *args, stats=ref_stats)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream
        B.moe_forward(p, *args, out=out, stats=stats, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.moe_forward(p, *args, out=out, stats=stats, workspace=ws)
    for rep in range(3):
        out.fill_(-1.0)
        stats.fill_(-1)
        junk = torch.randn(1 << 16, device="cuda").sum()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {rep}: output differs from the eager call"
        assert torch.equal(stats, ref_stats), f"replay {rep}: statistics differ"
        del junk
    print(f"[graph] {name}: 3 replays equal the eager call", flush=True)
