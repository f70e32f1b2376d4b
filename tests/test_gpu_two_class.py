"""GPU parity of the grouped FFN's two classes of experts: with bf16 weights,
at least 64 experts and more than 256 rows per expert on average, each
expert's tile height is chosen on the device from its row count (at most
160 rows: one 160-row tile, on the library's side stream; more: tall tiles on
the caller's stream).  The expert row counts are set through
moe_grouped_ffn's offsets so that both sides of every class and tile
boundary occur (0, 1, 32, 33, 64, 65, 159, 160, 161, 256, 257, 320, 321, 576,
577, ...), as well as layers whose experts all fall in one class.  Each
expert's rows are checked against the oracle's SwiGLU FFN, rows past the kept
ones must stay untouched, and each expert's rows must equal bit for bit a
call that holds that expert alone (fewer than 64 experts: one class, the
tile kind its row count picks), since every tile kind sums each row in the
same K order."""

import numpy as np
import pytest
import torch

import oracle as O
from mixture_experts_layer_wavefront_amd import binding as B
from mixture_experts_layer_wavefront_amd import workloads as W

from parity_util import BF16_TOL, bf16_err, host_f64

pytestmark = pytest.mark.gpu

E, K_TOP, T = 64, 4, 4200          # T k / E = 262.5 rows per expert > 256
BOUNDARY = [0, 1, 32, 33, 64, 65, 159, 160, 161, 255, 256, 257, 319, 320, 321, 576, 577,
            1280, 0, 2]


def _counts(kind):
    rng = np.random.default_rng({"mixed": 91, "all_small": 92, "all_big": 93}[kind])
    if kind == "mixed":
        c = BOUNDARY + rng.integers(0, 420, E - len(BOUNDARY)).tolist()
    elif kind == "all_small":
        c = rng.integers(0, 161, E).tolist()
        c[:4] = [160, 0, 1, 159]
    else:
        c = rng.integers(161, 262, E).tolist()
        c[:3] = [161, 257, 321]
    assert sum(c) <= T * K_TOP
    return c


@pytest.mark.parametrize("kind", ["mixed", "all_small", "all_big"])
def test_two_class_ffn(kind):
    d, dff = 264, 200
    counts = _counts(kind)
    R = T * K_TOP
    N = sum(counts)
    print(f"[two-class] {kind}: {N} rows, {sum(1 for c in counts if 0 < c <= 160)} small and "
          f"{sum(1 for c in counts if c > 160)} large experts", flush=True)
    wl = W.Workload("two_class", T, d, E, K_TOP, dff, W.BF16, W.TOPK_THEN_SOFTMAX, 0.0, 0.0, 94)
    host = W.make_host(wl)
    rng = np.random.default_rng(95)
    Xp_d = torch.from_numpy(rng.standard_normal((R, d)).astype(np.float32)).to("cuda").to(
        torch.bfloat16)
    Wd = {key: torch.from_numpy(host[key]).to("cuda").to(torch.bfloat16)
          for key in ("W_gate", "W_up", "W_down")}
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    p = B.problem(T, d, E, K_TOP, dff, 0.0, "bf16", W.TOPK_THEN_SOFTMAX, "f32")
    Y = torch.full((R, d), 7.0, dtype=torch.float32, device="cuda")
    B.moe_grouped_ffn(p, Xp_d, torch.from_numpy(off).to("cuda"), Wd["W_gate"], Wd["W_up"],
                      Wd["W_down"], Y)
    torch.cuda.synchronize()
    assert torch.all(Y[N:] == 7.0), "rows past the kept ones were written"
    Wh = {key: host_f64(v) for key, v in Wd.items()}
    Yo = O.grouped_ffn(host_f64(Xp_d)[:N], off, Wh["W_gate"], Wh["W_up"], Wh["W_down"])
    Yg = Y[:N].cpu().numpy()
    worst = 0.0
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        err = bf16_err(Yg[lo:hi], Yo[lo:hi])
        worst = max(worst, err)
        assert err <= BF16_TOL, f"expert {e} ({hi - lo} rows): err {err:.3e}"
        # the expert alone: one class, the tile kind its row count picks
        n = hi - lo
        p1 = B.problem(n, d, 1, 1, dff, 0.0, "bf16", W.TOPK_THEN_SOFTMAX, "f32")
        o2 = torch.tensor([0, n], dtype=torch.int32, device="cuda")
        Y1 = B.moe_grouped_ffn(p1, Xp_d[lo:hi].contiguous(), o2, Wd["W_gate"][e:e + 1],
                               Wd["W_up"][e:e + 1], Wd["W_down"][e:e + 1])
        torch.cuda.synchronize()
        assert torch.equal(Y1[:n], Y[lo:hi]), f"expert {e} ({n} rows) differs from its own call"
    print(f"[two-class] {kind}: worst err {worst:.3e}, every expert equals its own call",
          flush=True)
