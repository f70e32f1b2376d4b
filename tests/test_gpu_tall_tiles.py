"""GPU parity of the grouped FFN's tall M-tiles: with more than 256 rows per
expert on average, an expert's remainder of up to 64 rows joins its last
256-row tile (one tile of up to 320 rows instead of a tile of its own).  The
expert row counts are chosen through moe_grouped_ffn's offsets so that every
boundary occurs: exactly 320 rows (the largest tall tile), 257 (one row
merged), 321 (65 rows: not merged, a tile of its own), 576 (= 512 + 64, the
third tile tall), exactly 256, fewer than 256, an empty expert, and 300.
Both down-projection forms run: a single pass (d_ff = 200) and the two K
halves (d_ff = 2080).  Each expert's rows are checked against the oracle's
per-expert SwiGLU FFN, rows past the kept ones are not touched, and the
result is bit-identical to the same rows computed with the expert's rows
split into separate calls of at most 256 rows (no merge possible) wherever
both take the same K order (the few-row tiles of calls with at most 64 rows
run the down projection in one pass, not in two halves)."""

import numpy as np
import pytest
import torch

import oracle as O
from mixture_experts_layer_wavefront_amd import binding as B
from mixture_experts_layer_wavefront_amd import workloads as W

from parity_util import BF16_TOL, bf16_err, host_f64

pytestmark = pytest.mark.gpu

COUNTS = [320, 257, 321, 576, 256, 64, 0, 300]   # sum 2094
COUNTS8 = [576, 577, 640, 641, 512, 64, 0, 1088]  # sum 4098


@pytest.mark.parametrize("d, dff", [(264, 200), (520, 2080)])
def test_tall_tiles(d, dff):
    E, k, T = len(COUNTS), 2, 1100    # mean rows per expert 275 > 256
    R = T * k
    print(f"[tall] d={d} d_ff={dff} counts {COUNTS}", flush=True)
    wl = W.Workload("tall", T, d, E, k, dff, W.BF16, W.TOPK_THEN_SOFTMAX, 0.0, 0.0, 71)
    host = W.make_host(wl)
    rng = np.random.default_rng(72)
    N = sum(COUNTS)
    Xp = rng.standard_normal((R, d)).astype(np.float32)
    Xp_d = torch.from_numpy(Xp).to("cuda").to(torch.bfloat16)
    Wd = {key: torch.from_numpy(host[key]).to("cuda").to(torch.bfloat16)
          for key in ("W_gate", "W_up", "W_down")}
    off = np.concatenate([[0], np.cumsum(COUNTS)]).astype(np.int32)
    off_d = torch.from_numpy(off).to("cuda")
    p = B.problem(T, d, E, k, dff, 0.0, "bf16", W.TOPK_THEN_SOFTMAX, "f32")
    Y = torch.full((R, d), 7.0, dtype=torch.float32, device="cuda")
    B.moe_grouped_ffn(p, Xp_d, off_d, Wd["W_gate"], Wd["W_up"], Wd["W_down"], Y)
    torch.cuda.synchronize()
    assert torch.all(Y[N:] == 7.0), "rows past the kept ones were written"
    Xh = host_f64(Xp_d)
    Wh = {key: host_f64(v) for key, v in Wd.items()}
    Yo = O.grouped_ffn(Xh[:N], off, Wh["W_gate"], Wh["W_up"], Wh["W_down"])
    Yg = Y[:N].cpu().numpy()
    for e in range(E):
        lo, hi = off[e], off[e + 1]
        if hi > lo:
            err = bf16_err(Yg[lo:hi], Yo[lo:hi])
            print(f"[tall] expert {e}: {hi - lo} rows, err {err:.3e}", flush=True)
            assert err <= BF16_TOL
    # the same rows through calls whose experts hold at most 256 rows each:
    # each row's sums run in the same order, so the bits must agree
    pieces = []
    for e in range(E):
        c = COUNTS[e]
        pieces += [(e, s, min(256, c - s)) for s in range(0, c, 256)]
    for e, s, n in pieces:
        if dff >= 2048 and n <= 64:
            continue
        o2 = torch.tensor([0, n], dtype=torch.int32, device="cuda")
        p1 = B.problem(n, d, 1, 1, dff, 0.0, "bf16", W.TOPK_THEN_SOFTMAX, "f32")
        lo = int(off[e]) + s
        Y1 = B.moe_grouped_ffn(p1, Xp_d[lo:lo + n].contiguous(), o2, Wd["W_gate"][e:e + 1],
                               Wd["W_up"][e:e + 1], Wd["W_down"][e:e + 1])
        torch.cuda.synchronize()
        assert torch.equal(Y1[:n], Y[lo:lo + n]), f"expert {e} rows {s}..{s + n}"


def test_tall_tiles_fp8():
    """FP8 E4M3 expert weights on the same row counts: bit-identical to the
    bf16 path given the weights decoded to bf16 (power-of-two scales, same
    sums in the same order), and within the bf16 bar of the oracle.  FP8
    weights need d_model and d_ff multiples of 16."""
    d, dff = 272, 208
    # more than 512 rows per expert on average (FP8 weights take 256-row
    # tiles only then): 512 + 64 and 1024 + 64 merge, 512 + 65 does not
    counts = COUNTS8
    E, k, T = len(counts), 2, 2200
    R = T * k
    print(f"[tall] fp8 d={d} d_ff={dff} counts {counts}", flush=True)
    wl = W.Workload("tall8", T, d, E, k, dff, W.BF16, W.TOPK_THEN_SOFTMAX, 0.0, 0.0, 73)
    h8 = W.make_host_fp8(wl)
    rng = np.random.default_rng(74)
    N = sum(counts)
    Xp_d = torch.from_numpy(rng.standard_normal((R, d)).astype(np.float32)).to("cuda").to(
        torch.bfloat16)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    off_d = torch.from_numpy(off).to("cuda")
    Q = [torch.from_numpy(h8[q]).to("cuda") for q in ("Q_gate", "Q_up", "Q_down")]
    sc = torch.from_numpy(h8["scales"]).to("cuda")
    dec = [(Q[j].view(torch.float8_e4m3fn).to(torch.float32) * sc[:, j].view(E, 1, 1)).to(
        torch.bfloat16) for j in range(3)]
    p8 = B.problem(T, d, E, k, dff, 0.0, "bf16", W.TOPK_THEN_SOFTMAX, "f32", w_dtype="fp8")
    pb = B.problem(T, d, E, k, dff, 0.0, "bf16", W.TOPK_THEN_SOFTMAX, "f32")
    Y8 = B.moe_grouped_ffn_scaled(p8, Xp_d, off_d, *Q, sc)
    Yb = B.moe_grouped_ffn(pb, Xp_d, off_d, *dec)
    torch.cuda.synchronize()
    assert torch.equal(Y8[:N], Yb[:N]), "FP8 and decoded-bf16 grouped FFN differ"
    Yo = O.grouped_ffn(host_f64(Xp_d)[:N], off, *[host_f64(t) for t in dec])
    err = bf16_err(Y8[:N].cpu().numpy(), Yo)
    print(f"[tall] fp8: err {err:.3e}", flush=True)
    assert err <= BF16_TOL
