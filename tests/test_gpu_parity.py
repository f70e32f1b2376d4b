"""GPU parity of every stage and of the whole layer against the CPU oracle,
at sizes the oracle finishes in seconds that still span several tiles and
ragged tails (T not a multiple of 256, N and K not multiples of the tile),
both GEMM tile shapes, both gating orders, capacity with drops, and the
edge cases (T = 0, T = 1, one expert, k = E, everything routed to one
expert, tokens with every copy dropped, E = 256 with k = 32)."""

import numpy as np
import pytest
import torch

import oracle as O
from mixture_experts_layer_wavefront_amd import binding as B
from mixture_experts_layer_wavefront_amd import workloads as W

from parity_util import (bf16_err, check_permute, check_routing, emulated_tol,
                         host_f64, oracle_capacity, out_err, y_with_rounded_h,
                         out_tol, problem_of, run_stages, to_device)

pytestmark = pytest.mark.gpu

TK, ST = W.TOPK_THEN_SOFTMAX, W.SOFTMAX_THEN_TOPK
WL = W.Workload
SMALL = {
    # the tiny fp32 layer at its full size
    "tiny": W.WORKLOADS["tiny"],
    # Mixtral-like shape, scaled: N tail in the gate/up tiles (448 = 3.5 x 128)
    "mixtral_s": WL("mixtral_s", 512, 512, 8, 2, 448, W.BF16, TK, 0.0, 0.0, 12),
    # gpt-oss-like, Zipf skew: T tail, K tails (328, 200), several M tiles
    "gptoss_s": WL("gptoss_s", 1000, 328, 32, 4, 200, W.BF16, TK, 0.0, 1.2, 13),
    # DeepSeek-like softmax-then-topk, ~32 rows per expert: 32-row tile path
    "deepseek_s": WL("deepseek_s", 256, 512, 64, 8, 256, W.BF16, ST, 0.0, 0.0, 14),
    # Qwen3-like with capacity 1.25 and Zipf skew: drops
    "qwen_cap_s": WL("qwen_cap_s", 2048, 256, 32, 8, 192, W.BF16, TK, 1.25, 1.2, 15),
    # decode-like: ~3 rows per expert
    "decode_s": WL("decode_s", 24, 512, 64, 8, 320, W.BF16, TK, 0.0, 0.0, 16),
    # the widest routing the ABI takes
    "wide_k": WL("wide_k", 300, 64, 256, 32, 64, W.BF16, ST, 0.0, 0.0, 17),
    # 65..128 experts (expert-split router logits, EP = 128) with a token
    # tail (333 = 2 x 128 + 77) and d_model not a multiple of 32 (K tail of X)
    "wide_e": WL("wide_e", 333, 264, 100, 6, 128, W.BF16, ST, 0.0, 0.8, 19),
    # 256 experts (two expert groups of 128) with the same kinds of tails
    "wide_e256": WL("wide_e256", 200, 136, 256, 8, 64, W.BF16, TK, 0.0, 1.2, 20),
    # d_ff >= 2048 with few tiles: the down projection runs as two K halves
    # (d_ff / 2 = 1040 leaves a K tail in each half; N tail 520 = 2 x 256 + 8)
    "split_down": WL("split_down", 600, 520, 4, 2, 2080, W.BF16, TK, 0.0, 0.8, 18),
    # 16 experts averaging 375 rows with strong Zipf skew (2999, 2495, 418,
    # 68, 14 and 6 rows; ten experts without rows): tall tiles next to
    # nearly empty ones, with a down projection in two K halves
    "skew16": WL("skew16", 3000, 264, 16, 2, 2112, W.BF16, TK, 0.0, 1.2, 21),
    # fp32 layers on several 64 x 64 FMA tiles per expert: K tails (200 and
    # 136 are not multiples of 16), N tails (136 = 2 x 64 + 8, 200 = 3 x 64
    # + 8), ragged last M-tiles; then capacity drops with skew
    "f32_tiles": WL("f32_tiles", 700, 200, 6, 2, 136, W.F32, TK, 0.0, 0.8, 22),
    "f32_cap": WL("f32_cap", 500, 96, 16, 4, 72, W.F32, ST, 0.75, 1.2, 23),
}


def _run_and_check(wl, host=None, groups=None, h_emul=False):
    """Runs every stage and the whole layer and checks them.  `groups`
    (optional) maps a token-index array to a row population whose output
    scale differs by orders of magnitude from the rest; the output tolerance
    is applied to each population with its own RMS.  `h_emul` (bf16 layers
    with a tiny d_ff): each bar is the larger of the plain one and
    H_MARGIN times the error of the correctly rounded bf16-H emulation
    (parity_util.y_with_rounded_h) of the same comparison."""
    h_emul = h_emul and wl.dtype == W.BF16
    host = W.make_host(wl) if host is None else host
    print(f"[parity] {wl.name} T={wl.T} d={wl.d_model} E={wl.E} k={wl.top_k} "
          f"d_ff={wl.d_ff} {wl.dtype} cf={wl.capacity_factor}", flush=True)
    dev = to_device(host, wl)
    p = problem_of(wl)
    C = oracle_capacity(wl)
    o = O.moe_forward(host["X"], host["W_r"], host["bias"], host["W_gate"],
                      host["W_up"], host["W_down"], wl.top_k,
                      None if C is None else float(np.float32(wl.capacity_factor)),
                      wl.gating)
    assert o["C"] == C
    g = run_stages(p, dev)

    # router: ids bit-exact (near ties excluded), weights to 1e-4
    g_idx = g["idx"].cpu().numpy()
    n_near, differ = check_routing(g_idx, g["w"].cpu().numpy(), o["idx"],
                                   o["w"], o["near_tie"], o["logits"])
    # permute: the oracle's assignment of the GPU's ids, bit-exact
    a = check_permute(g, g_idx, wl.E, C, wl.T, wl.top_k)
    N = int(a["offsets"][-1])
    # X_perm rows are bit copies of X rows
    assert torch.equal(g["X_perm"][:N],
                       dev["X"][g["row_token"][:N].long()])
    # grouped FFN on the GPU's X_perm and offsets
    Yo = O.grouped_ffn(host_f64(g["X_perm"][:N]), a["offsets"], host["W_gate"],
                       host["W_up"], host["W_down"])
    Yg = g["Y"][:N].cpu().numpy()
    tol_y = out_tol(wl)
    if h_emul:
        Yr = y_with_rounded_h(host_f64(g["X_perm"][:N]), a["offsets"], host["W_gate"],
                              host["W_up"], host["W_down"])
        tol_y = emulated_tol(bf16_err(Yr, Yo))
        print(f"[parity] {wl.name}: Y_perm err {out_err(wl, Yg, Yo):.4f} / rms, "
              f"bf16-H emulation {bf16_err(Yr, Yo):.4f}, bar {tol_y:.4f}", flush=True)
    assert out_err(wl, Yg, Yo) <= tol_y, out_err(wl, Yg, Yo)
    # combine on the GPU's Y, dest rows and weights
    oc = O.combine(Yg, a["dest"], g["w"].cpu().numpy(), wl.T)
    assert out_err(wl, host_f64(g["out"]), oc) <= out_tol(wl)
    if h_emul:  # the layer output of the emulation, oracle routing throughout
        out_r = O.combine(y_with_rounded_h(o["X_perm"], o["offsets"], host["W_gate"],
                                           host["W_up"], host["W_down"]),
                          o["dest"], o["w"], wl.T)

    # the whole layer vs the oracle's own routing, near ties excluded
    stats = torch.empty(2 * wl.E + 2, dtype=torch.int32, device="cuda")
    out = B.moe_forward(p, dev["X"], dev["W_r"], dev["bias"], dev["W_gate"],
                        dev["W_up"], dev["W_down"], stats=stats)
    out2 = B.moe_forward(p, dev["X"], dev["W_r"], dev["bias"], dev["W_gate"],
                         dev["W_up"], dev["W_down"])
    torch.cuda.synchronize()
    assert torch.equal(out, out2), "two runs differ"          # deterministic
    assert torch.equal(out, g["out"]), "forward != stage-by-stage"
    s = stats.cpu().numpy()
    np.testing.assert_array_equal(s[:wl.E], a["counts"])
    np.testing.assert_array_equal(s[wl.E:2 * wl.E + 1], a["offsets"])
    assert s[-1] == a["dropped"]
    keep = ~o["near_tie"]
    if differ:  # a near tie flipped: later capacity decisions may cascade
        keep &= np.all((o["dest"] >= 0) == (a["dest"] >= 0), axis=1)
    # tokens whose every copy was dropped output exact zeros; the RMS of the
    # tolerance is taken over the rows that carry expert output
    gout = host_f64(out)
    empty = np.all(o["dest"] < 0, axis=1) & keep
    assert np.all(gout[empty] == 0.0)
    keep &= ~empty
    masks = [keep] if groups is None else [keep & m for m in groups(o)]
    for m in masks:
        err = out_err(wl, gout[m], o["out"][m])
        print(f"[parity] {wl.name}: out err {err:.3e} (tol {out_tol(wl)}) over "
              f"{int(m.sum())} rows, near ties {n_near}, dropped "
              f"{a['dropped']}, N {N}", flush=True)
        tol = out_tol(wl)
        if h_emul:
            tol = emulated_tol(bf16_err(out_r[m], o["out"][m]))
            print(f"[parity] {wl.name}: bf16-H emulation "
                  f"{bf16_err(out_r[m], o['out'][m]):.4f}, bar {tol:.4f}", flush=True)
        assert err <= tol
    return o, g, a


@pytest.mark.parametrize("name", list(SMALL))
def test_layer_parity(name):
    _run_and_check(SMALL[name])


# Shapes on either side of the few-token / few-copy paths: the K-split router
# (T <= 64, bf16) and the one-kernel permute (T*k <= 2048), with K not a
# multiple of the router's K split and expert counts for every router width.
BOUNDARY = {
    "copies_2048": WL("copies_2048", 64, 200, 64, 32, 96, W.BF16, TK, 0.0, 0.0, 31),
    "copies_2080": WL("copies_2080", 65, 200, 64, 32, 96, W.BF16, TK, 0.0, 0.0, 32),
    "k1_2048_tokens": WL("k1_2048_tokens", 2048, 64, 16, 1, 64, W.BF16, TK, 0.0, 0.0, 33),
    "few_tokens_E256": WL("few_tokens_E256", 40, 256, 256, 8, 64, W.BF16, ST, 0.0, 0.0, 34),
    # the first size on the matrix-core router with 256 experts: one token
    # tile of 65 rows (two waves without rows), two expert groups, K split 7
    "mfma_router_65_E256": WL("mfma_router_65_E256", 65, 200, 256, 8, 64, W.BF16, ST, 0.0,
                              0.0, 37),
    "few_tokens_E4": WL("few_tokens_E4", 10, 136, 4, 2, 64, W.BF16, TK, 0.0, 0.0, 35),
    "few_tokens_cap": WL("few_tokens_cap", 48, 128, 16, 4, 64, W.BF16, TK, 0.5, 1.2, 36),
}


@pytest.mark.parametrize("name", list(BOUNDARY))
def test_path_boundaries(name):
    _run_and_check(BOUNDARY[name])


def test_bf16_output_is_the_rounded_fp32_output():
    """out_dtype BF16 stores the same fp32 sum rounded once to bf16 (round to
    nearest even); against the oracle the error is the 2e-2 RMS bar plus that
    final rounding (<= 2^-8 relative)."""
    wl = SMALL["gptoss_s"]
    host = W.make_host(wl)
    dev = to_device(host, wl)
    args = (dev["X"], dev["W_r"], dev["bias"], dev["W_gate"], dev["W_up"],
            dev["W_down"])
    o32 = B.moe_forward(problem_of(wl, "f32"), *args)
    o16 = B.moe_forward(problem_of(wl, "bf16"), *args)
    torch.cuda.synchronize()
    assert o16.dtype == torch.bfloat16
    assert torch.equal(o16, o32.to(torch.bfloat16))
    o = O.moe_forward(host["X"], host["W_r"], host["bias"], host["W_gate"],
                      host["W_up"], host["W_down"], wl.top_k, None, wl.gating)
    keep = ~o["near_tie"]
    g, ref = host_f64(o16)[keep], o["out"][keep]
    r = float(np.sqrt(np.mean(ref ** 2)))
    assert np.all(np.abs(g - ref) <= 2e-2 * r + 2.0 ** -8 * np.abs(ref))


def test_single_expert_dense():
    _run_and_check(WL("one_expert", 100, 128, 1, 1, 96, W.BF16, TK, 0, 0, 21))


def test_k_equals_E():
    _run_and_check(WL("k_eq_E", 130, 64, 4, 4, 64, W.BF16, TK, 0, 0, 22))


def test_single_token():
    _run_and_check(WL("one_token", 1, 256, 16, 4, 128, W.BF16, TK, 0, 0, 23))


def test_all_to_one_expert_with_capacity():
    wl = WL("skew_all", 300, 64, 8, 2, 64, W.BF16, TK, 0.5, 0.0, 24)
    host = W.make_host(wl)
    host["bias"] = np.array([50.0] + [0.0] * 7, dtype=np.float32)
    # tokens that kept their expert-0 copy (gate ~1) and tokens left with only
    # their second copy (gate ~e^-50): two output scales 1e22 apart
    o, g, a = _run_and_check(
        wl, host, groups=lambda o: [o["dest"][:, 0] >= 0, o["dest"][:, 0] < 0])
    C = o["C"]
    assert a["counts"][0] == wl.T and a["kept"][0] == C   # C = 38
    assert np.all(a["dest"][C:, 0] == -1)


def test_all_copies_dropped_rows_are_zero():
    # C = 1: only the first token keeps anything
    wl = WL("drop_all", 40, 64, 2, 2, 64, W.BF16, TK, 0.02, 0.0, 25)
    o, g, a = _run_and_check(wl)
    assert o["C"] == 1
    out = g["out"].float().cpu().numpy()
    dropped_rows = np.all(a["dest"] < 0, axis=1)
    assert dropped_rows.sum() >= wl.T - 2
    assert np.all(out[dropped_rows] == 0.0)


def test_empty_batch_is_noop():
    wl = WL("empty", 0, 64, 8, 2, 64, W.BF16, TK, 0, 0, 26)
    p = problem_of(wl)
    X = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    W_r = torch.zeros((8, 64), device="cuda")
    Wg = torch.zeros((8, 64, 64), dtype=torch.bfloat16, device="cuda")
    out = B.moe_forward(p, X, W_r, None, Wg, Wg, Wg)
    idx, w = B.moe_route(p, X, W_r)
    perm = B.moe_permute(p, X, idx)
    torch.cuda.synchronize()
    assert out.shape == (0, 64)
    assert perm["counts"].sum().item() == 0
    assert perm["offsets"].cpu().numpy().tolist() == [0] * 9


def test_worked_example_on_gpu():
    """The pages' top-2 example through the router kernel: logits 2.0 (id 3)
    and 1.6 (id 5) renormalise to ~0.599 / ~0.401.  X is a one-hot token and
    W_r's column holds the logits."""
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                    "worked_example_top2.json")))
    logits = np.array(g["logits"], dtype=np.float32)
    p = B.problem(1, 8, 8, 2, 8, 0.0, "f32", 0)
    X = torch.zeros((1, 8), device="cuda")
    X[0, 0] = 1.0
    W_r = torch.zeros((8, 8), device="cuda")
    W_r[:, 0] = torch.from_numpy(logits)
    for gating in (0, 1):
        p.gating = gating
        idx, w = B.moe_route(p, X, W_r)
        torch.cuda.synchronize()
        assert idx.cpu().numpy()[0].tolist() == g["expected_idx"]
        np.testing.assert_allclose(w.cpu().numpy()[0], g["approx_weights"],
                                   atol=g["approx_tol"])
        np.testing.assert_allclose(w.cpu().numpy()[0],
                                   g["closed_form_weights"], rtol=1e-6)


def test_bad_arguments_raise_before_launch():
    p = B.problem(8, 64, 4, 5, 64)              # k > E
    X = torch.zeros((8, 64), dtype=torch.bfloat16, device="cuda")
    W_r = torch.zeros((4, 64), device="cuda")
    with pytest.raises(B.MoeError) as e:
        B.moe_route(p, X, W_r)
    assert e.value.status == B.MOE_ERR_INVALID_ARG
    p = B.problem(8, 64, 4, 2, 64)
    idx = torch.zeros((8, 2), dtype=torch.int32, device="cuda")
    small_ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(B.MoeError) as e:
        B.moe_permute(p, X, idx, workspace=small_ws)
    assert e.value.status == B.MOE_ERR_WORKSPACE
