"""Pins for the CPU oracle: each test checks the oracle against something
other than itself -- the pages' worked example, closed forms, invariants,
library routines, special cases and brute force on tiny inputs."""

import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle as O
from mixture_experts_layer_wavefront_amd import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _rand_layer(T, d, E, k, d_ff, seed, bias_scale=0.0):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((T, d)).astype(np.float32)
    W_r = (rng.standard_normal((E, d)) / np.sqrt(d)).astype(np.float32)
    bias = None
    if bias_scale:
        bias = (rng.standard_normal(E) * bias_scale).astype(np.float32)
    Wg = (rng.standard_normal((E, d_ff, d)) / np.sqrt(d)).astype(np.float32)
    Wu = (rng.standard_normal((E, d_ff, d)) / np.sqrt(d)).astype(np.float32)
    Wd = (rng.standard_normal((E, d, d_ff)) / np.sqrt(d_ff)).astype(np.float32)
    return X, W_r, bias, Wg, Wu, Wd


# ---------------------------------------------------------------- routing --
@pytest.mark.parametrize("gating", [O.TOPK_THEN_SOFTMAX, O.SOFTMAX_THEN_TOPK])
def test_worked_example_top2(gating):
    g = _gold("worked_example_top2.json")
    logits = np.array([g["logits"]], dtype=np.float32)
    idx, near = O.select_topk(logits, g["k"])
    assert idx[0].tolist() == g["expected_idx"]
    assert not near[0]
    w = O.gate_weights(logits, idx, gating)[0]
    np.testing.assert_allclose(w, g["approx_weights"], atol=g["approx_tol"])
    # 1.6 is not exactly representable in fp32 (the logits are fp32), so the
    # gap is 0.4 - 2.4e-8 and the weights sit ~1.4e-8 (relative) off sigmoid(0.4)
    np.testing.assert_allclose(w, g["closed_form_weights"], rtol=3e-8)
    # closed form of a two-way softmax: the logistic function of the fp32 gap
    gap = 2.0 - float(np.float32(1.6))
    assert w[0] == pytest.approx(1.0 / (1.0 + math.exp(-gap)), rel=1e-14)
    assert w[1] == pytest.approx(1.0 / (1.0 + math.exp(gap)), rel=1e-14)


def test_topk_set_is_brute_force_argmax_of_sum():
    rng = np.random.default_rng(1)
    for E, k in [(5, 1), (6, 2), (7, 3), (8, 4), (6, 6)]:
        L = rng.standard_normal((20, E)).astype(np.float32)
        idx, _ = O.select_topk(L, k)
        for t in range(L.shape[0]):
            best = max(itertools.combinations(range(E), k),
                       key=lambda s: sum(float(L[t, e]) for e in s))
            assert sorted(idx[t].tolist()) == sorted(best)
            # slots in descending logit order
            vals = L[t, idx[t]]
            assert np.all(np.diff(vals) <= 0)


def test_topk_ties_go_to_lower_id():
    L = np.zeros((1, 8), dtype=np.float32)
    idx, near = O.select_topk(L, 3)
    assert idx[0].tolist() == [0, 1, 2]
    assert near[0]
    L = np.array([[1.0, 3.0, 3.0, 2.0, 3.0]], dtype=np.float32)
    idx, _ = O.select_topk(L, 2)
    assert idx[0].tolist() == [1, 2]


def test_near_tie_flag():
    L = np.array([[3.0, 1.0, 1.0 + 5e-6, 0.0],
                  [3.0, 1.0, 1.5, 0.0]], dtype=np.float32)
    _, near = O.select_topk(L, 2)
    assert near.tolist() == [True, False]
    _, near = O.select_topk(L, 4)
    assert near.tolist() == [False, False]


def test_gating_orders_agree_and_match_library_softmax():
    rng = np.random.default_rng(2)
    L = (rng.standard_normal((50, 16)) * 3).astype(np.float32)
    idx, _ = O.select_topk(L, 4)
    w1 = O.gate_weights(L, idx, O.TOPK_THEN_SOFTMAX)
    w2 = O.gate_weights(L, idx, O.SOFTMAX_THEN_TOPK)
    np.testing.assert_allclose(w1, w2, rtol=1e-12, atol=1e-15)
    # softmax over the selected logits, by the library routine
    sel = np.take_along_axis(L.astype(np.float64), idx.astype(np.int64), 1)
    np.testing.assert_allclose(w1, scipy.special.softmax(sel, axis=1),
                               rtol=1e-12)
    np.testing.assert_allclose(w1.sum(1), 1.0, atol=1e-12)


def test_gate_weights_shift_invariant_and_overflow_safe():
    rng = np.random.default_rng(3)
    L = rng.standard_normal((10, 8)).astype(np.float32)
    idx, _ = O.select_topk(L, 2)
    for gating in (O.TOPK_THEN_SOFTMAX, O.SOFTMAX_THEN_TOPK):
        w = O.gate_weights(L, idx, gating)
        w_big = O.gate_weights(L.astype(np.float64) + 1000.0, idx, gating)
        np.testing.assert_allclose(w, w_big, rtol=1e-9)
        assert np.all(np.isfinite(w_big))


def test_router_logits_fp32_rounding_and_bias():
    rng = np.random.default_rng(4)
    X = rng.standard_normal((7, 33)).astype(np.float32)
    W = rng.standard_normal((5, 33)).astype(np.float32)
    b = rng.standard_normal(5).astype(np.float32)
    L = O.router_logits(X, W, b)
    assert L.dtype == np.float32
    # library fp64 product, then one rounding to fp32, then an fp32 add
    ref = (torch.from_numpy(X).double() @ torch.from_numpy(W).double().T)
    ref = ref.float() + torch.from_numpy(b)
    np.testing.assert_array_equal(L, ref.numpy())
    np.testing.assert_array_equal(O.router_logits(X, W, None),
                                  (torch.from_numpy(X).double()
                                   @ torch.from_numpy(W).double().T)
                                  .float().numpy())


# ------------------------------------------------------------- capacity --
def test_capacity_closed_forms():
    assert O.capacity(16384, 8, 128, 1.25) == 1280
    assert O.capacity(10, 2, 4, 1.0) == 5
    assert O.capacity(10, 1, 3, 1.25) == 5          # ceil(4.1667)
    assert O.capacity(10, 2, 4, 100.0) == 10        # capped at T
    assert O.capacity(10, 2, 4, 0.0) is None
    assert O.capacity(10, 2, 4, None) is None


def test_assign_hand_worked():
    g = _gold("assign_hand_worked.json")
    a = O.assign(np.array(g["idx"]), g["E"], g["C"])
    for key in ("counts", "kept", "offsets", "dest", "row_token"):
        assert np.asarray(a[key]).tolist() == g[key], key
    assert a["dropped"] == g["dropped"]


def _assign_by_expert(idx, E, C):
    """Independent formulation: per expert, the tokens that chose it in
    ascending order; the first C of them are kept."""
    T, k = idx.shape
    cap = T * k if C is None else C
    offsets = [0]
    lists = []
    for e in range(E):
        toks = [t for t in range(T) if e in idx[t].tolist()]
        lists.append(toks)
        offsets.append(offsets[-1] + min(len(toks), cap))
    dest = -np.ones((T, k), dtype=np.int64)
    for e in range(E):
        for pos, t in enumerate(lists[e][:cap]):
            j = idx[t].tolist().index(e)
            dest[t, j] = offsets[e] + pos
    return np.array(offsets), dest, [len(x) for x in lists]


@pytest.mark.parametrize("C", [None, 1, 3, 7, 1000])
def test_assign_invariants_and_brute_force(C):
    rng = np.random.default_rng(5)
    T, E, k = 37, 6, 3
    idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)])
    a = O.assign(idx, E, C)
    off_bf, dest_bf, counts_bf = _assign_by_expert(idx, E, C)
    np.testing.assert_array_equal(a["offsets"], off_bf)
    np.testing.assert_array_equal(a["dest"], dest_bf)
    np.testing.assert_array_equal(a["counts"], counts_bf)
    np.testing.assert_array_equal(a["counts"],
                                  np.bincount(idx.ravel(), minlength=E))
    N = int(a["offsets"][-1])
    assert a["kept"].sum() == T * k - a["dropped"] == N
    if C is not None:
        assert np.all(a["kept"] <= C)
    kept_dest = a["dest"][a["dest"] >= 0]
    assert sorted(kept_dest.tolist()) == list(range(N))        # bijection
    for e in range(E):
        rt = a["row_token"][a["offsets"][e]:a["offsets"][e + 1]]
        assert np.all(np.diff(rt) > 0)                          # stable
    for t in range(T):
        for j in range(k):
            if a["dest"][t, j] >= 0:
                assert a["row_token"][a["dest"][t, j]] == t


def test_gather_rows():
    X = np.arange(12, dtype=np.float32).reshape(4, 3)
    np.testing.assert_array_equal(O.gather_rows(X, [2, 0, 2]),
                                  X[[2, 0, 2]])


# -------------------------------------------------------------- the FFN --
def test_silu_values_and_library():
    z = np.array([-800.0, -5.0, -1.0, 0.0, 1.0, 5.0, 800.0])
    s = O.silu(z)
    assert s[3] == 0.0
    assert s[4] == pytest.approx(0.7310585786300049, rel=1e-15)
    assert s[0] == 0.0 and s[-1] == 800.0
    np.testing.assert_allclose(
        s, torch.nn.functional.silu(torch.from_numpy(z)).numpy(), rtol=1e-14)
    np.testing.assert_allclose(s, z * scipy.special.expit(z), rtol=1e-14)


def test_expert_ffn_matches_library_swiglu():
    rng = np.random.default_rng(6)
    A = rng.standard_normal((9, 16))
    Wg, Wu = rng.standard_normal((2, 24, 16))
    Wd = rng.standard_normal((16, 24))
    At, Wgt, Wut, Wdt = (torch.from_numpy(v) for v in (A, Wg, Wu, Wd))
    ref = torch.nn.functional.linear(
        torch.nn.functional.silu(torch.nn.functional.linear(At, Wgt))
        * torch.nn.functional.linear(At, Wut), Wdt)
    np.testing.assert_allclose(O.expert_ffn(A, Wg, Wu, Wd), ref.numpy(),
                               rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------- whole layer --
def _brute_force(X, W_r, bias, Wg, Wu, Wd, k, cf, gating):
    """Every expert on every token, masked by the gate matrix M[t, e]."""
    T = X.shape[0]
    E = W_r.shape[0]
    idx, w, _, _ = O.route(X, W_r, bias, k, gating)
    a = O.assign(idx, E, O.capacity(T, k, E, cf))
    M = np.zeros((T, E))
    for t in range(T):
        for j in range(k):
            if a["dest"][t, j] >= 0:
                M[t, idx[t, j]] = w[t, j]
    Xt = torch.from_numpy(X).double()
    out = torch.zeros(T, Wd.shape[1], dtype=torch.float64)
    for e in range(E):
        y = torch.nn.functional.linear(
            torch.nn.functional.silu(torch.nn.functional.linear(
                Xt, torch.from_numpy(Wg[e]).double()))
            * torch.nn.functional.linear(Xt, torch.from_numpy(Wu[e]).double()),
            torch.from_numpy(Wd[e]).double())
        out += torch.from_numpy(M[:, e])[:, None] * y
    return out.numpy()


@pytest.mark.parametrize("T,d,E,k,d_ff,cf,gating,bias", [
    (24, 16, 4, 2, 20, None, O.TOPK_THEN_SOFTMAX, 0.0),
    (24, 16, 4, 2, 20, None, O.SOFTMAX_THEN_TOPK, 0.0),
    (40, 8, 5, 3, 12, 0.6, O.TOPK_THEN_SOFTMAX, 2.0),
    (40, 8, 6, 1, 12, 1.0, O.SOFTMAX_THEN_TOPK, 3.0),
    (9, 8, 3, 3, 8, None, O.TOPK_THEN_SOFTMAX, 0.0),
])
def test_forward_matches_brute_force(T, d, E, k, d_ff, cf, gating, bias):
    X, W_r, b, Wg, Wu, Wd = _rand_layer(T, d, E, k, d_ff, seed=T + E,
                                        bias_scale=bias)
    res = O.moe_forward(X, W_r, b, Wg, Wu, Wd, k, cf, gating)
    ref = _brute_force(X, W_r, b, Wg, Wu, Wd, k, cf, gating)
    np.testing.assert_allclose(res["out"], ref, rtol=1e-10, atol=1e-12)
    # the permuted buffer really is a row gather of X
    np.testing.assert_array_equal(res["X_perm"], X[res["row_token"]])


def test_single_expert_is_dense_swiglu():
    X, W_r, b, Wg, Wu, Wd = _rand_layer(10, 16, 1, 1, 24, seed=7)
    res = O.moe_forward(X, W_r, b, Wg, Wu, Wd, 1)
    np.testing.assert_allclose(res["w"], 1.0)
    Xt = torch.from_numpy(X).double()
    ref = torch.nn.functional.linear(
        torch.nn.functional.silu(Xt @ torch.from_numpy(Wg[0]).double().T)
        * (Xt @ torch.from_numpy(Wu[0]).double().T),
        torch.from_numpy(Wd[0]).double())
    np.testing.assert_allclose(res["out"], ref.numpy(), rtol=1e-12,
                               atol=1e-12)


def test_identical_experts_give_dense_ffn_for_any_routing():
    X, W_r, b, Wg, Wu, Wd = _rand_layer(30, 16, 5, 3, 12, seed=8,
                                        bias_scale=1.0)
    Wg[:] = Wg[0]
    Wu[:] = Wu[0]
    Wd[:] = Wd[0]
    for gating in (O.TOPK_THEN_SOFTMAX, O.SOFTMAX_THEN_TOPK):
        res = O.moe_forward(X, W_r, b, Wg, Wu, Wd, 3, None, gating)
        dense = O.expert_ffn(X, Wg[0], Wu[0], Wd[0])
        np.testing.assert_allclose(res["out"], dense, rtol=1e-10, atol=1e-12)


def test_k_equals_E_is_full_softmax_mixture():
    X, W_r, b, Wg, Wu, Wd = _rand_layer(12, 8, 4, 4, 10, seed=9)
    res = O.moe_forward(X, W_r, b, Wg, Wu, Wd, 4)
    # logits are fp32 values (one rounding of the fp64 product)
    l32 = (X.astype(np.float64) @ W_r.astype(np.float64).T).astype(np.float32)
    p = scipy.special.softmax(l32.astype(np.float64), axis=1)
    ref = sum(p[:, e:e + 1] * O.expert_ffn(X, Wg[e], Wu[e], Wd[e])
              for e in range(4))
    np.testing.assert_allclose(res["out"], ref, rtol=1e-10, atol=1e-13)


def test_large_capacity_equals_no_capacity():
    X, W_r, b, Wg, Wu, Wd = _rand_layer(32, 8, 4, 2, 8, seed=10,
                                        bias_scale=1.0)
    r0 = O.moe_forward(X, W_r, b, Wg, Wu, Wd, 2, None)
    r1 = O.moe_forward(X, W_r, b, Wg, Wu, Wd, 2, 2.0)   # C = 32 = T
    assert r1["C"] == 32 and r1["dropped"] == 0
    np.testing.assert_array_equal(r0["out"], r1["out"])


def test_expert_relabelling_invariance():
    X, W_r, b, Wg, Wu, Wd = _rand_layer(40, 8, 6, 2, 8, seed=11,
                                        bias_scale=1.0)
    perm = np.random.default_rng(0).permutation(6)
    for cf in (None, 0.7):
        r0 = O.moe_forward(X, W_r, b, Wg, Wu, Wd, 2, cf)
        r1 = O.moe_forward(X, W_r[perm], b[perm], Wg[perm], Wu[perm],
                           Wd[perm], 2, cf)
        np.testing.assert_allclose(r0["out"], r1["out"], rtol=1e-12,
                                   atol=1e-14)


def test_token_permutation_equivariance_without_capacity():
    X, W_r, b, Wg, Wu, Wd = _rand_layer(25, 8, 5, 2, 8, seed=12)
    perm = np.random.default_rng(1).permutation(25)
    r0 = O.moe_forward(X, W_r, b, Wg, Wu, Wd, 2)
    r1 = O.moe_forward(X[perm], W_r, b, Wg, Wu, Wd, 2)
    np.testing.assert_allclose(r1["out"], r0["out"][perm], rtol=1e-12,
                               atol=1e-14)


def test_forced_skew_drops_all_but_first_C():
    T, E, k = 20, 4, 2
    X, W_r, _, Wg, Wu, Wd = _rand_layer(T, 8, E, k, 8, seed=13)
    b = np.array([100.0, 0, 0, 0], dtype=np.float32)   # everyone picks 0
    res = O.moe_forward(X, W_r, b, Wg, Wu, Wd, k, 0.4)  # C = ceil(4) = 4
    assert res["C"] == 4
    assert np.all(res["idx"][:, 0] == 0)
    assert res["counts"][0] == T and res["kept"][0] == 4
    assert res["row_token"][:4].tolist() == [0, 1, 2, 3]
    assert np.all(res["dest"][4:, 0] == -1)


def test_all_copies_dropped_gives_zero_row():
    T, E, k = 6, 2, 2
    X, W_r, _, Wg, Wu, Wd = _rand_layer(T, 8, E, k, 8, seed=14)
    res = O.moe_forward(X, W_r, None, Wg, Wu, Wd, k, 1.0 / 6)  # C = 1
    assert res["C"] == 1
    assert np.all(res["dest"][1:] == -1)
    assert np.all(res["out"][1:] == 0.0)
    assert np.any(res["out"][0] != 0.0)


def test_forward_tokens_matches_full_forward():
    X, W_r, b, Wg, Wu, Wd = _rand_layer(30, 8, 5, 2, 8, seed=15,
                                        bias_scale=2.0)
    res = O.moe_forward(X, W_r, b, Wg, Wu, Wd, 2, 0.5)
    toks = [0, 3, 17, 29]
    sub = O.moe_forward_tokens(toks, X, res["idx"], res["w"], res["dest"],
                               lambda e: (Wg[e], Wu[e], Wd[e]), X.shape[1])
    np.testing.assert_allclose(sub, res["out"][toks], rtol=1e-12, atol=1e-14)


# ------------------------------------------------------ input generators --
# ------------------------------------------------------------ fp8 weights --
def test_fp8_decode_closed_forms():
    d = O.fp8_e4m3_decode
    cases = {0x00: 0.0, 0x38: 1.0, 0x3C: 1.5, 0x40: 2.0, 0xC0: -2.0, 0x7E: 448.0,
             0xFE: -448.0, 0x01: 2.0 ** -9, 0x07: 7 / 8 * 2.0 ** -6,
             0x08: 2.0 ** -6, 0x30: 0.5, 0x37: 0.9375}
    for code, v in cases.items():
        assert d(np.uint8(code)) == v, hex(code)
    assert np.isnan(d(np.uint8(0x7F))) and np.isnan(d(np.uint8(0xFF)))
    assert np.signbit(d(np.uint8(0x80))) and d(np.uint8(0x80)) == 0.0


def test_fp8_decode_matches_library_on_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = O.fp8_e4m3_decode(codes)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok], ref[ok])
    # positive codes increase strictly up to the largest finite value
    pos = got[:0x7F]
    assert np.all(np.diff(pos) > 0)


def test_fp8_layer_is_the_layer_on_decoded_weights():
    """Weights that are exactly scale * decode(code) give the same layer
    whether passed decoded or as codes and scales."""
    rng = np.random.default_rng(81)
    T, d, E, k, dff = 20, 16, 4, 2, 12
    X, W_r, b, _, _, _ = _rand_layer(T, d, E, k, dff, seed=82)
    Qg = rng.integers(0, 256, (E, dff, d), dtype=np.uint8)
    Qu = rng.integers(0, 256, (E, dff, d), dtype=np.uint8)
    Qd = rng.integers(0, 256, (E, d, dff), dtype=np.uint8)
    for Q in (Qg, Qu, Qd):  # no NaN codes
        Q[(Q & 0x7F) == 0x7F] = 0x30
    sc = np.exp2(rng.integers(-8, -3, (E, 3))).astype(np.float32)
    res = O.moe_forward_fp8(X, W_r, b, Qg, Qu, Qd, sc, k)
    lib = lambda Q, s: (torch.from_numpy(Q).view(torch.float8_e4m3fn).double().numpy()
                        * s.reshape(-1, 1, 1))
    ref = O.moe_forward(X, W_r, b, lib(Qg, sc[:, 0]), lib(Qu, sc[:, 1]),
                        lib(Qd, sc[:, 2]), k)
    np.testing.assert_array_equal(res["out"], ref["out"])
    # a power-of-two scale is exact: halving the codes' values and doubling the
    # scale changes nothing (codes 0x38 = 1.0 and 0x30 = 0.5)
    one = np.full((E, dff, d), 0x38, np.uint8)
    half = np.full((E, dff, d), 0x30, np.uint8)
    np.testing.assert_array_equal(O.dequant_expert_weights(one, sc[:, 0]),
                                  O.dequant_expert_weights(half, 2 * sc[:, 0]))


# ------------------------------------------------------- router statistics --
def test_router_stats_uniform_router_closed_forms():
    """Equal logits: every mean probability is 1/E, the z-loss is (ln E)^2
    and the auxiliary loss is exactly 1 whatever the routing."""
    T, E, k = 7, 6, 2
    lg = np.full((T, E), 0.75, dtype=np.float32)
    idx, _ = O.select_topk(lg, k)
    w = O.gate_weights(lg, idx, O.TOPK_THEN_SOFTMAX)
    st = O.router_stats(lg, idx, w)
    np.testing.assert_allclose(st["mean_prob"], 1.0 / E, rtol=1e-14)
    np.testing.assert_allclose(st["z_loss"], (0.75 + math.log(E)) ** 2, rtol=1e-14)
    assert abs(st["aux_loss"] - 1.0) < 1e-14
    # ties go to the lower ids: experts 0 and 1 take every token at weight 1/2
    np.testing.assert_array_equal(st["count"], [T, T, 0, 0, 0, 0])
    np.testing.assert_allclose(st["importance"], [T / 2, T / 2, 0, 0, 0, 0])


def test_router_stats_worked_example():
    """The pages' top-2 token: logits 2.0 (id 3) and 1.6 (id 5) give
    importance sigma(0.4) and sigma(-0.4); z from the library logsumexp."""
    g = _gold("worked_example_top2.json")
    lg = np.array([g["logits"]], dtype=np.float32)
    idx, _ = O.select_topk(lg, 2)
    w = O.gate_weights(lg, idx, O.TOPK_THEN_SOFTMAX)
    st = O.router_stats(lg, idx, w)
    s = 1.0 / (1.0 + math.exp(-0.4))
    np.testing.assert_allclose(st["importance"][3], s, rtol=1e-7)
    np.testing.assert_allclose(st["importance"][5], 1 - s, rtol=1e-7)
    lse = scipy.special.logsumexp(lg.astype(np.float64)[0])
    np.testing.assert_allclose(st["z_loss"], lse ** 2, rtol=1e-13)
    np.testing.assert_allclose(st["mean_prob"],
                               scipy.special.softmax(lg.astype(np.float64)[0]), rtol=1e-13)


@pytest.mark.parametrize("gating", [O.TOPK_THEN_SOFTMAX, O.SOFTMAX_THEN_TOPK])
def test_router_stats_invariants_and_library(gating):
    rng = np.random.default_rng(61)
    T, E, k = 50, 9, 3
    lg = (rng.standard_normal((T, E)) * 3).astype(np.float32)
    idx, _ = O.select_topk(lg, k)
    w = O.gate_weights(lg, idx, gating)
    st = O.router_stats(lg, idx, w)
    # every token's weights sum to one, probabilities sum to one, counts to T k
    np.testing.assert_allclose(st["importance"].sum(), T, rtol=1e-12)
    np.testing.assert_allclose(st["mean_prob"].sum(), 1.0, rtol=1e-12)
    assert st["count"].sum() == T * k
    np.testing.assert_array_equal(st["count"], np.bincount(idx.ravel(), minlength=E))
    l64 = lg.astype(np.float64)
    np.testing.assert_allclose(st["mean_prob"], scipy.special.softmax(l64, axis=1).mean(0),
                               rtol=1e-12)
    np.testing.assert_allclose(st["z_loss"], np.mean(scipy.special.logsumexp(l64, axis=1) ** 2),
                               rtol=1e-12)
    imp = np.zeros(E)
    np.add.at(imp, idx.ravel(), w.ravel())
    np.testing.assert_allclose(st["importance"], imp, rtol=1e-12)
    f = np.bincount(idx.ravel(), minlength=E) / (T * k)
    np.testing.assert_allclose(st["aux_loss"], E * np.dot(f, st["mean_prob"]), rtol=1e-12)


def test_router_stats_all_to_one_expert():
    """k = 1 and every token on expert 0: aux = E * mean_prob[0]."""
    T, E = 11, 4
    lg = np.zeros((T, E), dtype=np.float32)
    lg[:, 0] = 5.0
    idx, _ = O.select_topk(lg, 1)
    w = O.gate_weights(lg, idx, O.TOPK_THEN_SOFTMAX)
    st = O.router_stats(lg, idx, w)
    p0 = math.exp(5.0) / (math.exp(5.0) + 3.0)
    np.testing.assert_allclose(st["aux_loss"], E * p0, rtol=1e-12)
    np.testing.assert_allclose(st["importance"], [T, 0, 0, 0])


# ----------------------------------------------------------- shared expert --
def _torch_swiglu(X, Wg, Wu, Wd):
    F = torch.nn.functional
    Xt = torch.from_numpy(np.asarray(X, dtype=np.float64))
    g, u, dn = (torch.from_numpy(np.asarray(v, dtype=np.float64)) for v in (Wg, Wu, Wd))
    return F.linear(F.silu(F.linear(Xt, g)) * F.linear(Xt, u), dn).numpy()


def test_shared_expert_is_library_swiglu_on_every_token():
    X, W_r, b, Wg, Wu, Wd = _rand_layer(17, 16, 4, 2, 12, seed=41)
    rng = np.random.default_rng(42)
    Sg, Su = rng.standard_normal((2, 20, 16)) / 4
    Sd = rng.standard_normal((16, 20)) / 4
    np.testing.assert_allclose(O.shared_expert_ffn(X, Sg, Su, Sd),
                               _torch_swiglu(X, Sg, Su, Sd), rtol=1e-12,
                               atol=1e-12)


def test_shared_expert_is_a_one_expert_routed_layer():
    """An E = 1, k = 1 routed layer sends every token to its expert with gate
    weight exactly 1: the same map as the shared expert."""
    X, W_r, b, Wg, Wu, Wd = _rand_layer(13, 8, 1, 1, 10, seed=43)
    routed = O.moe_forward(X, W_r, b, Wg, Wu, Wd, 1)["out"]
    np.testing.assert_allclose(O.shared_expert_ffn(X, Wg[0], Wu[0], Wd[0]),
                               routed, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("cf", [None, 0.5])
def test_layer_with_shared_expert_matches_brute_force(cf):
    X, W_r, b, Wg, Wu, Wd = _rand_layer(30, 8, 5, 2, 12, seed=44,
                                        bias_scale=1.0)
    rng = np.random.default_rng(45)
    Sg, Su = rng.standard_normal((2, 6, 8)) / 3
    Sd = rng.standard_normal((8, 6)) / 3
    res = O.moe_forward_shared(X, W_r, b, Wg, Wu, Wd, Sg, Su, Sd, 2, cf)
    ref = (_brute_force(X, W_r, b, Wg, Wu, Wd, 2, cf, O.TOPK_THEN_SOFTMAX)
           + _torch_swiglu(X, Sg, Su, Sd))
    np.testing.assert_allclose(res["out"], ref, rtol=1e-10, atol=1e-12)
    # a zero shared expert leaves the routed layer unchanged; tokens whose
    # copies were all dropped still get the shared expert's output
    z = O.moe_forward_shared(X, W_r, b, Wg, Wu, Wd, 0 * Sg, 0 * Su, 0 * Sd, 2, cf)
    np.testing.assert_array_equal(z["out"], O.moe_forward(X, W_r, b, Wg, Wu, Wd, 2, cf)["out"])
    if cf is not None:
        empty = np.all(res["dest"] < 0, axis=1)
        assert empty.any()
        np.testing.assert_allclose(res["out"][empty], _torch_swiglu(X[empty], Sg, Su, Sd),
                                   rtol=1e-12, atol=1e-12)


def test_round_bf16_matches_torch_conversion():
    rng = np.random.default_rng(16)
    x = (rng.standard_normal(100000) * 10.0 ** rng.integers(-5, 5, 100000)
         ).astype(np.float32)
    x[:4] = [0.0, -0.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8]  # ties
    ours = W.round_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(ours, ref)


def test_workloads_are_seeded_and_shaped():
    w = W.WORKLOADS["tiny"]
    a, b = W.make_host(w), W.make_host(w)
    for key in ("X", "W_r", "W_gate", "W_up", "W_down"):
        np.testing.assert_array_equal(a[key], b[key])
    assert a["X"].shape == (64, 128) and a["W_down"].shape == (8, 128, 256)
    assert a["bias"] is None
    w = W.WORKLOADS["gptoss"].replace(T=16, d_model=64, d_ff=64)
    W_r, bias = W.make_router(w)
    p = np.exp(bias.astype(np.float64))
    np.testing.assert_allclose(np.sort(p)[::-1] / p.max(),
                               np.arange(1, 33) ** -1.2, rtol=1e-5)


# -------------------------------------------------------------- backward --
def _fd_forward(X, W_r, b, Wg, Wu, Wd, idx, C, gating):
    """The layer in fp64 with the selection ``idx`` held fixed and fp64
    logits: the function whose derivatives the backward states."""
    T, E = X.shape[0], W_r.shape[0]
    l = np.asarray(X, np.float64) @ np.asarray(W_r, np.float64).T
    if b is not None:
        l = l + np.asarray(b, np.float64)
    w = O.gate_weights(l, idx, gating)
    a = O.assign(idx, E, C)
    Xp = np.asarray(X, np.float64)[a["row_token"]]
    Y = O.grouped_ffn(Xp, a["offsets"], Wg, Wu, Wd)
    return O.combine(Y, a["dest"], w, T)


@pytest.mark.parametrize("gating,cf,bias", [
    (O.TOPK_THEN_SOFTMAX, None, 0.0),
    (O.SOFTMAX_THEN_TOPK, None, 1.0),
    (O.TOPK_THEN_SOFTMAX, 0.6, 1.5),
])
def test_backward_matches_central_differences(gating, cf, bias):
    """Every coordinate of every gradient against a central difference of
    the loss sum(dout * out), selection fixed."""
    T, d, E, k, d_ff = 7, 6, 4, 2, 5
    X, W_r, b, Wg, Wu, Wd = _rand_layer(T, d, E, k, d_ff, seed=71, bias_scale=bias)
    if b is None:
        b = np.zeros(E, np.float32)
    X, W_r, b, Wg, Wu, Wd = (np.asarray(v, np.float64) for v in (X, W_r, b, Wg, Wu, Wd))
    dout = np.random.default_rng(72).standard_normal((T, d))
    g = O.moe_backward(X, W_r, b, Wg, Wu, Wd, dout, k, cf, gating)
    C = O.capacity(T, k, E, cf)
    if cf is not None:
        assert (g["dest"] < 0).any()
    params = dict(X=X, W_r=W_r, b=b, Wg=Wg, Wu=Wu, Wd=Wd)
    names = dict(X="dX", W_r="dW_r", b="dbias", Wg="dW_gate", Wu="dW_up", Wd="dW_down")
    h = 1e-6
    for pname, arr in params.items():
        fd = np.zeros_like(arr)
        for i in np.ndindex(arr.shape):
            old = arr[i]
            arr[i] = old + h
            lp = np.sum(dout * _fd_forward(**params, idx=g["idx"], C=C, gating=gating))
            arr[i] = old - h
            lm = np.sum(dout * _fd_forward(**params, idx=g["idx"], C=C, gating=gating))
            arr[i] = old
            fd[i] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(g[names[pname]], fd, rtol=2e-5, atol=2e-7,
                                   err_msg=pname)


def _torch_layer(X, W_r, b, Wg, Wu, Wd, idx, dest, gating):
    """Autograd reference: the layer written with torch ops (fp64), routing
    given by ``idx`` and ``dest``; gating 1 takes the full softmax, gathers
    the selected probabilities and renormalises them."""
    l = X @ W_r.T + b
    idx_t = torch.from_numpy(np.asarray(idx, np.int64))
    if gating == O.TOPK_THEN_SOFTMAX:
        w = torch.softmax(torch.gather(l, 1, idx_t), dim=1)
    else:
        p = torch.gather(torch.softmax(l, dim=1), 1, idx_t)
        w = p / p.sum(dim=1, keepdim=True)
    T, k = idx_t.shape
    out = torch.zeros(T, Wd.shape[1], dtype=torch.float64)
    for t in range(T):
        for j in range(k):
            if dest[t, j] >= 0:
                e = int(idx_t[t, j])
                x = X[t:t + 1]
                h = torch.nn.functional.silu(x @ Wg[e].T) * (x @ Wu[e].T)
                out[t] += w[t, j] * (h @ Wd[e].T)[0]
    return out


@pytest.mark.parametrize("gating,cf", [(O.TOPK_THEN_SOFTMAX, None),
                                       (O.SOFTMAX_THEN_TOPK, 0.7)])
def test_backward_matches_library_autograd(gating, cf):
    T, d, E, k, d_ff = 20, 8, 5, 3, 6
    X, W_r, b, Wg, Wu, Wd = _rand_layer(T, d, E, k, d_ff, seed=73, bias_scale=1.0)
    dout = np.random.default_rng(74).standard_normal((T, d))
    g = O.moe_backward(X, W_r, b, Wg, Wu, Wd, dout, k, cf, gating)
    leaves = [torch.from_numpy(np.asarray(v, np.float64)).requires_grad_()
              for v in (X, W_r, b, Wg, Wu, Wd)]
    out = _torch_layer(*leaves, g["idx"], g["dest"], gating)
    (out * torch.from_numpy(dout)).sum().backward()
    for leaf, name in zip(leaves, ("dX", "dW_r", "dbias", "dW_gate", "dW_up", "dW_down")):
        # the oracle's gate weights come from fp32-rounded logits
        np.testing.assert_allclose(g[name], leaf.grad.numpy(), rtol=1e-5, atol=1e-7,
                                   err_msg=name)


def test_backward_single_expert_is_dense_swiglu_backward():
    """E = 1, k = 1: every gate weight is 1, so the router gets no gradient
    and the rest is the dense SwiGLU FFN's backward."""
    X, W_r, b, Wg, Wu, Wd = _rand_layer(9, 8, 1, 1, 10, seed=75, bias_scale=1.0)
    dout = np.random.default_rng(76).standard_normal((9, 8))
    g = O.moe_backward(X, W_r, b, Wg, Wu, Wd, dout, 1)
    assert np.all(g["dW_r"] == 0) and np.all(g["dbias"] == 0)
    xs = [torch.from_numpy(np.asarray(v, np.float64)).requires_grad_()
          for v in (X, Wg[0], Wu[0], Wd[0])]
    y = torch.nn.functional.linear(
        torch.nn.functional.silu(torch.nn.functional.linear(xs[0], xs[1]))
        * torch.nn.functional.linear(xs[0], xs[2]), xs[3])
    (y * torch.from_numpy(dout)).sum().backward()
    for got, leaf in zip((g["dX"], g["dW_gate"][0], g["dW_up"][0], g["dW_down"][0]), xs):
        np.testing.assert_allclose(got, leaf.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_backward_top1_softmax_gives_no_router_gradient():
    """k = 1 with the softmax over the selected logits: w = 1 whatever the
    logits, so dW_r and dbias are exactly zero."""
    X, W_r, b, Wg, Wu, Wd = _rand_layer(15, 8, 4, 1, 6, seed=77, bias_scale=1.0)
    dout = np.random.default_rng(78).standard_normal((15, 8))
    g = O.moe_backward(X, W_r, b, Wg, Wu, Wd, dout, 1)
    assert np.all(g["dl"] == 0) and np.all(g["dW_r"] == 0) and np.all(g["dbias"] == 0)


def test_backward_identical_experts_match_dense_ffn():
    """Identical experts, no capacity: the layer is the dense FFN for any
    routing (the gate weights sum to 1), so the router gradient vanishes and
    the experts' weight gradients sum to the dense FFN's."""
    X, W_r, b, Wg, Wu, Wd = _rand_layer(16, 8, 4, 2, 6, seed=79, bias_scale=1.0)
    Wg[:], Wu[:], Wd[:] = Wg[0], Wu[0], Wd[0]
    dout = np.random.default_rng(80).standard_normal((16, 8))
    for gating in (O.TOPK_THEN_SOFTMAX, O.SOFTMAX_THEN_TOPK):
        g = O.moe_backward(X, W_r, b, Wg, Wu, Wd, dout, 2, None, gating)
        dA, dWg, dWu, dWd = O.expert_ffn_backward(X, Wg[0], Wu[0], Wd[0], dout)
        np.testing.assert_allclose(g["dW_r"], 0, atol=1e-12)
        np.testing.assert_allclose(g["dbias"], 0, atol=1e-12)
        np.testing.assert_allclose(g["dX"], dA, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(g["dW_gate"].sum(0), dWg, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(g["dW_up"].sum(0), dWu, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(g["dW_down"].sum(0), dWd, rtol=1e-10, atol=1e-12)


def test_backward_invariants_with_drops():
    """Each token's logit gradient sums to zero (so does dbias, and every
    column of dW_r); a token whose copies were all dropped passes no gradient
    through the experts and none to its logits; unused experts get zero
    weight gradients."""
    T, d, E, k, d_ff = 40, 8, 6, 2, 6
    X, W_r, b, Wg, Wu, Wd = _rand_layer(T, d, E, k, d_ff, seed=81)
    b = np.array([8, 7, -30, -30, -30, -30], np.float32)  # experts 0, 1 take everything
    dout = np.random.default_rng(82).standard_normal((T, d))
    g = O.moe_backward(X, W_r, b, Wg, Wu, Wd, dout, k, capacity_factor=0.9)
    np.testing.assert_allclose(g["dl"].sum(axis=1), 0, atol=1e-12)
    np.testing.assert_allclose(g["dbias"].sum(), 0, atol=1e-11)
    np.testing.assert_allclose(g["dW_r"].sum(axis=0), 0, atol=1e-10)
    gone = np.all(g["dest"] < 0, axis=1)
    assert gone.any()
    np.testing.assert_array_equal(g["dl"][gone], 0)
    np.testing.assert_allclose(g["dX"][gone], 0, atol=0)
    unused = np.diff(g["offsets"]) == 0
    assert unused.any()
    for name in ("dW_gate", "dW_up", "dW_down"):
        assert np.all(g[name][unused] == 0)
