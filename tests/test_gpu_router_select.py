"""Router selection with a group of 8 or 16 lanes per token (moe_route with at
least 128 tokens and k <= 8) against the one-wavefront-per-token selection
that moe_route_stats keeps, bit for bit (ids and gate weights), and both
against the oracle's routing: every group shape (E from 3 to 256), k from 1
to 8, both gating orders, a Zipf router bias, and exact ties between two
duplicated router rows (the lower expert id is taken first).  Cases with
fewer tokens or k > 8 run the wavefront kernel in both calls.

Ties and order: "Sparsely-Gated MoE 구현 관점에서 살펴보기" (molayo1419.me),
sections "Top-2 라우팅의 수치 예시" and "pure Python으로 Top-k Router 확인하기"."""

import numpy as np
import pytest
import torch

import oracle as O
from mixture_experts_layer_wavefront_amd import binding as B
from mixture_experts_layer_wavefront_amd import workloads as W

from parity_util import check_routing, problem_of, to_device

pytestmark = pytest.mark.gpu

TK, ST = W.TOPK_THEN_SOFTMAX, W.SOFTMAX_THEN_TOPK

# (T, E, k, gating, zipf, duplicated router rows or None)
CASES = {
    "E3_k1": (300, 3, 1, TK, 0.0, None),
    "E3_k3_st": (300, 3, 3, ST, 0.0, None),
    "E8_k2": (1030, 8, 2, TK, 0.0, (2, 5)),
    "E8_k8_st": (300, 8, 8, ST, 1.2, None),
    "E13_k5": (257, 13, 5, TK, 1.2, (4, 11)),
    "E16_k4_st": (300, 16, 4, ST, 0.0, None),
    "E24_k3": (300, 24, 3, TK, 0.0, (7, 20)),
    "E32_k4": (513, 32, 4, TK, 1.2, None),
    "E32_k8_st": (300, 32, 8, ST, 0.0, (1, 30)),
    "E50_k6": (300, 50, 6, TK, 0.0, None),
    "E64_k8": (300, 64, 8, TK, 1.2, (10, 63)),
    "E64_k1_st": (300, 64, 1, ST, 0.0, None),
    "E65_k2": (300, 65, 2, TK, 0.0, (0, 64)),
    "E100_k7_st": (300, 100, 7, ST, 1.2, None),
    "E128_k8": (700, 128, 8, TK, 1.2, (33, 97)),
    "E128_k8_st": (300, 128, 8, ST, 0.0, None),
    "E129_k3": (300, 129, 3, TK, 0.0, (64, 128)),
    "E200_k8_st": (300, 200, 8, ST, 1.2, (5, 150)),
    "E256_k8_st": (400, 256, 8, ST, 0.0, (100, 228)),
    "E256_k5": (300, 256, 5, TK, 1.2, None),
    # the wavefront kernel in both calls: fewer tokens, k > 8
    "few_tokens_E128_k8": (100, 128, 8, TK, 0.0, (3, 9)),
    "E64_k12": (300, 64, 12, TK, 0.0, None),
}


@pytest.mark.parametrize("name", list(CASES))
def test_group_select_matches_wavefront_select_and_oracle(name):
    T, E, k, gating, zipf, dup = CASES[name]
    wl = W.Workload(f"select_{name}", T, 64, E, k, 8, W.BF16, gating, 0.0, zipf,
                    3000 + sum(map(ord, name)))
    print(f"[select] {name} T={T} E={E} k={k} gating={gating} dup={dup}", flush=True)
    host = W.make_host(wl)
    if dup is not None:
        e1, e2 = dup
        host["W_r"][e2] = host["W_r"][e1]
        if host["bias"] is not None:
            host["bias"][e2] = host["bias"][e1]
    dev = to_device(host, wl)
    p = problem_of(wl)
    idx, w = B.moe_route(p, dev["X"], dev["W_r"], dev["bias"])
    idx1, w1, _ = B.moe_route_stats(p, dev["X"], dev["W_r"], dev["bias"])
    torch.cuda.synchronize()
    assert torch.equal(idx, idx1)
    assert torch.equal(w, w1)
    g_idx, g_w = idx.cpu().numpy(), w.cpu().numpy()
    o_idx, o_w, near, logits = O.route(host["X"], host["W_r"], host["bias"], k, gating)
    check_routing(g_idx, g_w, o_idx, o_w, near, logits)
    if dup is not None:
        e1, e2 = dup
        both = 0
        for t in range(T):
            row = g_idx[t].tolist()
            if e2 in row:
                # equal logits: the lower id comes first and is never left out
                assert e1 in row and row.index(e1) < row.index(e2), (t, row)
                both += 1
        print(f"[select] {name}: tokens selecting both tied experts {both}", flush=True)
