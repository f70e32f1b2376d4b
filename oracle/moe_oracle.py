"""CPU oracle for the forward and backward passes of one sparsely-gated MoE
FFN layer.

TEST INFRASTRUCTURE ONLY.  This module is the slow, plain, fp64 statement of
what the layer computes.  Only the test-suite, the package smoke check and the
``cpu_baseline`` leg of the benchmark may import or call it.  The HIP library
never imports it, links it or calls it, and it shares no code with that
library (no kernels, headers, helpers, tables or constants).

Sources (web pages, cited by title and section):

* [SG]   "Sparsely-Gated MoE 구현 관점에서 살펴보기: Router, Top-k, 부하 분산"
         (molayo1419.me) -- the method page.  Sections used: "Router를 텐서
         형태에서 추적하기" (router tensor shapes), "Top-2 라우팅의 수치 예시"
         (top-2 worked example), "순전파 과정(forward pass)은 디스패치와
         결합(combine)을 포함" (the five-step forward pipeline), "로드 밸런싱
         손실과 용량은 별개" (capacity and overflow), "pure Python으로 Top-k
         Router 확인하기" (stable softmax over the selected logits).
* [EP]   "5.3 Expert Parallelism" (sungeuns.github.io), section
         "3. 고도화된 최적화" / "최적화 2: GroupGEMM" (the per-expert loop).
* [HF]   "Expert를 똑같이 나눴는데도 GPU가 대기하는 이유: MoE의 토큰 쏠림"
         (portfolio.ywsung.com), table "실행 백엔드별 메커니즘과 최적
         시나리오" (the ``eager`` backend: a sequential per-expert loop, meant
         for correctness checking).
* [MOON] "가장 바쁜 랭크가 속도를 정합니다: MoonEP의 계획 코드를 직접
         돌려봤습니다" (thakicloud.com), section "설치 및 통합" (packed
         per-projection weights, ``cu_seqlens`` selecting each expert's rows,
         ``tokens_per_expert``).

Readings where the pages are silent or garbled (each also listed in the
repository's design notes):

* The expert FFN is SwiGLU: ``y = (silu(x Wg^T) * (x Wu^T)) Wd^T`` with
  ``silu(z) = z / (1 + exp(-z))``; no biases.  The pages do not define the
  expert FFN; this form is the one the workloads name.
* Weights are stored ``[E, out, in]`` so that every product is ``A @ W.T``, as
  in the router's ``X @ W_r.T`` ([SG] forward pipeline).
* Ties among equal logits go to the lower expert id; selected slots are
  ordered by descending logit.
* Capacity is ``C = min(T, ceil(cf * T * k / E))`` (the printed formula is
  lost in [SG] "capacity").  Overflow is resolved first-come in token order:
  each expert keeps its C lowest token ids.  A dropped copy contributes zero;
  the surviving weights are not renormalised; nothing is re-routed.
* Logits are fp32: the dot product is accumulated in fp64, rounded to fp32,
  then the fp32 bias is added in fp32.  Gate weights are computed in fp64.

Parity pins: every function here is pinned by ``tests/test_oracle.py``
against the worked example, closed forms, invariants, textbook special cases
and brute force; see the docstrings for which pin covers which step.
"""

from __future__ import annotations

import math

import numpy as np

TOPK_THEN_SOFTMAX = 0
SOFTMAX_THEN_TOPK = 1

# A token whose k-th and (k+1)-th fp32 logits differ by less than this is a
# near tie: its expert set is not decided robustly by fp32 rounding.
NEAR_TIE_GAP = 1e-5


def _f64(a):
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------------------
# O1  router logits            [SG] "Router를 텐서 형태에서 추적하기";
#                              [SG] forward pipeline, step 1 (X @ W_r.T)
# ---------------------------------------------------------------------------
def router_logits(X, W_r, bias=None):
    """Router logits ``l[t, e] = fp32(sum_i X[t,i] W_r[e,i]) + b[e]``.

    X: [T, d] (values exactly representable in fp32), W_r: [E, d] fp32,
    bias: [E] fp32 or None.  The dot products are accumulated in fp64 and
    rounded once to fp32; the bias is then added in fp32 arithmetic.
    Returns [T, E] float32.
    """
    l64 = _f64(X) @ _f64(W_r).T
    l32 = l64.astype(np.float32)
    if bias is not None:
        l32 = (l32 + np.asarray(bias, dtype=np.float32)).astype(np.float32)
    return l32


# ---------------------------------------------------------------------------
# O2/O3  top-k selection and gate weights
#        [SG] "Top-2 라우팅의 수치 예시" (select k largest, renormalise with
#        softmax over the selected logits; ids are 0-based);
#        [SG] "pure Python으로 Top-k Router 확인하기" (stable softmax: the max
#        selected logit is subtracted before exponentiating);
#        [SG] same example section, last paragraph (the other order:
#        softmax over all experts first, then top-k, then renormalise).
# ---------------------------------------------------------------------------
def select_topk(logits, k):
    """Per row, the k largest logits ordered by (logit desc, expert id asc).

    Returns (idx [T,k] int32, near_tie [T] bool).  ``near_tie[t]`` is set when
    k < E and the gap between the k-th and (k+1)-th largest logit is below
    ``NEAR_TIE_GAP``.
    """
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    # A stable sort of the negated logits orders equal logits by ascending id.
    order = np.argsort(-logits.astype(np.float64), axis=1, kind="stable")
    idx = order[:, :k].astype(np.int32)
    if k < E:
        srt = np.take_along_axis(logits, order, axis=1).astype(np.float64)
        near_tie = (srt[:, k - 1] - srt[:, k]) < NEAR_TIE_GAP
    else:
        near_tie = np.zeros(T, dtype=bool)
    return idx, near_tie


def gate_weights(logits, idx, gating):
    """Gate weights for the selected experts, in fp64.

    TOPK_THEN_SOFTMAX: ``w_j = exp(l_j - m) / sum_{j' in S} exp(l_j' - m)``
    with ``m`` the largest selected logit.
    SOFTMAX_THEN_TOPK: ``p = softmax(l)`` over all E experts (max-shifted),
    then ``w_j = p_j / sum_{j' in S} p_j'``.
    Returns [T, k] float64.
    """
    l = _f64(logits)
    sel = np.take_along_axis(l, np.asarray(idx, dtype=np.int64), axis=1)
    if gating == TOPK_THEN_SOFTMAX:
        m = sel.max(axis=1, keepdims=True)
        ex = np.exp(sel - m)
        return ex / ex.sum(axis=1, keepdims=True)
    if gating == SOFTMAX_THEN_TOPK:
        M = l.max(axis=1, keepdims=True)
        ex = np.exp(l - M)
        p = ex / ex.sum(axis=1, keepdims=True)
        psel = np.take_along_axis(p, np.asarray(idx, dtype=np.int64), axis=1)
        return psel / psel.sum(axis=1, keepdims=True)
    raise ValueError(f"unknown gating {gating}")


def route(X, W_r, bias, k, gating):
    """Router step: logits -> (topk_idx int32 [T,k], topk_w fp64 [T,k],
    near_tie bool [T], logits fp32 [T,E])."""
    logits = router_logits(X, W_r, bias)
    idx, near_tie = select_topk(logits, k)
    w = gate_weights(logits, idx, gating)
    return idx, w, near_tie, logits


# ---------------------------------------------------------------------------
# O4-O6  counts, capacity, slots      [SG] forward pipeline step 2 (assign
#        per-expert capacity slots); [SG] "로드 밸런싱 손실과 용량은 별개"
#        (capacity bounds the tokens one expert takes; overflow is dropped);
#        [MOON] "설치 및 통합" (tokens_per_expert, cu_seqlens);
#        [EP] "2. 디스패처 엔지니어링" (bincount of the routed ids).
# ---------------------------------------------------------------------------
def capacity(T, k, E, capacity_factor):
    """Per-expert capacity ``min(T, ceil(cf*T*k/E))``; None means unlimited
    (capacity_factor <= 0 or None)."""
    if capacity_factor is None or capacity_factor <= 0:
        return None
    return min(T, int(math.ceil(capacity_factor * T * k / E)))


def assign(idx, E, C):
    """Assign capacity slots, first-come in token-major order.

    Walks the copies (t, j) with t = 0..T-1 outer and j = 0..k-1 inner; copy
    (t, j) takes slot ``pos = fill[e]`` of expert ``e = idx[t, j]`` and is kept
    iff ``pos < C`` (always kept when C is None).

    Returns a dict with
      counts  [E]   int64  raw copies per expert (before capacity)
      kept    [E]   int64  min(counts, C)
      offsets [E+1] int64  exclusive prefix sum of kept (cu_seqlens)
      dest    [T,k] int64  row of the copy in expert-contiguous order, -1 if dropped
      row_token [N] int64  token id of each kept row
      dropped int          number of dropped copies
    """
    idx = np.asarray(idx)
    T, k = idx.shape
    counts = np.zeros(E, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            counts[idx[t, j]] += 1
    cap = np.iinfo(np.int64).max if C is None else int(C)
    kept = np.minimum(counts, cap)
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + kept[e]
    fill = np.zeros(E, dtype=np.int64)
    dest = np.full((T, k), -1, dtype=np.int64)
    row_token = np.full(int(offsets[E]), -1, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            pos = fill[e]
            fill[e] += 1
            if pos < cap:
                r = offsets[e] + pos
                dest[t, j] = r
                row_token[r] = t
    dropped = int((counts - kept).sum())
    return dict(counts=counts, kept=kept, offsets=offsets, dest=dest,
                row_token=row_token, dropped=dropped)


# ---------------------------------------------------------------------------
# O7  permute / dispatch           [SG] forward pipeline step 3 (reorder the
#                                  tokens in expert order and dispatch them)
# ---------------------------------------------------------------------------
def gather_rows(X, row_token):
    """``X_perm[r] = X[row_token[r]]`` (values copied unchanged)."""
    X = np.asarray(X)
    return X[np.asarray(row_token, dtype=np.int64)]


# ---------------------------------------------------------------------------
# O8  per-expert FFN, one expert at a time
#     [SG] forward pipeline step 4 (run each expert's FFN on its batch);
#     [EP] "최적화 2: GroupGEMM" (the plain loop over local experts);
#     [HF] backend table (``eager``: sequential loop per expert, for
#     correctness checking).
# ---------------------------------------------------------------------------
def silu(z):
    z = _f64(z)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_ffn(A, Wg, Wu, Wd):
    """One expert's SwiGLU FFN on the rows A [n, d], all in fp64:
    ``(silu(A Wg^T) * (A Wu^T)) Wd^T`` with Wg, Wu [d_ff, d] and Wd [d, d_ff].
    """
    A = _f64(A)
    G = A @ _f64(Wg).T
    U = A @ _f64(Wu).T
    H = silu(G) * U
    return H @ _f64(Wd).T


def grouped_ffn(X_perm, offsets, W_gate, W_up, W_down):
    """Loop over experts e = 0..E-1, each on its rows [offsets[e], offsets[e+1]).
    Returns Y_perm [N, d] fp64."""
    X_perm = _f64(X_perm)
    E = len(offsets) - 1
    d = W_down.shape[1]
    Y = np.zeros((int(offsets[E]), d), dtype=np.float64)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            Y[lo:hi] = expert_ffn(X_perm[lo:hi], W_gate[e], W_up[e], W_down[e])
    return Y


# ---------------------------------------------------------------------------
# O9  unpermute + gate-weighted combine
#     [SG] "Router를 텐서 형태에서 추적하기" (the layer output is the weighted
#     average of the selected experts' outputs; unselected experts contribute
#     nothing); [SG] forward pipeline step 5 (un-permute, combine with the
#     router weights, original token order).
# ---------------------------------------------------------------------------
def combine(Y_perm, dest, w, T):
    """``out[t] = sum_{j : dest[t,j] >= 0} w[t,j] * Y_perm[dest[t,j]]`` (fp64).
    A token whose copies were all dropped gets a zero row."""
    Y_perm = _f64(Y_perm)
    dest = np.asarray(dest)
    w = _f64(w)
    d = Y_perm.shape[1] if Y_perm.ndim == 2 else 0
    out = np.zeros((T, d), dtype=np.float64)
    for t in range(T):
        for j in range(dest.shape[1]):
            r = dest[t, j]
            if r >= 0:
                out[t] += w[t, j] * Y_perm[r]
    return out


# ---------------------------------------------------------------------------
# The whole layer.
# ---------------------------------------------------------------------------
def moe_forward(X, W_r, bias, W_gate, W_up, W_down, k, capacity_factor=None,
                gating=TOPK_THEN_SOFTMAX):
    """Forward pass of the layer, [SG] forward pipeline steps 1-5 in order.

    Returns a dict with ``out`` [T, d] fp64 plus every intermediate
    (idx, w, near_tie, logits, counts, kept, offsets, dest, row_token,
    dropped, C, X_perm, Y_perm).
    """
    X = np.asarray(X)
    T = X.shape[0]
    E = W_r.shape[0]
    idx, w, near_tie, logits = route(X, W_r, bias, k, gating)
    C = capacity(T, k, E, capacity_factor)
    a = assign(idx, E, C)
    X_perm = gather_rows(X, a["row_token"])
    Y_perm = grouped_ffn(X_perm, a["offsets"], W_gate, W_up, W_down)
    out = combine(Y_perm, a["dest"], w, T)
    res = dict(out=out, idx=idx, w=w, near_tie=near_tie, logits=logits, C=C,
               X_perm=X_perm, Y_perm=Y_perm)
    res.update(a)
    return res


# ---------------------------------------------------------------------------
# Expert weights stored as FP8 with a scale per expert and projection
#     [HF] sections "Weight Loading에서 텐서 구조 맞추기" and "적재 변환과
#     양자화 조합하기": once the experts sit in one packed tensor, a
#     per-expert quantisation step fits into weight loading.  Reading (the
#     page names no format): each expert's W_gate, W_up, W_down is stored as
#     FP8 E4M3 codes (the OCP "FN" variant: bias 7, no infinities, one NaN
#     pattern per sign, largest finite 448) times one fp32 scale per
#     (expert, projection); the layer is the same SwiGLU layer on the decoded
#     weights  W = scale * decode(code).  Activations stay as they are.
# ---------------------------------------------------------------------------
def fp8_e4m3_decode(codes):
    """Values (fp64) of FP8 E4M3 codes: bit 7 sign, bits 6..3 exponent (bias
    7), bits 2..0 mantissa; exponent 0 is subnormal (m/8 * 2^-6); exponent 15
    with mantissa 7 is NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6,
                   (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


def dequant_expert_weights(Q, scales):
    """Decoded weights ``scales[e] * decode(Q[e])`` (fp64) for codes Q
    [E, out, in] and one scale per expert [E]."""
    dec = fp8_e4m3_decode(Q)
    return dec * _f64(scales).reshape(-1, *([1] * (dec.ndim - 1)))


def moe_forward_fp8(X, W_r, bias, Qg, Qu, Qd, scales, k, capacity_factor=None,
                    gating=TOPK_THEN_SOFTMAX):
    """The layer with FP8 expert weights: ``moe_forward`` on the decoded
    weights; scales [E, 3] hold the (gate, up, down) scale of each expert."""
    sc = _f64(scales)
    return moe_forward(X, W_r, bias, dequant_expert_weights(Qg, sc[:, 0]),
                       dequant_expert_weights(Qu, sc[:, 1]),
                       dequant_expert_weights(Qd, sc[:, 2]), k, capacity_factor,
                       gating)


# ---------------------------------------------------------------------------
# Router statistics (monitoring; forward values only, no gradients)
#     [SG] "로드 밸런싱 손실과 용량은 별개": the Sparsely-Gated MoE auxiliary
#     loss balances expert importance and load; GShard's auxiliary loss uses
#     the dispatch fraction and the mean gate value; ST-MoE's router z-loss
#     keeps router logits small.  [HF] "라우팅 분포와 학습 안정성" asks for
#     routing-distribution monitoring hooks.  Readings (the pages print no
#     formula; these are the published definitions the names refer to):
#       importance[e] = sum_t of the gate weight token t gives expert e
#                       (0 when e is not selected)
#       count[e]      = copies routed to e (top-k selections, before capacity)
#       mean_prob[e]  = mean over tokens of softmax over all E logits
#       aux_loss      = E * sum_e (count[e] / (T k)) * mean_prob[e]
#                       (1 for a uniform router with any routing)
#       z_loss        = mean over tokens of (logsumexp_e logit[t, e])^2
#     The logits are the router's fp32 logits (bias included).
# ---------------------------------------------------------------------------
def router_stats(logits, idx, w):
    """Router statistics from fp32 logits [T, E], selected ids [T, k] and gate
    weights [T, k]; fp64.  Returns dict importance, count, mean_prob [E] and
    aux_loss, z_loss (floats)."""
    lg = _f64(logits)
    T, E = lg.shape
    idx = np.asarray(idx)
    w = _f64(w)
    k = idx.shape[1] if idx.ndim == 2 else 0
    importance = np.zeros(E)
    count = np.zeros(E)
    for t in range(T):
        for j in range(k):
            importance[idx[t, j]] += w[t, j]
            count[idx[t, j]] += 1.0
    m = lg.max(axis=1, keepdims=True)
    ex = np.exp(lg - m)
    Z = ex.sum(axis=1, keepdims=True)
    prob = ex / Z
    lse = (m + np.log(Z))[:, 0]
    mean_prob = prob.mean(axis=0) if T else np.zeros(E)
    aux = float(E * np.sum(count / max(T * k, 1) * mean_prob))
    z = float(np.mean(lse ** 2)) if T else 0.0
    return dict(importance=importance, count=count, mean_prob=mean_prob,
                aux_loss=aux, z_loss=z)


# ---------------------------------------------------------------------------
# Shared expert (the DeepSeek-V3 layer form)
#     [EP] section "최적화 1: 공유 전문가를 통한 연산-통신 오버랩": next to the
#     N routed experts the layer has one shared expert that every token goes
#     through; its output is computed while the routed tokens are dispatched.
#     Reading (the page gives no formula): the shared expert is the same
#     SwiGLU FFN applied to every row, added to the routed mixture with weight
#     one, ``out = shared(x) + sum_j w_j expert_j(x)``.
# ---------------------------------------------------------------------------
def shared_expert_ffn(X, Ws_gate, Ws_up, Ws_down):
    """The shared expert on every token: ``expert_ffn`` over all rows, fp64."""
    return expert_ffn(X, Ws_gate, Ws_up, Ws_down)


def moe_forward_shared(X, W_r, bias, W_gate, W_up, W_down, Ws_gate, Ws_up,
                       Ws_down, k, capacity_factor=None,
                       gating=TOPK_THEN_SOFTMAX):
    """The routed layer plus the shared expert: ``moe_forward`` with
    ``out += shared_expert_ffn(X)``; the dict also holds ``shared``."""
    res = moe_forward(X, W_r, bias, W_gate, W_up, W_down, k, capacity_factor,
                      gating)
    sh = shared_expert_ffn(X, Ws_gate, Ws_up, Ws_down)
    res["shared"] = sh
    res["out"] = res["out"] + sh
    return res


def moe_forward_tokens(tokens, X, idx, w, dest, expert_weights, d_out):
    """Layer output for a subset of tokens, given the full routing.

    ``out[t]`` depends on the other tokens only through which of t's copies
    capacity kept (``dest``), so once routing and assignment have been done
    for every token, the output of a token is its own weighted sum of expert
    FFNs.  The experts are visited one at a time (ascending id) so that only
    one expert's weights are held at once; ``expert_weights(e)`` returns
    (Wg, Wu, Wd) for expert e.  Returns [len(tokens), d_out] fp64.
    """
    tokens = [int(t) for t in tokens]
    k = idx.shape[1]
    y = {}
    need = {}
    for t in tokens:
        for j in range(k):
            if dest[t, j] >= 0:
                need.setdefault(int(idx[t, j]), []).append((t, j))
    for e in sorted(need):
        Wg, Wu, Wd = expert_weights(e)
        for (t, j) in need[e]:
            y[(t, j)] = expert_ffn(_f64(X[t])[None, :], Wg, Wu, Wd)[0]
    out = np.zeros((len(tokens), d_out), dtype=np.float64)
    for i, t in enumerate(tokens):
        for j in range(k):
            if (t, j) in y:
                out[i] += w[t, j] * y[(t, j)]
    return out


# ---------------------------------------------------------------------------
# Backward pass of the layer
#     [HF] "Unsloth와의 MoE 학습 경로": training runs the same grouped expert
#     GEMMs as inference, now with gradients; [MOON] "이 기술은 무엇인가":
#     in training the expert weights' gradients flow back in the backward
#     pass.  The pages print no formula.  Reading: the gradients of a scalar
#     loss whose gradient with respect to the layer output is ``dout``, by
#     the chain rule through each forward step, with the top-k selection and
#     the capacity assignment held fixed (both are piecewise constant in the
#     inputs, so no gradient flows through them) and the fp32 rounding of the
#     logits taken as the identity.
#       combine     dY_perm[r] = w[t,j] dout[t] and dw[t,j] = <dout[t], Y_perm[r]>
#                   for a kept copy r = dest[t,j]; a dropped copy has dw = 0
#       expert FFN  on its rows A with G = A Wg^T, U = A Wu^T,
#                   H = silu(G) U, Y = H Wd^T:
#                   dH = dY Wd, dWd = dY^T H, dG = dH U silu'(G),
#                   dU = dH silu(G), dWg = dG^T A, dWu = dU^T A,
#                   dA = dG Wg + dU Wu;  silu'(z) = s (1 + z (1 - s)), s = sigmoid(z)
#       permute     dX[t] = sum over t's kept copies of dA[dest[t,j]]
#       gate        both orders give the softmax of the selected logits (the
#                   renormalised top-k of the full softmax equals it), so
#                   dl[t, idx[t,j]] = w[t,j] (dw[t,j] - sum_i w[t,i] dw[t,i])
#                   and dl is zero at unselected experts
#       router      dW_r = dl^T X, dbias = sum_t dl[t], dX[t] += dl[t] W_r
# ---------------------------------------------------------------------------
def silu_grad(z):
    """Derivative of silu: ``s (1 + z (1 - s))`` with s = sigmoid(z), fp64."""
    z = _f64(z)
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-z))
    return s * (1.0 + z * (1.0 - s))


def expert_ffn_backward(A, Wg, Wu, Wd, dY):
    """Gradients of one expert's SwiGLU FFN on rows A [n, d] given dY [n, d]:
    returns (dA [n, d], dWg [d_ff, d], dWu [d_ff, d], dWd [d, d_ff]), fp64."""
    A, Wg, Wu, Wd, dY = (_f64(v) for v in (A, Wg, Wu, Wd, dY))
    G = A @ Wg.T
    U = A @ Wu.T
    H = silu(G) * U
    dH = dY @ Wd
    dWd = dY.T @ H
    dG = dH * U * silu_grad(G)
    dU = dH * silu(G)
    dWg = dG.T @ A
    dWu = dU.T @ A
    dA = dG @ Wg + dU @ Wu
    return dA, dWg, dWu, dWd


def gate_weights_backward(w, dw):
    """Logit gradient of the selected experts, ``w (dw - <w, dw>)`` per row
    ([T, k] fp64), for gate weights w [T, k] that are the softmax of the
    selected logits."""
    w, dw = _f64(w), _f64(dw)
    return w * (dw - np.sum(w * dw, axis=1, keepdims=True))


def moe_backward(X, W_r, bias, W_gate, W_up, W_down, dout, k,
                 capacity_factor=None, gating=TOPK_THEN_SOFTMAX, idx=None):
    """Gradients of the layer: the forward steps are redone in fp64 (logits
    in fp32 as in ``moe_forward``), then each step's backward in reverse
    order.  ``idx`` [T, k], when given, replaces the top-k selection (tests
    pass the ids another implementation selected, so that tokens with fp32
    near-ties are routed alike); the gate weights still come from this
    module's logits.

    Returns a dict with dX [T, d], dW_r [E, d], dbias [E], dW_gate, dW_up
    [E, d_ff, d], dW_down [E, d, d_ff] (all fp64) and the forward pieces
    (idx, w, dest, offsets, Y_perm, dw, dl).
    """
    X = np.asarray(X)
    T, d = X.shape
    E = W_r.shape[0]
    d_ff = W_gate.shape[1]
    logits = router_logits(X, W_r, bias)
    if idx is None:
        idx, _ = select_topk(logits, k)
    idx = np.asarray(idx, dtype=np.int64)
    w = gate_weights(logits, idx, gating)
    a = assign(idx, E, capacity(T, k, E, capacity_factor))
    dest, offsets = a["dest"], a["offsets"]
    X_perm = _f64(gather_rows(X, a["row_token"]))
    Y_perm = grouped_ffn(X_perm, offsets, W_gate, W_up, W_down)
    dout = _f64(dout)

    # combine
    N = int(offsets[E])
    dY_perm = np.zeros((N, d))
    dw = np.zeros((T, k))
    for t in range(T):
        for j in range(k):
            r = dest[t, j]
            if r >= 0:
                dY_perm[r] = w[t, j] * dout[t]
                dw[t, j] = np.dot(dout[t], Y_perm[r])

    # experts, one at a time
    dX_perm = np.zeros((N, d))
    dWg = np.zeros((E, d_ff, d))
    dWu = np.zeros((E, d_ff, d))
    dWd = np.zeros((E, d, d_ff))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            dX_perm[lo:hi], dWg[e], dWu[e], dWd[e] = expert_ffn_backward(
                X_perm[lo:hi], W_gate[e], W_up[e], W_down[e], dY_perm[lo:hi])

    # permute (transpose of the gather)
    dX = np.zeros((T, d))
    for t in range(T):
        for j in range(k):
            if dest[t, j] >= 0:
                dX[t] += dX_perm[dest[t, j]]

    # gate weights, router
    dl_sel = gate_weights_backward(w, dw)
    dl = np.zeros((T, E))
    for t in range(T):
        for j in range(k):
            dl[t, idx[t, j]] += dl_sel[t, j]
    dW_r = dl.T @ _f64(X)
    dbias = dl.sum(axis=0)
    dX += dl @ _f64(W_r)
    return dict(dX=dX, dW_r=dW_r, dbias=dbias, dW_gate=dWg, dW_up=dWu,
                dW_down=dWd, idx=idx, w=w, dest=dest, offsets=offsets,
                Y_perm=Y_perm, dw=dw, dl=dl)
