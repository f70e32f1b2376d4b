"""Seeded synthetic inputs for the MoE FFN layer.

This module only draws random numbers and arranges them into the layer's
input tensors.  It holds none of the layer's arithmetic (no routing, no
capacity, no FFN), so that the HIP library's tests and the CPU oracle can be
fed the same inputs without sharing any of the method's code.

Workloads (shapes of well-known MoE layers, used as shapes only; weights are
random):

=============  =====  =======  ===  ==  =====  =====  ==========  ========  ====
name           T      d_model  E    k   d_ff   dtype  gating      capacity  skew
=============  =====  =======  ===  ==  =====  =====  ==========  ========  ====
tiny           64     128      8    2   256    fp32   topk->smax  none      no
mixtral        4096   4096     8    2   14336  bf16   topk->smax  none      no
gptoss         8192   2880     32   4   2880   bf16   topk->smax  none      Zipf
deepseekv3     4096   7168     256  8   2048   bf16   smax->topk  none      no
qwen3_cap      16384  2048     128  8   768    bf16   topk->smax  cf 1.25   Zipf
qwen3_decode   32     2048     128  8   768    bf16   topk->smax  none      no
=============  =====  =======  ===  ==  =====  =====  ==========  ========  ====

Distributions: X ~ N(0, 1).  ``tiny``: every weight ~ N(0, variance
1/fan_in) in fp32 (fan_in = d_model for W_r, W_gate, W_up and d_ff for
W_down).  Other workloads: expert weights ~ N(0, std 0.02) rounded to bf16,
W_r ~ N(0, std 0.02) in fp32, X rounded to bf16.  Skewed workloads add a fixed
router bias ``b[e] = ln p[pi(e)]`` with ``p[r] ~ r**-1.2`` (Zipf exponent 1.2,
r = 1..E) and ``pi`` a seeded permutation of the experts.

Two generators are provided.  ``make_host`` draws every tensor with NumPy
(PCG64, one stream per (tensor, expert)) and is used for workloads small
enough for the oracle.  ``make_device`` draws the large expert weights with
torch's device generator (one seeded generator per (tensor, expert)) so that
the 22.5 GB DeepSeek-V3-shaped weights do not have to cross PCIe; X, W_r and
the bias still come from the NumPy streams.
"""

from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import numpy as np

F32 = "f32"
BF16 = "bf16"
TOPK_THEN_SOFTMAX = 0
SOFTMAX_THEN_TOPK = 1

# tensor ids of the per-tensor random streams
_X, _WR, _WG, _WU, _WD, _PERM = 0, 1, 2, 3, 4, 5
_SG, _SU, _SD = 6, 7, 8   # shared-expert projections
_DOUT = 9                  # upstream gradient of the layer output (backward)


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d_model: int
    E: int
    top_k: int
    d_ff: int
    dtype: str = BF16                 # activations and expert weights
    gating: int = TOPK_THEN_SOFTMAX
    capacity_factor: float = 0.0      # <= 0: no capacity limit
    zipf_s: float = 0.0               # > 0: add a Zipf(s) router bias
    seed: int = 0
    init: str = "std0.02"             # "std0.02" or "var1/fanin"

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", 64, 128, 8, 2, 256, F32, TOPK_THEN_SOFTMAX,
                     0.0, 0.0, 1, "var1/fanin"),
    "mixtral": Workload("mixtral", 4096, 4096, 8, 2, 14336, BF16,
                        TOPK_THEN_SOFTMAX, 0.0, 0.0, 2),
    "gptoss": Workload("gptoss", 8192, 2880, 32, 4, 2880, BF16,
                       TOPK_THEN_SOFTMAX, 0.0, 1.2, 3),
    "deepseekv3": Workload("deepseekv3", 4096, 7168, 256, 8, 2048, BF16,
                           SOFTMAX_THEN_TOPK, 0.0, 0.0, 4),
    "qwen3_cap": Workload("qwen3_cap", 16384, 2048, 128, 8, 768, BF16,
                          TOPK_THEN_SOFTMAX, 1.25, 1.2, 5),
    "qwen3_decode": Workload("qwen3_decode", 32, 2048, 128, 8, 768, BF16,
                             TOPK_THEN_SOFTMAX, 0.0, 0.0, 5),
}


def _rng(seed, tensor, expert=0):
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([int(seed), int(tensor), int(expert)])))


def round_bf16(x):
    """Round fp32 values to the nearest bf16 value (ties to even); returns
    fp32 arrays holding bf16-representable values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def bf16_bits(x):
    """The upper 16 bits of fp32 values that are already bf16-representable."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def _std(w: Workload, fan_in: int) -> float:
    if w.init == "var1/fanin":
        return 1.0 / np.sqrt(fan_in)
    return 0.02


def _normal(rng, shape, std, bf16):
    a = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a = (a * np.float32(std)).astype(np.float32)
    return round_bf16(a) if bf16 else a


def make_x(w: Workload, T=None):
    T = w.T if T is None else T
    return _normal(_rng(w.seed, _X), (T, w.d_model), 1.0, w.dtype == BF16)


def make_dout(w: Workload, T=None):
    """Upstream gradient dL/d(out) for the backward pass: [T, d] fp32,
    N(0, 1) entries."""
    T = w.T if T is None else T
    return _normal(_rng(w.seed, _DOUT), (T, w.d_model), 1.0, False)


def make_router(w: Workload):
    """(W_r [E, d] fp32, bias [E] fp32 or None)."""
    W_r = _normal(_rng(w.seed, _WR), (w.E, w.d_model), _std(w, w.d_model),
                  False)
    bias = None
    if w.zipf_s > 0:
        r = np.arange(1, w.E + 1, dtype=np.float64)
        p = r ** (-w.zipf_s)
        p /= p.sum()
        perm = _rng(w.seed, _PERM).permutation(w.E)
        bias = np.log(p[perm]).astype(np.float32)
    return W_r, bias


def make_expert(w: Workload, e: int):
    """Host weights of expert e: (Wg [d_ff, d], Wu [d_ff, d], Wd [d, d_ff])."""
    bf = w.dtype == BF16
    Wg = _normal(_rng(w.seed, _WG, e), (w.d_ff, w.d_model),
                 _std(w, w.d_model), bf)
    Wu = _normal(_rng(w.seed, _WU, e), (w.d_ff, w.d_model),
                 _std(w, w.d_model), bf)
    Wd = _normal(_rng(w.seed, _WD, e), (w.d_model, w.d_ff),
                 _std(w, w.d_ff), bf)
    return Wg, Wu, Wd


def _fp8_codes(W):
    """Per-tensor power-of-two scale s (largest |W| / s <= 448) and the
    nearest FP8 E4M3 codes of W / s (torch's conversion: round to nearest
    even).  W: torch fp32 tensor.  Returns (uint8 codes, float scale)."""
    import torch

    amax = float(W.abs().max())
    s = 2.0 ** np.ceil(np.log2(amax / 448.0)) if amax > 0 else 1.0
    q = (W / s).to(torch.float8_e4m3fn).view(torch.uint8)
    return q, float(s)


def make_host_fp8(w: Workload):
    """The layer's inputs with FP8 expert weights: X, W_r and bias as in
    make_host; per expert and projection the fp32 normal draw of make_expert
    (before any bf16 rounding) is stored as FP8 E4M3 codes with a
    power-of-two scale.  Returns dict X, W_r, bias, Q_gate, Q_up, Q_down
    (uint8 [E, out, in]) and scales (fp32 [E, 3]: gate, up, down)."""
    import torch

    X = make_x(w)
    W_r, bias = make_router(w)
    Qs = [np.empty((w.E, w.d_ff, w.d_model), np.uint8),
          np.empty((w.E, w.d_ff, w.d_model), np.uint8),
          np.empty((w.E, w.d_model, w.d_ff), np.uint8)]
    scales = np.empty((w.E, 3), np.float32)
    for e in range(w.E):
        for j, (tid, shape, fan) in enumerate(((_WG, (w.d_ff, w.d_model), w.d_model),
                                               (_WU, (w.d_ff, w.d_model), w.d_model),
                                               (_WD, (w.d_model, w.d_ff), w.d_ff))):
            W = _normal(_rng(w.seed, tid, e), shape, _std(w, fan), False)
            q, sc = _fp8_codes(torch.from_numpy(W))
            Qs[j][e] = q.numpy()
            scales[e, j] = sc
    return dict(X=X, W_r=W_r, bias=bias, Q_gate=Qs[0], Q_up=Qs[1], Q_down=Qs[2],
                scales=scales)


def make_device_fp8(w: Workload, device="cuda"):
    """make_device's inputs with FP8 expert weights (uint8 codes [E, out, in]
    and fp32 scales [E, 3]), drawn and quantised on the device with the same
    per-(tensor, expert) generators as make_device."""
    import torch

    X = torch.from_numpy(make_x(w)).to(device=device).to(torch.bfloat16)
    W_r, bias = make_router(w)
    W_r = torch.from_numpy(W_r).to(device)
    bias = None if bias is None else torch.from_numpy(bias).to(device)
    Qg = torch.empty((w.E, w.d_ff, w.d_model), dtype=torch.uint8, device=device)
    Qu = torch.empty_like(Qg)
    Qd = torch.empty((w.E, w.d_model, w.d_ff), dtype=torch.uint8, device=device)
    scales = torch.empty((w.E, 3), dtype=torch.float32)
    g = torch.Generator(device=device)
    for e in range(w.E):
        for j, (tid, dst, fan) in enumerate(((_WG, Qg, w.d_model), (_WU, Qu, w.d_model),
                                             (_WD, Qd, w.d_ff))):
            g.manual_seed((w.seed * 1_000_003 + tid * 65_537 + e) & (2**63 - 1))
            tmp = torch.randn(dst.shape[1:], generator=g, device=device,
                              dtype=torch.float32).mul_(_std(w, fan))
            q, sc = _fp8_codes(tmp)
            dst[e].copy_(q)
            scales[e, j] = sc
    return dict(X=X, W_r=W_r, bias=bias, Q_gate=Qg, Q_up=Qu, Q_down=Qd,
                scales=scales.to(device))


def make_shared(w: Workload, shared_d_ff: int):
    """Host weights of a shared expert with hidden size shared_d_ff:
    (Ws_gate [sdff, d], Ws_up [sdff, d], Ws_down [d, sdff]), drawn like the
    expert weights from their own streams."""
    bf = w.dtype == BF16
    Sg = _normal(_rng(w.seed, _SG), (shared_d_ff, w.d_model), _std(w, w.d_model), bf)
    Su = _normal(_rng(w.seed, _SU), (shared_d_ff, w.d_model), _std(w, w.d_model), bf)
    Sd = _normal(_rng(w.seed, _SD), (w.d_model, shared_d_ff), _std(w, shared_d_ff), bf)
    return Sg, Su, Sd


def make_shared_device(w: Workload, shared_d_ff: int, device="cuda"):
    """Shared-expert weights drawn on the device (one seeded torch generator
    per projection), in the activation dtype."""
    import torch

    tdt = torch.bfloat16 if w.dtype == BF16 else torch.float32
    g = torch.Generator(device=device)
    out = []
    for tid, shape, fan in ((_SG, (shared_d_ff, w.d_model), w.d_model),
                            (_SU, (shared_d_ff, w.d_model), w.d_model),
                            (_SD, (w.d_model, shared_d_ff), shared_d_ff)):
        g.manual_seed((w.seed * 1_000_003 + tid * 65_537) & (2**63 - 1))
        t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        out.append(t.mul_(_std(w, fan)).to(tdt))
    return tuple(out)


def make_host(w: Workload):
    """Every input of the layer as host fp32 arrays (bf16 workloads hold
    bf16-representable values).  Returns dict X, W_r, bias, W_gate, W_up,
    W_down with expert weights stacked [E, out, in]."""
    X = make_x(w)
    W_r, bias = make_router(w)
    Wg = np.empty((w.E, w.d_ff, w.d_model), np.float32)
    Wu = np.empty((w.E, w.d_ff, w.d_model), np.float32)
    Wd = np.empty((w.E, w.d_model, w.d_ff), np.float32)
    for e in range(w.E):
        Wg[e], Wu[e], Wd[e] = make_expert(w, e)
    return dict(X=X, W_r=W_r, bias=bias, W_gate=Wg, W_up=Wu, W_down=Wd)


def make_device(w: Workload, device="cuda"):
    """Inputs as torch tensors on ``device`` (activation dtype for X and the
    expert weights, fp32 for W_r and bias).  Expert weights are drawn on the
    device with one seeded torch generator per (tensor, expert)."""
    import torch

    tdt = torch.bfloat16 if w.dtype == BF16 else torch.float32
    X = torch.from_numpy(make_x(w)).to(device=device).to(tdt)
    W_r, bias = make_router(w)
    W_r = torch.from_numpy(W_r).to(device)
    bias = None if bias is None else torch.from_numpy(bias).to(device)
    Wg = torch.empty((w.E, w.d_ff, w.d_model), dtype=tdt, device=device)
    Wu = torch.empty_like(Wg)
    Wd = torch.empty((w.E, w.d_model, w.d_ff), dtype=tdt, device=device)
    g = torch.Generator(device=device)
    for e in range(w.E):
        for tid, dst, fan in ((_WG, Wg, w.d_model), (_WU, Wu, w.d_model),
                              (_WD, Wd, w.d_ff)):
            g.manual_seed((w.seed * 1_000_003 + tid * 65_537 + e) & (2**63 - 1))
            tmp = torch.randn(dst.shape[1:], generator=g, device=device,
                              dtype=torch.float32)
            dst[e].copy_(tmp.mul_(_std(w, fan)))
    return dict(X=X, W_r=W_r, bias=bias, W_gate=Wg, W_up=Wu, W_down=Wd)
