"""CPU checks of the C ABI: the library loads, exports every entry point
include/moe.h declares, and rejects bad arguments on the host before any
device work (these paths make no HIP call, so they run without a GPU)."""

import ctypes
import os
import re

import pytest

from mixture_experts_layer_wavefront_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = B.load()
    names = _declared()
    assert set(names) == set(B.SYMBOLS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for s in (B.MOE_OK, B.MOE_ERR_INVALID_ARG, B.MOE_ERR_UNSUPPORTED,
              B.MOE_ERR_WORKSPACE, B.MOE_ERR_HIP, B.MOE_ERR_SCRATCH_LIMIT):
        assert B.status_string(s).startswith("MOE_")


def test_capacity_and_rows_bound():
    p = B.problem(16384, 2048, 128, 8, 768, 1.25)
    assert B.capacity(p) == 1280
    assert B.rows_bound(p) == min(16384 * 8, 128 * 1280)
    p = B.problem(100, 64, 8, 2, 64, 0.5)           # C = ceil(12.5) = 13
    assert B.capacity(p) == 13 and B.rows_bound(p) == 8 * 13
    p = B.problem(10, 64, 4, 2, 64, 100.0)          # capped at T
    assert B.capacity(p) == 10 and B.rows_bound(p) == 20
    p = B.problem(4096, 4096, 8, 2, 14336)
    assert B.capacity(p) == -1 and B.rows_bound(p) == 8192


def test_workspace_sizes_cover_the_intermediates():
    p = B.problem(4096, 7168, 256, 8, 2048, 0.0, "bf16", 1)
    R = B.rows_bound(p)
    ws = B.workspace_bytes(p)
    # bf16: H (bf16) + Y_perm (fp32) at least; the FFN gathers the rows of X,
    # so no permuted copy of X is kept
    assert ws >= R * 2048 * 2 + R * 7168 * 4
    assert ws < R * 7168 * 2 + R * 2048 * 2 + R * 7168 * 4
    # fp32 layers keep X_perm (fp32) + H (fp32) + Y_perm (fp32)
    pf = B.problem(64, 256, 8, 2, 128, 0.0, "f32")
    Rf = B.rows_bound(pf)
    assert B.workspace_bytes(pf) >= Rf * 256 * 4 + Rf * 128 * 4 + Rf * 256 * 4
    assert B.grouped_ffn_workspace_bytes(p) >= R * 2048 * 2
    assert B.permute_workspace_bytes(p) >= 4096 * 8 * 4
    assert ws % 256 == 0


@pytest.mark.parametrize("kw,status", [
    (dict(T=8, d_model=64, E=4, top_k=5, d_ff=64), B.MOE_ERR_INVALID_ARG),
    (dict(T=-1, d_model=64, E=4, top_k=2, d_ff=64), B.MOE_ERR_INVALID_ARG),
    (dict(T=8, d_model=0, E=4, top_k=2, d_ff=64), B.MOE_ERR_INVALID_ARG),
    (dict(T=8, d_model=60, E=4, top_k=2, d_ff=64), B.MOE_ERR_UNSUPPORTED),
    (dict(T=8, d_model=64, E=4, top_k=2, d_ff=20), B.MOE_ERR_UNSUPPORTED),
    (dict(T=8, d_model=64, E=300, top_k=2, d_ff=64), B.MOE_ERR_UNSUPPORTED),
    (dict(T=8, d_model=64, E=64, top_k=40, d_ff=64), B.MOE_ERR_UNSUPPORTED),
])
def test_invalid_problems_rejected(kw, status):
    lib = B.load()
    p = B.problem(**kw)
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first
    r = lib.moe_route(ctypes.byref(p), fake, fake, None, fake, fake, fake, 1 << 40, None)
    assert r == status
    r = lib.moe_forward(ctypes.byref(p), fake, fake, None, fake, fake, fake,
                        fake, None, fake, 1 << 40, None)
    assert r == status
    assert lib.moe_workspace_bytes(ctypes.byref(p)) == 0


def test_mixed_dtypes_and_bad_enums_rejected():
    lib = B.load()
    p = B.problem(8, 64, 4, 2, 64)
    p.w_dtype = B.MOE_F32
    assert lib.moe_route(ctypes.byref(p), None, None, None, None, None, None,
                         0, None) == B.MOE_ERR_UNSUPPORTED
    p = B.problem(8, 64, 4, 2, 64)
    p.gating = 7
    assert lib.moe_route(ctypes.byref(p), None, None, None, None, None, None,
                         0, None) == B.MOE_ERR_INVALID_ARG
    p = B.problem(8, 64, 4, 2, 64, float("nan"))
    assert lib.moe_route(ctypes.byref(p), None, None, None, None, None, None,
                         0, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_route(None, None, None, None, None, None, None, 0,
                         None) == B.MOE_ERR_INVALID_ARG


def test_null_pointers_and_small_workspace_rejected():
    lib = B.load()
    p = B.problem(8, 64, 4, 2, 64)
    fake = ctypes.c_void_p(0x1000)
    assert lib.moe_route(ctypes.byref(p), None, fake, None, fake, fake, fake,
                         1 << 40, None) == B.MOE_ERR_INVALID_ARG
    need = lib.moe_route_workspace_bytes(ctypes.byref(p))
    assert need > 0
    assert lib.moe_route(ctypes.byref(p), fake, fake, None, fake, fake, fake,
                         need - 1, None) == B.MOE_ERR_WORKSPACE
    need = lib.moe_permute_workspace_bytes(ctypes.byref(p))
    r = lib.moe_permute(ctypes.byref(p), fake, fake, fake, fake, fake, fake,
                        fake, fake, fake, need - 1, None)
    assert r == B.MOE_ERR_WORKSPACE
    r = lib.moe_permute(ctypes.byref(p), fake, fake, fake, fake, fake, fake,
                        fake, fake, None, need, None)
    assert r == B.MOE_ERR_WORKSPACE
    need = lib.moe_workspace_bytes(ctypes.byref(p))
    r = lib.moe_forward(ctypes.byref(p), fake, fake, None, fake, fake, fake,
                        fake, None, fake, need - 1, None)
    assert r == B.MOE_ERR_WORKSPACE
    need = lib.moe_grouped_ffn_workspace_bytes(ctypes.byref(p))
    r = lib.moe_grouped_ffn(ctypes.byref(p), fake, fake, fake, fake, fake,
                            fake, fake, need - 1, None)
    assert r == B.MOE_ERR_WORKSPACE


def test_grouped_ffn_rows_arguments_checked_on_the_host():
    lib = B.load()
    fake = ctypes.c_void_p(0x1000)
    p = B.problem(8, 64, 4, 2, 64)
    need = lib.moe_grouped_ffn_workspace_bytes(ctypes.byref(p))
    args = lambda **kw: [kw.get(n, fake) for n in  # noqa: E731
                         ("X", "rt", "off", "wg", "wu", "wd")]
    call = lambda p, a, sc, ws: lib.moe_grouped_ffn_rows(  # noqa: E731
        ctypes.byref(p), *a, sc, fake, fake, ws, None)
    assert call(p, args(), None, need - 1) == B.MOE_ERR_WORKSPACE
    assert call(p, args(rt=None), None, need) == B.MOE_ERR_INVALID_ARG
    assert call(p, args(X=None), None, need) == B.MOE_ERR_INVALID_ARG
    # scales only with FP8 weights, and then required
    assert call(p, args(), fake, need) == B.MOE_ERR_INVALID_ARG
    p8 = B.problem(8, 64, 4, 2, 64, w_dtype="fp8")
    need8 = lib.moe_grouped_ffn_workspace_bytes(ctypes.byref(p8))
    assert call(p8, args(), None, need8) == B.MOE_ERR_INVALID_ARG
    # fp32 layers keep X_perm: unsupported here
    pf = B.problem(8, 64, 4, 2, 64, 0.0, "f32")
    assert call(pf, args(), None, 1 << 40) == B.MOE_ERR_UNSUPPORTED
    # X beyond one 32-bit buffer range
    pb = B.problem(1 << 18, 4096, 8, 2, 64)
    assert call(pb, args(), None, 1 << 50) == B.MOE_ERR_UNSUPPORTED


def test_shared_expert_arguments_checked_on_the_host():
    lib = B.load()
    p = B.problem(8, 64, 4, 2, 64)
    fake = ctypes.c_void_p(0x1000)
    base = lib.moe_workspace_bytes(ctypes.byref(p))
    need = lib.moe_forward_shared_workspace_bytes(ctypes.byref(p), 96)
    # the routed layer's workspace plus the shared FFN's H, schedule and rows
    assert need >= base + 8 * 96 * 2 + 8 * 64 * 4
    assert lib.moe_forward_shared_workspace_bytes(ctypes.byref(p), 12) == 0
    args = [fake] * 9
    for sdff, status in ((0, B.MOE_ERR_INVALID_ARG), (-8, B.MOE_ERR_INVALID_ARG),
                         (12, B.MOE_ERR_UNSUPPORTED), ((1 << 20) + 8, B.MOE_ERR_UNSUPPORTED)):
        assert lib.moe_forward_shared(ctypes.byref(p), sdff, *args, fake, None,
                                      fake, 1 << 40, None, None) == status
    # a missing shared weight, then a workspace one byte short
    bad = [fake] * 6 + [None] + [fake] * 2
    assert lib.moe_forward_shared(ctypes.byref(p), 96, *bad, fake, None, fake,
                                  need, None, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_forward_shared(ctypes.byref(p), 96, *args, fake, None, fake,
                                  need - 1, None, None) == B.MOE_ERR_WORKSPACE
    p0 = B.problem(0, 64, 4, 2, 64)
    assert lib.moe_forward_shared(ctypes.byref(p0), 96, *([None] * 9), None, None,
                                  None, 0, None, None) == B.MOE_OK


def test_fp8_weights_only_through_the_scaled_entry_points():
    lib = B.load()
    fake = ctypes.c_void_p(0x1000)
    p = B.problem(8, 64, 4, 2, 64, w_dtype="fp8")
    # sizes are defined; the unscaled entry points reject FP8 weights
    assert lib.moe_workspace_bytes(ctypes.byref(p)) > 0
    assert lib.moe_grouped_ffn_workspace_bytes(ctypes.byref(p)) > 0
    assert lib.moe_forward(ctypes.byref(p), fake, fake, None, fake, fake, fake,
                           fake, None, fake, 1 << 40, None) == B.MOE_ERR_UNSUPPORTED
    # FP8 needs bf16 activations and multiples of 16
    for kw in (dict(dtype="f32"), dict(d_model=72), dict(d_ff=72)):
        args = dict(T=8, d_model=64, E=4, top_k=2, d_ff=64, w_dtype="fp8")
        args.update(kw)
        q = B.problem(**args)
        assert lib.moe_forward_scaled(ctypes.byref(q), fake, fake, None, fake, fake,
                                      fake, fake, fake, None, fake, 1 << 40,
                                      None) == B.MOE_ERR_UNSUPPORTED
    # scales are required; the scaled entry points reject bf16 weights
    assert lib.moe_forward_scaled(ctypes.byref(p), fake, fake, None, fake, fake, fake,
                                  None, fake, None, fake, 1 << 40,
                                  None) == B.MOE_ERR_INVALID_ARG
    pb = B.problem(8, 64, 4, 2, 64)
    assert lib.moe_grouped_ffn_scaled(ctypes.byref(pb), fake, fake, fake, fake, fake,
                                      fake, fake, fake, 1 << 40,
                                      None) == B.MOE_ERR_UNSUPPORTED
    need = lib.moe_grouped_ffn_workspace_bytes(ctypes.byref(p))
    assert lib.moe_grouped_ffn_scaled(ctypes.byref(p), fake, fake, fake, fake, fake,
                                      fake, fake, fake, need - 1,
                                      None) == B.MOE_ERR_WORKSPACE


def test_empty_batch_is_a_noop_without_device_work():
    lib = B.load()
    p = B.problem(0, 64, 4, 2, 64)
    assert lib.moe_forward(ctypes.byref(p), None, None, None, None, None,
                           None, None, None, None, 0, None) == B.MOE_OK
    assert lib.moe_route(ctypes.byref(p), None, None, None, None, None, None,
                         0, None) == B.MOE_OK
    assert lib.moe_combine(ctypes.byref(p), None, None, None, None,
                           None) == B.MOE_OK


def test_binding_rejects_host_tensors():
    import torch
    p = B.problem(8, 64, 4, 2, 64)
    X = torch.zeros((8, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        B.moe_route(p, X, torch.zeros((4, 64)), topk_idx=X, topk_w=X)


def test_training_entry_points_checked_on_the_host():
    lib = B.load()
    fake = ctypes.c_void_p(0x1000)
    big = 1 << 40
    p = B.problem(64, 128, 8, 2, 256)
    S = lib.moe_train_state_bytes(ctypes.byref(p))
    W = lib.moe_backward_workspace_bytes(ctypes.byref(p))
    fw = lib.moe_workspace_bytes(ctypes.byref(p))
    R = lib.moe_rows_bound(ctypes.byref(p))
    # the state holds X_perm, G, U, H (bf16) and Y_perm (fp32) at least
    assert S >= R * (128 * 2 + 3 * 256 * 2 + 128 * 4)
    # the workspace holds dY, dG | dU (bf16) and dX_perm's two halves (fp32)
    assert W >= R * (128 * 2 + 2 * 256 * 2 + 2 * 128 * 4)

    def fwd(prob, state=fake, state_bytes=big, ws=fake, ws_bytes=big, X=fake):
        return lib.moe_forward_train(ctypes.byref(prob), X, fake, None, fake, fake,
                                     fake, fake, None, state, state_bytes, ws,
                                     ws_bytes, None)

    def bwd(prob, state=fake, state_bytes=big, ws=fake, ws_bytes=big, dout=fake,
            dbias=fake):
        return lib.moe_backward(ctypes.byref(prob), fake, fake, fake, fake, fake,
                                state, state_bytes, dout, fake, fake, dbias, fake,
                                fake, fake, ws, ws_bytes, None)

    # fp32 layers are not supported for training
    q = B.problem(64, 128, 8, 2, 256, dtype="f32")
    assert lib.moe_train_state_bytes(ctypes.byref(q)) == 0
    assert fwd(q) == B.MOE_ERR_UNSUPPORTED and bwd(q) == B.MOE_ERR_UNSUPPORTED
    # a state that is missing or too small, a workspace that is too small
    assert fwd(p, state=None) == B.MOE_ERR_INVALID_ARG
    assert fwd(p, state_bytes=S - 1) == B.MOE_ERR_INVALID_ARG
    assert fwd(p, ws_bytes=fw - 1) == B.MOE_ERR_WORKSPACE
    assert fwd(p, X=None) == B.MOE_ERR_INVALID_ARG
    assert bwd(p, state_bytes=S - 1) == B.MOE_ERR_INVALID_ARG
    assert bwd(p, ws_bytes=W - 1) == B.MOE_ERR_WORKSPACE
    assert bwd(p, ws=None) == B.MOE_ERR_WORKSPACE
    assert bwd(p, dout=None) == B.MOE_ERR_INVALID_ARG
    # an empty batch does nothing
    e = B.problem(0, 128, 8, 2, 256)
    assert fwd(e, state=None, ws=None) == B.MOE_OK
    assert bwd(e, state=None, ws=None, dout=None) == B.MOE_OK
    # an expert's rows of a saved activation must fit one 32-bit buffer range
    h = B.problem(1 << 20, 128, 8, 4, 256)
    assert lib.moe_train_state_bytes(ctypes.byref(h)) == 0
    assert bwd(h) == B.MOE_ERR_UNSUPPORTED
