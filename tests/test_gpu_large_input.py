"""GPU check of the forward path for an input too large for one 32-bit buffer
range (T * d_model * 2 bytes >= 2^31): there the grouped FFN cannot read the
rows of X in place, so moe_forward runs the permute with its row copy and
the grouped FFN on X_perm.  The layer output must equal the four stage entry
points run one after the other (the same kernels on the same rows) bit for
bit, and moe_grouped_ffn_rows must refuse the problem.  Inputs are seeded and
drawn on the device (2 GiB of X); no oracle runs at this size."""

import pytest
import torch

from mixture_experts_layer_wavefront_amd import binding as B

pytestmark = pytest.mark.gpu


def test_forward_beyond_one_buffer_range_uses_the_row_copy():
    T, d, E, k, dff = 1 << 17, 8192, 2, 1, 64     # T * d * 2 = 2^31 bytes
    print(f"[large] T={T} d={d} E={E} k={k} d_ff={dff}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(81)
    X = torch.randn((T, d), generator=g, device="cuda").to(torch.bfloat16)
    W_r = torch.randn((E, d), generator=g, device="cuda") * 0.02
    W_gate = (torch.randn((E, dff, d), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    W_up = (torch.randn((E, dff, d), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    W_down = (torch.randn((E, d, dff), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    p = B.problem(T, d, E, k, dff)
    out = B.moe_forward(p, X, W_r, None, W_gate, W_up, W_down)
    idx, w = B.moe_route(p, X, W_r, None)
    perm = B.moe_permute(p, X, idx)
    Y = B.moe_grouped_ffn(p, perm["X_perm"], perm["offsets"], W_gate, W_up, W_down)
    out2 = B.moe_combine(p, Y, perm["dest_row"], w)
    torch.cuda.synchronize()
    assert int(perm["offsets"][-1]) == T * k
    assert torch.isfinite(out).all()
    assert torch.equal(out, out2), "moe_forward differs from the stage entry points"
    del Y, out2
    with pytest.raises(B.MoeError) as ex:
        B.moe_grouped_ffn_rows(p, X, perm["row_token"], perm["offsets"], W_gate, W_up, W_down)
    assert ex.value.status == B.MOE_ERR_UNSUPPORTED
