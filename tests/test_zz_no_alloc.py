"""moe_dispatch_noalloc (the dispatch with the library's static per-GPU scratch, for callers that cannot
allocate) against moe_dispatch with a caller's workspace, through the C ABI, bit for bit: every layout
array and every kept send row. Two calls in a row on one GPU, the second with a smaller input, so the
second call runs over the scratch contents the first one left.
"""
import pytest
import torch

import combine_router_gemm_amd as moe

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else (t.view(torch.int32) if t.dtype == torch.float32 else t)


def _ids(T, E, k, hot, g):
    """Distinct expert ids per token; with `hot`, even tokens choose among the first k + 2 experts."""
    keys = torch.rand(T, E, generator=g, device="cuda")
    if hot and E > k + 2:
        keys[0::2, : k + 2] += 2.0
    return keys.argsort(dim=1, descending=True)[:, :k].to(torch.int32).contiguous()


CALLS = [
    # T, H, E, k, R, C, dtype, hot: a large skewed batch (overflow), then a smaller one with 4 ranks
    (16384, 1024, 256, 8, 1, 512, torch.bfloat16, True),
    (300, 256, 16, 2, 4, 40, torch.float32, False),
]


def _check(T, H, E, k, R, C, dtype, hot, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    x = torch.randn(T, H, generator=g, device="cuda").to(dtype)
    ids = _ids(T, E, k, hot, g)
    L_ref = moe.Layout(T, k, E, R, C, H, device="cuda")
    L_got = moe.Layout(T, k, E, R, C, H, device="cuda")
    send_ref = torch.empty(L_ref.rows_max, H, dtype=dtype, device="cuda")
    send_got = torch.empty_like(send_ref)
    ws = torch.empty(max(1, moe.moe_dispatch_workspace_bytes(T, k, E)), dtype=torch.uint8, device="cuda")
    moe.moe_dispatch(x, ids, L_ref, send_ref, workspace=ws)
    moe.moe_dispatch_noalloc(x, ids, L_got, send_got)
    torch.cuda.synchronize()
    for nm in ("expert_count", "expert_kept", "expert_overflow", "expert_offset", "pair_row"):
        assert torch.equal(getattr(L_got, nm), getattr(L_ref, nm)), nm
    n = int(L_ref.expert_offset[E].item())
    assert torch.equal(L_got.row_token[:n], L_ref.row_token[:n])
    assert torch.equal(L_got.row_slot[:n], L_ref.row_slot[:n])
    assert torch.equal(_bits(send_got[:n]), _bits(send_ref[:n]))
    return n, int(L_ref.expert_overflow.sum().item())


def test_noalloc_dispatch_equals_dispatch_on_two_calls_in_a_row():
    for i, c in enumerate(CALLS):
        print(f"\n[gpu] moe_dispatch_noalloc call {i}: T={c[0]} H={c[1]} E={c[2]} k={c[3]} R={c[4]} C={c[5]}",
              flush=True)
        n, over = _check(*c, seed=900 + i)
        print(f"[gpu] rows {n}, dropped pairs {over}")


def test_noalloc_dispatch_refuses_sizes_beyond_its_scratch():
    T, k, E = 131072, 8, 512
    assert moe.moe_dispatch_workspace_bytes(T, k, E) > moe.MOE_DISPATCH_NOALLOC_MAX_WORKSPACE
    L = moe.Layout(T, k, E, 1, 1, 8, device="cuda")
    x = torch.empty(T, 8, dtype=torch.bfloat16, device="cuda")
    ids = torch.zeros(T, k, dtype=torch.int32, device="cuda")
    send = torch.empty(L.rows_max, 8, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoeError, match="unsupported"):
        moe.moe_dispatch_noalloc(x, ids, L, send)
