"""Entry points on a stream other than torch's current stream.

The binding allocates a temporary workspace when the caller passes none. It is allocated on torch's
current stream and freed when the call returns, while the kernels that use it are queued on the given
stream; the caching allocator must not hand the block out again before they finish. Each call below
runs on a side stream, and right after it the current stream allocates blocks of the same size and
fills them with garbage. The results must equal the same calls on the current stream bit for bit.
A caller's workspace of any element type is sized in bytes.
"""
import pytest
import torch

import combine_router_gemm_amd as moe
import moe_workloads as W
from tests._hip_runner import run_layer

pytestmark = pytest.mark.gpu


def _bits(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16)
    if t.dtype == torch.float32:
        return t.view(torch.int32)
    return t


def _scribble(nbytes_list):
    """Allocate and fill blocks on the current stream (they would reuse a freed workspace block)."""
    keep = []
    for n in nbytes_list:
        b = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")
        b.fill_(0xA5)
        keep.append(b)
    return keep


# (name, T, H, E, k, F, R, C, dtype, routing): split-K router (few tokens), direct-to-LDS GEMM tiles
# with a plan, and weight-streaming tiles
CASES = [
    ("dl128", 900, 192, 4, 2, 192, 1, 400, "bf16", "zipf"),
    ("decode_R4", 64, 256, 16, 4, 128, 4, 20, "bf16", "uniform"),
    ("f32", 301, 40, 6, 2, 24, 3, 77, "f32", "zipf"),
]


@pytest.mark.parametrize("name,T,H,E,k,F,R,C,dtype,routing", CASES, ids=[c[0] for c in CASES])
def test_side_stream_equals_current_stream(name, T, H, E, k, F, R, C, dtype, routing):
    base = W.workload("tiny-fp32")
    cfg = W.small_config(base, seed=700 + [c[0] for c in CASES].index(name), name=name, T=T, H=H, E=E, k=k,
                         F=F, R=R, dtype=dtype, routing=routing)
    inp = W.make_inputs(cfg, device="cuda")
    inp["C"] = C
    print(f"\n[gpu] side-stream case {name}", flush=True)
    ref = run_layer(inp, k, R)

    side = torch.cuda.Stream()
    x = inp["x"]
    ws_sizes = [moe.moe_route_workspace_bytes(T, H, E, moe.MOE_BF16 if dtype == "bf16" else moe.MOE_F32),
                moe.moe_dispatch_workspace_bytes(T, k, E),
                moe.moe_expert_mlp_workspace_bytes(T, k, E, R, C, F, moe.MOE_BF16 if dtype == "bf16" else moe.MOE_F32)]
    # outputs are allocated up front (on the current stream) and only written by the side stream
    logits = torch.empty(T, E, dtype=torch.float32, device="cuda")
    ids = torch.empty(T, k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, k, dtype=torch.float32, device="cuda")
    L = moe.Layout(T, k, E, R, C, H, device="cuda")
    send_buf = torch.empty(L.rows_max, H, dtype=x.dtype, device="cuda")
    out_buf = torch.empty_like(send_buf)
    y = torch.empty(T, H, dtype=x.dtype, device="cuda")
    torch.cuda.synchronize()
    keep = []
    side.wait_stream(torch.cuda.current_stream())
    moe.moe_route(x, inp["w_router"], inp["bias"], k, logits, ids, w, stream=side)
    keep += _scribble(ws_sizes)
    moe.moe_dispatch(x, ids, L, send_buf, stream=side)
    keep += _scribble(ws_sizes)
    moe.moe_expert_mlp(send_buf, L, inp["w_gate_up"], inp["w_down"], out_buf, stream=side)
    keep += _scribble(ws_sizes)
    moe.moe_combine(out_buf, L, w, y, stream=side)
    torch.cuda.synchronize()
    n = int(ref["layout"].expert_offset[E].item())  # rows past the kept total are unspecified
    for key, got in (("logits", logits), ("ids", ids), ("w", w), ("send_buf", send_buf[:n]), ("out_buf", out_buf[:n]),
                     ("y", y)):
        want = ref[key][:n] if key in ("send_buf", "out_buf") else ref[key]
        assert torch.equal(_bits(got), _bits(want)), key
    for nm in ("expert_count", "expert_kept", "expert_overflow", "expert_offset", "pair_row"):
        assert torch.equal(getattr(L, nm), getattr(ref["layout"], nm)), nm

    # the fused-combine variant with a temporary workspace on the side stream
    out2 = torch.empty_like(send_buf)
    y2 = torch.empty_like(y)
    side.wait_stream(torch.cuda.current_stream())
    moe.moe_expert_mlp_combine(send_buf, L, inp["w_gate_up"], inp["w_down"], w, out2, y2, stream=side)
    keep += _scribble(ws_sizes)
    torch.cuda.synchronize()
    assert torch.equal(_bits(out2[:n]), _bits(out_buf[:n])) and torch.equal(_bits(y2), _bits(y))


def test_workspace_of_any_element_type_is_sized_in_bytes():
    base = W.workload("tiny-fp32")
    cfg = W.small_config(base, seed=710, name="ws-bytes", T=300, H=128, E=8, k=2, F=96, R=2, dtype="bf16",
                         routing="uniform")
    inp = W.make_inputs(cfg, device="cuda")
    T, H, E, k, F, R = cfg.T, cfg.H, cfg.E, cfg.k, cfg.F, cfg.R
    C = inp["C"]
    ref = run_layer(inp, k, R)
    L = moe.Layout(T, k, E, R, C, H, device="cuda")
    ids = ref["ids"]
    send_buf = torch.empty(L.rows_max, H, dtype=torch.bfloat16, device="cuda")
    nb = moe.moe_dispatch_workspace_bytes(T, k, E)
    ws = torch.empty((nb + 3) // 4, dtype=torch.float32, device="cuda")   # exactly enough bytes as fp32
    moe.moe_dispatch(inp["x"], ids, L, send_buf, workspace=ws)
    nb = moe.moe_expert_mlp_workspace_bytes(T, k, E, R, C, F, moe.MOE_BF16)
    ws2 = torch.empty((nb + 7) // 8, dtype=torch.int64, device="cuda")
    out_buf = torch.empty_like(send_buf)
    moe.moe_expert_mlp(send_buf, L, inp["w_gate_up"], inp["w_down"], out_buf, workspace=ws2)
    torch.cuda.synchronize()
    n = int(ref["layout"].expert_offset[E].item())
    assert torch.equal(_bits(send_buf[:n]), _bits(ref["send_buf"][:n]))
    assert torch.equal(_bits(out_buf[:n]), _bits(ref["out_buf"][:n]))
    with pytest.raises(moe.MoeError):
        moe.moe_expert_mlp(send_buf, L, inp["w_gate_up"], inp["w_down"], out_buf,
                           workspace=torch.empty(max(1, nb // 8 - 1), dtype=torch.int64, device="cuda"))
