"""GPU: one whole layer step (route -> dispatch -> expert MLP -> combine) captured in a HIP graph.

The entry points allocate nothing, never synchronise and only enqueue kernels on the caller's stream,
so a step can be captured and replayed. Each replay must reproduce the eager step bit for bit; eager
steps run between the replays. The shapes cover the fused router (E <= 16), the split-K router GEMM
with workspace, the 32- and 64-row weight-streaming GEMM tiles and the direct-to-LDS GEMM.
"""
import pytest
import torch

import combine_router_gemm_amd as moe
import moe_workloads as W

pytestmark = pytest.mark.gpu

CASES = [
    # name, T, H, E, k, F, R, C, routing
    ("fused_router_dec64", 200, 256, 8, 2, 128, 1, 60, "zipf"),
    ("router_gemm_dec32", 130, 1024, 64, 4, 128, 2, 8, "uniform"),
    ("direct_lds_gemm", 1200, 256, 4, 2, 192, 1, 600, "uniform"),
]


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


@pytest.mark.parametrize("name,T,H,E,k,F,R,C,routing", CASES, ids=[c[0] for c in CASES])
def test_graph_replay_matches_eager(name, T, H, E, k, F, R, C, routing):
    cfg = W.small_config(W.workload("mixtral8x7b-decode"), seed=300 + [c[0] for c in CASES].index(name), name=name,
                         T=T, H=H, E=E, k=k, F=F, R=R, dtype="bf16", routing=routing)
    dev = torch.device("cuda:0")
    inp = W.make_inputs(cfg, device=dev, T=T)
    x = inp["x"]
    print(f"\n[gpu] graph case {name}", flush=True)
    logits = torch.empty(T, E, dtype=torch.float32, device=dev)
    ids = torch.empty(T, k, dtype=torch.int32, device=dev)
    wts = torch.empty(T, k, dtype=torch.float32, device=dev)
    L = moe.Layout(T, k, E, R, C, H, device=dev)
    send_buf = torch.zeros(L.rows_max, H, dtype=x.dtype, device=dev)
    out_buf = torch.zeros_like(send_buf)
    y = torch.empty(T, H, dtype=x.dtype, device=dev)
    xdt = moe.MOE_BF16
    ws_r = torch.empty(max(1, moe.moe_route_workspace_bytes(T, H, E, xdt)), dtype=torch.uint8, device=dev)
    ws_d = torch.empty(max(1, moe.moe_dispatch_workspace_bytes(T, k, E)), dtype=torch.uint8, device=dev)
    ws_m = torch.empty(max(1, moe.moe_expert_mlp_workspace_bytes(T, k, E, R, C, F, xdt)), dtype=torch.uint8,
                       device=dev)

    def step():
        moe.moe_route(x, inp["w_router"], inp["bias"], k, logits, ids, wts, workspace=ws_r)
        moe.moe_dispatch(x, ids, L, send_buf, workspace=ws_d)
        moe.moe_expert_mlp(send_buf, L, inp["w_gate_up"], inp["w_down"], out_buf, workspace=ws_m)
        moe.moe_combine(out_buf, L, wts, y)

    step()
    torch.cuda.synchronize()
    total = int(L.expert_offset[-1].item())
    ref = [logits.clone(), ids.clone(), wts.clone(), send_buf[:total].clone(), out_buf[:total].clone(), y.clone()]

    # warm the capture stream, then capture one step
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for rep in range(3):
        for t in (logits, wts, y):
            t.fill_(-1.0)
        ids.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        got = [logits, ids, wts, send_buf[:total], out_buf[:total], y]
        for i, (a, b) in enumerate(zip(got, ref)):
            assert torch.equal(_bits(a), _bits(b)), f"replay {rep}: output {i} differs from the eager step"
        step()  # eager work between the replays
        torch.cuda.synchronize()


VARIANT_CASES = [
    # name, T, H, E, k, F, R, C, routing
    ("fp8_dispatch_sender_combine_dec64", 200, 256, 8, 2, 128, 2, 60, "zipf"),
    ("fp8_dispatch_sender_combine_direct_lds", 1200, 256, 4, 2, 192, 2, 600, "uniform"),
]


@pytest.mark.parametrize("name,T,H,E,k,F,R,C,routing", VARIANT_CASES, ids=[c[0] for c in VARIANT_CASES])
def test_graph_replay_fp8_and_sender_side_combine(name, T, H, E, k, F, R, C, routing):
    cfg = W.small_config(W.workload("mixtral8x7b-decode"), seed=320 + [c[0] for c in VARIANT_CASES].index(name),
                         name=name, T=T, H=H, E=E, k=k, F=F, R=R, dtype="bf16", routing=routing)
    dev = torch.device("cuda:0")
    inp = W.make_inputs(cfg, device=dev, T=T)
    x = inp["x"]
    print(f"\n[gpu] graph case {name}", flush=True)
    logits = torch.empty(T, E, dtype=torch.float32, device=dev)
    ids = torch.empty(T, k, dtype=torch.int32, device=dev)
    wts = torch.empty(T, k, dtype=torch.float32, device=dev)
    L = moe.Layout(T, k, E, R, C, H, device=dev)
    send_q = torch.zeros(L.rows_max, H, dtype=torch.uint8, device=dev)
    send_scale = torch.zeros(L.rows_max, H // moe.MOE_FP8_BLOCK, dtype=torch.float32, device=dev)
    out_buf = torch.zeros(L.rows_max, H, dtype=x.dtype, device=dev)
    partial = torch.zeros(R, T, H, dtype=x.dtype, device=dev)
    y = torch.empty(T, H, dtype=x.dtype, device=dev)
    xdt = moe.MOE_BF16
    ws_r = torch.empty(max(1, moe.moe_route_workspace_bytes(T, H, E, xdt)), dtype=torch.uint8, device=dev)
    ws_d = torch.empty(max(1, moe.moe_dispatch_workspace_bytes(T, k, E)), dtype=torch.uint8, device=dev)
    ws_m = torch.empty(max(1, moe.moe_expert_mlp_workspace_bytes(T, k, E, R, C, F, xdt)), dtype=torch.uint8,
                       device=dev)

    def step():
        moe.moe_route(x, inp["w_router"], inp["bias"], k, logits, ids, wts, workspace=ws_r)
        moe.moe_dispatch_fp8(x, ids, L, send_q, send_scale, workspace=ws_d)
        moe.moe_expert_mlp_fp8(send_q, send_scale, L, inp["w_gate_up"], inp["w_down"], out_buf, workspace=ws_m)
        moe.moe_combine_send(out_buf, L, wts, partial)
        moe.moe_combine_recv(partial, L, y)

    step()
    torch.cuda.synchronize()
    total = int(L.expert_offset[-1].item())
    ref = [ids.clone(), send_q[:total].clone(), send_scale[:total].clone(), out_buf[:total].clone(), y.clone()]

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for rep in range(3):
        y.fill_(-1.0)
        ids.fill_(-7)
        send_scale.fill_(-1.0)
        g.replay()
        torch.cuda.synchronize()
        got = [ids, send_q[:total], send_scale[:total], out_buf[:total], y]
        for i, (a, b) in enumerate(zip(got, ref)):
            assert torch.equal(_bits(a), _bits(b)), f"replay {rep}: output {i} differs from the eager step"
        step()
        torch.cuda.synchronize()
