"""GPU: the combine fused into the down GEMM (moe_expert_mlp_combine), through the C ABI.

The fused call must give the separate moe_expert_mlp + moe_combine results bit for bit: the same expert
outputs, and y from the same fp32 sums in the same slot order (the separate path is itself checked
against the oracle in test_gpu_parity.py). y is filled with a sentinel first, so every element must be
written, including the zero rows of fully dropped tokens; three calls in a row on the same workspace
check that the per-band counters are cleared and that no band is combined from stale rows.
"""
import numpy as np
import pytest
import torch

import combine_router_gemm_amd as moe
import moe_workloads as W
from tests._hip_runner import run_layer

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _check_fused(inp, out, k, R, calls=3):
    L = out["layout"]
    x = inp["x"]
    total = int(L.expert_offset[-1].item())
    xdt = moe.MOE_BF16 if x.dtype == torch.bfloat16 else moe.MOE_F32
    F = inp["w_gate_up"].shape[1] // 2
    ws = torch.empty(max(1, moe.moe_expert_mlp_combine_workspace_bytes(L.T, L.k, L.E, L.R, L.C, L.H, F, xdt)),
                     dtype=torch.uint8, device=x.device)
    ws.fill_(0xA5)  # counters start from garbage: the call must clear them
    for c in range(calls):
        ob = torch.zeros_like(out["out_buf"])
        y = torch.empty_like(out["y"])
        _bits(y).fill_(0x7FC1 if y.dtype == torch.bfloat16 else 0x7FC00001)
        moe.moe_expert_mlp_combine(out["send_buf"], L, inp["w_gate_up"], inp["w_down"], out["w"], ob, y,
                                   workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(_bits(ob[:total]), _bits(out["out_buf"][:total])), f"call {c}: expert outputs differ"
        diff = (_bits(y) != _bits(out["y"])).any(dim=1)
        assert not bool(diff.any()), f"call {c}: y differs from moe_combine on {int(diff.sum())} tokens"
    return total


@pytest.mark.parametrize("wl", list(W.WORKLOADS))
def test_fused_combine_full_size(wl):
    cfg = W.workload(wl)
    print(f"\n[gpu] fused combine: {W.describe(cfg)}", flush=True)
    inp = W.make_inputs(cfg, device="cuda")
    out = run_layer(inp, cfg.k, cfg.R)
    total = _check_fused(inp, out, cfg.k, cfg.R)
    print(f"[gpu] {wl}: fused combine equals moe_expert_mlp + moe_combine on {cfg.T} tokens, {total} rows")
    del out, inp
    torch.cuda.empty_cache()


EDGE = [
    # name, T, H, E, k, F, R, C, dtype, routing
    ("capacity0", 64, 64, 8, 2, 64, 1, 0, "bf16", "uniform"),
    ("T1", 1, 64, 8, 2, 64, 1, 1, "bf16", "uniform"),
    ("T0", 0, 64, 8, 2, 64, 1, 1, "bf16", "uniform"),
    ("k_eq_E", 70, 64, 8, 8, 64, 4, 70, "bf16", "uniform"),
    ("ragged_f32", 301, 40, 6, 2, 24, 3, 77, "f32", "zipf"),
    ("capacity_ge_T_f32", 96, 64, 8, 2, 64, 2, 101, "f32", "uniform"),
    ("R8_El2", 160, 64, 16, 4, 32, 8, 40, "bf16", "uniform"),
    ("E512_k8", 300, 64, 512, 8, 32, 8, 5, "bf16", "zipf"),
    ("hot_overflow", 512, 128, 64, 6, 64, 1, 48, "bf16", "hot8"),
    ("many_rows_tile_edges", 700, 128, 4, 2, 160, 1, 300, "bf16", "uniform"),
    ("dl128_ragged", 900, 192, 4, 2, 192, 1, 400, "bf16", "zipf"),
    ("dl256_ragged_R2", 2600, 320, 4, 2, 192, 2, 1100, "bf16", "zipf"),
    ("dec64_multi_mtile", 300, 128, 8, 2, 96, 1, 100, "bf16", "zipf"),
    ("H_not_multiple_of_band", 400, 200, 8, 2, 64, 1, 100, "bf16", "uniform"),
]


@pytest.mark.parametrize("name,T,H,E,k,F,R,C,dtype,routing", EDGE, ids=[e[0] for e in EDGE])
def test_fused_combine_edge_cases(name, T, H, E, k, F, R, C, dtype, routing):
    cfg = W.small_config(W.workload("tiny-fp32"), seed=600 + [e[0] for e in EDGE].index(name), name=name,
                         T=max(T, 1), H=H, E=E, k=k, F=F, R=R, dtype=dtype, routing=routing)
    inp = W.make_inputs(cfg, device="cuda", T=T)
    inp["C"] = C
    print(f"\n[gpu] fused combine edge case {name}", flush=True)
    out = run_layer(inp, k, R)
    _check_fused(inp, out, k, R)
