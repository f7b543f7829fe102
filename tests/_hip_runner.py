"""Helpers for the GPU tests: run the HIP path through the C ABI and move results to numpy.

The HIP path is called only through the binding of the C ABI (combine_router_gemm_amd); the oracle is
imported by the tests themselves. Inputs come from moe_workloads (seeded, synthetic).
"""
from __future__ import annotations

import numpy as np
import torch

import combine_router_gemm_amd as moe


def to_np(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy in the oracle's storage form (bf16 as uint16 bit patterns)."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def dt_name(t: torch.Tensor) -> str:
    return "bf16" if t.dtype == torch.bfloat16 else "f32"


class LazyExperts:
    """Indexable by local expert l: fetches that expert's weights from the device on first use."""

    def __init__(self, w: torch.Tensor):
        self.w = w
        self.cache = {}

    def __getitem__(self, l):
        l = int(l)
        if l not in self.cache:
            self.cache[l] = to_np(self.w[l])
        return self.cache[l]


def run_layer(inp: dict, k: int, R: int, stream=None) -> dict:
    """route -> dispatch -> expert MLP -> combine on the current device; returns device tensors."""
    x = inp["x"]
    dev = x.device
    T, H = x.shape
    E = inp["w_router"].shape[0]
    C = inp["C"]
    logits = torch.empty(T, E, dtype=torch.float32, device=dev)
    ids = torch.empty(T, k, dtype=torch.int32, device=dev)
    w = torch.empty(T, k, dtype=torch.float32, device=dev)
    moe.moe_route(x, inp["w_router"], inp["bias"], k, logits, ids, w, stream=stream)
    L = moe.Layout(T, k, E, R, C, H, device=dev)
    send_buf = torch.empty(L.rows_max, H, dtype=x.dtype, device=dev)
    moe.moe_dispatch(x, ids, L, send_buf, stream=stream)
    out_buf = torch.empty_like(send_buf)
    moe.moe_expert_mlp(send_buf, L, inp["w_gate_up"], inp["w_down"], out_buf, stream=stream)
    y = torch.empty(T, H, dtype=x.dtype, device=dev)
    moe.moe_combine(out_buf, L, w, y, stream=stream)
    torch.cuda.synchronize()
    return dict(logits=logits, ids=ids, w=w, layout=L, send_buf=send_buf, out_buf=out_buf, y=y)


def rowwise_rel_err(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per-row normwise relative error ||got - ref|| / ||ref|| (0/0 -> 0, x/0 -> inf)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.linalg.norm(got - ref, axis=-1)
    den = np.linalg.norm(ref, axis=-1)
    with np.errstate(divide="ignore", invalid="ignore"):
        out = np.where(den > 0, num / np.where(den > 0, den, 1.0), np.where(num > 0, np.inf, 0.0))
    return out


def run_layer_fp8(inp: dict, k: int, R: int, stream=None) -> dict:
    """route -> fp8 block-scaled dispatch -> expert MLP on the fp8 rows -> combine (bf16 activations)."""
    x = inp["x"]
    dev = x.device
    T, H = x.shape
    E = inp["w_router"].shape[0]
    C = inp["C"]
    logits = torch.empty(T, E, dtype=torch.float32, device=dev)
    ids = torch.empty(T, k, dtype=torch.int32, device=dev)
    w = torch.empty(T, k, dtype=torch.float32, device=dev)
    moe.moe_route(x, inp["w_router"], inp["bias"], k, logits, ids, w, stream=stream)
    L = moe.Layout(T, k, E, R, C, H, device=dev)
    send_q = torch.empty(L.rows_max, H, dtype=torch.uint8, device=dev)
    send_scale = torch.empty(L.rows_max, H // moe.MOE_FP8_BLOCK, dtype=torch.float32, device=dev)
    moe.moe_dispatch_fp8(x, ids, L, send_q, send_scale, stream=stream)
    out_buf = torch.empty(L.rows_max, H, dtype=x.dtype, device=dev)
    moe.moe_expert_mlp_fp8(send_q, send_scale, L, inp["w_gate_up"], inp["w_down"], out_buf, stream=stream)
    y = torch.empty(T, H, dtype=x.dtype, device=dev)
    moe.moe_combine(out_buf, L, w, y, stream=stream)
    torch.cuda.synchronize()
    return dict(logits=logits, ids=ids, w=w, layout=L, send_q=send_q, send_scale=send_scale, out_buf=out_buf, y=y)
