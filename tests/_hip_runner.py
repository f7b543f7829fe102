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


# Element-wise bound of an activation-type result against the oracle (relative tolerances are also
# checked per row, normwise): |got - ref| <= N_ULP ulp(ref) + ELEM_C rms(ref row).
#  bf16: both sides round the expert intermediate h and the output to bf16. The output may round to the
#        neighbouring value (1 ulp), and an h element whose float32 and float64 values straddle a rounding
#        point (about 1 in 1000) moves an output element by at most 2^-8 |h_f| |Wd_ef|, about 1e-3 of the
#        row's rms at F = 2048; 2^-6 of the rms is below the stated 2e-2 and leaves a 10x margin.
#  f32:  the stated fp32 tolerance, 1e-4 of the row's scale, covers the float32 sums of both GEMMs.
N_ULP = 2.0
ELEM_C = {"bf16": 2.0 ** -6, "f32": 1e-4}


def ulp(v, dt: str) -> np.ndarray:
    """Spacing of the storage format dt (bf16: 8 significant bits, f32: 24) at |v|, v in float64."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    frac, emin = (7, -133) if dt == "bf16" else (23, -149)
    _, e = np.frexp(a)                      # a = m 2^e, m in [0.5, 1): spacing 2^(e - 1 - frac)
    e = np.where(a > 0, e, emin + 1 + frac)
    return np.ldexp(1.0, np.maximum(e - 1 - frac, emin))


def rms_rows(ref) -> np.ndarray:
    ref = np.asarray(ref, dtype=np.float64)
    return np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True)) if ref.shape[-1] else np.zeros(ref.shape[:-1] + (1,))


def elementwise_ratio(got, ref, dt: str, c=None, n_ulp: float = N_ULP) -> np.ndarray:
    """|got - ref| / (n_ulp ulp(ref) + c rms(ref row)) per element (float64 inputs); a result passes
    where the ratio is at most 1. Non-finite results give inf."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    c = ELEM_C[dt] if c is None else c
    bound = n_ulp * ulp(ref, dt) + c * rms_rows(ref)
    with np.errstate(invalid="ignore"):
        r = np.abs(got - ref) / bound
    return np.where(np.isfinite(got), r, np.inf)


def sum_bound_ratio(got, ref, abs_sum, k: int, dt: str) -> np.ndarray:
    """|got - ref| / (ulp(ref) + (k + 1) 2^-24 abs_sum) per element: a float32 sum of k weighted rows,
    rounded once to dt, against the exact sum rounded once (abs_sum = sum of |w_j row_j|)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    bound = ulp(ref, dt) + (k + 1) * 2.0 ** -24 * np.asarray(abs_sum, dtype=np.float64)
    with np.errstate(invalid="ignore", divide="ignore"):
        r = np.abs(got - ref) / bound
    r = np.where(got == ref, 0.0, r)
    return np.where(np.isfinite(got), r, np.inf)


def combine_abs_sum(out_rows64, pair_row, w) -> np.ndarray:
    """sum over kept slots j of |w[t, j]| |out_rows[pair_row[t, j]]| per token and element (float64)."""
    pr = np.asarray(pair_row, dtype=np.int64)
    w = np.abs(np.asarray(w, dtype=np.float64))
    T, k = pr.shape
    H = out_rows64.shape[1]
    acc = np.zeros((T, H), dtype=np.float64)
    for j in range(k):
        m = pr[:, j] >= 0
        if m.any():
            acc[m] += w[m, j:j + 1] * np.abs(out_rows64[pr[m, j]])
    return acc


def layer_bound(y_ref64, out_rows64, pair_row, w, dt: str, c=None) -> np.ndarray:
    """Element-wise bound of a layer output whose expert rows each satisfy the element-wise bound
    N_ULP ulp(out) + c rms(out row): carried through the weighted sum, plus the combine's own rounding
    and float32 summation, ulp(y) + (k + 1) 2^-24 sum |w out|."""
    c = ELEM_C[dt] if c is None else c
    per_row = N_ULP * ulp(out_rows64, dt) + c * rms_rows(out_rows64)
    pr = np.asarray(pair_row, dtype=np.int64)
    k = pr.shape[1]
    return (ulp(y_ref64, dt) + combine_abs_sum(per_row, pr, w) +
            (k + 1) * 2.0 ** -24 * combine_abs_sum(out_rows64, pr, w))


def check_close(got64, ref64, dt: str, what: str, tol: float, bound=None, ratio=None) -> str:
    """Assert the per-row normwise error <= tol and the element-wise ratio <= 1 (the generic
    element-wise bound unless `bound` (absolute, per element) or `ratio` is given); every result
    finite. Returns a summary for the log."""
    got64 = np.asarray(got64, dtype=np.float64)
    ref64 = np.asarray(ref64, dtype=np.float64)
    assert np.all(np.isfinite(got64)), f"{what}: non-finite results"
    if got64.size == 0:
        return f"{what}: empty"
    err = rowwise_rel_err(got64, ref64)
    if ratio is None:
        if bound is None:
            ratio = elementwise_ratio(got64, ref64, dt)
        else:
            with np.errstate(invalid="ignore", divide="ignore"):
                ratio = np.where(got64 == ref64, 0.0, np.abs(got64 - ref64) / bound)
    worst = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    assert np.all(err <= tol), f"{what}: row {int(np.argmax(err))} normwise error {err.max():.3e} > {tol}"
    assert np.all(ratio <= 1.0), (f"{what}: element {tuple(int(i) for i in worst)} got {got64[worst]!r} ref "
                                  f"{ref64[worst]!r}, {ratio[worst]:.3f} x its bound")
    check_close.last = (int(err.shape[0]), float(err.max()), float(ratio.max()))
    return f"{what}: rows {err.shape[0]}, max normwise {err.max():.2e}, max element/bound {ratio.max():.3f}"


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
