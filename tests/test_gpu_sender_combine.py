"""GPU parity of the combine with sender-side partial accumulation (moe_combine_send, moe_combine_recv),
through the C ABI, on the GPU's own dispatch layout and expert outputs.

  partial  each present (rank, token) row within the combine tolerance (2e-2 bf16, 1e-4 fp32, per-row
           normwise) of the oracle's; absent slots keep the sentinel the buffer was filled with
  y        within the same tolerance of the oracle's receive side on the oracle's partials
  R = 1    y equals moe_combine's output bit for bit (one partial per token, summed in the same order)
  any R    |y_send - y_combine| <= u * (sum over ranks of |partial| + |y_send| + |y_combine|)
                                    + (k + R + 2) * 2^-24 * sum over kept slots of |w * row|,
           u the unit roundoff of the activation type: each partial adds one rounding, and both sides sum
           in fp32 (one fp32 rounding per addition; negligible for bf16, the same order as u for fp32)
The full-size workloads are checked on every token where T <= 4096 (all but the 16384-token skewed
prefill) and on 512 sampled tokens for that one; the edge shapes in full.
"""
import numpy as np
import pytest
import torch

import combine_router_gemm_amd as moe
import moe_workloads as W
import oracle
from oracle.sender_combine import combine_recv, combine_send
from tests._hip_runner import check_close, dt_name, rowwise_rel_err, run_layer, to_np, ulp

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-4}
UNIT = {"bf16": 2.0 ** -8, "f32": 2.0 ** -24}


def _sentinel(dtype):
    return torch.tensor([0x7FC1 if dtype == torch.bfloat16 else 0x7FC00001], dtype=torch.int64).item()


def _run_send_recv(out, layout, dtype):
    L = layout
    partial = torch.empty(L.R, L.T, L.H, dtype=dtype, device="cuda")
    bits = partial.view(torch.int16) if dtype == torch.bfloat16 else partial.view(torch.int32)
    bits.fill_(_sentinel(dtype))
    moe.moe_combine_send(out["out_buf"], L, out["w"], partial)
    y = torch.empty(L.T, L.H, dtype=dtype, device="cuda")
    moe.moe_combine_recv(partial, L, y)
    torch.cuda.synchronize()
    return partial, y


def _check(cfg_E, R, out, partial, y, tokens):
    """Compare the GPU partials and y of `tokens` with the oracle on the GPU's out_buf and layout."""
    dt = dt_name(out["y"])
    L = out["layout"]
    pr = to_np(L.pair_row)[tokens]
    off = to_np(L.expert_offset)
    used = np.unique(pr[pr >= 0])
    # monotone remap of the used rows keeps every row inside its rank segment
    new_off = np.searchsorted(used, off, side="left").astype(np.int64)
    pr_local = np.where(pr >= 0, np.searchsorted(used, np.maximum(pr, 0)), -1)
    ob = to_np(out["out_buf"][torch.as_tensor(used, device="cuda", dtype=torch.int64)]) if len(used) else \
        np.zeros((0, L.H), dtype=to_np(out["y"][:1]).dtype)
    w = to_np(out["w"])[tokens]
    ref_p, present = combine_send(ob, dt, pr_local, w, new_off, cfg_E, R)
    tok = torch.as_tensor(tokens, device="cuda", dtype=torch.int64)
    got_p = to_np(partial[:, tok])
    f = oracle.to_f64
    sent = _sentinel(partial.dtype)
    got_bits = got_p.view(np.int16 if dt == "bf16" else np.int32).astype(np.int64) & (0xFFFF if dt == "bf16" else 0xFFFFFFFF)
    # per (rank, token, element): sum over the token's kept slots on that rank of |w * row|
    k = pr_local.shape[1]
    seg = new_off[(np.arange(R + 1) * (cfg_E // R))]
    rank_of = np.searchsorted(seg, np.maximum(pr_local, 0), side="right") - 1
    obf = np.abs(f(ob, dt))
    terms_r = np.zeros((R, len(tokens), L.H))
    for j in range(k):
        m = pr_local[:, j] >= 0
        for r in np.unique(rank_of[m, j]):
            mm = m & (rank_of[:, j] == r)
            terms_r[r][mm] += np.abs(w[mm, j:j + 1].astype(np.float64)) * obf[pr_local[mm, j]]
    bound_y = np.zeros((len(tokens), L.H))
    for r in range(R):
        absent = ~present[r]
        assert np.all(got_bits[r][absent] == sent), f"rank {r}: a slot without kept pairs was written"
        if present[r].any():
            # a float32 sum of the rank's slots rounded once, against the exact sum rounded once
            ref_r = f(ref_p[r][present[r]], dt)
            b = ulp(ref_r, dt) + (k + 1) * 2.0 ** -24 * terms_r[r][present[r]]
            check_close(f(got_p[r][present[r]], dt), ref_r, dt, f"rank {r} partials", TOL[dt], bound=b)
            bound_y[present[r]] += b + (R + 1) * 2.0 ** -24 * np.abs(ref_r)
    ref_y = combine_recv(ref_p, dt, present)
    got_y = f(to_np(y)[tokens], dt)
    # the receive side: its own rounding, plus the partials' differences carried through the sum
    check_close(got_y, f(ref_y, dt), dt, "sender-side y", TOL[dt], bound=bound_y + ulp(f(ref_y, dt), dt))
    # against the receiver-side combine of the same GPU outputs
    y_comb = f(to_np(out["y"])[tokens], dt)
    mag = np.zeros_like(got_y)
    for r in range(R):
        mag[present[r]] += np.abs(f(got_p[r][present[r]], dt))
    terms = terms_r.sum(axis=0)  # sum over kept slots of |w * row|
    bound = UNIT[dt] * (mag + np.abs(got_y) + np.abs(y_comb)) + (k + R + 2) * 2.0 ** -24 * terms + 1e-30
    assert np.all(np.abs(got_y - y_comb) <= bound)
    assert np.all(got_y[(pr < 0).all(axis=1)] == 0.0)
    if R == 1:
        assert np.array_equal(to_np(y)[tokens], to_np(out["y"])[tokens]), "R = 1 must match moe_combine bit for bit"
    dev = rowwise_rel_err(got_y, y_comb)
    return int(present.sum()), int((pr >= 0).sum()), float(dev.max(initial=0.0))


@pytest.mark.parametrize("wl", list(W.WORKLOADS))
def test_sender_side_combine_full_size(wl):
    cfg = W.workload(wl)
    print(f"\n[gpu] sender-side combine: {W.describe(cfg)}", flush=True)
    inp = W.make_inputs(cfg, device="cuda")
    out = run_layer(inp, cfg.k, cfg.R)
    partial, y = _run_send_recv(out, out["layout"], inp["x"].dtype)
    tokens = np.arange(cfg.T) if cfg.T <= 4096 else np.sort(np.random.default_rng(3).choice(cfg.T, 512, replace=False))
    p_rows, k_rows, dev = _check(cfg.E, cfg.R, out, partial, y, tokens)
    print(f"[gpu] {wl}: partial rows {p_rows} vs kept rows {k_rows} ({p_rows / max(k_rows, 1):.3f}); "
          f"max per-token distance to moe_combine {dev:.2e}")
    del out, partial, y, inp
    torch.cuda.empty_cache()


EDGE = [
    # name, T, H, E, k, F, R, C, dtype, routing
    ("capacity0", 64, 64, 8, 2, 64, 2, 0, "bf16", "uniform"),
    ("T1_R4", 1, 64, 8, 2, 64, 4, 1, "bf16", "uniform"),
    ("T0", 0, 64, 8, 2, 64, 2, 1, "bf16", "uniform"),
    ("k_eq_E_R4", 70, 64, 8, 8, 64, 4, 70, "bf16", "uniform"),
    ("ragged_f32_R3", 301, 40, 6, 2, 24, 3, 77, "f32", "zipf"),
    ("R8_El2", 160, 64, 16, 4, 32, 8, 40, "bf16", "uniform"),
    ("E512_k8_R8", 300, 64, 512, 8, 32, 8, 5, "bf16", "zipf"),
    ("R512_one_expert_per_rank", 200, 72, 512, 8, 32, 512, 4, "bf16", "zipf"),
    ("hot_overflow_R4", 512, 128, 64, 6, 64, 4, 48, "bf16", "hot8"),
]


@pytest.mark.parametrize("name,T,H,E,k,F,R,C,dtype,routing", EDGE, ids=[e[0] for e in EDGE])
def test_sender_side_combine_edge_cases(name, T, H, E, k, F, R, C, dtype, routing):
    cfg = W.small_config(W.workload("tiny-fp32"), seed=500 + [e[0] for e in EDGE].index(name), name=name,
                         T=max(T, 1), H=H, E=E, k=k, F=F, R=R, dtype=dtype, routing=routing)
    inp = W.make_inputs(cfg, device="cuda", T=T)
    inp["C"] = C
    print(f"\n[gpu] sender-side combine edge case {name}", flush=True)
    out = run_layer(inp, k, R)
    partial, y = _run_send_recv(out, out["layout"], inp["x"].dtype)
    if T == 0:
        return
    _check(E, R, out, partial, y, np.arange(T))
