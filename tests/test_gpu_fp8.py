"""GPU parity of the fp8 block-scaled dispatch and of the expert MLP on its rows, through the C ABI.

The routing is the GPU's own (route is checked in test_gpu_parity.py); each stage is then checked on the
GPU's upstream output:
  F3 dispatch  every layout array bit-exact vs the oracle dispatch; E4M3 codes and block scales bit-exact
               vs the oracle's quantisation of the GPU's send rows (all rows for the Mixtral and Kimi-share
               decode batches, a sample of 2048 rows plus the first and last for the two prefill batches)
  F4 MLP       per-row normwise rel <= 2e-2 vs the oracle MLP on the GPU's decoded codes
  F6 layer     per-token normwise rel <= 2e-2 vs the oracle layer with fp8 dispatch (GPU ids); all-dropped
               tokens exactly 0
  fp8 vs bf16  the fp8 layer stays within 0.1 per-token normwise of the bf16 layer: E4M3 keeps 4
               significant bits, so each element carries up to 2^-4 relative rounding error (about 3 %
               normwise over a row), and gate * up roughly doubles it in the output (the oracle itself
               shows 4-5 %)
"""
import numpy as np
import pytest
import torch

import moe_workloads as W
import oracle
from oracle import fp8
from tests._hip_runner import LazyExperts, check_close, layer_bound, rowwise_rel_err, run_layer, run_layer_fp8, to_np

pytestmark = pytest.mark.gpu

TOL = 2e-2
FP8_VS_BF16 = 0.1
WORKLOADS = ["mixtral8x7b-decode", "dsv3-prefill-ep8-share", "kimik2-decode-ep8-share", "large-skewed-prefill"]
# workloads the oracle finishes whole in seconds (the others are sampled)
FULL = {"mixtral8x7b-decode", "kimik2-decode-ep8-share"}

_cache = {}


def _layer(wl):
    if wl not in _cache:
        cfg = W.workload(wl)
        print(f"\n[gpu] fp8 path: {W.describe(cfg)}", flush=True)
        inp = W.make_inputs(cfg, device="cuda")
        _cache.clear()
        _cache[wl] = (cfg, inp, run_layer_fp8(inp, cfg.k, cfg.R))
    return _cache[wl]


def _bias_np(inp):
    return None if inp["bias"] is None else to_np(inp["bias"])


def _check_dispatch(cfg, inp, out, rows=None):
    x = to_np(inp["x"])
    ids = to_np(out["ids"])
    lay, _ = oracle.dispatch(x, "bf16", ids, cfg.E, inp["C"], cfg.R)
    L = out["layout"]
    for name in ("expert_count", "expert_kept", "expert_overflow", "expert_offset", "pair_row"):
        assert np.array_equal(to_np(getattr(L, name)), getattr(lay, name)), name
    n = lay.total
    assert np.array_equal(to_np(L.row_token)[:n], lay.row_token)
    assert np.array_equal(to_np(L.row_slot)[:n], lay.row_slot)
    if rows is None:
        rows = np.arange(n)
    if len(rows) == 0:
        return lay
    idx = torch.as_tensor(rows, device="cuda", dtype=torch.int64)
    codes, scales = fp8.quantize_rows(x[lay.row_token[rows]])
    assert np.array_equal(to_np(out["send_q"][idx]), codes)
    assert np.array_equal(to_np(out["send_scale"][idx]), scales)
    return lay


@pytest.mark.parametrize("wl", WORKLOADS)
def test_f3_dispatch_fp8(wl):
    cfg, inp, out = _layer(wl)
    n = int(to_np(out["layout"].expert_offset)[cfg.E])
    rows = None
    if wl not in FULL and n > 2048:
        rows = np.unique(np.concatenate([[0, n - 1], np.random.default_rng(cfg.seed).choice(n, 2048, replace=False)]))
    _check_dispatch(cfg, inp, out, rows)
    print(f"[gpu] {wl}: fp8 rows checked {n if rows is None else len(rows)} of {n}")


@pytest.mark.parametrize("wl", WORKLOADS)
def test_f4_expert_mlp_fp8(wl):
    cfg, inp, out = _layer(wl)
    offset = to_np(out["layout"].expert_offset)
    rex = oracle.row_experts(offset, cfg.E)
    total = int(offset[cfg.E])
    if wl in FULL:
        rows = np.arange(total)
    else:
        rng = np.random.default_rng(100 + cfg.seed)
        local = rex % cfg.El
        chosen = rng.choice(np.unique(local), size=min(6, len(np.unique(local))), replace=False)
        rows = []
        for l in chosen:
            r = np.nonzero(local == l)[0]
            rows += [int(r[0]), int(r[-1])] + [int(v) for v in rng.choice(r, size=min(8, len(r)), replace=False)]
        rows = np.array(sorted(set(rows)), dtype=np.int64)
    if len(rows) == 0:
        return
    idx = torch.as_tensor(rows, device="cuda")
    a = fp8.dequantize_rows_bf16(to_np(out["send_q"][idx]), to_np(out["send_scale"][idx]))
    ref = oracle.expert_mlp(a, "bf16", rex[rows], cfg.El, LazyExperts(inp["w_gate_up"]), LazyExperts(inp["w_down"]),
                            cfg.F)
    got = to_np(out["out_buf"][idx])
    msg = check_close(oracle.to_f64(got, "bf16"), oracle.to_f64(ref, "bf16"), "bf16", f"{wl} fp8 MLP", TOL)
    print(f"[gpu] {msg}")


def _oracle_layer_fp8(cfg, inp, ids, C, tokens):
    """Oracle layer with fp8 dispatch for `tokens`, routing on the given ids."""
    x = to_np(inp["x"])
    bias = _bias_np(inp)
    sub_bias = None if bias is None else (bias if bias.ndim == 1 else bias[tokens])
    lg = oracle.router_logits(x[tokens], "bf16", to_np(inp["w_router"]), sub_bias)
    w = oracle.routing_weights(lg, ids[tokens])
    lay, codes, scales = fp8.dispatch_fp8(x, ids, cfg.E, C, cfg.R)
    rex = oracle.row_experts(lay.expert_offset, cfg.E)
    pr = lay.pair_row[tokens]
    used = np.unique(pr[pr >= 0])
    a = fp8.dequantize_rows_bf16(codes[used], scales[used]) if len(used) else np.zeros((0, cfg.H), np.uint16)
    out_rows = oracle.expert_mlp(a, "bf16", rex[used], cfg.El, LazyExperts(inp["w_gate_up"]),
                                 LazyExperts(inp["w_down"]), cfg.F) if len(used) else a
    remap = np.full(max(lay.total, 1), -1, dtype=np.int64)
    remap[used] = np.arange(len(used))
    pr_local = np.where(pr >= 0, remap[np.maximum(pr, 0)], -1)
    return oracle.combine(out_rows, "bf16", pr_local, w), out_rows, pr_local, w


def _check_layer(y64, ref, what):
    """The fp8 layer against the oracle's: row tolerance, and per element the expert-MLP element bound
    carried through the weighted sum."""
    y_ref, rows, pr_local, w = ref
    f = oracle.to_f64
    return check_close(y64, f(y_ref, "bf16"), "bf16", what, TOL,
                       bound=layer_bound(f(y_ref, "bf16"), f(rows, "bf16"), pr_local, w, "bf16"))


@pytest.mark.parametrize("wl", WORKLOADS)
def test_f6_layer_fp8_and_distance_to_bf16(wl):
    cfg, inp, out = _layer(wl)
    ids = to_np(out["ids"])
    tokens = np.arange(cfg.T) if wl in FULL else np.sort(np.random.default_rng(21).choice(cfg.T, 48, replace=False))
    ref = _oracle_layer_fp8(cfg, inp, ids, inp["C"], tokens)
    y = oracle.to_f64(to_np(out["y"])[tokens], "bf16")
    msg = _check_layer(y, ref, f"{wl} fp8 layer")
    dropped = (to_np(out["layout"].pair_row)[tokens] < 0).all(axis=1)
    assert np.all(y[dropped] == 0.0)
    # the same layer with bf16 dispatch
    bf = run_layer(inp, cfg.k, cfg.R)
    assert torch.equal(bf["ids"], out["ids"])
    yb = oracle.to_f64(to_np(bf["y"])[tokens], "bf16")
    live = ~dropped
    dev = rowwise_rel_err(y[live], yb[live])
    assert np.all(dev <= FP8_VS_BF16), f"fp8 vs bf16 worst token {dev.max():.3f}"
    print(f"[gpu] {msg}; distance to the bf16 layer mean {dev.mean():.3f}, max {dev.max():.3f}")
    del bf


def test_release():
    _cache.clear()
    torch.cuda.empty_cache()


EDGE = [
    # name, T, H, E, k, F, R, C, routing
    ("capacity0", 64, 128, 8, 2, 64, 1, 0, "uniform"),
    ("T0", 0, 128, 8, 2, 64, 1, 1, "uniform"),
    ("T1", 1, 128, 8, 2, 64, 1, 1, "uniform"),
    ("k_eq_E", 70, 256, 8, 8, 64, 4, 70, "uniform"),
    ("ragged_R3_three_blocks", 257, 384, 12, 4, 72, 3, 70, "zipf"),
    ("dec64_tiles", 300, 128, 8, 2, 96, 1, 100, "zipf"),
    ("register_staged_prefill_tiles", 700, 256, 4, 2, 192, 1, 300, "uniform"),
    ("extreme_rows", 200, 256, 8, 2, 64, 1, 60, "uniform"),
]


@pytest.mark.parametrize("name,T,H,E,k,F,R,C,routing", EDGE, ids=[e[0] for e in EDGE])
def test_fp8_edge_cases(name, T, H, E, k, F, R, C, routing):
    cfg = W.small_config(W.workload("mixtral8x7b-decode"), seed=400 + [e[0] for e in EDGE].index(name), name=name,
                         T=max(T, 1), H=H, E=E, k=k, F=F, R=R, dtype="bf16", routing=routing)
    inp = W.make_inputs(cfg, device="cuda", T=T)
    inp["C"] = C
    if name == "extreme_rows":
        # all-zero rows, rows scaled far up and far down, one row with a single nonzero element
        x = inp["x"].float()
        x[0] = 0.0
        x[1] *= 1.0e4
        x[2] *= 1.0e-4
        x[3] = 0.0
        x[3, 77] = -3.0
        x[4, :128] = 0.0
        inp["x"] = x.to(torch.bfloat16)
    print(f"\n[gpu] fp8 edge case {name}", flush=True)
    out = run_layer_fp8(inp, k, R)
    if T == 0:
        L = out["layout"]
        assert np.all(to_np(L.expert_count) == 0) and np.all(to_np(L.expert_offset) == 0)
        return
    lay = _check_dispatch(cfg, inp, out)
    n = lay.total
    rex = oracle.row_experts(lay.expert_offset, E)
    if n:
        a = fp8.dequantize_rows_bf16(to_np(out["send_q"][:n]), to_np(out["send_scale"][:n]))
        ref_ob = oracle.expert_mlp(a, "bf16", rex, E // R, to_np(inp["w_gate_up"]), to_np(inp["w_down"]), F)
        check_close(oracle.to_f64(to_np(out["out_buf"][:n]), "bf16"), oracle.to_f64(ref_ob, "bf16"), "bf16",
                    "fp8 MLP", TOL)
    ids = to_np(out["ids"])
    _check_layer(oracle.to_f64(to_np(out["y"]), "bf16"), _oracle_layer_fp8(cfg, inp, ids, C, np.arange(T)),
                 "fp8 layer")
