"""GPU parity: the HIP path (through the C ABI) against the CPU oracle, stage by stage.

Parity chain: each stage is checked on the GPU's own upstream output, so a top-k tie decided by the
last bit of an fp32 logit cannot cascade.
  P1 logits   per row max|d| <= 1e-5 * max|ref|               (router logits, fp32)
  P2 top-k    ids bit-exact vs oracle top-k of the GPU logits; weights rel <= 1e-5
  P3 dispatch every layout array and send_buf[:total] bit-exact vs oracle dispatch of the GPU ids
  P4 MLP      per-row normwise rel <= 2e-2 (bf16) / 1e-4 (fp32) vs oracle MLP of the GPU send_buf
  P5 combine  per-token normwise rel <= 2e-2 / 1e-4 vs oracle combine of the GPU out_buf
  P6 layer    oracle layer from x (routing on the GPU ids) vs y; all-dropped tokens exactly 0
The five workloads run at full size; where the oracle cannot finish the whole output in seconds
(expert MLP at 2.9-6 TFLOP) it checks sampled rows and tokens, including each sampled expert's first
and last rows and the rows around a 128-row tile edge.
"""
import numpy as np
import pytest
import torch

import moe_workloads as W
import oracle
from tests._hip_runner import LazyExperts, dt_name, rowwise_rel_err, run_layer, to_np

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-4}

_cache = {}


def _layer(wl):
    """Inputs (device) and HIP outputs of one full-size workload, computed once per session."""
    if wl not in _cache:
        cfg = W.workload(wl)
        print(f"\n[gpu] running {W.describe(cfg)}", flush=True)
        inp = W.make_inputs(cfg, device="cuda")
        out = run_layer(inp, cfg.k, cfg.R)
        _cache[wl] = (cfg, inp, out)
    return _cache[wl]


def _bias_np(inp):
    return None if inp["bias"] is None else to_np(inp["bias"])


WORKLOADS = list(W.WORKLOADS)
# workloads whose whole expert MLP the oracle finishes in seconds (the others are sampled)
FULL_MLP = {"tiny-fp32", "mixtral8x7b-decode", "kimik2-decode-ep8-share"}


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else (t.view(torch.int32) if t.dtype == torch.float32 else t)


@pytest.mark.parametrize("wl", WORKLOADS)
def test_p1_p2_route(wl):
    cfg, inp, out = _layer(wl)
    dt = dt_name(inp["x"])
    x = to_np(inp["x"])
    ref = oracle.router_logits(x, dt, to_np(inp["w_router"]), _bias_np(inp))
    got = to_np(out["logits"])
    err = np.abs(got.astype(np.float64) - ref).max(axis=1)
    scale = np.abs(ref.astype(np.float64)).max(axis=1)
    assert np.all(err <= 1e-5 * scale), f"worst row ratio {np.max(err / scale):.3e}"
    ids = to_np(out["ids"])
    assert np.array_equal(ids, oracle.topk_select(got, cfg.k))
    w_ref = oracle.routing_weights(got, ids)
    w = to_np(out["w"])
    assert np.all(np.abs(w.astype(np.float64) - w_ref) <= 1e-5 * np.abs(w_ref.astype(np.float64)) + 1e-30)
    # where the oracle's own fp32 logits pick different experts, the choice must be a near tie
    own = oracle.topk_select(ref, cfg.k)
    flips = np.nonzero((own != ids).any(axis=1))[0]
    for t in flips:
        srt = np.sort(ref[t].astype(np.float64))[::-1]
        gap = srt[cfg.k - 1] - srt[cfg.k]
        assert gap <= 2e-5 * scale[t], (t, gap)
    print(f"[gpu] {wl}: logits worst row ratio {np.max(err / scale):.2e}, top-k flips vs oracle's "
          f"own logits {len(flips)}")


@pytest.mark.parametrize("wl", WORKLOADS)
def test_p3_dispatch(wl):
    cfg, inp, out = _layer(wl)
    dt = dt_name(inp["x"])
    lay, sb = oracle.dispatch(to_np(inp["x"]), dt, to_np(out["ids"]), cfg.E, inp["C"], cfg.R)
    L = out["layout"]
    for name in ("expert_count", "expert_kept", "expert_overflow", "expert_offset", "pair_row"):
        assert np.array_equal(to_np(getattr(L, name)), getattr(lay, name)), name
    n = lay.total
    assert np.array_equal(to_np(L.row_token)[:n], lay.row_token)
    assert np.array_equal(to_np(L.row_slot)[:n], lay.row_slot)
    assert np.array_equal(to_np(out["send_buf"][:n]), sb)
    # the invariants the pages state: counts = router histogram, overflow = max(count - C, 0)
    ids = to_np(out["ids"])
    assert np.array_equal(lay.expert_count, np.bincount(ids.ravel(), minlength=cfg.E))
    print(f"[gpu] {wl}: rows {n} of {cfg.T * cfg.k} pairs, overflow {int(lay.expert_overflow.sum())}, "
          f"experts over capacity {int((lay.expert_overflow > 0).sum())}")


def _sample_rows(offset_l, BM=128, per_expert=10, max_experts=6, seed=0):
    """Rows of a few local experts: first, last, around a tile edge, and random ones."""
    rng = np.random.default_rng(seed)
    El = len(offset_l) - 1
    nonempty = [l for l in range(El) if offset_l[l + 1] > offset_l[l]]
    if not nonempty:
        return {}
    chosen = sorted(set([nonempty[0], nonempty[-1]] + list(
        rng.choice(nonempty, size=min(max_experts, len(nonempty)), replace=False))))
    out = {}
    for l in chosen:
        lo, hi = offset_l[l], offset_l[l + 1]
        m = hi - lo
        cand = {0, m - 1, min(BM - 1, m - 1), min(BM, m - 1)}
        cand |= set(rng.integers(0, m, size=per_expert).tolist())
        out[l] = sorted(lo + c for c in cand)
    return out


@pytest.mark.parametrize("wl", WORKLOADS)
def test_p4_expert_mlp(wl):
    cfg, inp, out = _layer(wl)
    dt = dt_name(inp["x"])
    L = out["layout"]
    offset = to_np(L.expert_offset)
    rex = oracle.row_experts(offset, cfg.E)
    total = int(offset[cfg.E])
    if wl in FULL_MLP:
        rows = np.arange(total)
    else:
        # plan order groups rows by local expert; sample per local expert over all rank segments
        El = cfg.El
        local = rex % El
        rows = []
        per_l = [np.nonzero(local == l)[0] for l in range(El)]
        off_l = np.concatenate([[0], np.cumsum([len(p) for p in per_l])])
        for l, picks in _sample_rows(off_l, seed=cfg.seed).items():
            rows += [int(per_l[l][p - off_l[l]]) for p in picks]
        rows = np.array(sorted(set(rows)), dtype=np.int64)
    sb = to_np(out["send_buf"][torch.as_tensor(rows, device="cuda")]) if len(rows) else None
    if len(rows) == 0:
        return
    ref = oracle.expert_mlp(sb, dt, rex[rows], cfg.El, LazyExperts(inp["w_gate_up"]),
                            LazyExperts(inp["w_down"]), cfg.F)
    got = to_np(out["out_buf"][torch.as_tensor(rows, device="cuda")])
    f = oracle.to_f64
    err = rowwise_rel_err(f(got, dt), f(ref, dt))
    assert np.all(err <= TOL[dt]), f"max rel err {err.max():.3e} over {len(rows)} rows"
    print(f"[gpu] {wl}: MLP rows checked {len(rows)}, max rel err {err.max():.2e}")


@pytest.mark.parametrize("wl", WORKLOADS)
def test_p5_combine(wl):
    cfg, inp, out = _layer(wl)
    dt = dt_name(inp["x"])
    L = out["layout"]
    pr = to_np(L.pair_row)
    w = to_np(out["w"])
    T = cfg.T
    tokens = np.arange(T) if T <= 4096 else np.sort(np.random.default_rng(5).choice(T, 2048, replace=False))
    sub_pr = pr[tokens]
    used = np.unique(sub_pr[sub_pr >= 0])
    remap = np.full(max(int(L.rows_max), 1), -1, dtype=np.int64)
    remap[used] = np.arange(len(used))
    ob = to_np(out["out_buf"][torch.as_tensor(used, device="cuda", dtype=torch.int64)]) if len(used) else \
        np.zeros((0, cfg.H), dtype=to_np(out["y"][:1]).dtype)
    pr_local = np.where(sub_pr >= 0, remap[np.maximum(sub_pr, 0)], -1)
    ref = oracle.combine(ob, dt, pr_local, w[tokens])
    got = to_np(out["y"])[tokens]
    f = oracle.to_f64
    err = rowwise_rel_err(f(got, dt), f(ref, dt))
    assert np.all(err <= TOL[dt]), f"max rel err {err.max():.3e}"
    dropped = (sub_pr < 0).all(axis=1)
    assert np.all(f(got, dt)[dropped] == 0.0)
    print(f"[gpu] {wl}: combine tokens {len(tokens)}, fully dropped {int(dropped.sum())}, "
          f"max rel err {err.max():.2e}")


def _oracle_layer_tokens(cfg, inp, ids, C, tokens):
    """Oracle layer output for `tokens`, routing on the given ids (weights from the oracle's logits).

    Dispatch positions depend on every token, so dispatch runs on all ids; the expert MLP runs only
    on the rows of the chosen tokens."""
    dt = dt_name(inp["x"])
    x = to_np(inp["x"])
    bias = _bias_np(inp)
    sub_bias = None if bias is None else (bias if bias.ndim == 1 else bias[tokens])
    lg = oracle.router_logits(x[tokens], dt, to_np(inp["w_router"]), sub_bias)
    w = oracle.routing_weights(lg, ids[tokens])
    lay, sb = oracle.dispatch(x, dt, ids, cfg.E, C, cfg.R)
    rex = oracle.row_experts(lay.expert_offset, cfg.E)
    pr = lay.pair_row[tokens]
    used = np.unique(pr[pr >= 0])
    out_rows = oracle.expert_mlp(sb[used], dt, rex[used], cfg.El, LazyExperts(inp["w_gate_up"]),
                                 LazyExperts(inp["w_down"]), cfg.F) if len(used) else sb[:0]
    remap = np.full(max(lay.total, 1), -1, dtype=np.int64)
    remap[used] = np.arange(len(used))
    pr_local = np.where(pr >= 0, remap[np.maximum(pr, 0)], -1)
    return oracle.combine(out_rows, dt, pr_local, w)


@pytest.mark.parametrize("wl", WORKLOADS)
def test_p6_layer_end_to_end(wl):
    cfg, inp, out = _layer(wl)
    dt = dt_name(inp["x"])
    ids = to_np(out["ids"])
    if wl in FULL_MLP:
        tokens = np.arange(cfg.T)
    else:
        tokens = np.sort(np.random.default_rng(11).choice(cfg.T, 48, replace=False))
    ref = _oracle_layer_tokens(cfg, inp, ids, inp["C"], tokens)
    got = to_np(out["y"])[tokens]
    f = oracle.to_f64
    err = rowwise_rel_err(f(got, dt), f(ref, dt))
    assert np.all(err <= TOL[dt]), f"max rel err {err.max():.3e}"
    print(f"[gpu] {wl}: layer tokens {len(tokens)}, max rel err {err.max():.2e}")


def test_determinism_bitwise():
    cfg, inp, out = _layer("dsv3-prefill-ep8-share")
    again = run_layer(inp, cfg.k, cfg.R)
    for key in ("logits", "ids", "w", "send_buf", "out_buf", "y"):
        assert torch.equal(_bits(out[key]), _bits(again[key])), key


def test_release_full_size_buffers():
    _cache.clear()
    torch.cuda.empty_cache()


# --------------------------------------------------------------------------------------------------
# edge cases at sizes the oracle finishes in full
# --------------------------------------------------------------------------------------------------

EDGE = [
    # name, T, H, E, k, F, R, C, dtype, routing
    ("capacity0", 64, 64, 8, 2, 64, 1, 0, "bf16", "uniform"),
    ("capacity_ge_T", 96, 64, 8, 2, 64, 2, 101, "f32", "uniform"),
    ("k1", 200, 128, 8, 1, 96, 1, 20, "bf16", "uniform"),
    ("k_eq_E", 70, 64, 8, 8, 64, 4, 70, "bf16", "uniform"),
    ("E10_R2", 130, 96, 10, 3, 48, 2, 30, "bf16", "uniform"),
    ("ragged_R3", 257, 136, 12, 4, 72, 3, 70, "bf16", "zipf"),
    ("ragged_f32", 301, 40, 6, 2, 24, 3, 77, "f32", "zipf"),
    ("T1", 1, 64, 8, 2, 64, 1, 1, "bf16", "uniform"),
    ("T0", 0, 64, 8, 2, 64, 1, 1, "bf16", "uniform"),
    ("R8_El2", 160, 64, 16, 4, 32, 8, 40, "bf16", "uniform"),
    ("E512_k8", 300, 64, 512, 8, 32, 8, 5, "bf16", "zipf"),
    ("hot_overflow", 512, 128, 64, 6, 64, 1, 48, "bf16", "hot8"),
    ("many_rows_tile_edges", 700, 128, 4, 2, 160, 1, 300, "bf16", "uniform"),
    # direct-to-LDS grouped GEMM: 128-row tiles (400 rows per expert), then 256-row tiles (2200 rows per
    # local expert); F = 192 and H = 192 / 320 leave a ragged last column tile in both GEMMs
    ("dl128_ragged", 900, 192, 4, 2, 192, 1, 400, "bf16", "zipf"),
    ("dl256_ragged_R2", 2600, 320, 4, 2, 192, 2, 1100, "bf16", "zipf"),
    # 64-row weight-streaming tiles (capacity 75 rows per expert on average), hot experts over 64 rows
    ("dec64_multi_mtile", 300, 128, 8, 2, 96, 1, 100, "bf16", "zipf"),
    # one counting block (T <= 256) scans all 512 experts itself
    ("E512_one_block", 200, 64, 512, 8, 32, 8, 4, "bf16", "zipf"),
]


@pytest.mark.parametrize("name,T,H,E,k,F,R,C,dtype,routing", EDGE, ids=[e[0] for e in EDGE])
def test_edge_cases(name, T, H, E, k, F, R, C, dtype, routing):
    base = W.workload("tiny-fp32")
    cfg = W.small_config(base, seed=100 + EDGE.index(next(e for e in EDGE if e[0] == name)), name=name,
                         T=max(T, 1), H=H, E=E, k=k, F=F, R=R, dtype=dtype, routing=routing)
    inp = W.make_inputs(cfg, device="cuda", T=T)
    inp["C"] = C
    print(f"\n[gpu] edge case {name}", flush=True)
    out = run_layer(inp, k, R)
    check_layer_full(cfg, inp, out, T, E, k, F, R, C)


def check_layer_full(cfg, inp, out, T, E, k, F, R, C):
    """Every stage of a small layer against the whole oracle (route on the GPU logits, dispatch and send
    rows bit-exact, expert MLP, combine and the layer within the activation type's tolerance)."""
    if T == 0:
        L = out["layout"]
        assert np.all(to_np(L.expert_count) == 0) and np.all(to_np(L.expert_offset) == 0)
        return
    dt = dt_name(inp["x"])
    ids = to_np(out["ids"])
    got_lg = to_np(out["logits"])
    assert np.array_equal(ids, oracle.topk_select(got_lg, k))
    lay, sb = oracle.dispatch(to_np(inp["x"]), dt, ids, E, C, R)
    L = out["layout"]
    for nm in ("expert_count", "expert_kept", "expert_overflow", "expert_offset", "pair_row"):
        assert np.array_equal(to_np(getattr(L, nm)), getattr(lay, nm)), nm
    n = lay.total
    assert np.array_equal(to_np(L.row_token)[:n], lay.row_token)
    assert np.array_equal(to_np(out["send_buf"][:n]), sb)
    rex = oracle.row_experts(lay.expert_offset, E)
    if n:
        ref_ob = oracle.expert_mlp(to_np(out["send_buf"][:n]), dt, rex, E // R, to_np(inp["w_gate_up"]),
                                   to_np(inp["w_down"]), F)
        err = rowwise_rel_err(oracle.to_f64(to_np(out["out_buf"][:n]), dt), oracle.to_f64(ref_ob, dt))
        assert np.all(err <= TOL[dt]), f"MLP max rel err {err.max():.3e}"
    ref_y = oracle.combine(to_np(out["out_buf"]), dt, lay.pair_row, to_np(out["w"]))
    y = oracle.to_f64(to_np(out["y"]), dt)
    err = rowwise_rel_err(y, oracle.to_f64(ref_y, dt))
    assert np.all(err <= TOL[dt]), f"combine max rel err {err.max():.3e}"
    dropped = (lay.pair_row < 0).all(axis=1)
    assert np.all(y[dropped] == 0.0)
    full = _oracle_layer_tokens(cfg, inp, ids, C, np.arange(T))
    err = rowwise_rel_err(y, oracle.to_f64(full, dt))
    assert np.all(err <= TOL[dt]), f"layer max rel err {err.max():.3e}"
