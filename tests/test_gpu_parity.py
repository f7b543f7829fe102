"""GPU parity: the HIP path (through the C ABI) against the CPU oracle, stage by stage.

Parity chain: each stage is checked on the GPU's own upstream output, so a top-k tie decided by the
last bit of an fp32 logit cannot cascade.
  P1 logits   per row max|d| <= 1e-5 * max|ref|               (router logits, fp32)
  P2 top-k    ids bit-exact vs oracle top-k of the GPU logits; weights rel <= 1e-5
  P3 dispatch every layout array and send_buf[:total] bit-exact vs oracle dispatch of the GPU ids
  P4 MLP      every row of every local expert: per-row normwise rel <= 2e-2 (bf16) / 1e-4 (fp32) and
              per element |d| <= 2 ulp(ref) + c rms(ref row) (c = 2^-6 bf16, 1e-4 fp32) vs the oracle MLP
              of the GPU send_buf; the oracle holds one local expert's weights at a time, in chunks of
              experts for the prefill workloads
  P5 combine  every token: per element |d| <= ulp(ref) + (k + 1) 2^-24 sum_j |w_j out_j| (a float32 sum
              rounded once, against the exact sum rounded once) vs oracle combine of the GPU out_buf
  P6 layer    every token: the oracle layer from x (routing on the GPU ids); per element the P4 bound
              carried through the weighted sum; all-dropped tokens exactly 0
The five workloads run at full size, in the launch configuration the benchmark times.
"""
import numpy as np
import pytest
import torch

import moe_workloads as W
import oracle
from tests._hip_runner import (check_close, combine_abs_sum, dt_name, layer_bound, run_layer, sum_bound_ratio,
                               to_np)

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-4}

_cache = {}
_oracle_rows = {}


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
# chunks of local experts for the expert-MLP check (the oracle converts one expert's weights at a time)
CHUNKS = {"tiny-fp32": 1, "mixtral8x7b-decode": 2, "dsv3-prefill-ep8-share": 2, "kimik2-decode-ep8-share": 1,
          "large-skewed-prefill": 8}
P4_CASES = [(wl, c) for wl in WORKLOADS for c in range(CHUNKS[wl])]


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else (t.view(torch.int32) if t.dtype == torch.float32 else t)


def p1_check(got_lg, ref_lg):
    """P1: per row max|d| <= 1e-5 max|ref|; returns the worst row's ratio."""
    err = np.abs(got_lg.astype(np.float64) - ref_lg).max(axis=1)
    scale = np.abs(ref_lg.astype(np.float64)).max(axis=1)
    ratio = np.where(scale > 0, err / np.where(scale > 0, scale, 1.0), np.where(err > 0, np.inf, 0.0))
    assert np.all(ratio <= 1e-5), f"worst row ratio {np.max(ratio):.3e}"
    return float(ratio.max()) if ratio.size else 0.0


@pytest.mark.parametrize("wl", WORKLOADS)
def test_p1_p2_route(wl):
    cfg, inp, out = _layer(wl)
    dt = dt_name(inp["x"])
    x = to_np(inp["x"])
    ref = oracle.router_logits(x, dt, to_np(inp["w_router"]), _bias_np(inp))
    got = to_np(out["logits"])
    worst = p1_check(got, ref)
    ids = to_np(out["ids"])
    assert np.array_equal(ids, oracle.topk_select(got, cfg.k))
    w_ref = oracle.routing_weights(got, ids)
    w = to_np(out["w"])
    assert np.all(np.abs(w.astype(np.float64) - w_ref) <= 1e-5 * np.abs(w_ref.astype(np.float64)) + 1e-30)
    # where the oracle's own fp32 logits pick different experts, the choice must be a near tie
    own = oracle.topk_select(ref, cfg.k)
    flips = np.nonzero((own != ids).any(axis=1))[0]
    scale = np.abs(ref.astype(np.float64)).max(axis=1)
    for t in flips:
        srt = np.sort(ref[t].astype(np.float64))[::-1]
        gap = srt[cfg.k - 1] - srt[cfg.k]
        assert gap <= 2e-5 * scale[t], (t, gap)
    print(f"[gpu] {wl}: logits worst row max|d|/max|ref| {worst:.2e} (bound 1e-5), top-k flips vs oracle's "
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


def _oracle_mlp_chunk(wl, chunk):
    """The oracle's expert MLP on every GPU send row of local experts [El*chunk/n, El*(chunk+1)/n): a dict
    l -> (send-row indices, oracle output rows in storage form). Cached for the layer check."""
    key = (wl, chunk)
    if key in _oracle_rows:
        return _oracle_rows[key]
    cfg, inp, out = _layer(wl)
    dt = dt_name(inp["x"])
    El, nch = cfg.El, CHUNKS[wl]
    offset = to_np(out["layout"].expert_offset)
    rex = oracle.row_experts(offset, cfg.E)
    local = rex % El
    res = {}
    for l in range(El * chunk // nch, El * (chunk + 1) // nch):
        rows = np.nonzero(local == l)[0]
        if len(rows) == 0:
            continue
        sb = to_np(out["send_buf"][torch.as_tensor(rows, device="cuda")])
        ref = oracle.expert_mlp(sb, dt, rex[rows], El, {l: to_np(inp["w_gate_up"][l])},
                                {l: to_np(inp["w_down"][l])}, cfg.F)
        res[l] = (rows, ref)
    _oracle_rows[key] = res
    return res


@pytest.mark.parametrize("wl,chunk", P4_CASES, ids=[f"{c[0]}-{c[1]}" for c in P4_CASES])
def test_p4_expert_mlp(wl, chunk):
    cfg, inp, out = _layer(wl)
    dt = dt_name(inp["x"])
    res = _oracle_mlp_chunk(wl, chunk)
    f = oracle.to_f64
    n_rows, worst_err, worst_ratio = 0, 0.0, 0.0
    for l, (rows, ref) in res.items():
        got = to_np(out["out_buf"][torch.as_tensor(rows, device="cuda")])
        check_close(f(got, dt), f(ref, dt), dt, f"{wl} MLP local expert {l}", TOL[dt])
        n, e, r = check_close.last
        n_rows, worst_err, worst_ratio = n_rows + n, max(worst_err, e), max(worst_ratio, r)
    El, nch = cfg.El, CHUNKS[wl]
    local = oracle.row_experts(to_np(out["layout"].expert_offset), cfg.E) % El
    lo, hi = El * chunk // nch, El * (chunk + 1) // nch
    assert n_rows == int(((local >= lo) & (local < hi)).sum())   # every row of these experts
    print(f"[gpu] {wl}: MLP local experts {lo}..{hi - 1}: {n_rows} rows, max normwise {worst_err:.2e}, "
          f"max element/bound {worst_ratio:.3f}")


@pytest.mark.parametrize("wl", WORKLOADS)
def test_p5_combine(wl):
    cfg, inp, out = _layer(wl)
    dt = dt_name(inp["x"])
    L = out["layout"]
    pr = to_np(L.pair_row)
    w = to_np(out["w"])
    total = int(to_np(L.expert_offset)[cfg.E])
    ob = to_np(out["out_buf"][:total])
    ref = oracle.combine(ob, dt, pr, w)
    got = to_np(out["y"])
    f = oracle.to_f64
    ob64 = f(ob, dt)
    ratio = sum_bound_ratio(f(got, dt), f(ref, dt), combine_abs_sum(ob64, pr, w), cfg.k, dt)
    msg = check_close(f(got, dt), f(ref, dt), dt, f"{wl} combine", TOL[dt], ratio=ratio)
    dropped = (pr < 0).all(axis=1)
    assert np.all(f(got, dt)[dropped] == 0.0)
    print(f"[gpu] {msg}; fully dropped tokens {int(dropped.sum())}")


def _oracle_layer(cfg, inp, ids, C, tokens, out_rows=None, wgu=None, wdn=None):
    """Oracle layer for `tokens`, routing on the given ids (weights from the oracle's logits). Returns
    (y, the oracle's expert-output rows of the tokens' kept slots, their pair -> row map, weights).

    Dispatch positions depend on every token, so dispatch runs on all ids. out_rows: the oracle's expert
    outputs of every send row, if already computed; else the MLP runs on the rows of `tokens` with the
    weights wgu / wdn (indexable by local expert)."""
    dt = dt_name(inp["x"])
    x = to_np(inp["x"])
    bias = _bias_np(inp)
    sub_bias = None if bias is None else (bias if bias.ndim == 1 else bias[tokens])
    lg = oracle.router_logits(x[tokens], dt, to_np(inp["w_router"]), sub_bias)
    w = oracle.routing_weights(lg, ids[tokens])
    lay, sb = oracle.dispatch(x, dt, ids, cfg.E, C, cfg.R)
    pr = lay.pair_row[tokens]
    used = np.unique(pr[pr >= 0])
    if out_rows is not None:
        rows = out_rows[used]
    else:
        rex = oracle.row_experts(lay.expert_offset, cfg.E)
        rows = oracle.expert_mlp(sb[used], dt, rex[used], cfg.El, wgu, wdn, cfg.F) if len(used) else sb[:0]
    remap = np.full(max(lay.total, 1), -1, dtype=np.int64)
    remap[used] = np.arange(len(used))
    pr_local = np.where(pr >= 0, remap[np.maximum(pr, 0)], -1)
    return oracle.combine(rows, dt, pr_local, w), rows, pr_local, w, (lay, sb)


@pytest.mark.parametrize("wl", WORKLOADS)
def test_p6_layer_end_to_end(wl):
    cfg, inp, out = _layer(wl)
    dt = dt_name(inp["x"])
    ids = to_np(out["ids"])
    total = int(to_np(out["layout"].expert_offset)[cfg.E])
    # the oracle's expert outputs of every send row, from the P4 chunks (computed here if P4 did not run).
    # They were computed on the GPU's send rows; the oracle's own dispatch below must give the same rows.
    store = np.empty((total, cfg.H), dtype=to_np(out["send_buf"][:1]).dtype)
    for c in range(CHUNKS[wl]):
        for l, (rows, ref) in _oracle_mlp_chunk(wl, c).items():
            store[rows] = ref
    tokens = np.arange(cfg.T)
    y_ref, rows, pr_local, w, (lay, sb) = _oracle_layer(cfg, inp, ids, inp["C"], tokens, out_rows=store)
    assert np.array_equal(sb, to_np(out["send_buf"][:total]))
    got = to_np(out["y"])
    f = oracle.to_f64
    bound = layer_bound(f(y_ref, dt), f(rows, dt), pr_local, w, dt)
    msg = check_close(f(got, dt), f(y_ref, dt), dt, f"{wl} layer", TOL[dt], bound=bound)
    dropped = (pr_local < 0).all(axis=1)
    assert np.all(f(got, dt)[dropped] == 0.0)
    print(f"[gpu] {msg}")


def test_determinism_bitwise():
    cfg, inp, out = _layer("dsv3-prefill-ep8-share")
    again = run_layer(inp, cfg.k, cfg.R)
    for key in ("logits", "ids", "w", "send_buf", "out_buf", "y"):
        assert torch.equal(_bits(out[key]), _bits(again[key])), key


def test_release_full_size_buffers():
    _cache.clear()
    _oracle_rows.clear()
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
    # loaded-to-LDS grouped GEMM: 320-row whole-expert tiles (400 rows per expert; 3-stage K loops, so no
    # cross-tile prefetch), then 256-row ping-pong tiles (2200 rows per local expert); F = 192 and
    # H = 192 / 320 leave a ragged last column tile in both GEMMs
    ("dl128_ragged", 900, 192, 4, 2, 192, 1, 400, "bf16", "zipf"),
    # whole-expert tiles, two per workgroup (512 tiles per GEMM), even K-stage counts: the next tile's first
    # stage is prefetched during the current one
    ("xs_two_tiles_per_wg", 4096, 1024, 128, 8, 512, 1, 300, "bf16", "uniform"),
    # 128-row direct-to-LDS tiles (capacity 200 rows per expert), ragged
    ("dl128_cap200", 700, 128, 8, 2, 128, 2, 200, "bf16", "zipf"),
    ("dl256_ragged_R2", 2600, 320, 4, 2, 192, 2, 1100, "bf16", "zipf"),
    # 64-row weight-streaming tiles (capacity 75 rows per expert on average), hot experts over 64 rows
    ("dec64_multi_mtile", 300, 128, 8, 2, 96, 1, 100, "bf16", "zipf"),
    # one counting block (T <= 256) scans all 512 experts itself
    ("E512_one_block", 200, 64, 512, 8, 32, 8, 4, "bf16", "zipf"),
    # whole-expert gate/up GEMM with a K-split last round: about 288 M tiles x 10 N tiles (F 1280) leave 1-16 tail
    # tiles per XCD range of 256 workgroups, each cut into two K halves (4 stages -> 2 + 2) that meet through the
    # split counters; the hot-8 routing drops about 61K pairs, so h has rows free past the kept rows for the fp32
    # partials (64 split tiles with this seed)
    ("xs_split_tail_hot8", 16384, 256, 256, 8, 1280, 1, 512, "bf16", "hot8"),
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
    """Every stage of a small layer against the whole oracle: logits (P1), top-k ids on the GPU logits,
    every layout array and send row bit-exact, expert MLP, combine and the layer within the activation
    type's row and element bounds."""
    if T == 0:
        L = out["layout"]
        assert np.all(to_np(L.expert_count) == 0) and np.all(to_np(L.expert_offset) == 0)
        return
    dt = dt_name(inp["x"])
    f = oracle.to_f64
    ids = to_np(out["ids"])
    got_lg = to_np(out["logits"])
    p1_check(got_lg, oracle.router_logits(to_np(inp["x"]), dt, to_np(inp["w_router"]), _bias_np(inp)))
    assert np.array_equal(ids, oracle.topk_select(got_lg, k))
    w_ref = oracle.routing_weights(got_lg, ids)
    assert np.all(np.abs(to_np(out["w"]).astype(np.float64) - w_ref) <= 1e-5 * np.abs(w_ref.astype(np.float64)) + 1e-30)
    lay, sb = oracle.dispatch(to_np(inp["x"]), dt, ids, E, C, R)
    L = out["layout"]
    for nm in ("expert_count", "expert_kept", "expert_overflow", "expert_offset", "pair_row"):
        assert np.array_equal(to_np(getattr(L, nm)), getattr(lay, nm)), nm
    n = lay.total
    assert np.array_equal(to_np(L.row_token)[:n], lay.row_token)
    assert np.array_equal(to_np(L.row_slot)[:n], lay.row_slot)
    assert np.array_equal(to_np(out["send_buf"][:n]), sb)
    rex = oracle.row_experts(lay.expert_offset, E)
    wgu, wdn = to_np(inp["w_gate_up"]), to_np(inp["w_down"])
    if n:
        ref_ob = oracle.expert_mlp(to_np(out["send_buf"][:n]), dt, rex, E // R, wgu, wdn, F)
        check_close(f(to_np(out["out_buf"][:n]), dt), f(ref_ob, dt), dt, "MLP", TOL[dt])
    ob = to_np(out["out_buf"][:n])
    ref_y = oracle.combine(ob, dt, lay.pair_row, to_np(out["w"]))
    y = f(to_np(out["y"]), dt)
    ratio = sum_bound_ratio(y, f(ref_y, dt), combine_abs_sum(f(ob, dt), lay.pair_row, to_np(out["w"])), k, dt)
    check_close(y, f(ref_y, dt), dt, "combine", TOL[dt], ratio=ratio)
    dropped = (lay.pair_row < 0).all(axis=1)
    assert np.all(y[dropped] == 0.0)
    full, rows, pr_local, w, _ = _oracle_layer(cfg, inp, ids, C, np.arange(T), wgu=wgu, wdn=wdn)
    check_close(y, f(full, dt), dt, "layer", TOL[dt], bound=layer_bound(f(full, dt), f(rows, dt), pr_local, w, dt))
