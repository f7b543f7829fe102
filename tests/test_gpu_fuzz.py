"""GPU fuzz of the index-heavy stages through the C ABI, against the oracle, bit for bit.

* dispatch: about 200 seeded cases of given top-k ids (no routing): token counts at and around the 256-token
  counting-block edges, 1..512 experts, 1..8 slots, 1..8 ranks, capacity 0, 1, tight and >= T, and uniform,
  skewed and single-expert id patterns. Every layout array and every send row must equal the oracle's; bf16
  cases with H = 128 also run the fp8 dispatch (codes and scales bit-exact).
* top-k with exact ties: one-hot router rows make every logit exactly a chosen input value (from a small set
  including -0 and +0, optionally plus a per-expert bias), so most rows hold ties; the ids must equal the
  oracle's top-k of the GPU logits (descending, ties to the lower id, -0 == +0) on every router kernel (the
  fused small-E kernel, and the split-K GEMM with the lane-interleaved or the row-contiguous top-k kernel).
"""
import numpy as np
import pytest
import torch

import combine_router_gemm_amd as moe
import oracle
from oracle import fp8
from tests._hip_runner import to_np

pytestmark = pytest.mark.gpu


def _ids(rng, T, E, k, pattern):
    if T == 0:
        return np.zeros((0, k), np.int32)
    if pattern == "uniform":
        return np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    if pattern == "skew":  # expert popularity ~ 1 / (e + 1)
        p = 1.0 / np.arange(1, E + 1)
        p /= p.sum()
        return np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    # "same": every token picks experts 0..k-1 (in a random order)
    return np.stack([rng.permutation(k) for _ in range(T)]).astype(np.int32)


def _dispatch_cases():
    rng = np.random.default_rng(99)
    cases = []
    edges = [0, 1, 2, 255, 256, 257, 511, 512, 513, 1023, 1024, 1025, 4097]
    for i in range(200):
        E = int(rng.choice([1, 2, 3, 5, 8, 12, 16, 33, 64, 128, 256, 384, 512]))
        k = int(rng.integers(1, min(8, E) + 1))
        R = int(rng.choice([d for d in range(1, 9) if E % d == 0]))
        T = int(rng.choice(edges)) if i % 3 == 0 else int(rng.integers(0, 3000))
        cmode = rng.integers(0, 4)
        C = [0, 1, max(1, (T * k) // max(E, 1) // 2), T + 1][cmode]
        H = int(rng.choice([8, 16, 128]))
        dt = "bf16" if rng.random() < 0.7 else "f32"
        pattern = str(rng.choice(["uniform", "skew", "same"]))
        cases.append((i, T, H, E, k, R, C, dt, pattern))
    return cases


DISPATCH_CASES = _dispatch_cases()


def test_dispatch_fuzz():
    rng = np.random.default_rng(7)
    dev = torch.device("cuda:0")
    for (i, T, H, E, k, R, C, dt, pattern) in DISPATCH_CASES:
        print(f"[gpu] dispatch fuzz {i}: T={T} H={H} E={E} k={k} R={R} C={C} {dt} {pattern}", flush=True)
        ids = _ids(rng, T, E, k, pattern)
        tdt = torch.bfloat16 if dt == "bf16" else torch.float32
        x = torch.randn(T, H, generator=torch.Generator().manual_seed(i)).to(tdt).to(dev)
        L = moe.Layout(T, k, E, R, C, H, device=dev)
        send = torch.zeros(L.rows_max, H, dtype=tdt, device=dev)
        ids_d = torch.as_tensor(ids, device=dev)
        moe.moe_dispatch(x, ids_d, L, send)
        torch.cuda.synchronize()
        lay, sb = oracle.dispatch(to_np(x), dt, ids, E, C, R)
        for nm in ("expert_count", "expert_kept", "expert_overflow", "expert_offset", "pair_row"):
            assert np.array_equal(to_np(getattr(L, nm)), getattr(lay, nm)), (i, nm)
        n = lay.total
        assert np.array_equal(to_np(L.row_token)[:n], lay.row_token), i
        assert np.array_equal(to_np(L.row_slot)[:n], lay.row_slot), i
        assert np.array_equal(to_np(send[:n]), sb), i
        if dt == "bf16" and H == 128:
            q = torch.zeros(L.rows_max, H, dtype=torch.uint8, device=dev)
            sc = torch.zeros(L.rows_max, 1, dtype=torch.float32, device=dev)
            L8 = moe.Layout(T, k, E, R, C, H, device=dev)
            moe.moe_dispatch_fp8(x, ids_d, L8, q, sc)
            torch.cuda.synchronize()
            assert np.array_equal(to_np(L8.pair_row), lay.pair_row), i
            if n:
                codes, scales = fp8.quantize_rows(sb)
                assert np.array_equal(to_np(q[:n]), codes) and np.array_equal(to_np(sc[:n]), scales), i


TOPK_CASES = [
    # T, E, k, bias
    (300, 8, 2, None), (300, 16, 8, "vec"), (257, 12, 3, "rows"), (5000, 8, 4, None),   # fused small-E router
    (300, 64, 8, None), (700, 256, 8, "vec"), (129, 512, 8, "rows"), (2000, 40, 5, None),  # split-K router
]


# E a multiple of 64 takes the row-contiguous top-k kernel: 2 to 8 values per lane (float4, float2 and single
# loads), one split (the partial sums are the logits buffer) or several (extra zero-weight columns of x), few
# tokens (all splits loaded at once) or many (four at a time), and a logits buffer only 4-byte aligned
TOPK_ROWS_CASES = [
    # T, E, k, bias, H, logits offset (floats)
    (300, 128, 8, None, 128, 0), (1100, 192, 6, "vec", 2048, 0), (200, 320, 8, "rows", 4096, 0),
    (700, 384, 8, None, 7168, 0), (50, 448, 7, "vec", 448, 1), (129, 512, 8, "rows", 1024, 1),
    (1500, 256, 8, "rows", 256, 1), (3, 384, 8, None, 384, 0),
    # 2048+ tokens with H % 64 == 0 take the plane GEMM: ragged token and expert tiles, one or several splits
    (2500, 256, 8, "rows", 256, 0), (4100, 384, 8, None, 7168, 1), (2300, 448, 7, "vec", 1024, 0),
]


@pytest.mark.parametrize("T,E,k,bias", TOPK_CASES, ids=[f"T{c[0]}_E{c[1]}_k{c[2]}_{c[3]}" for c in TOPK_CASES])
def test_topk_exact_ties(T, E, k, bias):
    _check_topk_ties(T, E, k, bias, ((E + 7) // 8) * 8, 0)


@pytest.mark.parametrize("T,E,k,bias,H,off", TOPK_ROWS_CASES,
                         ids=[f"T{c[0]}_E{c[1]}_k{c[2]}_{c[3]}_H{c[4]}_off{c[5]}" for c in TOPK_ROWS_CASES])
def test_topk_exact_ties_row_kernel(T, E, k, bias, H, off):
    _check_topk_ties(T, E, k, bias, H, off)


def _check_topk_ties(T, E, k, bias, H, off):
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(T * 1000 + E)
    vals = np.array([-2.0, -1.0, -0.0, 0.0, 0.5, 1.0, 2.0], dtype=np.float32)
    xv = rng.choice(vals, size=(T, H)).astype(np.float32)
    x = torch.as_tensor(xv).to(torch.bfloat16).to(dev)        # every value is exact in bf16
    w = torch.zeros(E, H, dtype=torch.float32)
    w[torch.arange(E), torch.arange(E)] = 1.0                  # logit e = x[:, e] (+ bias)
    w = w.to(dev)
    b = None
    if bias == "vec":
        b = torch.as_tensor(rng.choice([0.0, 1.0, -1.0], size=E).astype(np.float32), device=dev)
    elif bias == "rows":
        b = torch.as_tensor(rng.choice([0.0, 0.5], size=(T, E)).astype(np.float32), device=dev)
    logits = torch.empty(T * E + off, dtype=torch.float32, device=dev)[off:].view(T, E)
    ids = torch.empty(T, k, dtype=torch.int32, device=dev)
    wts = torch.empty(T, k, dtype=torch.float32, device=dev)
    moe.moe_route(x, w, b, k, logits, ids, wts)
    torch.cuda.synchronize()
    lg = to_np(logits)
    expect = xv[:, :E] + (0.0 if b is None else to_np(b))
    assert np.array_equal(lg, expect.astype(np.float32))      # -0 and +0 compare equal
    got = to_np(ids)
    assert np.array_equal(got, oracle.topk_select(lg, k))
    ref_w = oracle.routing_weights(lg, got)
    assert np.all(np.abs(to_np(wts).astype(np.float64) - ref_w) <= 1e-6 * np.abs(ref_w) + 1e-30)
    ties = int((np.sort(lg, axis=1)[:, ::-1][:, k - 1] == np.sort(lg, axis=1)[:, ::-1][:, k]).sum()) if k < E else 0
    print(f"[gpu] top-k ties T={T} E={E} k={k}: {ties} rows with a tie at the k-th place")


# non-finite logits: a [T, E] bias of 0, NaN, +inf or -inf on one-hot router rows. A NaN logit ranks as -inf
# and ties (also among infinities and NaN) go to the lower id, on every router kernel: fused small-E,
# split-K with the lane-interleaved top-k, split-K with the row-contiguous top-k, and the plane GEMM
NONFINITE_CASES = [(300, 8, 2), (257, 16, 8), (300, 40, 5), (129, 64, 8), (700, 256, 8), (50, 384, 8), (2200, 256, 8)]


@pytest.mark.parametrize("T,E,k", NONFINITE_CASES, ids=[f"T{c[0]}_E{c[1]}_k{c[2]}" for c in NONFINITE_CASES])
def test_topk_nonfinite_logits(T, E, k):
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(T * 7 + E)
    H = ((E + 7) // 8) * 8
    xv = rng.choice(np.array([-1.0, -0.0, 0.0, 1.0], dtype=np.float32), size=(T, H)).astype(np.float32)
    x = torch.as_tensor(xv).to(torch.bfloat16).to(dev)
    w = torch.zeros(E, H, dtype=torch.float32)
    w[torch.arange(E), torch.arange(E)] = 1.0
    w = w.to(dev)
    special = np.array([np.nan, np.inf, -np.inf], dtype=np.float32)
    bv = np.where(rng.random((T, E)) < 0.3, rng.choice(special, size=(T, E)), 0.0).astype(np.float32)
    bv[: T // 8] = np.nan                                   # rows with every logit NaN
    bv[T // 8: T // 4] = np.where(rng.random((T // 4 - T // 8, E)) < 0.8, -np.inf, np.nan)
    b = torch.as_tensor(bv, device=dev)
    logits = torch.empty(T, E, dtype=torch.float32, device=dev)
    ids = torch.empty(T, k, dtype=torch.int32, device=dev)
    wts = torch.empty(T, k, dtype=torch.float32, device=dev)
    moe.moe_route(x, w, b, k, logits, ids, wts)
    torch.cuda.synchronize()
    lg = to_np(logits)
    expect = xv[:, :E] + bv
    assert np.array_equal(lg, expect, equal_nan=True)
    got = to_np(ids)
    assert np.array_equal(got, oracle.topk_select(lg, k))
    # the weights are specified where every selected logit is finite
    sel = np.take_along_axis(lg, got.astype(np.int64), axis=1)
    fin = np.isfinite(sel).all(axis=1)
    ref_w = oracle.routing_weights(lg[fin], got[fin])
    assert np.all(np.abs(to_np(wts)[fin].astype(np.float64) - ref_w) <= 1e-6 * np.abs(ref_w) + 1e-30)
    print(f"[gpu] non-finite top-k T={T} E={E} k={k}: {int((~fin).sum())} rows select a non-finite logit")
