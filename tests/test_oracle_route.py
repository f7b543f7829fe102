"""Pins for the oracle's router: logits, top-k selection and routing weights.

Router and top-K: "Efficient and portable mixture-of-experts communication", section "Introductie"
(a small linear layer scores the experts, the top-K are chosen, the output is a weighted average with
weights derived from the router's distribution).
"""
import itertools
import math

import numpy as np
import pytest

from oracle import router_logits, routing_weights, topk_select, topk_softmax
from oracle.numerics import f64_to_bf16_bits


def test_logits_one_hot_rows_read_the_router_weight_exactly():
    # x = e_h has a single nonzero product, so logits[:, e] = W_r[e, h] + bias exactly
    rng = np.random.default_rng(0)
    E, H = 5, 7
    w = rng.standard_normal((E, H)).astype(np.float32)
    bias = rng.standard_normal(E).astype(np.float32)
    x = np.eye(H, dtype=np.float32)
    lg = router_logits(x, "f32", w)
    assert np.array_equal(lg, w.T)
    lgb = router_logits(x, "f32", w, bias)
    assert np.array_equal(lgb, (w.T.astype(np.float64) + bias).astype(np.float32))


def test_logits_against_exact_sums_by_brute_force():
    # math.fsum gives the correctly rounded sum of the exact products (float32 * float32 products
    # are exact in float64); the oracle must agree to float32 rounding
    rng = np.random.default_rng(1)
    T, E, H = 3, 4, 33
    x = rng.standard_normal((T, H)).astype(np.float32)
    xb = f64_to_bf16_bits(x.astype(np.float64))
    w = (rng.standard_normal((E, H)) * 0.02).astype(np.float32)
    bias = np.arange(T * E, dtype=np.float32).reshape(T, E) * 0.25
    for dt, xs in (("f32", x), ("bf16", xb)):
        lg = router_logits(xs, dt, w, bias)
        xv = x if dt == "f32" else (xb.astype(np.uint32) << 16).view(np.float32)
        for t in range(T):
            for e in range(E):
                exact = math.fsum([float(xv[t, h]) * float(w[e, h]) for h in range(H)]
                                  + [float(bias[t, e])])
                assert lg[t, e] == np.float32(exact)


def test_bias_row_stride_forms_agree():
    rng = np.random.default_rng(2)
    T, E, H = 4, 6, 8
    x = rng.standard_normal((T, H)).astype(np.float32)
    w = rng.standard_normal((E, H)).astype(np.float32)
    b = rng.standard_normal(E).astype(np.float32)
    assert np.array_equal(router_logits(x, "f32", w, b),
                          router_logits(x, "f32", w, np.tile(b, (T, 1))))


def _brute_topk(row, k):
    """Independent definition: expert e takes slot r = #{e' : v[e'] > v[e] or (v[e'] == v[e] and
    e' < e)}; it is selected iff r < k."""
    E = len(row)
    slots = [None] * k
    for e in range(E):
        r = sum(1 for f in range(E) if row[f] > row[e] or (row[f] == row[e] and f < e))
        if r < k:
            slots[r] = e
    return slots


@pytest.mark.parametrize("E", [1, 2, 3, 4])
def test_topk_brute_force_over_every_tie_pattern(E):
    values = [-1.0, -0.0, 0.0, 1.0, 2.0]
    rows = np.array(list(itertools.product(values, repeat=E)), dtype=np.float32)
    for k in range(1, E + 1):
        ids = topk_select(rows, k)
        for i, row in enumerate(rows):
            assert list(ids[i]) == _brute_topk(list(row), k), (row, k)


def _brute_topk_nan_as_minus_inf(row, k):
    """The same definition with a NaN score replaced by -inf before any comparison."""
    return _brute_topk([float("-inf") if math.isnan(v) else v for v in row], k)


@pytest.mark.parametrize("E", [1, 2, 3])
def test_topk_brute_force_with_infinities_and_nan(E):
    # NaN ranks as -inf; infinities order like any other value; ties (also among -inf and NaN) go to
    # the lower expert id
    values = [float("-inf"), -1.0, -0.0, 0.0, 1.0, float("inf"), float("nan")]
    rows = np.array(list(itertools.product(values, repeat=E)), dtype=np.float32)
    for k in range(1, E + 1):
        ids = topk_select(rows, k)
        for i, row in enumerate(rows):
            assert list(ids[i]) == _brute_topk_nan_as_minus_inf(list(row), k), (row, k)


def test_topk_negative_zero_equals_positive_zero():
    lg = np.array([[-0.0, 0.0, -1.0], [0.0, -0.0, -1.0]], dtype=np.float32)
    ids = topk_select(lg, 2)
    assert ids.tolist() == [[0, 1], [0, 1]]


def test_weights_closed_forms():
    rng = np.random.default_rng(4)
    lg = rng.standard_normal((64, 16)).astype(np.float32)
    # k = 1: the single weight is exactly 1
    _, w1 = topk_softmax(lg, 1)
    assert np.all(w1 == 1.0)
    # k equal logits: every weight is exactly 1/k (k a power of two, so 1/k is exact)
    for k in (2, 4, 8):
        eq = np.zeros((3, 16), dtype=np.float32)
        eq[:, :k] = 3.5
        eq[:, k:] = -10.0
        ids, w = topk_softmax(eq, k)
        assert ids[:, :k].tolist() == [list(range(k))] * 3
        assert np.all(w == np.float32(1.0 / k))
    # ratios are exp of logit differences and the weights sum to 1
    ids, w = topk_softmax(lg, 4)
    for t in range(lg.shape[0]):
        sel = lg[t, ids[t]]
        assert abs(float(w[t].astype(np.float64).sum()) - 1.0) < 4e-7
        for a in range(4):
            assert math.isclose(float(w[t, a]) / float(w[t, 0]),
                                math.exp(float(sel[a]) - float(sel[0])), rel_tol=3e-7)


def test_weights_are_renormalised_over_the_selected_experts_only():
    # a softmax over all E experts (then selecting k) would not sum to 1
    lg = np.array([[2.0, 1.0, 0.5, 0.25]], dtype=np.float32)
    ids, w = topk_softmax(lg, 2)
    assert ids.tolist() == [[0, 1]]
    expect0 = 1.0 / (1.0 + math.exp(-1.0))
    assert w[0, 0] == np.float32(expect0)
    assert w[0, 1] == np.float32(1.0 - expect0) or abs(float(w[0, 1]) - (1 - expect0)) < 1e-7


def test_routing_weights_follow_given_ids():
    lg = np.array([[0.0, 1.0, 2.0]], dtype=np.float32)
    w = routing_weights(lg, np.array([[2, 0]]))
    assert abs(float(w[0, 0]) - 1.0 / (1.0 + math.exp(-2.0))) < 1e-7
