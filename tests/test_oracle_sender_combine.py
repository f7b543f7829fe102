"""Pins for the oracle's combine with sender-side partial accumulation (oracle/sender_combine.py).

Checked against: the receiver-side combine (R = 1 must agree bit for bit; exact inputs must agree for
any R), a brute force over tokens, slots and ranks that takes each pair's rank from its expert id
(ids // El) rather than from the layout offsets, and the rounding bound of one extra bf16 rounding
per partial row.
"""
import numpy as np
import pytest

from oracle.moe import combine, dispatch
from oracle.numerics import bf16_bits_to_f64, f64_to_bf16_bits, from_f64, to_f64
from oracle.sender_combine import combine_recv, combine_send, combine_sender_side, row_ranks


def _routing(seed, T, E, k, C, R, H, dt="bf16", exact=False):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    x = f64_to_bf16_bits(rng.standard_normal((T, H))) if dt == "bf16" else rng.standard_normal((T, H)).astype(np.float32)
    lay, _ = dispatch(x, dt, ids, E, C, R)
    n = lay.total
    if exact:
        # small integers and dyadic weights: every partial and total is exact in bf16 and fp32
        vals = rng.integers(-3, 4, size=(n, H)).astype(np.float64)
        w = rng.choice([0.25, 0.5, 1.0], size=(T, k)).astype(np.float32)
    else:
        vals = rng.standard_normal((n, H))
        w = rng.uniform(0.05, 1.0, size=(T, k)).astype(np.float32)
    out_buf = from_f64(vals, dt)
    return ids, lay, out_buf, w


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_one_rank_equals_receiver_side_combine_bit_for_bit(dt):
    ids, lay, ob, w = _routing(1, T=90, E=8, k=3, C=20, R=1, H=40, dt=dt)
    assert lay.total < 90 * 3                      # some pairs dropped
    res = combine_sender_side(ob, dt, lay.pair_row, w, lay.expert_offset, 8, 1)
    assert np.array_equal(res["y"], combine(ob, dt, lay.pair_row, w))
    assert res["partial_rows"] == int(((lay.pair_row >= 0).any(axis=1)).sum())


@pytest.mark.parametrize("R", [2, 4, 8])
def test_partials_and_presence_against_brute_force_over_expert_ids(R):
    E, k, T, H = 16, 4, 60, 24
    El = E // R
    ids, lay, ob, w = _routing(2 + R, T=T, E=E, k=k, C=12, R=R, H=H, exact=True)
    partial, present = combine_send(ob, "bf16", lay.pair_row, w, lay.expert_offset, E, R)
    ref_present = np.zeros((R, T), dtype=bool)
    for t in range(T):
        for r in range(R):
            acc = np.zeros(H)
            for j in range(k):
                if lay.pair_row[t, j] >= 0 and ids[t, j] // El == r:
                    ref_present[r, t] = True
                    acc += float(w[t, j]) * bf16_bits_to_f64(ob[lay.pair_row[t, j]])
            if ref_present[r, t]:
                assert np.array_equal(bf16_bits_to_f64(partial[r, t]), acc), (t, r)
            else:
                assert not np.any(bf16_bits_to_f64(partial[r, t]))
    assert np.array_equal(present, ref_present)
    # exact inputs: the sender-side total equals the receiver-side combine for any R
    y = combine_recv(partial, "bf16", present)
    assert np.array_equal(y, combine(ob, "bf16", lay.pair_row, w))


def test_row_ranks_follow_the_expert_ids_and_handle_empty_ranks():
    E, R, k, T = 12, 4, 2, 30
    ids = np.array([[e % 3, (e % 3) + 6] for e in range(T)], dtype=np.int32)   # ranks 1 and 3 stay empty
    x = f64_to_bf16_bits(np.ones((T, 8)))
    lay, _ = dispatch(x, "bf16", ids, E, 100, R)
    rk = row_ranks(lay.pair_row, lay.expert_offset, E // R, R)
    assert np.array_equal(rk, np.where(lay.pair_row >= 0, ids // (E // R), -1))
    assert np.array_equal(row_ranks([-1], lay.expert_offset, 3, 4), [-1])


def test_one_extra_rounding_per_partial_bounds_the_difference():
    E, R, k, T, H = 32, 8, 8, 64, 64
    ids, lay, ob, w = _routing(7, T=T, E=E, k=k, C=64, R=R, H=H)
    res = combine_sender_side(ob, "bf16", lay.pair_row, w, lay.expert_offset, E, R)
    y_recv = bf16_bits_to_f64(combine(ob, "bf16", lay.pair_row, w))
    y_send = bf16_bits_to_f64(res["y"])
    p = np.abs(bf16_bits_to_f64(res["partial"])).sum(axis=0)        # sum over ranks of |partial|
    u = 2.0 ** -8                                                   # bf16 unit roundoff
    # each partial carries at most u relative error; each side's final rounding adds at most u |y|
    bound = u * p + u * (np.abs(y_recv) + np.abs(y_send)) + 1e-30
    assert np.all(np.abs(y_send - y_recv) <= bound)
    assert np.any(y_send != y_recv)                                 # the extra rounding is visible
    assert res["partial_rows"] < res["kept_rows"]                   # fewer rows cross the link


def test_fully_dropped_tokens_give_zero_and_k1_sends_every_row():
    ids, lay, ob, w = _routing(9, T=50, E=8, k=1, C=3, R=4, H=16)
    res = combine_sender_side(ob, "bf16", lay.pair_row, w, lay.expert_offset, 8, 4)
    dropped = (lay.pair_row < 0).all(axis=1)
    assert dropped.any() and not np.any(bf16_bits_to_f64(res["y"][dropped]))
    assert res["partial_rows"] == res["kept_rows"]
    # with k = 1 the partial is already the weighted row: the receive side only rounds it again
    assert np.array_equal(res["y"], combine(ob, "bf16", lay.pair_row, w))
