"""Pins for the oracle's dispatch (histogram -> cumulative sum -> pack, with capacity and overflow).

Definitions: "80. MoE Expert Parallel Benchmark", Step 2 (assigned, capacity, overflow =
max(assigned - capacity, 0), effective = sum(assigned - overflow)); "Enabling trillion-parameter models
on AWS EFA", section "Диспетчеризация и комбинирование" (count per expert, cumulative sum to offsets,
pack into contiguous per-peer buffers); "Efficient and portable mixture-of-experts communication",
section "Dispatch" (the receiver keeps source rank, expert and token index per row).
"""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import dispatch, row_experts

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "dispatch_worked_example.json")


def _brute_dispatch(ids, E, C):
    """Independent formulation: for every expert, filter the tokens routed to it in token order; the
    first C are kept; experts are laid out one after another in id order."""
    T, k = len(ids), len(ids[0])
    rows = []                     # (token, slot)
    pair_row = [[-1] * k for _ in range(T)]
    for e in range(E):
        routed = [(t, ids[t].index(e)) for t in range(T) if e in ids[t]]
        for (t, j) in routed[:C]:
            pair_row[t][j] = len(rows)
            rows.append((t, j))
    counts = [sum(1 for t in range(T) if e in ids[t]) for e in range(E)]
    return rows, pair_row, counts


def test_worked_example_golden():
    g = json.load(open(GOLDEN))
    x = np.arange(g["T"] * 4, dtype=np.float32).reshape(g["T"], 4)
    lay, sb = dispatch(x, "f32", np.array(g["ids"]), g["E"], g["C"], g["R"])
    assert lay.expert_count.tolist() == g["expert_count"]
    assert lay.expert_kept.tolist() == g["expert_kept"]
    assert lay.expert_overflow.tolist() == g["expert_overflow"]
    assert lay.effective == g["effective_tokens"]
    assert lay.expert_offset.tolist() == g["expert_offset"]
    assert lay.row_token.tolist() == g["row_token"]
    assert lay.row_slot.tolist() == g["row_slot"]
    assert lay.pair_row.tolist() == g["pair_row"]
    assert np.array_equal(sb, x[g["row_token"]])
    dropped = [t for t in range(g["T"]) if all(r < 0 for r in lay.pair_row[t])]
    assert dropped == g["fully_dropped_tokens"]


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (2, 2, 1), (2, 3, 2), (3, 2, 2), (3, 4, 1), (3, 4, 2)])
def test_brute_force_every_assignment(T, E, k):
    per_token = list(itertools.permutations(range(E), k))
    x = (np.arange(T * 2, dtype=np.float32) + 1).reshape(T, 2)
    for assignment in itertools.product(per_token, repeat=T):
        ids = [list(a) for a in assignment]
        for R in [r for r in (1, 2, 4) if E % r == 0]:
            for C in range(0, T + 1):
                lay, sb = dispatch(x, "f32", np.array(ids, dtype=np.int32), E, C, R)
                rows, pair_row, counts = _brute_dispatch(ids, E, C)
                assert lay.expert_count.tolist() == counts
                assert lay.pair_row.tolist() == pair_row
                assert lay.row_token.tolist() == [t for t, _ in rows]
                assert lay.row_slot.tolist() == [j for _, j in rows]
                assert np.array_equal(sb, x[[t for t, _ in rows]].reshape(len(rows), 2))


def _random_ids(rng, T, E, k, p=None):
    ids = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        ids[t] = rng.choice(E, size=k, replace=False, p=p)
    return ids


@pytest.mark.parametrize("T,E,k,C,R,skew", [
    (300, 16, 4, 60, 1, False), (300, 16, 4, 20, 4, True), (128, 384, 8, 4, 8, True),
    (257, 8, 2, 80, 1, False), (64, 8, 8, 64, 2, False), (100, 10, 1, 0, 5, False)])
def test_invariants(T, E, k, C, R, skew):
    rng = np.random.default_rng(T * 7 + E)
    p = None
    if skew:
        p = 1.0 / np.arange(1, E + 1) ** 1.2
        p /= p.sum()
    ids = _random_ids(rng, T, E, k, p)
    x = rng.standard_normal((T, 3)).astype(np.float32)
    lay, sb = dispatch(x, "f32", ids, E, C, R)
    count = lay.expert_count.astype(np.int64)
    # per-expert counts equal the router histogram
    assert np.array_equal(count, np.bincount(ids.ravel(), minlength=E))
    # overflow and effective tokens ("80. MoE Expert Parallel Benchmark", Step 2)
    assert np.array_equal(lay.expert_overflow, np.maximum(count - C, 0))
    assert np.array_equal(lay.expert_kept, count - lay.expert_overflow)
    assert lay.effective == int(lay.expert_kept.sum()) == lay.total
    assert lay.expert_offset[0] == 0 and np.all(np.diff(lay.expert_offset) == lay.expert_kept)
    # rows of an expert: the first kept[e] tokens routed to e, strictly increasing
    rex = row_experts(lay.expert_offset, E)
    for e in range(E):
        seg = lay.row_token[lay.expert_offset[e]:lay.expert_offset[e + 1]]
        routed = np.nonzero((ids == e).any(axis=1))[0]
        assert np.array_equal(seg, routed[:lay.expert_kept[e]])
        assert np.all(np.diff(seg) > 0)
    # pair_row and (row_token, row_slot) are mutually inverse
    for r in range(lay.total):
        t, j = lay.row_token[r], lay.row_slot[r]
        assert lay.pair_row[t, j] == r and ids[t, j] == rex[r]
    kept_pairs = lay.pair_row[lay.pair_row >= 0]
    assert np.array_equal(np.sort(kept_pairs), np.arange(lay.total))
    # rank segments are contiguous: rank r owns rows of experts [r*El, (r+1)*El)
    El = E // R
    for r in range(R):
        lo, hi = lay.expert_offset[r * El], lay.expert_offset[(r + 1) * El]
        assert np.all((rex[lo:hi] // El) == r)
    assert np.array_equal(sb, x[lay.row_token])


def test_special_cases():
    rng = np.random.default_rng(9)
    ids = _random_ids(rng, 50, 6, 3)
    x = rng.standard_normal((50, 2)).astype(np.float32)
    lay0, sb0 = dispatch(x, "f32", ids, 6, 0)
    assert lay0.total == 0 and sb0.shape[0] == 0 and np.all(lay0.pair_row == -1)
    layT, _ = dispatch(x, "f32", ids, 6, 50)
    assert np.all(layT.expert_overflow == 0) and layT.total == 150
    # C >= T never drops: capacity above T changes nothing
    layB, _ = dispatch(x, "f32", ids, 6, 500)
    assert np.array_equal(layB.pair_row, layT.pair_row)
