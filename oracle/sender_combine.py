"""Combine with sender-side partial accumulation: the expert side sums, per token and per destination
rank, the weighted rows it holds, and the token's own side sums those partial rows.

TEST INFRASTRUCTURE ONLY: this module is part of the CPU oracle the HIP path is checked against. Only
the tests, the smoke check and the benchmark's CPU-baseline leg may import it.

"Enabling trillion-parameter models on AWS EFA", section "Оценка" (the dispatch/combine latency part):
the pages' combine accumulates only at the receiver, one row per kept (token, expert) pair crossing the
link; DeepEP accumulates at the sender, which moves fewer bytes at a possible cost in precision. The
readings taken here (the page gives no more detail):

* Rank of a row: the row lies in rank r's segment of the dispatch layout, expert_offset[r * El] <= row
  < expert_offset[(r + 1) * El] (El = E / R experts per rank).
* Send side: for every token t and every rank r holding at least one kept pair of t,
      partial[r, t] = sum over kept slots j of t on rank r, ascending j, of w[t, j] * out_buf[pair_row[t, j]],
  accumulated exactly and rounded once to the activation type (the precision cost: one extra rounding
  per partial). Slots (r, t) with no kept pair are not written. The buffer is rank-major [R, T, H], so
  what rank r sends back to a source is one contiguous block.
* Receive side: y[t] = sum over present r, ascending, of partial[r, t], accumulated exactly and rounded
  once; a token with no kept pair gets 0.
* With R = 1 there is one partial per token, which is the receiver-side sum already rounded once, so
  the two combines agree bit for bit.
"""
from __future__ import annotations

import numpy as np

from .numerics import from_f64, to_f64


def row_ranks(rows, expert_offset, El: int, R: int) -> np.ndarray:
    """Rank of each row index (-1 for a negative index), from the rank segments of the layout."""
    off = np.asarray(expert_offset, dtype=np.int64)
    bounds = off[np.arange(R + 1) * El]              # rank r owns rows [bounds[r], bounds[r+1])
    rows = np.asarray(rows, dtype=np.int64)
    r = np.searchsorted(bounds, rows, side="right") - 1
    return np.where(rows >= 0, r, -1)


def combine_send(out_buf, dt: str, pair_row, topk_w, expert_offset, E: int, R: int):
    """Partial rows per (rank, token). Returns (partial [R, T, H] storage form dt, zero where absent;
    present [R, T] bool)."""
    pr = np.asarray(pair_row, dtype=np.int64)
    w = np.asarray(topk_w, dtype=np.float32).astype(np.float64)
    T, k = pr.shape
    ob = np.asarray(out_buf)
    H = ob.shape[1]
    El = E // R
    rk = row_ranks(pr, expert_offset, El, R)
    acc = np.zeros((R, T, H), dtype=np.float64)
    present = np.zeros((R, T), dtype=bool)
    for j in range(k):                               # ascending slots inside each (rank, token)
        m = pr[:, j] >= 0
        if not m.any():
            continue
        t = np.nonzero(m)[0]
        r = rk[t, j]
        acc[r, t] += w[t, j:j + 1] * to_f64(ob[pr[t, j]], dt)
        present[r, t] = True
    return from_f64(acc, dt), present


def combine_recv(partial, dt: str, present) -> np.ndarray:
    """y[t] = sum over present ranks r (ascending) of partial[r, t], rounded once."""
    p = to_f64(np.asarray(partial), dt)
    pres = np.asarray(present, dtype=bool)
    y = np.zeros(p.shape[1:], dtype=np.float64)
    for r in range(p.shape[0]):
        y[pres[r]] += p[r][pres[r]]
    return from_f64(y, dt)


def combine_sender_side(out_buf, dt: str, pair_row, topk_w, expert_offset, E: int, R: int) -> dict:
    """Both halves; also the rows that cross the link each way of the exchange (one per present
    (rank, token) here, one per kept pair with the receiver-side combine)."""
    partial, present = combine_send(out_buf, dt, pair_row, topk_w, expert_offset, E, R)
    y = combine_recv(partial, dt, present)
    return dict(partial=partial, present=present, y=y, partial_rows=int(present.sum()),
                kept_rows=int((np.asarray(pair_row) >= 0).sum()))
