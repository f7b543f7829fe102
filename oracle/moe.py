"""Plain, slow CPU oracle of one GPU's share of an expert-parallel MoE layer.

TEST INFRASTRUCTURE ONLY. This module is the reference the HIP path is checked against; only the
tests, the smoke check and the benchmark's CPU-baseline leg may import it. It shares no code with the
HIP path and imports nothing from it.

Arithmetic is float64 unless a step states a rounding. Activations and expert weights are carried in
their storage form: float32 arrays for "f32", uint16 bfloat16 bit patterns for "bf16".

The layer (sources are cited by page title and section):
  route    -- a small linear router gives a score per expert; the k best experts are chosen and their
              weights come from the router's probability distribution ("Efficient and portable
              mixture-of-experts communication", section "Introductie"; "Enabling trillion-parameter
              models on AWS EFA", section "Введение").
  dispatch -- count tokens per expert, take the cumulative sum of the counts to get offsets, pack the
              tokens into contiguous per-destination buffers ("Enabling trillion-parameter models on
              AWS EFA", section "Диспетчеризация и комбинирование"; "Efficient and portable ...",
              section "Dispatch"), with a per-expert capacity, overflow = max(assigned - capacity, 0)
              and effective tokens = sum(assigned - overflow) ("80. MoE Expert Parallel Benchmark",
              Step 2).
  experts  -- each expert is a small MLP applied to the rows routed to it ("DistributedMoE",
              section "Основные компоненты"; "Enabling trillion-parameter models on AWS EFA", section
              "MoE all-to-all через EFA"), here the SwiGLU form.
  combine  -- the output of a token is the router-weighted sum of its experts' outputs, written into
              caller-owned tensors ("Efficient and portable ...", sections "Introductie" and "Combine").

Readings taken where the pages are silent (each is listed in the design notes):
  * top-k is taken on the fp32 logits, descending, ties to the lower expert id, -0 == +0;
  * the k weights are the softmax over the k selected logits (they sum to 1);
  * capacity C is an integer input; pairs are admitted first come first served in row-major
    (token, slot) order; a dropped pair contributes nothing and the kept weights are not renormalised;
  * rows are laid out in expert-id order, each expert's rows in token order, with no padding; with R
    destination ranks and El = E / R experts per rank, rank r owns experts [r*El, (r+1)*El);
  * a row routed to expert e is multiplied by local expert weights W[e mod El] (one GPU plays one rank
    and its R incoming segments are the R rank segments of its own send buffer);
  * the gate and up projections g = x Wg^T and u = x Wu^T are float32 values (the precision of
    the matrix units' accumulators); h = silu(g) * u is stored in the activation type;
  * a NaN router score ranks as -inf in the top-k selection.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

from .numerics import from_f64, round_to_f32, to_f64

__all__ = ["router_logits", "topk_select", "routing_weights", "topk_softmax", "Layout", "dispatch",
           "expert_mlp", "combine", "moe_layer", "row_experts", "silu"]


# --------------------------------------------------------------------------------------------------
# route
# --------------------------------------------------------------------------------------------------

def router_logits(x, dt: str, w_router, bias=None) -> np.ndarray:
    """logits[t, e] = sum_h x[t, h] * W_r[e, h] + bias, in float64, rounded once to float32.

    The router is "a small linear layer" producing one score per expert ("Efficient and portable
    mixture-of-experts communication", section "Introductie"). x: [T, H] in storage form dt;
    w_router: [E, H] float32; bias: None, [E] or [T, E] float32. Returns [T, E] float32.
    """
    x64 = to_f64(x, dt)
    w64 = np.asarray(w_router, dtype=np.float32).astype(np.float64)
    acc = x64 @ w64.T
    if bias is not None:
        acc = acc + np.asarray(bias, dtype=np.float32).astype(np.float64)
    return round_to_f32(acc)


def topk_select(logits, k: int) -> np.ndarray:
    """The k experts with the largest logits per token; slot 0 holds the best.

    Top-K selection over the router's scores ("Efficient and portable mixture-of-experts
    communication", section "Introductie"). Order: descending logit; equal logits are ordered by the
    lower expert id; -0 and +0 compare equal. The pages do not say how a NaN score ranks; here it ranks
    as -inf (so it is chosen only when fewer than k scores are larger than -inf, and then by expert id
    like every other tie). Written as a stable sort of the negated values, so equal keys keep index
    order. Returns ids [T, k] int32.
    """
    lg = np.asarray(logits, dtype=np.float32).astype(np.float64)
    lg = np.where(np.isnan(lg), -np.inf, lg)
    order = np.argsort(-lg, axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def routing_weights(logits, ids) -> np.ndarray:
    """Weights of the selected experts: the router's distribution restricted to the k selected
    experts and renormalised, w_j = exp(l_j - m) / sum_i exp(l_i - m) with m the largest selected
    logit, in float64, rounded to float32 ("Efficient and portable mixture-of-experts communication",
    section "Introductie": the weights derive from the router's probability distribution)."""
    lg = np.asarray(logits, dtype=np.float32)
    sel = np.take_along_axis(lg, np.asarray(ids, dtype=np.int64), axis=1).astype(np.float64)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    return round_to_f32(z / z.sum(axis=1, keepdims=True))


def topk_softmax(logits, k: int) -> tuple[np.ndarray, np.ndarray]:
    """(ids [T, k] int32, weights [T, k] float32): top-k selection, then its routing weights."""
    ids = topk_select(logits, k)
    return ids, routing_weights(logits, ids)


# --------------------------------------------------------------------------------------------------
# dispatch
# --------------------------------------------------------------------------------------------------

@dataclasses.dataclass
class Layout:
    """Where every (token, slot) pair went.

    expert_count[e]    tokens routed to expert e (the router histogram)
    expert_kept[e]     min(count, C)
    expert_overflow[e] max(count - C, 0)
    expert_offset[E+1] exclusive cumulative sum of kept; [E] = total rows. Rank r's segment is rows
                       [expert_offset[r*El], expert_offset[(r+1)*El]).
    row_token[rows]    source token of each row; row_slot[rows] its k-slot
    pair_row[T, k]     row of each pair, -1 if dropped
    """
    T: int
    k: int
    E: int
    R: int
    C: int
    expert_count: np.ndarray
    expert_kept: np.ndarray
    expert_overflow: np.ndarray
    expert_offset: np.ndarray
    row_token: np.ndarray
    row_slot: np.ndarray
    pair_row: np.ndarray

    @property
    def El(self) -> int:
        return self.E // self.R

    @property
    def total(self) -> int:
        return int(self.expert_offset[self.E])

    @property
    def effective(self) -> int:
        """Effective tokens: sum over experts of (assigned - overflow) ("80. MoE Expert Parallel
        Benchmark", Step 2)."""
        return int((self.expert_count - self.expert_overflow).sum())


def dispatch(x, dt: str, ids, E: int, C: int, R: int = 1):
    """Partition (token, slot) pairs by expert into contiguous, rank-aligned per-expert rows.

    Follows the send side of "Enabling trillion-parameter models on AWS EFA", section
    "Диспетчеризация и комбинирование": count tokens per expert, turn the counts into offsets by a
    cumulative sum, then pack each token into its expert's contiguous region. Capacity and overflow
    follow "80. MoE Expert Parallel Benchmark", Step 2. Pairs are visited in row-major (t, j) order,
    so each expert's rows are in token order and the first C pairs routed to an expert are kept.

    x: [T, H] storage form dt; ids: [T, k] int. Returns (Layout, send_buf [total, H] in storage form).
    """
    ids = np.asarray(ids)
    T, k = ids.shape
    if E % R != 0:
        raise ValueError("E must be a multiple of R")
    count = np.zeros(E, dtype=np.int64)
    pos = np.zeros((T, k), dtype=np.int64)
    for t in range(T):                    # counting pass in row-major pair order
        for j in range(k):
            e = int(ids[t, j])
            pos[t, j] = count[e]
            count[e] += 1
    kept = np.minimum(count, C)
    overflow = np.maximum(count - C, 0)
    offset = np.zeros(E + 1, dtype=np.int64)
    offset[1:] = np.cumsum(kept)
    total = int(offset[E])
    row_token = np.empty(total, dtype=np.int64)
    row_slot = np.empty(total, dtype=np.int64)
    pair_row = np.full((T, k), -1, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            if pos[t, j] < C:
                r = offset[ids[t, j]] + pos[t, j]
                pair_row[t, j] = r
                row_token[r] = t
                row_slot[r] = j
    xs = np.asarray(x)
    send_buf = xs[row_token] if total else xs[:0]
    lay = Layout(T=T, k=k, E=E, R=R, C=C,
                 expert_count=count.astype(np.int32), expert_kept=kept.astype(np.int32),
                 expert_overflow=overflow.astype(np.int32), expert_offset=offset.astype(np.int32),
                 row_token=row_token.astype(np.int32), row_slot=row_slot.astype(np.int32),
                 pair_row=pair_row.astype(np.int32))
    return lay, send_buf


def row_experts(expert_offset, E: int) -> np.ndarray:
    """Global expert id of every row, read off the offsets (row r belongs to e with
    offset[e] <= r < offset[e+1])."""
    off = np.asarray(expert_offset, dtype=np.int64)
    counts = off[1:E + 1] - off[:E]
    return np.repeat(np.arange(E, dtype=np.int64), counts)


# --------------------------------------------------------------------------------------------------
# expert MLP
# --------------------------------------------------------------------------------------------------

def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z * sigmoid(z) = z / (1 + exp(-z))."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_mlp(rows, dt: str, row_expert, El: int, w_gate_up, w_down, F: int) -> np.ndarray:
    """SwiGLU expert MLP on dispatched rows.

    Each row routed to global expert e uses local expert l = e mod El:
        g = x Wg[l]^T,  u = x Wu[l]^T       (Wg = w_gate_up[l][:F], Wu = w_gate_up[l][F:]),
                                             each summed exactly (float64) and rounded to float32
        h = silu(g) * u, rounded to the activation type
        out = h Wd[l]^T, rounded to the activation type
    The expert is a small MLP run on the tokens dispatched to it ("DistributedMoE", section
    "Основные компоненты": the expert block runs the expert MLP on the activations it receives);
    the gated form is SwiGLU (Shazeer, "GLU Variants Improve Transformer", 2020).

    rows: [n, H] storage form; row_expert: [n] global expert ids; w_gate_up: indexable by l giving
    [2F, H]; w_down: indexable by l giving [H, F] (storage form dt). Returns [n, H] storage form dt.
    """
    rows = np.asarray(rows)
    row_expert = np.asarray(row_expert, dtype=np.int64)
    n = rows.shape[0]
    H = rows.shape[1] if rows.ndim == 2 else 0
    out = np.zeros((n, H), dtype=np.float64)
    local = row_expert % El
    for l in np.unique(local):
        sel = np.nonzero(local == l)[0]
        xa = to_f64(rows[sel], dt)
        wgu = to_f64(np.asarray(w_gate_up[int(l)]), dt)
        wd = to_f64(np.asarray(w_down[int(l)]), dt)
        # the gate and up projections are formed as float32 values (one rounding of each exact sum),
        # then h = silu(g) * u is evaluated on them in float64 and rounded to the activation type
        g = round_to_f32(xa @ wgu[:F].T).astype(np.float64)
        u = round_to_f32(xa @ wgu[F:2 * F].T).astype(np.float64)
        h = to_f64(from_f64(silu(g) * u, dt), dt)
        out[sel] = h @ wd.T
    return from_f64(out, dt)


# --------------------------------------------------------------------------------------------------
# combine
# --------------------------------------------------------------------------------------------------

def combine(out_buf, dt: str, pair_row, topk_w) -> np.ndarray:
    """y[t] = sum over kept slots j (ascending) of w[t, j] * out_buf[pair_row[t, j]], rounded once.

    The weighted sum of the expert outputs of each token, using the routing table to choose the rows
    and the weights ("Efficient and portable mixture-of-experts communication", section "Combine").
    A token whose pairs were all dropped gets y = 0.
    out_buf: [rows, H] storage form dt; pair_row: [T, k]; topk_w: [T, k] float32.
    Returns y [T, H] storage form dt.
    """
    pr = np.asarray(pair_row, dtype=np.int64)
    w = np.asarray(topk_w, dtype=np.float32).astype(np.float64)
    T, k = pr.shape
    ob = np.asarray(out_buf)
    H = ob.shape[1]
    y = np.zeros((T, H), dtype=np.float64)
    for j in range(k):
        m = pr[:, j] >= 0
        if m.any():
            y[m] += w[m, j:j + 1] * to_f64(ob[pr[m, j]], dt)
    return from_f64(y, dt)


# --------------------------------------------------------------------------------------------------
# whole layer
# --------------------------------------------------------------------------------------------------

def moe_layer(x, dt: str, w_router, bias, k: int, C: int, R: int, w_gate_up, w_down, F: int,
              ids: Optional[np.ndarray] = None) -> dict:
    """route -> dispatch -> expert MLP -> combine, all on the CPU.

    If `ids` is given (the selection another implementation made on its own fp32 logits), routing
    follows those ids and their weights are recomputed from this oracle's logits.
    """
    logits = router_logits(x, dt, w_router, bias)
    if ids is None:
        ids = topk_select(logits, k)
    ids = np.asarray(ids, dtype=np.int32)
    w = routing_weights(logits, ids)
    E = np.asarray(w_router).shape[0]
    lay, send_buf = dispatch(x, dt, ids, E, C, R)
    rex = row_experts(lay.expert_offset, E)
    out_buf = expert_mlp(send_buf, dt, rex, E // R, w_gate_up, w_down, F)
    y = combine(out_buf, dt, lay.pair_row, w)
    return dict(logits=logits, ids=ids, weights=w, layout=lay, send_buf=send_buf, out_buf=out_buf,
                y=y)
