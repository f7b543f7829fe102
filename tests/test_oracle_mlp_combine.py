"""Pins for the oracle's expert SwiGLU MLP, combine, and the whole layer.

Combine is the router-weighted sum of each token's expert outputs ("Efficient and portable
mixture-of-experts communication", sections "Introductie" and "Combine"). The pins use special cases
with closed forms or a dense torch formulation that never goes through dispatch.
"""
import math

import numpy as np
import pytest
import torch

from oracle import combine, dispatch, expert_mlp, moe_layer, row_experts, topk_softmax
from oracle.numerics import bf16_bits_to_f64, f64_to_bf16_bits


def _dense_swiglu_torch(x, wgu, wd, F, act):
    """Dense SwiGLU FFN with torch CPU ops: silu(x Wg^T) * (x Wu^T), stored in the activation type,
    then times Wd^T."""
    x = torch.from_numpy(x).double()
    g = x @ torch.from_numpy(wgu[:F]).double().T
    u = x @ torch.from_numpy(wgu[F:]).double().T
    h = torch.nn.functional.silu(g) * u
    h = h.to(act).double()
    return (h @ torch.from_numpy(wd).double().T).to(act)


def test_single_expert_reduces_to_dense_swiglu():
    # E = 1, k = 1, C = T: every token goes once through the only expert
    rng = np.random.default_rng(0)
    T, H, F = 37, 24, 40
    x = rng.standard_normal((T, H)).astype(np.float32)
    wgu = (rng.standard_normal((2 * F, H)) * 0.2).astype(np.float32)
    wd = (rng.standard_normal((H, F)) * 0.2).astype(np.float32)
    lay, sb = dispatch(x, "f32", np.zeros((T, 1), dtype=np.int32), 1, T)
    out = expert_mlp(sb, "f32", row_experts(lay.expert_offset, 1), 1, [wgu], [wd], F)
    ref = _dense_swiglu_torch(x, wgu, wd, F, torch.float32).numpy()
    assert np.array_equal(out, ref) or np.max(np.abs(out - ref)) <= 2 * np.spacing(np.abs(ref)).max()


def test_scalar_closed_form_and_gate_up_order():
    # H = F = 1: out = wd * silu(x wg) * (x wu)
    x = np.array([[2.0]], dtype=np.float32)
    wgu = np.array([[1.0], [0.5]], dtype=np.float32)     # gate row first, then up row
    wd = np.array([[3.0]], dtype=np.float32)
    out = expert_mlp(x, "f32", [0], 1, [wgu], [wd], 1)
    expect = 3.0 * (2.0 / (1.0 + math.exp(-2.0))) * 1.0
    assert out[0, 0] == np.float32(expect)
    swapped = expert_mlp(x, "f32", [0], 1, [wgu[::-1].copy()], [wd], 1)
    expect_sw = 3.0 * (1.0 / (1.0 + math.exp(-1.0))) * 2.0
    assert swapped[0, 0] == np.float32(expect_sw) and swapped[0, 0] != out[0, 0]


def test_gate_is_rounded_to_float32_before_the_activation():
    # g = 1 + 2^-24 exactly (two products summed in float64); as a float32 value it is 1.0 (half-way,
    # ties to even), and silu(1.0) and silu(1 + 2^-24) round to different float32 values, so the output
    # shows which g the activation saw
    x = np.array([[1.0, 1.0]], dtype=np.float32)
    wgu = np.array([[1.0, 2.0 ** -24], [1.0, 0.0]], dtype=np.float32)   # gate row, then up row (u = 1)
    wd = np.array([[1.0, 0.0]], dtype=np.float32).T.copy()               # [H=2, F=1]: out = [h, 0]
    out = expert_mlp(x, "f32", [0], 1, [wgu], [wd], 1)
    h_f32_gate = np.float32(1.0 / (1.0 + math.exp(-1.0)))
    h_exact_gate = np.float32((1.0 + 2.0 ** -24) / (1.0 + math.exp(-(1.0 + 2.0 ** -24))))
    assert h_f32_gate != h_exact_gate
    assert out[0, 0] == h_f32_gate and out[0, 1] == 0.0


def test_zero_down_projection_gives_zero():
    rng = np.random.default_rng(1)
    x = f64_to_bf16_bits(rng.standard_normal((5, 16)))
    wgu = f64_to_bf16_bits(rng.standard_normal((2, 32, 16)) * 0.1)
    wd = np.zeros((2, 16, 16), dtype=np.uint16)
    out = expert_mlp(x, "bf16", [0, 1, 1, 0, 1], 2, wgu, wd, 16)
    assert np.all(bf16_bits_to_f64(out) == 0.0)


def test_row_uses_local_expert_e_mod_El():
    # R = 2 ranks of El = 2 experts: a row of global expert 3 uses local weights W[1]
    rng = np.random.default_rng(2)
    H, F = 8, 12
    rows = rng.standard_normal((4, H)).astype(np.float32)
    wgu = (rng.standard_normal((2, 2 * F, H)) * 0.3).astype(np.float32)
    wd = (rng.standard_normal((2, H, F)) * 0.3).astype(np.float32)
    out = expert_mlp(rows, "f32", [0, 1, 2, 3], 2, wgu, wd, F)
    for r, l in zip(range(4), [0, 1, 0, 1]):
        ref = _dense_swiglu_torch(rows[r:r + 1], wgu[l], wd[l], F, torch.float32).numpy()
        assert np.max(np.abs(out[r] - ref[0])) <= 2 * np.spacing(np.abs(ref)).max()


def test_bf16_mlp_close_to_dense_torch():
    rng = np.random.default_rng(3)
    T, H, F = 20, 32, 48
    x = f64_to_bf16_bits(rng.standard_normal((T, H)))
    wgu = f64_to_bf16_bits(rng.standard_normal((2 * F, H)) * 0.1)
    wd = f64_to_bf16_bits(rng.standard_normal((H, F)) * 0.1)
    out = bf16_bits_to_f64(expert_mlp(x, "bf16", np.zeros(T), 1, [wgu], [wd], F))
    ref = _dense_swiglu_torch(bf16_bits_to_f64(x), bf16_bits_to_f64(wgu), bf16_bits_to_f64(wd), F,
                              torch.bfloat16).double().numpy()
    # torch narrows float64 -> bfloat16 through float32 (two roundings): allow one bf16 ulp
    assert np.all(np.abs(out - ref) <= np.abs(ref) * 2.0 ** -7 + 1e-30)


def _layout_and_weights(rng, T, E, k, C, R=1):
    lg = rng.standard_normal((T, E)).astype(np.float32)
    ids, w = topk_softmax(lg, k)
    return ids, w


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_combine_identity_experts_reproduce_input(dt):
    # identity experts: out_buf = send_buf, so y = (sum of kept weights) * x; no drops -> y = x
    rng = np.random.default_rng(4)
    T, E, k, H = 64, 8, 2, 16
    xf = rng.standard_normal((T, H))
    x = f64_to_bf16_bits(xf) if dt == "bf16" else xf.astype(np.float32)
    ids, w = _layout_and_weights(rng, T, E, k, T)
    lay, sb = dispatch(x, dt, ids, E, T)
    y = combine(sb, dt, lay.pair_row, w)
    xv = bf16_bits_to_f64(x) if dt == "bf16" else x.astype(np.float64)
    yv = bf16_bits_to_f64(y) if dt == "bf16" else y.astype(np.float64)
    ulp = 2.0 ** -7 if dt == "bf16" else 2.0 ** -22
    assert np.all(np.abs(yv - xv) <= np.abs(xv) * ulp + 1e-30)
    # with a small capacity, y = (sum of kept weights) * x, and all-dropped tokens give exactly 0
    lay2, sb2 = dispatch(x, dt, ids, E, 3)
    y2 = combine(sb2, dt, lay2.pair_row, w)
    y2v = bf16_bits_to_f64(y2) if dt == "bf16" else y2.astype(np.float64)
    wk = np.where(lay2.pair_row >= 0, w.astype(np.float64), 0.0).sum(axis=1)
    assert np.all(np.abs(y2v - wk[:, None] * xv) <= np.abs(wk[:, None] * xv) * ulp + 1e-30)
    dropped = (lay2.pair_row < 0).all(axis=1)
    assert dropped.any() and np.all(y2v[dropped] == 0.0)


def test_combine_k1_is_an_exact_gather():
    rng = np.random.default_rng(5)
    T, E, H = 40, 5, 8
    x = f64_to_bf16_bits(rng.standard_normal((T, H)))
    ids, w = _layout_and_weights(rng, T, E, 1, T)
    assert np.all(w == 1.0)
    lay, sb = dispatch(x, "bf16", ids, E, T)
    out_buf = sb[::-1].copy()                   # any rows: combine must gather them exactly
    y = combine(out_buf, "bf16", lay.pair_row, w)
    assert np.array_equal(y, out_buf[lay.pair_row[:, 0]])


@pytest.mark.parametrize("R", [1, 2])
def test_layer_against_per_token_dense_formulation(R):
    # without drops the layer is y[t] = sum_j w[t,j] * FFN_{ids[t,j] mod El}(x[t]); computed per
    # token with torch, never going through dispatch
    rng = np.random.default_rng(6 + R)
    T, H, E, k, F = 24, 16, 4, 2, 20
    El = E // R
    x = rng.standard_normal((T, H)).astype(np.float32)
    wr = (rng.standard_normal((E, H)) * 0.3).astype(np.float32)
    wgu = (rng.standard_normal((El, 2 * F, H)) * 0.2).astype(np.float32)
    wd = (rng.standard_normal((El, H, F)) * 0.2).astype(np.float32)
    res = moe_layer(x, "f32", wr, None, k, T, R, wgu, wd, F)
    ids, w = res["ids"], res["weights"]
    for t in range(T):
        acc = torch.zeros(H, dtype=torch.float64)
        for j in range(k):
            l = int(ids[t, j]) % El
            acc += float(w[t, j]) * _dense_swiglu_torch(x[t:t + 1], wgu[l], wd[l], F,
                                                         torch.float32)[0].double()
        assert np.allclose(res["y"][t], acc.numpy(), rtol=1e-6, atol=1e-7)
