"""GPU parity on seeded random layer shapes, through the C ABI.

24 shapes drawn from a fixed seed across the kernels' regimes: direct-to-LDS prefill tiles, 64- and 32-row
weight-streaming tiles, fp32, and the register-staged bf16 fallback, plus unconstrained draws. They cover
1..3000 tokens, hidden and FFN widths that are any multiple of 8, 4..512 experts, 1..8 slots, 1..8 ranks (and
one expert per rank), capacity factors from 0.5 to "no drop", and uniform, Zipf and hot-expert routing. Each shape
runs at a size the oracle finishes in seconds:
  * every stage against the whole oracle (test_gpu_parity.check_layer_full);
  * the fused combine, bit for bit against moe_expert_mlp + moe_combine;
  * the sender-side combine against the oracle;
  * for bf16 shapes with H % 128 == 0, the fp8 dispatch (codes and scales bit-exact) and the fp8 layer.
The environment variable MOE_RANDOM_SHAPES raises the number of shapes.
"""
import math
import os

import numpy as np
import pytest
import torch

import moe_workloads as W
from tests._hip_runner import run_layer, run_layer_fp8, to_np
from tests.test_gpu_fp8 import _check_dispatch, _check_layer, _oracle_layer_fp8
from tests.test_gpu_fused_combine import _check_fused
from tests.test_gpu_parity import check_layer_full
from tests.test_gpu_sender_combine import _check as _check_sender
from tests.test_gpu_sender_combine import _run_send_recv

import oracle

pytestmark = pytest.mark.gpu


def _draw(rng, kind):
    for _ in range(100000):
        dt = "f32" if kind == "f32" else ("bf16" if kind != "any" else str(rng.choice(["bf16", "bf16", "bf16", "f32"])))
        E = int(rng.choice([4, 6, 8, 12, 16, 32, 64, 160, 256, 512]))
        divs = [d for d in range(1, 9) if E % d == 0]
        R = int(rng.choice(divs + ([E] if E <= 512 and rng.random() < 0.1 else [])))
        k = int(rng.integers(1, min(8, E) + 1))
        T = int(math.exp(rng.uniform(0.0, math.log(3000.0))))
        H = 8 * int(rng.integers(1, 129))
        F = 8 * int(rng.integers(1, 65))
        cf = float(rng.choice([0.0, 0.5, 1.0, 1.25, 2.0]))
        C = T if cf == 0.0 else math.ceil(cf * T * k / E)
        routing = str(rng.choice(["uniform", "zipf", "hot8"] if E >= 8 else ["uniform", "zipf"]))
        per_expert = min(T * k, E * C) // (E // R)
        ok = T * k * H * F <= 3e9
        if kind == "dl":
            ok = ok and dt == "bf16" and H % 64 == 0 and F % 64 == 0 and per_expert >= 128
        elif kind == "dec64":
            ok = ok and dt == "bf16" and 32 <= per_expert < 128
        elif kind == "dec32":
            ok = ok and dt == "bf16" and per_expert < 32
        elif kind == "regpre":
            ok = ok and dt == "bf16" and per_expert >= 128 and (H % 64 != 0 or F % 64 != 0)
        if ok:
            return dict(T=T, H=H, E=E, k=k, F=F, R=R, C=C, dtype=dt, routing=routing)
    raise RuntimeError(f"no shape of kind {kind}")


def _shapes():
    """The 24 default shapes; MOE_RANDOM_SHAPES=N (N > 24) draws N - 24 more from the same stream, cycling
    through the regimes (a longer run: `MOE_RANDOM_SHAPES=600 pytest tests/test_gpu_random_shapes.py`)."""
    rng = np.random.default_rng(20261203)
    kinds = ["dl"] * 4 + ["dec64"] * 4 + ["dec32"] * 4 + ["f32"] * 3 + ["regpre"] * 2 + ["any"] * 7
    more = ["dl", "dec64", "dec32", "f32", "regpre", "any", "any", "any"]
    n = max(len(kinds), int(os.environ.get("MOE_RANDOM_SHAPES", len(kinds))))
    kinds += [more[i % len(more)] for i in range(n - len(kinds))]
    return [(kind, _draw(rng, kind)) for kind in kinds]


SHAPES = _shapes()


def _id(i, kind, s):
    return f"{i:02d}_{kind}_T{s['T']}_H{s['H']}_E{s['E']}_k{s['k']}_F{s['F']}_R{s['R']}_C{s['C']}_{s['dtype']}_{s['routing']}"


@pytest.mark.parametrize("i,kind,s", [(i, kd, s) for i, (kd, s) in enumerate(SHAPES)],
                         ids=[_id(i, kd, s) for i, (kd, s) in enumerate(SHAPES)])
def test_random_shape(i, kind, s):
    T, H, E, k, F, R, C = s["T"], s["H"], s["E"], s["k"], s["F"], s["R"], s["C"]
    cfg = W.small_config(W.workload("tiny-fp32"), seed=700 + i, name=f"random{i}", T=T, H=H, E=E, k=k, F=F, R=R,
                         dtype=s["dtype"], routing=s["routing"])
    print(f"\n[gpu] random shape {_id(i, kind, s)}", flush=True)
    inp = W.make_inputs(cfg, device="cuda", T=T)
    inp["C"] = C
    out = run_layer(inp, k, R)
    check_layer_full(cfg, inp, out, T, E, k, F, R, C)
    _check_fused(inp, out, k, R, calls=1)
    partial, y = _run_send_recv(out, out["layout"], inp["x"].dtype)
    _check_sender(E, R, out, partial, y, np.arange(T))
    if s["dtype"] == "bf16" and H % 128 == 0:
        o8 = run_layer_fp8(inp, k, R)
        assert torch.equal(o8["ids"], out["ids"])
        _check_dispatch(cfg, inp, o8)
        ref = _oracle_layer_fp8(cfg, inp, to_np(o8["ids"]), C, np.arange(T))
        _check_layer(oracle.to_f64(to_np(o8["y"]), "bf16"), ref, "fp8 layer")
