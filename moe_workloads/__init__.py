"""Seeded synthetic inputs for the MoE-layer hot path (shared by the oracle tests and the HIP path).

This module holds the five workload shapes and the seeded generators only. It contains none of the
method's arithmetic (no routing, no dispatch, no expert math): it draws activations, router weights,
expert weights and the additive logit bias that gives each workload its routing structure.

Shapes follow the pages:
  * tiny fp32 layer (256 tokens, hidden 128, 8 experts, top-2, FFN 256, capacity factor 1.25);
  * Mixtral-8x7B-shaped decode (hidden 4096, 8 experts, top-2, FFN 14336; the model is named in the
    "Introductie" section of "Efficient and portable mixture-of-experts communication");
  * DeepSeek-V3 / Kimi-K2-shaped layers (hidden 7168, 256 / 384 experts, top-8, 128 decode or 4096
    prefill tokens), the shapes of the "Оценка" (evaluation) section of "Enabling trillion-parameter
    models on AWS EFA";
  * routing shapes "balanced" and "skewed" (hot spots, long tail, overflow) from Step 1 of
    "80. MoE Expert Parallel Benchmark".

Seeds are per (config, tensor, expert): ``(cfg << 32) | (tensor_id << 16) | l`` with tensor ids
0 = x, 1 = router weight, 2 = w_gate_up[l], 3 = w_down[l], 4 = routing structure.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

__all__ = ["MoEConfig", "WORKLOADS", "workload", "capacity", "rows_max", "make_inputs", "make_routing_bias",
           "make_expert_weights", "seed_for"]


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    """One synthetic MoE-layer workload.

    T tokens of hidden size H, E experts of which each token picks k, expert FFN width F.
    R destination ranks in the layout (El = E / R local experts per rank). The capacity factor is the
    rational ``cf_num / cf_den``; ``cf_num == 0`` means "no capacity drop" (capacity = T).
    ``dtype`` is the activation / expert-weight type ("f32" or "bf16"); the router is always fp32.
    ``routing`` is the routing structure: "uniform", "balanced", "zipf" or "hot8".
    ``seed`` selects the workload's random streams (see seed_for).
    """
    seed: int
    name: str
    T: int
    H: int
    E: int
    k: int
    F: int
    R: int
    cf_num: int
    cf_den: int
    dtype: str
    routing: str

    @property
    def El(self) -> int:
        return self.E // self.R


# the five workloads, by name (the order is the benchmark's listing order)
WORKLOADS = {c.name: c for c in (
    MoEConfig(1, "tiny-fp32", T=256, H=128, E=8, k=2, F=256, R=1, cf_num=5, cf_den=4,
              dtype="f32", routing="uniform"),
    MoEConfig(2, "mixtral8x7b-decode", T=128, H=4096, E=8, k=2, F=14336, R=1, cf_num=0, cf_den=1,
              dtype="bf16", routing="uniform"),
    MoEConfig(3, "dsv3-prefill-ep8-share", T=4096, H=7168, E=256, k=8, F=2048, R=8, cf_num=1,
              cf_den=1, dtype="bf16", routing="balanced"),
    MoEConfig(4, "kimik2-decode-ep8-share", T=128, H=7168, E=384, k=8, F=2048, R=8, cf_num=5,
              cf_den=4, dtype="bf16", routing="zipf"),
    MoEConfig(5, "large-skewed-prefill", T=16384, H=7168, E=256, k=8, F=2048, R=1, cf_num=1,
              cf_den=1, dtype="bf16", routing="hot8"),
)}


def workload(name: str) -> MoEConfig:
    """The workload called `name`."""
    try:
        return WORKLOADS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; choose from {list(WORKLOADS)}") from None


def capacity(cfg: MoEConfig, T: Optional[int] = None) -> int:
    """Per-expert capacity C = ceil(cf * T * k / E), in exact integer arithmetic; T when no drop.

    `T` overrides the config's token count (for cut-down test inputs).
    """
    T = cfg.T if T is None else T
    if cfg.cf_num == 0:
        return T
    num = cfg.cf_num * T * cfg.k
    den = cfg.cf_den * cfg.E
    return -(-num // den)


def rows_max(T: int, k: int, E: int, C: int) -> int:
    """Worst-case number of dispatched rows: min(T*k, E*C)."""
    return min(T * k, E * C)


def seed_for(seed: int, tensor_id: int, l: int = 0) -> int:
    return (seed << 32) | (tensor_id << 16) | l


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _act_dtype(cfg: MoEConfig) -> torch.dtype:
    return torch.float32 if cfg.dtype == "f32" else torch.bfloat16


def make_routing_bias(cfg: MoEConfig, device="cpu") -> tuple[Optional[torch.Tensor], int]:
    """Additive fp32 logit bias that gives the workload its routing structure.

    Returns (bias, row_stride): bias is None (uniform), an [E] tensor (row stride 0) or a
    [T, E] tensor (row stride E).
      * balanced: +64 on S_t = {pi_E((pi_T(t)*k + j) mod E) : j < k} for seeded permutations
        pi_E, pi_T, so that every expert receives exactly T*k/E tokens;
      * zipf: b_e = -1.2 * ln(e + 1), i.e. expert popularity multiplied by a Zipf(1.2) pmf;
      * hot8: +16 on experts 0..7 for even tokens (half of the tokens go to 8 hot experts).
    """
    T, E, k = cfg.T, cfg.E, cfg.k
    if cfg.routing == "uniform":
        return None, 0
    if cfg.routing == "zipf":
        e = torch.arange(E, dtype=torch.float64)
        return (-1.2 * torch.log(e + 1.0)).to(torch.float32).to(device), 0
    if cfg.routing == "balanced":
        g = _gen("cpu", seed_for(cfg.seed, 4))
        pi_E = torch.randperm(E, generator=g)
        pi_T = torch.randperm(T, generator=g)
        cols = (pi_T.view(T, 1) * k + torch.arange(k).view(1, k)) % E
        bias = torch.zeros(T, E, dtype=torch.float32)
        bias.scatter_(1, pi_E[cols], 64.0)
        return bias.to(device), E
    if cfg.routing == "hot8":
        bias = torch.zeros(T, E, dtype=torch.float32)
        bias[0::2, :8] = 16.0
        return bias.to(device), E
    raise ValueError(f"unknown routing structure {cfg.routing!r}")


def make_expert_weights(cfg: MoEConfig, l: int, device="cpu") -> tuple[torch.Tensor, torch.Tensor]:
    """Weights of local expert l: w_gate_up [2F, H] (rows 0..F-1 gate, F..2F-1 up), w_down [H, F].

    N(0, 0.02^2) drawn in fp32 then rounded to the activation type (round-to-nearest-even).
    """
    dt = _act_dtype(cfg)
    gu = torch.randn(2 * cfg.F, cfg.H, generator=_gen(device, seed_for(cfg.seed, 2, l)),
                     device=device, dtype=torch.float32).mul_(0.02).to(dt)
    dn = torch.randn(cfg.H, cfg.F, generator=_gen(device, seed_for(cfg.seed, 3, l)),
                     device=device, dtype=torch.float32).mul_(0.02).to(dt)
    return gu, dn


def make_inputs(cfg: MoEConfig, device="cpu", T: Optional[int] = None,
                with_experts: bool = True) -> dict:
    """All inputs of one layer, on `device`.

    x [T, H] ~ N(0, 1) in the activation type; w_router [E, H] ~ N(0, 0.02^2) fp32; the routing
    bias; and (if with_experts) w_gate_up [El, 2F, H], w_down [El, H, F] in the activation type.
    `T` may shrink the token count (the bias is then cut to the first T rows).
    """
    T_full = cfg.T
    T = T_full if T is None else T
    dt = _act_dtype(cfg)
    x = torch.randn(T_full, cfg.H, generator=_gen(device, seed_for(cfg.seed, 0)), device=device,
                    dtype=torch.float32)[:T].to(dt).contiguous()
    w_router = torch.randn(cfg.E, cfg.H, generator=_gen(device, seed_for(cfg.seed, 1)),
                           device=device, dtype=torch.float32).mul_(0.02)
    bias, stride = make_routing_bias(cfg, device)
    if bias is not None and stride != 0:
        bias = bias[:T].contiguous()
    out = dict(x=x, w_router=w_router, bias=bias, bias_stride=stride, T=T, C=capacity(cfg, T))
    if with_experts:
        El = cfg.El
        w_gu = torch.empty(El, 2 * cfg.F, cfg.H, dtype=dt, device=device)
        w_dn = torch.empty(El, cfg.H, cfg.F, dtype=dt, device=device)
        for l in range(El):
            gu, dn = make_expert_weights(cfg, l, device)
            w_gu[l].copy_(gu)
            w_dn[l].copy_(dn)
            del gu, dn
        out["w_gate_up"] = w_gu
        out["w_down"] = w_dn
    return out


def small_config(base: MoEConfig, **overrides) -> MoEConfig:
    """A copy of `base` with some fields replaced (for edge-case tests)."""
    return dataclasses.replace(base, **overrides)


def describe(cfg: MoEConfig) -> str:
    return (f"{cfg.name}: T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.k} F={cfg.F} "
            f"R={cfg.R} C={capacity(cfg)} {cfg.dtype} {cfg.routing}")

