"""Seeded synthetic inputs for the MoE layer workloads.

This module is shared by the tests, the benchmark and the checker. It holds
only shapes, value distributions and seeds: none of the layer's arithmetic
(no routing, capacity, dispatch, FFN or combine) lives here.

Workloads (all synthetic; no dataset or trained weights exist for them):

  tiny_f32      T=8,     d=16,   d_ff=64,    E=2,   k=1, c=1.0,  fp32, ReLU,
                raw softmax gate (no renormalisation), zero biases
  small_bf16    T=4096,  d=1024, d_ff=4096,  E=8,   k=2, c=1.25, bf16, tanh-GELU,
                renormalised gates, every bias ~ N(0, 0.01)
  mid_bf16      T=16384, d=4096, d_ff=14336, E=8,   k=2, c=1.25, bf16, tanh-GELU,
                renormalised gates, zero biases (8 sequences x 2048 tokens,
                routed as one group)
  skewed_bf16   T=8192,  d=2048, d_ff=1024,  E=64,  k=4, c=1.0,  bf16, tanh-GELU,
                renormalised gates, router bias 2*ln(1/(rank+1)) over a seeded
                random ranking of the experts (Zipf(2)-skewed loads), other
                biases zero
  large_e_bf16  T=4096,  d=4096, d_ff=2048,  E=256, k=8, c=1.25, bf16, tanh-GELU,
                renormalised gates, router bias ~ N(0, 0.1), other biases zero

Dropless variants (capacity C = T, so no assignment is ever dropped):

  skewed_dropless_bf16  skewed_bf16's tensors with C = T: the hottest
                expert takes most of the 8192 tokens
  decode_bf16   mid_bf16's layer at decode size, T=64, C = T

Re-routing variant:

  skewed_reroute_bf16  skewed_bf16 with rank-major priority and two rounds
                of overflow re-routing to the next candidate experts

N(0, v) names the variance v. x ~ N(0, 1); W_r and W1 ~ N(0, 1/d); W2 ~ N(0, 1/d_ff).
Values are drawn in fp32 and rounded to bf16 (round to nearest even) for the
bf16 workloads; biases are always fp32.

Every tensor (and, for expert weights, every expert's slice) has its own
generator seeded from (0x4D6F45, workload seed id, tensor id, expert, user
seed), so any slice can be regenerated alone.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math

import torch

MAGIC = 0x4D6F45

TENSOR_IDS = {"x": 1, "W_r": 2, "b_r": 3, "W1": 4, "b1": 5, "W2": 6, "b2": 7, "dy": 8}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str              # "f32" or "bf16"
    T: int
    d: int
    d_ff: int
    E: int
    k: int
    c: float                # capacity factor
    act: str                # "relu" or "gelu_tanh"
    renormalize: bool
    router_bias: str        # "zero", "normal" or "zipf"
    router_bias_var: float  # variance when router_bias == "normal"
    ffn_bias_var: float     # variance of b1 and b2 (0 means zero biases)
    seed_id: int
    dropless: bool = False  # capacity C = T instead of ceil(c T k / E)
    priority: str = "token"  # "token" or "rank": order arrivals at a full expert are served
    reroute: int = 0        # rounds of overflow re-routing to the next candidate

    def scaled(self, **changes) -> "Workload":
        """Same recipe at other sizes (used for parity tests the oracle can
        finish in seconds)."""
        name = changes.pop("name", None) or (
            self.name + "@" + ",".join(f"{k}={v}" for k, v in sorted(changes.items())))
        return dataclasses.replace(self, name=name, **changes)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", "f32", 8, 16, 64, 2, 1, 1.0, "relu", False,
                         "zero", 0.0, 0.0, 1),
    "small_bf16": Workload("small_bf16", "bf16", 4096, 1024, 4096, 8, 2, 1.25, "gelu_tanh",
                           True, "normal", 0.01, 0.01, 2),
    "mid_bf16": Workload("mid_bf16", "bf16", 16384, 4096, 14336, 8, 2, 1.25, "gelu_tanh",
                         True, "zero", 0.0, 0.0, 3),
    "skewed_bf16": Workload("skewed_bf16", "bf16", 8192, 2048, 1024, 64, 4, 1.0, "gelu_tanh",
                            True, "zipf", 0.0, 0.0, 4),
    "large_e_bf16": Workload("large_e_bf16", "bf16", 4096, 4096, 2048, 256, 8, 1.25,
                             "gelu_tanh", True, "normal", 0.1, 0.0, 5),
}
WORKLOADS["skewed_dropless_bf16"] = WORKLOADS["skewed_bf16"].scaled(name="skewed_dropless_bf16",
                                                                    dropless=True)
WORKLOADS["decode_bf16"] = WORKLOADS["mid_bf16"].scaled(name="decode_bf16", T=64, dropless=True)
WORKLOADS["skewed_reroute_bf16"] = WORKLOADS["skewed_bf16"].scaled(name="skewed_reroute_bf16",
                                                                   priority="rank", reroute=2)


def _seed(*ids) -> int:
    h = hashlib.sha256(repr((MAGIC,) + tuple(ids)).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, *ids) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(*ids))
    return g


def _normal(shape, var, device, gen, out_dtype):
    v = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if var != 1.0:
        v.mul_(math.sqrt(var))
    return v.to(out_dtype)


def make_x(w: Workload, device, seed: int = 0) -> torch.Tensor:
    g = _gen(device, w.seed_id, TENSOR_IDS["x"], 0, seed)
    return _normal((w.T, w.d), 1.0, device, g, w.torch_dtype)


def make_dy(w: Workload, device, seed: int = 0) -> torch.Tensor:
    """Upstream gradient dL/dy [T, d] ~ N(0, 1) in the workload dtype, for the
    backward pass."""
    g = _gen(device, w.seed_id, TENSOR_IDS["dy"], 0, seed)
    return _normal((w.T, w.d), 1.0, device, g, w.torch_dtype)


def make_router(w: Workload, device, seed: int = 0):
    """(W_r [E, d] in the workload dtype, b_r [E] fp32)."""
    g = _gen(device, w.seed_id, TENSOR_IDS["W_r"], 0, seed)
    W_r = _normal((w.E, w.d), 1.0 / w.d, device, g, w.torch_dtype)
    g = _gen(device, w.seed_id, TENSOR_IDS["b_r"], 0, seed)
    if w.router_bias == "zero":
        b_r = torch.zeros(w.E, dtype=torch.float32, device=device)
    elif w.router_bias == "normal":
        b_r = _normal((w.E,), w.router_bias_var, device, g, torch.float32)
    elif w.router_bias == "zipf":
        # a random ranking of the experts; expert i gets 2*ln(1/(rank_i + 1))
        rank = torch.randperm(w.E, generator=g, device=device).to(torch.float64)
        b_r = (2.0 * torch.log(1.0 / (rank + 1.0))).to(torch.float32)
    else:
        raise ValueError(w.router_bias)
    return W_r, b_r


def make_expert(w: Workload, e: int, device, seed: int = 0):
    """One expert's (W1 [d_ff, d], b1 [d_ff], W2 [d, d_ff], b2 [d])."""
    dt = w.torch_dtype
    W1 = _normal((w.d_ff, w.d), 1.0 / w.d, device,
                 _gen(device, w.seed_id, TENSOR_IDS["W1"], e, seed), dt)
    W2 = _normal((w.d, w.d_ff), 1.0 / w.d_ff, device,
                 _gen(device, w.seed_id, TENSOR_IDS["W2"], e, seed), dt)
    if w.ffn_bias_var > 0:
        b1 = _normal((w.d_ff,), w.ffn_bias_var, device,
                     _gen(device, w.seed_id, TENSOR_IDS["b1"], e, seed), torch.float32)
        b2 = _normal((w.d,), w.ffn_bias_var, device,
                     _gen(device, w.seed_id, TENSOR_IDS["b2"], e, seed), torch.float32)
    else:
        b1 = torch.zeros(w.d_ff, dtype=torch.float32, device=device)
        b2 = torch.zeros(w.d, dtype=torch.float32, device=device)
    return W1, b1, W2, b2


def make_experts(w: Workload, device, seed: int = 0):
    """Stacked expert weights: W1 [E, d_ff, d], b1 [E, d_ff], W2 [E, d, d_ff], b2 [E, d]."""
    dt = w.torch_dtype
    W1 = torch.empty((w.E, w.d_ff, w.d), dtype=dt, device=device)
    W2 = torch.empty((w.E, w.d, w.d_ff), dtype=dt, device=device)
    b1 = torch.empty((w.E, w.d_ff), dtype=torch.float32, device=device)
    b2 = torch.empty((w.E, w.d), dtype=torch.float32, device=device)
    for e in range(w.E):
        W1[e], b1[e], W2[e], b2[e] = make_expert(w, e, device, seed)
    return W1, b1, W2, b2


def make_inputs(w: Workload, device, seed: int = 0) -> dict:
    x = make_x(w, device, seed)
    W_r, b_r = make_router(w, device, seed)
    W1, b1, W2, b2 = make_experts(w, device, seed)
    return {"x": x, "W_r": W_r, "b_r": b_r, "W1": W1, "b1": b1, "W2": W2, "b2": b2}


def to_numpy_bits(t: torch.Tensor):
    """Host copy of a tensor's stored values: bf16 as uint16 bit patterns,
    fp32 as float32, int32 as int32."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    return t.numpy()
