"""Seeded synthetic inputs for the MoE layer workloads.

This module only draws random numbers; it holds none of the layer's
arithmetic.  The same bytes feed the HIP library and, in the tests and the
CPU-baseline measurement, the CPU oracle.

Seeding: workload ``c`` has a base seed B; tensor ``j`` of it is drawn from a
fresh ``torch.Generator`` seeded with ``B + j`` (j: 0 x, 1 router weight,
2 gate, 3 up, 4 down, 5-7 shared gate/up/down, 8 expert bias, 9 skew
permutation).  Tensors that decide the routing (x, router weight, bias) are
always drawn on the CPU so that every machine gets identical bytes; expert
weights may be drawn on the GPU for speed (they never decide a routing).

Distributions (std, not variance, everywhere except where noted):
  x ~ N(0, 1); router weight ~ N(0, 1/H) in *variance* (std H^-1/2), so that
  logits are ~N(0, 1); expert and shared weights ~ N(0, 0.02); expert bias
  ~ N(0, 0.05) where a workload asks for one.
"""
from __future__ import annotations

import dataclasses
import math
import os

import torch


@dataclasses.dataclass(frozen=True)
class LayerShape:
    """Shape and dtype of one MoE layer workload."""
    name: str
    T: int
    H: int
    E: int = 256
    n_group: int = 8
    topk_group: int = 4
    top_k: int = 8
    I: int = 512
    I_shared: int = 512
    scale: float = 2.5
    dtype: str = "bf16"          # activations and expert weights: "bf16" or "f32"
    bias: str = "none"           # "none", "normal" (std 0.05) or "skew"
    seed: int = 0
    layers: int = 1              # > 1: a residual stack of independent layers

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32


# The five workloads: a tiny fp32 layer, the full-size layer at 512 and 16384
# tokens, a skewed-routing layer at 65536 tokens and a 19-layer stack.
WORKLOADS = {
    "tiny_f32": LayerShape("tiny_f32", T=256, H=512, I=128, I_shared=128, dtype="f32", seed=0),
    "full_t512": LayerShape("full_t512", T=512, H=2048, seed=1000),
    "full_t16k_bias": LayerShape("full_t16k_bias", T=16384, H=2048, bias="normal", seed=2000),
    "skew_t64k": LayerShape("skew_t64k", T=65536, H=2048, bias="skew", seed=3000),
    "stack19_t8k": LayerShape("stack19_t8k", T=8192, H=2048, seed=4000, layers=19),
}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal(shape, std: float, seed: int, device, dtype) -> torch.Tensor:
    g = _gen(seed, device)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def skew_offsets(E: int, n_group: int, seed: int, hot_groups: int = 2, hot_per_group: int = 10,
                 amp: float = 12.0, s: float = 1.2) -> torch.Tensor:
    """Per-expert logit offsets o_e = amp * rank_e^(-s) (a Zipf law).  Ranks
    1..hot_groups*hot_per_group go to seeded experts inside `hot_groups`
    seeded groups; the other ranks are spread at random over the rest."""
    g = _gen(seed, "cpu")
    gsize = E // n_group
    groups = torch.randperm(n_group, generator=g)[:hot_groups]
    hot = []
    for grp in groups.tolist():
        members = torch.randperm(gsize, generator=g)[:hot_per_group] + grp * gsize
        hot += members.tolist()
    hot_order = torch.randperm(len(hot), generator=g).tolist()
    hot = [hot[i] for i in hot_order]
    rest = [e for e in range(E) if e not in set(hot)]
    rest_order = torch.randperm(len(rest), generator=g).tolist()
    ordered = hot + [rest[i] for i in rest_order]
    off = torch.empty(E, dtype=torch.float32)
    for rank, e in enumerate(ordered, start=1):
        off[e] = amp * rank ** (-s)
    return off


def router_inputs(shape: LayerShape, layer: int = 0):
    """(x [T,H], router weight [E,H] fp32, expert bias [E] fp32 or None) on the
    CPU.  For the skewed workload the bias is returned as None: it comes from
    the first routing pass and is stored with the tests (``skew_bias``)."""
    B = shape.seed + 100 * layer
    x = _normal((shape.T, shape.H), 1.0, B + 0, "cpu", shape.torch_dtype)
    wr = _normal((shape.E, shape.H), 1.0 / math.sqrt(shape.H), B + 1, "cpu", torch.float32)
    bias = None
    if shape.bias == "normal":
        bias = _normal((shape.E,), 0.05, B + 8, "cpu", torch.float32)
    if shape.bias == "skew":
        # constant input channel 0 carries the per-expert offset into the logits
        x[:, 0] = 1.0
        wr[:, 0] = skew_offsets(shape.E, shape.n_group, B + 9)
    return x, wr, bias


SKEW_BIAS_FILE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                              "tests", "golden", "skew_t64k_expert_bias.txt")


def skew_bias() -> torch.Tensor:
    """The skewed workload's expert bias [E] fp32, as stored next to the tests
    (the load-balancing update of the first, unbiased routing pass's counts;
    tests/golden/make_skew_bias.py writes it from the oracle)."""
    vals = [float(line) for line in open(SKEW_BIAS_FILE) if line.strip() and line[0] != "#"]
    return torch.tensor(vals, dtype=torch.float32)


def expert_weights(shape: LayerShape, device="cpu", layer: int = 0):
    """dict(w_gate, w_up, w_down [E][I][H], ws_gate, ws_up, ws_down [I_s][H])."""
    B = shape.seed + 100 * layer
    dt = shape.torch_dtype
    E, I, H, Is = shape.E, shape.I, shape.H, shape.I_shared
    out = dict(
        w_gate=_normal((E, I, H), 0.02, B + 2, device, dt),
        w_up=_normal((E, I, H), 0.02, B + 3, device, dt),
        w_down=_normal((E, I, H), 0.02, B + 4, device, dt),
        ws_gate=None, ws_up=None, ws_down=None,
    )
    if Is > 0:
        out["ws_gate"] = _normal((Is, H), 0.02, B + 5, device, dt)
        out["ws_up"] = _normal((Is, H), 0.02, B + 6, device, dt)
        out["ws_down"] = _normal((Is, H), 0.02, B + 7, device, dt)
    return out


def small_shape(T: int, H: int = 256, I: int = 64, I_shared: int = 64, dtype: str = "bf16",
                bias: str = "none", seed: int = 77, E: int = 256, n_group: int = 8,
                topk_group: int = 4, top_k: int = 8) -> LayerShape:
    """A reduced layer for fast tests (same structure, smaller H and I)."""
    return LayerShape(f"small_T{T}_H{H}_I{I}", T=T, H=H, E=E, n_group=n_group,
                      topk_group=topk_group, top_k=top_k, I=I, I_shared=I_shared, dtype=dtype,
                      bias=bias, seed=seed)


def to_numpy_bits(t: torch.Tensor):
    """Host numpy view for the oracle: fp32 stays fp32, bf16 becomes uint16 bits."""
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    if t.dtype == torch.float32:
        return t.numpy()
    raise TypeError(t.dtype)
