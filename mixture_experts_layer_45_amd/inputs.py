"""Seeded synthetic inputs for the sparse MoE layer forward.

This module only draws random tensors and lists workload shapes: it holds none
of the layer's arithmetic, so both the HIP path and the CPU oracle can take
their inputs from it.  Every tensor comes from its own torch.Generator, seeded
from (seed, tensor id, expert); expert-indexed weights are drawn one expert at
a time so a single expert can be regenerated on its own.

Layouts (shared with the C ABI):
  x            [T, h]
  w_router     [H, E, d]        d = h / H; row e holds expert e's router weights
  w_gate/w_up  [H*E, f, d]      out-major: f rows of d inputs
  w_down       [H*E, d, f]
  sh_gate/up   [f, h]; sh_down [h, f]   (always-on shared expert)
  w_o          [h, h]           out-major
  logit_bias   [H*E] fp32 (added to the router logits)
  select_bias  [H*E] fp32 (added to the sigmoid routing key only)

Weights are N(0, 1/fan_in) and activations N(0, 1), drawn in fp32 and rounded
to the workload's dtype (bf16 by round-to-nearest-even).
"""
import math

import torch

# Workload shapes.  The pages describe top-2 GShard and top-1 Switch gates, a
# sigmoid router with a selection bias, capacity factors with token dropping
# and a multi-head variant; these are synthetic layers of those kinds.
CONFIGS = {
    # tiny fp32 layer: 8 experts, top-2 softmax, SwiGLU 64->128->64, no capacity
    "tiny_f32": dict(T=256, h=64, H=1, E=8, K=2, f=128, n_shared=0, has_wo=0, dtype="f32",
                     score="softmax", act="swiglu", capacity_factor=0.0, alpha=0.01,
                     logit_bias=None, select_bias=None),
    # top-2 softmax over 8 experts, SwiGLU 4096->14336->4096, capacity factor 1.25
    "top2_e8_h4096": dict(T=8192, h=4096, H=1, E=8, K=2, f=14336, n_shared=0, has_wo=0,
                          dtype="bf16", score="softmax", act="swiglu", capacity_factor=1.25,
                          alpha=0.01, logit_bias=None, select_bias=None),
    # 256 fine-grained experts + 1 shared, top-8 by sigmoid + bias, SwiGLU 7168->2048->7168
    "sigmoid_top8_e256_shared": dict(T=4096, h=7168, H=1, E=256, K=8, f=2048, n_shared=1,
                                     has_wo=0, dtype="bf16", score="sigmoid", act="swiglu",
                                     capacity_factor=0.0, alpha=0.01, logit_bias=None,
                                     select_bias="uniform0.1"),
    # Switch top-1 over 64 experts with Zipf-like logit bias, GELU 2048->8192->2048, CF 1.0
    "switch_top1_e64_zipf": dict(T=16384, h=2048, H=1, E=64, K=1, f=8192, n_shared=0, has_wo=0,
                                 dtype="bf16", score="softmax", act="gelu", capacity_factor=1.0,
                                 alpha=0.01, logit_bias="zipf", select_bias=None),
    # multi-head: 8 heads of 512, 32 experts per head, top-4, SwiGLU 512->1024->512, W_o 4096^2
    "multihead_h8_e32_top4": dict(T=8192, h=4096, H=8, E=32, K=4, f=1024, n_shared=0, has_wo=1,
                                  dtype="bf16", score="softmax", act="swiglu",
                                  capacity_factor=0.0, alpha=0.01, logit_bias=None,
                                  select_bias=None),
}

# the workload the throughput figure is quoted on
BENCH_WORKLOAD = "top2_e8_h4096"

_TENSOR_ID = dict(x=0, w_router=1, bias=2, w_gate=3, w_up=4, w_down=5,
                  sh_gate=6, sh_up=7, sh_down=8, w_o=9, logits=10)


def variant(name, **over):
    """A copy of a named workload with some fields replaced (smaller test shapes)."""
    cfg = dict(CONFIGS[name])
    cfg.update(over)
    cfg["name"] = name if not over else name + "[" + ",".join(f"{k}={v}" for k, v in sorted(over.items())) + "]"
    return cfg


def torch_dtype(cfg):
    return torch.bfloat16 if cfg["dtype"] == "bf16" else torch.float32


def _gen(device, seed, tid, e=0):
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1000 + tid) * 100003 + e)
    return g


def _normal(shape, std, device, dtype, gen):
    t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    t.mul_(std)
    return t.to(dtype)


def _per_expert(n, shape, std, device, dtype, seed, tid, first=0):
    out = torch.empty((n,) + tuple(shape), device=device, dtype=dtype)
    for e in range(n):
        out[e].copy_(_normal(shape, std, device, dtype, _gen(device, seed, tid, first + e)))
    return out


def make_inputs(cfg, device="cpu", seed=0, with_weights=True):
    """All layer inputs for one workload as torch tensors on `device`."""
    T, h, H, E, f = cfg["T"], cfg["h"], cfg.get("H", 1), cfg["E"], cfg["f"]
    d = h // H
    Et = H * E
    dt = torch_dtype(cfg)
    out = {}
    out["x"] = _normal((T, h), 1.0, device, dt, _gen(device, seed, _TENSOR_ID["x"]))
    if not with_weights:
        return out
    out["w_router"] = _normal((H, E, d), 1.0 / math.sqrt(d), device, dt,
                              _gen(device, seed, _TENSOR_ID["w_router"]))
    out.update(make_biases(cfg, device, seed))
    gelu = cfg.get("act", "swiglu") == "gelu"
    out["w_gate"] = _per_expert(Et, (f, d), 1.0 / math.sqrt(d), device, dt, seed, _TENSOR_ID["w_gate"])
    out["w_up"] = None if gelu else _per_expert(Et, (f, d), 1.0 / math.sqrt(d), device, dt, seed,
                                                _TENSOR_ID["w_up"])
    out["w_down"] = _per_expert(Et, (d, f), 1.0 / math.sqrt(f), device, dt, seed, _TENSOR_ID["w_down"])
    if cfg.get("n_shared", 0):
        out["sh_gate"] = _normal((f, h), 1.0 / math.sqrt(h), device, dt, _gen(device, seed, _TENSOR_ID["sh_gate"]))
        out["sh_up"] = None if gelu else _normal((f, h), 1.0 / math.sqrt(h), device, dt,
                                                 _gen(device, seed, _TENSOR_ID["sh_up"]))
        out["sh_down"] = _normal((h, f), 1.0 / math.sqrt(f), device, dt, _gen(device, seed, _TENSOR_ID["sh_down"]))
    else:
        out["sh_gate"] = out["sh_up"] = out["sh_down"] = None
    out["w_o"] = (_normal((h, h), 1.0 / math.sqrt(h), device, dt, _gen(device, seed, _TENSOR_ID["w_o"]))
                  if cfg.get("has_wo", 0) else None)
    return out


def make_biases(cfg, device="cpu", seed=0):
    """logit_bias and select_bias of a workload (None where it has none)."""
    E, Et = cfg["E"], cfg.get("H", 1) * cfg["E"]
    out = {}
    if cfg.get("logit_bias") == "zipf":
        # expert e (rank e+1 in popularity) gets 2*ln(1/(e+1)), the same in every head
        ranks = torch.arange(1, E + 1, dtype=torch.float64)
        out["logit_bias"] = (2.0 * torch.log(1.0 / ranks)).to(torch.float32).repeat(cfg.get("H", 1)).to(device)
    else:
        out["logit_bias"] = None
    if cfg.get("select_bias") == "uniform0.1":
        g = _gen(device, seed, _TENSOR_ID["bias"])
        out["select_bias"] = torch.rand((Et,), generator=g, device=device, dtype=torch.float32) * 0.2 - 0.1
    else:
        out["select_bias"] = None
    return out


def make_logits(cfg, device="cpu", seed=0, tie_every=0, T=None):
    """Synthetic router logits [T*H, E] ~ N(0,1) fp32.  With tie_every = n > 0,
    every n-th row copies its largest value into another slot, so the rows hold
    exact ties at the top."""
    T = cfg["T"] if T is None else T
    S, E = T * cfg.get("H", 1), cfg["E"]
    lg = torch.randn((S, E), generator=_gen(device, seed, _TENSOR_ID["logits"]), device=device,
                     dtype=torch.float32)
    if tie_every and E > 1:
        rows = torch.arange(0, S, tie_every, device=device)
        top = lg[rows].argmax(dim=1)
        other = (top + 1 + (rows % (E - 1))) % E
        lg[rows, other] = lg[rows, top]
    return lg


def make_routing(cfg, device="cpu", seed=0, T=None, skew=0.0):
    """Synthetic top-K expert ids [T*H, K] int32 (distinct per row, global ids
    head*E + e), drawn from a Zipf-like popularity when skew > 0."""
    T = cfg["T"] if T is None else T
    H, E, K = cfg.get("H", 1), cfg["E"], cfg["K"]
    S = T * H
    g = _gen(device, seed, _TENSOR_ID["logits"], 7)
    w = torch.arange(1, E + 1, dtype=torch.float64, device=device).pow(-skew)
    w = w.expand(S, E)
    pick = torch.multinomial(w.to(torch.float32), K, replacement=False, generator=g)
    heads = (torch.arange(S, device=device) % H).unsqueeze(1)
    return (pick + heads * E).to(torch.int32)
