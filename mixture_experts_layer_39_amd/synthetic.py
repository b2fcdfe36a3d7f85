"""Seeded synthetic inputs for the MoE layer workloads.

This module only draws numbers: it holds none of the layer's arithmetic, so
both the HIP path and the CPU oracle can be fed from it.  Every tensor is drawn
in float32 from ``torch.randn`` with one seeded generator in a fixed order
(x, router weight or logits, W1, b1, W2, b2, upstream gradient), scaled by the
workload's standard deviation and cast to the workload's storage dtype (bf16
by round-to-nearest-even).  The cast tensors *are* the inputs.

Workloads (shapes from the five benchmark configurations of the layer):
  tiny_fp32   T=64,    d=32,   E=4,   k=1, Linear(32->64)+ReLU+Linear(64->32), fp32,
              capacity_factor 1.0, min_capacity 4, logits given ~ N(0,1), weights N(0,0.1)
  top2_e8     T=4096,  d=512,  E=8,   k=2, one Linear(512->512)+bias, bf16, cf 1.0
  top2_e64    T=16384, d=2048, E=64,  k=2, 2048->5120->2048 GELU, bf16, cf 1.25
  skew_e16    T=32768, d=4096, E=16,  k=2, 4096->14336->4096 GELU, bf16, cf 2.0,
              router bias ln(p_e) with p_e proportional to (e+1)^-1.2 (Zipf s=1.2)
  nodrop_e128 T=65536, d=4096, E=128, k=2, 4096->1536->4096 GELU, bf16, no drop,
              plus an N(0,1) upstream gradient for the expert backward
  nodrop_e128_layer  the same layer with an N(0,1) upstream gradient of the
              layer output [T, d] for the whole layer's backward
  random_e64  the top2_e64 layer and inputs with the seeded random gate
              options of a training step on (router input jitter, sampled
              second expert)
  residual_e64 the top2_e64 layer as a residual MoE (PR-MoE): after the
              layer's tensors, a dense MLP of the expert's shape (W1 [h, d],
              b1, W2 [d, h], b2) and the mixing coefficient Linear (W_c [2, d]
              ~ N(0, 0.02), b_c [2] fp32 ~ N(0, 1))
Activations and upstream gradients ~ N(0,1); weights and biases ~ N(0, 0.02)
unless stated.
"""
from __future__ import annotations

import math

import torch

ACT_NONE, ACT_RELU, ACT_GELU = 0, 1, 2

WORKLOADS = {
    "tiny_fp32": dict(T=64, d=32, E=4, k=1, h=64, act=ACT_RELU, dtype="f32",
                      cf=1.0, min_cap=4, drop=True, wstd=0.1, logits_given=True,
                      zipf=None, seed=1001),
    "top2_e8": dict(T=4096, d=512, E=8, k=2, h=0, act=ACT_NONE, dtype="bf16",
                    cf=1.0, min_cap=4, drop=True, wstd=0.02, logits_given=False,
                    zipf=None, seed=1002),
    "top2_e64": dict(T=16384, d=2048, E=64, k=2, h=5120, act=ACT_GELU, dtype="bf16",
                     cf=1.25, min_cap=4, drop=True, wstd=0.02, logits_given=False,
                     zipf=None, seed=1003),
    "skew_e16": dict(T=32768, d=4096, E=16, k=2, h=14336, act=ACT_GELU, dtype="bf16",
                     cf=2.0, min_cap=4, drop=True, wstd=0.02, logits_given=False,
                     zipf=1.2, seed=1004),
    "nodrop_e128": dict(T=65536, d=4096, E=128, k=2, h=1536, act=ACT_GELU, dtype="bf16",
                        cf=1.0, min_cap=4, drop=False, wstd=0.02, logits_given=False,
                        zipf=None, seed=1005, backward=True),
    "random_e64": dict(T=16384, d=2048, E=64, k=2, h=5120, act=ACT_GELU, dtype="bf16",
                       cf=1.25, min_cap=4, drop=True, wstd=0.02, logits_given=False,
                       zipf=None, seed=1003, random_gate=True),
    "residual_e64": dict(T=16384, d=2048, E=64, k=2, h=5120, act=ACT_GELU, dtype="bf16",
                         cf=1.25, min_cap=4, drop=True, wstd=0.02, logits_given=False,
                         zipf=None, seed=1006, residual=True),
    "nodrop_e128_layer": dict(T=65536, d=4096, E=128, k=2, h=1536, act=ACT_GELU, dtype="bf16",
                              cf=1.0, min_cap=4, drop=False, wstd=0.02, logits_given=False,
                              zipf=None, seed=1005, backward="layer"),
}


def spec(name, **overrides):
    """A copy of a named workload with some fields replaced (smaller T, ...)."""
    s = dict(WORKLOADS[name])
    s["name"] = name
    s.update(overrides)
    return s


def zipf_router_bias(E, s):
    """b[e] = ln p_e, p_e = (e+1)^-s / sum_i i^-s: expert popularity ~ Zipf(s)."""
    z = [(e + 1) ** (-s) for e in range(E)]
    tot = sum(z)
    return torch.tensor([math.log(v / tot) for v in z], dtype=torch.float32)


def _draw(g, shape, std, device):
    return torch.randn(*shape, generator=g, device=device, dtype=torch.float32) * std


def make_inputs(sp, device="cpu", seed=None, n_rows_grad=None):
    """Draw one workload's tensors on ``device``.

    Returns a dict with x, w_router (or None), b_router (or None), logits
    (given logits, or None), w1, b1, w2 (or None), b2 (or None) and, for
    workloads with a backward, dy of shape [n_rows_grad, d] (default: k*T
    dispatched rows for the expert backward, T token rows for the layer's).
    """
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(sp["seed"] if seed is None else seed)
    dt = torch.bfloat16 if sp["dtype"] == "bf16" else torch.float32
    T, d, E, h = sp["T"], sp["d"], sp["E"], sp["h"]
    std = sp["wstd"]
    out = {}
    out["x"] = _draw(g, (T, d), 1.0, dev).to(dt)
    if sp.get("logits_given"):
        out["logits"] = _draw(g, (T, E), 1.0, dev)
        out["w_router"] = None
    else:
        out["logits"] = None
        out["w_router"] = _draw(g, (E, d), std, dev).to(dt)
    out["b_router"] = zipf_router_bias(E, sp["zipf"]).to(dev) if sp.get("zipf") else None
    hid = h if h > 0 else d
    out["w1"] = _draw(g, (E, hid, d), std, dev).to(dt)
    out["b1"] = _draw(g, (E, hid), std, dev).to(dt)
    if h > 0:
        out["w2"] = _draw(g, (E, d, h), std, dev).to(dt)
        out["b2"] = _draw(g, (E, d), std, dev).to(dt)
    else:
        out["w2"] = None
        out["b2"] = None
    if sp.get("backward"):
        n = (T if sp["backward"] == "layer" else sp["k"] * T) if n_rows_grad is None else n_rows_grad
        out["dy"] = _draw(g, (n, d), 1.0, dev).to(dt)
    if sp.get("residual"):
        out["mlp_w1"] = _draw(g, (hid, d), std, dev).to(dt)
        out["mlp_b1"] = _draw(g, (hid,), std, dev).to(dt)
        out["mlp_w2"] = _draw(g, (d, h), std, dev).to(dt) if h > 0 else None
        out["mlp_b2"] = _draw(g, (d,), std, dev).to(dt) if h > 0 else None
        out["coef_w"] = _draw(g, (2, d), std, dev).to(dt)
        out["coef_b"] = _draw(g, (2,), 1.0, dev)
    return out
