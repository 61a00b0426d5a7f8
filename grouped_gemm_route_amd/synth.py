"""Seeded synthetic inputs for the MoE layer workloads.

This module only draws inputs: router logits, hidden states and expert
weights.  It holds none of the layer's arithmetic, so both the HIP path and
the CPU oracle can take their inputs from it.

No trained weights or routing traces are used.  The inputs are synthetic.
Their shapes and routing skew follow what the pages describe: routing is
skewed ("MoE 专家并行的 All-to-All 通信瓶颈", section "专家越多，通信为什么越重":
a few experts take most tokens), and in one incident 70% of the tokens
landed on 16% of the experts ("MoE 推理服务工程真相 2026", section 5.2).

Recipe:
  * logits  float32 N(0,1) of shape [N, E], plus a per-expert bias:
      - "zipf": bias_e = -2.2 * ln(pi(e) + 1) for a seeded permutation pi
        (twice the log of a Zipf(s=1.1) weight of the expert's rank);
      - "hot":  +hot_bias on the first round(0.16 E) experts of a seeded
        permutation;
  * x       N(0,1) [N, d], stored in the activation type;
  * weights N(0, std = 1/sqrt(fan_in)), stored in the activation type:
      w_gate, w_up [E, ffn, d] (fan_in d), w_down [E, d, ffn] (fan_in ffn).
Every tensor and every expert has its own seed, so one expert's weights can
be regenerated alone.  Values are drawn in float32 with torch's generator on
the requested device and rounded to bf16 by torch (round-to-nearest-even).
"""
from __future__ import annotations

import math
import zlib

import torch

# The five layer shapes, and the dropless / C=1.0 pair of the last one.
CONFIGS = {
    "tiny_f32": dict(N=256, d=128, ffn=256, E=8, K=2, W=4, act="f32",
                     bias="none", C=None),
    "dense8": dict(N=4096, d=4096, ffn=14336, E=8, K=2, W=8, act="bf16",
                   bias="none", C=None),
    "fine128_zipf_c1.25": dict(N=8192, d=2048, ffn=768, E=128, K=8, W=8,
                               act="bf16", bias="zipf", C=1.25),
    "decode256": dict(N=16, d=7168, ffn=2048, E=256, K=8, W=8, act="bf16",
                      bias="none", C=None),
    "prefill256_hot": dict(N=32768, d=7168, ffn=2048, E=256, K=8, W=8,
                           act="bf16", bias="hot", hot_bias=4.0, C=None),
    "prefill256_hot_c1.0": dict(N=32768, d=7168, ffn=2048, E=256, K=8, W=8,
                                act="bf16", bias="hot", hot_bias=4.0, C=1.0),
    # the same hot set with the bias that puts ~70% of assignments on it
    # (70.1% with these seeds), the share the skewed-prefill workload names
    "prefill256_cal": dict(N=32768, d=7168, ffn=2048, E=256, K=8, W=8,
                           act="bf16", bias="hot", hot_bias=1.2, C=None),
    "prefill256_cal_c1.0": dict(N=32768, d=7168, ffn=2048, E=256, K=8, W=8,
                                act="bf16", bias="hot", hot_bias=1.2, C=1.0),
}

TORCH_DTYPE = {"bf16": torch.bfloat16, "f32": torch.float32}


def config(name, **overrides):
    """A copy of a named config with fields overridden (for test shapes)."""
    cfg = dict(CONFIGS[name]) if name in CONFIGS else {}
    cfg.update(overrides)
    cfg.setdefault("bias", "none")
    cfg.setdefault("C", None)
    cfg["name"] = overrides.get("name", name)
    return cfg


def _seed(cfg, tensor, index=0):
    base = cfg.get("seed", 0)
    key = f"{cfg['name']}|{tensor}|{index}|{base}".encode()
    return zlib.crc32(key) & 0x7FFFFFFF


def _gen(cfg, tensor, index, device):
    g = torch.Generator(device=device)
    g.manual_seed(_seed(cfg, tensor, index))
    return g


def expert_bias(cfg):
    """Per-expert logit bias, float32 [E] on the CPU."""
    E = cfg["E"]
    kind = cfg.get("bias", "none")
    if kind == "none":
        return torch.zeros(E, dtype=torch.float32)
    g = _gen(cfg, "bias_perm", 0, "cpu")
    perm = torch.randperm(E, generator=g)
    if kind == "zipf":
        ranks = perm.to(torch.float64) + 1.0
        return (-2.2 * torch.log(ranks)).to(torch.float32)
    if kind == "hot":
        n_hot = int(round(0.16 * E))
        b = torch.zeros(E, dtype=torch.float64)
        b[perm[:n_hot]] = cfg.get("hot_bias", 4.0)
        return b.to(torch.float32)
    raise ValueError(f"unknown bias {kind!r}")


def make_logits(cfg, device="cpu"):
    N, E = cfg["N"], cfg["E"]
    g = _gen(cfg, "logits", 0, device)
    z = torch.randn(N, E, generator=g, device=device, dtype=torch.float32)
    return z + expert_bias(cfg).to(device)


def make_x(cfg, device="cpu"):
    g = _gen(cfg, "x", 0, device)
    z = torch.randn(cfg["N"], cfg["d"], generator=g, device=device,
                    dtype=torch.float32)
    return z.to(TORCH_DTYPE[cfg["act"]])


def expert_weights(cfg, e, device="cpu"):
    """(w_gate [ffn, d], w_up [ffn, d], w_down [d, ffn]) of expert e."""
    d, ffn = cfg["d"], cfg["ffn"]
    dt = TORCH_DTYPE[cfg["act"]]
    out = []
    for name, shape, fan_in in (("w_gate", (ffn, d), d), ("w_up", (ffn, d), d),
                                ("w_down", (d, ffn), ffn)):
        g = _gen(cfg, name, e, device)
        z = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
        out.append((z * (1.0 / math.sqrt(fan_in))).to(dt))
    return tuple(out)


def make_weights(cfg, device="cpu"):
    """All experts' weights: w_gate, w_up [E, ffn, d]; w_down [E, d, ffn]."""
    E, d, ffn = cfg["E"], cfg["d"], cfg["ffn"]
    dt = TORCH_DTYPE[cfg["act"]]
    wg = torch.empty(E, ffn, d, dtype=dt, device=device)
    wu = torch.empty(E, ffn, d, dtype=dt, device=device)
    wd = torch.empty(E, d, ffn, dtype=dt, device=device)
    for e in range(E):
        a, b, c = expert_weights(cfg, e, device)
        wg[e].copy_(a)
        wu[e].copy_(b)
        wd[e].copy_(c)
    return wg, wu, wd


def make_shared_weights(cfg, device="cpu", ffn_s=None):
    """The dense MLP of a Residual-MoE layer as one expert: w_gate, w_up
    [1, ffn_s, d] and w_down [1, d, ffn_s] (ffn_s defaults to the experts'
    width), N(0, std = 1/sqrt(fan_in)), activation type."""
    d = cfg["d"]
    ffn_s = ffn_s or cfg["ffn"]
    dt = TORCH_DTYPE[cfg["act"]]
    out = []
    for name, shape, fan_in in (("shared_gate", (1, ffn_s, d), d), ("shared_up", (1, ffn_s, d), d),
                                ("shared_down", (1, d, ffn_s), ffn_s)):
        g = _gen(cfg, name, 0, device)
        z = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
        out.append((z * (1.0 / math.sqrt(fan_in))).to(dt))
    return tuple(out)


def make_router(cfg, device="cpu"):
    """Router weights w_router [E, d], N(0, std = 1/sqrt(d)), activation type."""
    g = _gen(cfg, "w_router", 0, device)
    z = torch.randn(cfg["E"], cfg["d"], generator=g, device=device, dtype=torch.float32)
    return (z * (1.0 / math.sqrt(cfg["d"]))).to(TORCH_DTYPE[cfg["act"]])


def make_inputs(cfg, device="cpu", weights=True):
    """logits, x and (optionally) the three weight tensors of a config."""
    res = {"logits": make_logits(cfg, device), "x": make_x(cfg, device)}
    if weights:
        res["w_gate"], res["w_up"], res["w_down"] = make_weights(cfg, device)
    return res
