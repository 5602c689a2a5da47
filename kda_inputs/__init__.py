"""Seeded synthetic inputs for the KDA forward workloads.

This module is the ONLY code shared by the HIP-path tests/bench and the fp64
oracle: it draws the inputs and holds none of the method's arithmetic (no
decay, no delta rule, no conv, no normalisation of the conv prologue).  The
L2 normalisation of q and k below is part of the *input recipe* of the
non-conv workloads (q, k ~ N(0,1), then unit length per head), not the
method's own QK norm, which runs inside the conv prologue on raw inputs.

Draws use torch generators on the requested device, seeded per
(seed, tensor id, block) so that any 4096-token block (or decode step) can be
re-drawn on its own.  Values are drawn in fp32, shaped, then rounded
(round-to-nearest-even) to the stored dtype; consumers that need the oracle's
view upcast those stored values exactly.

Workloads, by name (shapes from the KDA deployment the pages describe: 32
linear-attention heads, head dim 128, kernel-4 conv, 8K pretraining context,
262,144 served context; decode batch 256):

  TINY          tiny fp32 prefill       B1 T64 H2 D16 C16, all fp32
  PREFILL       model-shaped prefill    B1 T8192 H32 D128 C64, bf16 q/k/v,
                                        fp32 g/beta
  CONV_PREFILL  prefill + conv prologue B8 T4096 H32 D128 C64, raw x over
                                        4096 channels
  DECODE        decode step             N256 H32 D128, fp32 state, bf16
                                        inputs, 1000 steps
  LONG          long-context prefill    B1 T262144 H32 D128 C64, slow
                                        forgetting
"""
from __future__ import annotations

import hashlib

import torch
import torch.nn.functional as F

BLOCK = 4096  # tokens per independently seeded block

SEED_BASE = 7400

TINY = "kda_prefill_tiny_fp32"
PREFILL = "kda_prefill_b1_t8192_h32_d128"
CONV_PREFILL = "kda_prefill_conv4_b8_t4096_h32_d128"
DECODE = "kda_decode_n256_h32_d128_x1000"
LONG = "kda_prefill_b1_t262144_h32_d128"

# each workload draws from its own seed
WORKLOADS = {
    TINY: dict(kind="prefill", seed=SEED_BASE + 0, B=1, T=64, H=2, Dk=16,
               Dv=16, chunk=16, qkv="f32", gate="f32", gate_kind="softplus",
               conv_width=0),
    PREFILL: dict(kind="prefill", seed=SEED_BASE + 1, B=1, T=8192, H=32,
                  Dk=128, Dv=128, chunk=64, qkv="bf16", gate="f32",
                  gate_kind="softplus", conv_width=0),
    CONV_PREFILL: dict(kind="prefill", seed=SEED_BASE + 2, B=8, T=4096, H=32,
                       Dk=128, Dv=128, chunk=64, qkv="bf16", gate="f32",
                       gate_kind="softplus", conv_width=4),
    DECODE: dict(kind="decode", seed=SEED_BASE + 3, N=256, H=32, Dk=128,
                 Dv=128, steps=1000, qkv="bf16", gate="bf16", state_std=0.1),
    LONG: dict(kind="prefill", seed=SEED_BASE + 4, B=1, T=262144, H=32,
               Dk=128, Dv=128, chunk=64, qkv="bf16", gate="f32",
               gate_kind="slow", conv_width=0),
}


def workload(name: str) -> dict:
    """The workload's parameters (a copy), with its name."""
    return dict(WORKLOADS[name], name=name)


_DT = {"f32": torch.float32, "bf16": torch.bfloat16}

# tensor ids (part of each draw's seed)
_ID = dict(q=1, k=2, v=3, g=4, beta=5, s0=6, xq=7, xk=8, xv=9, wq=10, wk=11,
           wv=12, state=13)


def torch_dtype(name: str) -> torch.dtype:
    return _DT[name]


def _seed_of(*parts) -> int:
    h = hashlib.blake2b(repr(parts).encode(), digest_size=8).digest()
    return int.from_bytes(h, "little") & ((1 << 63) - 1)


def _randn(shape, device, *parts) -> torch.Tensor:
    gen = torch.Generator(device=device)
    gen.manual_seed(_seed_of(*parts))
    return torch.randn(shape, generator=gen, device=device,
                       dtype=torch.float32)


def _unit(x: torch.Tensor) -> torch.Tensor:
    """Input recipe: scale each head vector (last dim) to unit length."""
    return x / x.norm(dim=-1, keepdim=True).clamp_min(1e-30)


def _gate(z: torch.Tensor, gate_kind: str) -> torch.Tensor:
    """Log-decay draws.  'softplus': g = -softplus(z), z ~ N(0,1).
    'slow': g = log1p(-0.002 * sigmoid(z)) so E[exp g] = 0.999 exactly
    (E[sigmoid(z)] = 1/2 by symmetry)."""
    if gate_kind == "softplus":
        return -F.softplus(z)
    if gate_kind == "slow":
        return torch.log1p(-0.002 * torch.sigmoid(z))
    raise ValueError(gate_kind)


def prefill_inputs(B, T, H, Dk, Dv, qkv="bf16", gate="f32",
                   gate_kind="softplus", conv_width=0, seed=SEED_BASE,
                   device="cpu", with_s0=False, s0_std=0.1,
                   gate_per_head=False, beta_max=1.0):
    """Draw one prefill batch.  Returns a dict with q,k,g [B,T,H,Dk],
    v [B,T,H,Dv], beta [B,T,H] (and s0 [B,H,Dk,Dv] fp32 if with_s0).
    With conv_width > 0 it also holds raw xq,xk [B,T,H*Dk], xv [B,T,H*Dv]
    (qkv dtype, N(0,1)) and fp32 taps wq,wk [H*Dk,W], wv [H*Dv,W] ~ N(0,1/4);
    q, k, v are then absent (the conv prologue makes them).
    gate_per_head: g is [B,T,H] (one log-decay per token-head, same
    distribution).  beta_max: beta = beta_max * sigmoid(z) (2.0 for the
    "negative eigenvalues" range (0,2))."""
    qdt, gdt = _DT[qkv], _DT[gate]
    out = {}

    def blocks(name, feat, fn, dtype):
        parts = []
        for b in range(B):
            for t0 in range(0, T, BLOCK):
                n = min(BLOCK, T - t0)
                z = _randn((n,) + feat, device, seed, _ID[name], b, t0 // BLOCK)
                parts.append(fn(z).to(dtype))
        return torch.cat(parts, 0).reshape((B, T) + feat)

    if conv_width:
        out["xq"] = blocks("xq", (H * Dk,), lambda z: z, qdt)
        out["xk"] = blocks("xk", (H * Dk,), lambda z: z, qdt)
        out["xv"] = blocks("xv", (H * Dv,), lambda z: z, qdt)
        for name, C in (("wq", H * Dk), ("wk", H * Dk), ("wv", H * Dv)):
            out[name] = 0.5 * _randn((C, conv_width), device, seed, _ID[name])
    else:
        out["q"] = blocks("q", (H, Dk), _unit, qdt)
        out["k"] = blocks("k", (H, Dk), _unit, qdt)
        out["v"] = blocks("v", (H, Dv), lambda z: z, qdt)
    out["g"] = blocks("g", (H,) if gate_per_head else (H, Dk),
                      lambda z: _gate(z, gate_kind), gdt)
    out["beta"] = blocks("beta", (H,),
                         lambda z: beta_max * torch.sigmoid(z), gdt)
    if with_s0:
        out["s0"] = s0_std * _randn((B, H, Dk, Dv), device, seed, _ID["s0"])
    return out


def workload_prefill_inputs(name: str, device="cpu", seed=None, **over):
    """The named prefill workload's inputs (fields in `over` replace the
    workload's own)."""
    c = workload(name)
    c.update(over)
    return prefill_inputs(c["B"], c["T"], c["H"], c["Dk"], c["Dv"],
                          qkv=c["qkv"], gate=c["gate"],
                          gate_kind=c["gate_kind"],
                          conv_width=c["conv_width"],
                          seed=c["seed"] if seed is None else seed,
                          device=device)


def decode_state(N, H, Dk, Dv, std=0.1, seed=WORKLOADS[DECODE]["seed"], device="cpu"):
    """Initial decode state, fp32 N(0, std^2) ('N(0,0.01)' read as variance
    0.01, std 0.1), layout [N,H,Dk,Dv]."""
    return std * _randn((N, H, Dk, Dv), device, seed, _ID["state"])


def decode_step_inputs(N, H, Dk, Dv, step, qkv="bf16", gate="bf16",
                       seed=WORKLOADS[DECODE]["seed"], device="cpu",
                       gate_per_head=False,
                       beta_max=1.0):
    """Fresh single-token inputs for decode step `step`, distributed as the
    tiny workload: q,k unit per head, v ~ N(0,1), g = -softplus(N(0,1)),
    beta = sigmoid(N(0,1))."""
    qdt, gdt = _DT[qkv], _DT[gate]
    r = lambda name, shape: _randn(shape, device, seed, _ID[name], "step",
                                   step)
    return dict(
        q=_unit(r("q", (N, H, Dk))).to(qdt),
        k=_unit(r("k", (N, H, Dk))).to(qdt),
        v=r("v", (N, H, Dv)).to(qdt),
        g=(-F.softplus(r("g", (N, H) if gate_per_head else (N, H, Dk)))
           ).to(gdt),
        beta=(beta_max * torch.sigmoid(r("beta", (N, H)))).to(gdt),
    )
