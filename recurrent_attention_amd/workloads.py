"""Seeded synthetic inputs shared by the GPU path's tests/bench and the oracle.

This module draws random numbers and nothing else: it holds none of the
recurrence's arithmetic.  Both sides of a parity check receive the very
tensors made here (the oracle widened to fp64 on the host).

Workloads (named by what they are, with their sizes):

=====================================  ======================================
name                                   contents
=====================================  ======================================
``linear_elu1_L64_d16_fp32``           1 x 1 head, L=64, d=16, fp32 N(0,1),
                                       phi = elu+1, normalised, A_t = 1, C=16
``linear_elu1_B4H8_L2048_d64``         B=4, H=8, L=2048, d=64, bf16
                                       N(0,1)/sqrt(d), elu+1, normalised, C=64
``retention_B2H16_L8192_d128``         B=2, H=16, L=8192, d=128, bf16,
                                       gamma_h = 1 - 2^(-5-3h/15), C=64
``gla_B1H16_L32768_d128``              B=1, H=16, L=32768, d=128, bf16,
                                       log alpha = logsigmoid(g)/16, g~N(0,1)
                                       per token/head/channel, C=64
``decode_retention_256x32_d128``       256 sequences x 32 heads, d=128, fp32
                                       S ~ N(0,1), one bf16 token per step,
                                       gamma = 0.97, 1000 steps
``scalar_gate_B1H16_L32768_d128``      as the GLA workload with one gate per
                                       token and head (log alpha =
                                       logsigmoid(g)/16, g ~ N(0,1) [B,H,L])
``delta_B16H16_L4096_d128``            delta rule: B=16, H=16, L=4096, d=128,
                                       bf16; q N(0,1)/sqrt(d), unit-norm k,
                                       v N(0,1), beta = sigmoid(N(0,1))
``gla_varlen_32seq_H16_d128``          32 packed sequences, lengths uniform
                                       in [1, 4096] (seed 7), H=16, d=128,
                                       bf16, GLA gates as above, C=64
=====================================  ======================================

Draw order for prefill workloads: one ``torch.Generator`` seeded with
``seed`` draws q, k, v (each ``randn([B,H,L,d])`` in fp32, scaled by 1/sqrt(d)
in fp32, then rounded to bf16 with round-to-nearest-even), then the gate
pre-activation g.  The decode workload draws S0, then the tokens step by
step.  A backward draws, from its own generator, dout like the tokens and
then dS_final ~ N(0,1).  Streams drawn on a CUDA device differ from CPU
streams (different generators); every run is self-consistent because the
oracle receives the same tensors.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

GATE_NONE, GATE_GAMMA, GATE_DIAG, GATE_SCALAR = 0, 1, 2, 3
PHI_IDENTITY, PHI_ELU1 = 0, 1


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    L: int
    dk: int
    dv: int
    dtype: torch.dtype
    gate_mode: int
    phi: int
    normalize: bool
    chunk: int
    scale_inputs: bool = True          # N(0,1)/sqrt(d) when True
    gamma: tuple = field(default=())   # per-head decays (GAMMA)
    steps: int = 0                     # decode workloads only

    @property
    def tokens(self) -> int:
        return self.B * self.L


def retention_gammas(H: int):
    """gamma_h = 1 - 2^(-5 - 3h/15): the retention workload's per-head decays."""
    return tuple(1.0 - 2.0 ** (-5.0 - 3.0 * h / 15.0) for h in range(H))


WORKLOADS = {
    w.name: w for w in [
        Workload("linear_elu1_L64_d16_fp32", 1, 1, 64, 16, 16, torch.float32,
                 GATE_NONE, PHI_ELU1, True, 16, scale_inputs=False),
        Workload("linear_elu1_B4H8_L2048_d64", 4, 8, 2048, 64, 64,
                 torch.bfloat16, GATE_NONE, PHI_ELU1, True, 64),
        Workload("retention_B2H16_L8192_d128", 2, 16, 8192, 128, 128,
                 torch.bfloat16, GATE_GAMMA, PHI_IDENTITY, False, 64,
                 gamma=retention_gammas(16)),
        Workload("gla_B1H16_L32768_d128", 1, 16, 32768, 128, 128,
                 torch.bfloat16, GATE_DIAG, PHI_IDENTITY, False, 64),
        Workload("scalar_gate_B1H16_L32768_d128", 1, 16, 32768, 128, 128,
                 torch.bfloat16, GATE_SCALAR, PHI_IDENTITY, False, 64),
        Workload("decode_retention_256x32_d128", 256, 32, 1, 128, 128,
                 torch.bfloat16, GATE_GAMMA, PHI_IDENTITY, False, 0,
                 gamma=(0.97,) * 32, steps=1000),
    ]
}

PREFILL_HEADLINE = "gla_B1H16_L32768_d128"
DECODE_HEADLINE = "decode_retention_256x32_d128"
VARLEN_HEADLINE = "gla_varlen_32seq_H16_d128"
DELTA_HEADLINE = "delta_B16H16_L4096_d128"
DELTA_SPEC = {"B": 16, "H": 16, "L": 4096, "d": 128}
VARLEN_SPEC = {"n": 32, "lo": 1, "hi": 4096, "seed": 7, "H": 16, "d": 128, "chunk": 64}


def varlen_lengths(n, lo, hi, seed):
    """Seeded sequence lengths: n integers uniform in [lo, hi]."""
    gen = generator(seed)
    return torch.randint(lo, hi + 1, (n,), generator=gen).tolist()


def generator(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _tokens(gen, shape, d, dtype, scale, device):
    x = torch.randn(shape, generator=gen, dtype=torch.float32, device=device)
    if scale:
        x = x * torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32, device=device)
    return x.to(dtype)


def prefill_inputs(B, H, L, dk, dv, dtype=torch.bfloat16, gate_mode=GATE_NONE,
                   seed=0, device="cpu", scale_inputs=True, gamma=None,
                   with_state=False, state_scale=1.0):
    """Seeded q, k, v [B,H,L,d] (+ gate, + optional S0/z0) as a dict."""
    gen = generator(seed, device)
    q = _tokens(gen, (B, H, L, dk), dk, dtype, scale_inputs, device)
    k = _tokens(gen, (B, H, L, dk), dk, dtype, scale_inputs, device)
    v = _tokens(gen, (B, H, L, dv), dv, dtype, scale_inputs, device)
    out = {"q": q, "k": k, "v": v, "gamma": None, "log_alpha": None}
    if gate_mode == GATE_GAMMA:
        out["gamma"] = torch.tensor(
            gamma if gamma is not None else retention_gammas(H),
            dtype=torch.float32)
    elif gate_mode == GATE_DIAG:
        g = torch.randn((B, H, L, dk), generator=gen, dtype=torch.float32,
                        device=device)
        # alpha = sigmoid(g)^(1/16), kept in log space
        out["log_alpha"] = torch.nn.functional.logsigmoid(g) / 16.0
    elif gate_mode == GATE_SCALAR:
        # one gate per token and head, drawn like the diagonal ones
        g = torch.randn((B, H, L), generator=gen, dtype=torch.float32, device=device)
        out["log_alpha"] = torch.nn.functional.logsigmoid(g) / 16.0
    if with_state:
        out["S0"] = state_scale * torch.randn((B, H, dk, dv), generator=gen,
                                              dtype=torch.float32, device=device)
        # z0 >= 1 keeps the normaliser away from zero
        out["z0"] = 1.0 + torch.randn((B, H, dk), generator=gen,
                                      dtype=torch.float32, device=device).abs()
    return out


def workload_inputs(name: str, seed: int = 0, device="cpu", L=None, B=None):
    """Inputs of a named prefill workload (optionally with L or B overridden)."""
    w = WORKLOADS[name]
    return prefill_inputs(B or w.B, w.H, L or w.L, w.dk, w.dv, w.dtype,
                          w.gate_mode, seed=seed, device=device,
                          scale_inputs=w.scale_inputs,
                          gamma=w.gamma if w.gate_mode == GATE_GAMMA else None)


def delta_inputs(B, H, L, dk, dv, dtype=torch.bfloat16, seed=0, device="cpu",
                 with_state=False):
    """Seeded inputs of the delta rule: q ~ N(0,1)/sqrt(d_k); k = a N(0,1)
    row scaled to unit norm (in fp32, then rounded to dtype); v ~ N(0,1);
    beta = sigmoid(N(0,1)) in fp32 [B,H,L]; S0 ~ N(0,1) when asked."""
    gen = generator(seed, device)
    q = _tokens(gen, (B, H, L, dk), dk, dtype, True, device)
    k = torch.randn((B, H, L, dk), generator=gen, dtype=torch.float32, device=device)
    k = (k / k.norm(dim=-1, keepdim=True)).to(dtype)
    v = torch.randn((B, H, L, dv), generator=gen, dtype=torch.float32, device=device).to(dtype)
    beta = torch.sigmoid(torch.randn((B, H, L), generator=gen, dtype=torch.float32, device=device))
    out = {"q": q, "k": k, "v": v, "beta": beta, "S0": None}
    if with_state:
        out["S0"] = torch.randn((B, H, dk, dv), generator=gen, dtype=torch.float32, device=device)
    return out


def backward_inputs(B, H, L, dk, dv, dtype=torch.bfloat16, seed=100, device="cpu",
                    scale_inputs=True, with_state_grad=True):
    """Seeded gradients for a prefill backward: dout [B,H,L,dv] drawn like the
    tokens, and dS_final ~ N(0,1) fp32 [B,H,dk,dv] when asked."""
    gen = generator(seed, device)
    dout = _tokens(gen, (B, H, L, dv), dv, dtype, scale_inputs, device)
    dS = None
    if with_state_grad:
        dS = torch.randn((B, H, dk, dv), generator=gen, dtype=torch.float32, device=device)
    return {"dout": dout, "dS_final": dS}


def decode_state(nseq, H, dk, dv, seed=0, device="cpu", with_z=False):
    """S0 ~ N(0,1) fp32 [nseq,H,dk,dv] (+ z0 = 1 + |N(0,1)| when asked)."""
    gen = generator(seed, device)
    S = torch.randn((nseq, H, dk, dv), generator=gen, dtype=torch.float32,
                    device=device)
    z = None
    if with_z:
        z = 1.0 + torch.randn((nseq, H, dk), generator=gen, dtype=torch.float32,
                              device=device).abs()
    return S, z


def decode_tokens(nseq, H, dk, dv, steps, seed=1, device="cpu",
                  dtype=torch.bfloat16, scale_inputs=True, gate=False):
    """Per-step tokens q, k, v [steps,nseq,H,d] (+ log-gates when asked)."""
    gen = generator(seed, device)
    q = _tokens(gen, (steps, nseq, H, dk), dk, dtype, scale_inputs, device)
    k = _tokens(gen, (steps, nseq, H, dk), dk, dtype, scale_inputs, device)
    v = _tokens(gen, (steps, nseq, H, dv), dv, dtype, scale_inputs, device)
    la = None
    if gate:
        g = torch.randn((steps, nseq, H, dk), generator=gen,
                        dtype=torch.float32, device=device)
        la = torch.nn.functional.logsigmoid(g) / 16.0
    return q, k, v, la
