"""Seeded synthetic inputs for the block-scaled FP4 path.

This module only draws random tensors with the shapes and value distributions of
the workloads below.  It holds none of the quantisation arithmetic, so the HIP
library and the CPU oracle can both consume its bytes without sharing any of
the method's code.  Every generator is a pure function of its seed and sizes.

Large workloads are drawn on whatever device is passed (the GPU for benchmark
sizes); the bytes are identical for every consumer of one call, which is all
parity needs.  Reproducibility across devices is not promised: torch's CPU and
GPU generators are different streams.

Workloads (sizes are the defaults of each function):

* ``tiny_roundtrip`` - one 64x256 fp32 tensor X_r ~ N(0,1); X_t = X_r*(1+e),
  e ~ N(0, 1e-3).
* ``moe_expert_weights_layer`` - one layer of 64 experts of [2048x768] bf16
  weights ~ N(0, 0.02), 0.1% of entries x20; training copy
  X_t = bf16(X_r + N(0, 1e-3*|X_r|)).  48 such layers form the MoE-weights
  workload.
* ``activations`` - [32768 x 4096] bf16 Student-t(4) values with 8 fixed outlier
  channels x50; training copy perturbed by uniform relative noise of +-2^-8.
* ``kv_cache`` - one layer's K and V cache [32768 tokens x 8 heads x 128] bf16,
  K with 4 outlier channels per head x20, V ~ N(0,1); training copies perturbed by
  uniform relative noise of +-2^-8.  Quantized per token-head (blocks of 16 along
  head_dim).
* ``transpose_source`` - [8192 x 8192] bf16 ~ N(0,1).
* ``grouped_gemm_inputs`` - 32 experts with Zipf(1.1) token counts summing to
  16384; A = bf16 N(0,1) [tokens x 2048]; expert weights bf16 N(0,0.02)
  [32 x 768 x 2048] in [n][k] layout.
"""
from __future__ import annotations

import math

import torch

__all__ = [
    "tiny_roundtrip",
    "moe_expert_weights_layer",
    "activations",
    "kv_cache",
    "transpose_source",
    "zipf_counts",
    "group_offsets",
    "grouped_gemm_inputs",
    "random_nvfp4",
]


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(int(seed))
    return g


def tiny_roundtrip(seed: int = 1, rows: int = 64, cols: int = 256):
    """fp32 X_r ~ N(0,1) and X_t = X_r * (1 + e), e ~ N(0, 1e-3), on the CPU."""
    g = _gen(seed, "cpu")
    xr = torch.randn(rows, cols, generator=g, dtype=torch.float32)
    e = torch.randn(rows, cols, generator=g, dtype=torch.float32) * 1e-3
    xt = xr * (1.0 + e)
    return xr.contiguous(), xt.contiguous()


def moe_expert_weights_layer(layer: int, experts: int = 64, rows: int = 2048,
                             cols: int = 768, device="cpu", seed: int = 2):
    """One layer of MoE expert weights, rollout copy and training copy (bf16).

    X_r = bf16(w), w ~ N(0, 0.02) with a Bernoulli(0.001) mask of entries x20.
    X_t = bf16(X_r + z * 1e-3 * |X_r|), z ~ N(0,1).
    """
    g = _gen(seed * 1_000_003 + 7919 * int(layer), device)
    shape = (experts, rows, cols)
    w = torch.randn(shape, generator=g, device=device, dtype=torch.float32) * 0.02
    mask = torch.rand(shape, generator=g, device=device) < 1e-3
    w = torch.where(mask, w * 20.0, w)
    del mask
    xr = w.to(torch.bfloat16)
    del w
    xrf = xr.float()
    z = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    xt = (xrf + z * (1e-3 * xrf.abs())).to(torch.bfloat16)
    return xr.contiguous(), xt.contiguous()


def activations(tokens: int = 32768, hidden: int = 4096, device="cpu", seed: int = 3,
                outlier_channels: int = 8, outlier_scale: float = 50.0):
    """Student-t(4) activations with fixed outlier channels, rollout and training copies.

    t = z * sqrt(4 / c), c ~ chi^2_4 drawn as -2*ln(u1*u2), u in (0, 1].
    The training copy is bf16(X_r * (1 + u)), u ~ U(-2^-8, 2^-8).
    """
    g = _gen(seed, device)
    shape = (tokens, hidden)
    z = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    u1 = 1.0 - torch.rand(shape, generator=g, device=device, dtype=torch.float32)
    u2 = 1.0 - torch.rand(shape, generator=g, device=device, dtype=torch.float32)
    chi2 = -2.0 * torch.log(u1 * u2)
    del u1, u2
    t = z * torch.sqrt(4.0 / chi2)
    del z, chi2
    gc = _gen(seed + 17, "cpu")
    ch = torch.randperm(hidden, generator=gc)[:outlier_channels].to(device)
    t[:, ch] *= outlier_scale
    xr = t.to(torch.bfloat16)
    del t
    u = (torch.rand(shape, generator=g, device=device, dtype=torch.float32) * 2.0 - 1.0) * 2.0 ** -8
    xt = (xr.float() * (1.0 + u)).to(torch.bfloat16)
    return xr.contiguous(), xt.contiguous(), ch.cpu()


def kv_cache(tokens: int = 32768, heads: int = 8, head_dim: int = 128, device="cpu", seed: int = 6,
             outlier_channels: int = 4, outlier_scale: float = 20.0):
    """One layer's K and V cache [tokens][heads][head_dim] bf16, rollout and training
    copies.  K ~ N(0, 1) with `outlier_channels` fixed head_dim channels per head
    scaled x`outlier_scale` (keys concentrate magnitude in a few channels); V ~ N(0, 1).
    Training copies are bf16(X_r * (1 + u)), u ~ U(-2^-8, 2^-8), as for activations.
    Returns (k_r, k_t, v_r, v_t, outlier channel ids [heads, outlier_channels])."""
    g = _gen(seed, device)
    shape = (tokens, heads, head_dim)
    kr = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    gc = _gen(seed + 17, "cpu")
    ch = torch.stack([torch.randperm(head_dim, generator=gc)[:outlier_channels] for _ in range(heads)])
    for h in range(heads):
        kr[:, h, ch[h].to(device)] *= outlier_scale
    kr = kr.to(torch.bfloat16)
    vr = torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)

    def trainer_copy(x):
        u = (torch.rand(shape, generator=g, device=device, dtype=torch.float32) * 2.0 - 1.0) * 2.0 ** -8
        return (x.float() * (1.0 + u)).to(torch.bfloat16)

    kt = trainer_copy(kr)
    vt = trainer_copy(vr)
    return kr.contiguous(), kt.contiguous(), vr.contiguous(), vt.contiguous(), ch


def transpose_source(rows: int = 8192, cols: int = 8192, device="cpu", seed: int = 4):
    """bf16 N(0,1) matrix that is nearest-quantised before the transpose step."""
    g = _gen(seed, device)
    return torch.randn(rows, cols, generator=g, device=device,
                       dtype=torch.float32).to(torch.bfloat16).contiguous()


def zipf_counts(groups: int = 32, total: int = 16384, s: float = 1.1):
    """Deterministic Zipf(s) group sizes summing to ``total``.

    p_e is proportional to e^-s for e = 1..groups; counts are floor(total*p_e)
    plus one each for the largest fractional remainders (ties to the lower index).
    """
    w = [float(e) ** (-s) for e in range(1, groups + 1)]
    z = math.fsum(w)
    exact = [total * x / z for x in w]
    base = [int(math.floor(v)) for v in exact]
    rem = total - sum(base)
    order = sorted(range(groups), key=lambda i: (-(exact[i] - base[i]), i))
    for i in order[:rem]:
        base[i] += 1
    return base


def group_offsets(counts):
    off = [0]
    for c in counts:
        off.append(off[-1] + int(c))
    return torch.tensor(off, dtype=torch.int32)


def grouped_gemm_inputs(groups: int = 32, tokens: int = 16384, k: int = 2048, n: int = 768,
                        device="cpu", seed: int = 5, s: float = 1.1, counts=None):
    """Activations A [tokens x k] bf16 ~ N(0,1), expert weights [groups x n x k] bf16
    ~ N(0, 0.02) (k contiguous), and int32 group offsets [groups+1]."""
    if counts is None:
        counts = zipf_counts(groups, tokens, s)
    assert sum(counts) == tokens and len(counts) == groups
    g = _gen(seed, device)
    a = torch.randn(tokens, k, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
    w = (torch.randn(groups, n, k, generator=g, device=device, dtype=torch.float32) * 0.02
         ).to(torch.bfloat16)
    return a.contiguous(), w.contiguous(), group_offsets(counts)


def random_nvfp4(batch: int, rows: int, cols: int, seed: int = 11, device="cpu",
                 zero_block_frac: float = 0.0):
    """Uniformly random NVFP4 storage: any 4-bit code, E4M3 scale bytes drawn from
    the finite non-negative codes 0x00..0x7E, and a positive fp32 tensor scale.

    Used to exercise the transpose step on arbitrary stored tensors, including
    subnormal and zero block scales.
    """
    g = _gen(seed, device)
    codes = torch.randint(0, 256, (batch, rows, cols // 2), generator=g, device=device,
                          dtype=torch.int32).to(torch.uint8)
    scales = torch.randint(0, 0x7F, (batch, rows, cols // 16), generator=g, device=device,
                           dtype=torch.int32).to(torch.uint8)
    if zero_block_frac > 0:
        z = torch.rand((batch, rows, cols // 16), generator=g, device=device) < zero_block_frac
        scales = torch.where(z, torch.zeros_like(scales), scales)
    ts = (torch.rand((batch,), generator=g, device=device, dtype=torch.float32) + 0.5)
    return codes.contiguous(), scales.contiguous(), ts.contiguous()
