"""Seeded synthetic inputs for the GDN recurrent decode step.

This module is shared by the tests, the smoke check and the benchmark.  It
holds only random draws and the distribution transforms that shape them; it
holds none of the step's arithmetic, and neither the HIP library nor the CPU
oracle imports it.  Both sides always consume the very same fp32 arrays (the
oracle receives host copies of whatever the GPU received), so the choice of
random generator affects how realistic a workload is, never parity.

Distributions (the workloads of "Kestrel_VLLM #24: GDN linear attention on
GPU", section 6, at vh=48, kh=16, kd=vd=128, dim=5120, ck=4):
  state S ~ N(0, 0.02)                       (sigma is a standard deviation)
  q, k   ~ N(0, 1), then scaled to unit L2 norm per key head; q additionally
           scaled by 1/sqrt(kd)
  v      ~ N(0, 1)
  g      = -softplus(z), beta = sigmoid(z'), z, z' ~ N(0, 1) per value head
  "alpha-uniform" variant: alpha ~ U[0.5, 1], g = ln(alpha), beta ~ U(0, 1)
Front end: x ~ N(0, 1) [B][dim]; Wa, Wb ~ N(0, 0.01) [vh][dim]; raw conv
input and initial history ~ N(0, 1); conv_w, A_log, dt_bias ~ N(0, 0.5).
Projections (in_proj_qkv, in_proj_z, out_proj) ~ N(0, 0.02); gated-norm
weight ~ 1 + N(0, 0.1).
The transforms run in float64 and are rounded once to fp32.
"""
from __future__ import annotations

import math

import torch

DIMS128 = (48, 16, 128, 128)   # vh, kh, kd, vd
DIMS64 = (96, 32, 64, 64)
FE_DIM = 5120
CONV_K = 4


def conv_dim_of(dims):
    vh, kh, kd, vd = dims
    return 2 * kh * kd + vh * vd


def make_gen(seed: int, device) -> torch.Generator:
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    return gen


def _normal(gen, shape, std, device):
    t = torch.randn(shape, generator=gen, dtype=torch.float32, device=device)
    if std != 1.0:
        t.mul_(std)
    return t


def state(gen, n_units, dims, std=0.02, device="cpu"):
    """Initial state S [N][vh][kd][vd] ~ N(0, std)."""
    vh, kh, kd, vd = dims
    return _normal(gen, (n_units, vh, kd, vd), std, device)


def _unit_rows(z64):
    return z64 / torch.linalg.vector_norm(z64, dim=-1, keepdim=True)


def step_inputs(gen, n_units, dims, M=1, gate="softplus", device="cpu"):
    """q, k [M][N][kh][kd]; v [M][N][vh][vd]; g, beta [M][N][vh] (fp32).

    gate="softplus": g = -softplus(N(0,1)), beta = sigmoid(N(0,1)).
    gate="alpha-uniform": alpha ~ U[0.5, 1], g = ln(alpha), beta ~ U(0, 1).
    Draw order: q, k, v, then the gate draws, then the beta draws.
    """
    vh, kh, kd, vd = dims
    q = torch.randn((M, n_units, kh, kd), generator=gen, dtype=torch.float64, device=device)
    k = torch.randn((M, n_units, kh, kd), generator=gen, dtype=torch.float64, device=device)
    q = (_unit_rows(q) * (1.0 / math.sqrt(kd))).float()
    k = _unit_rows(k).float()
    v = _normal(gen, (M, n_units, vh, vd), 1.0, device)
    if gate == "softplus":
        zg = torch.randn((M, n_units, vh), generator=gen, dtype=torch.float64, device=device)
        zb = torch.randn((M, n_units, vh), generator=gen, dtype=torch.float64, device=device)
        g = (-torch.nn.functional.softplus(zg)).float()
        beta = torch.sigmoid(zb).float()
    elif gate == "alpha-uniform":
        a = torch.rand((M, n_units, vh), generator=gen, dtype=torch.float64, device=device)
        g = torch.log(0.5 + 0.5 * a).float()
        beta = torch.rand((M, n_units, vh), generator=gen, dtype=torch.float64, device=device).float()
    else:
        raise ValueError(gate)
    return dict(q=q.contiguous(), k=k.contiguous(), v=v, g=g.contiguous(),
                beta=beta.contiguous())


def frontend_weights(gen, dims, dim=FE_DIM, ck=CONV_K, device="cpu"):
    """Wa, Wb [vh][dim] ~ N(0, 0.01); A_log, dt_bias [vh] and conv_w
    [conv_dim][ck] ~ N(0, 0.5)."""
    vh = dims[0]
    cd = conv_dim_of(dims)
    return dict(
        Wa=_normal(gen, (vh, dim), 0.01, device),
        Wb=_normal(gen, (vh, dim), 0.01, device),
        A_log=_normal(gen, (vh,), 0.5, device),
        dt_bias=_normal(gen, (vh,), 0.5, device),
        conv_w=_normal(gen, (cd, ck), 0.5, device),
    )


def proj_weights(gen, dims, dim=FE_DIM, std=0.02, device="cpu"):
    """Projection weights of one layer, all ~ N(0, std): W_qkv [conv_dim][dim]
    (conv input), W_z [vh*vd][dim] (output gate), W_out [dim][vh*vd]; and the
    gated-norm weight norm_w [vd] ~ 1 + N(0, 0.1)."""
    vh, kh, kd, vd = dims
    cd = conv_dim_of(dims)
    return dict(
        W_qkv=_normal(gen, (cd, dim), std, device),
        W_z=_normal(gen, (vh * vd, dim), std, device),
        W_out=_normal(gen, (dim, vh * vd), std, device),
        norm_w=1.0 + _normal(gen, (vd,), 0.1, device),
    )


def q4_weights(gen, R, C, std=0.02, device="cpu"):
    """A random 4-bit weight matrix [R][C] in the source format: q uint8
    [R][C/2] (every byte value equally likely, so every 4-bit value -8..7 in
    either nibble) and scale float16 [R][C/32], drawn uniform in
    [0.5, 1.5] x std / 4.61 (4.61 ~ the spread of a uniform 4-bit value), so
    the decoded weights have about the spread of proj_weights."""
    q = torch.randint(0, 256, (R, C // 2), generator=gen, dtype=torch.int32, device=device)
    u = torch.rand((R, C // 32), generator=gen, dtype=torch.float32, device=device)
    return q.to(torch.uint8), ((0.5 + u) * (std / 4.61)).to(torch.float16)


def proj_weights_q4(gen, dims, dim=FE_DIM, std=0.02, device="cpu"):
    """proj_weights with the three large matrices as 4-bit weights: dict of
    (q, scale) pairs for W_qkv, W_z, W_out, and the f32 norm_w."""
    vh, kh, kd, vd = dims
    cd = conv_dim_of(dims)
    return dict(
        W_qkv=q4_weights(gen, cd, dim, std, device),
        W_z=q4_weights(gen, vh * vd, dim, std, device),
        W_out=q4_weights(gen, dim, vh * vd, std, device),
        norm_w=1.0 + _normal(gen, (vd,), 0.1, device),
    )


def frontend_inputs(gen, B, dims, T=1, dim=FE_DIM, ck=CONV_K, device="cpu"):
    """x [T][B][dim] ~ N(0,1); raw conv input xc_raw [T][B][conv_dim] ~ N(0,1);
    initial history hist [B][ck-1][conv_dim] ~ N(0,1)."""
    cd = conv_dim_of(dims)
    return dict(
        x=_normal(gen, (T, B, dim), 1.0, device),
        xc_raw=_normal(gen, (T, B, cd), 1.0, device),
        hist=_normal(gen, (B, ck - 1, cd), 1.0, device),
    )


# The benchmarked workloads, with their sizes.  "units" = sequences x layers.
WORKLOADS = {
    0: dict(name="single sequence, 1 layer, 64 sequential decode steps",
            seqs=1, layers=1, dims=DIMS128, steps=64, gate="softplus", seed=0),
    1: dict(name="batched decode, 64 sequences x 48 layers, one step",
            seqs=64, layers=48, dims=DIMS128, steps=100, gate="softplus", seed=1),
    2: dict(name="speculative verify, 32 sequences x 48 layers, M=8 drafts",
            seqs=32, layers=48, dims=DIMS128, M=8, gate="softplus", seed=2),
    3: dict(name="front end + step, 128 sequences x 1 layer, 32 steps",
            seqs=128, layers=1, dims=DIMS128, steps=32, gate=None, seed=3),
    4: dict(name="large batch, 512 sequences x 8 layers, 50 steps",
            seqs=512, layers=8, dims=DIMS128, steps=50, gate="alpha-uniform", seed=4),
    5: dict(name="large batch kd=vd=64, 512 sequences x 8 layers, 50 steps",
            seqs=512, layers=8, dims=DIMS64, steps=50, gate="alpha-uniform", seed=5),
    6: dict(name="verify with front end, 128 sequences x 1 layer, M=8 drafts",
            seqs=128, layers=1, dims=DIMS128, M=8, gate=None, seed=6),
    7: dict(name="batched decode with gated RMSNorm output, 64 sequences x 48 layers",
            seqs=64, layers=48, dims=DIMS128, steps=100, gate="softplus", seed=7, gated=True),
    8: dict(name="whole-layer decode with f32 projections, 1 sequence x 8 layers",
            seqs=1, layers=8, dims=DIMS128, gate=None, seed=8),
    9: dict(name="whole-layer decode with f32 projections, 64 sequences x 8 layers",
            seqs=64, layers=8, dims=DIMS128, gate=None, seed=9),
    10: dict(name="whole-layer speculative verify with f32 projections, 1 sequence x 8 layers, "
                  "M=8 drafts", seqs=1, layers=8, dims=DIMS128, M=8, gate=None, seed=10),
    11: dict(name="whole-layer decode with 4-bit projections, 1 sequence x 8 layers",
             seqs=1, layers=8, dims=DIMS128, gate=None, seed=11, q4=True),
    12: dict(name="whole-layer speculative verify with 4-bit projections, 1 sequence x 8 "
                  "layers, M=8 drafts", seqs=1, layers=8, dims=DIMS128, M=8, gate=None, seed=12,
             q4=True),
}
