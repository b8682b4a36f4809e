"""Seeded synthetic inputs for the selective-SSM scan workloads.

This module only draws numbers; it holds none of the scan's arithmetic.  Both
the fp64 oracle (``oracle/``) and the HIP path receive the tensors it returns,
so the two sides always read identical stored values.

Recipe (one generator for every workload, ``torch.Generator`` seeded with the
workload index unless a seed is given):

* draw order, all fp32 normal draws: ``u``, ``delta_raw``, ``z`` ~ N(0,1) over
  (B,L,D); ``B``, ``C`` ~ N(0,1) over (B,L,N); ``D`` ~ N(0,1) over (D); then
  ``dt`` = exp(U[ln 1e-3, ln 1e-1]) over (D);
* ``delta_bias`` = log(expm1(dt)), the inverse of softplus, so that
  softplus(delta_bias) = dt, a per-channel step size between 1e-3 and 1e-1;
* ``A[d, n] = -(n + 1)`` (real, diagonal, negative), fp32;
* bf16 workloads round u, delta_raw, z, B, C to bf16 (round-to-nearest-even)
  right after drawing; A, D, delta_bias and states stay fp32;
* large tensors are drawn in blocks of ``_BLOCK`` elements along their
  flattened order and converted block by block, so that host memory stays
  bounded; the block size is part of the recipe.

The pages' workloads are Mamba language models trained on text corpora,
million-length DNA and synthetic recall tasks (Mamba paper, "Sonuçlar" section
of the reading guide).  No dataset or checkpoint is used here: the shapes are
the layer shapes listed in ``WORKLOADS`` and Gaussian draws stand in for the
outputs of the input projections that feed the scan.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import torch

_BLOCK = 1 << 26  # elements per draw block


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seqlen: int
    dim: int
    dstate: int
    io_dtype: torch.dtype
    kind: str  # "fwd", "decode", "fwd+bwd"
    steps: int = 1  # decode steps
    outputs: tuple = field(default=("y",))


WORKLOADS = {
    0: Workload("tiny-fp32-fwd", 1, 64, 32, 4, torch.float32, "fwd", outputs=("y", "h_final")),
    1: Workload("mamba-370m-layer-fwd", 8, 2048, 2048, 16, torch.float32, "fwd",
                outputs=("y", "h_final")),
    2: Workload("mamba-2.8b-layer-fwd", 4, 4096, 5120, 16, torch.bfloat16, "fwd", outputs=("y",)),
    3: Workload("decode-state-update", 256, 1, 5120, 16, torch.bfloat16, "decode", steps=64,
                outputs=("y", "state")),
    4: Workload("million-length-fwd-bwd", 1, 1 << 20, 1024, 16, torch.bfloat16, "fwd+bwd",
                outputs=("y", "chunk_states", "du", "ddelta", "dA", "dB", "dC", "dD", "dz")),
    # the one scan length the pages state (a 32K context), at the Mamba-2.8b width
    5: Workload("mamba-2.8b-32k-fwd", 1, 32768, 5120, 16, torch.bfloat16, "fwd", outputs=("y",)),
}


def _gen(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal(gen: torch.Generator, shape, dtype=torch.float32, device="cpu", std: float = 1.0):
    """N(0, std^2) draws in fp32, converted to ``dtype`` block by block."""
    numel = 1
    for s in shape:
        numel *= int(s)
    out = torch.empty(numel, dtype=dtype, device=device)
    for start in range(0, numel, _BLOCK):
        n = min(_BLOCK, numel - start)
        blk = torch.randn(n, generator=gen, dtype=torch.float32, device=device)
        if std != 1.0:
            blk.mul_(std)
        out[start:start + n] = blk.to(dtype)
    return out.view(*shape)


def log_uniform(gen: torch.Generator, shape, lo: float, hi: float, device="cpu"):
    """exp(U[ln lo, ln hi]) in fp32."""
    r = torch.rand(*shape, generator=gen, dtype=torch.float32, device=device)
    return torch.exp(r * (math.log(hi) - math.log(lo)) + math.log(lo))


def inverse_softplus(x: torch.Tensor) -> torch.Tensor:
    """log(expm1(x)), computed in fp64 then rounded to fp32 (input recipe only)."""
    return torch.log(torch.expm1(x.double())).float()


def state_space_A(dim: int, dstate: int, device="cpu") -> torch.Tensor:
    n = torch.arange(1, dstate + 1, dtype=torch.float32, device=device)
    return (-n).unsqueeze(0).expand(dim, dstate).contiguous()


def scan_inputs(batch: int, seqlen: int, dim: int, dstate: int, io_dtype=torch.float32,
                seed: int = 0, device="cpu", with_z: bool = True, with_D: bool = True,
                with_bias: bool = True):
    """Inputs of one forward scan, drawn in the recipe's order.

    Returns a dict with u, delta (raw, before bias and softplus), z, B, C in
    ``io_dtype`` and A, D, delta_bias in fp32.  Optional parts that are
    switched off are still drawn (so the other tensors do not change) and
    returned as ``None``.
    """
    g = _gen(seed, device)
    shp = (batch, seqlen, dim)
    u = normal(g, shp, io_dtype, device)
    delta = normal(g, shp, io_dtype, device)
    z = normal(g, shp, io_dtype, device)
    Bm = normal(g, (batch, seqlen, dstate), io_dtype, device)
    Cm = normal(g, (batch, seqlen, dstate), io_dtype, device)
    Dskip = normal(g, (dim,), torch.float32, device)
    dt = log_uniform(g, (dim,), 1e-3, 1e-1, device)
    bias = inverse_softplus(dt)
    return dict(u=u, delta=delta, A=state_space_A(dim, dstate, device), B=Bm, C=Cm,
                D=Dskip if with_D else None, z=z if with_z else None,
                delta_bias=bias if with_bias else None, delta_softplus=True)


def cotangent(like: torch.Tensor, seed: int, device=None) -> torch.Tensor:
    """dy ~ N(0,1) with ``like``'s shape and dtype, from its own seeded stream."""
    g = _gen(seed + 1_000_003, device or like.device)
    return normal(g, like.shape, like.dtype, device or like.device)


def decode_inputs(batch: int, dim: int, dstate: int, steps: int, io_dtype=torch.bfloat16,
                  seed: int = 3, device="cpu", state_std: float = 0.1):
    """Initial fp32 state (B,D,N) ~ N(0, state_std^2) and per-step token inputs.

    Draw order: state, then u, delta_raw, z over (steps,B,D), B, C over
    (steps,B,N), D over (D), dt over (D).
    """
    g = _gen(seed, device)
    state = normal(g, (batch, dim, dstate), torch.float32, device, std=state_std)
    shp = (steps, batch, dim)
    u = normal(g, shp, io_dtype, device)
    delta = normal(g, shp, io_dtype, device)
    z = normal(g, shp, io_dtype, device)
    Bm = normal(g, (steps, batch, dstate), io_dtype, device)
    Cm = normal(g, (steps, batch, dstate), io_dtype, device)
    Dskip = normal(g, (dim,), torch.float32, device)
    dt = log_uniform(g, (dim,), 1e-3, 1e-1, device)
    return dict(state=state, u=u, delta=delta, A=state_space_A(dim, dstate, device), B=Bm,
                C=Cm, D=Dskip, z=z, delta_bias=inverse_softplus(dt), delta_softplus=True)


def conv_inputs(dim: int, width: int = 4, seed: int = 0, device="cpu", with_bias: bool = True):
    """Taps (dim, width) ~ N(0, 0.5^2) and bias (dim) ~ N(0, 0.3^2), fp32, of the
    causal depthwise convolution in front of the scan (drawn in that order from
    their own generator, seed + 2,000,003)."""
    g = _gen(seed + 2_000_003, device)
    w = normal(g, (dim, width), torch.float32, device, std=0.5)
    b = normal(g, (dim,), torch.float32, device, std=0.3)
    return w, (b if with_bias else None)


def workload_inputs(index: int, device="cpu", seed: Optional[int] = None):
    w = WORKLOADS[index]
    s = index if seed is None else seed
    if w.kind == "decode":
        return decode_inputs(w.batch, w.dim, w.dstate, w.steps, w.io_dtype, s, device)
    return scan_inputs(w.batch, w.seqlen, w.dim, w.dstate, w.io_dtype, s, device)


def algorithmic_bytes_fwd(batch, seqlen, dim, dstate, io_bytes, *, with_z=True, with_D=True,
                          with_bias=True, h0=False, h_final=False, chunk_states_bytes=0):
    """Bytes a forward scan must move: every input read once, every output written once."""
    bld = batch * seqlen * dim
    bln = batch * seqlen * dstate
    total = bld * io_bytes * (2 + (1 if with_z else 0))  # u, delta, z
    total += bld * io_bytes  # y
    total += 2 * bln * io_bytes  # B, C
    total += dim * dstate * 4  # A
    total += dim * 4 * ((1 if with_D else 0) + (1 if with_bias else 0))
    total += batch * dim * dstate * 4 * ((1 if h0 else 0) + (1 if h_final else 0))
    return total + chunk_states_bytes


def algorithmic_bytes_decode(batch, dim, dstate, io_bytes):
    """Bytes of one decode step: state in and out, token inputs, parameters, y."""
    bd = batch * dim
    return (2 * bd * dstate * 4 + 3 * bd * io_bytes + 2 * batch * dstate * io_bytes
            + dim * dstate * 4 + 2 * dim * 4 + bd * io_bytes)


def algorithmic_bytes_bwd(batch, seqlen, dim, dstate, io_bytes, chunk_len=32):
    """Bytes a backward must move: u, delta, z, dy in and du, ddelta, dz out
    (B,L,D); B, C in and dB, dC out (B,L,N); the chunk-boundary states in; A,
    D, bias in and dA, dD, dbias out."""
    K = -(-seqlen // chunk_len)
    return (7 * batch * seqlen * dim * io_bytes + 4 * batch * seqlen * dstate * io_bytes
            + batch * K * dstate * dim * 4 + dim * dstate * 4 * 2 + dim * 4 * 4)
