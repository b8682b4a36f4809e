"""Torch-facing wrappers of the C ABI: shape/dtype/device checks, output and
workspace allocation with ``torch.empty``, and the call on the current stream.
Every step of the scan itself runs in the HIP library; nothing here computes.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import _lib

_IO = {torch.float32: _lib.SSM_F32, torch.bfloat16: _lib.SSM_BF16}


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _need(name, t, shape, dtype, device, optional=False):
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _io_code(u: torch.Tensor) -> int:
    if u.dtype not in _IO:
        raise TypeError(f"io dtype must be float32 or bfloat16, got {u.dtype}")
    return _IO[u.dtype]


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def chunk_len() -> int:
    return int(_lib.load().ssm_scan_chunk_len())


def scan_fwd_plan(batch, seqlen, dim, dstate, dtype=torch.float32, zoh=False, reverse=False,
                  per_token=False, accumulate=False, conv_width=0) -> dict:
    """How the forward would run these sizes on the current device (a host
    query, nothing is launched): ``kernel`` ("all-purpose" or
    "wave-specialised"), ``tile_channels``, ``segments``, ``segment_len`` and
    ``first_pass_len`` (steps per piece of a split's first pass)."""
    if dtype not in _IO:
        raise TypeError(f"io dtype must be float32 or bfloat16, got {dtype}")
    lib = _lib.load()
    flags = ((_lib.FLAG_ZOH if zoh else 0) | (_lib.FLAG_REVERSE if reverse else 0)
             | (_lib.FLAG_DELTA_PER_TOKEN if per_token else 0)
             | (_lib.FLAG_ACCUMULATE if accumulate else 0))
    plan = _lib.FwdPlan()
    _lib.check(lib.ssm_scan_fwd_plan(batch, seqlen, dim, dstate, _IO[dtype], flags, conv_width,
                                     plan))
    return {"kernel": ("all-purpose", "wave-specialised")[plan.kernel],
            "tile_channels": int(plan.tile_channels), "segments": int(plan.segments),
            "segment_len": int(plan.segment_len), "first_pass_len": int(plan.first_pass_len)}


def _flags(delta, u, zoh=False, reverse=False, accumulate=False):
    f = (_lib.FLAG_ZOH if zoh else 0) | (_lib.FLAG_REVERSE if reverse else 0)
    if accumulate:
        f |= _lib.FLAG_ACCUMULATE
    if isinstance(delta, torch.Tensor) and delta.dim() == 2:
        f |= _lib.FLAG_DELTA_PER_TOKEN
    return f


def _check_common(u, delta, A, B, C, D, z, delta_bias, h0):
    if not isinstance(u, torch.Tensor) or u.dim() != 3:
        raise ValueError("u must be a (batch, seqlen, dim) tensor")
    if not isinstance(A, torch.Tensor) or A.dim() != 2:
        raise ValueError("A must be a (dim, dstate) tensor")
    Bsz, L, Dm = u.shape
    N = A.shape[1]
    dev, io = u.device, u.dtype
    if dev.type != "cuda":
        raise ValueError(f"tensors must be on a GPU device, got {dev}")
    _io_code(u)
    _need("u", u, (Bsz, L, Dm), io, dev)
    if isinstance(delta, torch.Tensor) and delta.dim() == 2:  # one step size per token
        _need("delta", delta, (Bsz, L), io, dev)
    else:
        _need("delta", delta, (Bsz, L, Dm), io, dev)
    _need("A", A, (Dm, N), torch.float32, dev)
    _need("B", B, (Bsz, L, N), io, dev)
    _need("C", C, (Bsz, L, N), io, dev)
    _need("D", D, (Dm,), torch.float32, dev, optional=True)
    _need("z", z, (Bsz, L, Dm), io, dev, optional=True)
    _need("delta_bias", delta_bias, (Dm,), torch.float32, dev, optional=True)
    _need("h0", h0, (Bsz, Dm, N), torch.float32, dev, optional=True)
    return Bsz, L, Dm, N


def scan_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True, h0=None,
             return_final_state=False, save_chunk_states=False, zoh=False, reverse=False,
             out=None):
    """Forward selective scan.  Returns (y, h_final or None, chunk_states or None);
    chunk_states is (batch, K, dstate, dim) with K = ceil(seqlen / chunk_len()).

    Options: ``zoh`` uses the exact zero-order-hold input term; ``reverse``
    scans from the last step to the first; a (batch, seqlen) ``delta`` is one
    step size per token; ``out`` (a tensor like u) receives y += result."""
    Bsz, L, Dm, N = _check_common(u, delta, A, B, C, D, z, delta_bias, h0)
    lib = _lib.load()
    io = _io_code(u)
    dev = u.device
    if out is not None:
        _need("out", out, (Bsz, L, Dm), u.dtype, dev)
        y = out
    else:
        y = torch.empty_like(u)
    flags = _flags(delta, u, zoh, reverse, accumulate=out is not None)
    hf = torch.empty((Bsz, Dm, N), dtype=torch.float32, device=dev) if return_final_state else None
    cs = None
    if save_chunk_states:
        K = -(-L // chunk_len())
        cs = torch.empty((Bsz, K, N, Dm), dtype=torch.float32, device=dev)
    wsb = int(lib.ssm_scan_fwd_workspace_bytes(Bsz, L, Dm, N, io))
    if wsb < 0:
        raise ValueError("invalid sizes for the forward workspace query")
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev) if wsb > 0 else None
    with torch.cuda.device(dev):
        st = lib.ssm_scan_fwd_ex(Bsz, L, Dm, N, io, _ptr(u), _ptr(delta), _ptr(A), _ptr(B),
                                 _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
                                 int(bool(delta_softplus)), _ptr(h0), _ptr(hf), _ptr(y), _ptr(cs),
                                 _ptr(ws), wsb, _stream(dev), flags)
    _lib.check(st)
    return y, hf, cs


def scan_bwd(u, delta, A, B, C, D, z, delta_bias, delta_softplus, h0, chunk_states, dy,
             dh_final=None, want_ddelta_bias=True, want_dh0=True, zoh=False, reverse=False):
    """Backward of scan_fwd (same options; ddelta has delta's shape).  Returns a
    dict: du, ddelta, dA, dB, dC, dD, dz, ddelta_bias, dh0."""
    Bsz, L, Dm, N = _check_common(u, delta, A, B, C, D, z, delta_bias, h0)
    lib = _lib.load()
    io = _io_code(u)
    dev = u.device
    K = -(-L // chunk_len())
    _need("chunk_states", chunk_states, (Bsz, K, N, Dm), torch.float32, dev)
    _need("dy", dy, (Bsz, L, Dm), u.dtype, dev)
    _need("dh_final", dh_final, (Bsz, Dm, N), torch.float32, dev, optional=True)
    f32 = dict(dtype=torch.float32, device=dev)
    g = dict(du=torch.empty_like(u), ddelta=torch.empty_like(delta), dA=torch.empty((Dm, N), **f32),
             dB=torch.empty_like(B), dC=torch.empty_like(C),
             dD=torch.empty((Dm,), **f32) if D is not None else None,
             dz=torch.empty_like(u) if z is not None else None,
             ddelta_bias=torch.empty((Dm,), **f32) if (delta_bias is not None and want_ddelta_bias)
             else None,
             dh0=torch.empty((Bsz, Dm, N), **f32) if want_dh0 else None)
    wsb = int(lib.ssm_scan_bwd_workspace_bytes(Bsz, L, Dm, N, io))
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        st = lib.ssm_scan_bwd_ex(Bsz, L, Dm, N, io, _ptr(u), _ptr(delta), _ptr(A), _ptr(B),
                                 _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
                                 int(bool(delta_softplus)), _ptr(h0), _ptr(chunk_states), _ptr(dy),
                                 _ptr(dh_final), _ptr(g["du"]), _ptr(g["ddelta"]), _ptr(g["dA"]),
                                 _ptr(g["dB"]), _ptr(g["dC"]), _ptr(g["dD"]), _ptr(g["dz"]),
                                 _ptr(g["ddelta_bias"]), _ptr(g["dh0"]), _ptr(ws), wsb,
                                 _stream(dev), _flags(delta, u, zoh, reverse))
    _lib.check(st)
    return g


def _check_conv(x, conv_w, conv_b, dev):
    if not isinstance(conv_w, torch.Tensor) or conv_w.dim() != 2:
        raise ValueError("conv_w must be a (dim, width) tensor")
    Dm, K = conv_w.shape
    if not 1 <= K <= 4:
        raise ValueError(f"convolution width {K} not in 1..4")
    _need("conv_w", conv_w, (Dm, K), torch.float32, dev)
    _need("conv_b", conv_b, (Dm,), torch.float32, dev, optional=True)
    return K


def scan_fwd_conv(x, conv_w, conv_b, delta, A, B, C, D=None, z=None, delta_bias=None,
                  delta_softplus=True, h0=None, return_final_state=False, save_chunk_states=False,
                  zoh=False, out=None):
    """The scan fed by the fused causal depthwise convolution:
    u = silu(conv_b + sum_k conv_w[:, k] x[t - (K-1) + k]), then scan_fwd on u
    (u is never written to memory).  Returns (y, h_final or None, chunk_states or None)."""
    Bsz, L, Dm, N = _check_common(x, delta, A, B, C, D, z, delta_bias, h0)
    K = _check_conv(x, conv_w, conv_b, x.device)
    lib = _lib.load()
    io = _io_code(x)
    dev = x.device
    if out is not None:
        _need("out", out, (Bsz, L, Dm), x.dtype, dev)
        y = out
    else:
        y = torch.empty_like(x)
    flags = _flags(delta, x, zoh, False, accumulate=out is not None)
    hf = torch.empty((Bsz, Dm, N), dtype=torch.float32, device=dev) if return_final_state else None
    cs = None
    if save_chunk_states:
        cs = torch.empty((Bsz, -(-L // chunk_len()), N, Dm), dtype=torch.float32, device=dev)
    wsb = int(lib.ssm_scan_fwd_workspace_bytes(Bsz, L, Dm, N, io))
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev) if wsb > 0 else None
    with torch.cuda.device(dev):
        st = lib.ssm_scan_fwd_conv(Bsz, L, Dm, N, io, _ptr(x), _ptr(conv_w), _ptr(conv_b), K,
                                   _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                   _ptr(delta_bias), int(bool(delta_softplus)), _ptr(h0), _ptr(hf),
                                   _ptr(y), _ptr(cs), _ptr(ws), wsb, _stream(dev), flags)
    _lib.check(st)
    return y, hf, cs


def scan_bwd_conv(x, conv_w, conv_b, delta, A, B, C, D, z, delta_bias, delta_softplus, h0,
                  chunk_states, dy, dh_final=None, want_ddelta_bias=True, want_dh0=True, zoh=False):
    """Backward of scan_fwd_conv.  Returns a dict: dx, dconv_w, dconv_b, ddelta, dA, dB, dC,
    dD, dz, ddelta_bias, dh0."""
    Bsz, L, Dm, N = _check_common(x, delta, A, B, C, D, z, delta_bias, h0)
    K = _check_conv(x, conv_w, conv_b, x.device)
    lib = _lib.load()
    io = _io_code(x)
    dev = x.device
    _need("chunk_states", chunk_states, (Bsz, -(-L // chunk_len()), N, Dm), torch.float32, dev)
    _need("dy", dy, (Bsz, L, Dm), x.dtype, dev)
    _need("dh_final", dh_final, (Bsz, Dm, N), torch.float32, dev, optional=True)
    f32 = dict(dtype=torch.float32, device=dev)
    g = dict(dx=torch.empty_like(x), dconv_w=torch.empty((Dm, K), **f32),
             dconv_b=torch.empty((Dm,), **f32) if conv_b is not None else None,
             ddelta=torch.empty_like(delta), dA=torch.empty((Dm, N), **f32),
             dB=torch.empty_like(B), dC=torch.empty_like(C),
             dD=torch.empty((Dm,), **f32) if D is not None else None,
             dz=torch.empty_like(x) if z is not None else None,
             ddelta_bias=torch.empty((Dm,), **f32) if (delta_bias is not None and want_ddelta_bias)
             else None,
             dh0=torch.empty((Bsz, Dm, N), **f32) if want_dh0 else None)
    wsb = int(lib.ssm_scan_bwd_conv_workspace_bytes(Bsz, L, Dm, N, io))
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        st = lib.ssm_scan_bwd_conv(Bsz, L, Dm, N, io, _ptr(x), _ptr(conv_w), _ptr(conv_b), K,
                                   _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                   _ptr(delta_bias), int(bool(delta_softplus)), _ptr(h0),
                                   _ptr(chunk_states), _ptr(dy), _ptr(dh_final), _ptr(g["dx"]),
                                   _ptr(g["dconv_w"]), _ptr(g["dconv_b"]), _ptr(g["ddelta"]),
                                   _ptr(g["dA"]), _ptr(g["dB"]), _ptr(g["dC"]), _ptr(g["dD"]),
                                   _ptr(g["dz"]), _ptr(g["ddelta_bias"]), _ptr(g["dh0"]), _ptr(ws),
                                   wsb, _stream(dev), _flags(delta, x, zoh))
    _lib.check(st)
    return g


def state_update(state, u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True,
                 zoh=False):
    """One decode step; ``state`` (batch, dim, dstate) fp32 is updated in place.  Returns y.
    ``zoh`` uses the exact zero-order-hold input term."""
    if not isinstance(state, torch.Tensor) or state.dim() != 3:
        raise ValueError("state must be a (batch, dim, dstate) tensor")
    Bsz, Dm, N = state.shape
    dev = state.device
    if dev.type != "cuda":
        raise ValueError(f"tensors must be on a GPU device, got {dev}")
    if not isinstance(u, torch.Tensor):
        raise TypeError("u must be a torch.Tensor")
    io = _io_code(u)
    _need("state", state, (Bsz, Dm, N), torch.float32, dev)
    _need("u", u, (Bsz, Dm), u.dtype, dev)
    _need("delta", delta, (Bsz, Dm), u.dtype, dev)
    _need("A", A, (Dm, N), torch.float32, dev)
    _need("B", B, (Bsz, N), u.dtype, dev)
    _need("C", C, (Bsz, N), u.dtype, dev)
    _need("D", D, (Dm,), torch.float32, dev, optional=True)
    _need("z", z, (Bsz, Dm), u.dtype, dev, optional=True)
    _need("delta_bias", delta_bias, (Dm,), torch.float32, dev, optional=True)
    lib = _lib.load()
    y = torch.empty_like(u)
    with torch.cuda.device(dev):
        st = lib.ssm_state_update_ex(Bsz, Dm, N, io, _ptr(state), _ptr(u), _ptr(delta), _ptr(A),
                                     _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
                                     int(bool(delta_softplus)), _ptr(y), _stream(dev),
                                     _lib.FLAG_ZOH if zoh else 0)
    _lib.check(st)
    return y


def affine_scan(a, b, h0=None, reverse=False):
    """Scan of affine maps along the last axis: h[..., i] = a[..., i] h[..., i-1]
    + b[..., i] in scan order (last to first if ``reverse``), starting from h0
    (shape a.shape[:-1], zeros if None).  a, b fp32 on one GPU, same shape."""
    if not isinstance(a, torch.Tensor) or a.dim() < 1:
        raise ValueError("a must be a tensor with at least one dimension")
    dev = a.device
    if dev.type != "cuda":
        raise ValueError(f"tensors must be on a GPU device, got {dev}")
    _need("a", a, tuple(a.shape), torch.float32, dev)
    _need("b", b, tuple(a.shape), torch.float32, dev)
    _need("h0", h0, tuple(a.shape[:-1]), torch.float32, dev, optional=True)
    length = a.shape[-1]
    rows = a.numel() // max(length, 1)
    h = torch.empty_like(a)
    with torch.cuda.device(dev):
        st = _lib.load().ssm_affine_scan(rows, length, _ptr(a), _ptr(b), _ptr(h0), _ptr(h),
                                         int(bool(reverse)), _stream(dev))
    _lib.check(st)
    return h


class SelectiveScanFn(torch.autograd.Function):
    """Autograd wrapper: forward saves the chunk-boundary states, backward
    recomputes the states inside each chunk from them."""

    @staticmethod
    def forward(ctx, u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True,
                h0=None, zoh=False, reverse=False):
        y, hf, cs = scan_fwd(u, delta, A, B, C, D, z, delta_bias, delta_softplus, h0,
                             return_final_state=True, save_chunk_states=True, zoh=zoh,
                             reverse=reverse)
        ctx.delta_softplus = bool(delta_softplus)
        ctx.zoh, ctx.reverse = bool(zoh), bool(reverse)
        ctx.save_for_backward(u, delta, A, B, C, D, z, delta_bias, h0, cs)
        return y, hf

    @staticmethod
    def backward(ctx, dy, dhf):
        u, delta, A, B, C, D, z, delta_bias, h0, cs = ctx.saved_tensors
        g = scan_bwd(u, delta, A, B, C, D, z, delta_bias, ctx.delta_softplus, h0, cs,
                     dy.contiguous(), None if dhf is None else dhf.contiguous(),
                     want_ddelta_bias=delta_bias is not None, want_dh0=h0 is not None,
                     zoh=ctx.zoh, reverse=ctx.reverse)
        return (g["du"], g["ddelta"], g["dA"], g["dB"], g["dC"], g["dD"], g["dz"],
                g["ddelta_bias"], None, g["dh0"], None, None)


def selective_scan(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True,
                   h0=None, zoh=False, reverse=False):
    """Differentiable scan; returns (y, h_final)."""
    return SelectiveScanFn.apply(u, delta, A, B, C, D, z, delta_bias, delta_softplus, h0, zoh,
                                 reverse)


def bidirectional_scan(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True,
                       zoh=False):
    """Both scan directions summed: y = (S_fwd(u) + S_rev(u) + D u) * silu(z), where
    S_fwd and S_rev are the state contributions sum_n C h of the forward and the
    reverse recurrence.  Two launches; the second adds into the first's output."""
    y, _, _ = scan_fwd(u, delta, A, B, C, D, z, delta_bias, delta_softplus, zoh=zoh)
    scan_fwd(u, delta, A, B, C, None, z, delta_bias, delta_softplus, zoh=zoh, reverse=True, out=y)
    return y


class ConvScanFn(torch.autograd.Function):
    """Autograd wrapper of the scan fed by the fused causal convolution."""

    @staticmethod
    def forward(ctx, x, conv_w, conv_b, delta, A, B, C, D=None, z=None, delta_bias=None,
                delta_softplus=True, h0=None, zoh=False):
        y, hf, cs = scan_fwd_conv(x, conv_w, conv_b, delta, A, B, C, D, z, delta_bias,
                                  delta_softplus, h0, return_final_state=True,
                                  save_chunk_states=True, zoh=zoh)
        ctx.delta_softplus, ctx.zoh = bool(delta_softplus), bool(zoh)
        ctx.save_for_backward(x, conv_w, conv_b, delta, A, B, C, D, z, delta_bias, h0, cs)
        return y, hf

    @staticmethod
    def backward(ctx, dy, dhf):
        x, conv_w, conv_b, delta, A, B, C, D, z, delta_bias, h0, cs = ctx.saved_tensors
        g = scan_bwd_conv(x, conv_w, conv_b, delta, A, B, C, D, z, delta_bias, ctx.delta_softplus,
                          h0, cs, dy.contiguous(), None if dhf is None else dhf.contiguous(),
                          want_ddelta_bias=delta_bias is not None, want_dh0=h0 is not None,
                          zoh=ctx.zoh)
        return (g["dx"], g["dconv_w"], g["dconv_b"], g["ddelta"], g["dA"], g["dB"], g["dC"],
                g["dD"], g["dz"], g["ddelta_bias"], None, g["dh0"], None)


def conv_selective_scan(x, conv_w, conv_b, delta, A, B, C, D=None, z=None, delta_bias=None,
                        delta_softplus=True, h0=None, zoh=False):
    """Differentiable scan behind the fused causal convolution; returns (y, h_final)."""
    return ConvScanFn.apply(x, conv_w, conv_b, delta, A, B, C, D, z, delta_bias, delta_softplus,
                            h0, zoh)
