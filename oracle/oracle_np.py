"""NumPy fp64 twin of the C oracle, written independently of it.

Test infrastructure only.  It vectorises over (batch, channel, state) and
steps through time in a Python loop, so it is meant for small and medium
shapes.  Softplus uses ``numpy.logaddexp(0, x)`` and the sigmoid uses
``scipy.special.expit``, so neither shares a formula with the C version.

Same definition as ``ssm_oracle.c``: Mamba (Gu & Dao) per the reading guide's
"Yöntem" discretisation equations and "Seçim Mekanizması (S6)" delta equation,
the input term delta*B*u of the sequential loop quoted on the mamba-minimal
news page, the D*u skip and SiLU gate of the Mamba block.
"""
from __future__ import annotations

import numpy as np
from scipy.special import expit


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):
        import torch
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _step_sizes(delta, delta_bias, delta_softplus):
    s = delta if delta_bias is None else delta + delta_bias
    return (np.logaddexp(0.0, s) if delta_softplus else s), s


def scan_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True, h0=None,
             chunk_len=None, return_states=False):
    u, delta, A, B, C, D, z, delta_bias, h0 = map(_f64, (u, delta, A, B, C, D, z, delta_bias, h0))
    Bsz, L, Dm = u.shape
    N = A.shape[1]
    dt, _ = _step_sizes(delta, delta_bias, delta_softplus)
    h = np.zeros((Bsz, Dm, N)) if h0 is None else h0.copy()
    y = np.empty((Bsz, L, Dm))
    states = np.empty((Bsz, L, Dm, N)) if return_states else None
    chunks = []
    for t in range(L):
        if chunk_len and t % chunk_len == 0:
            chunks.append(h.copy())
        decay = np.exp(dt[:, t, :, None] * A[None, :, :])
        inject = dt[:, t, :, None] * u[:, t, :, None] * B[:, t, None, :]
        h = decay * h + inject
        if return_states:
            states[:, t] = h
        y[:, t, :] = np.einsum("bdn,bn->bd", h, C[:, t, :])
    if D is not None:
        y = y + D[None, None, :] * u
    if z is not None:
        y = y * (z * expit(z))
    cs = np.stack(chunks, axis=1) if chunk_len else None
    if return_states:
        return y, h, cs, states
    return y, h, cs


def scan_bwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True, h0=None,
             dy=None, dh_final=None):
    u, delta, A, B, C, D, z, delta_bias, h0, dy, dh_final = map(
        _f64, (u, delta, A, B, C, D, z, delta_bias, h0, dy, dh_final))
    Bsz, L, Dm = u.shape
    N = A.shape[1]
    dt, s = _step_sizes(delta, delta_bias, delta_softplus)
    hinit = np.zeros((Bsz, Dm, N)) if h0 is None else h0
    _, _, _, H = scan_fwd(u, delta, A, B, C, None, None, delta_bias, delta_softplus, h0,
                          return_states=True)
    pre = np.einsum("bldn,bln->bld", H, C)
    if D is not None:
        pre = pre + D * u
    if z is not None:
        sig = expit(z)
        e = dy * z * sig
        dz = dy * pre * (sig + z * sig * (1.0 - sig))
    else:
        e = dy.copy()
        dz = None
    lam_next = np.zeros((Bsz, Dm, N)) if dh_final is None else dh_final.copy()
    du = np.empty_like(u)
    ddt = np.empty_like(u)
    dA = np.zeros((Dm, N))
    dB = np.empty((Bsz, L, N))
    dC = np.empty((Bsz, L, N))
    for t in range(L - 1, -1, -1):
        decay = np.exp(dt[:, t, :, None] * A[None])
        hprev = H[:, t - 1] if t > 0 else hinit
        lam = e[:, t, :, None] * C[:, t, None, :] + lam_next
        dC[:, t] = np.einsum("bd,bdn->bn", e[:, t], H[:, t])
        dB[:, t] = np.einsum("bdn,bd->bn", lam, dt[:, t] * u[:, t])
        du[:, t] = np.einsum("bdn,bn->bd", lam, B[:, t]) * dt[:, t]
        ddt[:, t] = (np.einsum("bdn,bdn->bd", lam, hprev * decay * A[None])
                     + np.einsum("bdn,bn->bd", lam, B[:, t]) * u[:, t])
        dA += np.einsum("bdn,bd->dn", lam * hprev * decay, dt[:, t])
        lam_next = decay * lam
    if D is not None:
        du = du + D * e
    dD = (e * u).sum(axis=(0, 1)) if D is not None else None
    ddelta = ddt * expit(s) if delta_softplus else ddt
    dbias = ddelta.sum(axis=(0, 1)) if delta_bias is not None else None
    return dict(du=du, ddelta=ddelta, dA=dA, dB=dB, dC=dC, dD=dD, dz=dz, ddelta_bias=dbias,
                dh0=lam_next)


def state_update(state, u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True):
    state, u, delta, A, B, C, D, z, delta_bias = map(
        _f64, (state, u, delta, A, B, C, D, z, delta_bias))
    dt, _ = _step_sizes(delta, delta_bias, delta_softplus)
    new = np.exp(dt[:, :, None] * A[None]) * state + (dt * u)[:, :, None] * B[:, None, :]
    y = np.einsum("bdn,bn->bd", new, C)
    if D is not None:
        y = y + D * u
    if z is not None:
        y = y * z * expit(z)
    return new, y
