"""NumPy fp64 twin of the C oracle, written independently of it.

Test infrastructure only.  It vectorises over (batch, channel, state) and
steps through time in a Python loop, so it is meant for small and medium
shapes.  Softplus uses ``numpy.logaddexp(0, x)`` and the sigmoid uses
``scipy.special.expit``, so neither shares a formula with the C version.

Same definition as ``ssm_oracle.c``: Mamba (Gu & Dao) per the reading guide's
"Yöntem" equations (zero-order hold of A, the linear recurrence of the state,
the output as the state contracted with C) and its "Seçim Mekanizması (S6)"
step-size equation, with the first-order input term delta*B*u (the reading
taken for the discretisation of B), the D*u skip and the SiLU gate of the
Mamba block.
"""
from __future__ import annotations

import numpy as np
from scipy.signal import lfilter
from scipy.special import expit


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):
        import torch
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _step_sizes(delta, delta_bias, delta_softplus, dim):
    """Step sizes (B,L,D) and their pre-softplus argument; a (B,L) delta is
    one raw value per token, the same for every channel."""
    if delta.ndim == 2:
        delta = np.repeat(delta[:, :, None], dim, axis=2)
    s = delta if delta_bias is None else delta + delta_bias
    return (np.logaddexp(0.0, s) if delta_softplus else s), s


def _coef(dt_t, A, zoh):
    """Input coefficient per (b, d, n) of one step: dt, or expm1(dt A)/A for
    the exact zero-order hold (dt where A = 0)."""
    x = dt_t[:, :, None] * A[None]
    if not zoh:
        return np.broadcast_to(dt_t[:, :, None], x.shape)
    safe = np.where(A == 0.0, 1.0, A)[None]
    return np.where(A[None] == 0.0, dt_t[:, :, None], np.expm1(x) / safe)


def _dcoef_dA(dt_t, A):
    """d/dA of expm1(dt A)/A: dt^2 (x e^x - e^x + 1)/x^2 with x = dt A, by
    its Taylor series where the closed form loses digits."""
    dt3 = dt_t[:, :, None]
    x = dt3 * A[None]
    series = sum(x ** k * (k + 1) / float(np.prod(np.arange(1, k + 3))) for k in range(9))
    small = np.abs(x) < 5e-2
    xs = np.where(small, 1.0, x)
    closed = (xs * np.exp(xs) - np.expm1(xs)) / (xs * xs)
    return dt3 * dt3 * np.where(small, series, closed)


def scan_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True, h0=None,
             chunk_len=None, return_states=False, zoh=False, reverse=False):
    """``zoh``: exact zero-order-hold input coefficient; ``reverse``: the scan
    runs from the last step to the first (states are returned in scan order)."""
    u, delta, A, B, C, D, z, delta_bias, h0 = map(_f64, (u, delta, A, B, C, D, z, delta_bias, h0))
    Bsz, L, Dm = u.shape
    N = A.shape[1]
    dt, _ = _step_sizes(delta, delta_bias, delta_softplus, Dm)
    h = np.zeros((Bsz, Dm, N)) if h0 is None else h0.copy()
    y = np.empty((Bsz, L, Dm))
    states = np.empty((Bsz, L, Dm, N)) if return_states else None
    chunks = []
    order = range(L - 1, -1, -1) if reverse else range(L)
    for k, t in enumerate(order):
        if chunk_len and k % chunk_len == 0:
            chunks.append(h.copy())
        # one step of the discrete recurrence ("Yöntem"): the state decays by
        # exp(dt A) per (b, d, n) and takes in the input term coef * B_t * u_t
        Abar = np.exp(dt[:, t, :, None] * A[None, :, :])
        Bbar_u = (_coef(dt[:, t], A, zoh) * B[:, t, None, :]) * u[:, t, :, None]
        h = Abar * h + Bbar_u
        if return_states:
            states[:, k] = h
        # output: the state contracted with C_t over the state index
        y[:, t, :] = (h * C[:, t][:, None, :]).sum(axis=2)
    if D is not None:
        y = y + D[None, None, :] * u
    if z is not None:
        y = y * (z * expit(z))
    cs = np.stack(chunks, axis=1) if chunk_len else None
    if return_states:
        return y, h, cs, states
    return y, h, cs


def scan_bwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True, h0=None,
             dy=None, dh_final=None, zoh=False, reverse=False):
    u, delta, A, B, C, D, z, delta_bias, h0, dy, dh_final = map(
        _f64, (u, delta, A, B, C, D, z, delta_bias, h0, dy, dh_final))
    Bsz, L, Dm = u.shape
    N = A.shape[1]
    per_token = delta.ndim == 2
    dt, s = _step_sizes(delta, delta_bias, delta_softplus, Dm)
    hinit = np.zeros((Bsz, Dm, N)) if h0 is None else h0
    _, _, _, Hs = scan_fwd(u, delta, A, B, C, None, None, delta_bias, delta_softplus, h0,
                           return_states=True, zoh=zoh, reverse=reverse)
    order = list(range(L - 1, -1, -1)) if reverse else list(range(L))
    H = np.empty_like(Hs)  # states by memory row
    H[:, order] = Hs
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
    for k in range(L - 1, -1, -1):
        t = order[k]
        decay = np.exp(dt[:, t, :, None] * A[None])
        cf = _coef(dt[:, t], A, zoh)
        hprev = Hs[:, k - 1] if k > 0 else hinit
        lam = e[:, t, :, None] * C[:, t, None, :] + lam_next
        lamBu = lam * B[:, t, None, :] * u[:, t, :, None]
        dC[:, t] = np.einsum("bd,bdn->bn", e[:, t], H[:, t])
        dB[:, t] = np.einsum("bdn,bdn->bn", lam, cf * u[:, t, :, None])
        du[:, t] = np.einsum("bdn,bdn->bd", lam * cf, np.broadcast_to(B[:, t, None, :], lam.shape))
        dcoef_ddt = decay if zoh else 1.0
        ddt[:, t] = (np.einsum("bdn,bdn->bd", lam, hprev * decay * A[None])
                     + (lamBu * dcoef_ddt).sum(axis=2))
        dA += np.einsum("bdn,bd->dn", lam * hprev * decay, dt[:, t])
        if zoh:
            dA += (lamBu * _dcoef_dA(dt[:, t], A)).sum(axis=0)
        lam_next = decay * lam
    if D is not None:
        du = du + D * e
    dD = (e * u).sum(axis=(0, 1)) if D is not None else None
    ddelta = ddt * expit(s) if delta_softplus else ddt
    dbias = ddelta.sum(axis=(0, 1)) if delta_bias is not None else None
    if per_token:
        ddelta = ddelta.sum(axis=2)
    return dict(du=du, ddelta=ddelta, dA=dA, dB=dB, dC=dC, dD=dD, dz=dz, ddelta_bias=dbias,
                dh0=lam_next)


def state_update(state, u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True,
                 zoh=False):
    state, u, delta, A, B, C, D, z, delta_bias = map(
        _f64, (state, u, delta, A, B, C, D, z, delta_bias))
    s = delta if delta_bias is None else delta + delta_bias
    dt = np.logaddexp(0.0, s) if delta_softplus else s
    new = (np.exp(dt[:, :, None] * A[None]) * state
           + _coef(dt, A, zoh) * u[:, :, None] * B[:, None, :])
    y = (new * C[:, None, :]).sum(axis=2)
    if D is not None:
        y = y + D * u
    if z is not None:
        y = y * z * expit(z)
    return new, y


def conv1d_silu(x, w, bias=None):
    """Causal depthwise convolution as an FIR filter along time per channel
    (``scipy.signal.lfilter`` with taps w[d, ::-1], zero initial conditions),
    then SiLU.  Returns (u, pre)."""
    x, w, bias = map(_f64, (x, w, bias))
    pre = np.empty_like(x)
    for d in range(x.shape[2]):
        pre[:, :, d] = lfilter(w[d, ::-1], [1.0], x[:, :, d], axis=1)
    if bias is not None:
        pre = pre + bias
    return pre * expit(pre), pre


def conv1d_silu_bwd(x, w, bias, du):
    """Backward of conv1d_silu: the transposed filter runs backwards in time."""
    x, w, bias, du = map(_f64, (x, w, bias, du))
    _, pre = conv1d_silu(x, w, bias)
    sig = expit(pre)
    g = du * (sig + pre * sig * (1.0 - sig))
    K = w.shape[1]
    dx = np.empty_like(x)
    for d in range(x.shape[2]):
        dx[:, :, d] = lfilter(w[d, ::-1], [1.0], g[:, ::-1, d], axis=1)[:, ::-1]
    L = x.shape[1]
    dw = np.empty_like(w)
    for k in range(K):
        s = K - 1 - k  # tap k reads x shifted by s steps
        dw[:, k] = np.einsum("bld,bld->d", x[:, :L - s], g[:, s:]) if s < L else 0.0
    db = g.sum(axis=(0, 1)) if bias is not None else None
    return dx, dw, db
