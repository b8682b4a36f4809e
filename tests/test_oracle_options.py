"""Pins of the oracle's options: the exact zero-order-hold input term, the
reverse scan direction and one step size per token.

Each option is pinned by something other than its own code: a closed form the
mathematics fixes, a special case that reduces to an already pinned path, or
central differences of the forward.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch
from scipy.special import expit

from oracle import oracle_c, oracle_np
from tests.helpers import nmax_err, rand_problem

GRAD_OF = dict(u="du", delta="ddelta", A="dA", B="dB", C="dC", D="dD", z="dz",
               delta_bias="ddelta_bias", h0="dh0")
IMPLS = pytest.mark.parametrize("impl", [oracle_c, oracle_np], ids=["c", "np"])


def _np(t):
    return None if t is None else (t.numpy() if hasattr(t, "numpy") else np.asarray(t))


# --------------------------------------------------------------------------
# P-3z  Under the exact zero-order hold, A = -1 and a softplus step size give
# the gated RNN of the reading guide's "Seçim Mekanizması (S6)" section
# exactly: exp(-softplus(s)) = 1 - sigmoid(s) and expm1(-softplus(s))/(-1) =
# sigmoid(s), so h_t = (1 - g_t) h_{t-1} + g_t B_t u_t with g_t = sigmoid(s_t).
# --------------------------------------------------------------------------
@IMPLS
def test_p3z_zoh_is_the_gated_rnn(impl):
    rng = np.random.default_rng(3)
    Bsz, L, D = 2, 40, 3
    u = rng.normal(size=(Bsz, L, D))
    raw = rng.normal(size=(Bsz, L, D)) * 3
    bias = rng.normal(size=D)
    Bm = rng.normal(size=(Bsz, L, 1))
    Cm = rng.normal(size=(Bsz, L, 1))
    h0 = rng.normal(size=(Bsz, D, 1))
    y, hf, _ = impl.scan_fwd(u, raw, -np.ones((D, 1)), Bm, Cm, None, None, bias, True, h0, zoh=True)
    g = expit(raw + bias)
    h = h0[:, :, 0].copy()
    ref = np.empty((Bsz, L, D))
    for t in range(L):
        h = (1.0 - g[:, t]) * h + g[:, t] * Bm[:, t] * u[:, t]
        ref[:, t] = Cm[:, t] * h
    assert np.abs(y - ref).max() < 1e-13
    assert np.abs(hf[:, :, 0] - h).max() < 1e-13


# --------------------------------------------------------------------------
# P-12  Fixed point of the exact hold: with u and B constant in time, the
# state h* = -B u / A satisfies exp(dt A) h* + expm1(dt A)/A B u = h* for every
# dt, so a scan started there stays there whatever the step sizes are, and
# y_t = C_t h* + D u.  (The first-order form has no such fixed point.)
# --------------------------------------------------------------------------
@IMPLS
def test_p12_zoh_fixed_point(impl):
    rng = np.random.default_rng(4)
    Bsz, L, D, N = 2, 30, 4, 3
    u = np.repeat(rng.normal(size=(Bsz, 1, D)), L, axis=1)
    Bm = np.repeat(rng.normal(size=(Bsz, 1, N)), L, axis=1)
    Cm = rng.normal(size=(Bsz, L, N))
    A = -(rng.random(size=(D, N)) * 3 + 0.2)
    Dk = rng.normal(size=D)
    raw = rng.normal(size=(Bsz, L, D)) * 2
    hstar = -Bm[:, 0, None, :] * u[:, 0, :, None] / A[None]
    y, hf, _ = impl.scan_fwd(u, raw, A, Bm, Cm, Dk, None, None, True, hstar, zoh=True)
    assert nmax_err(hf, hstar) < 1e-13
    ref = np.einsum("bln,bdn->bld", Cm, hstar) + Dk * u
    assert nmax_err(y, ref) < 1e-13
    y1, hf1, _ = impl.scan_fwd(u, raw, A, Bm, Cm, Dk, None, None, True, hstar, zoh=False)
    assert nmax_err(hf1, hstar) > 1e-3  # the first-order input term drifts away


# --------------------------------------------------------------------------
# P-13  As A -> 0 both input terms tend to dt B u: the exact hold agrees with
# the first-order form to O(dt A).
# --------------------------------------------------------------------------
@IMPLS
def test_p13_zoh_small_A_limit(impl):
    p = {k: _np(v) for k, v in rand_problem(2, 25, 3, 4, seed=9, with_h0=True).items()}
    p["A"] = p["A"] * 1e-9
    y0, h0f, _ = impl.scan_fwd(**p)
    y1, h1f, _ = impl.scan_fwd(**p, zoh=True)
    assert nmax_err(y1, y0) < 1e-8 and nmax_err(h1f, h0f) < 1e-8


# --------------------------------------------------------------------------
# P-14  The reverse scan is the forward scan of the time-reversed inputs,
# reversed back (forward path already pinned by P-1..P-11).  Chunk slot k of
# the reverse scan is the state before scan step k*T.  The same holds for
# every gradient (time-indexed ones reversed).
# --------------------------------------------------------------------------
def _flip(p, keys=("u", "delta", "B", "C", "z", "dy")):
    return {k: (v[:, ::-1].copy() if k in keys and v is not None else v) for k, v in p.items()}


@IMPLS
@pytest.mark.parametrize("zoh", [False, True])
def test_p14_reverse_is_flipped_forward(impl, zoh):
    p = {k: _np(v) for k, v in rand_problem(2, 23, 3, 4, seed=12, with_h0=True).items()}
    y, hf, cs = impl.scan_fwd(**p, chunk_len=5, reverse=True, zoh=zoh)
    yf, hff, csf = impl.scan_fwd(**_flip(p), chunk_len=5, zoh=zoh)
    assert np.abs(y - yf[:, ::-1]).max() < 1e-12
    assert np.abs(hf - hff).max() < 1e-12
    assert np.abs(cs - csf).max() < 1e-12
    rng = np.random.default_rng(1)
    dy = rng.normal(size=y.shape)
    G = rng.normal(size=hf.shape)
    g = impl.scan_bwd(**p, dy=dy, dh_final=G, reverse=True, zoh=zoh)
    gf = impl.scan_bwd(**_flip(dict(p, dy=dy)), dh_final=G, zoh=zoh)
    for k in ("du", "ddelta", "dB", "dC", "dz"):
        assert np.abs(g[k] - gf[k][:, ::-1]).max() < 1e-11, k
    for k in ("dA", "dD", "ddelta_bias", "dh0"):
        assert np.abs(g[k] - gf[k]).max() < 1e-11, k


# --------------------------------------------------------------------------
# P-15  One step size per token is the full (B,L,D) step size with that value
# repeated over channels; its gradient is the full gradient summed over them.
# --------------------------------------------------------------------------
@IMPLS
@pytest.mark.parametrize("zoh,reverse", [(False, False), (True, True)])
def test_p15_per_token_delta_is_broadcast(impl, zoh, reverse):
    p = {k: _np(v) for k, v in rand_problem(2, 17, 5, 2, seed=13, with_h0=True).items()}
    tok = p["delta"][:, :, 0].copy()
    full = dict(p, delta=np.repeat(tok[:, :, None], 5, axis=2))
    y, hf, _ = impl.scan_fwd(**dict(p, delta=tok), zoh=zoh, reverse=reverse)
    yf, hff, _ = impl.scan_fwd(**full, zoh=zoh, reverse=reverse)
    assert np.abs(y - yf).max() < 1e-13 and np.abs(hf - hff).max() < 1e-13
    dy = np.random.default_rng(2).normal(size=y.shape)
    g = impl.scan_bwd(**dict(p, delta=tok), dy=dy, zoh=zoh, reverse=reverse)
    gf = impl.scan_bwd(**full, dy=dy, zoh=zoh, reverse=reverse)
    assert g["ddelta"].shape == tok.shape
    assert np.abs(g["ddelta"] - gf["ddelta"].sum(axis=2)).max() < 1e-12
    for k in ("du", "dA", "dB", "dC", "dD", "dz", "ddelta_bias", "dh0"):
        assert np.abs(g[k] - gf[k]).max() < 1e-12, k


# --------------------------------------------------------------------------
# P-9z  The options' backward is the gradient of their forward: central
# differences on every element of every differentiable input.
# --------------------------------------------------------------------------
@IMPLS
@pytest.mark.parametrize("zoh,reverse,per_token", [(True, False, False), (False, True, True),
                                                    (True, True, True)],
                         ids=["zoh", "reverse-token", "all"])
def test_p9z_options_backward_matches_finite_differences(impl, zoh, reverse, per_token):
    Bsz, L, D, N = 2, 5, 3, 2
    p = {k: _np(v) for k, v in rand_problem(Bsz, L, D, N, seed=41, with_h0=True).items()}
    if per_token:
        p["delta"] = p["delta"][:, :, 0].copy()
    rng = np.random.default_rng(6)
    w = rng.normal(size=(Bsz, L, D))
    G = rng.normal(size=(Bsz, D, N))
    kw = dict(zoh=zoh, reverse=reverse)
    grads = impl.scan_bwd(**p, dy=w, dh_final=G, **kw)

    def loss(q):
        y, hf, _ = impl.scan_fwd(**q, **kw)
        return float((y * w).sum() + (hf * G).sum())

    eps = 1e-6
    for name, gname in GRAD_OF.items():
        base = p[name]
        fd = np.empty(base.shape)
        for i in range(base.size):
            vals = []
            for sgn in (1, -1):
                x = base.copy().reshape(-1)
                x[i] += sgn * eps
                vals.append(loss(dict(p, **{name: x.reshape(base.shape)})))
            fd.reshape(-1)[i] = (vals[0] - vals[1]) / (2 * eps)
        err = nmax_err(grads[gname], fd)
        assert err < 5e-7, (name, err)


@pytest.mark.parametrize("zoh,reverse,per_token", [(True, False, False), (True, True, True)])
def test_p11_options_twins_agree(zoh, reverse, per_token):
    p = {k: _np(v) for k, v in rand_problem(3, 40, 6, 4, seed=17, with_h0=True).items()}
    if per_token:
        p["delta"] = p["delta"][:, :, 0].copy()
    kw = dict(zoh=zoh, reverse=reverse)
    yc, hc, cc = oracle_c.scan_fwd(**p, chunk_len=7, nthreads=3, **kw)
    yn, hn, cn = oracle_np.scan_fwd(**p, chunk_len=7, **kw)
    assert nmax_err(yc, yn) < 1e-12 and nmax_err(hc, hn) < 1e-12
    assert nmax_err(cc, np.moveaxis(cn, 0, 0)) < 1e-12
    dy = np.random.default_rng(8).normal(size=yc.shape)
    gc = oracle_c.scan_bwd(**p, dy=dy, nthreads=3, **kw)
    gn = oracle_np.scan_bwd(**p, dy=dy, **kw)
    for k in gc:
        if gc[k] is not None:
            assert nmax_err(gc[k], gn[k]) < 1e-11, k


# --------------------------------------------------------------------------
# P-7z  One decode step with the exact hold equals a one-step scan with it.
# --------------------------------------------------------------------------
@IMPLS
def test_p7z_decode_zoh_is_one_step_scan(impl):
    p = {k: _np(v) for k, v in rand_problem(2, 1, 5, 4, seed=21, with_h0=True).items()}
    y, hf, _ = impl.scan_fwd(**p, zoh=True)
    st, yd = impl.state_update(p["h0"], p["u"][:, 0], p["delta"][:, 0], p["A"], p["B"][:, 0],
                               p["C"][:, 0], p["D"], p["z"][:, 0], p["delta_bias"], True, zoh=True)
    assert np.abs(st - hf).max() < 1e-14 and np.abs(yd - y[:, 0]).max() < 1e-14
