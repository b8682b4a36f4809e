"""Pins of the oracle's causal depthwise convolution + SiLU (the Mamba block's
Conv1d in front of the selective SSM) and of the scan fed by it."""
from __future__ import annotations

import numpy as np
import pytest

from oracle import oracle_c, oracle_np
from tests.helpers import nmax_err, rand_problem


def _conv_problem(B=2, L=13, D=3, K=4, seed=0):
    rng = np.random.default_rng(seed)
    return rng.normal(size=(B, L, D)), rng.normal(size=(D, K)) * 0.5, rng.normal(size=D) * 0.3


# --------------------------------------------------------------------------
# P-16  The convolution is a causal FIR filter along time per channel: brute
# force on the definition, K = 1 is pointwise, and a unit impulse returns the
# taps in reverse order (tap K-1 multiplies the current step).
# --------------------------------------------------------------------------
@pytest.mark.parametrize("impl", [oracle_c, oracle_np], ids=["c", "np"])
def test_p16_conv_definition(impl):
    x, w, b = _conv_problem()
    u, pre = impl.conv1d_silu(x, w, b)
    B, L, D = x.shape
    K = w.shape[1]
    ref = np.zeros_like(x)
    for t in range(L):
        for k in range(K):
            s = t - (K - 1) + k
            if s >= 0:
                ref[:, t] += w[:, k] * x[:, s]
    ref += b
    assert np.abs(pre - ref).max() < 1e-13
    assert np.abs(u - ref / (1 + np.exp(-ref))).max() < 1e-13
    u1, pre1 = impl.conv1d_silu(x, w[:, :1], b)
    assert np.abs(pre1 - (x * w[:, 0] + b)).max() < 1e-14
    imp = np.zeros((1, 8, 3))
    imp[0, 0] = 1.0
    _, pi = impl.conv1d_silu(imp, w, None)
    for k in range(4):
        assert np.allclose(pi[0, k], w[:, 3 - k])
    assert np.abs(pi[0, 4:]).max() == 0.0


@pytest.mark.parametrize("impl", [oracle_c, oracle_np], ids=["c", "np"])
@pytest.mark.parametrize("K", [1, 2, 4])
def test_p17_conv_backward_finite_differences(impl, K):
    x, w, b = _conv_problem(K=K, seed=K)
    du = np.random.default_rng(9).normal(size=x.shape)
    dx, dw, db = impl.conv1d_silu_bwd(x, w, b, du)

    def loss(xx, ww, bb):
        return float((impl.conv1d_silu(xx, ww, bb)[0] * du).sum())

    eps = 1e-6
    for arr, grad in ((x, dx), (w, dw), (b, db)):
        fd = np.empty(arr.shape)
        for i in range(arr.size):
            vals = []
            for sg in (1, -1):
                a2 = arr.copy().reshape(-1)
                a2[i] += sg * eps
                a2 = a2.reshape(arr.shape)
                args = [x, w, b]
                args[[id(x), id(w), id(b)].index(id(arr))] = a2
                vals.append(loss(*args))
            fd.reshape(-1)[i] = (vals[0] - vals[1]) / (2 * eps)
        assert nmax_err(grad, fd) < 2e-7


def test_conv_twins_agree():
    x, w, b = _conv_problem(B=3, L=50, D=5, K=3, seed=4)
    uc, pc = oracle_c.conv1d_silu(x, w, b)
    un, pn = oracle_np.conv1d_silu(x, w, b)
    assert nmax_err(uc, un) < 1e-13 and nmax_err(pc, pn) < 1e-13
    du = np.random.default_rng(1).normal(size=x.shape)
    for a, c in zip(oracle_c.conv1d_silu_bwd(x, w, b, du), oracle_np.conv1d_silu_bwd(x, w, b, du)):
        assert nmax_err(a, c) < 1e-12


# --------------------------------------------------------------------------
# P-18  The scan fed by the convolution: its gradient matches central
# differences of the composed forward for every input, including x, the taps
# and the conv bias.
# --------------------------------------------------------------------------
def test_p18_conv_scan_backward_finite_differences():
    p = {k: (v.numpy() if hasattr(v, "numpy") else v)
         for k, v in rand_problem(2, 7, 3, 2, seed=51, with_h0=True).items()}
    x, w, cb = _conv_problem(2, 7, 3, 3, seed=8)
    rng = np.random.default_rng(3)
    dy = rng.normal(size=x.shape)
    G = rng.normal(size=(2, 3, 2))
    base = dict(x=x, conv_w=w, conv_b=cb, delta=p["delta"], A=p["A"], B=p["B"], C=p["C"],
                D=p["D"], z=p["z"], delta_bias=p["delta_bias"], h0=p["h0"])
    g = oracle_c.scan_bwd_conv(**base, dy=dy, dh_final=G)

    def loss(q):
        y, hf, _ = oracle_c.scan_fwd_conv(**q)
        return float((y * dy).sum() + (hf * G).sum())

    eps = 1e-6
    for name, gname in (("x", "dx"), ("conv_w", "dconv_w"), ("conv_b", "dconv_b"),
                        ("delta", "ddelta"), ("A", "dA"), ("h0", "dh0")):
        arr = base[name]
        fd = np.empty(arr.shape)
        for i in range(arr.size):
            vals = []
            for sg in (1, -1):
                a2 = arr.copy().reshape(-1)
                a2[i] += sg * eps
                vals.append(loss(dict(base, **{name: a2.reshape(arr.shape)})))
            fd.reshape(-1)[i] = (vals[0] - vals[1]) / (2 * eps)
        assert nmax_err(g[gname], fd) < 5e-7, name
