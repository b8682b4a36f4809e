"""Pins of the fp64 oracle against closed forms, identities and brute force.

Each test runs both oracle implementations (C and NumPy) against a result
fixed by the mathematics, not by either implementation.  The pages print no
worked numeric example, so there are no printed values to pin against.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import pytest
import torch
from scipy.special import expit

from oracle import oracle_c, oracle_np
from tests.helpers import nmax_err, rand_problem

IMPLS = [pytest.param(oracle_c, id="c"), pytest.param(oracle_np, id="np")]


def _np(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


# --------------------------------------------------------------------------
# P-1  geometric series: constant step size, B, C, u (time-invariant, N > 1).
# With q = exp(A*delta) the recurrence h_t = q h_{t-1} + delta*beta*u0 has the
# closed form h_t = q^(t+1) h0 + delta*beta*u0 * (1 - q^(t+1)) / (1 - q).
# --------------------------------------------------------------------------
@pytest.mark.parametrize("impl", IMPLS)
@pytest.mark.parametrize("softplus", [False, True])
def test_p1_geometric_series(impl, softplus):
    rng = np.random.default_rng(11)
    Bsz, L, D, N = 2, 37, 5, 3
    A = -rng.uniform(0.2, 3.0, size=(D, N))
    bias = rng.uniform(0.01, 0.5, size=D) if not softplus else rng.uniform(-4.0, 1.0, size=D)
    # step size per channel, computed here from the definition of softplus
    dt = np.array([math.log(1.0 + math.exp(b)) if softplus else b for b in bias])
    beta = rng.normal(size=(Bsz, N))
    c = rng.normal(size=(Bsz, N))
    u0 = rng.normal(size=(Bsz, D))
    h0 = rng.normal(size=(Bsz, D, N))
    Dsk = rng.normal(size=D)
    u = np.broadcast_to(u0[:, None, :], (Bsz, L, D)).copy()
    Bm = np.broadcast_to(beta[:, None, :], (Bsz, L, N)).copy()
    Cm = np.broadcast_to(c[:, None, :], (Bsz, L, N)).copy()
    delta = np.zeros((Bsz, L, D))
    y, hf, _ = impl.scan_fwd(u, delta, A, Bm, Cm, Dsk, None, bias, softplus, h0)
    q = np.exp(A[None, :, :] * dt[None, :, None])  # (1, D, N)
    drive = dt[None, :, None] * beta[:, None, :] * u0[:, :, None]  # (B, D, N)
    yexp = np.empty((Bsz, L, D))
    for t in range(L):
        qt = q ** (t + 1)
        h = qt * h0 + drive * (1.0 - qt) / (1.0 - q)
        yexp[:, t, :] = np.einsum("bdn,bn->bd", h, c) + Dsk[None, :] * u0
    assert nmax_err(y, yexp) < 1e-12
    assert nmax_err(hf, h) < 1e-12


# --------------------------------------------------------------------------
# P-2  convolution form.  With delta, B, C time-invariant the scan is a causal
# convolution of u with K_k = sum_n C_n exp(A_n delta k) B_n delta, plus D*u,
# then gated (the pages' LTI equivalence of recurrence and global convolution).
# --------------------------------------------------------------------------
@pytest.mark.parametrize("impl", IMPLS)
def test_p2_convolution_form(impl):
    rng = np.random.default_rng(5)
    Bsz, L, D, N = 2, 53, 4, 3
    A = -rng.uniform(0.05, 2.0, size=(D, N))
    raw = rng.normal(size=(Bsz, D))
    bias = rng.normal(size=D) * 0.5 - 1.0
    beta = rng.normal(size=(Bsz, N))
    c = rng.normal(size=(Bsz, N))
    u = rng.normal(size=(Bsz, L, D))
    z = rng.normal(size=(Bsz, L, D)) * 2
    Dsk = rng.normal(size=D)
    delta = np.broadcast_to(raw[:, None, :], (Bsz, L, D)).copy()
    Bm = np.broadcast_to(beta[:, None, :], (Bsz, L, N)).copy()
    Cm = np.broadcast_to(c[:, None, :], (Bsz, L, N)).copy()
    y, _, _ = impl.scan_fwd(u, delta, A, Bm, Cm, Dsk, z, bias, True, None)
    yexp = np.empty_like(y)
    k = np.arange(L)
    for b in range(Bsz):
        for d in range(D):
            dt = np.logaddexp(0.0, raw[b, d] + bias[d])
            K = (c[b][None, :] * np.exp(np.outer(k, A[d]) * dt) * beta[b][None, :] * dt).sum(axis=1)
            conv = np.convolve(u[b, :, d], K)[:L]
            pre = conv + Dsk[d] * u[b, :, d]
            yexp[b, :, d] = pre * z[b, :, d] * expit(z[b, :, d])
    assert nmax_err(y, yexp) < 1e-12


# --------------------------------------------------------------------------
# P-3  RNN-gate identity (reading guide, S6 section and the Q&A on Delta):
# with N = 1 and A = -1, exp(-softplus(s)) = 1 - sigmoid(s), so
# h_t = (1 - g_t) h_{t-1} + softplus(s_t) B_t u_t with g_t = sigmoid(s_t).
# --------------------------------------------------------------------------
@pytest.mark.parametrize("impl", IMPLS)
def test_p3_rnn_gate(impl):
    rng = np.random.default_rng(7)
    Bsz, L, D = 3, 41, 6
    u = rng.normal(size=(Bsz, L, D))
    raw = rng.normal(size=(Bsz, L, D)) * 2.0
    bias = rng.normal(size=D)
    Bm = rng.normal(size=(Bsz, L, 1))
    Cm = rng.normal(size=(Bsz, L, 1))
    h0 = rng.normal(size=(Bsz, D, 1))
    A = -np.ones((D, 1))
    y, hf, _ = impl.scan_fwd(u, raw, A, Bm, Cm, None, None, bias, True, h0)
    s = raw + bias
    g = expit(s)
    h = h0[:, :, 0].copy()
    yexp = np.empty_like(y)
    for t in range(L):
        h = (1.0 - g[:, t]) * h + np.logaddexp(0.0, s[:, t]) * Bm[:, t, :] * u[:, t]
        yexp[:, t] = Cm[:, t, :] * h
    assert nmax_err(y, yexp) < 1e-12
    assert nmax_err(hf[:, :, 0], h) < 1e-12


# --------------------------------------------------------------------------
# P-4  limits of the step size (reading guide, Q&A on Delta): a vanishing
# step keeps the state and ignores the input; a huge step resets the state
# to the current input term.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("impl", IMPLS)
def test_p4_small_step_keeps_state(impl):
    p = rand_problem(2, 17, 5, 3, seed=3, with_h0=True)
    p["delta_bias"] = torch.full((5,), -900.0, dtype=torch.float64)  # softplus underflows to 0
    y, hf, _ = impl.scan_fwd(**p)
    h0 = p["h0"].numpy()
    pre = np.einsum("bdn,bln->bld", h0, p["C"].numpy()) + p["D"].numpy() * p["u"].numpy()
    z = p["z"].numpy()
    assert nmax_err(hf, h0) == 0.0
    assert nmax_err(y, pre * z * expit(z)) < 1e-14


@pytest.mark.parametrize("impl", IMPLS)
def test_p4_large_step_resets_state(impl):
    p = rand_problem(2, 17, 5, 3, seed=4, with_h0=True, with_z=False, with_D=False)
    p["delta_bias"] = torch.full((5,), 900.0, dtype=torch.float64)
    y, hf, _ = impl.scan_fwd(**p)
    dt = (p["delta"] + p["delta_bias"]).numpy()  # softplus(x) = x for huge x
    hexp = dt[:, :, :, None] * p["u"].numpy()[:, :, :, None] * p["B"].numpy()[:, :, None, :]
    yexp = np.einsum("bldn,bln->bld", hexp, p["C"].numpy())
    assert nmax_err(hf, hexp[:, -1]) < 1e-15
    assert nmax_err(y, yexp) < 1e-14


# --------------------------------------------------------------------------
# P-5  chunk split: the scan over L equals the scan over L1 followed by the
# scan over the rest started from the first part's final state.  Chunk states
# are the states at multiples of the chunk length.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("impl", IMPLS)
def test_p5_chunk_split_and_chunk_states(impl):
    p = rand_problem(2, 45, 4, 3, seed=9, with_h0=True)
    y, hf, cs = impl.scan_fwd(**p, chunk_len=8)
    L1 = 19
    first = {k: (v[:, :L1] if k in ("u", "delta", "z", "B", "C") else v) for k, v in p.items()}
    second = {k: (v[:, L1:] if k in ("u", "delta", "z", "B", "C") else v) for k, v in p.items()}
    y1, h1, _ = impl.scan_fwd(**first)
    second["h0"] = torch.from_numpy(h1)
    y2, h2, _ = impl.scan_fwd(**second)
    assert nmax_err(np.concatenate([y1, y2], axis=1), y) < 1e-13
    assert nmax_err(h2, hf) < 1e-13
    assert cs.shape == (2, 6, 4, 3)
    assert nmax_err(cs[:, 0], p["h0"]) == 0.0
    for k in range(1, 6):
        part = {kk: (v[:, :8 * k] if kk in ("u", "delta", "z", "B", "C") else v)
                for kk, v in p.items()}
        _, hk, _ = impl.scan_fwd(**part)
        assert nmax_err(cs[:, k], hk) < 1e-13


# --------------------------------------------------------------------------
# P-6  brute force: the recurrence unrolled into its explicit sum
# h_t = (prod_{r<=t} a_r) h0 + sum_{s<=t} (prod_{s<r<=t} a_r) delta_s B_s u_s,
# evaluated term by term (O(L^2)), on shapes where B, L, D, N all differ.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("impl", IMPLS)
def test_p6_unrolled_sum(impl):
    Bsz, L, D, N = 2, 9, 3, 4
    p = rand_problem(Bsz, L, D, N, seed=21, with_h0=True)
    y, hf, _ = impl.scan_fwd(**p)
    u, raw, A = p["u"].numpy(), p["delta"].numpy(), p["A"].numpy()
    Bm, Cm, Dsk, z = p["B"].numpy(), p["C"].numpy(), p["D"].numpy(), p["z"].numpy()
    bias, h0 = p["delta_bias"].numpy(), p["h0"].numpy()
    yexp = np.zeros((Bsz, L, D))
    hlast = np.zeros((Bsz, D, N))
    for b in range(Bsz):
        for d in range(D):
            dt = [math.log1p(math.exp(raw[b, t, d] + bias[d])) for t in range(L)]
            for n in range(N):
                a = [math.exp(dt[t] * A[d, n]) for t in range(L)]
                for t in range(L):
                    h = math.prod(a[0:t + 1]) * h0[b, d, n]
                    for s in range(t + 1):
                        h += math.prod(a[s + 1:t + 1]) * dt[s] * Bm[b, s, n] * u[b, s, d]
                    yexp[b, t, d] += Cm[b, t, n] * h
                    if t == L - 1:
                        hlast[b, d, n] = h
            for t in range(L):
                zz = z[b, t, d]
                yexp[b, t, d] = (yexp[b, t, d] + Dsk[d] * u[b, t, d]) * zz / (1.0 + math.exp(-zz))
    assert nmax_err(y, yexp) < 1e-12
    assert nmax_err(hf, hlast) < 1e-12


def test_p6_combine_is_associative():
    """The pair operator (a1,b1)o(a2,b2) = (a1 a2, a2 b1 + b2) composes two
    affine steps h -> a h + b; any bracketing gives the left fold exactly."""
    rng = np.random.default_rng(0)
    pairs = [(Fraction(int(rng.integers(-9, 10)), int(rng.integers(1, 7))),
              Fraction(int(rng.integers(-9, 10)), int(rng.integers(1, 7)))) for _ in range(16)]

    def comb(p, q):
        return (p[0] * q[0], q[0] * p[1] + q[1])

    left = pairs[0]
    for q in pairs[1:]:
        left = comb(left, q)

    def tree(xs):
        if len(xs) == 1:
            return xs[0]
        m = len(xs) // 2
        return comb(tree(xs[:m]), tree(xs[m:]))

    assert tree(pairs) == left
    h = Fraction(3, 7)
    for a, b in pairs:
        h = a * h + b
    assert left[0] * Fraction(3, 7) + left[1] == h


# --------------------------------------------------------------------------
# P-7  decode: L single-token updates equal one scan of length L.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("impl", IMPLS)
def test_p7_decode_equals_scan(impl):
    p = rand_problem(3, 12, 5, 4, seed=13, with_h0=True)
    y, hf, _ = impl.scan_fwd(**p)
    st = p["h0"].numpy()
    for t in range(12):
        st, yt = impl.state_update(st, p["u"][:, t], p["delta"][:, t], p["A"], p["B"][:, t],
                                   p["C"][:, t], p["D"], p["z"][:, t], p["delta_bias"], True)
        assert nmax_err(yt, y[:, t]) < 1e-14
    assert nmax_err(st, hf) < 1e-14


# --------------------------------------------------------------------------
# P-8  superposition: without the gate the scan is linear in (u, h0) when
# delta, B, C are held fixed.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("impl", IMPLS)
def test_p8_superposition(impl):
    p = rand_problem(2, 23, 4, 3, seed=17, with_h0=True, with_z=False)
    g = torch.Generator().manual_seed(99)
    u2 = torch.randn(p["u"].shape, generator=g, dtype=torch.float64)
    h2 = torch.randn(p["h0"].shape, generator=g, dtype=torch.float64)
    al, be = 0.7, -1.3
    y1, f1, _ = impl.scan_fwd(**p)
    q = dict(p, u=u2, h0=h2)
    y2, f2, _ = impl.scan_fwd(**q)
    r = dict(p, u=al * p["u"] + be * u2, h0=al * p["h0"] + be * h2)
    y3, f3, _ = impl.scan_fwd(**r)
    assert nmax_err(y3, al * y1 + be * y2) < 1e-13
    assert nmax_err(f3, al * f1 + be * f2) < 1e-13


# --------------------------------------------------------------------------
# P-10 the elementwise functions against library routines.
# --------------------------------------------------------------------------
def test_p10_softplus_silu(oracle_lib):
    for x in [-800.0, -40.0, -9.0, -1e-3, 0.0, 1e-8, 0.5, 3.0, 25.0, 700.0]:
        assert oracle_lib.softplus(x) == pytest.approx(float(np.logaddexp(0.0, x)), rel=1e-15,
                                                       abs=1e-300)
        assert oracle_lib.silu(x) == pytest.approx(x * float(expit(x)), rel=1e-15, abs=1e-300)


# --------------------------------------------------------------------------
# P-19 the scan of affine maps (the fold the library's wave-wide scan and the
# segment composition compute): exact against a fold in rational arithmetic,
# equal to the recurrence's own state trajectory, and reversal.
# --------------------------------------------------------------------------
def test_p19_affine_scan_exact_rational_fold(oracle_lib):
    """a = k/8, b, h0 small integers: every value is exact in fp64, so the fp64
    fold must equal the fold in fractions.Fraction digit for digit."""
    rng = np.random.default_rng(19)
    rows, length = 3, 14
    a = rng.integers(-8, 9, size=(rows, length)) / 8.0
    b = rng.integers(-10, 11, size=(rows, length)).astype(np.float64)
    h0 = rng.integers(-5, 6, size=rows).astype(np.float64)
    for reverse in (False, True):
        got = oracle_lib.affine_scan(a, b, h0, reverse=reverse)
        for r in range(rows):
            s = Fraction(int(h0[r]))
            order = range(length - 1, -1, -1) if reverse else range(length)
            for i in order:
                s = Fraction(int(a[r, i] * 8), 8) * s + Fraction(int(b[r, i]))
                assert got[r, i] == float(s) and Fraction(got[r, i]) == s


def test_p19_affine_scan_is_the_recurrence(oracle_lib):
    """With a_t = exp(dt_t A) and b_t = dt_t B_t u_t (one channel, one state),
    the fold is the scan's state trajectory, which the NumPy twin returns."""
    p = rand_problem(1, 40, 1, 1, seed=29, with_h0=True, with_z=False, with_D=False)
    _, _, _, states = oracle_np.scan_fwd(**p, return_states=True)
    dt = np.logaddexp(0.0, (p["delta"] + p["delta_bias"]).numpy()[0, :, 0])
    a = np.exp(dt * p["A"].numpy()[0, 0])
    b = dt * p["B"].numpy()[0, :, 0] * p["u"].numpy()[0, :, 0]
    h = oracle_lib.affine_scan(a[None], b[None], p["h0"].numpy()[0, 0][None])
    assert nmax_err(h[0], states[0, :, 0, 0]) < 1e-14


def test_p19_affine_scan_reverse_is_flipped_forward(oracle_lib):
    rng = np.random.default_rng(3)
    a, b = rng.uniform(0.2, 1.0, (2, 30)), rng.standard_normal((2, 30))
    h0 = rng.standard_normal(2)
    rev = oracle_lib.affine_scan(a, b, h0, reverse=True)
    fwd = oracle_lib.affine_scan(a[:, ::-1], b[:, ::-1], h0)
    assert np.array_equal(rev, fwd[:, ::-1])
