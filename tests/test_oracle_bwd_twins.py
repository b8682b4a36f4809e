"""Oracle backward against central finite differences of the oracle forward,
and the C oracle against its independent NumPy twin."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import oracle_c, oracle_np
from tests.helpers import nmax_err, rand_problem
from workloads import WORKLOADS, decode_inputs, scan_inputs

GRAD_OF = dict(u="du", delta="ddelta", A="dA", B="dB", C="dC", D="dD", z="dz",
               delta_bias="ddelta_bias", h0="dh0")


def _loss(impl, p, w, G):
    y, hf, _ = impl.scan_fwd(**p)
    return float((y * w).sum() + (hf * G).sum())


# --------------------------------------------------------------------------
# P-9  backward = gradient of the forward: central differences, every element
# of every differentiable input, loss = <y, dy> + <h_final, dh_final>.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("impl", [oracle_c, oracle_np], ids=["c", "np"])
@pytest.mark.parametrize("opts", [dict(), dict(softplus=False, with_z=False, with_D=False,
                                                  with_bias=False)], ids=["all", "bare"])
def test_p9_backward_matches_finite_differences(impl, opts):
    Bsz, L, D, N = 2, 6, 3, 2
    p = rand_problem(Bsz, L, D, N, seed=31, with_h0=True, **opts)
    g = torch.Generator().manual_seed(5)
    w = torch.randn(Bsz, L, D, generator=g, dtype=torch.float64).numpy()
    G = torch.randn(Bsz, D, N, generator=g, dtype=torch.float64).numpy()
    grads = impl.scan_bwd(**p, dy=w, dh_final=G)
    eps = 1e-6
    for name, gname in GRAD_OF.items():
        if p.get(name) is None:
            assert grads[gname] is None or name == "h0"
            continue
        base = p[name].clone()
        fd = np.empty(base.shape)
        for i in range(base.numel()):
            vals = []
            for sgn in (1, -1):
                x = base.clone().view(-1)
                x[i] += sgn * eps
                vals.append(_loss(impl, dict(p, **{name: x.view(base.shape)}), w, G))
            fd.reshape(-1)[i] = (vals[0] - vals[1]) / (2 * eps)
        err = nmax_err(grads[gname], fd)
        assert err < 2e-7, (name, err)


@pytest.mark.parametrize("impl", [oracle_c, oracle_np], ids=["c", "np"])
@pytest.mark.parametrize("opts", [dict(), dict(zoh=True), dict(reverse=True)],
                         ids=["plain", "zoh", "reverse"])
def test_p9_dot_product_linear_part(impl, opts):
    """Without the gate, and with delta, B, C fixed, (y, h_final) is linear in
    (u, h0), so the backward's du, dh0 must be the exact adjoint of that map:
    <J v, w> = <v, J^T w> for random v = (v_u, v_h0) and w = (w_y, w_h) to
    rounding (the forward applied to v is J v itself)."""
    kw = {k: v for k, v in opts.items()}
    p = rand_problem(2, 19, 5, 4, seed=41, with_h0=True, with_z=False)
    g = torch.Generator().manual_seed(8)
    vu = torch.randn(p["u"].shape, generator=g, dtype=torch.float64)
    vh = torch.randn(p["h0"].shape, generator=g, dtype=torch.float64)
    wy = torch.randn(p["u"].shape, generator=g, dtype=torch.float64).numpy()
    wh = torch.randn(p["h0"].shape, generator=g, dtype=torch.float64).numpy()
    q = dict(p, u=vu, h0=vh, D=p["D"])
    yv, hv, _ = impl.scan_fwd(**q, **kw)
    lhs = float((yv * wy).sum() + (hv * wh).sum())
    gr = impl.scan_bwd(**q, dy=wy, dh_final=wh, **kw)
    rhs = float((gr["du"] * vu.numpy()).sum() + (gr["dh0"] * vh.numpy()).sum())
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs)), (lhs, rhs)


@pytest.mark.parametrize("impl", [oracle_c, oracle_np], ids=["c", "np"])
def test_p9_dot_product_full_map(impl):
    """The whole nonlinear map, all nine inputs at once: the directional
    derivative along a random direction v (central difference of the fp64
    forward) equals <v, J^T w> from the backward."""
    p = rand_problem(2, 9, 3, 2, seed=43, with_h0=True)
    g = torch.Generator().manual_seed(9)
    w = torch.randn(p["u"].shape, generator=g, dtype=torch.float64).numpy()
    G = torch.randn(p["h0"].shape, generator=g, dtype=torch.float64).numpy()
    names = [k for k in GRAD_OF if p.get(k) is not None]
    v = {k: torch.randn(p[k].shape, generator=g, dtype=torch.float64) for k in names}
    grads = impl.scan_bwd(**p, dy=w, dh_final=G)
    rhs = sum(float((grads[GRAD_OF[k]] * v[k].numpy()).sum()) for k in names)
    eps = 1e-6
    plus = dict(p, **{k: p[k] + eps * v[k] for k in names})
    minus = dict(p, **{k: p[k] - eps * v[k] for k in names})
    lhs = (_loss(impl, plus, w, G) - _loss(impl, minus, w, G)) / (2 * eps)
    assert abs(lhs - rhs) <= 1e-7 * max(1.0, abs(rhs)), (lhs, rhs)


def test_p9_backward_without_final_cotangent():
    p = rand_problem(1, 5, 2, 3, seed=2)
    w = np.random.default_rng(0).normal(size=(1, 5, 2))
    a = oracle_c.scan_bwd(**p, dy=w)
    b = oracle_c.scan_bwd(**p, dy=w, dh_final=np.zeros((1, 2, 3)))
    for k in a:
        if a[k] is not None:
            assert np.array_equal(a[k], b[k]), k


# --------------------------------------------------------------------------
# P-11 the two oracles agree (they share no code).
# --------------------------------------------------------------------------
def _twins_fwd(p, chunk_len=None):
    yc, hc, cc = oracle_c.scan_fwd(**p, chunk_len=chunk_len, nthreads=3)
    yn, hn, cn = oracle_np.scan_fwd(**p, chunk_len=chunk_len)
    assert nmax_err(yc, yn) < 1e-12
    assert nmax_err(hc, hn) < 1e-12
    if chunk_len:
        assert nmax_err(cc, cn) < 1e-12


def test_p11_twins_workload0():
    w = WORKLOADS[0]
    p = scan_inputs(w.batch, w.seqlen, w.dim, w.dstate, w.io_dtype, seed=0)
    _twins_fwd(p, chunk_len=16)


@pytest.mark.parametrize("seed", range(4))
def test_p11_twins_random(seed):
    rng = np.random.default_rng(seed)
    Bsz, L, D, N = (int(rng.integers(1, 4)), int(rng.integers(1, 70)), int(rng.integers(1, 9)),
                    int(rng.choice([1, 2, 4, 8, 16])))
    opts = dict(with_z=bool(seed % 2), with_D=bool(seed % 3), with_bias=seed != 2,
                with_h0=seed > 1, softplus=seed != 3)
    p = rand_problem(Bsz, L, D, N, seed=seed, **opts)
    _twins_fwd(p, chunk_len=int(rng.integers(1, 20)))
    dy = rng.normal(size=(Bsz, L, D))
    G = rng.normal(size=(Bsz, D, N))
    gc = oracle_c.scan_bwd(**p, dy=dy, dh_final=G, nthreads=2)
    gn = oracle_np.scan_bwd(**p, dy=dy, dh_final=G)
    for k, v in gc.items():
        if v is None:
            assert gn[k] is None, k
        else:
            assert nmax_err(v, gn[k]) < 1e-12, k


def test_p11_twins_mamba370m_slice():
    """Workload 1's value distributions at its full length, a few channels."""
    p = scan_inputs(2, 2048, 16, 16, torch.float32, seed=1)
    _twins_fwd(p)


def test_p11_twins_decode():
    d = decode_inputs(4, 24, 16, 3, torch.bfloat16, seed=3)
    sc = sn = d["state"]
    for t in range(3):
        args = [d["u"][t], d["delta"][t], d["A"], d["B"][t], d["C"][t], d["D"], d["z"][t],
                d["delta_bias"], True]
        sc, yc = oracle_c.state_update(sc, *args)
        sn, yn = oracle_np.state_update(sn, *args)
        assert nmax_err(yc, yn) < 1e-12
        assert nmax_err(sc, sn) < 1e-12
