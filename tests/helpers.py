"""Shared test helpers: error metric and small random problems."""
from __future__ import annotations

import numpy as np
import torch


def nmax_err(got, ref) -> float:
    """max_i |got - ref| / max_i |ref| over one output tensor (0 if both are 0)."""
    got = np.asarray(got.detach().cpu().double() if hasattr(got, "detach") else got, np.float64)
    ref = np.asarray(ref.detach().cpu().double() if hasattr(ref, "detach") else ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if got.size == 0:
        return 0.0
    assert not np.isnan(got).any(), "NaN in result"
    scale = np.abs(ref).max()
    diff = np.abs(got - ref).max()
    if scale == 0.0:
        return float(diff)
    return float(diff / scale)


def rand_problem(B, L, D, N, seed=0, *, with_z=True, with_D=True, with_bias=True, with_h0=False,
                 softplus=True, dtype=torch.float64):
    """A random scan problem with generic (non-structured) A, for oracle pins."""
    g = torch.Generator().manual_seed(seed)
    r = lambda *s: torch.randn(*s, generator=g, dtype=torch.float64)
    p = dict(
        u=r(B, L, D), delta=r(B, L, D) * 0.5 - (1.0 if softplus else -0.5),
        A=-torch.rand(D, N, generator=g, dtype=torch.float64) * 2.0 - 0.1,
        B=r(B, L, N), C=r(B, L, N),
        D=r(D) if with_D else None, z=r(B, L, D) if with_z else None,
        delta_bias=(r(D) * 0.3) if with_bias else None, delta_softplus=softplus,
        h0=r(B, D, N) if with_h0 else None)
    if dtype != torch.float64:
        p = {k: (v.to(dtype) if isinstance(v, torch.Tensor) else v) for k, v in p.items()}
    return p


def parity_report(name, got, ref) -> dict:
    """The per-output-tensor error reported beside the gated metric: the
    normalised max error, the largest per-element relative error over entries
    with |ref| >= 1e-3 max|ref|, its index, and the NaN count (which must be 0).
    Printed, so that it appears in the test log."""
    g = np.asarray(got.detach().cpu().double() if hasattr(got, "detach") else got, np.float64)
    r = np.asarray(ref.detach().cpu().double() if hasattr(ref, "detach") else ref, np.float64)
    nan = int(np.isnan(g).sum())
    scale = float(np.abs(r).max()) if r.size else 0.0
    mask = np.abs(r) >= 1e-3 * scale
    rel = np.where(mask, np.abs(g - r) / np.where(mask, np.abs(r), 1.0), 0.0)
    worst = np.unravel_index(int(np.argmax(rel)), rel.shape) if rel.size else ()
    rep = {"tensor": name, "nmax_err": nmax_err(g, r) if not nan else float("nan"),
           "max_rel_err_significant": float(rel.max()) if rel.size else 0.0,
           "worst_index": tuple(int(i) for i in worst), "nan_count": nan}
    print("parity", rep, flush=True)
    return rep
