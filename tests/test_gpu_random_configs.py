"""Seeded random configurations: the HIP forward and backward against the fp64
oracle on shapes, dtypes and option sets drawn together, so that combinations
no hand-picked case names (ragged channel tiles with per-token steps, reverse
scans with the exact hold and no gate, sequence splits with a start state ...)
are compared element by element as well.  The draw is fixed (one seed), so
every run checks the same cases.  Tolerances are the parity bounds of the
other tests: max|gpu - oracle| / max|oracle| <= 1e-4 (fp32), 2e-2 (bf16).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import oracle_c
from tests.helpers import nmax_err
from tests.test_gpu_conv import _check_bwd as _check_bwd_conv
from tests.test_gpu_conv import _conv_problem, _gpu_fwd as _gpu_fwd_conv, _okw
from tests.test_gpu_options import _check_bwd, _check_fwd, _with_opts
from tests.test_gpu_parity import TOL, _problem, _to

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ssm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import selective_state_space_10_amd as m
    m.load()
    return m


def _draw_cases(n_short=60, n_long=12, seed=20240611):
    """Short cases: up to 3 rows, up to 1200 steps, up to 320 channels.  Long
    cases: one row, 8200-14000 steps, few channels, so the launcher splits the
    sequence into segments."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n_short + n_long):
        long = i >= n_short
        if long:
            B, L, D = 1, int(rng.integers(8200, 14001)), int(8 * rng.integers(1, 4))
        else:
            B = int(rng.integers(1, 4))
            L = int(np.exp(rng.uniform(0.0, np.log(1200.0))))
            D = int(8 * rng.integers(1, 41))
        N = int(rng.choice([1, 2, 4, 8, 16]))
        dtype = torch.float32 if rng.random() < 0.5 else torch.bfloat16
        flags = dict(z=rng.random() < 0.7, Dskip=rng.random() < 0.7, bias=rng.random() < 0.7,
                     softplus=rng.random() < 0.8, h0=rng.random() < 0.5,
                     generic_A=rng.random() < 0.5)
        opts = dict(zoh=bool(rng.random() < 0.3), reverse=bool(rng.random() < 0.3),
                    tok=bool(rng.random() < 0.3))
        cases.append((B, L, D, N, dtype, {k: bool(v) for k, v in flags.items()}, opts, 1000 + i))
    return cases


CASES = _draw_cases()


def _case_id(c):
    B, L, D, N, dtype, flags, opts, _ = c
    on = [k for k, v in {**flags, **opts}.items() if v]
    return f"{B}x{L}x{D}x{N}-{'f32' if dtype == torch.float32 else 'bf16'}-" + "+".join(on)


@pytest.mark.parametrize("case", CASES, ids=[_case_id(c) for c in CASES])
def test_random_config_fwd_bwd(ssm, case):
    B, L, D, N, dtype, flags, opts, seed = case
    print(f"case {_case_id(case)} seed {seed}", flush=True)
    p = _with_opts(_problem(B, L, D, N, dtype, seed=seed, **flags), opts["tok"])
    _check_fwd(ssm, p, TOL[dtype], zoh=opts["zoh"], reverse=opts["reverse"])
    _check_bwd(ssm, p, TOL[dtype], zoh=opts["zoh"], reverse=opts["reverse"], seed=seed)


def _draw_conv_cases(n_short=24, n_long=4, seed=20240612):
    """The fused causal convolution in front of the scan (forward in time
    only): width 1-4, with or without the convolution's bias, the gate, the
    skip term, one step size per token and the exact hold."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n_short + n_long):
        if i >= n_short:
            B, L, D = 1, int(rng.integers(8200, 12001)), int(8 * rng.integers(1, 3))
        else:
            B = int(rng.integers(1, 4))
            L = int(np.exp(rng.uniform(0.0, np.log(900.0))))
            D = int(8 * rng.integers(1, 31))
        N = int(rng.choice([1, 2, 4, 8, 16]))
        dtype = torch.float32 if rng.random() < 0.5 else torch.bfloat16
        K = int(rng.integers(1, 5))
        kw = dict(bias=bool(rng.random() < 0.7), tok=bool(rng.random() < 0.3),
                  z=bool(rng.random() < 0.7), Dskip=bool(rng.random() < 0.7),
                  generic_A=bool(rng.random() < 0.5))
        cases.append((B, L, D, N, dtype, K, kw, bool(rng.random() < 0.3), 2000 + i))
    return cases


CONV_CASES = _draw_conv_cases()


def _conv_case_id(c):
    B, L, D, N, dtype, K, kw, zoh, _ = c
    on = [k for k, v in {**kw, "zoh": zoh}.items() if v]
    return f"{B}x{L}x{D}x{N}-k{K}-{'f32' if dtype == torch.float32 else 'bf16'}-" + "+".join(on)


@pytest.mark.parametrize("case", CONV_CASES, ids=[_conv_case_id(c) for c in CONV_CASES])
def test_random_config_conv_fwd_bwd(ssm, case):
    B, L, D, N, dtype, K, kw, zoh, seed = case
    print(f"case {_conv_case_id(case)} seed {seed}", flush=True)
    p = _conv_problem(B, L, D, N, dtype, K, seed=seed, **kw)
    tol = TOL[dtype]
    y, hf, cs = _gpu_fwd_conv(ssm, _to(p, "cuda"), zoh, return_final_state=True,
                              save_chunk_states=True)
    torch.cuda.synchronize()
    yo, hfo, cso = oracle_c.scan_fwd_conv(**_okw(p), chunk_len=ssm.chunk_len(), zoh=zoh)
    assert nmax_err(y, yo) <= tol
    assert nmax_err(hf, hfo) <= tol
    assert nmax_err(cs.permute(0, 1, 3, 2), cso) <= tol
    _check_bwd_conv(ssm, p, tol, zoh=zoh, seed=seed)
