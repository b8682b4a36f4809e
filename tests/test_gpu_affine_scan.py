"""The wave-wide associative scan of affine maps (ssm_affine_scan, and the
segment composition of split sequences that uses the same primitive) against
the oracle's sequential fold, through the C ABI.

Inputs chosen so that every product and sum is exact in fp32 (a in {-1, 0,
1}, or powers of two with a single non-zero input term, integer b) make any
association of the scan give the same bits, so those cases are compared bit
for bit: a wrong lane shift, a missing identity or a wrong carry between
pieces of 64 changes integers.  Random inputs are compared within a bound."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import oracle_c
from tests.helpers import nmax_err

pytestmark = pytest.mark.gpu

LENGTHS = [1, 2, 17, 63, 64, 65, 128, 130, 1000]


@pytest.fixture(scope="module")
def ssm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import selective_state_space_10_amd as m
    m.load()
    return m


def _run(ssm, a, b, h0, reverse):
    print(f"affine scan rows={a.shape[0]} len={a.shape[1]} reverse={reverse}", flush=True)
    ga = torch.from_numpy(a.astype(np.float32)).cuda()
    gb = torch.from_numpy(b.astype(np.float32)).cuda()
    gh = None if h0 is None else torch.from_numpy(h0.astype(np.float32)).cuda()
    h = ssm.affine_scan(ga, gb, gh, reverse=reverse)
    torch.cuda.synchronize()
    return h.cpu().numpy(), oracle_c.affine_scan(a, b, h0, reverse=reverse)


@pytest.mark.parametrize("length", LENGTHS)
@pytest.mark.parametrize("reverse", [False, True])
def test_exact_signs_and_resets(ssm, length, reverse):
    """a in {-1, 0, 1} (sign flips and resets), integer b and h0: exact."""
    rng = np.random.default_rng(length + 7 * reverse)
    rows = 5
    a = rng.choice([-1.0, 0.0, 1.0, 1.0, 1.0], size=(rows, length))
    b = rng.integers(-50, 51, size=(rows, length)).astype(np.float64)
    h0 = rng.integers(-9, 10, size=rows).astype(np.float64)
    got, ref = _run(ssm, a, b, h0, reverse)
    assert np.array_equal(got.astype(np.float64), ref)


@pytest.mark.parametrize("length", [1, 5, 64, 65, 150])
@pytest.mark.parametrize("reverse", [False, True])
def test_exact_powers_of_two(ssm, length, reverse):
    """a = 2^k (k in -1..1) and a single non-zero input term at the first
    position in scan order: every state is h0 or b times a product of powers
    of two, exact in fp32."""
    rng = np.random.default_rng(100 + length)
    rows = 3
    a = 2.0 ** rng.integers(-1, 2, size=(rows, length))
    b = np.zeros((rows, length))
    first = length - 1 if reverse else 0
    b[:, first] = rng.integers(1, 100, size=rows)
    h0 = rng.integers(-4, 5, size=rows).astype(np.float64)
    got, ref = _run(ssm, a, b, h0, reverse)
    assert np.array_equal(got.astype(np.float64), ref)


@pytest.mark.parametrize("length", [64, 200, 4097])
def test_random_maps(ssm, length):
    """Decay factors in (0.5, 1) and Gaussian inputs, as in the recurrence:
    within fp32 rounding of the fp64 fold."""
    rng = np.random.default_rng(length)
    rows = 7
    a = rng.uniform(0.5, 1.0, size=(rows, length))
    b = rng.standard_normal((rows, length))
    for reverse in (False, True):
        got, ref = _run(ssm, a, b, None, reverse)
        assert nmax_err(got, ref) <= 1e-5


def test_rows_beyond_one_workgroup(ssm):
    """Rows not a multiple of the four waves of a workgroup (whole waves leave)."""
    rng = np.random.default_rng(5)
    a = rng.choice([-1.0, 1.0], size=(4097, 3))
    b = rng.integers(-9, 10, size=(4097, 3)).astype(np.float64)
    got, ref = _run(ssm, a, b, None, False)
    assert np.array_equal(got.astype(np.float64), ref)
