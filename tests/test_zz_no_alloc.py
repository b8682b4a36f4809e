"""The allocation-free forward (ssm_scan_fwd_noalloc) against the forward
with a caller workspace (ssm_scan_fwd_ex), through the C ABI: two calls in a
row on split sequences (so the static scratch is what the kernels use), the
second smaller, each identical to the workspace entry point and within the
oracle bound."""
from __future__ import annotations

import pytest
import torch

from oracle import oracle_c
from tests.helpers import nmax_err
from workloads import scan_inputs

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}
IO = {torch.float32: 0, torch.bfloat16: 1}


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import selective_state_space_10_amd as m
    return m.load()


def _p(t):
    return None if t is None else t.data_ptr()


def _run(lib, B, L, D, N, dtype, flags, seed):
    print(f"no-alloc forward B={B} L={L} D={D} N={N} {dtype} flags={flags}", flush=True)
    p = {k: (v.cuda() if isinstance(v, torch.Tensor) else v)
         for k, v in scan_inputs(B, L, D, N, dtype, seed=seed).items()}
    h0 = torch.randn(B, D, N, generator=torch.Generator().manual_seed(seed)).cuda()
    K = -(-L // lib.ssm_scan_chunk_len())
    stream = torch.cuda.current_stream().cuda_stream
    outs = []
    for noalloc in (False, True):
        y = torch.full_like(p["u"], float("nan"))
        hf = torch.full((B, D, N), float("nan"), device="cuda")
        cs = torch.full((B, K, N, D), float("nan"), device="cuda")
        ins = (B, L, D, N, IO[dtype], _p(p["u"]), _p(p["delta"]), _p(p["A"]), _p(p["B"]),
               _p(p["C"]), _p(p["D"]), _p(p["z"]), _p(p["delta_bias"]), 1, _p(h0), _p(hf), _p(y),
               _p(cs))
        if noalloc:
            st = lib.ssm_scan_fwd_noalloc(*ins, stream, flags)
        else:
            wsb = lib.ssm_scan_fwd_workspace_bytes(B, L, D, N, IO[dtype])
            assert 0 < wsb <= 16 << 20  # a split: the workspace (or the scratch) is used
            ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
            st = lib.ssm_scan_fwd_ex(*ins, _p(ws), wsb, stream, flags)
        assert st == 0, lib.ssm_last_error()
        torch.cuda.synchronize()
        outs.append((y, hf, cs))
    (y0, h0f, c0), (y1, h1f, c1) = outs
    assert torch.equal(y0, y1) and torch.equal(h0f, h1f) and torch.equal(c0, c1)
    pc = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in p.items()}
    yo, hfo, _ = oracle_c.scan_fwd(pc["u"], pc["delta"], pc["A"], pc["B"], pc["C"], pc["D"],
                                   pc["z"], pc["delta_bias"], True, h0.cpu(),
                                   reverse=bool(flags & 2))
    assert nmax_err(y1, yo) <= TOL[dtype]
    assert nmax_err(h1f, hfo) <= TOL[dtype]


def test_noalloc_forward_matches_the_workspace_forward(lib):
    _run(lib, 1, 20000, 24, 16, torch.float32, 0, seed=1)
    _run(lib, 1, 9000, 16, 16, torch.bfloat16, 2, seed=2)  # smaller, reverse direction


def test_noalloc_forward_with_first_pass_pieces(lib):
    """Splits whose first pass runs in pieces (the pieces' end states and the
    segments' start states share the static scratch): 6 segments of 2 pieces,
    then a smaller one of 3 segments of 2 pieces in reverse."""
    _run(lib, 1, 24576, 24, 16, torch.float32, 0, seed=5)
    _run(lib, 1, 12288, 16, 16, torch.bfloat16, 2, seed=6)


def test_noalloc_forward_without_split_and_other_states(lib):
    """Sizes that need no workspace, and a split with 4 states (the
    all-purpose kernel's split)."""
    _run_plain = _run
    B, L, D, N = 2, 300, 72, 16
    assert lib.ssm_scan_fwd_workspace_bytes(B, L, D, N, 0) == 0
    p = {k: (v.cuda() if isinstance(v, torch.Tensor) else v)
         for k, v in scan_inputs(B, L, D, N, torch.float32, seed=3).items()}
    y = torch.empty_like(p["u"])
    st = lib.ssm_scan_fwd_noalloc(B, L, D, N, 0, _p(p["u"]), _p(p["delta"]), _p(p["A"]),
                                  _p(p["B"]), _p(p["C"]), _p(p["D"]), _p(p["z"]),
                                  _p(p["delta_bias"]), 1, None, None, _p(y), None,
                                  torch.cuda.current_stream().cuda_stream, 0)
    assert st == 0
    torch.cuda.synchronize()
    pc = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in p.items()}
    yo, _, _ = oracle_c.scan_fwd(pc["u"], pc["delta"], pc["A"], pc["B"], pc["C"], pc["D"],
                                 pc["z"], pc["delta_bias"], True)
    assert nmax_err(y, yo) <= 1e-4
    _run_plain(lib, 2, 9000, 24, 4, torch.float32, 0, seed=4)
