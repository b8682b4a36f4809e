"""HIP path with options (exact zero-order hold, reverse direction, one step
size per token, accumulation into y) against the fp64 oracle with the same
options, element by element, through the C ABI.  Same tolerances as the plain
path: max|gpu - oracle| / max|oracle| <= 1e-4 (fp32 inputs), 2e-2 (bf16)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import oracle_c
from tests.helpers import nmax_err
from tests.test_gpu_parity import GRADS, TOL, _oracle_kwargs, _problem, _slice_channels, _to
from workloads import WORKLOADS, cotangent, decode_inputs, workload_inputs

pytestmark = pytest.mark.gpu

OPTS = [dict(zoh=True), dict(reverse=True), dict(tok=True), dict(zoh=True, reverse=True, tok=True)]
OPT_IDS = ["zoh", "reverse", "per-token", "all"]


@pytest.fixture(scope="module")
def ssm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import selective_state_space_10_amd as m
    m.load()
    return m


def _with_opts(p, tok):
    if tok:  # one raw step size per token
        p = dict(p, delta=p["delta"][:, :, 0].contiguous())
    return p


def _fwd(ssm, p, zoh=False, reverse=False, **kw):
    return ssm.scan_fwd(p["u"], p["delta"], p["A"], p["B"], p["C"], p.get("D"), p.get("z"),
                        p.get("delta_bias"), p.get("delta_softplus", True), p.get("h0"),
                        zoh=zoh, reverse=reverse, **kw)


def _check_fwd(ssm, p, tol, zoh=False, reverse=False):
    T = ssm.chunk_len()
    y, hf, cs = _fwd(ssm, _to(p, "cuda"), zoh, reverse, return_final_state=True,
                     save_chunk_states=True)
    torch.cuda.synchronize()
    yo, hfo, cso = oracle_c.scan_fwd(**_oracle_kwargs(p), chunk_len=T, zoh=zoh, reverse=reverse)
    assert nmax_err(y, yo) <= tol
    assert nmax_err(hf, hfo) <= tol
    assert nmax_err(cs.permute(0, 1, 3, 2), cso) <= tol


@pytest.mark.parametrize("opts", OPTS, ids=OPT_IDS)
@pytest.mark.parametrize("B,L,D,N,dtype", [
    (2, 300, 72, 16, torch.float32), (2, 300, 72, 16, torch.bfloat16),
    (3, 97, 136, 8, torch.float32), (2, 45, 64, 1, torch.float32), (1, 70, 16, 2, torch.bfloat16)])
def test_fwd_options_small(ssm, opts, B, L, D, N, dtype):
    p = _with_opts(_problem(B, L, D, N, dtype, seed=L + N, h0=True, generic_A=True), opts.get("tok"))
    _check_fwd(ssm, p, TOL[dtype], opts.get("zoh", False), opts.get("reverse", False))


@pytest.mark.parametrize("zoh", [True, False], ids=["zoh", "no-zoh"])
@pytest.mark.parametrize("B,L,D,N,dtype", [(1, 10000, 16, 16, torch.float32),
                                           (2, 9000, 24, 8, torch.bfloat16),
                                           (1, 9001, 72, 16, torch.bfloat16)])
def test_fwd_options_sequence_split(ssm, B, L, D, N, dtype, zoh):
    """Reverse direction and one step size per token over a split sequence
    (16 states without the exact hold: segments scanned by the wave-specialised
    kernel)."""
    p = _with_opts(_problem(B, L, D, N, dtype, seed=7, h0=True), True)
    _check_fwd(ssm, p, TOL[dtype], zoh=zoh, reverse=True)


@pytest.mark.parametrize("opts", [dict(), dict(zoh=True, reverse=True, tok=True)], ids=["plain", "all"])
@pytest.mark.parametrize("B,L,D,dtype", [(1, 24576, 24, torch.float32), (2, 12288, 16, torch.bfloat16)])
def test_fwd_split_first_pass_in_pieces(ssm, B, L, D, dtype, opts):
    """A split whose first pass leaves most CUs idle cuts each segment into
    pieces for that pass (ssm_scan_fwd_plan reports their length); the start
    states of the segments are the composition of the pieces' maps."""
    p = _with_opts(_problem(B, L, D, 16, dtype, seed=L % 101, h0=True, generic_A=True), opts.get("tok"))
    plan = ssm.scan_fwd_plan(B, L, D, 16, dtype, zoh=opts.get("zoh", False),
                             reverse=opts.get("reverse", False), per_token=opts.get("tok", False))
    assert plan["segments"] > 1 and plan["segment_len"] // plan["first_pass_len"] >= 2, plan
    _check_fwd(ssm, p, TOL[dtype], opts.get("zoh", False), opts.get("reverse", False))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_fwd_accumulate_and_bidirectional(ssm, dtype):
    p = _problem(2, 150, 72, 16, dtype, seed=31)
    pg = _to(p, "cuda")
    base = torch.randn(p["u"].shape, generator=torch.Generator().manual_seed(3)).to(dtype)
    out = base.cuda().clone()
    _fwd(ssm, pg, zoh=True, out=out)
    torch.cuda.synchronize()
    yo, _, _ = oracle_c.scan_fwd(**_oracle_kwargs(p), zoh=True)
    ref = yo + base.double().numpy()
    assert nmax_err(out, ref) <= TOL[dtype]
    yb = ssm.bidirectional_scan(pg["u"], pg["delta"], pg["A"], pg["B"], pg["C"], pg["D"], pg["z"],
                                pg["delta_bias"], True)
    torch.cuda.synchronize()
    ok = _oracle_kwargs(p)
    yf, _, _ = oracle_c.scan_fwd(**ok)
    yr, _, _ = oracle_c.scan_fwd(**dict(ok, D=None), reverse=True)
    # bf16: the forward launch rounds y, the reverse launch adds to it and
    # rounds again; emulated on the oracle's outputs that costs at most about
    # 4e-3 of max|y| here, within the bf16 bound
    assert nmax_err(yb, yf + yr) <= TOL[dtype]


def test_bidirectional_sequence_split(ssm):
    """Both directions over a split sequence (the reverse launch accumulates
    into y)."""
    p = _problem(1, 10000, 16, 16, torch.float32, seed=13)
    pg = _to(p, "cuda")
    yb = ssm.bidirectional_scan(pg["u"], pg["delta"], pg["A"], pg["B"], pg["C"], pg["D"], pg["z"],
                                pg["delta_bias"], True)
    torch.cuda.synchronize()
    ok = _oracle_kwargs(p)
    yf, _, _ = oracle_c.scan_fwd(**ok)
    yr, _, _ = oracle_c.scan_fwd(**dict(ok, D=None), reverse=True)
    assert nmax_err(yb, yf + yr) <= TOL[torch.float32]


def test_fwd_zoh_workload1_full_size(ssm):
    """The Mamba-370m shape with the exact hold, on sampled channels."""
    w = WORKLOADS[1]
    p = workload_inputs(1, device="cuda")
    y, hf, _ = _fwd(ssm, p, zoh=True, return_final_state=True)
    torch.cuda.synchronize()
    g = torch.Generator().manual_seed(11)
    sel = torch.randperm(w.dim, generator=g)[:16].sort().values
    ps = _slice_channels(p, sel.cuda())
    yo, hfo, _ = oracle_c.scan_fwd(**_oracle_kwargs(ps), zoh=True)
    assert nmax_err(y[:, :, sel.cuda()], yo) <= TOL[w.io_dtype]
    assert nmax_err(hf[:, sel.cuda()], hfo) <= TOL[w.io_dtype]


def _check_bwd(ssm, p, tol, zoh=False, reverse=False, seed=0):
    pg = _to(p, "cuda")
    y, hf, cs = _fwd(ssm, pg, zoh, reverse, return_final_state=True, save_chunk_states=True)
    dy = cotangent(y, seed)
    dhf = torch.randn(hf.shape, generator=torch.Generator().manual_seed(seed)).cuda()
    gr = ssm.scan_bwd(pg["u"], pg["delta"], pg["A"], pg["B"], pg["C"], pg.get("D"), pg.get("z"),
                      pg.get("delta_bias"), p.get("delta_softplus", True), pg.get("h0"), cs, dy,
                      dhf, zoh=zoh, reverse=reverse)
    torch.cuda.synchronize()
    go = oracle_c.scan_bwd(**_oracle_kwargs(p), dy=dy.cpu(), dh_final=dhf.cpu(), zoh=zoh,
                           reverse=reverse)
    for k in GRADS:
        if go[k] is None or gr.get(k) is None:
            continue
        assert tuple(gr[k].shape) == go[k].shape, k
        err = nmax_err(gr[k], go[k])
        assert err <= tol, (k, err)


@pytest.mark.parametrize("opts", OPTS, ids=OPT_IDS)
@pytest.mark.parametrize("B,L,D,N,dtype", [
    (2, 300, 72, 16, torch.float32), (2, 300, 72, 16, torch.bfloat16),
    (3, 97, 136, 8, torch.float32), (2, 45, 64, 1, torch.float32)])
def test_bwd_options_small(ssm, opts, B, L, D, N, dtype):
    p = _with_opts(_problem(B, L, D, N, dtype, seed=L + 2 * N, h0=True, generic_A=True),
                   opts.get("tok"))
    _check_bwd(ssm, p, TOL[dtype], opts.get("zoh", False), opts.get("reverse", False), seed=N)


@pytest.mark.parametrize("B,L,D,N,dtype", [(1, 5000, 16, 16, torch.float32),
                                           (1, 6000, 8, 16, torch.bfloat16)])
def test_bwd_options_sequence_split(ssm, B, L, D, N, dtype):
    p = _with_opts(_problem(B, L, D, N, dtype, seed=5, h0=True), True)
    _check_bwd(ssm, p, TOL[dtype], zoh=True, reverse=True, seed=L)


@pytest.mark.parametrize("N", [1, 4, 16])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_decode_zoh(ssm, N, dtype):
    d = decode_inputs(3, 72, N, 4, dtype, seed=N + 50)
    dg = _to(d, "cuda")
    state = dg["state"].clone()
    so = d["state"]
    for t in range(4):
        yt = ssm.state_update(state, dg["u"][t], dg["delta"][t], dg["A"], dg["B"][t], dg["C"][t],
                              dg["D"], dg["z"][t], dg["delta_bias"], True, zoh=True)
        so, yo = oracle_c.state_update(so, d["u"][t], d["delta"][t], d["A"], d["B"][t], d["C"][t],
                                       d["D"], d["z"][t], d["delta_bias"], True, zoh=True)
        torch.cuda.synchronize()
        assert nmax_err(yt, yo) <= TOL[dtype]
    assert nmax_err(state, so) <= TOL[dtype]


def test_autograd_with_options(ssm):
    p = _to(_problem(2, 130, 64, 16, torch.float32, seed=23, h0=True), "cuda")
    leaves = {k: p[k].clone().requires_grad_(True) for k in
              ("u", "delta", "A", "B", "C", "D", "z", "delta_bias", "h0")}
    y, hf = ssm.selective_scan(leaves["u"], leaves["delta"], leaves["A"], leaves["B"],
                               leaves["C"], leaves["D"], leaves["z"], leaves["delta_bias"], True,
                               leaves["h0"], zoh=True, reverse=True)
    dy = cotangent(y.detach(), 2)
    (y * dy).sum().backward()
    pc = {k: v.detach().cpu() for k, v in p.items() if isinstance(v, torch.Tensor)}
    pc["delta_softplus"] = True
    go = oracle_c.scan_bwd(**_oracle_kwargs(pc), dy=dy.cpu(), zoh=True, reverse=True)
    names = dict(u="du", delta="ddelta", A="dA", B="dB", C="dC", D="dD", z="dz",
                 delta_bias="ddelta_bias", h0="dh0")
    for k, g in names.items():
        assert nmax_err(leaves[k].grad, go[g]) <= 1e-4, k
