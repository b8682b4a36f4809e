"""HIP path against the fp64 oracle, element by element, through the C ABI.

Tolerance (per output tensor): max|gpu - oracle| / max|oracle| <= 1e-4 for
fp32 inputs and <= 2e-2 for bf16 inputs (fp32 arithmetic on the GPU).  Small
shapes are compared in full; the full-size workloads are compared on sampled
channels (channels are independent recurrences, so the oracle runs on the
sliced channels), or through a cotangent that is zero outside the sampled
channels for sums over channels.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import oracle_c
from tests.helpers import nmax_err, parity_report
from workloads import WORKLOADS, cotangent, decode_inputs, scan_inputs, workload_inputs

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


@pytest.fixture(scope="module")
def ssm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import selective_state_space_10_amd as m
    m.load()
    return m


def _to(p, device):
    return {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in p.items()}


def _slice_channels(p, sel):
    """Inputs restricted to channels `sel` (a 1-D index tensor)."""
    out = {}
    for k, v in p.items():
        if not isinstance(v, torch.Tensor):
            out[k] = v
        elif k in ("u", "delta", "z", "dy"):
            out[k] = v[:, :, sel].cpu()
        elif k in ("A", "D", "delta_bias"):
            out[k] = v[sel].cpu()
        elif k in ("h0", "state", "dh_final"):
            out[k] = v[:, sel].cpu()
        else:  # B, C shared by all channels
            out[k] = v.cpu()
    return out


def _oracle_kwargs(p):
    keys = ("u", "delta", "A", "B", "C", "D", "z", "delta_bias", "delta_softplus", "h0")
    return {k: p.get(k) for k in keys}


def _gpu_fwd(ssm, p, **kw):
    return ssm.scan_fwd(p["u"], p["delta"], p["A"], p["B"], p["C"], p.get("D"), p.get("z"),
                        p.get("delta_bias"), p.get("delta_softplus", True), p.get("h0"), **kw)


def _problem(B, L, D, N, dtype, seed, *, z=True, Dskip=True, bias=True, softplus=True, h0=False,
             generic_A=False):
    p = scan_inputs(B, L, D, N, dtype, seed=seed, with_z=z, with_D=Dskip, with_bias=bias)
    g = torch.Generator().manual_seed(seed + 77)
    if not softplus:  # step size used as given: keep it positive
        p["delta_softplus"] = False
        p["delta"] = (p["delta"].float().abs() * 0.05).to(dtype)
        if p.get("delta_bias") is not None:
            p["delta_bias"] = torch.rand(D, generator=g) * 0.05 + 1e-3
    if h0:
        p["h0"] = torch.randn(B, D, N, generator=g)
    if generic_A:
        p["A"] = -(torch.rand(D, N, generator=g) * 8 + 0.05)
    return p


def _check_fwd(ssm, p, tol, chunk=True):
    T = ssm.chunk_len()
    pg = _to(p, "cuda")
    y, hf, cs = _gpu_fwd(ssm, pg, return_final_state=True, save_chunk_states=chunk)
    torch.cuda.synchronize()
    yo, hfo, cso = oracle_c.scan_fwd(**_oracle_kwargs(p), chunk_len=T if chunk else None)
    assert nmax_err(y, yo) <= tol
    assert nmax_err(hf, hfo) <= tol
    if chunk:  # the library keeps chunk states as (B, K, N, D), the oracle as (B, K, D, N)
        assert nmax_err(cs.permute(0, 1, 3, 2), cso) <= tol
    return y


SMALL = [
    # B, L, D, N, dtype
    (1, 64, 32, 4, torch.float32),  # workload 0's shape
    (2, 300, 72, 16, torch.float32),  # 2 channel tiles (ragged), 2 chunks (ragged)
    (2, 300, 72, 16, torch.bfloat16),
    (3, 97, 136, 8, torch.float32),
    (3, 97, 136, 8, torch.bfloat16),
    (2, 45, 64, 2, torch.float32),
    (2, 45, 64, 1, torch.bfloat16),
    (1, 1, 8, 16, torch.float32),  # single step, smallest dim
    (1, 513, 8, 4, torch.float32),  # length just past two chunks
]


@pytest.mark.parametrize("B,L,D,N,dtype", SMALL)
def test_fwd_small(ssm, B, L, D, N, dtype):
    _check_fwd(ssm, _problem(B, L, D, N, dtype, seed=B * 1000 + L + N), TOL[dtype])


@pytest.mark.parametrize("B,L,D,N,dtype", [
    (1, 10000, 16, 16, torch.float32), (1, 10000, 16, 16, torch.bfloat16),
    (2, 9000, 24, 8, torch.float32), (1, 12289, 8, 2, torch.float32)])
def test_fwd_sequence_split(ssm, B, L, D, N, dtype):
    """Few channels and a long sequence: the forward splits the sequence into
    segments (local end states, then their composition, then the scan of each
    segment from its true initial state)."""
    lib = ssm.load()
    assert lib.ssm_scan_fwd_workspace_bytes(B, L, D, N, 0 if dtype == torch.float32 else 1) > 0
    _check_fwd(ssm, _problem(B, L, D, N, dtype, seed=L % 97, h0=True), TOL[dtype])


def test_fwd_workload0(ssm):
    p = workload_inputs(0)
    _check_fwd(ssm, p, TOL[torch.float32])


@pytest.mark.parametrize("opts", [
    dict(z=False), dict(Dskip=False), dict(bias=False), dict(softplus=False),
    dict(h0=True), dict(generic_A=True), dict(z=False, Dskip=False, bias=False, softplus=False)],
    ids=["no-z", "no-D", "no-bias", "no-softplus", "h0", "generic-A", "bare"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_fwd_options(ssm, opts, dtype):
    _check_fwd(ssm, _problem(2, 130, 72, 16, dtype, seed=5, **opts), TOL[dtype])


@pytest.mark.parametrize("bias", [-30.0, 30.0, -12.0])
def test_fwd_extreme_step_sizes(ssm, bias):
    """Tiny steps (state kept) and huge steps (state reset)."""
    p = _problem(1, 80, 16, 16, torch.float32, seed=9, h0=True)
    p["delta_bias"] = torch.full((16,), bias)
    _check_fwd(ssm, p, TOL[torch.float32])


def test_softplus_accuracy_single_step(ssm):
    """L = 1, N = 1, h0 = 0: y = C * softplus(raw + bias) * B * u isolates the
    step-size nonlinearity over raw values from -20 to 25."""
    D = 4096
    raw = torch.linspace(-20.0, 25.0, D).view(1, 1, D)
    p = dict(u=torch.ones(1, 1, D), delta=raw, A=-torch.ones(D, 1), B=torch.ones(1, 1, 1),
             C=torch.ones(1, 1, 1), D=None, z=None, delta_bias=torch.zeros(D), delta_softplus=True)
    pg = _to(p, "cuda")
    y, _, _ = _gpu_fwd(ssm, pg)
    ref = np.logaddexp(0.0, raw.double().numpy())
    rel = np.abs(y.cpu().double().numpy() - ref) / ref
    assert rel.max() < 2e-6, float(rel.max())


def _sampled_fwd(ssm, idx, nsample, seed_dev="cuda"):
    w = WORKLOADS[idx]
    p = workload_inputs(idx, device=seed_dev)
    T = ssm.chunk_len()
    want_cs = "chunk_states" in w.outputs
    y, hf, cs = _gpu_fwd(ssm, p, return_final_state=True, save_chunk_states=want_cs)
    torch.cuda.synchronize()
    g = torch.Generator().manual_seed(idx)
    sel = torch.randperm(w.dim, generator=g)[:nsample].sort().values
    sel = torch.cat([sel, torch.tensor([0, w.dim - 1])]).unique()
    ps = _slice_channels(p, sel.to(p["u"].device))
    yo, hfo, cso = oracle_c.scan_fwd(**_oracle_kwargs(ps), chunk_len=T if want_cs else None)
    tol = TOL[w.io_dtype]
    for name, got, ref in (("y", y[:, :, sel.cuda()], yo), ("h_final", hf[:, sel.cuda()], hfo)):
        rep = parity_report(f"{w.name}:{name}", got, ref)
        assert rep["nan_count"] == 0 and rep["nmax_err"] <= tol
    if want_cs:
        assert nmax_err(cs[:, :, :, sel.cuda()].permute(0, 1, 3, 2), cso) <= tol
    return p, y


def test_fwd_workload1_full_size(ssm):
    _sampled_fwd(ssm, 1, 24)


def test_fwd_workload2_full_size(ssm):
    _sampled_fwd(ssm, 2, 12)


def test_fwd_workload4_full_size(ssm):
    _sampled_fwd(ssm, 4, 4)


def test_fwd_32k_context_full_size(ssm):
    """Batch 1, length 32768 (the context length the pages state), 5120
    channels, bf16: too few channel tiles for the GPU, so the launcher splits
    the sequence; sampled channels against the oracle."""
    w = WORKLOADS[5]
    plan = ssm.scan_fwd_plan(w.batch, w.seqlen, w.dim, w.dstate, w.io_dtype)
    assert plan["segments"] > 1, plan
    _sampled_fwd(ssm, 5, 8)


@pytest.mark.parametrize("reverse", [False, True], ids=["forward", "reverse"])
@pytest.mark.parametrize("L", [65472, 65536])
def test_fwd_rows_near_2gib(ssm, L, reverse):
    """8192 fp32 channels: 65472 steps are the most the 16-state kernel
    addresses with 32-bit offsets (its largest offsets, just under 2^31); at
    65536 a batch row of each (B,L,D) array spans 2 GiB and the forward takes
    the all-purpose kernel with 64-bit offsets. Sampled channels against the
    oracle."""
    from tests.test_gpu_options import _fwd as _fwd_opts
    D = 8192
    p = scan_inputs(1, L, D, 16, torch.float32, seed=12, device="cuda")
    y, hf, _ = _fwd_opts(ssm, p, reverse=reverse, return_final_state=True)
    torch.cuda.synchronize()
    sel = torch.tensor([0, 1, 2, 3, 4100, 4101, 4102, 4103, D - 4, D - 3, D - 2, D - 1])
    ps = _slice_channels(p, sel.cuda())
    y_s, hf_s = y[:, :, sel.cuda()].cpu(), hf[:, sel.cuda()].cpu()
    del p, y, hf
    torch.cuda.empty_cache()
    yo, hfo, _ = oracle_c.scan_fwd(**_oracle_kwargs(ps), reverse=reverse)
    assert nmax_err(y_s, yo) <= 1e-4
    assert nmax_err(hf_s, hfo) <= 1e-4


def test_fwd_deterministic_and_stream(ssm):
    p = _to(_problem(2, 400, 136, 16, torch.float32, seed=3, h0=True), "cuda")
    y1, h1, c1 = _gpu_fwd(ssm, p, return_final_state=True, save_chunk_states=True)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        y2, h2, c2 = _gpu_fwd(ssm, p, return_final_state=True, save_chunk_states=True)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(h1, h2) and torch.equal(c1, c2)


# ---------------------------------------------------------------- decode


def _decode_check(ssm, d, steps, tol, sel=None, zoh=False):
    dg = _to(d, "cuda")
    state = dg["state"].clone()
    ys = []
    for t in range(steps):
        ys.append(ssm.state_update(state, dg["u"][t], dg["delta"][t], dg["A"], dg["B"][t],
                                   dg["C"][t], dg.get("D"), None if dg.get("z") is None
                                   else dg["z"][t], dg.get("delta_bias"),
                                   d.get("delta_softplus", True), zoh=zoh))
    torch.cuda.synchronize()
    yg = torch.stack(ys)
    if sel is None:
        sel = torch.arange(d["state"].shape[1])
    so = d["state"][:, sel]
    yo = []
    for t in range(steps):
        so, yt = oracle_c.state_update(
            so, d["u"][t][:, sel], d["delta"][t][:, sel], d["A"][sel], d["B"][t], d["C"][t],
            None if d.get("D") is None else d["D"][sel],
            None if d.get("z") is None else d["z"][t][:, sel],
            None if d.get("delta_bias") is None else d["delta_bias"][sel],
            d.get("delta_softplus", True), zoh=zoh)
        yo.append(yt)
    assert nmax_err(yg[:, :, sel.cuda()], np.stack(yo)) <= tol
    assert nmax_err(state[:, sel.cuda()], so) <= tol


@pytest.mark.parametrize("N", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_decode_small(ssm, N, dtype):
    d = decode_inputs(3, 72, N, 5, dtype, seed=N)
    _decode_check(ssm, d, 5, TOL[dtype])


def test_decode_no_optionals(ssm):
    d = decode_inputs(2, 16, 16, 3, torch.float32, seed=1)
    d["D"] = d["z"] = d["delta_bias"] = None
    d["delta"] = d["delta"].abs() * 0.1
    d["delta_softplus"] = False
    _decode_check(ssm, d, 3, TOL[torch.float32])


@pytest.mark.parametrize("N", [4, 16])
def test_decode_more_rows_than_one_grid(ssm, N):
    """65537 batch rows (more than a 16-bit grid index): every row is updated."""
    d = decode_inputs(65537, 8, N, 2, torch.bfloat16, seed=33)
    _decode_check(ssm, d, 2, TOL[torch.bfloat16])


def test_decode_workload3_full_size(ssm):
    w = WORKLOADS[3]
    d = decode_inputs(w.batch, w.dim, w.dstate, w.steps, w.io_dtype, seed=3)
    g = torch.Generator().manual_seed(3)
    sel = torch.randperm(w.dim, generator=g)[:16].sort().values
    _decode_check(ssm, d, w.steps, TOL[w.io_dtype], sel=sel)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_decode_unaligned_token_b_c(ssm, dtype):
    """B and C only aligned to their element, which the state update allows:
    the same result as the aligned call, and the oracle's."""
    def misalign(x):
        buf = torch.empty(x.numel() + 1, dtype=x.dtype, device=x.device)
        buf[1:].copy_(x.reshape(-1))
        return buf[1:].view(x.shape)

    d = decode_inputs(3, 72, 16, 2, dtype, seed=21)
    dg = _to(d, "cuda")
    st_a, st_u = dg["state"].clone(), dg["state"].clone()
    so = d["state"]
    for t in range(2):
        Bu, Cu = misalign(dg["B"][t]), misalign(dg["C"][t])
        assert Bu.data_ptr() % (4 * Bu.element_size()) != 0
        args = (dg["u"][t], dg["delta"][t], dg["A"])
        rest = (dg["D"], dg["z"][t], dg["delta_bias"], True)
        ya = ssm.state_update(st_a, *args, dg["B"][t], dg["C"][t], *rest)
        yu = ssm.state_update(st_u, *args, Bu, Cu, *rest)
        so, yo = oracle_c.state_update(so, d["u"][t], d["delta"][t], d["A"], d["B"][t], d["C"][t],
                                       d["D"], d["z"][t], d["delta_bias"], True)
        torch.cuda.synchronize()
        assert torch.equal(ya, yu)
        assert nmax_err(yu, yo) <= TOL[dtype]
    assert torch.equal(st_a, st_u)
    assert nmax_err(st_u, so) <= TOL[dtype]


def test_decode_matches_scan_on_gpu(ssm):
    """64 single-token updates equal one 64-step scan (both on the GPU)."""
    p = _to(_problem(2, 64, 72, 16, torch.float32, seed=12, h0=True), "cuda")
    y, hf, _ = _gpu_fwd(ssm, p, return_final_state=True)
    state = p["h0"].clone()
    for t in range(64):
        yt = ssm.state_update(state, p["u"][:, t].contiguous(), p["delta"][:, t].contiguous(),
                              p["A"], p["B"][:, t].contiguous(), p["C"][:, t].contiguous(), p["D"],
                              p["z"][:, t].contiguous(), p["delta_bias"], True)
        assert nmax_err(yt, y[:, t]) <= 1e-5
    assert nmax_err(state, hf) <= 1e-5


# ---------------------------------------------------------------- backward

GRADS = ("du", "ddelta", "dA", "dB", "dC", "dD", "dz", "ddelta_bias", "dh0")


def _check_bwd(ssm, p, tol, dh_final=True, seed=0):
    pg = _to(p, "cuda")
    y, hf, cs = _gpu_fwd(ssm, pg, return_final_state=True, save_chunk_states=True)
    dy = cotangent(y, seed)
    g = torch.Generator().manual_seed(seed)
    dhf = torch.randn(hf.shape, generator=g).cuda() if dh_final else None
    gr = ssm.scan_bwd(pg["u"], pg["delta"], pg["A"], pg["B"], pg["C"], pg.get("D"), pg.get("z"),
                      pg.get("delta_bias"), p.get("delta_softplus", True), pg.get("h0"), cs, dy, dhf)
    torch.cuda.synchronize()
    go = oracle_c.scan_bwd(**_oracle_kwargs(p), dy=dy.cpu(), dh_final=None if dhf is None
                           else dhf.cpu())
    for k in GRADS:
        if go[k] is None or gr.get(k) is None:
            continue
        err = nmax_err(gr[k], go[k])
        assert err <= tol, (k, err)
    return gr


@pytest.mark.parametrize("B,L,D,N,dtype", [
    (2, 300, 72, 16, torch.float32), (2, 300, 72, 16, torch.bfloat16),
    (1, 64, 32, 4, torch.float32), (3, 97, 136, 8, torch.bfloat16), (2, 45, 64, 1, torch.float32),
    (1, 600, 16, 2, torch.float32)])
def test_bwd_small(ssm, B, L, D, N, dtype):
    _check_bwd(ssm, _problem(B, L, D, N, dtype, seed=L + N, h0=True), TOL[dtype])


@pytest.mark.parametrize("opts", [dict(z=False), dict(Dskip=False, bias=False),
                                  dict(softplus=False), dict(generic_A=True)],
                         ids=["no-z", "no-D-no-bias", "no-softplus", "generic-A"])
def test_bwd_options(ssm, opts):
    _check_bwd(ssm, _problem(2, 200, 64, 16, torch.float32, seed=4, **opts), 1e-4,
               dh_final=False)


@pytest.mark.parametrize("B,L,D,N,dtype", [
    (1, 5000, 16, 16, torch.float32), (2, 9000, 24, 8, torch.float32),
    (1, 6000, 8, 16, torch.bfloat16), (1, 4500, 8, 1, torch.float32),
    # segments of the shortest length, 512 steps: 16 of them (composed by the
    # wave-wide scan) and 8 (composed by the per-thread fold)
    (1, 8192, 8, 16, torch.float32), (1, 4096, 16, 16, torch.bfloat16)])
def test_bwd_sequence_split(ssm, B, L, D, N, dtype):
    """Few channels and a long sequence: the backward splits the sequence into
    segments (local adjoint carries, their composition from the right, then the
    full backward of each segment)."""
    _check_bwd(ssm, _problem(B, L, D, N, dtype, seed=L % 89, h0=True), TOL[dtype], seed=L)


def test_bwd_deterministic(ssm):
    p = _to(_problem(2, 300, 72, 16, torch.bfloat16, seed=8, h0=True), "cuda")
    y, hf, cs = _gpu_fwd(ssm, p, return_final_state=True, save_chunk_states=True)
    dy = cotangent(y, 1)
    args = (p["u"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"], p["delta_bias"], True,
            p["h0"], cs, dy)
    g1 = ssm.scan_bwd(*args)
    g2 = ssm.scan_bwd(*args)
    for k in GRADS:
        if g1[k] is not None:
            assert torch.equal(g1[k], g2[k]), k


def test_bwd_workload4_full_size(ssm):
    """Full million-length shape in the benchmark's launch configuration.  The
    cotangent is zero outside a few sampled channels, so the sums over channels
    (dB, dC) are sums over those channels only and the oracle can compute them;
    every gradient of the other channels must be exactly zero."""
    w = WORKLOADS[4]
    p = workload_inputs(4, device="cuda")
    y, hf, cs = _gpu_fwd(ssm, p, return_final_state=True, save_chunk_states=True)
    sel = torch.tensor([0, 333, 640, w.dim - 1])
    mask = torch.zeros(w.dim, dtype=torch.bool)
    mask[sel] = True
    dy = cotangent(y, 4)
    dy[:, :, ~mask.cuda()] = 0
    gr = ssm.scan_bwd(p["u"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"],
                      p["delta_bias"], True, None, cs, dy)
    torch.cuda.synchronize()
    ps = _slice_channels(dict(p, dy=dy), sel.cuda())
    go = oracle_c.scan_bwd(**_oracle_kwargs(ps), dy=ps["dy"])
    tol = TOL[w.io_dtype]
    sc = sel.cuda()
    for k in ("du", "ddelta", "dz"):
        assert parity_report(f"million-length:{k}", gr[k][:, :, sc], go[k])["nmax_err"] <= tol, k
        assert int(torch.count_nonzero(gr[k][:, :, ~mask.cuda()])) == 0, k
    for k in ("dB", "dC"):
        assert parity_report(f"million-length:{k}", gr[k], go[k])["nmax_err"] <= tol, k
    assert parity_report("million-length:dA", gr["dA"][sc], go["dA"])["nmax_err"] <= tol
    for k in ("dD", "ddelta_bias"):
        assert nmax_err(gr[k][sc], go[k]) <= tol, k


def test_bwd_workload1_shape_full_size(ssm):
    """Backward at the Mamba-370m layer shape (fp32, 8 batch rows, 32 channel
    tiles, no sequence split), as the benchmark runs it.  The cotangent is zero
    outside sampled channels in every tile position the staging of the channel
    sums distinguishes (first and last of a tile, both lane parities), so the
    oracle computes dB and dC over those channels; all gradients of the other
    channels must be exactly zero."""
    w = WORKLOADS[1]
    p = workload_inputs(1, device="cuda")
    y, hf, cs = _gpu_fwd(ssm, p, return_final_state=True, save_chunk_states=True)
    sel = torch.tensor([0, 1, 62, 63, 64, 777, 1030, 1500, w.dim - 2, w.dim - 1])
    mask = torch.zeros(w.dim, dtype=torch.bool)
    mask[sel] = True
    dy = cotangent(y, 1)
    dy[:, :, ~mask.cuda()] = 0
    gr = ssm.scan_bwd(p["u"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"],
                      p["delta_bias"], True, None, cs, dy)
    torch.cuda.synchronize()
    ps = _slice_channels(dict(p, dy=dy), sel.cuda())
    go = oracle_c.scan_bwd(**_oracle_kwargs(ps), dy=ps["dy"])
    tol = TOL[w.io_dtype]
    sc = sel.cuda()
    for k in ("du", "ddelta", "dz"):
        assert nmax_err(gr[k][:, :, sc], go[k]) <= tol, k
        assert int(torch.count_nonzero(gr[k][:, :, ~mask.cuda()])) == 0, k
    for k in ("dB", "dC"):
        assert nmax_err(gr[k], go[k]) <= tol, k
    for k in ("dA", "dD", "ddelta_bias"):
        assert nmax_err(gr[k][sc], go[k]) <= tol, k
        assert int(torch.count_nonzero(gr[k][~mask.cuda()])) == 0, k


def test_autograd_function(ssm):
    p = _to(_problem(2, 150, 64, 16, torch.float32, seed=21, h0=True), "cuda")
    leaves = {k: p[k].clone().requires_grad_(True) for k in
              ("u", "delta", "A", "B", "C", "D", "z", "delta_bias", "h0")}
    y, hf = ssm.selective_scan(leaves["u"], leaves["delta"], leaves["A"], leaves["B"],
                               leaves["C"], leaves["D"], leaves["z"], leaves["delta_bias"], True,
                               leaves["h0"])
    dy = cotangent(y.detach(), 2)
    (y * dy).sum().backward()
    pc = {k: v.detach().cpu() for k, v in p.items() if isinstance(v, torch.Tensor)}
    pc["delta_softplus"] = True
    go = oracle_c.scan_bwd(**_oracle_kwargs(pc), dy=dy.cpu())
    names = dict(u="du", delta="ddelta", A="dA", B="dB", C="dC", D="dD", z="dz",
                 delta_bias="ddelta_bias", h0="dh0")
    for k, g in names.items():
        assert nmax_err(leaves[k].grad, go[g]) <= 1e-4, k
