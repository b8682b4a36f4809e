"""Edge cases of the HIP path against the oracle: lengths around the chunk
length, the smallest channel count, many short rows, NaN propagation, and
inputs the binding must refuse."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import oracle_c
from tests.helpers import nmax_err
from tests.test_gpu_parity import TOL, _check_bwd, _check_fwd, _gpu_fwd, _problem, _to

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ssm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import selective_state_space_10_amd as m
    m.load()
    return m


@pytest.mark.parametrize("L", [1, 2, 15, 16, 17, 31, 32, 33, 47, 48, 49, 63, 64, 65])
def test_lengths_around_the_chunk(ssm, L):
    """One chunk is 32 steps and the 16-state forward stages 16-step sub-chunks:
    lengths just below, at and above one to four sub-chunks."""
    p = _problem(2, L, 72, 16, torch.float32, seed=L, h0=True)
    _check_fwd(ssm, p, 1e-4)
    _check_bwd(ssm, p, 1e-4, seed=L)


@pytest.mark.parametrize("L", [1, 2, 15, 16, 17, 31, 33, 49])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_reverse_lengths_around_the_chunk(ssm, L, dtype):
    """The reverse direction with one step size per token at lengths below,
    at and above a 16-step sub-chunk: loads of steps past the end are clamped
    to the segment's first row in memory."""
    from tests.test_gpu_options import _check_fwd as _check_fwd_opts, _with_opts
    p = _with_opts(_problem(2, L, 72, 16, dtype, seed=100 + L, h0=True), True)
    _check_fwd_opts(ssm, p, TOL[dtype], reverse=True)


@pytest.mark.parametrize("B,L,D,N,dtype", [(1, 40, 8, 16, torch.float32),
                                           (5, 33, 8, 4, torch.bfloat16),
                                           (64, 7, 64, 16, torch.float32),
                                           (3, 50, 200, 16, torch.bfloat16)])
def test_small_channel_counts_and_short_rows(ssm, B, L, D, N, dtype):
    """8 channels (one partially filled tile), many short rows, and a channel
    count that leaves a 8-channel tail in the last 64-channel tile."""
    p = _problem(B, L, D, N, dtype, seed=B + L + D, h0=True)
    _check_fwd(ssm, p, TOL[dtype])
    _check_bwd(ssm, p, TOL[dtype], seed=B)


def test_more_batch_rows_than_one_grid_row_range(ssm):
    """65537 batch rows (more than a 16-bit grid index): forward and backward
    cover every row."""
    p = _problem(65537, 3, 8, 4, torch.bfloat16, seed=65, h0=True)
    _check_fwd(ssm, p, TOL[torch.bfloat16])
    _check_bwd(ssm, p, TOL[torch.bfloat16], seed=65)


def _assert_plan(ssm, p, tile, zoh=False, reverse=False, conv=0):
    """The forward reaches the wave-specialised kernel on `tile`-channel tiles
    for this problem (the launch plan the launcher itself follows)."""
    Bsz, L, D = p["u" if "u" in p else "x"].shape
    plan = ssm.scan_fwd_plan(Bsz, L, D, p["A"].shape[1], p["B"].dtype, zoh=zoh, reverse=reverse,
                             per_token=p["delta"].dim() == 2, conv_width=conv)
    assert plan == {"kernel": "wave-specialised", "tile_channels": tile, "segments": 1,
                    "segment_len": 0, "first_pass_len": 0}, plan


@pytest.mark.parametrize("opts", [dict(), dict(zoh=True), dict(reverse=True, tok=True)],
                         ids=["plain", "zoh", "reverse-per-token"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_many_channel_tiles(ssm, dtype, opts):
    """More tiles than one round over the compute units: 12 rows x 32 tiles of
    64 or 12 x 26 of 80 need two rounds, while 12 x 64 tiles of 32 take one
    round of two workgroups per compute unit and half a round of one, so the
    16-state forward takes 32-channel tiles (the last one ragged: 24 of 32
    channels)."""
    from tests.test_gpu_options import _check_fwd as _check_fwd_opts, _with_opts
    p = _with_opts(_problem(12, 40, 2040, 16, dtype, seed=41, h0=True), opts.get("tok", False))
    _assert_plan(ssm, p, 32, opts.get("zoh", False), opts.get("reverse", False))
    _check_fwd_opts(ssm, p, TOL[dtype], opts.get("zoh", False), opts.get("reverse", False))


@pytest.mark.parametrize("opts", [dict(), dict(zoh=True, tok=True)], ids=["plain", "zoh-per-token"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_many_channel_tiles_fused_conv(ssm, dtype, opts):
    """The fused convolution at 12 x 2040 channels: on 32-channel tiles (12 x 64
    tiles) in bf16, on 64-channel tiles in fp32 (whose 32-channel variant is
    never the fastest), against the oracle's convolution followed by its scan."""
    from tests.test_gpu_conv import _conv_problem, _gpu_fwd as _conv_fwd, _okw
    zoh = opts.get("zoh", False)
    p = _conv_problem(12, 40, 2040, 16, dtype, 4, seed=47, tok=opts.get("tok", False))
    _assert_plan(ssm, p, 32 if dtype == torch.bfloat16 else 64, zoh=zoh, conv=4)
    T = ssm.chunk_len()
    y, hf, cs = _conv_fwd(ssm, _to(p, "cuda"), zoh, return_final_state=True, save_chunk_states=True)
    torch.cuda.synchronize()
    yo, hfo, cso = oracle_c.scan_fwd_conv(**_okw(p), chunk_len=T, zoh=zoh)
    assert nmax_err(y, yo) <= TOL[dtype]
    assert nmax_err(hf, hfo) <= TOL[dtype]
    assert nmax_err(cs.permute(0, 1, 3, 2), cso) <= TOL[dtype]


@pytest.mark.parametrize("opts", [dict(), dict(zoh=True, tok=True, bias=False)],
                         ids=["plain", "zoh-per-token-no-bias"])
@pytest.mark.parametrize("D,dtype", [(5120, torch.float32), (5120, torch.bfloat16),
                                     (5112, torch.bfloat16)], ids=["5120-f32", "5120-bf16", "5112-bf16"])
def test_eighty_channel_tiles_fused_conv(ssm, D, dtype, opts):
    """The fused convolution on 80-channel tiles (4 rows of 5120 or 5112
    channels: one round of 64 or 65 tiles per row over 256 compute units, where
    64-channel tiles would need two), the last tile ragged for 5112, against the
    oracle's convolution followed by its scan."""
    from tests.test_gpu_conv import _conv_problem, _gpu_fwd as _conv_fwd, _okw
    opts = dict(opts)
    zoh = opts.pop("zoh", False)
    p = _conv_problem(4, 48, D, 16, dtype, 4, seed=D % 97, **opts)
    _assert_plan(ssm, p, 80, zoh=zoh, conv=4)
    T = ssm.chunk_len()
    y, hf, cs = _conv_fwd(ssm, _to(p, "cuda"), zoh, return_final_state=True, save_chunk_states=True)
    torch.cuda.synchronize()
    yo, hfo, cso = oracle_c.scan_fwd_conv(**_okw(p), chunk_len=T, zoh=zoh)
    assert nmax_err(y, yo) <= TOL[dtype]
    assert nmax_err(hf, hfo) <= TOL[dtype]
    assert nmax_err(cs.permute(0, 1, 3, 2), cso) <= TOL[dtype]


@pytest.mark.parametrize("opts", [dict(), dict(zoh=True), dict(reverse=True, tok=True)],
                         ids=["plain", "zoh", "reverse-per-token"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_eighty_channel_tiles(ssm, dtype, opts):
    """20480 channels in one row: 320 tiles of 64 channels would need a second
    round over 256 compute units, 256 tiles of 80 need one, so the 16-state
    forward takes 80-channel tiles there (on a 256-CU device)."""
    from tests.test_gpu_options import _check_fwd as _check_fwd_opts, _with_opts
    p = _with_opts(_problem(1, 37, 20480, 16, dtype, seed=43, h0=True), opts.get("tok", False))
    _assert_plan(ssm, p, 80, opts.get("zoh", False), opts.get("reverse", False))
    _check_fwd_opts(ssm, p, TOL[dtype], opts.get("zoh", False), opts.get("reverse", False))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_two_full_rounds_of_64_channel_tiles(ssm, dtype):
    """16 rows x 32 tiles of 64 channels: exactly two rounds over 256 compute
    units, which the forward prefers to 32-channel tiles (two rounds of two
    workgroups per compute unit) and to 80-channel tiles (two rounds, 416
    tiles)."""
    p = _problem(16, 24, 2048, 16, dtype, seed=45, h0=True)
    _assert_plan(ssm, p, 64)
    _check_fwd(ssm, p, TOL[dtype])


@pytest.mark.parametrize("z,Dskip", [(True, True), (False, False)], ids=["gated", "no-gate-no-skip"])
def test_eighty_channel_tiles_ragged(ssm, z, Dskip):
    """16408 channels: 257 tiles of 64, 206 tiles of 80 of which the last holds
    8 channels."""
    p = _problem(1, 20, 16408, 16, torch.float32, seed=44, z=z, Dskip=Dskip, h0=True)
    _check_fwd(ssm, p, 1e-4)


def test_nan_propagates_in_its_channel_only(ssm):
    """A NaN input poisons its own channel from that step on (through the
    state) and nothing else: channels are independent recurrences."""
    p = _to(_problem(1, 100, 72, 16, torch.float32, seed=2), "cuda")
    p["u"][0, 40, 5] = float("nan")
    y, hf, _ = _gpu_fwd(ssm, p, return_final_state=True)
    torch.cuda.synchronize()
    yc = y[0].cpu()
    assert torch.isfinite(yc[:40]).all()
    assert torch.isnan(yc[40:, 5]).all()
    others = torch.cat([yc[:, :5], yc[:, 6:]], dim=1)
    assert torch.isfinite(others).all()
    assert torch.isnan(hf[0, 5]).all() and torch.isfinite(torch.cat([hf[0, :5], hf[0, 6:]])).all()


def test_decode_matches_scan_for_many_small_rows(ssm):
    p = _to(_problem(32, 3, 8, 16, torch.float32, seed=6, h0=True), "cuda")
    y, hf, _ = _gpu_fwd(ssm, p, return_final_state=True)
    state = p["h0"].clone()
    for t in range(3):
        yt = ssm.state_update(state, p["u"][:, t].contiguous(), p["delta"][:, t].contiguous(),
                              p["A"], p["B"][:, t].contiguous(), p["C"][:, t].contiguous(),
                              p["D"], p["z"][:, t].contiguous(), p["delta_bias"], True)
        assert nmax_err(yt, y[:, t]) <= 1e-5
    assert nmax_err(state, hf) <= 1e-5


def test_binding_refuses_bad_inputs(ssm):
    p = _to(_problem(2, 40, 16, 4, torch.float32, seed=1), "cuda")
    args = [p["u"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"], p["delta_bias"]]
    with pytest.raises(ValueError, match="contiguous"):
        ssm.scan_fwd(p["u"].transpose(1, 2).contiguous().transpose(1, 2), *args[1:])
    with pytest.raises(TypeError, match="dtype"):
        ssm.scan_fwd(args[0], args[1], args[2].double(), *args[3:])
    with pytest.raises(ValueError, match="shape"):
        ssm.scan_fwd(args[0], args[1], args[2][:8], *args[3:])
    with pytest.raises(TypeError, match="io dtype"):
        ssm.scan_fwd(args[0].half(), *args[1:])
    with pytest.raises(ValueError, match="width"):
        ssm.scan_fwd_conv(args[0], torch.zeros(16, 5, device="cuda"), None, *args[1:5])
