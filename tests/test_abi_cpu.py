"""The C-ABI library loads, exports every symbol the header declares, and
rejects invalid arguments before touching the GPU.  No kernel is launched: every
call here fails validation, so these run without a GPU."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "ssm_scan.h")

OK, NULL_ARG, BAD_SHAPE, UNSUPPORTED, ALIGNMENT, WORKSPACE, HIP = range(7)
FAKE = 0x10000  # aligned, never dereferenced: every call below fails validation first


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssm_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from selective_state_space_10_amd import _lib
    return _lib.load()


def test_every_declared_symbol_is_exported(lib):
    from selective_state_space_10_amd import _lib
    names = _declared()
    assert len(names) >= 10
    assert sorted(_lib.EXPORTS) == names
    for n in names:
        assert hasattr(lib, n), n


def test_probe_library_exports_its_header():
    """The vector-ALU probe library (a measurement tool the benchmark loads)
    exports exactly what include/ssm_alu_probe.h declares, and refuses bad
    arguments without a device."""
    from selective_state_space_10_amd import build
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "ssm_alu_probe.h")).read(),
                  flags=re.S)
    names = sorted(set(re.findall(r"\b(ssm_[a-z0-9_]+)\s*\(", text)))
    assert names == ["ssm_probe_instructions_per_lane", "ssm_probe_valu", "ssm_probe_wave_placement"]
    probe = ctypes.CDLL(build.PROBE_LIB)
    for n in names:
        assert hasattr(probe, n), n
    probe.ssm_probe_instructions_per_lane.restype = ctypes.c_int64
    probe.ssm_probe_instructions_per_lane.argtypes = [ctypes.c_int, ctypes.c_int64]
    assert probe.ssm_probe_instructions_per_lane(0, 10) == 10 * 64
    assert probe.ssm_probe_instructions_per_lane(2, 10) == 10 * 64 * 5
    probe.ssm_probe_valu.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p,
                                     ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    wg = ctypes.c_int(0)
    assert probe.ssm_probe_valu(0, 5, 10, FAKE, 1 << 20, ctypes.addressof(wg), None) == 1
    assert probe.ssm_probe_valu(5, 1, 10, FAKE, 1 << 20, ctypes.addressof(wg), None) == 1
    assert probe.ssm_probe_valu(0, 1, 10, None, 1 << 20, ctypes.addressof(wg), None) == 1


def test_binding_signatures_match_the_header(lib):
    """Each ctypes prototype has as many arguments as the header declares."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    protos = re.findall(r"\b(ssm_[a-z0-9_]+)\s*\(([^)]*)\)\s*;", text)
    assert len(protos) == len(_declared())
    for name, params in protos:
        n = 0 if params.strip() in ("", "void") else len(params.split(","))
        assert len(getattr(lib, name).argtypes) == n, name


def test_version_and_queries(lib):
    assert lib.ssm_abi_version() == 4
    T = lib.ssm_scan_chunk_len()
    assert T >= 16 and T & (T - 1) == 0
    assert lib.ssm_scan_chunk_states_bytes(2, T * 3 + 1, 64, 16) == 2 * 4 * 64 * 16 * 4
    assert lib.ssm_scan_chunk_states_bytes(0, 5, 8, 4) == -1
    assert lib.ssm_scan_fwd_workspace_bytes(1, 64, 32, 4, 0) >= 0
    assert lib.ssm_scan_bwd_workspace_bytes(1, 64, 32, 4, 1) > 0
    assert lib.ssm_scan_bwd_workspace_bytes(1, 64, 33, 4, 1) == -1
    for s in range(7):
        assert lib.ssm_status_string(s)
    assert lib.ssm_status_string(99) == b"unknown status"


@pytest.mark.parametrize("L,D,io,nseg_uncapped", [(1 << 20, 1024, 0, 64), (1 << 22, 4096, 0, 16),
                                                  (1 << 22, 4096, 1, 16)])
def test_fwd_split_segments_fit_32bit_offsets(lib, L, D, io, nseg_uncapped):
    """A split sequence's segments are what the forward workspace holds
    (per segment: two (D,N) state arrays and a D-vector of step-size sums). The
    forward kernel addresses a segment with 32-bit byte offsets, so a segment
    of a (B,L,D) array, plus 64 rows of slack, stays below 2^31 bytes: long
    segments are cut into more."""
    N, sz = 16, (4, 2)[io]
    wsb = lib.ssm_scan_fwd_workspace_bytes(1, L, D, N, io)
    nseg, rem = divmod(wsb, 4 * D * (2 * N + 1))
    assert wsb > 0 and rem == 0
    seg = -(-L // nseg)
    seg = -(-seg // 32) * 32
    fits = (seg + 64) * D * sz < 1 << 31
    assert fits
    if (-(-L // nseg_uncapped) + 64) * D * sz < 1 << 31:
        assert nseg == nseg_uncapped
    else:
        assert nseg > nseg_uncapped


def _fwd(lib, B=1, L=16, D=8, N=4, io=0, **kw):
    p = dict(u=FAKE, delta=FAKE, A=FAKE, Bm=FAKE, Cm=FAKE, Dskip=None, z=None, bias=None,
             h0=None, hf=None, y=FAKE, cs=None, ws=None)
    p.update(kw)
    return lib.ssm_scan_fwd(B, L, D, N, io, p["u"], p["delta"], p["A"], p["Bm"], p["Cm"],
                            p["Dskip"], p["z"], p["bias"], 1, p["h0"], p["hf"], p["y"], p["cs"],
                            p["ws"], kw.get("wsb", 0), None)


@pytest.mark.parametrize("sizes,status", [
    (dict(B=0), BAD_SHAPE), (dict(L=0), BAD_SHAPE), (dict(D=0), BAD_SHAPE), (dict(N=0), BAD_SHAPE),
    (dict(L=-3), BAD_SHAPE), (dict(B=1 << 40, L=1 << 40), BAD_SHAPE),
    (dict(N=3), UNSUPPORTED), (dict(N=32), UNSUPPORTED), (dict(D=12), UNSUPPORTED),
    (dict(B=1 << 31), UNSUPPORTED), (dict(D=(1 << 36) + 8), UNSUPPORTED),
    (dict(io=2), UNSUPPORTED)])
def test_fwd_rejects_bad_sizes(lib, sizes, status):
    assert _fwd(lib, **sizes) == status
    assert lib.ssm_last_error()


@pytest.mark.parametrize("name", ["u", "delta", "A", "Bm", "Cm", "y"])
def test_fwd_rejects_null_required(lib, name):
    assert _fwd(lib, **{name: None}) == NULL_ARG
    assert b"NULL" in lib.ssm_last_error()


@pytest.mark.parametrize("name", ["u", "A", "z", "h0", "cs", "Dskip"])
def test_fwd_rejects_misaligned(lib, name):
    kw = {name: FAKE + 4}
    if name in ("u", "A"):
        kw["Dskip"] = None
    assert _fwd(lib, **kw) == ALIGNMENT


def _bwd(lib, B=1, L=16, D=8, N=4, io=0, wsb=0, **kw):
    p = dict(u=FAKE, delta=FAKE, A=FAKE, Bm=FAKE, Cm=FAKE, Dskip=None, z=None, bias=None, h0=None,
             cs=FAKE, dy=FAKE, dhf=None, du=FAKE, ddelta=FAKE, dA=FAKE, dB=FAKE, dC=FAKE,
             dD=None, dz=None, dbias=None, dh0=None, ws=FAKE)
    p.update(kw)
    return lib.ssm_scan_bwd(B, L, D, N, io, p["u"], p["delta"], p["A"], p["Bm"], p["Cm"],
                            p["Dskip"], p["z"], p["bias"], 1, p["h0"], p["cs"], p["dy"], p["dhf"],
                            p["du"], p["ddelta"], p["dA"], p["dB"], p["dC"], p["dD"], p["dz"],
                            p["dbias"], p["dh0"], p["ws"], wsb, None)


def test_bwd_validation(lib):
    assert _bwd(lib) == WORKSPACE  # everything valid except the workspace size
    assert _bwd(lib, cs=None) == NULL_ARG
    assert _bwd(lib, ws=None) == NULL_ARG
    assert _bwd(lib, Dskip=FAKE) == NULL_ARG  # dD missing while Dskip given
    assert _bwd(lib, dD=FAKE) == NULL_ARG
    assert _bwd(lib, z=FAKE) == NULL_ARG  # dz missing while z given
    assert _bwd(lib, dy=FAKE + 8) == ALIGNMENT
    assert _bwd(lib, L=0) == BAD_SHAPE
    need = lib.ssm_scan_bwd_workspace_bytes(1, 16, 8, 4, 0)
    assert _bwd(lib, wsb=need - 1) == WORKSPACE


def test_decode_validation(lib):
    f = lib.ssm_state_update
    args = [FAKE] * 6 + [None, None, None]
    assert f(0, 8, 4, 0, *args, 1, FAKE, None) == BAD_SHAPE
    assert f(2, 8, 5, 0, *args, 1, FAKE, None) == UNSUPPORTED
    assert f(2, 8, 4, 0, None, *args[1:], 1, FAKE, None) == NULL_ARG
    assert f(2, 8, 4, 0, *args, 1, None, None) == NULL_ARG
    assert f(2, 8, 4, 0, FAKE + 2, *args[1:], 1, FAKE, None) == ALIGNMENT  # state
    assert f(2, 8, 4, 0, *args[:3], FAKE + 8, *args[4:], 1, FAKE, None) == ALIGNMENT  # A
    assert f(2, 8, 4, 1, *args[:4], FAKE + 1, *args[5:], 1, FAKE, None) == ALIGNMENT  # odd bf16


def test_decode_rejects_dim_beyond_the_grid(lib):
    """The decode kernel's lane index is 64-bit (more than 2^31 lanes per
    batch row are addressed correctly); channel counts above 2^36, whose lanes
    would not fit the grid, are rejected before any launch."""
    f = lib.ssm_state_update
    args = [FAKE] * 6 + [None, None, None]
    assert f(1, (1 << 36) + 8, 16, 0, *args, 1, FAKE, None) == UNSUPPORTED
    assert b"2^36" in lib.ssm_last_error()


ZOH, REV, TOK, ACC = 1, 2, 4, 8


@pytest.mark.parametrize("sizes,io,flags,conv,expect", [
    ((8, 2048, 2048, 16), 0, 0, 0, (1, 64, 1)),        # Mamba-370m layer: 256 tiles of 64
    ((8, 2048, 2048, 16), 0, ZOH, 4, (1, 64, 1)),
    ((4, 4096, 5120, 16), 1, 0, 0, (1, 80, 1)),        # Mamba-2.8b layer: 256 tiles of 80
    ((4, 4096, 5120, 16), 1, 0, 4, (1, 80, 1)),        # ... with the fused convolution too
    ((4, 4096, 5120, 16), 0, 0, 4, (1, 80, 1)),        # fp32 with the convolution: 80 costs 102
    ((12, 40, 2040, 16), 0, 0, 0, (1, 32, 1)),         # 1.5 rounds of 32-channel tiles
    ((12, 40, 2040, 16), 1, ZOH, 0, (1, 32, 1)),
    ((12, 40, 2040, 16), 0, REV | TOK, 0, (1, 32, 1)),
    ((12, 40, 2040, 16), 1, 0, 4, (1, 32, 1)),
    ((12, 40, 2040, 16), 0, 0, 4, (1, 64, 1)),         # fp32 with the convolution: never 32
    ((16, 24, 2048, 16), 0, 0, 0, (1, 64, 1)),         # two full rounds of 64-channel tiles
    ((8, 4096, 5120, 16), 1, 0, 0, (1, 80, 1)),        # two full rounds of 80-channel tiles
    ((8, 4096, 5120, 16), 1, 0, 4, (1, 80, 1)),        # ... and with the convolution
    ((8, 4096, 5120, 16), 0, 0, 4, (1, 64, 1)),        # fp32: 3 rounds of 64 beat 2 of 80
    ((8, 40, 3336, 16), 0, 0, 0, (1, 64, 1)),          # 424 tiles of 64: two rounds beat 32
    ((1, 37, 20480, 16), 0, 0, 0, (1, 80, 1)),
    ((1, 1 << 20, 1024, 16), 1, 0, 0, (1, 64, 64)),    # million-length: 64 segments, four rounds
    ((1, 32768, 5120, 16), 1, 0, 0, (1, 64, 3)),       # 32K context: 3 x 80 tiles fill one round
    ((1, 65536, 8192, 16), 0, 0, 0, (0, 64, 1)),       # a row spans 2 GiB: 64-bit offsets
    ((2, 300, 72, 8), 0, 0, 0, (0, 64, 1)),
    ((3, 97, 136, 8), 0, ZOH, 0, (0, 32, 1)),
    ((1, 12289, 8, 2), 0, 0, 0, (0, 64, 3)),           # 2 states: one wave covers 64 channels
])
def test_fwd_plan_query(lib, sizes, io, flags, conv, expect):
    """The launch plan the forward follows (kernel, channels per workgroup,
    segments) for shapes the GPU tests and the benchmark use, on a device
    with 256 compute units (or none, which the query takes as 256)."""
    from selective_state_space_10_amd import _lib
    plan = _lib.FwdPlan()
    assert lib.ssm_scan_fwd_plan(*sizes, io, flags, conv, ctypes.byref(plan)) == OK
    assert (plan.kernel, plan.tile_channels, plan.segments) == expect
    assert (plan.segment_len == 0) == (plan.segments == 1) == (plan.first_pass_len == 0)
    if plan.segments > 1:
        B, L, D, N = sizes
        assert plan.segments == -(-L // plan.segment_len)
        # the first pass cuts every segment into whole pieces of whole chunks
        assert plan.segment_len % plan.first_pass_len == 0 and plan.first_pass_len % 32 == 0
        rows = -(-L // plan.first_pass_len)  # pieces over the whole length
        assert lib.ssm_scan_fwd_workspace_bytes(*sizes, io) == 4 * B * D * (rows * (N + 1) + plan.segments * N)


@pytest.mark.parametrize("sizes,io,segment_len,first_pass_len", [
    ((1, 32768, 5120, 16), 1, 10944, 3648),       # 32K context: 2 x 80 first-pass tiles, cut in 3
    ((1, 1 << 20, 1024, 16), 1, 16384, 16384),    # million-length: the first pass fills 4 rounds
    ((1, 24576, 24, 16), 0, 4096, 2048),          # one tile: pieces no shorter than 2048 steps
    ((1, 13868, 16, 16), 1, 4640, 4640),          # no whole-chunk piece of 2048 steps or more
    ((2, 9000, 24, 8), 0, 4512, 4512),            # other state counts: no pieces
])
def test_fwd_plan_first_pass_pieces(lib, sizes, io, segment_len, first_pass_len):
    """How a split's first pass is cut: pieces where whole rounds of them over
    256 compute units save at least 5% of its time, none elsewhere."""
    from selective_state_space_10_amd import _lib
    plan = _lib.FwdPlan()
    assert lib.ssm_scan_fwd_plan(*sizes, io, 0, 0, ctypes.byref(plan)) == OK
    assert (plan.segment_len, plan.first_pass_len) == (segment_len, first_pass_len)


def test_noalloc_forward_rejects_oversized_scratch(lib):
    """The allocation-free forward holds a fixed scratch of 16 MiB: sizes whose
    forward workspace is larger are refused before anything is enqueued (and
    before the device is touched), like every other invalid argument."""
    B, L, D, N = 1, 1 << 22, 4096, 16
    need = lib.ssm_scan_fwd_workspace_bytes(B, L, D, N, 0)
    assert need > 16 << 20
    args = (B, L, D, N, 0, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, 1, None, None, FAKE,
            None, None)
    assert lib.ssm_scan_fwd_noalloc(*args, 0) == WORKSPACE
    assert b"allocation-free" in lib.ssm_last_error()
    assert lib.ssm_scan_fwd_noalloc(1, 0, D, N, 0, *args[5:], 0) == BAD_SHAPE
    # within the scratch (the million-length shape needs about 2 MiB)
    assert 0 < lib.ssm_scan_fwd_workspace_bytes(1, 1 << 20, 1024, 16, 1) <= 16 << 20


def test_affine_scan_validation(lib):
    f = lib.ssm_affine_scan
    assert f(0, 4, FAKE, FAKE, None, FAKE, 0, None) == BAD_SHAPE
    assert f(2, 0, FAKE, FAKE, None, FAKE, 0, None) == BAD_SHAPE
    assert f(2, 4, None, FAKE, None, FAKE, 0, None) == NULL_ARG
    assert f(2, 4, FAKE, FAKE, None, None, 0, None) == NULL_ARG
    assert f(2, 4, FAKE + 2, FAKE, None, FAKE, 0, None) == ALIGNMENT
    assert f(2, 4, FAKE, FAKE, None, FAKE, 2, None) == UNSUPPORTED
    assert f(1 << 40, 1 << 30, FAKE, FAKE, None, FAKE, 0, None) == BAD_SHAPE


def test_fwd_plan_query_validates(lib):
    from selective_state_space_10_amd import _lib
    plan = _lib.FwdPlan()
    assert lib.ssm_scan_fwd_plan(1, 0, 8, 4, 0, 0, 0, ctypes.byref(plan)) == BAD_SHAPE
    assert lib.ssm_scan_fwd_plan(1, 16, 8, 4, 0, 16, 0, ctypes.byref(plan)) == UNSUPPORTED
    assert lib.ssm_scan_fwd_plan(1, 16, 8, 4, 0, 0, 5, ctypes.byref(plan)) == UNSUPPORTED
    assert lib.ssm_scan_fwd_plan(1, 16, 8, 4, 0, REV, 4, ctypes.byref(plan)) == UNSUPPORTED
    assert lib.ssm_scan_fwd_plan(1, 16, 8, 4, 0, 0, 0, None) == NULL_ARG


def test_option_flags_are_validated(lib):
    """Unknown option bits, and bits that do not apply to an entry point, are
    rejected before anything is enqueued."""
    fargs = (1, 16, 8, 4, 0, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, 1, None, None, FAKE,
             None, None, 0, None)
    assert lib.ssm_scan_fwd_ex(*fargs, 16) == UNSUPPORTED
    assert lib.ssm_scan_fwd_ex(*fargs, -1) == UNSUPPORTED
    assert lib.ssm_scan_fwd_ex(*fargs[:1], 0, *fargs[2:], 1) == BAD_SHAPE  # sizes still checked
    bargs = (1, 16, 8, 4, 0, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, 1, None, FAKE, FAKE,
             None, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, None, FAKE, 0, None)
    assert lib.ssm_scan_bwd_ex(*bargs, 8) == UNSUPPORTED  # accumulate is forward-only
    assert lib.ssm_scan_bwd_ex(*bargs, 32) == UNSUPPORTED
    assert lib.ssm_scan_bwd_ex(*bargs, 7) == WORKSPACE  # valid bits: fails later, on the workspace
    dargs = (2, 8, 4, 0) + (FAKE,) * 6 + (None, None, None, 1, FAKE, None)
    assert lib.ssm_state_update_ex(*dargs, 2) == UNSUPPORTED  # no direction for one token
    assert lib.ssm_state_update_ex(*dargs, 4) == UNSUPPORTED
    assert b"SSM_FLAG_ZOH" in lib.ssm_last_error()
    cargs = (1, 16, 8, 4, 0, FAKE, FAKE, None)
    rest = (FAKE, FAKE, FAKE, FAKE, None, None, None, 1, None, None, FAKE, None, None, 0, None)
    assert lib.ssm_scan_fwd_conv(*cargs, 4, *rest, 2) == UNSUPPORTED  # no reverse with the conv
    assert lib.ssm_scan_fwd_conv(*cargs, 5, *rest, 0) == UNSUPPORTED  # width above 4
    assert lib.ssm_scan_fwd_conv(*cargs, 0, *rest, 0) == UNSUPPORTED
    assert lib.ssm_scan_fwd_conv(1, 16, 8, 4, 0, FAKE, None, None, 4, *rest, 0) == NULL_ARG


def test_last_error_is_thread_local(lib):
    import threading
    assert _fwd(lib, L=0) == BAD_SHAPE
    seen = {}

    def other():
        seen["msg"] = lib.ssm_last_error()

    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen["msg"] == b""
    assert lib.ssm_last_error() != b""


def test_python_binding_rejects_cpu_tensors():
    import torch
    from selective_state_space_10_amd import scan_fwd
    x = torch.zeros(1, 4, 8)
    A = -torch.ones(8, 4)
    with pytest.raises(ValueError, match="GPU"):
        scan_fwd(x, x, A, torch.zeros(1, 4, 4), torch.zeros(1, 4, 4))


def test_header_compiles_as_c_and_cpp(tmp_path):
    """The C ABI header is plain C: it compiles with gcc as C11 and as C++."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    src = tmp_path / "use.c"
    src.write_text('#include "ssm_scan.h"\nint main(void) { return SSM_OK + SSM_FLAG_ZOH - 1; }\n')
    inc = os.path.dirname(HEADER)
    for lang in (["-x", "c", "-std=c11"], ["-x", "c++", "-std=c++17"]):
        r = subprocess.run(["gcc", *lang, "-Wall", "-Werror", "-fsyntax-only", "-I", inc, str(src)],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr


def test_missing_library_fails_loudly(monkeypatch):
    """No fallback: without the built HIP library the loader raises."""
    import selective_state_space_10_amd._lib as L
    monkeypatch.setattr(L, "_lib", None)
    monkeypatch.setattr(L, "LIB_PATH", os.path.join(ROOT, "no-such-dir", "libssm_scan.so"))
    with pytest.raises(ImportError, match="not built"):
        L.load()
