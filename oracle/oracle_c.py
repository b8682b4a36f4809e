"""ctypes front-end of the fp64 C oracle (``ssm_oracle.c``).

Test infrastructure only: tests, the smoke check and bench.py's CPU-baseline
leg call it; the HIP path never does.  Inputs may be numpy arrays or CPU torch
tensors of any float dtype; they are upcast exactly to fp64.  Outputs are fp64
numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssm_oracle.c")
# ORACLE_LIB_OVERRIDE points the loader at another build (used to check that
# the pins fail on deliberately broken copies of the oracle).
_LIB_PATH = os.environ.get("ORACLE_LIB_OVERRIDE") or os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (fp64, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                               "-fno-fast-math", "-Wall", "-o", tmp, _SRC, "-lm", "-lpthread"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def build_sanitized(path: str) -> str:
    """Compile the oracle with AddressSanitizer and UndefinedBehaviorSanitizer
    (any undefined-behaviour report aborts) into ``path``, for a test run of the
    oracle's checks against it (load it with ORACLE_LIB_OVERRIDE=path and the
    ASan runtime preloaded).  Same floating-point flags as build()."""
    tmp = path + ".tmp"
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                           "-fno-fast-math", "-Wall", "-fno-omit-frame-pointer",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                           "-o", tmp, _SRC, "-lm", "-lpthread"])
    os.replace(tmp, path)
    return path


def _load():
    global _lib
    if _lib is None:
        if not os.environ.get("ORACLE_LIB_OVERRIDE") and (not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I = ctypes.c_int64
        CI = ctypes.c_int
        lib.oracle_scan_fwd.argtypes = [I, I, I, I] + [P] * 8 + [CI, P, P, P, I, P, CI]
        lib.oracle_scan_fwd.restype = CI
        lib.oracle_scan_fwd_ex.argtypes = lib.oracle_scan_fwd.argtypes + [CI]
        lib.oracle_scan_fwd_ex.restype = CI
        lib.oracle_scan_bwd.argtypes = [I, I, I, I] + [P] * 8 + [CI, P, P, P] + [P] * 9 + [CI]
        lib.oracle_scan_bwd.restype = CI
        lib.oracle_scan_bwd_ex.argtypes = lib.oracle_scan_bwd.argtypes + [CI]
        lib.oracle_scan_bwd_ex.restype = CI
        lib.oracle_state_update.argtypes = [I, I, I, P, P, P, P, P, P, P, P, P, CI, P]
        lib.oracle_state_update.restype = CI
        lib.oracle_state_update_ex.argtypes = lib.oracle_state_update.argtypes + [CI]
        lib.oracle_state_update_ex.restype = CI
        lib.oracle_conv1d_silu.argtypes = [I, I, I, I, P, P, P, P, P]
        lib.oracle_conv1d_silu.restype = CI
        lib.oracle_conv1d_silu_bwd.argtypes = [I, I, I, I, P, P, P, P, P, P, P]
        lib.oracle_conv1d_silu_bwd.restype = CI
        lib.oracle_affine_scan.argtypes = [I, I, P, P, P, P, CI]
        lib.oracle_affine_scan.restype = CI
        for f in ("oracle_softplus", "oracle_sigmoid", "oracle_silu"):
            getattr(lib, f).argtypes = [ctypes.c_double]
            getattr(lib, f).restype = ctypes.c_double
        _lib = lib
    return _lib


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor
        import torch
        x = x.detach().to("cpu", torch.float64).contiguous().numpy()
    return np.ascontiguousarray(x, dtype=np.float64)


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


ZOH, REVERSE, DELTA_PER_TOKEN = 1, 2, 4


def _flags(zoh, reverse, delta, u):
    f = (ZOH if zoh else 0) | (REVERSE if reverse else 0)
    if delta.ndim == 2:  # one raw step size per token, (B, L)
        if delta.shape != u.shape[:2]:
            raise ValueError("a per-token delta must be (batch, seqlen)")
        f |= DELTA_PER_TOKEN
    return f


def scan_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True, h0=None,
             chunk_len=None, nthreads=None, zoh=False, reverse=False):
    """Returns (y, h_final, chunk_states or None) in fp64.  ``zoh``: exact
    zero-order-hold input term; ``reverse``: scan from the last step to the
    first; a (batch, seqlen) ``delta`` is one step size per token."""
    u, delta, A, B, C = map(_f64, (u, delta, A, B, C))
    D, z, delta_bias, h0 = map(_f64, (D, z, delta_bias, h0))
    Bsz, L, Dm = u.shape
    N = A.shape[1]
    y = np.empty((Bsz, L, Dm))
    hf = np.empty((Bsz, Dm, N))
    cs = None
    if chunk_len:
        K = (L + chunk_len - 1) // chunk_len
        cs = np.empty((Bsz, K, Dm, N))
    rc = _load().oracle_scan_fwd_ex(Bsz, L, Dm, N, _p(u), _p(delta), _p(A), _p(B), _p(C), _p(D),
                                    _p(z), _p(delta_bias), int(bool(delta_softplus)), _p(h0), _p(y),
                                    _p(hf), int(chunk_len or 0), _p(cs),
                                    int(nthreads or default_threads()),
                                    _flags(zoh, reverse, delta, u))
    if rc != 0:
        raise ValueError(f"oracle_scan_fwd failed ({rc})")
    return y, hf, cs


def scan_bwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True, h0=None,
             dy=None, dh_final=None, nthreads=None, zoh=False, reverse=False):
    """Returns a dict of fp64 gradients: du, ddelta, dA, dB, dC, dD, dz, ddelta_bias, dh0
    (options as in scan_fwd; ddelta has delta's shape)."""
    u, delta, A, B, C = map(_f64, (u, delta, A, B, C))
    D, z, delta_bias, h0, dy, dh_final = map(_f64, (D, z, delta_bias, h0, dy, dh_final))
    Bsz, L, Dm = u.shape
    N = A.shape[1]
    out = dict(du=np.empty_like(u), ddelta=np.empty_like(delta), dA=np.empty((Dm, N)),
               dB=np.empty((Bsz, L, N)), dC=np.empty((Bsz, L, N)),
               dD=np.empty(Dm) if D is not None else None,
               dz=np.empty_like(u) if z is not None else None,
               ddelta_bias=np.empty(Dm) if delta_bias is not None else None,
               dh0=np.empty((Bsz, Dm, N)))
    rc = _load().oracle_scan_bwd_ex(Bsz, L, Dm, N, _p(u), _p(delta), _p(A), _p(B), _p(C), _p(D),
                                    _p(z), _p(delta_bias), int(bool(delta_softplus)), _p(h0), _p(dy),
                                    _p(dh_final), _p(out["du"]), _p(out["ddelta"]), _p(out["dA"]),
                                    _p(out["dB"]), _p(out["dC"]), _p(out["dD"]), _p(out["dz"]),
                                    _p(out["ddelta_bias"]), _p(out["dh0"]),
                                    int(nthreads or default_threads()),
                                    _flags(zoh, reverse, delta, u))
    if rc != 0:
        raise ValueError(f"oracle_scan_bwd failed ({rc})")
    return out


def state_update(state, u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True,
                 zoh=False):
    """One decode step. Returns (new_state, y) in fp64; the input is not modified."""
    st = _f64(state).copy()
    u, delta, A, B, C = map(_f64, (u, delta, A, B, C))
    D, z, delta_bias = map(_f64, (D, z, delta_bias))
    Bsz, Dm, N = st.shape
    y = np.empty((Bsz, Dm))
    rc = _load().oracle_state_update_ex(Bsz, Dm, N, _p(st), _p(u), _p(delta), _p(A), _p(B), _p(C),
                                        _p(D), _p(z), _p(delta_bias), int(bool(delta_softplus)),
                                        _p(y), ZOH if zoh else 0)
    if rc != 0:
        raise ValueError(f"oracle_state_update failed ({rc})")
    return st, y


def affine_scan(a, b, h0=None, reverse=False):
    """Sequential fold of h -> a h + b along the last axis from h0 (zeros if
    None); returns every state, fp64, a's shape."""
    a, b, h0 = _f64(a), _f64(b), _f64(h0)
    if a.shape != b.shape or a.ndim < 1:
        raise ValueError("a and b must have one shape")
    length = a.shape[-1]
    rows = a.size // length
    h = np.empty_like(a)
    if h0 is not None and h0.size != rows:
        raise ValueError("h0 must hold one state per row")
    rc = _load().oracle_affine_scan(rows, length, _p(a), _p(b), _p(h0), _p(h), int(bool(reverse)))
    if rc != 0:
        raise ValueError(f"oracle_affine_scan failed ({rc})")
    return h


def conv1d_silu(x, w, bias=None):
    """Causal depthwise convolution of width K = w.shape[1] over time, then SiLU.
    Returns (u, pre), both (B, L, D) fp64."""
    x, w, bias = _f64(x), _f64(w), _f64(bias)
    Bsz, L, Dm = x.shape
    u = np.empty_like(x)
    pre = np.empty_like(x)
    rc = _load().oracle_conv1d_silu(Bsz, L, Dm, w.shape[1], _p(x), _p(w), _p(bias), _p(pre), _p(u))
    if rc != 0:
        raise ValueError(f"oracle_conv1d_silu failed ({rc})")
    return u, pre


def conv1d_silu_bwd(x, w, bias, du):
    """Backward of conv1d_silu: returns (dx, dw, dbias or None)."""
    x, w, bias, du = _f64(x), _f64(w), _f64(bias), _f64(du)
    Bsz, L, Dm = x.shape
    dx = np.empty_like(x)
    dw = np.empty_like(w)
    db = np.empty(Dm) if bias is not None else None
    rc = _load().oracle_conv1d_silu_bwd(Bsz, L, Dm, w.shape[1], _p(x), _p(w), _p(bias), _p(du),
                                        _p(dx), _p(dw), _p(db))
    if rc != 0:
        raise ValueError(f"oracle_conv1d_silu_bwd failed ({rc})")
    return dx, dw, db


def scan_fwd_conv(x, conv_w, conv_b, delta, A, B, C, D=None, z=None, delta_bias=None,
                  delta_softplus=True, h0=None, chunk_len=None, nthreads=None, zoh=False):
    """The scan fed by the convolution: u = silu(conv(x)), then scan_fwd."""
    u, _ = conv1d_silu(x, conv_w, conv_b)
    return scan_fwd(u, delta, A, B, C, D, z, delta_bias, delta_softplus, h0, chunk_len,
                    nthreads, zoh=zoh)


def scan_bwd_conv(x, conv_w, conv_b, delta, A, B, C, D=None, z=None, delta_bias=None,
                  delta_softplus=True, h0=None, dy=None, dh_final=None, nthreads=None, zoh=False):
    """Backward of scan_fwd_conv: the scan gradients with du replaced by dx,
    plus dconv_w and dconv_b."""
    u, _ = conv1d_silu(x, conv_w, conv_b)
    g = scan_bwd(u, delta, A, B, C, D, z, delta_bias, delta_softplus, h0, dy, dh_final,
                 nthreads, zoh=zoh)
    dx, dw, db = conv1d_silu_bwd(x, conv_w, conv_b, g.pop("du"))
    g.update(dx=dx, dconv_w=dw, dconv_b=db)
    return g


def softplus(x: float) -> float:
    return _load().oracle_softplus(float(x))


def silu(x: float) -> float:
    return _load().oracle_silu(float(x))
