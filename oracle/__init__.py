"""Oracle for the Mamba-2 SSD core and its block shell (CPU, float64).

TEST INFRASTRUCTURE ONLY: tests, the smoke check and the benchmark's CPU
baseline leg may call it; the product path (the HIP library and its Python
binding) never imports it, and this package imports nothing from the product.

The arithmetic lives in ``ssd_oracle.c`` (plain C, sequential in time, f64);
this module converts numpy arrays to float64, calls it through ctypes and
returns float64 arrays.  Each function cites the passage it follows on the
burn_dragon_kernel 0.5.0 page "src/sequence/mamba2/backward.rs":

  ssd_fwd   -> ssd_forward_state_history_reference (recurrence) and the
               block backward's y readout
  ssd_bwd   -> ssd_backward_reference (reverse-time loop) + d(initial state)
  conv_fwd/conv_bwd -> depthwise_conv_preact_with_history, silu, conv tap loop
  rmsnorm_fwd/rmsnorm_bwd -> rmsnorm_gated_{forward,backward}_from_inv_rms
  dt_softplus_fwd/dt_softplus_bwd -> the dt_pre / softplus lines of
               tensorized_mamba2_backward_impl and the grad_dt_pre /
               grad_dt_bias lines after its fused backward (elementwise, so
               written here in numpy float64)

Parity pins (tests/test_oracle_*.py): the dual quadratic form of the forward,
central finite differences of every gradient, the A->0 and T=1 closed forms,
skip paths, group replication, linearity, the decay-gradient rectangle
identity, a hand-worked example under tests/golden/, and brute-force checks of
the shell ops.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import numpy as np

from .build import build_oracle, oracle_lib_path

_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        path = oracle_lib_path()
        if not os.path.exists(path):
            build_oracle()
        lib = ctypes.CDLL(path)
        i64, dp, cint, cdbl = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_double
        lib.ssd_oracle_fwd.argtypes = [i64] * 7 + [dp] * 10 + [cint]
        lib.ssd_oracle_bwd.argtypes = [i64] * 6 + [dp] * 16 + [cint]
        lib.conv_oracle_fwd.argtypes = [i64] * 4 + [dp] * 5
        lib.conv_oracle_bwd.argtypes = [i64] * 4 + [dp] * 7
        lib.rmsnorm_oracle_fwd.argtypes = [i64, i64, cdbl] + [dp] * 5
        lib.rmsnorm_oracle_bwd.argtypes = [i64, i64] + [dp] * 8
        for f in (lib.ssd_oracle_fwd, lib.ssd_oracle_bwd, lib.conv_oracle_fwd, lib.conv_oracle_bwd,
                  lib.rmsnorm_oracle_fwd, lib.rmsnorm_oracle_bwd):
            f.restype = cint
        _LIB = lib
    return _LIB


def default_threads() -> int:
    """Threads for the oracle's (batch, head) units: the CPUs this process may
    run on, at most 16 (one GPU's share of the host's cores on the machines
    the benchmark runs on, whatever the host's total)."""
    try:
        avail = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        avail = os.cpu_count() or 1
    return max(1, min(16, avail))


def _f64(a) -> Optional[np.ndarray]:
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dims(x, B, dt):
    b, T, H, P = x.shape
    N = B.shape[-1]
    G = B.shape[2]
    assert B.shape == (b, T, G, N) and dt.shape == (b, T, H)
    return b, T, H, P, N, G


def ssd_fwd(x, dt, A_log, B, C, D, h0=None, chunk: int = 0, nthreads: Optional[int] = None,
            want_y: bool = True) -> Dict[str, np.ndarray]:
    """Sequential forward.  Returns y [b,T,H,P], final [b,H,P,N] and, when
    ``chunk`` > 0, chunk_states [b,T/chunk,H,P,N] (state entering each chunk)."""
    x, dt, A_log, B, C, D, h0 = map(_f64, (x, dt, A_log, B, C, D, h0))
    b, T, H, P, N, G = _dims(x, B, dt)
    y = np.empty((b, T, H, P)) if want_y else None
    final = np.empty((b, H, P, N))
    cs = np.empty((b, T // chunk, H, P, N)) if chunk > 0 else None
    rc = _lib().ssd_oracle_fwd(b, T, H, P, N, G, chunk, *map(_ptr, (x, dt, A_log, B, C, D, h0, y, final, cs)),
                               nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"ssd_oracle_fwd failed ({rc})")
    out = {"final": final}
    if want_y:
        out["y"] = y
    if cs is not None:
        out["chunk_states"] = cs
    return out


def ssd_bwd(x, dt, A_log, B, C, D, dy, h0=None, nthreads: Optional[int] = None,
            dfinal=None) -> Dict[str, np.ndarray]:
    """Sequential analytic backward of L = sum(dy * y) + sum(dfinal * final).
    Returns dx, ddt, dA_log, dB, dC, dD and dh0 (gradient of the initial
    state; zeros state is used when h0 is None and dh0 is still returned).
    dfinal [b,H,P,N] (None: zeros) is the gradient of the state after the last
    step: it is the reverse-time loop's carry before its first step."""
    x, dt, A_log, B, C, D, h0, dy, dfinal = map(_f64, (x, dt, A_log, B, C, D, h0, dy, dfinal))
    b, T, H, P, N, G = _dims(x, B, dt)
    dx = np.empty_like(x)
    ddt = np.empty_like(dt)
    dA = np.empty(H)
    dB = np.empty_like(B)
    dC = np.empty_like(C)
    dD = np.empty(H)
    dh0 = np.empty((b, H, P, N))
    rc = _lib().ssd_oracle_bwd(b, T, H, P, N, G,
                               *map(_ptr, (x, dt, A_log, B, C, D, h0, dy, dfinal, dx, ddt, dA, dB, dC, dD, dh0)),
                               nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"ssd_oracle_bwd failed ({rc})")
    return dict(dx=dx, ddt=ddt, dA_log=dA, dB=dB, dC=dC, dD=dD, dh0=dh0)


def conv_fwd(xbc, w, bias):
    """Causal depthwise conv (zero initial state) + SiLU on [b,T,channels].
    Returns (preact, act)."""
    xbc, w, bias = map(_f64, (xbc, w, bias))
    b, T, cd = xbc.shape
    K = w.shape[1]
    pre = np.empty_like(xbc)
    act = np.empty_like(xbc)
    rc = _lib().conv_oracle_fwd(b, T, cd, K, *map(_ptr, (xbc, w, bias, pre, act)))
    if rc != 0:
        raise ValueError("conv_oracle_fwd failed")
    return pre, act


def conv_bwd(xbc, w, bias, gact):
    """Backward of conv_fwd's act.  Returns (dxbc, dw, dbias)."""
    xbc, w, bias, gact = map(_f64, (xbc, w, bias, gact))
    b, T, cd = xbc.shape
    K = w.shape[1]
    dx = np.empty_like(xbc)
    dw = np.empty_like(w)
    db = np.empty(cd)
    rc = _lib().conv_oracle_bwd(b, T, cd, K, *map(_ptr, (xbc, w, bias, gact, dx, dw, db)))
    if rc != 0:
        raise ValueError("conv_oracle_bwd failed")
    return dx, dw, db


def rmsnorm_fwd(y, z, w, eps: float):
    """RMSNorm over the last axis, then gate by silu(z).  Returns (out, inv_rms)."""
    y, z, w = map(_f64, (y, z, w))
    width = y.shape[-1]
    rows = y.size // width
    out = np.empty_like(y)
    inv = np.empty(y.shape[:-1])
    rc = _lib().rmsnorm_oracle_fwd(rows, width, float(eps), *map(_ptr, (y, z, w, out, inv)))
    if rc != 0:
        raise ValueError("rmsnorm_oracle_fwd failed")
    return out, inv


def rmsnorm_bwd(y, z, w, inv_rms, g):
    """Backward with the saved inv_rms.  Returns (dy, dz, dw)."""
    y, z, w, inv_rms, g = map(_f64, (y, z, w, inv_rms, g))
    width = y.shape[-1]
    rows = y.size // width
    dy = np.empty_like(y)
    dz = np.empty_like(y)
    dw = np.empty(width)
    rc = _lib().rmsnorm_oracle_bwd(rows, width, *map(_ptr, (y, z, w, inv_rms, g, dy, dz, dw)))
    if rc != 0:
        raise ValueError("rmsnorm_oracle_bwd failed")
    return dy, dz, dw


def dt_softplus_fwd(dt_raw, dt_bias):
    """dt = softplus(dt_raw + dt_bias) with beta 1, i.e. log(1 + e^v), over
    [..., H] (the burn_dragon_kernel backward.rs page: dt_pre = dt_raw + dt_bias, dt = softplus(dt_pre, 1.0)).
    np.logaddexp(0, v) is log(e^0 + e^v), the same function, without overflow."""
    v = _f64(dt_raw) + _f64(dt_bias)
    return np.logaddexp(0.0, v)


def dt_softplus_bwd(dt_raw, dt_bias, ddt):
    """Gradient through dt_softplus_fwd (the burn_dragon_kernel
    backward.rs page: grad_dt_pre = grad_dt *
    sigmoid(dt_pre); grad_dt_bias sums it over batch and time; grad_dt_raw is
    grad_dt_pre).  Returns (ddt_raw [..., H], d_dt_bias [H])."""
    v = _f64(dt_raw) + _f64(dt_bias)
    g = _f64(ddt) / (1.0 + np.exp(-v))
    H = g.shape[-1]
    return g, g.reshape(-1, H).sum(axis=0)
