"""ctypes binding of libssd_mi355x.so (argument marshalling only)."""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libssd_mi355x.so"
_lib = None

SSD_F32, SSD_BF16 = 0, 1
_STATUS = {0: "SSD_OK", -1: "SSD_ERR_INVALID_ARG", -2: "SSD_ERR_SHAPE", -3: "SSD_ERR_DTYPE",
           -4: "SSD_ERR_WORKSPACE", -5: "SSD_ERR_HIP", -6: "SSD_ERR_ALIGN"}


class SSDError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


class Problem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("nheads", ctypes.c_int64),
                ("headdim", ctypes.c_int64), ("dstate", ctypes.c_int64), ("ngroups", ctypes.c_int64),
                ("chunk", ctypes.c_int64), ("act_dtype", ctypes.c_int32), ("dy_dtype", ctypes.c_int32)]


def library_path() -> str:
    return os.path.join(_HERE, _LIB_NAME)


def load_library():
    """Load the HIP library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m selective_state_space_mamba_amd.build`")
    lib = ctypes.CDLL(path)
    vp, sz, i64, i32, f32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
    pp = ctypes.POINTER(Problem)
    lib.ssd_workspace_bytes.argtypes = [pp, ctypes.c_int, ctypes.c_int]
    lib.ssd_workspace_bytes.restype = sz
    lib.ssd_fwd.argtypes = [pp] + [vp] * 10 + [vp, sz, vp]
    lib.ssd_fwd.restype = ctypes.c_int
    lib.ssd_bwd.argtypes = [pp] + [vp] * 17 + [vp, sz, vp]
    lib.ssd_bwd.restype = ctypes.c_int
    lib.ssd_fwd_ex.argtypes = [pp] + [vp] * 11 + [vp, sz, vp]
    lib.ssd_fwd_ex.restype = ctypes.c_int
    lib.ssd_bwd_ex.argtypes = [pp] + [vp] * 18 + [vp, sz, vp]
    lib.ssd_bwd_ex.restype = ctypes.c_int
    lib.ssd_bwd_noalloc.argtypes = [pp] + [vp] * 17 + [vp]
    lib.ssd_bwd_noalloc.restype = ctypes.c_int
    lib.mamba2_conv1d_silu_fwd.argtypes = [i64] * 6 + [i32] + [vp] * 6 + [vp]
    lib.mamba2_conv1d_silu_fwd.restype = ctypes.c_int
    lib.mamba2_conv1d_silu_bwd_workspace_bytes.argtypes = [i64] * 6
    lib.mamba2_conv1d_silu_bwd_workspace_bytes.restype = sz
    lib.mamba2_conv1d_silu_bwd.argtypes = [i64] * 6 + [i32] + [vp] * 6 + [i32, vp, i64, vp, vp] + [vp, sz, vp]
    lib.mamba2_conv1d_silu_bwd.restype = ctypes.c_int
    lib.mamba2_rmsnorm_gated_fwd.argtypes = [i64, i64, f32, i32] + [vp] * 5 + [vp]
    lib.mamba2_rmsnorm_gated_fwd.restype = ctypes.c_int
    lib.mamba2_rmsnorm_gated_bwd_workspace_bytes.argtypes = [i64, i64]
    lib.mamba2_rmsnorm_gated_bwd_workspace_bytes.restype = sz
    lib.mamba2_rmsnorm_gated_bwd.argtypes = [i64, i64, i32, i32, i32, i32] + [vp] * 7 + [i64, vp] + [vp, sz, vp]
    lib.mamba2_rmsnorm_gated_bwd.restype = ctypes.c_int
    lib.ssd_dt_softplus_fwd.argtypes = [i64, i64, i32] + [vp] * 3 + [vp]
    lib.ssd_dt_softplus_fwd.restype = ctypes.c_int
    lib.ssd_dt_softplus_bwd_workspace_bytes.argtypes = [i64, i64]
    lib.ssd_dt_softplus_bwd_workspace_bytes.restype = sz
    lib.ssd_dt_softplus_bwd.argtypes = [i64, i64, i32] + [vp] * 3 + [i32, vp, i64, vp] + [vp, sz, vp]
    lib.ssd_dt_softplus_bwd.restype = ctypes.c_int
    lib.ssd_gemm.argtypes = [i32, i32, i64, i64, i64, f32, vp, i64, vp, i64, f32, vp, i32, i64, vp]
    lib.ssd_gemm.restype = ctypes.c_int
    lib.ssd_cast_f32_to_bf16.argtypes = [i64, vp, vp, vp]
    lib.ssd_cast_f32_to_bf16.restype = ctypes.c_int
    lib.ssd_last_error.argtypes = []
    lib.ssd_last_error.restype = ctypes.c_char_p
    lib.ssd_version.argtypes = []
    lib.ssd_version.restype = ctypes.c_char_p
    lib.ssd_profile_enable.argtypes = [ctypes.c_int]
    lib.ssd_profile_enable.restype = ctypes.c_int
    lib.ssd_profile_only.argtypes = [ctypes.c_char_p]
    lib.ssd_profile_only.restype = ctypes.c_int
    lib.ssd_profile_kernel_ms.argtypes = [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                                          ctypes.POINTER(ctypes.c_int64)]
    lib.ssd_profile_kernel_ms.restype = ctypes.c_int
    _lib = lib
    return lib


def version() -> str:
    return load_library().ssd_version().decode()


def profile_enable(on: bool = True) -> None:
    """Clear earlier per-kernel timing records and turn recording on or off."""
    _check(load_library().ssd_profile_enable(int(on)))


def profile_only(kernel: str = "") -> None:
    """Record only this kernel's launches from now on ("" records every kernel)."""
    _check(load_library().ssd_profile_only(kernel.encode()))


def profile_kernel_ms(kernel: str) -> Tuple[float, int]:
    """(summed milliseconds, launches) of one kernel since profile_enable."""
    ms, n = ctypes.c_double(0.0), ctypes.c_int64(0)
    _check(load_library().ssd_profile_kernel_ms(kernel.encode(), ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def _check(rc: int):
    if rc != 0:
        raise SSDError(rc, load_library().ssd_last_error().decode())


def _code(dtype: torch.dtype) -> int:
    if dtype == torch.float32:
        return SSD_F32
    if dtype == torch.bfloat16:
        return SSD_BF16
    raise TypeError(f"unsupported dtype {dtype}: use float32 or bfloat16")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _need(t: torch.Tensor, name: str, shape, dtype=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _need_rows(t: torch.Tensor, name: str, shape, dtype, device) -> int:
    """Check an output whose rows (all but the last axis, flattened) may lie a
    fixed stride apart, e.g. a column slice of a wider matrix; returns that
    stride in elements."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dim() < 2 or t.stride(-1) != 1:
        raise ValueError(f"{name} must have unit stride along its last axis")
    ld = t.stride(-2)
    expect = ld
    for i in range(t.dim() - 2, -1, -1):
        if t.shape[i] > 1 and t.stride(i) != expect:
            raise ValueError(f"{name}'s rows must lie a fixed stride apart")
        expect *= t.shape[i]
    if ld < shape[-1]:
        raise ValueError(f"{name}'s row stride {ld} is below its row length {shape[-1]}")
    return ld


def _need_workspace(ws: Optional[torch.Tensor], device) -> int:
    """Byte size of a caller-supplied workspace (a contiguous uint8 device buffer)."""
    if ws is None:
        return 0
    if not isinstance(ws, torch.Tensor) or ws.dtype != torch.uint8:
        raise TypeError("workspace must be a torch.uint8 tensor")
    if not ws.is_contiguous():
        raise ValueError("workspace must be contiguous")
    if ws.device != device:
        raise ValueError(f"workspace is on {ws.device}, expected {device}")
    return ws.numel()


def _on_gpu(t: torch.Tensor, name: str):
    # the library takes device pointers only: a host pointer handed to a kernel
    # would fault the GPU, so host tensors are refused here
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU (cuda/hip device) tensor")


def make_problem(x: torch.Tensor, B: torch.Tensor, chunk: int, dy_dtype: Optional[torch.dtype] = None) -> Problem:
    b, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    act = _code(x.dtype)
    return Problem(b, T, H, P, N, G, chunk, act, _code(dy_dtype) if dy_dtype is not None else act)


def ssd_workspace_bytes(prob: Problem, for_backward: bool, has_chunk_states: bool) -> int:
    return int(load_library().ssd_workspace_bytes(ctypes.byref(prob), int(for_backward), int(has_chunk_states)))


def _check_inputs(x, dt, A_log, B, C, D, init_state):
    _on_gpu(x, "x")
    if x.dim() != 4 or B.dim() != 4:
        raise ValueError("x must be [b, T, H, P] and B, C [b, T, G, N]")
    b, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    dev = x.device
    _need(x, "x", (b, T, H, P), device=dev)
    _need(dt, "dt", (b, T, H), x.dtype, dev)
    _need(B, "B", (b, T, G, N), x.dtype, dev)
    _need(C, "C", (b, T, G, N), x.dtype, dev)
    _need(A_log, "A_log", (H,), torch.float32, dev)
    _need(D, "D", (H,), torch.float32, dev)
    if init_state is not None:
        _need(init_state, "init_state", (b, H, P, N), torch.float32, dev)
    return b, T, H, P, N, G


def ssd_fwd(x, dt, A_log, B, C, D, init_state=None, chunk: int = 256, want_chunk_states: bool = True,
            want_final_state: bool = True, out: Optional[Dict[str, torch.Tensor]] = None,
            workspace: Optional[torch.Tensor] = None, stream=None
            ) -> Tuple[torch.Tensor, Optional[torch.Tensor], Optional[torch.Tensor]]:
    """SSD forward.  Returns (y, final_state, chunk_states); the last two are
    None when not requested.  `out` may hold preallocated y / final_state /
    chunk_states; `workspace` a preallocated uint8 device buffer."""
    r = _fwd(x, dt, A_log, B, C, D, init_state, chunk, want_chunk_states, False, want_final_state, out, workspace,
             stream)
    return r["y"], r["final_state"], r["chunk_states"]


def ssd_fwd_ex(x, dt, A_log, B, C, D, init_state=None, chunk: int = 256, want_chunk_states: bool = False,
               want_chunk_states_bf16: bool = True, want_final_state: bool = True,
               out: Optional[Dict[str, torch.Tensor]] = None, workspace: Optional[torch.Tensor] = None,
               stream=None) -> Dict[str, Optional[torch.Tensor]]:
    """ssd_fwd_ex: the forward with the chunk states also (or only) in bf16,
    for problems the bf16 kernels run.  Returns a dict of y, final_state,
    chunk_states (f32) and chunk_states_bf16, None for those not requested;
    `out` may hold any of them preallocated."""
    return _fwd(x, dt, A_log, B, C, D, init_state, chunk, want_chunk_states, want_chunk_states_bf16,
                want_final_state, out, workspace, stream)


def _fwd(x, dt, A_log, B, C, D, init_state, chunk, want_chunk_states, want_chunk_states_bf16, want_final_state,
         out, workspace, stream) -> Dict[str, Optional[torch.Tensor]]:
    lib = load_library()
    b, T, H, P, N, G = _check_inputs(x, dt, A_log, B, C, D, init_state)
    prob = make_problem(x, B, chunk)
    out = out or {}
    nc = T // chunk if chunk > 0 else 0
    y = out.get("y")
    if y is None:
        y = torch.empty((b, T, H, P), dtype=x.dtype, device=x.device)
    _need(y, "out['y']", (b, T, H, P), x.dtype, x.device)
    fin = out.get("final_state")
    if fin is None and want_final_state:
        fin = torch.empty((b, H, P, N), dtype=torch.float32, device=x.device)
    if fin is not None:
        _need(fin, "out['final_state']", (b, H, P, N), torch.float32, x.device)
    cs = out.get("chunk_states")
    if cs is None and want_chunk_states:
        cs = torch.empty((b, nc, H, P, N), dtype=torch.float32, device=x.device)
    if cs is not None:
        _need(cs, "out['chunk_states']", (b, nc, H, P, N), torch.float32, x.device)
    csb = out.get("chunk_states_bf16")
    if csb is None and want_chunk_states_bf16:
        csb = torch.empty((b, nc, H, P, N), dtype=torch.bfloat16, device=x.device)
    if csb is not None:
        _need(csb, "out['chunk_states_bf16']", (b, nc, H, P, N), torch.bfloat16, x.device)
    need = lib.ssd_workspace_bytes(ctypes.byref(prob), 0, int(cs is not None))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    wsz = _need_workspace(workspace, x.device)
    _check(lib.ssd_fwd_ex(ctypes.byref(prob), _ptr(x), _ptr(dt), _ptr(A_log), _ptr(B), _ptr(C), _ptr(D),
                          _ptr(init_state), _ptr(y), _ptr(fin), _ptr(cs), _ptr(csb), _ptr(workspace), wsz,
                          _stream(stream)))
    return {"y": y, "final_state": fin, "chunk_states": cs, "chunk_states_bf16": csb}


def ssd_bwd(x, dt, A_log, B, C, D, dy, init_state=None, chunk_states=None, chunk: int = 256,
            want_d_init_state: bool = True, out: Optional[Dict[str, torch.Tensor]] = None,
            workspace: Optional[torch.Tensor] = None, stream=None,
            d_final_state: Optional[torch.Tensor] = None,
            chunk_states_bf16: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """SSD backward of sum(dy * y) + sum(d_final_state * final_state).
    Returns dx, ddt, dA_log, dB, dC, dD (f32) and d_init_state (f32, or None
    when not requested).  `chunk_states_bf16` is the bf16 history that
    ssd_fwd_ex wrote (ssd_bwd_ex of the library)."""
    lib = load_library()
    b, T, H, P, N, G = _check_inputs(x, dt, A_log, B, C, D, init_state)
    if dy.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("dy must be float32 or bfloat16")
    _need(dy, "dy", (b, T, H, P), device=x.device)
    if d_final_state is not None:
        _need(d_final_state, "d_final_state", (b, H, P, N), torch.float32, x.device)
    if chunk_states is not None:
        _need(chunk_states, "chunk_states", (b, T // chunk, H, P, N), torch.float32, x.device)
    if chunk_states_bf16 is not None:
        _need(chunk_states_bf16, "chunk_states_bf16", (b, T // chunk, H, P, N), torch.bfloat16, x.device)
    prob = make_problem(x, B, chunk, dy.dtype)
    out = dict(out or {})
    f32 = dict(dtype=torch.float32, device=x.device)
    shapes = dict(dx=(b, T, H, P), ddt=(b, T, H), dA_log=(H,), dB=(b, T, G, N), dC=(b, T, G, N), dD=(H,))
    for k, s in shapes.items():
        if out.get(k) is None:
            out[k] = torch.empty(s, **f32)
        _need(out[k], f"out['{k}']", s, torch.float32, x.device)
    if want_d_init_state and out.get("d_init_state") is None:
        out["d_init_state"] = torch.empty((b, H, P, N), **f32)
    dinit = out.get("d_init_state")
    if dinit is not None:
        _need(dinit, "out['d_init_state']", (b, H, P, N), torch.float32, x.device)
    need = lib.ssd_workspace_bytes(ctypes.byref(prob), 1, int(chunk_states is not None))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    wsz = _need_workspace(workspace, x.device)
    _check(lib.ssd_bwd_ex(ctypes.byref(prob), _ptr(x), _ptr(dt), _ptr(A_log), _ptr(B), _ptr(C), _ptr(D),
                          _ptr(init_state), _ptr(chunk_states), _ptr(chunk_states_bf16), _ptr(dy),
                          _ptr(d_final_state), _ptr(out["dx"]), _ptr(out["ddt"]), _ptr(out["dA_log"]),
                          _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dD"]), _ptr(dinit), _ptr(workspace), wsz,
                          _stream(stream)))
    out["d_init_state"] = dinit
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20  # SSD_NOALLOC_SCRATCH_BYTES of include/ssd.h


def ssd_bwd_noalloc(x, dt, A_log, B, C, D, dy, out: Dict[str, torch.Tensor], init_state=None, chunk_states=None,
                    chunk: int = 256, stream=None, d_final_state: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """ssd_bwd through the entry point that allocates nothing (the library's
    static scratch instead of a workspace).  `out` must hold every output
    (dx, ddt, dA_log, dB, dC, dD, and d_init_state or None); nothing is
    allocated here either."""
    lib = load_library()
    b, T, H, P, N, G = _check_inputs(x, dt, A_log, B, C, D, init_state)
    if dy.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("dy must be float32 or bfloat16")
    _need(dy, "dy", (b, T, H, P), device=x.device)
    if d_final_state is not None:
        _need(d_final_state, "d_final_state", (b, H, P, N), torch.float32, x.device)
    if chunk_states is not None:
        _need(chunk_states, "chunk_states", (b, T // chunk, H, P, N), torch.float32, x.device)
    shapes = dict(dx=(b, T, H, P), ddt=(b, T, H), dA_log=(H,), dB=(b, T, G, N), dC=(b, T, G, N), dD=(H,))
    for k, s_ in shapes.items():
        if out.get(k) is None:
            raise ValueError(f"out['{k}'] is required")
        _need(out[k], f"out['{k}']", s_, torch.float32, x.device)
    dinit = out.get("d_init_state")
    if dinit is not None:
        _need(dinit, "out['d_init_state']", (b, H, P, N), torch.float32, x.device)
    prob = make_problem(x, B, chunk, dy.dtype)
    _check(lib.ssd_bwd_noalloc(ctypes.byref(prob), _ptr(x), _ptr(dt), _ptr(A_log), _ptr(B), _ptr(C), _ptr(D),
                               _ptr(init_state), _ptr(chunk_states), _ptr(dy), _ptr(d_final_state), _ptr(out["dx"]),
                               _ptr(out["ddt"]), _ptr(out["dA_log"]), _ptr(out["dB"]), _ptr(out["dC"]),
                               _ptr(out["dD"]), _ptr(dinit), _stream(stream)))
    return out


def conv1d_silu_fwd(xbc, w, bias, d_inner: int, ngroups: int, dstate: int, stream=None):
    """Causal depthwise conv1d + SiLU on xbc [b,T,conv_dim]; returns
    (x [b,T,d_inner], B [b,T,G,N], C [b,T,G,N]) in xbc's dtype."""
    _on_gpu(xbc, "xbc")
    lib = load_library()
    b, T, cd = xbc.shape
    K = w.shape[1]
    _need(xbc, "xbc", (b, T, d_inner + 2 * ngroups * dstate), device=xbc.device)
    _need(w, "w", (cd, K), torch.float32, xbc.device)
    if bias is not None:
        _need(bias, "bias", (cd,), torch.float32, xbc.device)
    xo = torch.empty((b, T, d_inner), dtype=xbc.dtype, device=xbc.device)
    Bo = torch.empty((b, T, ngroups, dstate), dtype=xbc.dtype, device=xbc.device)
    Co = torch.empty_like(Bo)
    _check(lib.mamba2_conv1d_silu_fwd(b, T, d_inner, ngroups, dstate, K, _code(xbc.dtype), _ptr(xbc), _ptr(w),
                                      _ptr(bias), _ptr(xo), _ptr(Bo), _ptr(Co), _stream(stream)))
    return xo, Bo, Co


def conv1d_silu_bwd(xbc, w, bias, dx, dB, dC, d_inner: int, ngroups: int, dstate: int, workspace=None,
                    stream=None, dxbc_dtype=torch.float32, out=None):
    """Backward of conv1d_silu_fwd given f32 gradients of its outputs; returns
    (dxbc [b,T,conv_dim] in dxbc_dtype (f32, or bf16 rounded to nearest even),
    dw [conv_dim,d_conv] f32, dbias [conv_dim] f32).  `out` may give dxbc: its
    rows may lie a fixed stride apart (a column slice of a wider matrix, with
    the stride a multiple of 4)."""
    _on_gpu(xbc, "xbc")
    lib = load_library()
    b, T, cd = xbc.shape
    K = w.shape[1]
    _need(dx, "dx", (b, T, d_inner), torch.float32, xbc.device)
    _need(dB, "dB", (b, T, ngroups, dstate), torch.float32, xbc.device)
    _need(dC, "dC", (b, T, ngroups, dstate), torch.float32, xbc.device)
    if dxbc_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("dxbc_dtype must be torch.float32 or torch.bfloat16")
    f32 = dict(dtype=torch.float32, device=xbc.device)
    if out is None:
        dxbc = torch.empty((b, T, cd), dtype=dxbc_dtype, device=xbc.device)
        ld = cd
    else:
        dxbc = out
        ld = _need_rows(dxbc, "out (dxbc)", (b, T, cd), dxbc_dtype, xbc.device)
    dw = torch.empty((cd, K), **f32)
    db = torch.empty((cd,), **f32)
    need = lib.mamba2_conv1d_silu_bwd_workspace_bytes(b, T, d_inner, ngroups, dstate, K)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=xbc.device)
    wsz = _need_workspace(workspace, xbc.device)
    _check(lib.mamba2_conv1d_silu_bwd(b, T, d_inner, ngroups, dstate, K, _code(xbc.dtype), _ptr(xbc), _ptr(w),
                                      _ptr(bias), _ptr(dx), _ptr(dB), _ptr(dC), _code(dxbc_dtype), _ptr(dxbc), ld,
                                      _ptr(dw), _ptr(db),
                                      _ptr(workspace), wsz, _stream(stream)))
    return dxbc, dw, db


def rmsnorm_gated_fwd(y, z, w, eps: float = 1e-5, stream=None):
    """RMSNorm over the last axis of y, times w * silu(z).  Returns
    (out in y's dtype, inv_rms f32 over the leading axes)."""
    _on_gpu(y, "y")
    lib = load_library()
    width = y.shape[-1]
    rows = y.numel() // width if width else 0
    _need(z, "z", tuple(y.shape), y.dtype, y.device)
    _need(w, "w", (width,), torch.float32, y.device)
    if not y.is_contiguous():
        raise ValueError("y must be contiguous")
    out = torch.empty_like(y)
    inv = torch.empty(tuple(y.shape[:-1]), dtype=torch.float32, device=y.device)
    _check(lib.mamba2_rmsnorm_gated_fwd(rows, width, float(eps), _code(y.dtype), _ptr(y), _ptr(z), _ptr(w),
                                        _ptr(out), _ptr(inv), _stream(stream)))
    return out, inv


def rmsnorm_gated_bwd(y, z, w, inv_rms, g, workspace=None, stream=None, dy_dtype=torch.float32,
                      dz_dtype=torch.float32, dz_out=None):
    """Backward of rmsnorm_gated_fwd with the saved inv_rms; returns
    (dy in dy_dtype, dz in dz_dtype, dw f32); bf16 outputs are rounded to
    nearest even.  dz_out may give dz: its rows may lie a fixed stride apart
    (a column slice of a wider matrix, the stride a multiple of 8)."""
    _on_gpu(y, "y")
    lib = load_library()
    width = y.shape[-1]
    rows = y.numel() // width if width else 0
    _need(z, "z", tuple(y.shape), y.dtype, y.device)
    _need(w, "w", (width,), torch.float32, y.device)
    _need(inv_rms, "inv_rms", tuple(y.shape[:-1]), torch.float32, y.device)
    _need(g, "g", tuple(y.shape), None, y.device)
    for name, dt_ in (("dy_dtype", dy_dtype), ("dz_dtype", dz_dtype)):
        if dt_ not in (torch.float32, torch.bfloat16):
            raise TypeError(f"{name} must be torch.float32 or torch.bfloat16")
    f32 = dict(dtype=torch.float32, device=y.device)
    dy = torch.empty(tuple(y.shape), dtype=dy_dtype, device=y.device)
    if dz_out is None:
        dz = torch.empty(tuple(y.shape), dtype=dz_dtype, device=y.device)
        zld = width
    else:
        dz = dz_out
        zld = _need_rows(dz, "dz_out", tuple(y.shape), dz_dtype, y.device)
    dw = torch.empty((width,), **f32)
    need = lib.mamba2_rmsnorm_gated_bwd_workspace_bytes(rows, width)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=y.device)
    wsz = _need_workspace(workspace, y.device)
    _check(lib.mamba2_rmsnorm_gated_bwd(rows, width, _code(y.dtype), _code(g.dtype), _code(dy_dtype),
                                        _code(dz_dtype), _ptr(y), _ptr(z), _ptr(w),
                                        _ptr(inv_rms), _ptr(g), _ptr(dy), _ptr(dz), zld, _ptr(dw), _ptr(workspace), wsz,
                                        _stream(stream)))
    return dy, dz, dw


def dt_softplus_fwd(dt_raw, dt_bias, out=None, stream=None):
    """dt = softplus(dt_raw + dt_bias) over [..., H] in dt_raw's dtype (the form
    ssd_fwd / ssd_bwd take as dt)."""
    _on_gpu(dt_raw, "dt_raw")
    lib = load_library()
    H = dt_raw.shape[-1]
    rows = dt_raw.numel() // H if H else 0
    _need(dt_raw, "dt_raw", tuple(dt_raw.shape), None, dt_raw.device)
    _need(dt_bias, "dt_bias", (H,), torch.float32, dt_raw.device)
    dt = torch.empty_like(dt_raw) if out is None else out
    _need(dt, "out", tuple(dt_raw.shape), dt_raw.dtype, dt_raw.device)
    _check(lib.ssd_dt_softplus_fwd(rows, H, _code(dt_raw.dtype), _ptr(dt_raw), _ptr(dt_bias), _ptr(dt),
                                   _stream(stream)))
    return dt


def dt_softplus_bwd(dt_raw, dt_bias, ddt, workspace=None, out=None, stream=None, out_dtype=torch.float32):
    """Backward of dt_softplus_fwd: returns (ddt_raw [..., H] in out_dtype (f32,
    or bf16 rounded to nearest even), d_dt_bias f32 [H]) from ddt, the gradient
    of dt that ssd_bwd returns.  A given ddt_raw (out[0]) may have its rows a
    fixed stride apart (a column slice of a wider matrix)."""
    _on_gpu(dt_raw, "dt_raw")
    lib = load_library()
    H = dt_raw.shape[-1]
    rows = dt_raw.numel() // H if H else 0
    _need(dt_raw, "dt_raw", tuple(dt_raw.shape), None, dt_raw.device)
    _need(dt_bias, "dt_bias", (H,), torch.float32, dt_raw.device)
    _need(ddt, "ddt", tuple(dt_raw.shape), torch.float32, dt_raw.device)
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out_dtype must be torch.float32 or torch.bfloat16")
    f32 = dict(dtype=torch.float32, device=dt_raw.device)
    if out is None:
        out = (torch.empty(tuple(dt_raw.shape), dtype=out_dtype, device=dt_raw.device), torch.empty((H,), **f32))
    ddt_raw, d_bias = out
    ld = _need_rows(ddt_raw, "out[0] (ddt_raw)", tuple(dt_raw.shape), out_dtype, dt_raw.device) \
        if ddt_raw.dim() >= 2 else H
    if ddt_raw.dim() < 2:
        _need(ddt_raw, "out[0] (ddt_raw)", tuple(dt_raw.shape), out_dtype, dt_raw.device)
    _need(d_bias, "out[1] (d_dt_bias)", (H,), torch.float32, dt_raw.device)
    need = lib.ssd_dt_softplus_bwd_workspace_bytes(rows, H)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dt_raw.device)
    wsz = _need_workspace(workspace, dt_raw.device)
    _check(lib.ssd_dt_softplus_bwd(rows, H, _code(dt_raw.dtype), _ptr(dt_raw), _ptr(dt_bias), _ptr(ddt),
                                   _code(out_dtype), _ptr(ddt_raw), ld, _ptr(d_bias), _ptr(workspace), wsz,
                                   _stream(stream)))
    return ddt_raw, d_bias


def gemm(A, B, trans_a: bool = False, trans_b: bool = False, out=None, out_dtype=torch.bfloat16,
         alpha: float = 1.0, beta: float = 0.0, stream=None):
    """out[m,n] = alpha * op(A) @ op(B) + beta * out for 2-D contiguous bf16 A, B
    (op transposes when trans_*); out in out_dtype (bf16 or f32)."""
    _on_gpu(A, "A")
    lib = load_library()
    _on_gpu(B, "B")
    if B.device != A.device:
        raise ValueError(f"B is on {B.device}, expected {A.device}")
    if A.dtype != torch.bfloat16 or B.dtype != torch.bfloat16:
        raise TypeError("gemm takes bfloat16 operands")
    if A.dim() != 2 or B.dim() != 2 or not A.is_contiguous() or not B.is_contiguous():
        raise ValueError("gemm takes contiguous 2-D operands")
    m, k = (A.shape[1], A.shape[0]) if trans_a else (A.shape[0], A.shape[1])
    kb, n = (B.shape[1], B.shape[0]) if trans_b else (B.shape[0], B.shape[1])
    if kb != k:
        raise ValueError(f"gemm: inner sizes {k} and {kb} differ")
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=A.device)
    _need(out, "out", (m, n), None, A.device)
    _check(lib.ssd_gemm(int(trans_a), int(trans_b), m, n, k, float(alpha), _ptr(A), A.shape[1], _ptr(B),
                        B.shape[1], float(beta), _ptr(out), _code(out.dtype), n, _stream(stream)))
    return out


def cast_bf16(src, out=None, stream=None):
    """bf16 copy (round to nearest even) of a contiguous f32 tensor."""
    _on_gpu(src, "src")
    lib = load_library()
    if src.dtype != torch.float32 or not src.is_contiguous():
        raise TypeError("cast_bf16 takes a contiguous float32 tensor")
    if out is None:
        out = torch.empty(src.shape, dtype=torch.bfloat16, device=src.device)
    _need(out, "out", tuple(src.shape), torch.bfloat16, src.device)
    _check(lib.ssd_cast_f32_to_bf16(src.numel(), _ptr(src), _ptr(out), _stream(stream)))
    return out
