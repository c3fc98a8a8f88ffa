"""C-ABI checks that need no GPU: the library loads, exports every function
include/ssd.h declares, and rejects bad arguments with the documented status
before enqueuing anything (these paths make no HIP call)."""
import ctypes
import os
import re

import pytest

from selective_state_space_mamba_amd import _binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bd.library_path()):
        from selective_state_space_mamba_amd.build import build
        build()
    return bd.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "sizeof")))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("ssd_fwd", "ssd_bwd", "ssd_fwd_ex", "ssd_bwd_ex", "ssd_workspace_bytes", "ssd_last_error",
              "mamba2_conv1d_silu_fwd",
              "mamba2_conv1d_silu_bwd", "mamba2_rmsnorm_gated_fwd", "mamba2_rmsnorm_gated_bwd",
              "ssd_dt_softplus_fwd", "ssd_dt_softplus_bwd", "ssd_dt_softplus_bwd_workspace_bytes"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for n in declared_functions():
        assert hasattr(lib, n), n
    assert "gfx950" in lib.ssd_version().decode()


def prob(**kw):
    base = dict(batch=2, seqlen=512, nheads=8, headdim=64, dstate=128, ngroups=2, chunk=256, act_dtype=0, dy_dtype=0)
    base.update(kw)
    return bd.Problem(**base)


FAKE = 1 << 20  # a 16-byte aligned non-null address that is never dereferenced


def call_fwd(lib, p, ws_bytes=1 << 30, misalign=None, null=None):
    ptrs = {k: ctypes.c_void_p(FAKE) for k in ("x", "dt", "A_log", "B", "C", "D", "y", "ws")}
    if misalign:
        ptrs[misalign] = ctypes.c_void_p(FAKE + 2)
    if null:
        ptrs[null] = None
    return lib.ssd_fwd(ctypes.byref(p), ptrs["x"], ptrs["dt"], ptrs["A_log"], ptrs["B"], ptrs["C"], ptrs["D"],
                       None, ptrs["y"], None, None, ptrs["ws"], ws_bytes, None)


def call_bwd(lib, p, ws_bytes=1 << 30, misalign=None, null=None):
    names = ("x", "dt", "A_log", "B", "C", "D", "dy", "dx", "ddt", "dA_log", "dB", "dC", "dD", "ws")
    ptrs = {k: ctypes.c_void_p(FAKE) for k in names}
    if misalign:
        ptrs[misalign] = ctypes.c_void_p(FAKE + 4)
    if null:
        ptrs[null] = None
    return lib.ssd_bwd(ctypes.byref(p), ptrs["x"], ptrs["dt"], ptrs["A_log"], ptrs["B"], ptrs["C"], ptrs["D"],
                       None, None, ptrs["dy"], None, ptrs["dx"], ptrs["ddt"], ptrs["dA_log"], ptrs["dB"],
                       ptrs["dC"], ptrs["dD"], None, ptrs["ws"], ws_bytes, None)


@pytest.mark.parametrize("kw,status,text", [
    (dict(act_dtype=7), -3, "act_dtype"),
    (dict(dy_dtype=-1), -3, "dy_dtype"),
    (dict(headdim=65), -2, "headdim"),
    (dict(dstate=129), -2, "dstate"),
    (dict(chunk=512, seqlen=1024), -2, "chunk"),
    (dict(seqlen=500), -2, "multiple of chunk"),
    (dict(nheads=6, ngroups=4), -2, "multiple of ngroups"),
    (dict(nheads=0), -1, "must be > 0"),
    (dict(batch=-1), -1, ">= 0"),
])
def test_invalid_problem_statements(lib, kw, status, text):
    p = prob(**kw)
    for f in (call_fwd, call_bwd):
        assert f(lib, p) == status
        assert text in lib.ssd_last_error().decode()
    assert lib.ssd_workspace_bytes(ctypes.byref(p), 1, 0) == 0


def test_null_problem(lib):
    assert lib.ssd_fwd(None, *([None] * 10), None, 0, None) == -1
    assert "null" in lib.ssd_last_error().decode()


@pytest.mark.parametrize("which", ["x", "dt", "B", "C", "y", "A_log", "D"])
def test_fwd_null_required_pointer(lib, which):
    assert call_fwd(lib, prob(), null=which) == -1


@pytest.mark.parametrize("which", ["dy", "dx", "ddt", "dB", "dC", "dA_log", "dD"])
def test_bwd_null_required_pointer(lib, which):
    assert call_bwd(lib, prob(), null=which) == -1


def test_misaligned_pointer(lib):
    assert call_fwd(lib, prob(), misalign="B") == -6
    assert call_bwd(lib, prob(), misalign="dy") == -6


def test_workspace_too_small(lib):
    p = prob()
    need_f = lib.ssd_workspace_bytes(ctypes.byref(p), 0, 0)
    need_b = lib.ssd_workspace_bytes(ctypes.byref(p), 1, 0)
    assert need_f > 0 and need_b > need_f
    assert call_fwd(lib, p, ws_bytes=need_f - 1) == -4
    assert call_bwd(lib, p, ws_bytes=need_b - 1) == -4
    assert call_bwd(lib, p, null="ws") == -4
    assert "workspace" in lib.ssd_last_error().decode()


def test_workspace_sizes_follow_the_plan(lib):
    # forward: the chunk states, unless the caller passes them, and the
    # per-chunk total log-decay [b, nc, H] of the two-pass f32 state form
    p = prob()
    nc = 512 // 256
    states = 4 * 2 * nc * 8 * 64 * 128
    send = 256  # 4 * 2 * nc * 8 bytes, rounded up to the 256-byte alignment
    assert lib.ssd_workspace_bytes(ctypes.byref(p), 0, 0) == states + send
    assert lib.ssd_workspace_bytes(ctypes.byref(p), 0, 1) == send
    # backward needs at least the state gradients, plus the states in recompute mode
    wb1 = lib.ssd_workspace_bytes(ctypes.byref(p), 1, 1)
    wb0 = lib.ssd_workspace_bytes(ctypes.byref(p), 1, 0)
    assert wb1 >= states and wb0 == wb1 + states


def test_bf16_workspace_sizes(lib, monkeypatch):
    # bf16 problems: the forward keeps only the bf16 copy of the states (its
    # output kernel reads that), whether or not the caller takes the f32
    # ones; the fused backward reads the states only in bf16, so it needs no
    # f32 slot for recomputed states either
    monkeypatch.delenv("SSD_BF16_BWD", raising=False)
    p = prob(act_dtype=1, dy_dtype=1)
    nc = 512 // 256
    states = 4 * 2 * nc * 8 * 64 * 128
    send = 256
    assert lib.ssd_workspace_bytes(ctypes.byref(p), 0, 0) == states // 2 + send
    assert lib.ssd_workspace_bytes(ctypes.byref(p), 0, 1) == states // 2 + send
    assert lib.ssd_workspace_bytes(ctypes.byref(p), 1, 0) == lib.ssd_workspace_bytes(ctypes.byref(p), 1, 1)


def test_bf16_history_needs_a_bf16_problem(lib):
    # an f32 problem (or bf16 activations with f32 dy in the backward) has no
    # bf16 history: rejected before any launch
    f = ctypes.c_void_p(FAKE)
    for kw in (dict(), dict(act_dtype=1, dy_dtype=0), dict(act_dtype=1, dy_dtype=1, headdim=60)):
        p = prob(**kw)
        assert lib.ssd_bwd_ex(ctypes.byref(p), f, f, f, f, f, f, None, None, f, f, None, f, f, f, f, f, f, None, f,
                              1 << 30, None) == -1
        assert "chunk_states_bf16" in lib.ssd_last_error().decode()
    for kw in (dict(), dict(act_dtype=1, headdim=60)):
        p = prob(**kw)
        assert lib.ssd_fwd_ex(ctypes.byref(p), f, f, f, f, f, f, None, f, None, None, f, f, 1 << 30, None) == -1
        assert "chunk_states_bf16" in lib.ssd_last_error().decode()


def test_shell_argument_checks(lib):
    f = ctypes.c_void_p(FAKE)
    assert lib.mamba2_conv1d_silu_fwd(1, 8, 64, 1, 16, 9, 0, f, f, f, f, f, f, None) == -2  # d_conv > 8
    assert lib.mamba2_conv1d_silu_fwd(1, 8, 64, 1, 16, 4, 5, f, f, f, f, f, f, None) == -3
    assert lib.mamba2_conv1d_silu_fwd(1, 8, 64, 1, 16, 4, 0, None, f, f, f, f, f, None) == -1
    assert lib.mamba2_rmsnorm_gated_fwd(4, 5000, 1e-5, 0, f, f, f, f, f, None) == -2
    assert lib.mamba2_rmsnorm_gated_fwd(4, 64, 1e-5, 0, f, None, f, f, f, None) == -1
    need = lib.mamba2_rmsnorm_gated_bwd_workspace_bytes(100, 64)
    assert need > 0
    assert lib.mamba2_rmsnorm_gated_bwd(100, 64, 0, 0, 0, 0, f, f, f, f, f, f, f, 0, f, f, need - 1, None) == -4
    assert lib.mamba2_rmsnorm_gated_bwd(100, 64, 0, 0, 7, 0, f, f, f, f, f, f, f, 0, f, f, need, None) == -3
    assert lib.mamba2_rmsnorm_gated_bwd(100, 64, 0, 0, 0, 7, f, f, f, f, f, f, f, 0, f, f, need, None) == -3
    # dz_ld below width, or above it but not a multiple of 8
    assert lib.mamba2_rmsnorm_gated_bwd(100, 64, 0, 0, 0, 0, f, f, f, f, f, f, f, 60, f, f, need, None) == -1
    assert lib.mamba2_rmsnorm_gated_bwd(100, 64, 0, 0, 0, 0, f, f, f, f, f, f, f, 68, f, f, need, None) == -1
    cneed = lib.mamba2_conv1d_silu_bwd_workspace_bytes(2, 300, 64, 1, 16, 4)
    assert cneed > 0
    assert lib.mamba2_conv1d_silu_bwd(2, 300, 64, 1, 16, 4, 0, f, f, f, f, f, f, 7, f, 0, f, f, f, cneed, None) == -3
    # dxbc_ld below conv_dim (96) or not a multiple of 4
    assert lib.mamba2_conv1d_silu_bwd(2, 300, 64, 1, 16, 4, 0, f, f, f, f, f, f, 0, f, 92, f, f, f, cneed, None) == -1
    assert lib.mamba2_conv1d_silu_bwd(2, 300, 64, 1, 16, 4, 0, f, f, f, f, f, f, 0, f, 98, f, f, f, cneed, None) == -1
    # a packed row of a conv_dim that is not a multiple of 4 (65 + 2 * 1 = 67) passes the stride
    # check: the call stops at the next one, the (too small) workspace, before any launch
    need67 = lib.mamba2_conv1d_silu_bwd_workspace_bytes(2, 300, 65, 1, 1, 4)
    assert lib.mamba2_conv1d_silu_bwd(2, 300, 65, 1, 1, 4, 0, f, f, f, f, f, f, 0, f, 67, f, f, f, need67 - 1,
                                      None) == -4
    dneed = lib.ssd_dt_softplus_bwd_workspace_bytes(100, 8)
    assert lib.ssd_dt_softplus_bwd(100, 8, 0, f, f, f, 7, f, 0, f, f, dneed, None) == -3
    assert lib.ssd_dt_softplus_bwd(100, 8, 0, f, f, f, 0, f, 4, f, f, dneed, None) == -1  # ld below nheads


def test_dt_softplus_argument_checks(lib):
    f = ctypes.c_void_p(FAKE)
    lib.ssd_dt_softplus_bwd_workspace_bytes.restype = ctypes.c_size_t
    i64 = ctypes.c_int64
    assert lib.ssd_dt_softplus_fwd(i64(10), i64(4), 3, f, f, f, None) == -3      # unknown dtype
    assert lib.ssd_dt_softplus_fwd(i64(10), i64(0), 0, f, f, f, None) == -1      # no heads
    assert lib.ssd_dt_softplus_fwd(i64(10), i64(4), 0, f, None, f, None) == -1   # bias required
    assert lib.ssd_dt_softplus_fwd(i64(10), i64(4), 0, ctypes.c_void_p(FAKE + 4), f, f, None) == -6
    need = lib.ssd_dt_softplus_bwd_workspace_bytes(i64(100), i64(4))
    assert need >= 2 * 4 * 4  # two 64-row partials of 4 heads (at most 64 rows each)
    assert lib.ssd_dt_softplus_bwd(i64(100), i64(4), 0, f, f, f, 0, f, i64(0), f, f, ctypes.c_size_t(need - 1),
                                   None) == -4
    assert lib.ssd_dt_softplus_bwd(i64(100), i64(4), 0, f, f, f, 0, None, i64(0), f, f, ctypes.c_size_t(need),
                                   None) == -1


def test_product_path_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "selective_state_space_mamba_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".cpp", ".hip", ".hpp", ".h")):
                text = open(os.path.join(dirpath, fn)).read()
                assert "oracle" not in text.lower(), fn


def test_gemm_and_cast_argument_checks(lib):
    f = ctypes.c_void_p(FAKE)
    i64 = ctypes.c_int64
    # c_dtype unknown, negative size, row stride shorter than the row, misaligned
    assert lib.ssd_gemm(0, 0, i64(4), i64(4), i64(4), 1.0, f, i64(4), f, i64(4), 0.0, f, 9, i64(4), None) == -3
    assert lib.ssd_gemm(0, 0, i64(-1), i64(4), i64(4), 1.0, f, i64(4), f, i64(4), 0.0, f, 0, i64(4), None) == -1
    assert lib.ssd_gemm(0, 1, i64(4), i64(8), i64(16), 1.0, f, i64(16), f, i64(8), 0.0, f, 0, i64(8), None) == -2
    assert lib.ssd_gemm(0, 0, i64(4), i64(4), i64(4), 1.0, ctypes.c_void_p(FAKE + 2), i64(4), f, i64(4), 0.0, f, 0,
                        i64(4), None) == -6
    assert lib.ssd_gemm(0, 0, i64(0), i64(4), i64(4), 1.0, None, i64(4), None, i64(4), 0.0, None, 0, i64(4), None) == 0
    assert lib.ssd_cast_f32_to_bf16(i64(-1), f, f, None) == -1
    assert lib.ssd_cast_f32_to_bf16(i64(8), None, f, None) == -1
    assert lib.ssd_cast_f32_to_bf16(i64(0), None, None, None) == 0


def test_launch_grid_limit(lib):
    # 65535 batch rows of 65536 one-step chunks: one workgroup per (row, chunk,
    # head, block) would be 2^32 workgroups; rejected before any launch
    p = prob(batch=65535, seqlen=65536, chunk=1, nheads=1, headdim=1, dstate=1, ngroups=1)
    for f in (call_fwd, call_bwd):
        assert f(lib, p) == -2
        assert "launch grid" in lib.ssd_last_error().decode()
    assert lib.ssd_workspace_bytes(ctypes.byref(p), 1, 0) == 0


def _bf16_state_copy_bytes(lib, **kw):
    # the bf16 kernel family keeps a bf16 copy of the chunk states (and per-block
    # row-sum slots) in the backward workspace; the general kernels (here: bf16
    # activations with an f32 dy) do not, with everything else the same
    a = lib.ssd_workspace_bytes(ctypes.byref(prob(act_dtype=1, dy_dtype=1, **kw)), 1, 1)
    b = lib.ssd_workspace_bytes(ctypes.byref(prob(act_dtype=1, dy_dtype=0, **kw)), 1, 1)
    return a - b


def test_bf16_family_offset_bounds(lib):
    big = dict(batch=1, nheads=64, headdim=64, dstate=128, ngroups=8, chunk=256)
    states = lambda T: 4 * (T // 256) * 64 * 64 * 128
    # a 262144-step row holds 2 GiB of bf16 x: the chunk-state kernel's
    # descriptors start at each chunk, so the bf16 family still applies
    assert _bf16_state_copy_bytes(lib, seqlen=262144, **big) >= states(262144) // 2
    # 2^23 steps of 64 heads: a head's row of the [b, H, T] per-head sums
    # spans 2^31 bytes, past a descriptor's 32-bit range -> general kernels
    assert _bf16_state_copy_bytes(lib, seqlen=1 << 23, **big) == 0


@pytest.fixture
def meta_binding(monkeypatch, lib):
    # meta tensors carry shapes, dtypes and devices but no memory: every
    # binding check runs, and a check that is missing lets a null pointer
    # reach the library, which then answers SSDError (not the ValueError /
    # TypeError the binding raises)
    monkeypatch.setattr(bd, "_on_gpu", lambda t, name: None)
    b, T, H, P, N, G = 1, 256, 4, 64, 32, 2
    m = dict(device="meta")
    t = dict(x=torch.empty((b, T, H, P), **m), dt=torch.empty((b, T, H), **m), B=torch.empty((b, T, G, N), **m),
             C=torch.empty((b, T, G, N), **m), A_log=torch.empty(H, **m), D=torch.empty(H, **m))
    return t, (b, T, H, P, N, G)


import torch  # noqa: E402


@pytest.mark.parametrize("key,shape,dtype", [
    ("y", (1, 256, 4, 32), torch.float32),
    ("y", (1, 256, 4, 64), torch.bfloat16),
    ("final_state", (1, 4, 64, 16), torch.float32),
    ("chunk_states", (1, 1, 4, 64, 32), torch.bfloat16),
])
def test_binding_checks_fwd_out_buffers(meta_binding, key, shape, dtype):
    t, _ = meta_binding
    bad = {key: torch.empty(shape, dtype=dtype, device="meta")}
    with pytest.raises((ValueError, TypeError), match=key):
        bd.ssd_fwd(t["x"], t["dt"], t["A_log"], t["B"], t["C"], t["D"], chunk=256, out=bad)


@pytest.mark.parametrize("key,shape,dtype", [
    ("dx", (1, 256, 4, 32), torch.float32),
    ("dx", (1, 256, 4, 64), torch.bfloat16),
    ("ddt", (1, 256, 3), torch.float32),
    ("dA_log", (5,), torch.float32),
    ("dB", (1, 256, 2, 16), torch.float32),
    ("dC", (1, 256, 2, 32), torch.float64),
    ("dD", (4, 1), torch.float32),
    ("d_init_state", (1, 4, 64, 31), torch.float32),
])
def test_binding_checks_bwd_out_buffers(meta_binding, key, shape, dtype):
    t, _ = meta_binding
    bad = {key: torch.empty(shape, dtype=dtype, device="meta")}
    with pytest.raises((ValueError, TypeError), match=key):
        bd.ssd_bwd(t["x"], t["dt"], t["A_log"], t["B"], t["C"], t["D"], t["x"], chunk=256, out=bad)


def test_binding_checks_workspace_and_dt_outputs(meta_binding):
    t, (b, T, H, P, N, G) = meta_binding
    with pytest.raises(TypeError, match="workspace"):
        bd.ssd_fwd(t["x"], t["dt"], t["A_log"], t["B"], t["C"], t["D"], chunk=256,
                   workspace=torch.empty(100, dtype=torch.float32, device="meta"))
    raw, bias, ddt = t["dt"], t["A_log"], torch.empty((b, T, H), device="meta")
    with pytest.raises(ValueError, match="ddt_raw"):
        bd.dt_softplus_bwd(raw, bias, ddt, out=(torch.empty((b, T, H + 1), device="meta"), torch.empty(H, device="meta")))
    with pytest.raises(ValueError, match="d_dt_bias"):
        bd.dt_softplus_bwd(raw, bias, ddt, out=(torch.empty((b, T, H), device="meta"), torch.empty(H + 1, device="meta")))


def test_binding_refuses_host_tensors(lib):
    x = torch.zeros((1, 16, 2, 8))
    B = torch.zeros((1, 16, 1, 4))
    with pytest.raises(ValueError, match="GPU"):
        bd.ssd_fwd(x, torch.zeros((1, 16, 2)), torch.zeros(2), B, B, torch.zeros(2), chunk=16)
    with pytest.raises(ValueError, match="GPU"):
        bd.rmsnorm_gated_fwd(torch.zeros((4, 8)), torch.zeros((4, 8)), torch.ones(8))


def test_noalloc_scratch_size_matches_the_header():
    text = open(HEADER).read()
    m = re.search(r"#define SSD_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == bd.NOALLOC_SCRATCH_BYTES


def test_noalloc_refuses_a_problem_past_its_scratch_before_any_launch(lib):
    # the f32 grouped-sized problem in recompute mode needs more scratch than
    # the static array holds: refused before anything touches a device
    p = prob(batch=4, seqlen=2048, nheads=32, ngroups=8)
    assert lib.ssd_workspace_bytes(ctypes.byref(p), 1, 0) > bd.NOALLOC_SCRATCH_BYTES
    f = ctypes.c_void_p(FAKE)
    rc = lib.ssd_bwd_noalloc(ctypes.byref(p), f, f, f, f, f, f, None, None, f, None, f, f, f, f, f, f, None, None)
    assert rc == -4 and "static scratch" in lib.ssd_last_error().decode()
