"""GPU parity of the block-shell ops (conv1d+SiLU, RMSNorm-gated) and of the
whole block-core slice (conv -> SSD -> RMSNorm-gated, and back) against the
oracle on the same seeded inputs."""
import numpy as np
import pytest
import torch

import oracle
import selective_state_space_mamba_amd as ssd
from ssd_inputs import CONFIGS, Stored, make_inputs
from tests.gpu_util import TOL, dev, host, relerr

pytestmark = pytest.mark.gpu


def conv_case(seed, b, T, d_inner, G, N, K, dtype):
    rng = np.random.default_rng(seed)
    cd = d_inner + 2 * G * N
    xbc = Stored(rng.standard_normal((b, T, cd)).astype(np.float32), dtype)
    w = (0.5 * rng.standard_normal((cd, K))).astype(np.float32)
    bias = (0.1 * rng.standard_normal(cd)).astype(np.float32)
    gact = rng.standard_normal((b, T, cd)).astype(np.float32)
    return xbc, w, bias, gact


@pytest.mark.parametrize("b,T,d_inner,G,N,K,dtype", [
    (2, 300, 64, 1, 16, 4, "f32"),   # T not a multiple of the 128-step run
    (2, 300, 64, 2, 16, 4, "bf16"),
    (1, 2, 32, 1, 8, 4, "f32"),      # fewer steps than taps
    (3, 129, 48, 1, 8, 1, "f32"),
    (3, 129, 48, 1, 8, 3, "f32"),
    (1, 64, 40, 1, 8, 8, "f32"),
    (2, 200, 36, 1, 6, 4, "bf16"),   # channel counts not multiples of 8: the scalar kernels
    (2, 70, 20, 2, 2, 2, "f32"),
    (8, 2048, 3072, 1, 128, 4, "bf16"),  # the block-slice shape
])
def test_conv1d_silu(b, T, d_inner, G, N, K, dtype):
    xbc, w, bias, gact = conv_case(11, b, T, d_inner, G, N, K, dtype)
    xo, Bo, Co = ssd.conv1d_silu_fwd(dev(xbc), dev(w), dev(bias), d_inner, G, N)
    gx = gact[..., :d_inner]
    gB = gact[..., d_inner:d_inner + G * N].reshape(b, T, G, N)
    gC = gact[..., d_inner + G * N:].reshape(b, T, G, N)
    dxbc, dw, db = ssd.conv1d_silu_bwd(dev(xbc), dev(w), dev(bias), dev(gx), dev(gB), dev(gC), d_inner, G, N)
    torch.cuda.synchronize()
    _, act = oracle.conv_fwd(xbc.values, w, bias)
    rdx, rdw, rdb = oracle.conv_bwd(xbc.values, w, bias, gact)
    got_act = np.concatenate([host(xo), host(Bo).reshape(b, T, -1), host(Co).reshape(b, T, -1)], axis=-1)
    tol = TOL[dtype]
    errs = {"act": relerr(got_act, act), "dxbc": relerr(host(dxbc), rdx), "dw": relerr(host(dw), rdw),
            "dbias": relerr(host(db), rdb)}
    print("[parity conv]", errs, flush=True)
    assert all(v <= tol for v in errs.values()), errs


@pytest.mark.parametrize("rows,width,dtype,gdtype,dydtype", [
    ((3, 5), 64, "f32", "f32", "f32"),
    ((2, 37), 200, "bf16", "f32", "f32"),
    ((2, 37), 200, "bf16", "f32", "bf16"),
    ((1, 1), 4096, "f32", "bf16", "f32"),     # wider than the vector kernels hold: scalar kernels
    ((5, 7), 2048, "f32", "f32", "f32"),
    ((3, 33), 100, "bf16", "bf16", "bf16"),   # width not a multiple of 8: scalar kernels
    ((8, 2048), 3072, "bf16", "bf16", "f32"),  # the block-slice shape
    ((8, 2048), 3072, "bf16", "bf16", "bf16"),
])
def test_rmsnorm_gated(rows, width, dtype, gdtype, dydtype):
    rng = np.random.default_rng(12)
    y = Stored(rng.standard_normal(rows + (width,)).astype(np.float32), dtype)
    z = Stored(rng.standard_normal(rows + (width,)).astype(np.float32), dtype)
    w = (1.0 + 0.1 * rng.standard_normal(width)).astype(np.float32)
    g = Stored(rng.standard_normal(rows + (width,)).astype(np.float32), gdtype)
    out, inv = ssd.rmsnorm_gated_fwd(dev(y), dev(z), dev(w), 1e-5)
    dy, dz, dw = ssd.rmsnorm_gated_bwd(dev(y), dev(z), dev(w), inv, dev(g),
                                       dy_dtype=torch.bfloat16 if dydtype == "bf16" else torch.float32)
    torch.cuda.synchronize()
    assert dy.dtype == (torch.bfloat16 if dydtype == "bf16" else torch.float32)
    rout, rinv = oracle.rmsnorm_fwd(y.values, z.values, w, 1e-5)
    rdy, rdz, rdw = oracle.rmsnorm_bwd(y.values, z.values, w, rinv, g.values)
    tol = TOL["bf16" if "bf16" in (dtype, gdtype, dydtype) else "f32"]
    errs = {"out": relerr(host(out), rout), "inv_rms": relerr(host(inv), rinv), "dy": relerr(host(dy), rdy),
            "dz": relerr(host(dz), rdz), "dw": relerr(host(dw), rdw)}
    print("[parity rmsnorm]", errs, flush=True)
    assert all(v <= tol for v in errs.values()), errs


@pytest.mark.parametrize("b,T,d_inner,G,N,K,dtype", [
    (2, 300, 64, 2, 16, 4, "bf16"),      # vector kernel
    (2, 300, 64, 1, 16, 3, "f32"),
    (2, 200, 36, 1, 6, 4, "bf16"),       # scalar kernel
    (8, 2048, 3072, 1, 128, 4, "bf16"),  # the block-slice shape
])
def test_conv1d_silu_bwd_bf16_dxbc_is_the_cast(b, T, d_inner, G, N, K, dtype):
    """dxbc written in bf16 by the kernel equals, bit for bit, the f32 dxbc
    rounded by ssd_cast_f32_to_bf16; the other outputs do not change."""
    xbc, w, bias, gact = conv_case(13, b, T, d_inner, G, N, K, dtype)
    gx = dev(np.ascontiguousarray(gact[..., :d_inner]))
    gB = dev(np.ascontiguousarray(gact[..., d_inner:d_inner + G * N].reshape(b, T, G, N)))
    gC = dev(np.ascontiguousarray(gact[..., d_inner + G * N:].reshape(b, T, G, N)))
    args = (dev(xbc), dev(w), dev(bias), gx, gB, gC, d_inner, G, N)
    d32, dw32, db32 = ssd.conv1d_silu_bwd(*args)
    d16, dw16, db16 = ssd.conv1d_silu_bwd(*args, dxbc_dtype=torch.bfloat16)
    ref = ssd.cast_bf16(d32.reshape(-1)).view(d16.shape)
    torch.cuda.synchronize()
    assert d16.dtype == torch.bfloat16
    assert torch.equal(d16.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(dw16, dw32) and torch.equal(db16, db32)


@pytest.mark.parametrize("rows,width,dtype,gdtype", [
    ((2, 37), 200, "bf16", "f32"),      # vector kernel
    ((8, 2048), 3072, "bf16", "bf16"),  # the block-slice shape
    ((3, 33), 100, "bf16", "bf16"),     # scalar kernel
    ((1, 1), 4096, "f32", "bf16"),
])
def test_rmsnorm_gated_bwd_bf16_dz_is_the_cast(rows, width, dtype, gdtype):
    """dz written in bf16 by the kernel equals, bit for bit, the f32 dz rounded
    by ssd_cast_f32_to_bf16; dy and dw do not change."""
    rng = np.random.default_rng(14)
    y = Stored(rng.standard_normal(rows + (width,)).astype(np.float32), dtype)
    z = Stored(rng.standard_normal(rows + (width,)).astype(np.float32), dtype)
    w = (1.0 + 0.1 * rng.standard_normal(width)).astype(np.float32)
    g = Stored(rng.standard_normal(rows + (width,)).astype(np.float32), gdtype)
    _, inv = ssd.rmsnorm_gated_fwd(dev(y), dev(z), dev(w), 1e-5)
    args = (dev(y), dev(z), dev(w), inv, dev(g))
    dy32, dz32, dw32 = ssd.rmsnorm_gated_bwd(*args)
    dy16, dz16, dw16 = ssd.rmsnorm_gated_bwd(*args, dz_dtype=torch.bfloat16)
    ref = ssd.cast_bf16(dz32.reshape(-1)).view(dz16.shape)
    # the same bf16 dz written as the first column block of a wider matrix
    n = int(np.prod(rows))
    ld = -(-(width + 64) // 8) * 8  # a wider row stride must be a multiple of 8
    wide = torch.full((n, ld), float("nan"), dtype=torch.bfloat16, device=dz16.device)
    ssd.rmsnorm_gated_bwd(*args, dz_dtype=torch.bfloat16, dz_out=wide[:, :width].view(rows + (width,)))
    torch.cuda.synchronize()
    assert dz16.dtype == torch.bfloat16
    assert torch.equal(dz16.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(dy16, dy32) and torch.equal(dw16, dw32)
    assert torch.equal(wide[:, :width].reshape(dz16.shape).view(torch.int16), dz16.view(torch.int16))
    assert torch.isnan(wide[:, width:]).all()


@pytest.mark.parametrize("b,T,d_inner,G,N,K,H", [
    (2, 300, 64, 2, 16, 4, 4),           # vector conv kernel
    (2, 200, 36, 1, 6, 4, 4),            # scalar conv kernel (conv_dim 48)
    (4, 2048, 3072, 1, 128, 4, 48),      # the block training shape, four batch rows
])
def test_side_by_side_gradient_outputs(b, T, d_inner, G, N, K, H):
    """The conv backward's bf16 dxbc and the dt backward's bf16 ddt_raw written
    as the two column blocks of one [b*T, conv_dim + H] matrix equal, bit for
    bit, the same outputs written on their own, and fill every column."""
    xbc, w, bias, gact = conv_case(15, b, T, d_inner, G, N, K, "bf16")
    cd = d_inner + 2 * G * N
    gx = dev(np.ascontiguousarray(gact[..., :d_inner]))
    gB = dev(np.ascontiguousarray(gact[..., d_inner:d_inner + G * N].reshape(b, T, G, N)))
    gC = dev(np.ascontiguousarray(gact[..., d_inner + G * N:].reshape(b, T, G, N)))
    rng = np.random.default_rng(16)
    raw = dev(Stored(rng.standard_normal((b, T, H)).astype(np.float32), "bf16"))
    dtb = dev(rng.standard_normal(H).astype(np.float32))
    ddt = dev(rng.standard_normal((b, T, H)).astype(np.float32))
    cargs = (dev(xbc), dev(w), dev(bias), gx, gB, gC, d_inner, G, N)
    dx_ref, _, _ = ssd.conv1d_silu_bwd(*cargs, dxbc_dtype=torch.bfloat16)
    dd_ref, db_ref = ssd.dt_softplus_bwd(raw, dtb, ddt, out_dtype=torch.bfloat16)
    gxd = torch.full((b * T, cd + H), float("nan"), dtype=torch.bfloat16, device=dx_ref.device)
    ssd.conv1d_silu_bwd(*cargs, dxbc_dtype=torch.bfloat16, out=gxd[:, :cd].view(b, T, cd))
    _, db = ssd.dt_softplus_bwd(raw, dtb, ddt, out_dtype=torch.bfloat16,
                                out=(gxd[:, cd:].view(b, T, H), torch.empty(H, device=dx_ref.device)))
    torch.cuda.synchronize()
    assert torch.equal(gxd[:, :cd].reshape(b, T, cd).view(torch.int16), dx_ref.view(torch.int16))
    assert torch.equal(gxd[:, cd:].reshape(b, T, H).view(torch.int16), dd_ref.view(torch.int16))
    assert torch.equal(db, db_ref)
    assert not torch.isnan(gxd).any()


def test_block_slice_end_to_end():
    """dt activation and conv1d+SiLU -> SSD -> RMSNorm-gated forward and the
    backward through all of them at the block-slice size, against the oracle chain run in f64 from the
    same generated inputs.  The HIP chain stores its intermediates in bf16,
    including the gradient that the RMSNorm backward hands to the SSD backward
    (so the SSD backward runs its bf16 kernels), exactly as bench.py runs it."""
    cfg = CONFIGS["block"]
    d = make_inputs(cfg)
    b, T, H, P, N, G, Q, di = cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.dstate, cfg.ngroups, cfg.chunk, cfg.d_inner
    xbc, z, gout = dev(d["xBC"]), dev(d["z"]), dev(d["gout"])
    cw, cb, nw = dev(d["conv_w"]), dev(d["conv_b"]), dev(d["norm_w"])
    A_log, D = dev(d["A_log"]), dev(d["D"])
    raw, bias = dev(d["dt_raw"]), dev(d["dt_bias"])
    dt = ssd.dt_softplus_fwd(raw, bias)
    xs, Bs, Cs = ssd.conv1d_silu_fwd(xbc, cw, cb, di, G, N)
    y, _, cs = ssd.ssd_fwd(xs.view(b, T, H, P), dt, A_log, Bs, Cs, D, chunk=Q)
    out, inv = ssd.rmsnorm_gated_fwd(y.view(b, T, di), z, nw, cfg.norm_eps)
    gy, gz, gw = ssd.rmsnorm_gated_bwd(y.view(b, T, di), z, nw, inv, gout, dy_dtype=torch.bfloat16)
    g = ssd.ssd_bwd(xs.view(b, T, H, P), dt, A_log, Bs, Cs, D, gy.view(b, T, H, P), chunk_states=cs, chunk=Q)
    dxbc, dcw, dcb = ssd.conv1d_silu_bwd(xbc, cw, cb, g["dx"].view(b, T, di), g["dB"], g["dC"], di, G, N)
    g_raw, g_bias = ssd.dt_softplus_bwd(raw, bias, g["ddt"])
    torch.cuda.synchronize()

    _, act = oracle.conv_fwd(d["xBC"].values, d["conv_w"], d["conv_b"])
    rx = act[..., :di].reshape(b, T, H, P)
    rB = act[..., di:di + G * N].reshape(b, T, G, N)
    rC = act[..., di + G * N:].reshape(b, T, G, N)
    r_dt = oracle.dt_softplus_fwd(d["dt_raw"].values, d["dt_bias"])
    sargs = (rx, r_dt, d["A_log"], rB, rC, d["D"])
    ry = oracle.ssd_fwd(*sargs)["y"].reshape(b, T, di)
    rout, rinv = oracle.rmsnorm_fwd(ry, d["z"].values, d["norm_w"], cfg.norm_eps)
    rgy, rgz, rgw = oracle.rmsnorm_bwd(ry, d["z"].values, d["norm_w"], rinv, d["gout"].values)
    rg = oracle.ssd_bwd(*sargs, rgy.reshape(b, T, H, P))
    gact = np.concatenate([rg["dx"].reshape(b, T, di), rg["dB"].reshape(b, T, -1), rg["dC"].reshape(b, T, -1)], -1)
    rdxbc, rdcw, rdcb = oracle.conv_bwd(d["xBC"].values, d["conv_w"], d["conv_b"], gact)
    r_raw, r_bias = oracle.dt_softplus_bwd(d["dt_raw"].values, d["dt_bias"], rg["ddt"])
    errs = {"out": relerr(host(out), rout), "dz": relerr(host(gz), rgz), "dnorm_w": relerr(host(gw), rgw),
            "ddt": relerr(host(g["ddt"]), rg["ddt"]), "dA_log": relerr(host(g["dA_log"]), rg["dA_log"]),
            "dD": relerr(host(g["dD"]), rg["dD"]), "dxbc": relerr(host(dxbc), rdxbc),
            "dconv_w": relerr(host(dcw), rdcw), "dconv_b": relerr(host(dcb), rdcb),
            "ddt_raw": relerr(host(g_raw), r_raw), "d_dt_bias": relerr(host(g_bias), r_bias)}
    print("[parity block chain]", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    assert all(v <= TOL["bf16"] for v in errs.values()), errs


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_autograd_block_core(dtype):
    """mamba2_block_core's autograd gradients of sum(gout * out) + <dfinal,
    final> with a carried initial state, against the oracle chain."""
    from ssd_inputs import SSDConfig
    cfg = SSDConfig("blk_ag", 2, 256, 4, 64, 64, 1, 128, dtype, init_state=True, shell=True, seed=91)
    d = make_inputs(cfg)
    b, T, H, P, N, G, Q, di = cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.dstate, cfg.ngroups, cfg.chunk, cfg.d_inner
    dfin = np.random.default_rng(92).standard_normal((b, H, P, N)).astype(np.float32)
    xbc, raw, z = (dev(d[k]).requires_grad_() for k in ("xBC", "dt_raw", "z"))
    cw, cb, bias, A_log, D, nw = (dev(d[k]).requires_grad_() for k in ("conv_w", "conv_b", "dt_bias", "A_log", "D", "norm_w"))
    h0 = dev(d["h0"]).requires_grad_()
    out, fin = ssd.mamba2_block_core(xbc, raw, z, cw, cb, bias, A_log, D, nw, ngroups=G, dstate=N, headdim=P,
                                     chunk=Q, eps=cfg.norm_eps, init_state=h0)
    loss = (out.float() * dev(d["gout"]).float()).sum() + (fin * dev(dfin)).sum()
    loss.backward()
    torch.cuda.synchronize()

    _, act = oracle.conv_fwd(d["xBC"].values, d["conv_w"], d["conv_b"])
    rx = act[..., :di].reshape(b, T, H, P)
    rB = act[..., di:di + G * N].reshape(b, T, G, N)
    rC = act[..., di + G * N:].reshape(b, T, G, N)
    r_dt = oracle.dt_softplus_fwd(d["dt_raw"].values, d["dt_bias"])
    sargs = (rx, r_dt, d["A_log"], rB, rC, d["D"])
    rf = oracle.ssd_fwd(*sargs, d["h0"])
    ry = rf["y"].reshape(b, T, di)
    rout, rinv = oracle.rmsnorm_fwd(ry, d["z"].values, d["norm_w"], cfg.norm_eps)
    rgy, rgz, rgw = oracle.rmsnorm_bwd(ry, d["z"].values, d["norm_w"], rinv, d["gout"].values)
    rg = oracle.ssd_bwd(*sargs, rgy.reshape(b, T, H, P), d["h0"], dfinal=dfin)
    gact = np.concatenate([rg["dx"].reshape(b, T, di), rg["dB"].reshape(b, T, -1), rg["dC"].reshape(b, T, -1)], -1)
    rdxbc, rdcw, rdcb = oracle.conv_bwd(d["xBC"].values, d["conv_w"], d["conv_b"], gact)
    r_raw, r_bias = oracle.dt_softplus_bwd(d["dt_raw"].values, d["dt_bias"], rg["ddt"])
    errs = {"out": relerr(host(out), rout), "final": relerr(host(fin), rf["final"]),
            "dxbc": relerr(host(xbc.grad), rdxbc), "ddt_raw": relerr(host(raw.grad), r_raw),
            "dz": relerr(host(z.grad), rgz), "dconv_w": relerr(host(cw.grad), rdcw),
            "dconv_b": relerr(host(cb.grad), rdcb), "d_dt_bias": relerr(host(bias.grad), r_bias),
            "dA_log": relerr(host(A_log.grad), rg["dA_log"]), "dD": relerr(host(D.grad), rg["dD"]),
            "dnorm_w": relerr(host(nw.grad), rgw), "dh0": relerr(host(h0.grad), rg["dh0"])}
    print("[parity block core autograd]", dtype, {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    assert all(v <= TOL[dtype] for v in errs.values()), errs


def _full_block_problem(size):
    """Inputs of one mamba2_block call: the small shape (2 x 256 steps, 4
    heads, d_model 128, carried initial state and a final-state gradient), or
    the block training workload's shape at one batch row (2048 steps, 48 heads
    of 64, d_state 128, d_model 1536, no initial state), with its weights and
    output gradient drawn as the benchmark draws them."""
    from ssd_inputs import CONFIGS, SSDConfig
    if size in ("small", "odd"):
        # odd: three heads and d_state 66, so conv_dim (324) is not a multiple
        # of 8 and the gradients of xbc and dt_raw take a product each instead
        # of one together (and the SSD takes its general kernels)
        nh, ns = (3, 66) if size == "odd" else (4, 64)
        cfg = SSDConfig("blk_full", 2, 256, nh, 64, ns, 1, 128, "bf16", init_state=True, shell=True, seed=93)
        d = make_inputs(cfg)
        b, T, H, P, N = cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.dstate
        di, cd, dm = cfg.d_inner, cfg.conv_dim, 128
        rng = np.random.default_rng(94)
        u = Stored(rng.standard_normal((b, T, dm)).astype(np.float32), "bf16")
        Wz, Wx, Wd = (Stored((rng.standard_normal((o, dm)) / np.sqrt(dm)).astype(np.float32), "bf16")
                      for o in (di, cd, H))
        Wo = Stored((rng.standard_normal((dm, di)) / np.sqrt(di)).astype(np.float32), "bf16")
        go = Stored(rng.standard_normal((b, T, dm)).astype(np.float32), "bf16")
        dfin = rng.standard_normal((b, H, P, N)).astype(np.float32)
        return cfg, d, dm, (u, Wz, Wx, Wd, Wo, go), d["h0"], dfin
    cfg = CONFIGS["block_train"].with_(batch=1)
    d = make_inputs(cfg)
    return cfg, d, cfg.d_model, tuple(d[k] for k in ("u", "W_z", "W_xbc", "W_dt", "W_out", "go")), None, None


@pytest.mark.parametrize("size", ["small", "odd", "bench"])
def test_autograd_full_block_with_projections(size):
    """mamba2_block (in_proj parts, block slice, out_proj; bf16) against the
    oracle chain with the projections as f64 matrix products; `bench` is the
    block training workload's shape (d_model 1536, 48 heads) at one batch row."""
    cfg, d, dm, (u, Wz, Wx, Wd, Wo, go), h0_np, dfin = _full_block_problem(size)
    b, T, H, P, N, G, Q, di = cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.dstate, cfg.ngroups, cfg.chunk, cfg.d_inner
    print(f"[parity full block {size}] b={b} T={T} H={H} d_model={dm}", flush=True)

    tu, tWz, tWx, tWd, tWo = (dev(a).requires_grad_() for a in (u, Wz, Wx, Wd, Wo))
    cw, cb, bias, A_log, D, nw = (dev(d[k]).requires_grad_() for k in ("conv_w", "conv_b", "dt_bias", "A_log", "D", "norm_w"))
    h0 = dev(h0_np).requires_grad_() if h0_np is not None else None
    o, fin = ssd.mamba2_block(tu, tWz, tWx, tWd, cw, cb, bias, A_log, D, nw, tWo, ngroups=G, dstate=N, headdim=P,
                              chunk=Q, eps=cfg.norm_eps, init_state=h0)
    loss = (o.float() * dev(go).float()).sum()
    if dfin is not None:
        loss = loss + (fin * dev(dfin)).sum()
    loss.backward()
    torch.cuda.synchronize()

    U, WZ, WX, WD, WO, GO = (a.values.astype(np.float64) for a in (u, Wz, Wx, Wd, Wo, go))
    z, xbc, raw = U @ WZ.T, U @ WX.T, U @ WD.T
    _, act = oracle.conv_fwd(xbc, d["conv_w"], d["conv_b"])
    rx = act[..., :di].reshape(b, T, H, P)
    rB = act[..., di:di + G * N].reshape(b, T, G, N)
    rC = act[..., di + G * N:].reshape(b, T, G, N)
    r_dt = oracle.dt_softplus_fwd(raw, d["dt_bias"])
    sargs = (rx, r_dt, d["A_log"], rB, rC, d["D"])
    rf = oracle.ssd_fwd(*sargs, h0_np)
    ry = rf["y"].reshape(b, T, di)
    rout, rinv = oracle.rmsnorm_fwd(ry, z, d["norm_w"], cfg.norm_eps)
    ro = rout @ WO.T
    gout = GO @ WO
    r_dWo = GO.reshape(-1, dm).T @ rout.reshape(-1, di)
    rgy, rgz, rgw = oracle.rmsnorm_bwd(ry, z, d["norm_w"], rinv, gout)
    rg = oracle.ssd_bwd(*sargs, rgy.reshape(b, T, H, P), h0_np, dfinal=dfin)
    gact = np.concatenate([rg["dx"].reshape(b, T, di), rg["dB"].reshape(b, T, -1), rg["dC"].reshape(b, T, -1)], -1)
    rdxbc, rdcw, rdcb = oracle.conv_bwd(xbc, d["conv_w"], d["conv_b"], gact)
    r_raw, r_bias = oracle.dt_softplus_bwd(raw, d["dt_bias"], rg["ddt"])
    r_du = rgz @ WZ + rdxbc @ WX + r_raw @ WD
    flat = lambda a: a.reshape(-1, a.shape[-1])
    errs = {"o": relerr(host(o), ro), "final": relerr(host(fin), rf["final"]), "du": relerr(host(tu.grad), r_du),
            "dW_z": relerr(host(tWz.grad), flat(rgz).T @ flat(U)),
            "dW_xbc": relerr(host(tWx.grad), flat(rdxbc).T @ flat(U)),
            "dW_dt": relerr(host(tWd.grad), flat(r_raw).T @ flat(U)), "dW_out": relerr(host(tWo.grad), r_dWo),
            "dconv_w": relerr(host(cw.grad), rdcw), "dconv_b": relerr(host(cb.grad), rdcb),
            "d_dt_bias": relerr(host(bias.grad), r_bias), "dA_log": relerr(host(A_log.grad), rg["dA_log"]),
            "dD": relerr(host(D.grad), rg["dD"]), "dnorm_w": relerr(host(nw.grad), rgw)}
    if h0 is not None:
        errs["dh0"] = relerr(host(h0.grad), rg["dh0"])
    print(f"[parity full block {size}]", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    assert all(v <= TOL["bf16"] for v in errs.values()), errs


@pytest.mark.parametrize("ta,tb", [(False, False), (False, True), (True, False), (True, True)])
@pytest.mark.parametrize("m,n,k", [(1, 1, 1), (37, 45, 13), (128, 96, 257)])
def test_gemm_entry_point(ta, tb, m, n, k):
    """ssd_gemm against a float64 product of the same bf16 operands: both
    transposes, odd sizes, f32 and bf16 results, beta accumulation."""
    rng = np.random.default_rng(m * 1000 + n * 10 + k)
    a = Stored(rng.standard_normal((k, m) if ta else (m, k)).astype(np.float32), "bf16")
    b = Stored(rng.standard_normal((n, k) if tb else (k, n)).astype(np.float32), "bf16")
    c0 = rng.standard_normal((m, n)).astype(np.float32)
    A = a.values.astype(np.float64).T if ta else a.values.astype(np.float64)
    B = b.values.astype(np.float64).T if tb else b.values.astype(np.float64)
    ref = A @ B
    got32 = ssd.gemm(dev(a), dev(b), trans_a=ta, trans_b=tb, out_dtype=torch.float32)
    acc = dev(c0)
    ssd.gemm(dev(a), dev(b), trans_a=ta, trans_b=tb, out=acc, alpha=0.5, beta=1.0)
    got16 = ssd.gemm(dev(a), dev(b), trans_a=ta, trans_b=tb)
    torch.cuda.synchronize()
    assert got16.dtype == torch.bfloat16
    assert relerr(host(got32), ref) <= 1e-5
    assert relerr(host(acc), 0.5 * ref + c0) <= 1e-5
    assert relerr(host(got16), ref) <= TOL["bf16"]


@pytest.mark.parametrize("n", [1, 3, 4, 1027])
def test_cast_bf16_entry_point(n):
    src = np.random.default_rng(n).standard_normal(n).astype(np.float32) * 100
    got = ssd.cast_bf16(dev(src))
    torch.cuda.synchronize()
    expect = Stored(src, "bf16").raw  # round to nearest even
    assert np.array_equal(got.cpu().view(torch.int16).numpy().view(np.uint16), expect)
