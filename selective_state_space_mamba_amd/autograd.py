"""Differentiable ops over the C ABI.

``ssd_scan`` wraps ssd_fwd / ssd_bwd (and, with ``dt_bias``, the dt activation
dt = softplus(dt_raw + dt_bias) in front of the core) in one
``torch.autograd.Function``: the forward saves the chunk states that ssd_fwd
writes (in bf16 for the problems the bf16 kernels run, which read them only in
bf16: ssd_fwd_ex), the backward hands them to ssd_bwd together with the
gradients of y and of the final state.  The dt gradient stays f32 between ssd_bwd and the
softplus backward inside the one function.

``mamba2_block_core`` does the same for the block slice between the input and
output projections of a Mamba-2 block: dt activation, causal depthwise conv1d
+ SiLU split into x / B / C, the SSD, and the RMSNorm-gated output.
``mamba2_block`` adds the projections (bf16 GEMMs through the library's
rocBLAS entry point).

Every computation runs in the library's kernels; the functions only route
tensors.  Gradients come back in f32 (autograd casts them to a bf16 input's
dtype).
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import _binding as _b


def _fwd_with_history(x, dt, A_log, B, C, D, init_state, chunk):
    """ssd_fwd keeping the chunk states for the backward: (y, final_state,
    f32 states or None, bf16 states or None).  bf16 problems with headdim and
    d_state multiples of 8 keep them in bf16 (the library refuses the bf16
    history for problems its bf16 kernels do not run, e.g. past their size
    limits: those keep the f32 states)."""
    if x.dtype == torch.bfloat16 and x.shape[-1] % 8 == 0 and B.shape[-1] % 8 == 0:
        try:
            r = _b.ssd_fwd_ex(x, dt, A_log, B, C, D, init_state, chunk=chunk)
            return r["y"], r["final_state"], None, r["chunk_states_bf16"]
        except _b.SSDError as e:
            if "chunk_states_bf16" not in str(e):
                raise
    y, fin, cs = _b.ssd_fwd(x, dt, A_log, B, C, D, init_state, chunk=chunk)
    return y, fin, cs, None


def _history_args(cs, csb, dy):
    """The saved history as ssd_bwd's arguments: the bf16 one only for a bf16
    dy (an f32 dy takes the general kernels, which recompute the f32 states)."""
    return dict(chunk_states=cs, chunk_states_bf16=csb if dy.dtype == torch.bfloat16 else None)


class _SSDScan(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, dt_in, A_log, B, C, D, init_state, dt_bias, chunk):
        dt = _b.dt_softplus_fwd(dt_in, dt_bias) if dt_bias is not None else dt_in
        y, fin, cs, csb = _fwd_with_history(x, dt, A_log, B, C, D, init_state, chunk)
        ctx.save_for_backward(x, dt_in, dt, A_log, B, C, D, init_state, dt_bias, cs, csb)
        ctx.chunk = chunk
        return y, fin

    @staticmethod
    def backward(ctx, gy, gfin):
        x, dt_in, dt, A_log, B, C, D, init_state, dt_bias, cs, csb = ctx.saved_tensors
        if gy is None:
            gy = torch.zeros_like(x)
        gy = gy.contiguous()
        g = _b.ssd_bwd(x, dt, A_log, B, C, D, gy, init_state, chunk=ctx.chunk, **_history_args(cs, csb, gy),
                       want_d_init_state=init_state is not None and ctx.needs_input_grad[6],
                       d_final_state=None if gfin is None else gfin.float().contiguous())
        ddt, d_bias = g["ddt"], None
        if dt_bias is not None:
            ddt, d_bias = _b.dt_softplus_bwd(dt_in, dt_bias, ddt)
        return g["dx"], ddt, g["dA_log"], g["dB"], g["dC"], g["dD"], g["d_init_state"], d_bias, None


def ssd_scan(x: torch.Tensor, dt: torch.Tensor, A_log: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
             D: torch.Tensor, init_state: Optional[torch.Tensor] = None, chunk: int = 256,
             dt_bias: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Differentiable Mamba-2 SSD.  x [b,T,H,P], dt [b,T,H], B, C [b,T,G,N]
    (f32 or bf16, one dtype), A_log, D [H] f32, init_state [b,H,P,N] f32 or
    None.  With dt_bias [H] (f32), ``dt`` is the pre-activation and the op
    uses softplus(dt + dt_bias).  Returns (y [b,T,H,P], final_state [b,H,P,N]);
    gradients flow to every tensor argument."""
    return _SSDScan.apply(x, dt, A_log, B, C, D, init_state, dt_bias, chunk)


def _core_fwd(xbc, dt_raw, z, conv_w, conv_b, dt_bias, A_log, D, norm_w, init_state, dims):
    """Forward of the block slice; returns (out, final_state, tensors saved for _core_bwd)."""
    ngroups, dstate, headdim, chunk, eps = dims
    b, T, _ = xbc.shape
    d_inner = z.shape[-1]
    H = d_inner // headdim
    dt = _b.dt_softplus_fwd(dt_raw, dt_bias)
    xs, Bs, Cs = _b.conv1d_silu_fwd(xbc, conv_w, conv_b, d_inner, ngroups, dstate)
    xs = xs.view(b, T, H, headdim)
    y, fin, cs, csb = _fwd_with_history(xs, dt, A_log, Bs, Cs, D, init_state, chunk)
    out, inv = _b.rmsnorm_gated_fwd(y.view(b, T, d_inner), z, norm_w, eps)
    return out, fin, (dt, xs, Bs, Cs, y, inv, cs, csb)


def _core_bwd(xbc, dt_raw, z, conv_w, conv_b, dt_bias, A_log, D, norm_w, init_state, saved, dims, gout, gfin,
              want_dh0, act_grad_dtype=torch.float32, gin=None):
    """Backward of the block slice: (dxbc, ddt_raw, dz, dconv_w, dconv_b, d_dt_bias,
    dA_log, dD, dnorm_w, d_init_state), f32 but for dz, dxbc and ddt_raw, which
    the kernels write in act_grad_dtype (bf16: rounded to nearest even, the
    values a cast of the f32 gradients gives); with gin ([b*T, >= d_inner +
    conv_dim + H] in act_grad_dtype) dz, dxbc and ddt_raw go into its first
    three column blocks."""
    dt, xs, Bs, Cs, y, inv, cs, csb = saved
    ngroups, dstate, headdim, chunk, eps = dims
    b, T, d_inner = z.shape
    H = d_inner // headdim
    # the gradient handed to the SSD backward is stored in the activation
    # dtype, as the block-slice step does
    cd = xbc.shape[-1]
    gy, gz, gnw = _b.rmsnorm_gated_bwd(y.view(b, T, d_inner), z, norm_w, inv, gout, dy_dtype=xbc.dtype,
                                       dz_dtype=act_grad_dtype,
                                       dz_out=None if gin is None else gin[:, :d_inner].view(b, T, d_inner))
    gy = gy.view(b, T, H, headdim)
    g = _b.ssd_bwd(xs, dt, A_log, Bs, Cs, D, gy, init_state, **_history_args(cs, csb, gy),
                   chunk=chunk, want_d_init_state=want_dh0,
                   d_final_state=None if gfin is None else gfin.float().contiguous())
    o = d_inner + cd  # the dt_raw block's first column in gin
    dxbc, dcw, dcb = _b.conv1d_silu_bwd(xbc, conv_w, conv_b, g["dx"].view(b, T, d_inner), g["dB"], g["dC"],
                                        d_inner, ngroups, dstate, dxbc_dtype=act_grad_dtype,
                                        out=None if gin is None else gin[:, d_inner:o].view(b, T, cd))
    ddt_out = None if gin is None else (gin[:, o:o + H].view(b, T, H),
                                        torch.empty(H, dtype=torch.float32, device=xbc.device))
    ddt_raw, d_bias = _b.dt_softplus_bwd(dt_raw, dt_bias, g["ddt"], out=ddt_out, out_dtype=act_grad_dtype)
    return dxbc, ddt_raw, gz, dcw, dcb, d_bias, g["dA_log"], g["dD"], gnw, g["d_init_state"]


class _BlockCore(torch.autograd.Function):
    @staticmethod
    def forward(ctx, xbc, dt_raw, z, conv_w, conv_b, dt_bias, A_log, D, norm_w, init_state, dims):
        out, fin, saved = _core_fwd(xbc, dt_raw, z, conv_w, conv_b, dt_bias, A_log, D, norm_w, init_state, dims)
        ctx.save_for_backward(xbc, dt_raw, z, conv_w, conv_b, dt_bias, A_log, D, norm_w, init_state, *saved)
        ctx.dims = dims
        return out, fin

    @staticmethod
    def backward(ctx, gout, gfin):
        t = ctx.saved_tensors
        if gout is None:
            gout = torch.zeros_like(t[2])
        grads = _core_bwd(*t[:10], t[10:], ctx.dims, gout.contiguous(), gfin,
                          t[9] is not None and ctx.needs_input_grad[9])
        return (*grads, None)


def mamba2_block_core(xbc: torch.Tensor, dt_raw: torch.Tensor, z: torch.Tensor, conv_w: torch.Tensor,
                      conv_b: torch.Tensor, dt_bias: torch.Tensor, A_log: torch.Tensor, D: torch.Tensor,
                      norm_w: torch.Tensor, *, ngroups: int, dstate: int, headdim: int, chunk: int = 256,
                      eps: float = 1e-5, init_state: Optional[torch.Tensor] = None
                      ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Differentiable Mamba-2 block slice.  xbc [b,T,d_inner + 2*ngroups*dstate]
    (channels x, B, C), dt_raw [b,T,H] and z [b,T,d_inner] in one dtype (f32 or
    bf16); conv_w [conv_dim, d_conv], conv_b [conv_dim], dt_bias, A_log, D [H]
    and norm_w [d_inner] f32; init_state [b,H,headdim,dstate] f32 or None.
    Returns (out [b,T,d_inner] = RMSNorm(y) * norm_w * silu(z), final_state)."""
    return _BlockCore.apply(xbc, dt_raw, z, conv_w, conv_b, dt_bias, A_log, D, norm_w, init_state,
                            (ngroups, dstate, headdim, chunk, eps))


class _Block(torch.autograd.Function):
    @staticmethod
    def forward(ctx, u, W_z, W_xbc, W_dt, conv_w, conv_b, dt_bias, A_log, D, norm_w, W_out, init_state, dims):
        b, T, dm = u.shape
        u2 = u.reshape(b * T, dm)
        z = _b.gemm(u2, W_z, trans_b=True).view(b, T, -1)
        xbc = _b.gemm(u2, W_xbc, trans_b=True).view(b, T, -1)
        dt_raw = _b.gemm(u2, W_dt, trans_b=True).view(b, T, -1)
        out, fin, saved = _core_fwd(xbc, dt_raw, z, conv_w, conv_b, dt_bias, A_log, D, norm_w, init_state, dims)
        o = _b.gemm(out.view(b * T, -1), W_out, trans_b=True).view(b, T, dm)
        ctx.save_for_backward(u, W_z, W_xbc, W_dt, W_out, out, xbc, dt_raw, z, conv_w, conv_b, dt_bias, A_log, D,
                              norm_w, init_state, *saved)
        ctx.dims = dims
        return o, fin

    @staticmethod
    def backward(ctx, go, gfin):
        t = ctx.saved_tensors
        u, W_z, W_xbc, W_dt, W_out, out = t[:6]
        b, T, dm = u.shape
        u2 = u.reshape(b * T, dm)
        if go is None:
            go = torch.zeros_like(u)
        go2 = go.contiguous().view(b * T, dm)
        # the gradient of the slice's output, in the activation dtype (bf16)
        gout = _b.gemm(go2, W_out).view(b, T, -1)
        dW_out = _b.gemm(go2, out.view(b * T, -1), trans_a=True, out_dtype=torch.float32)
        init_state = t[15]
        # the gradients of z, xbc and dt_raw come out of their kernels in bf16,
        # the operand dtype of the products below (the same values as a cast of
        # the f32 gradients), side by side, so that one product against
        # [W_z; W_xbc; W_dt] gives du and one the weight gradients (rows padded
        # with zero columns to a multiple of 64, the products' k-tile; the
        # blocks start 16-byte aligned when d_inner and conv_dim are multiples
        # of 8, otherwise each gradient takes its own products)
        di, cd, H = W_z.shape[0], W_xbc.shape[0], W_dt.shape[0]
        side = di % 8 == 0 and cd % 8 == 0
        nin = di + cd + H
        ninp = -(-nin // 64) * 64
        gin = None
        if side:
            gin = torch.empty((b * T, ninp), dtype=torch.bfloat16, device=u.device)
            gin[:, nin:].zero_()
        (dxbc, ddt_raw, dz, dcw, dcb, d_bias, dA, dD, dnw, dh0) = _core_bwd(
            *t[6:16], t[16:], ctx.dims, gout, gfin, init_state is not None and ctx.needs_input_grad[11],
            act_grad_dtype=torch.bfloat16, gin=gin)
        if side:
            Win = torch.cat([W_z, W_xbc, W_dt, W_dt.new_zeros((ninp - nin, W_dt.shape[1]))], dim=0)
            du = _b.gemm(gin, Win, out_dtype=torch.float32)
            dWin = _b.gemm(gin, u2, trans_a=True, out_dtype=torch.float32)
            dWz, dWx, dWd = dWin[:di], dWin[di:di + cd], dWin[di + cd:nin]
        else:
            du = None
            dWs = []
            for gr, W in ((dz, W_z), (dxbc, W_xbc), (ddt_raw, W_dt)):
                g2 = gr.reshape(b * T, -1)
                du = _b.gemm(g2, W, out=du, out_dtype=torch.float32, beta=0.0 if du is None else 1.0)
                dWs.append(_b.gemm(g2, u2, trans_a=True, out_dtype=torch.float32))
            dWz, dWx, dWd = dWs
        return (du.view(b, T, dm), dWz, dWx, dWd, dcw, dcb, d_bias, dA, dD, dnw, dW_out, dh0, None)


def mamba2_block(u: torch.Tensor, W_z: torch.Tensor, W_xbc: torch.Tensor, W_dt: torch.Tensor,
                 conv_w: torch.Tensor, conv_b: torch.Tensor, dt_bias: torch.Tensor, A_log: torch.Tensor,
                 D: torch.Tensor, norm_w: torch.Tensor, W_out: torch.Tensor, *, ngroups: int, dstate: int,
                 headdim: int, chunk: int = 256, eps: float = 1e-5, init_state: Optional[torch.Tensor] = None
                 ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Differentiable Mamba-2 block with its projections, bf16 activations and
    weights: z, xbc, dt_raw = u W_z^T, u W_xbc^T, u W_dt^T (the three parts of
    in_proj, [out_features, d_model] each), the block slice of
    mamba2_block_core, and o = out W_out^T (W_out [d_model, d_inner]).  The
    projections run through ssd_gemm (hipBLASLt, f32 accumulation); the
    gradient entering the slice from out_proj is bf16 and the slice's
    gradients of z, xbc and dt_raw are rounded to bf16 for the backward
    products (z and xbc by the kernels that form them).  Returns
    (o [b,T,d_model], final_state)."""
    return _Block.apply(u, W_z, W_xbc, W_dt, conv_w, conv_b, dt_bias, A_log, D, norm_w, W_out, init_state,
                        (ngroups, dstate, headdim, chunk, eps))
