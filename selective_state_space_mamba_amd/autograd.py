"""Differentiable ops over the C ABI.

``ssd_scan`` wraps ssd_fwd / ssd_bwd (and, with ``dt_bias``, the dt activation
dt = softplus(dt_raw + dt_bias) in front of the core) in one
``torch.autograd.Function``: the forward saves the chunk states that ssd_fwd
writes, the backward hands them to ssd_bwd together with the gradients of y
and of the final state.  The dt gradient stays f32 between ssd_bwd and the
softplus backward inside the one function.

``mamba2_block_core`` does the same for the block slice between the input and
output projections of a Mamba-2 block: dt activation, causal depthwise conv1d
+ SiLU split into x / B / C, the SSD, and the RMSNorm-gated output.

Every computation runs in the library's kernels; the functions only route
tensors.  Gradients come back in f32 (autograd casts them to a bf16 input's
dtype).
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import _binding as _b


class _SSDScan(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, dt_in, A_log, B, C, D, init_state, dt_bias, chunk):
        dt = _b.dt_softplus_fwd(dt_in, dt_bias) if dt_bias is not None else dt_in
        y, fin, cs = _b.ssd_fwd(x, dt, A_log, B, C, D, init_state, chunk=chunk)
        ctx.save_for_backward(x, dt_in, dt, A_log, B, C, D, init_state, dt_bias, cs)
        ctx.chunk = chunk
        return y, fin

    @staticmethod
    def backward(ctx, gy, gfin):
        x, dt_in, dt, A_log, B, C, D, init_state, dt_bias, cs = ctx.saved_tensors
        if gy is None:
            gy = torch.zeros_like(x)
        g = _b.ssd_bwd(x, dt, A_log, B, C, D, gy.contiguous(), init_state, chunk_states=cs, chunk=ctx.chunk,
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


class _BlockCore(torch.autograd.Function):
    @staticmethod
    def forward(ctx, xbc, dt_raw, z, conv_w, conv_b, dt_bias, A_log, D, norm_w, init_state, dims):
        ngroups, dstate, headdim, chunk, eps = dims
        b, T, _ = xbc.shape
        d_inner = z.shape[-1]
        H = d_inner // headdim
        dt = _b.dt_softplus_fwd(dt_raw, dt_bias)
        xs, Bs, Cs = _b.conv1d_silu_fwd(xbc, conv_w, conv_b, d_inner, ngroups, dstate)
        xs = xs.view(b, T, H, headdim)
        y, fin, cs = _b.ssd_fwd(xs, dt, A_log, Bs, Cs, D, init_state, chunk=chunk)
        out, inv = _b.rmsnorm_gated_fwd(y.view(b, T, d_inner), z, norm_w, eps)
        ctx.save_for_backward(xbc, dt_raw, z, conv_w, conv_b, dt_bias, A_log, D, norm_w, init_state,
                              dt, xs, Bs, Cs, y, inv, cs)
        ctx.dims = dims
        return out, fin

    @staticmethod
    def backward(ctx, gout, gfin):
        (xbc, dt_raw, z, conv_w, conv_b, dt_bias, A_log, D, norm_w, init_state,
         dt, xs, Bs, Cs, y, inv, cs) = ctx.saved_tensors
        ngroups, dstate, headdim, chunk, eps = ctx.dims
        b, T, d_inner = z.shape
        H = d_inner // headdim
        if gout is None:
            gout = torch.zeros_like(z)
        # the gradient handed to the SSD backward is stored in the activation
        # dtype, as the block-slice step does
        gy, gz, gnw = _b.rmsnorm_gated_bwd(y.view(b, T, d_inner), z, norm_w, inv, gout.contiguous(),
                                           dy_dtype=xbc.dtype)
        g = _b.ssd_bwd(xs, dt, A_log, Bs, Cs, D, gy.view(b, T, H, headdim), init_state, chunk_states=cs,
                       chunk=chunk, want_d_init_state=init_state is not None and ctx.needs_input_grad[9],
                       d_final_state=None if gfin is None else gfin.float().contiguous())
        dxbc, dcw, dcb = _b.conv1d_silu_bwd(xbc, conv_w, conv_b, g["dx"].view(b, T, d_inner), g["dB"], g["dC"],
                                            d_inner, ngroups, dstate)
        ddt_raw, d_bias = _b.dt_softplus_bwd(dt_raw, dt_bias, g["ddt"])
        return (dxbc, ddt_raw, gz, dcw, dcb, d_bias, g["dA_log"], g["dD"], gnw, g["d_init_state"], None)


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
