"""Differentiable SSD op over the C ABI.

``ssd_scan`` wraps ssd_fwd / ssd_bwd (and, with ``dt_bias``, the dt activation
dt = softplus(dt_raw + dt_bias) in front of the core) in one
``torch.autograd.Function``: the forward saves the chunk states that ssd_fwd
writes, the backward hands them to ssd_bwd together with the gradients of y
and of the final state.  Every computation runs in the library's kernels; the
function only routes tensors.  The dt gradient stays f32 between ssd_bwd and
the softplus backward inside the one function.  Gradients come back in f32
(autograd casts them to a bf16 input's dtype).
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
