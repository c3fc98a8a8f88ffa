"""Seeded synthetic inputs for the Mamba-2 SSD core and its block shell.

This module is shared by the oracle side (tests, CPU baseline) and the HIP side
(tests, bench). It draws random numbers and rounds them to the storage dtype; it
holds none of the method's arithmetic (no recurrence, no gradient).

Workloads (sizes follow the five synthetic SSD configurations the method is
measured on, plus the deterministic shape from the parity test on the page
burn_dragon_kernel ``src/sequence/mamba2/backward.rs``, ``make_realistic_cuda_inputs``):

  tiny        b=1  T=64    H=2  P=8  N=4   G=1 Q=16  f32
  m130        b=2  T=1024  H=24 P=64 N=128 G=1 Q=256 f32   (130M-shaped)
  grouped     b=4  T=2048  H=32 P=64 N=128 G=8 Q=256 bf16  (4 heads/group)
  long        b=1  T=16384 H=64 P=64 N=128 G=1 Q=256 f32   carried h0 ~ N(0, 0.1)
  block       b=8  T=2048  H=48 P=64 N=128 G=1 Q=256 bf16  + conv1d/SiLU and
                                                        RMSNorm-gated shell
  p1test      b=1  T=32    H=4  P=64 N=16  G=4 Q=16  f32   the page's test pattern

Distributions: x, B, C, dy ~ N(0,1); dt = softplus(N(0,1) + dt_bias_h) with
dt_bias ~ U(-4,-2) per head; A_log ~ U(log 1, log 16); D ~ N(0,1); initial
state zero except where stated.  bf16 workloads round every activation
(x, dt, B, C, dy; xBC and z for the shell) from f32 to bf16 with
round-to-nearest-even; the same rounded values feed both sides.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class SSDConfig:
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    chunk: int
    dtype: str  # "f32" or "bf16": storage dtype of x, dt, B, C, dy, y
    init_state: bool = False
    shell: bool = False  # conv1d+SiLU before and RMSNorm-gated after the core
    d_model: int = 0  # > 0: also the block's in/out projections from and to d_model
    d_conv: int = 4
    norm_eps: float = 1e-5
    seed: int = 0

    @property
    def hpg(self) -> int:
        return self.nheads // self.ngroups

    @property
    def nchunks(self) -> int:
        return self.seqlen // self.chunk

    @property
    def d_inner(self) -> int:
        return self.nheads * self.headdim

    @property
    def conv_dim(self) -> int:
        return self.d_inner + 2 * self.ngroups * self.dstate

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen

    def with_(self, **kw) -> "SSDConfig":
        return dataclasses.replace(self, **kw)


CONFIGS: Dict[str, SSDConfig] = {
    "tiny": SSDConfig("tiny", 1, 64, 2, 8, 4, 1, 16, "f32", seed=1000),
    "m130": SSDConfig("m130", 2, 1024, 24, 64, 128, 1, 256, "f32", seed=1001),
    "grouped": SSDConfig("grouped", 4, 2048, 32, 64, 128, 8, 256, "bf16", seed=1002),
    "long": SSDConfig("long", 1, 16384, 64, 64, 128, 1, 256, "f32",
                      init_state=True, seed=1003),
    "block": SSDConfig("block", 8, 2048, 48, 64, 128, 1, 256, "bf16",
                       shell=True, seed=1004),
    # the block slice's sizes with the block's projections, d_model = d_inner / 2
    "block_train": SSDConfig("block_train", 8, 2048, 48, 64, 128, 1, 256, "bf16",
                             shell=True, d_model=1536, seed=1004),
}
# The five configurations in the order the workload list gives them.
CONFIG_ORDER = ["tiny", "m130", "grouped", "long", "block"]

P1TEST = SSDConfig("p1test", 1, 32, 4, 64, 16, 4, 16, "f32", init_state=True, seed=0)


# --------------------------------------------------------------------------
# bf16 storage
# --------------------------------------------------------------------------

def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round f32 values to bf16 (round-to-nearest-even) and return the raw
    16-bit patterns as uint16. NaN is not expected in generated data."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_bf16(a: np.ndarray) -> np.ndarray:
    """f32 array holding the bf16-rounded values of ``a``."""
    return bf16_to_f32(bf16_bits(a))


class Stored:
    """An activation as it is stored on the device: ``values`` holds the f32
    values (already bf16-rounded for bf16 storage) and ``raw`` the array that is
    copied to the device (float32, or uint16 bf16 bit patterns)."""

    def __init__(self, values: np.ndarray, dtype: str):
        self.dtype = dtype
        if dtype == "bf16":
            self.raw = bf16_bits(values)
            self.values = bf16_to_f32(self.raw)
        elif dtype == "f32":
            self.values = np.ascontiguousarray(values, dtype=np.float32)
            self.raw = self.values
        else:
            raise ValueError(f"unknown dtype {dtype}")

    @property
    def shape(self):
        return self.values.shape


def _softplus(v: np.ndarray) -> np.ndarray:
    # log(1 + e^v) without overflow; used only to draw dt's distribution.
    return np.logaddexp(0.0, v).astype(np.float32)


def make_inputs(cfg: SSDConfig, seed: Optional[int] = None) -> Dict[str, object]:
    """Draw one workload.  Returns a dict of Stored activations and f32 params.

    Keys: x [b,T,H,P], dt [b,T,H], B, C [b,T,G,N], dy [b,T,H,P] (Stored);
    A_log, D [H], dt_bias [H], h0 [b,H,P,N] or None (f32 numpy); dt_raw
    [b,T,H] (Stored), the N(0,1) draw that dt is the softplus of after adding
    dt_bias.
    Shell workloads add xBC [b,T,conv_dim], z [b,T,d_inner], gout [b,T,d_inner]
    (Stored) and conv_w [conv_dim,d_conv], conv_b [conv_dim], norm_w [d_inner]
    (f32).  For shell workloads x, B, C, dy are still drawn (same order) so the
    core can also be exercised alone on this shape.
    """
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    b, T, H, P, N, G = cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.dstate, cfg.ngroups
    f32 = np.float32
    out: Dict[str, object] = {}
    x = rng.standard_normal((b, T, H, P), dtype=f32)
    Bm = rng.standard_normal((b, T, G, N), dtype=f32)
    Cm = rng.standard_normal((b, T, G, N), dtype=f32)
    dt_noise = rng.standard_normal((b, T, H), dtype=f32)
    dt_bias = rng.uniform(-4.0, -2.0, size=H).astype(f32)
    A_log = rng.uniform(np.log(1.0), np.log(16.0), size=H).astype(f32)
    D = rng.standard_normal(H, dtype=f32)
    h0 = (0.1 * rng.standard_normal((b, H, P, N), dtype=f32)).astype(f32) if cfg.init_state else None
    dy = rng.standard_normal((b, T, H, P), dtype=f32)
    dt = _softplus(dt_noise + dt_bias[None, None, :])
    out.update(
        x=Stored(x, cfg.dtype), B=Stored(Bm, cfg.dtype), C=Stored(Cm, cfg.dtype),
        dt=Stored(dt, cfg.dtype), dy=Stored(dy, cfg.dtype),
        A_log=A_log, D=D, dt_bias=dt_bias, h0=h0,
        dt_raw=Stored(dt_noise, cfg.dtype),  # the pre-activation, for the fused dt activation
    )
    if cfg.shell:
        cd, di, K = cfg.conv_dim, cfg.d_inner, cfg.d_conv
        xbc = rng.standard_normal((b, T, cd), dtype=f32)
        conv_w = (0.5 * rng.standard_normal((cd, K), dtype=f32)).astype(f32)
        conv_b = (0.1 * rng.standard_normal(cd, dtype=f32)).astype(f32)
        z = rng.standard_normal((b, T, di), dtype=f32)
        norm_w = (1.0 + 0.1 * rng.standard_normal(di, dtype=f32)).astype(f32)
        gout = rng.standard_normal((b, T, di), dtype=f32)
        out.update(xBC=Stored(xbc, cfg.dtype), z=Stored(z, cfg.dtype), gout=Stored(gout, cfg.dtype),
                   conv_w=conv_w, conv_b=conv_b, norm_w=norm_w)
    if cfg.d_model:
        # projections: u ~ N(0,1); weights [out, in] ~ N(0, 1/in), so that the
        # projected activations are about N(0,1); the gradient of the block's
        # output ~ N(0,1)
        dm, di, cd = cfg.d_model, cfg.d_inner, cfg.conv_dim
        u = rng.standard_normal((b, T, dm), dtype=f32)
        w_z, w_xbc, w_dt = ((rng.standard_normal((o, dm), dtype=f32) / np.sqrt(dm)).astype(f32) for o in (di, cd, H))
        w_out = (rng.standard_normal((dm, di), dtype=f32) / np.sqrt(di)).astype(f32)
        go = rng.standard_normal((b, T, dm), dtype=f32)
        out.update(u=Stored(u, cfg.dtype), W_z=Stored(w_z, cfg.dtype), W_xbc=Stored(w_xbc, cfg.dtype),
                   W_dt=Stored(w_dt, cfg.dtype), W_out=Stored(w_out, cfg.dtype), go=Stored(go, cfg.dtype))
    return out


def make_p1test_inputs() -> Dict[str, object]:
    """The deterministic ``(idx % prime) / prime - offset`` pattern of the
    parity test of the page (burn_dragon_kernel src/sequence/mamba2/backward.rs, tests module,
    ``make_realistic_cuda_inputs``): b=1, T=32, G=4, one head per group,
    P=64, N=16, with a nonzero initial state.  Flat index order is the
    row-major order of the page's grouped shapes, which is the same memory
    order as our [b,T,H,P] / [b,T,G,N] / [b,H,P,N] layouts."""
    cfg = P1TEST
    b, T, H, P, N, G = cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.dstate, cfg.ngroups

    def pattern(count, prime, offset):
        idx = np.arange(count, dtype=np.int64)
        return ((idx % prime).astype(np.float32) / np.float32(prime) + np.float32(offset)).astype(np.float32)

    x = pattern(b * T * H * P, 257, -0.5).reshape(b, T, H, P)
    Bm = pattern(b * T * G * N, 263, -0.5).reshape(b, T, G, N)
    Cm = pattern(b * T * G * N, 269, -0.5).reshape(b, T, G, N)
    dt = pattern(b * T * H, 271, 0.05).reshape(b, T, H)
    A_log = pattern(H, 277, -0.25)
    D = pattern(H, 281, -0.25)
    h0 = pattern(b * H * P * N, 283, -0.5).reshape(b, H, P, N)
    dy = pattern(b * T * H * P, 293, -0.5).reshape(b, T, H, P)
    return dict(x=Stored(x, "f32"), B=Stored(Bm, "f32"), C=Stored(Cm, "f32"), dt=Stored(dt, "f32"),
                dy=Stored(dy, "f32"), A_log=A_log, D=D, dt_bias=None, h0=h0)
