"""Helpers for the GPU parity tests: move seeded inputs to the device, run the
HIP path through the binding, run the oracle on the same values, compare."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from ssd_inputs import SSDConfig, Stored

DEV = "cuda:0"

# Parity bars: max|gpu - ref| / max|ref| per output tensor.
TOL = {"f32": 1e-4, "bf16": 2e-2}


def dev(a, dtype: str | None = None) -> torch.Tensor | None:
    """A Stored activation (raw bits/values) or an f32 numpy array -> device tensor."""
    if a is None:
        return None
    if isinstance(a, Stored):
        if a.dtype == "bf16":
            return torch.from_numpy(a.raw.view(np.int16)).view(torch.bfloat16).to(DEV)
        return torch.from_numpy(np.ascontiguousarray(a.raw)).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def host(t: torch.Tensor | None) -> np.ndarray | None:
    if t is None:
        return None
    return t.detach().float().cpu().numpy().astype(np.float64)


def relerr(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if not np.all(np.isfinite(got)):
        return float("inf")
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    if den == 0.0:
        return num
    return num / den


def gpu_ssd(cfg: SSDConfig, d: dict, chunk: int | None = None, save_states: bool = True, dy=None,
            dfinal: np.ndarray | None = None):
    """Runs ssd_fwd then ssd_bwd on the device; returns host f64 arrays."""
    import selective_state_space_mamba_amd as ssd
    Q = chunk or cfg.chunk
    x, dt, B, C = dev(d["x"]), dev(d["dt"]), dev(d["B"]), dev(d["C"])
    A_log, D = dev(d["A_log"]), dev(d["D"])
    h0 = dev(d["h0"]) if d.get("h0") is not None else None
    dyd = dev(d["dy"]) if dy is None else dy
    y, fin, cs = ssd.ssd_fwd(x, dt, A_log, B, C, D, h0, chunk=Q, want_chunk_states=True)
    g = ssd.ssd_bwd(x, dt, A_log, B, C, D, dyd, h0, chunk_states=cs if save_states else None, chunk=Q,
                    d_final_state=dev(dfinal))
    torch.cuda.synchronize()
    out = {"y": host(y), "final": host(fin), "chunk_states": host(cs)}
    out.update({k: host(v) for k, v in g.items()})
    return out


def oracle_ssd(d: dict, chunk: int, dy_values=None, dfinal: np.ndarray | None = None):
    args = (d["x"].values, d["dt"].values, d["A_log"], d["B"].values, d["C"].values, d["D"])
    f = oracle.ssd_fwd(*args, d.get("h0"), chunk=chunk)
    g = oracle.ssd_bwd(*args, d["dy"].values if dy_values is None else dy_values, d.get("h0"), dfinal=dfinal)
    out = {"y": f["y"], "final": f["final"], "chunk_states": f["chunk_states"]}
    out.update(g)
    out["d_init_state"] = out.pop("dh0")
    return out


SSD_KEYS = ("y", "final", "chunk_states", "dx", "ddt", "dA_log", "dB", "dC", "dD", "d_init_state")


def compare(got: dict, ref: dict, tol: float, keys=SSD_KEYS, label: str = ""):
    errs = {k: relerr(got[k], ref[k]) for k in keys}
    bad = {k: v for k, v in errs.items() if not v <= tol}
    print(f"[parity {label}] " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    assert not bad, f"{label}: outside {tol:g}: {bad}"
    return errs
