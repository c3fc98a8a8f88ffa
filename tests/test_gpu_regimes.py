"""GPU parity of the SSD core in the method's edge regimes, against the oracle.

The workload inputs (A in [-16, -1], dt mostly 0.02-0.3) never reach these:

  a_to_zero   A_log = -60: A = -e^-60, every decay is 1 in f32, the state sums
              every input of the sequence (the inter-chunk states and their
              bf16 copies grow over all chunks);
  saturating  A_log = 14: dt A <= -100 on every step (dt >= 3e-4 here), so
              every decay underflows and only the diagonal term of each step
              survives (the factorised off-diagonal decays and the carried
              column factors run through zeros and denormals);
  c_zero      C = 0: y = D x, dx = D dy, dB = ddt = dA_log = d(h0) = 0 exactly,
              dC = sum_p dy h (the skip path of the readout);
  b_zero      B = 0 with a zero initial state: the state stays 0, y = D x,
              dC = ddt = dA_log = 0 exactly, dB and d(h0) from the adjoint;
  mixed       even heads A -> 0, odd heads saturating, in the same groups.

Each regime runs on three kernel paths: f32 (general kernels), bf16 (the bf16
family) and bf16 activations with an f32 dy (general kernels on bf16
operands), at a grouped-like shape (4 chunks of 256, 4 heads per group) and at
a ragged one (headdim 40, d_state 72, chunk 80: partial tiles and a 16-row
tail block).  Every output is compared element by element: max|gpu - ref| /
max(max|ref|, floor) within 1e-4 (f32) or 2e-2 (bf16 operands).  The floor is
1 for the outputs whose exact value is 0 or below 1e-30 in the regime (dA_log
and d(h0) under saturating decay, and the exact zeros of the skip paths), i.e.
those are held to the same bound in absolute terms.
"""
import numpy as np
import pytest

from ssd_inputs import SSDConfig, Stored, make_inputs
from tests.gpu_util import SSD_KEYS, TOL, dev, gpu_ssd, oracle_ssd, relerr

pytestmark = pytest.mark.gpu

SHAPES = {
    "grouped": dict(batch=1, seqlen=1024, nheads=16, headdim=64, dstate=128, ngroups=4, chunk=256),
    "ragged": dict(batch=2, seqlen=240, nheads=6, headdim=40, dstate=72, ngroups=3, chunk=80),
}
# (activation dtype, dy dtype)
PATHS = {"f32": ("f32", "f32"), "bf16": ("bf16", "bf16"), "bf16_dy_f32": ("bf16", "f32")}


def regime_inputs(regime: str, cfg: SSDConfig):
    d = make_inputs(cfg)
    H = cfg.nheads
    zero_floor = ()
    if regime == "a_to_zero":
        d["A_log"] = np.full(H, -60.0, np.float32)
    elif regime == "saturating":
        d["A_log"] = np.full(H, 14.0, np.float32)
        zero_floor = ("dA_log", "d_init_state")
    elif regime == "mixed":
        d["A_log"] = np.where(np.arange(H) % 2 == 0, -60.0, 14.0).astype(np.float32)
    elif regime == "c_zero":
        d["C"] = Stored(np.zeros(d["C"].shape, np.float32), cfg.dtype)
        zero_floor = ("dB", "ddt", "dA_log", "d_init_state")
    elif regime == "b_zero":
        d["B"] = Stored(np.zeros(d["B"].shape, np.float32), cfg.dtype)
        d["h0"] = None
        zero_floor = ("dC", "ddt", "dA_log", "chunk_states", "final")
    else:
        raise ValueError(regime)
    return d, zero_floor


def check(got, ref, tol, floor_keys, label):
    errs = {}
    for k in SSD_KEYS:
        if k in floor_keys:
            den = max(float(np.max(np.abs(ref[k]))), 1.0)
            errs[k] = float(np.max(np.abs(got[k] - ref[k]))) / den if np.all(np.isfinite(got[k])) else float("inf")
        else:
            errs[k] = relerr(got[k], ref[k])
    print(f"[regime {label}] " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"{label}: outside {tol:g}: {bad}"


@pytest.mark.parametrize("shape", list(SHAPES))
@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("regime", ["a_to_zero", "saturating", "mixed", "c_zero", "b_zero"])
def test_edge_regime_parity(regime, path, shape):
    act, dyt = PATHS[path]
    cfg = SSDConfig("regime", dtype=act, init_state=True, seed=31, **SHAPES[shape])
    d, floor_keys = regime_inputs(regime, cfg)
    label = f"{regime} {path} {shape}"
    print(f"[regime {label}] running", flush=True)
    dy_dev, dy_vals = None, None
    if dyt != act:
        dy_vals = np.random.default_rng(32).standard_normal(d["x"].shape).astype(np.float32)
        dy_dev = dev(dy_vals)
    got = gpu_ssd(cfg, d, dy=dy_dev)
    ref = oracle_ssd(d, cfg.chunk, dy_values=dy_vals)
    check(got, ref, TOL["bf16" if act == "bf16" else "f32"], floor_keys, label)
    if regime in ("c_zero", "b_zero"):
        # the exact zeros of the skip paths come out exactly
        for k in floor_keys:
            assert np.count_nonzero(got[k]) == 0, (label, k)
