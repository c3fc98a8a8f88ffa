"""GPU test of ssd_bwd_noalloc, the backward entry point that allocates
nothing (its scratch is the library's static per-GPU array): through the C ABI
its outputs equal ssd_bwd's on the same inputs, on two calls in a row, the
second with a smaller problem (the array keeps the first call's contents), and
a third on another kernel family; a problem whose scratch need exceeds the
array is refused; a call changes no device memory usage.  Runs last in the
suite (collected after every other test)."""
import numpy as np
import pytest
import torch

from ssd_inputs import SSDConfig, make_inputs
from tests.gpu_util import TOL, dev, relerr

pytestmark = pytest.mark.gpu

KEYS = ("dx", "ddt", "dA_log", "dB", "dC", "dD", "d_init_state")


def _run(cfg):
    import selective_state_space_mamba_amd as ssd
    d = make_inputs(cfg)
    x, dt, B, C = dev(d["x"]), dev(d["dt"]), dev(d["B"]), dev(d["C"])
    A_log, D, dy = dev(d["A_log"]), dev(d["D"]), dev(d["dy"])
    h0 = dev(d["h0"]) if d.get("h0") is not None else None
    y, fin, cs = ssd.ssd_fwd(x, dt, A_log, B, C, D, h0, chunk=cfg.chunk)
    ref = ssd.ssd_bwd(x, dt, A_log, B, C, D, dy, h0, chunk_states=cs, chunk=cfg.chunk)
    out = {k: torch.full_like(v, float("nan")) for k, v in ref.items()}
    got = ssd.ssd_bwd_noalloc(x, dt, A_log, B, C, D, dy, out, h0, chunk_states=cs, chunk=cfg.chunk)
    torch.cuda.synchronize()
    return ref, got, (x, dt, A_log, B, C, D, dy, h0, cs)


def _same(ref, got, tol, label):
    for k in KEYS:
        a, b = ref[k].cpu().numpy(), got[k].cpu().numpy()
        e = relerr(b, a)
        print(f"[no_alloc {label}] {k} rel err {e:.2e}", flush=True)
        assert e <= tol, (label, k, e)
        assert np.array_equal(a, b), (label, k)  # same kernels, fixed-order sums: identical bits


def test_noalloc_matches_ssd_bwd_on_consecutive_calls():
    big = SSDConfig("na1", 2, 1024, 16, 64, 128, 4, 256, "bf16", init_state=True, seed=41)
    small = SSDConfig("na2", 1, 512, 8, 64, 128, 2, 128, "bf16", init_state=True, seed=42)
    f32 = SSDConfig("na3", 1, 240, 6, 40, 72, 3, 80, "f32", init_state=True, seed=43)
    for cfg in (big, small, f32):
        print(f"[no_alloc] {cfg}", flush=True)
        ref, got, _ = _run(cfg)
        _same(ref, got, TOL[cfg.dtype], cfg.name)


def test_noalloc_allocates_no_device_memory():
    import selective_state_space_mamba_amd as ssd
    cfg = SSDConfig("na4", 1, 512, 8, 64, 128, 2, 256, "bf16", seed=44)
    _, got, (x, dt, A_log, B, C, D, dy, h0, cs) = _run(cfg)  # the static array is in place from here on
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    for _ in range(3):
        ssd.ssd_bwd_noalloc(x, dt, A_log, B, C, D, dy, got, h0, chunk_states=cs, chunk=cfg.chunk)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 == free0, (free0, free1)


def test_noalloc_refuses_problems_past_its_scratch():
    import selective_state_space_mamba_amd as ssd
    # the grouped workload's shape at twice its batch, without saved chunk
    # states (recomputed into the scratch): more than the static array holds
    b, T, H, P, N, G, Q = 8, 2048, 32, 64, 128, 8, 256
    bf = dict(dtype=torch.bfloat16, device="cuda:0")
    f32 = dict(dtype=torch.float32, device="cuda:0")
    x = torch.zeros((b, T, H, P), **bf)
    dt = torch.zeros((b, T, H), **bf)
    Bm = torch.zeros((b, T, G, N), **bf)
    A_log, D = torch.zeros(H, **f32), torch.zeros(H, **f32)
    prob = ssd._binding.make_problem(x, Bm, Q, torch.bfloat16)
    assert ssd.ssd_workspace_bytes(prob, True, False) > ssd.NOALLOC_SCRATCH_BYTES
    out = dict(dx=torch.empty((b, T, H, P), **f32), ddt=torch.empty((b, T, H), **f32), dA_log=torch.empty(H, **f32),
               dB=torch.empty((b, T, G, N), **f32), dC=torch.empty((b, T, G, N), **f32), dD=torch.empty(H, **f32))
    with pytest.raises(ssd.SSDError, match="static scratch"):
        ssd.ssd_bwd_noalloc(x, dt, A_log, Bm, Bm, D, x, out, None, chunk_states=None, chunk=Q)
