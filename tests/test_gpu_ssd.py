"""GPU parity of the SSD core (HIP path through the C ABI) against the oracle.

Every output tensor (y, final state, chunk states, dx, ddt, dA_log, dB, dC,
dD, d_init_state) is compared element by element with the f64 oracle on the
same seeded inputs: max|gpu - oracle| / max|oracle| <= 1e-4 for f32 runs and
<= 2e-2 for bf16-input runs.  The workload configurations run at their full
sizes (the largest is the bench's own launch shape); smaller cases cover
ragged tiles, chunk-size edge cases, both history modes, determinism and
empty problems.
"""
import numpy as np
import pytest
import torch

from ssd_inputs import CONFIGS, P1TEST, SSDConfig, make_inputs, make_p1test_inputs
from tests.gpu_util import TOL, compare, dev, gpu_ssd, host, oracle_ssd

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny", "m130", "grouped", "long", "block"])
def test_workload_parity_full_size(name):
    cfg = CONFIGS[name]
    d = make_inputs(cfg)
    got = gpu_ssd(cfg, d)
    ref = oracle_ssd(d, cfg.chunk)
    compare(got, ref, TOL[cfg.dtype], label=name)


@pytest.mark.parametrize("chunk", [16, 32])
@pytest.mark.parametrize("saved", [True, False])
def test_page_test_pattern(chunk, saved):
    # The deterministic inputs of the page's parity tests (b=1, T=32, G=4, one
    # head per group, P=64, N=16, nonzero initial state), with and without the
    # saved history.  Both our relative bar and the page's absolute 5e-4 hold.
    d = make_p1test_inputs()
    got = gpu_ssd(P1TEST, d, chunk=chunk, save_states=saved)
    ref = oracle_ssd(d, chunk)
    compare(got, ref, TOL["f32"], label=f"p1test Q={chunk} saved={saved}")
    for k in ("dx", "dB", "dC", "ddt", "dA_log", "dD"):
        assert np.max(np.abs(got[k] - ref[k])) <= 5e-4, k


RAGGED = SSDConfig("ragged", 2, 240, 6, 40, 72, 3, 80, "f32", init_state=True, seed=77)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ragged_tiles(dtype):
    # chunk 80 = one full 64-row block + a 16-row tail; headdim 40 and d_state
    # 72 leave partial 16-wide tiles; 3 groups of 2 heads; carried state.
    cfg = RAGGED.with_(dtype=dtype)
    d = make_inputs(cfg)
    compare(gpu_ssd(cfg, d), oracle_ssd(d, cfg.chunk), TOL[dtype], label=f"ragged {dtype}")


@pytest.mark.parametrize("chunk", [1, 7, 48, 64, 128, 256])
def test_chunk_lengths(chunk):
    seqlen = {1: 64, 7: 1792, 48: 480}.get(chunk, 512)
    cfg = SSDConfig("chunks", 1, seqlen, 4, 64, 128, 2, chunk, "f32", init_state=True, seed=5)
    d = make_inputs(cfg)
    compare(gpu_ssd(cfg, d), oracle_ssd(d, chunk), TOL["f32"], label=f"chunk={chunk}")


@pytest.mark.parametrize("chunk", [32, 64, 128, 192, 200])
def test_chunk_lengths_bf16(chunk):
    # the bf16 kernels at chunk lengths other than the workloads' 256: a half
    # block at 32, one, two and three 64-row blocks per chunk, and four with an
    # 8-row tail at 200 (the fused backward's W area with one, three and six
    # block pairs)
    seqlen = {192: 576, 200: 600}.get(chunk, 512)
    cfg = SSDConfig("chunks_bf16", 2, seqlen, 8, 64, 128, 2, chunk, "bf16", init_state=True, seed=15)
    d = make_inputs(cfg)
    compare(gpu_ssd(cfg, d), oracle_ssd(d, chunk), TOL["bf16"], label=f"bf16 chunk={chunk}")


def test_f32_three_heads_per_group():
    # the f32 two-pass state form and the general kernels with an odd number of
    # heads per group (3 groups of 3) and 40-wide headdim
    cfg = SSDConfig("f32_hpg3", 2, 768, 9, 40, 64, 3, 256, "f32", init_state=True, seed=16)
    d = make_inputs(cfg)
    compare(gpu_ssd(cfg, d), oracle_ssd(d, cfg.chunk), TOL["f32"], label="f32 hpg=3 P=40")


@pytest.mark.parametrize("dy_dtype", ["f32", "f32dy_bf16act"])
def test_paired_general_blocks(dy_dtype):
    # the general forward output, column and row kernels with paired blocks
    # (a workgroup takes blocks k and nb - 1 - k): 64 chunks of 200 steps (three
    # full 64-row blocks and an 8-row tail) give 2 * 32 * 2 = 128 block pairs,
    # so two head splits of three heads fill 256 workgroups; ragged headdim and
    # d_state; carried state.  With bf16 activations and f32 dy the backward
    # takes the same general kernels.
    act = "f32" if dy_dtype == "f32" else "bf16"
    cfg = SSDConfig("paired", 2, 6400, 6, 40, 72, 1, 200, act, init_state=True, seed=51)
    d = make_inputs(cfg)
    if act == "f32":
        got, ref = gpu_ssd(cfg, d), oracle_ssd(d, cfg.chunk)
    else:
        dy = np.random.default_rng(52).standard_normal(d["x"].shape).astype(np.float32)
        got, ref = gpu_ssd(cfg, d, dy=dev(dy)), oracle_ssd(d, cfg.chunk, dy_values=dy)
    compare(got, ref, TOL[act], label=f"paired general {dy_dtype}")


def test_many_chunks_bf16():
    # 256 chunks per head with 16-step chunks and a 32-wide d_state: the final
    # workgroup of the fused backward kernel sums 512 chunk partials per head
    # (every other test has at most 64)
    cfg = SSDConfig("many", 2, 2048, 4, 64, 32, 2, 16, "bf16", init_state=True, seed=12)
    d = make_inputs(cfg)
    compare(gpu_ssd(cfg, d), oracle_ssd(d, cfg.chunk), TOL["bf16"], label="256 chunks per head, bf16")


def test_many_heads_bf16():
    # 520 heads in 40 groups of 13, two batch rows of four chunks: the fused
    # backward kernel takes all 13 heads of a group per workgroup (its ddt
    # epilogue in two rounds of eight heads), and the last workgroup's dA_log
    # and dD sums run over more heads than its 512 threads (two rounds)
    cfg = SSDConfig("many_heads", 2, 1024, 520, 8, 8, 40, 256, "bf16", init_state=True, seed=41)
    d = make_inputs(cfg)
    got = gpu_ssd(cfg, d)
    ref = oracle_ssd(d, cfg.chunk)
    compare(got, ref, TOL["bf16"], label="many heads")


@pytest.mark.parametrize("dtype,saved", [("f32", True), ("bf16", False), ("bf16", True)])
def test_final_state_gradient(dtype, saved):
    # With d_final_state the reverse state pass starts from it (consecutive
    # segments of one sequence chain their backward passes this way); every
    # gradient changes through Gamma of the last chunk.
    cfg = SSDConfig("dfinal", 2, 512, 8, 64, 128, 2, 128, dtype, init_state=True, seed=21)
    d = make_inputs(cfg)
    dfin = (0.5 * np.random.default_rng(22).standard_normal((2, 8, 64, 128))).astype(np.float32)
    compare(gpu_ssd(cfg, d, save_states=saved, dfinal=dfin), oracle_ssd(d, cfg.chunk, dfinal=dfin), TOL[dtype],
            label=f"d_final_state {dtype} saved={saved}")


def test_single_chunk_whole_sequence():
    cfg = SSDConfig("one", 3, 256, 8, 64, 128, 8, 256, "bf16", init_state=True, seed=6)
    d = make_inputs(cfg)
    compare(gpu_ssd(cfg, d), oracle_ssd(d, 256), TOL["bf16"], label="T=Q bf16")


def test_f32_dy_with_bf16_activations():
    # The block slice feeds the core an f32 dy (from the RMSNorm-gated backward)
    # with bf16 activations.
    cfg = SSDConfig("mixed", 2, 512, 8, 64, 128, 1, 128, "bf16", seed=8)
    d = make_inputs(cfg)
    rng = np.random.default_rng(9)
    dy = rng.standard_normal(d["x"].shape).astype(np.float32)
    got = gpu_ssd(cfg, d, dy=dev(dy))
    ref = oracle_ssd(d, cfg.chunk, dy_values=dy)
    compare(got, ref, TOL["bf16"], label="dy f32 / act bf16")


def test_recompute_matches_saved_history_bitwise():
    cfg = SSDConfig("modes", 2, 1024, 8, 64, 128, 2, 256, "bf16", init_state=True, seed=10)
    d = make_inputs(cfg)
    a = gpu_ssd(cfg, d, save_states=True)
    b = gpu_ssd(cfg, d, save_states=False)
    for k in ("dx", "ddt", "dA_log", "dB", "dC", "dD", "d_init_state"):
        assert np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("cfg", [
    SSDConfig("hist", 2, 1024, 8, 64, 128, 2, 256, "bf16", init_state=True, seed=21),
    SSDConfig("hist_ragged", 2, 240, 6, 40, 72, 3, 80, "bf16", init_state=True, seed=22),
    # 320 chunk-state workgroups, more than the CUs: the 64-step-slab kernels
    SSDConfig("hist_rounds", 2, 1024, 80, 64, 128, 4, 256, "bf16", init_state=True, seed=23),
], ids=["full_tiles", "ragged", "several_rounds"])
def test_bf16_history(cfg):
    # ssd_fwd_ex writes the bf16 copy of the chunk states (the round to
    # nearest even of the f32 ones) and the same y as ssd_fwd; ssd_bwd_ex with
    # only that copy gives the gradients of the f32 history and of the
    # recompute mode bit for bit (the backward reads the states only in
    # bf16), within the bf16 bar of the oracle
    import selective_state_space_mamba_amd as ssd
    d = make_inputs(cfg)
    x, dt, B, C = dev(d["x"]), dev(d["dt"]), dev(d["B"]), dev(d["C"])
    A_log, D, h0, dy = dev(d["A_log"]), dev(d["D"]), dev(d["h0"]), dev(d["dy"])
    Q = cfg.chunk
    y0, fin0, cs0 = ssd.ssd_fwd(x, dt, A_log, B, C, D, h0, chunk=Q)
    r = ssd.ssd_fwd_ex(x, dt, A_log, B, C, D, h0, chunk=Q, want_chunk_states=True, want_chunk_states_bf16=True)
    r1 = ssd.ssd_fwd_ex(x, dt, A_log, B, C, D, h0, chunk=Q)  # the bf16 history alone
    torch.cuda.synchronize()
    assert torch.equal(r["y"], y0) and torch.equal(r["final_state"], fin0) and torch.equal(r["chunk_states"], cs0)
    assert r1["chunk_states"] is None and torch.equal(r1["y"], y0) and torch.equal(r1["final_state"], fin0)
    assert torch.equal(r["chunk_states_bf16"], cs0.to(torch.bfloat16))
    assert torch.equal(r1["chunk_states_bf16"], r["chunk_states_bf16"])
    g_bf = ssd.ssd_bwd(x, dt, A_log, B, C, D, dy, h0, chunk_states_bf16=r1["chunk_states_bf16"], chunk=Q)
    g_f32 = ssd.ssd_bwd(x, dt, A_log, B, C, D, dy, h0, chunk_states=cs0, chunk=Q)
    g_re = ssd.ssd_bwd(x, dt, A_log, B, C, D, dy, h0, chunk=Q)
    torch.cuda.synchronize()
    for k in ("dx", "ddt", "dA_log", "dB", "dC", "dD", "d_init_state"):
        assert torch.equal(g_bf[k], g_f32[k]), k
        assert torch.equal(g_bf[k], g_re[k]), k
    got = {"y": host(r1["y"]), "final": host(r1["final_state"]), "chunk_states": host(r["chunk_states"])}
    got.update({k: host(v) for k, v in g_bf.items()})
    compare(got, oracle_ssd(d, Q), TOL["bf16"], label=f"bf16 history {cfg.name}")


def test_deterministic_bitwise():
    cfg = CONFIGS["grouped"].with_(batch=1, seqlen=1024)
    d = make_inputs(cfg)
    a = gpu_ssd(cfg, d)
    b = gpu_ssd(cfg, d)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_empty_problems():
    import selective_state_space_mamba_amd as ssd
    for b, T in ((0, 256), (2, 0)):
        x = torch.zeros((b, T, 4, 8), device="cuda:0")
        dt = torch.zeros((b, T, 4), device="cuda:0")
        B = torch.zeros((b, T, 2, 16), device="cuda:0")
        A_log = torch.zeros(4, device="cuda:0")
        D = torch.ones(4, device="cuda:0")
        h0 = torch.randn((b, 4, 8, 16), device="cuda:0")
        y, fin, cs = ssd.ssd_fwd(x, dt, A_log, B, B, D, h0, chunk=16)
        g = ssd.ssd_bwd(x, dt, A_log, B, B, D, x, h0, chunk_states=cs, chunk=16)
        torch.cuda.synchronize()
        assert y.shape == x.shape and torch.equal(fin, h0)
        assert torch.count_nonzero(g["dA_log"]) == 0 and torch.count_nonzero(g["dD"]) == 0
        assert torch.count_nonzero(g["d_init_state"]) == 0
        # no steps: the final state is the initial one, so is its gradient
        dfin = torch.randn((b, 4, 8, 16), device="cuda:0")
        g = ssd.ssd_bwd(x, dt, A_log, B, B, D, x, h0, chunk_states=cs, chunk=16, d_final_state=dfin)
        torch.cuda.synchronize()
        assert torch.equal(g["d_init_state"], dfin)


def test_errors_are_raised_not_hidden():
    import selective_state_space_mamba_amd as ssd
    x = torch.zeros((1, 100, 4, 8), device="cuda:0")
    dt = torch.zeros((1, 100, 4), device="cuda:0")
    B = torch.zeros((1, 100, 2, 16), device="cuda:0")
    A_log = torch.zeros(4, device="cuda:0")
    with pytest.raises(ssd.SSDError, match="multiple of chunk"):
        ssd.ssd_fwd(x, dt, A_log, B, B, A_log, chunk=64)


@pytest.mark.parametrize("dy_f32", [True, False])
def test_repeated_backward_bitwise(dy_f32):
    # 48 heads per group: long per-workgroup head loops and many workgroup-wide
    # sums in the decay-gradient pass; every repeat must give the same bits
    # (a data race in a block reduction showed up here as run-to-run dA_log
    # differences).
    cfg = CONFIGS["block"].with_(batch=2)
    d = make_inputs(cfg)
    x, dt, B, C = dev(d["x"]), dev(d["dt"]), dev(d["B"]), dev(d["C"])
    A_log, D = dev(d["A_log"]), dev(d["D"])
    dy = dev(d["dy"]).float() if dy_f32 else dev(d["dy"])
    import selective_state_space_mamba_amd as ssd
    y, fin, cs = ssd.ssd_fwd(x, dt, A_log, B, C, D, chunk=cfg.chunk)
    first = None
    for _ in range(6):
        g = ssd.ssd_bwd(x, dt, A_log, B, C, D, dy, chunk_states=cs, chunk=cfg.chunk)
        got = {k: host(g[k]) for k in ("dA_log", "ddt", "dD")}
        if first is None:
            first = got
        for k in got:
            assert np.array_equal(got[k], first[k]), k
