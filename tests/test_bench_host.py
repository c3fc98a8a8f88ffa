"""Host-side logic of bench.py: the algorithmic byte and flop counts its
rooflines divide by, the choice of roof, and the one-GPU guard."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from ssd_inputs import CONFIGS  # noqa: E402


def test_grouped_workload_algorithmic_bytes():
    cfg = CONFIGS["grouped"]
    tok = cfg.batch * cfg.seqlen
    HP, GN, H = 32 * 64, 8 * 128, 32
    # x, dt, B, C, dy read once in bf16; dx, ddt, dB, dC written once in f32
    assert bench.backward_algorithmic_bytes(cfg) == (2 * HP * 2 + 2 * GN * 2 + H * 2 + HP * 4 + 2 * GN * 4 + H * 4) * tok
    assert round(bench.backward_algorithmic_bytes(cfg) / 1e6, 1) == 236.5
    # the column kernel: x, B, C, dt, dy, Gamma in; dx, dB, three per-row sums out
    sg = 32 * 64 * 128 * 2 / 256
    col = HP * 2 + 2 * GN * 2 + H * 2 + HP * 2 + sg + HP * 4 + GN * 4 + 3 * H * 4
    assert bench.algorithmic_bytes(cfg, "chunk_bwd_col") == col * tok
    assert round(bench.algorithmic_bytes(cfg, "chunk_bwd_col") / 1e6, 1) == 221.8


def test_method_bytes_exclude_intermediates():
    cfg = CONFIGS["grouped"]
    tok = cfg.batch * cfg.seqlen
    HP, GN, H = 32 * 64, 8 * 128, 32
    # the column kernel moves x, B, C, dt, dy (bf16) and dx, dB (f32) of the
    # method; Gamma and the per-row sums are intermediates
    assert bench.method_bytes(cfg, "chunk_bwd_col") == (HP * 2 + 2 * GN * 2 + H * 2 + HP * 2 + HP * 4 + GN * 4) * tok
    assert round(bench.method_bytes(cfg, "chunk_bwd_col") / 1e6, 1) == 201.9
    # chunk states are an optional output, not counted
    assert bench.method_bytes(cfg, "chunk_state_fwd") == (HP * 2 + GN * 2 + H * 2) * tok


def test_roof_choice_follows_machine_balance():
    # bf16 grouped column kernel: about 97 flop/B, below 2.5 PFLOP/s / 8 TB/s
    r = bench.roofline_entry(CONFIGS["grouped"], "chunk_bwd_col", 88e-6)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert abs(r["frac"] - bench.method_bytes(CONFIGS["grouped"], "chunk_bwd_col") / 88e-6 / 8e12) < 1e-4
    assert r["with_intermediates_gbs"] > r["achieved"]
    # f32 long column kernel: above 157.3 TFLOP/s / 8 TB/s
    r = bench.roofline_entry(CONFIGS["long"], "chunk_bwd_col", 1.9e-3)
    assert r["bound"] == "mfma" and r["peak"] == 157.3
    assert abs(r["frac"] - bench.algorithmic_flops(CONFIGS["long"], "chunk_bwd_col") / 1.9e-3 / 157.3e12) < 1e-4


def test_projection_flops():
    cfg = CONFIGS["block_train"]
    per_pass = 2.0 * cfg.tokens * cfg.d_model * (cfg.d_inner + cfg.conv_dim + cfg.nheads + cfg.d_inner)
    assert bench.train_step_flops(cfg) == 3 * per_pass


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2 and "one GPU" in res.stderr


def test_fused_method_bytes_include_ddt():
    # the fused backward kernel also writes ddt (the dt kernel's work)
    cfg = CONFIGS["grouped"]
    HP, GN, H = cfg.nheads * cfg.headdim, cfg.ngroups * cfg.dstate, cfg.nheads
    tok = cfg.batch * cfg.seqlen
    assert bench.method_bytes(cfg, "chunk_bwd_fused") == (HP * 2 + 2 * GN * 2 + H * 2 + HP * 2 + HP * 4 + 2 * GN * 4
                                                          + H * 4) * tok
    # so the fused kernel alone reads and writes every byte the whole backward must move
    assert bench.method_bytes(cfg, "chunk_bwd_fused") == bench.backward_algorithmic_bytes(cfg)
