#!/usr/bin/env python3
"""SSD fwd+bwd throughput on one MI355X.

One step = ssd_fwd (saving the chunk states) + ssd_bwd (reading them) over one
batch of synthetic input already resident in HBM; for the block-slice workload
the step also runs the dt activation (softplus of dt_raw + dt_bias), conv1d+SiLU
and RMSNorm-gated, forward and backward.
Prints ONE JSON line on stdout (progress goes to stderr).

After the warm-up, an untimed pass of the same number of steps records HIP
events around every kernel (per-kernel times, `kernel_ms`).  The timed region
then records events around the dominant kernel only: its live average duration
gives `roofline`, and the other kernels run back to back as they do without
profiling.

The default workload is the grouped bf16 configuration (b=4, T=2048, H=32,
P=64, N=128, G=8, chunk 256), the one the performance target is quoted on.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "SSD fwd+bwd tokens/sec on 1 MI355X; achieved HBM GB/s and MFMA % of peak"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}  # MI355X dense matrix-core peaks
KERNELS_FWD = ["chunk_state_fwd", "chunk_out_fwd"]
KERNELS_BWD = ["chunk_state_bwd", "chunk_bwd_fused", "chunk_bwd_col", "chunk_bwd_row", "bwd_dt", "bwd_split_sum"]
KERNELS_SHELL = ["dt_softplus_fwd", "conv1d_silu_fwd", "rmsnorm_gated_fwd", "rmsnorm_gated_bwd", "conv1d_silu_bwd",
                 "dt_softplus_bwd"]
KERNEL_SOURCES = {
    "chunk_state_fwd": ["ssd_state.hip", "ssd_state_bf16.hip", "ssd_async.hpp", "ssd_common.hpp"],
    "chunk_state_bwd": ["ssd_state.hip", "ssd_state_bf16.hip", "ssd_async.hpp", "ssd_common.hpp"],
    "chunk_out_fwd": ["ssd_chunk_fwd.hip", "ssd_fwd_bf16.hip", "ssd_async.hpp", "ssd_common.hpp"],
    "chunk_bwd_col": ["ssd_chunk_bwd.hip", "ssd_bwd_bf16.hip", "ssd_async.hpp", "ssd_common.hpp"],
    "chunk_bwd_row": ["ssd_chunk_bwd.hip", "ssd_bwd_bf16.hip", "ssd_async.hpp", "ssd_common.hpp"],
    "chunk_bwd_fused": ["ssd_bwd_fused.hip", "ssd_async.hpp", "ssd_common.hpp"],
    "bwd_dt": ["ssd_chunk_bwd.hip", "ssd_common.hpp"],
}


# Device kernels behind each profiled launch (bf16 variant first), as
# substrings of the kernel names rocprofv3 records.
DEVICE_KERNELS = {
    "chunk_state_fwd": ("chunk_state_bf16_kernel<false", "chunk_state_kernel"),
    "chunk_state_bwd": ("chunk_state_bf16_kernel<true", "chunk_state_kernel"),
    "chunk_out_fwd": ("out_fwd_bf16_kernel", "chunk_out_fwd_kernel"),
    "chunk_bwd_col": ("bwd_col_bf16_kernel", "chunk_bwd_col_kernel"),
    "chunk_bwd_row": ("bwd_row_bf16_kernel", "chunk_bwd_row_kernel"),
    "chunk_bwd_fused": ("bwd_fused_bf16_kernel",),
    "bwd_dt": ("bwd_dt_kernel",),
}


def _device_match(kernel: str, name: str) -> bool:
    """Whether the recorded kernel name holds one of the kernel's device names
    followed by its argument or template list (or the next template argument)."""
    for n in DEVICE_KERNELS.get(kernel, (kernel + "_kernel",)):
        i = name.find(n)
        while i >= 0:
            if name[i + len(n):i + len(n) + 1] in ("(", "<", ">", ","):
                return True
            i = name.find(n, i + 1)
    return False


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def method_bytes(cfg, kernel: str) -> float:
    """The method's own inputs and outputs that one launch reads or writes,
    each once, at their storage dtypes: x, dt, B, C, dy, y and the gradients
    dx, ddt, dB, dC.  Intermediates (the chunk states and their gradients, the
    per-head row and column sums) are not counted; the saved chunk states are
    an optional output and are reported apart.  This is the denominator of the
    headline roofline."""
    s_a = 2 if cfg.dtype == "bf16" else 4
    s_y = s_a
    HP, GN, H = cfg.nheads * cfg.headdim, cfg.ngroups * cfg.dstate, cfg.nheads
    per_token = {
        "chunk_state_fwd": HP * s_a + GN * s_a + H * s_a,
        "chunk_out_fwd": 2 * HP * s_a + 2 * GN * s_a + H * s_a,
        "chunk_state_bwd": HP * s_y + GN * s_a + H * s_a,
        "chunk_bwd_col": HP * s_a + 2 * GN * s_a + H * s_a + HP * s_y + HP * 4 + GN * 4,
        "chunk_bwd_row": HP * s_a + 2 * GN * s_a + H * s_a + HP * s_y + GN * 4,
        # dx, dB, dC and (the dt kernel's work folded in) ddt
        "chunk_bwd_fused": HP * s_a + 2 * GN * s_a + H * s_a + HP * s_y + HP * 4 + 2 * GN * 4 + H * 4,
        "bwd_dt": H * s_a + H * 4,
    }
    return per_token[kernel] * cfg.batch * cfg.seqlen


# The saved state history a step keeps between its forward and backward: in
# bf16 (ssd_fwd_ex / ssd_bwd_ex) for problems the bf16 kernels run, which read
# the states only in bf16; --f32-history keeps the f32 one instead.
F32_HISTORY = False


def bf16_family(cfg) -> bool:
    return cfg.dtype == "bf16" and cfg.headdim % 8 == 0 and cfg.dstate % 8 == 0


def bf16_history(cfg) -> bool:
    return bf16_family(cfg) and not F32_HISTORY


def algorithmic_bytes(cfg, kernel: str) -> float:
    """Bytes one launch must move at minimum counting its intermediates too:
    each input it needs read once and each output written once, at the storage
    dtypes (the per-token figures are the per_token expressions below)."""
    s_a = 2 if cfg.dtype == "bf16" else 4
    s_y = s_a
    tok = cfg.batch * cfg.seqlen
    HP, GN, H = cfg.nheads * cfg.headdim, cfg.ngroups * cfg.dstate, cfg.nheads
    st = H * cfg.headdim * cfg.dstate * 4 / cfg.chunk  # chunk states per token (f32)
    sg = H * cfg.headdim * cfg.dstate * s_a / cfg.chunk  # state gradients per token (operand dtype)
    # the chunk states each kernel writes or reads: the bf16 family's output
    # and fused kernels read the bf16 copy (st / 2); with the bf16 history the
    # forward pass writes only that copy and the reverse pass reads no states,
    # with the f32 one the forward writes both and the reverse pass reads the
    # f32 states and writes the bf16 copy
    if bf16_family(cfg):
        st_fwd, st_out, st_rev = (st / 2, st / 2, 0.0) if bf16_history(cfg) else (1.5 * st, st / 2, 1.5 * st)
    else:
        st_fwd = st_out = st_rev = st
    per_token = {
        "chunk_state_fwd": HP * s_a + GN * s_a + H * s_a + st_fwd,
        "chunk_out_fwd": HP * s_a + 2 * GN * s_a + H * s_a + st_out + HP * s_a,
        "chunk_state_bwd": HP * s_y + GN * s_a + H * s_a + st_rev + sg,
        "chunk_bwd_col": HP * s_a + 2 * GN * s_a + H * s_a + HP * s_y + sg + HP * 4 + GN * 4 + 3 * H * 4,
        "chunk_bwd_row": HP * s_a + 2 * GN * s_a + H * s_a + HP * s_y + st + GN * 4 + 2 * H * 4,
        # + Gamma and the bf16 states in; the per-head column sums, diagonal,
        # R', readout term and the row sums of M (one slot per 64-column block
        # at or before a row's block, (nb + 1) / 2 on average) out, and read
        # back for ddt (written, H * 4)
        "chunk_bwd_fused": (HP * s_a + 2 * GN * s_a + H * s_a + HP * s_y + 2 * sg + HP * 4 + 2 * GN * 4
                            + 2 * (4 * H * 4 + H * 4 * (cfg.chunk // 64 + 1) / 2) + H * 4),
        "bwd_dt": H * s_a + 5 * H * 4 + H * 4,
    }
    return per_token[kernel] * tok


def backward_algorithmic_bytes(cfg) -> float:
    """Bytes the whole backward must move: x, dt, B, C, dy read once, dx, ddt,
    dB, dC written once (f32); saved chunk states excluded."""
    s_a = 2 if cfg.dtype == "bf16" else 4
    HP, GN, H = cfg.nheads * cfg.headdim, cfg.ngroups * cfg.dstate, cfg.nheads
    return (2 * HP * s_a + 2 * GN * s_a + H * s_a + HP * 4 + 2 * GN * 4 + H * 4) * cfg.batch * cfg.seqlen


def algorithmic_flops(cfg, kernel: str) -> float:
    """Useful MFMA flops of one launch (causal halves counted once)."""
    Q, P, N, H, G = cfg.chunk, cfg.headdim, cfg.dstate, cfg.nheads, cfg.ngroups
    tok = cfg.batch * cfg.seqlen
    per_token = {
        "chunk_state_fwd": 2 * H * P * N,
        "chunk_out_fwd": 2 * (0.5 * G * Q * N + 0.5 * H * Q * P + H * P * N),
        "chunk_state_bwd": 2 * H * P * N,
        "chunk_bwd_col": 2 * (0.5 * G * Q * N + 0.5 * G * Q * N + H * Q * P + 2 * H * P * N),
        "chunk_bwd_row": 2 * (0.5 * G * Q * N + 0.5 * G * Q * N + 0.5 * H * Q * P + H * P * N),
        # C.B^T once; dB and dC; yx and dx; B Gamma^T, x Gamma and dy H_c
        "chunk_bwd_fused": 2 * (1.5 * G * Q * N + H * Q * P + 3 * H * P * N),
        "bwd_dt": 0.0,
    }
    return per_token[kernel] * tok


def source_digest(kernel: str) -> str:
    """Digest of the code of the kernel's source files: comments removed and
    white space collapsed, so that a change of comments keeps the counters
    taken with that code."""
    h = hashlib.sha256()
    for fn in KERNEL_SOURCES.get(kernel, []):
        with open(os.path.join(ROOT, "selective_state_space_mamba_amd", "csrc", fn), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when there is none or the kernel's sources changed since."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_hbm_counters.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_src = re.search(r"^source_digest:\s*(\S+)", text, re.M)
    m_b = re.search(r"^hbm_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    if not m_src or not m_b or m_src.group(1) != source_digest(kernel):
        return None
    return float(m_b.group(1))


def _counter_rows(d: str):
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        rows.extend(csv.DictReader(open(f)))
    return rows


def write_counter_summary(fetch_dir: str, write_dir: str, kernel: str, workload: str, copy_mb: int) -> None:
    """HBM bytes per launch of `kernel` (or of each kernel of a comma list)
    from rocprofv3 FETCH_SIZE / WRITE_SIZE runs (KiB per dispatch), each scaled
    by what the same counter reads for the plain copy of `copy_mb` MiB that
    --calibrate-copy-mb ran in those runs."""
    if "," in kernel:
        for k in kernel.split(","):
            write_counter_summary(fetch_dir, write_dir, k, workload, copy_mb)
        return
    if copy_mb <= 0:
        raise SystemExit("--counter-summary needs --calibrate-copy-mb (the calibration copy size)")
    known = float(copy_mb << 20)
    out = {}
    for label, d, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        rows = [r for r in _counter_rows(d) if r["Counter_Name"] == counter]
        kv = [float(r["Counter_Value"]) for r in rows if _device_match(kernel, r["Kernel_Name"])]
        copies = sorted(float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"])
        if not kv or not copies:
            raise SystemExit(f"no {counter} rows for {kernel} or for the calibration copy in {d}")
        cal = copies[-3:]  # the calibration copies are the largest ones
        factor = known / (sum(cal) / len(cal) * 1024.0)
        out[label] = (sum(kv) / len(kv), len(kv), sum(cal) / len(cal), factor)
    fetch_b = out["fetch"][0] * 1024.0 * out["fetch"][3]
    write_b = out["write"][0] * 1024.0 * out["write"][3]
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_hbm_counters.txt")
    lines = [
        f"HBM traffic of {kernel} on the {workload} workload (rocprofv3 counters, per launch)",
        "",
        "Commands (repository root, one MI355X, TMPDIR=/tmp):",
        f"  rocprofv3 --pmc FETCH_SIZE -f csv -d <FETCH_DIR> -o run -- python3 bench.py --workload {workload} "
        f"--steps 2 --warmup 1 --no-cpu-baseline --calibrate-copy-mb {copy_mb}",
        f"  rocprofv3 --pmc WRITE_SIZE -f csv -d <WRITE_DIR> -o run -- python3 bench.py --workload {workload} "
        f"--steps 2 --warmup 1 --no-cpu-baseline --calibrate-copy-mb {copy_mb}",
        f"  python3 bench.py --workload {workload} --kernel {kernel} --calibrate-copy-mb {copy_mb} "
        "--counter-summary <FETCH_DIR> <WRITE_DIR>",
        "",
        f"FETCH_SIZE: {out['fetch'][0]:.1f} KiB per launch (mean of {out['fetch'][1]} launches); "
        f"the {copy_mb} MiB copy reads {out['fetch'][2]:.1f} KiB -> scale {out['fetch'][3]:.4f}",
        f"WRITE_SIZE: {out['write'][0]:.1f} KiB per launch (mean of {out['write'][1]} launches); "
        f"the {copy_mb} MiB copy writes {out['write'][2]:.1f} KiB -> scale {out['write'][3]:.4f}",
        f"fetch_bytes_per_launch: {fetch_b:.0f}",
        f"write_bytes_per_launch: {write_b:.0f}",
        f"hbm_bytes_per_launch: {fetch_b + write_b:.0f}",
        f"method_bytes_per_launch: {method_bytes(CONFIGS_BY_NAME()[workload], kernel):.0f}",
        f"algorithmic_bytes_per_launch (with intermediates): {algorithmic_bytes(CONFIGS_BY_NAME()[workload], kernel):.0f}",
        f"source_digest: {source_digest(kernel)}",
        "",
        "The digest covers the kernel's source files; bench.py reports this traffic only while it matches.",
    ]
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(path)


def CONFIGS_BY_NAME():
    from ssd_inputs import CONFIGS
    return CONFIGS


def _kernel_base(name: str) -> str:
    """Kernel name with its template arguments, without namespace and parameters."""
    return name.split("(")[0].replace("void ", "").replace("ssd::", "").strip()


def write_mfma_summary(d: str, workload: str) -> None:
    """Per-kernel MFMA utilisation and counted MFMA flops from one rocprofv3
    --pmc MfmaUtil MfmaFlopsBF16 MfmaFlopsF32 run (MfmaUtil = MFMA busy
    cycles / (GPU busy cycles x SIMDs); MfmaFlops* = MFMA MOPs x 512)."""
    rows = _counter_rows(d)
    if not rows:
        raise SystemExit(f"no counter rows under {d}")
    acc = {}
    for r in rows:
        k = _kernel_base(r["Kernel_Name"])
        acc.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    # bench kernel of each device kernel whose name says which one it is (the
    # chunk-state kernels serve both directions and are listed only)
    bench_of = {dev: k for k, devs in DEVICE_KERNELS.items() for dev in devs if not k.startswith("chunk_state")}
    lines = [f"MFMA counters per kernel on the {workload} workload (rocprofv3, per launch)", "",
             "Command (repository root, one MI355X, TMPDIR=/tmp):",
             f"  rocprofv3 --pmc MfmaUtil MfmaFlopsBF16 MfmaFlopsF32 -f csv -d <DIR> -o run -- python3 bench.py "
             f"--workload {workload} --steps 2 --warmup 1 --no-cpu-baseline",
             f"  python3 bench.py --workload {workload} --mfma-summary <DIR>", "",
             "MfmaUtil is 100 x SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x SIMDs), the share of SIMD cycles",
             "the matrix cores were busy during the launch; MfmaFlops* count 512 flops per MFMA MOP (all issued",
             "MFMAs, including the masked halves of diagonal tiles and zero padding).", "",
             "| kernel | launches | MfmaUtil % | counted MFMA GFLOP per launch (bf16 + f32) |",
             "|---|---|---|---|"]
    out = {}
    for k in sorted(acc):
        c = acc[k]
        if "MfmaUtil" not in c:
            continue
        n = len(c["MfmaUtil"])
        util = sum(c["MfmaUtil"]) / n
        fl = sum(sum(c.get(x, [0.0])) / max(1, len(c.get(x, []))) for x in ("MfmaFlopsBF16", "MfmaFlopsF32"))
        lines.append(f"| `{k}` | {n} | {util:.2f} | {fl / 1e9:.3f} |")
        if k.split("<")[0] in bench_of:
            out[bench_of[k.split("<")[0]]] = (util, fl)
    lines.append("")
    for k, (util, fl) in sorted(out.items()):
        lines.append(f"mfma_util_pct {k}: {util:.3f}")
        lines.append(f"mfma_flops_per_launch {k}: {fl:.0f}")
        lines.append(f"source_digest {k}: {source_digest(k)}")
    lines += ["", "The digests cover each kernel's source files; bench.py reports a kernel's utilisation only while",
              "its digest matches."]
    path = os.path.join(ROOT, "profiles", f"mfma_counters_{workload}.txt")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(path)


def measured_mfma_util(kernel: str, workload: str):
    path = os.path.join(ROOT, "profiles", f"mfma_counters_{workload}.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_u = re.search(rf"^mfma_util_pct {re.escape(kernel)}:\s*([0-9.eE+-]+)", text, re.M)
    m_d = re.search(rf"^source_digest {re.escape(kernel)}:\s*(\S+)", text, re.M)
    if not m_u or not m_d or m_d.group(1) != source_digest(kernel):
        return None
    return float(m_u.group(1))


def to_dev(a):
    import numpy as np
    import torch
    from ssd_inputs import Stored
    if a is None:
        return None
    if isinstance(a, Stored):
        if a.dtype == "bf16":
            return torch.from_numpy(a.raw.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a.raw)).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def roofline_entry(cfg, kernel: str, t_s: float) -> dict:
    """Roofline of one launch of `kernel` taking t_s seconds.  `achieved`
    counts the method's inputs and outputs the launch moves (method_bytes); the
    figure with its intermediates counted too is `with_intermediates_gbs`.  The
    roof that bounds it is HBM when its algorithmic flops per byte fall below
    the machine balance of the operand dtype's MFMA peak over the HBM peak, and
    that MFMA peak above it."""
    alg = method_bytes(cfg, kernel)
    flops = algorithmic_flops(cfg, kernel)
    achieved = alg / t_s / 1e9
    tflops = flops / t_s / 1e12
    traffic = measured_traffic(kernel, cfg.name)
    mfma_peak = MFMA_PEAK_TFLOPS["bf16" if cfg.dtype == "bf16" else "f32"]
    if flops / alg > mfma_peak * 1e3 / HBM_PEAK_GBS:
        r = {"bound": "mfma", "achieved": round(tflops, 2), "peak": mfma_peak, "unit": "TFLOP/s",
             "frac": round(tflops / mfma_peak, 4), "traffic": traffic, "hbm_gbs": round(achieved, 1)}
    else:
        r = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic, "mfma_tflops": round(tflops, 2)}
    r.update({"scope": "dominant kernel (per launch)", "kernel": kernel, "kernel_ms": round(t_s * 1e3, 4),
              "algorithmic_bytes": alg, "algorithmic_flops": flops,
              "with_intermediates_gbs": round(algorithmic_bytes(cfg, kernel) / t_s / 1e9, 1),
              "mfma_util_pct": measured_mfma_util(kernel, cfg.name)})
    return r


def make_step(cfg, d):
    import torch
    import selective_state_space_mamba_amd as ssd
    x, dt, B, C = to_dev(d["x"]), to_dev(d["dt"]), to_dev(d["B"]), to_dev(d["C"])
    A_log, D, h0 = to_dev(d["A_log"]), to_dev(d["D"]), to_dev(d.get("h0"))
    dy = to_dev(d["dy"])
    f32 = dict(dtype=torch.float32, device="cuda")
    b, T, H, P, N, G, Q = cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.dstate, cfg.ngroups, cfg.chunk
    hist = "chunk_states_bf16" if bf16_history(cfg) else "chunk_states"
    fo = {"y": torch.empty_like(x), "final_state": torch.empty((b, H, P, N), **f32),
          hist: torch.empty((b, T // Q, H, P, N), dtype=torch.bfloat16 if bf16_history(cfg) else torch.float32,
                            device="cuda")}
    go = {"dx": torch.empty((b, T, H, P), **f32), "ddt": torch.empty((b, T, H), **f32),
          "dA_log": torch.empty(H, **f32), "dB": torch.empty((b, T, G, N), **f32),
          "dC": torch.empty((b, T, G, N), **f32), "dD": torch.empty(H, **f32),
          "d_init_state": torch.empty((b, H, P, N), **f32)}
    if not cfg.shell:
        prob = ssd._binding.make_problem(x, B, Q, dy.dtype)
        f32h = hist == "chunk_states"
        wsf = torch.empty(max(1, ssd.ssd_workspace_bytes(prob, False, f32h)), dtype=torch.uint8, device="cuda")
        wsb = torch.empty(max(1, ssd.ssd_workspace_bytes(prob, True, f32h)), dtype=torch.uint8, device="cuda")

        def step():
            ssd.ssd_fwd_ex(x, dt, A_log, B, C, D, h0, chunk=Q, want_chunk_states=f32h, want_chunk_states_bf16=not f32h,
                           out=fo, workspace=wsf)
            ssd.ssd_bwd(x, dt, A_log, B, C, D, dy, h0, chunk_states=fo.get("chunk_states"),
                        chunk_states_bf16=fo.get("chunk_states_bf16"), chunk=Q, out=go, workspace=wsb)
        return step

    if cfg.d_model:
        return make_train_step(cfg, d)
    xbc, z, gout = to_dev(d["xBC"]), to_dev(d["z"]), to_dev(d["gout"])
    dt_raw, dt_bias = to_dev(d["dt_raw"]), to_dev(d["dt_bias"])
    conv_w, conv_b, norm_w = to_dev(d["conv_w"]), to_dev(d["conv_b"]), to_dev(d["norm_w"])
    di = cfg.d_inner
    lib = ssd.load_library()
    K = conv_w.shape[1]
    u8 = dict(dtype=torch.uint8, device="cuda")
    prob = ssd._binding.make_problem(x.view(b, T, H, P), B, Q, torch.bfloat16)
    f32h = hist == "chunk_states"
    wsf = torch.empty(max(1, ssd.ssd_workspace_bytes(prob, False, f32h)), **u8)
    wsb = torch.empty(max(1, ssd.ssd_workspace_bytes(prob, True, f32h)), **u8)
    wsr = torch.empty(max(1, lib.mamba2_rmsnorm_gated_bwd_workspace_bytes(b * T, di)), **u8)
    wsc = torch.empty(max(1, lib.mamba2_conv1d_silu_bwd_workspace_bytes(b, T, di, G, N, K)), **u8)
    wsd = torch.empty(max(1, lib.ssd_dt_softplus_bwd_workspace_bytes(b * T, H)), **u8)
    dt = torch.empty_like(dt_raw)

    def step():
        ssd.dt_softplus_fwd(dt_raw, dt_bias, out=dt)
        xs, Bs, Cs = ssd.conv1d_silu_fwd(xbc, conv_w, conv_b, di, G, N)
        xs = xs.view(b, T, H, P)
        r = ssd.ssd_fwd_ex(xs, dt, A_log, Bs, Cs, D, h0, chunk=Q, want_chunk_states=f32h,
                           want_chunk_states_bf16=not f32h, out=fo, workspace=wsf)
        y = r["y"]
        out, inv = ssd.rmsnorm_gated_fwd(y.view(b, T, di), z, norm_w, cfg.norm_eps)
        gy, gz, gw = ssd.rmsnorm_gated_bwd(y.view(b, T, di), z, norm_w, inv, gout, workspace=wsr,
                                           dy_dtype=torch.bfloat16)
        g = ssd.ssd_bwd(xs, dt, A_log, Bs, Cs, D, gy.view(b, T, H, P), h0, chunk_states=r["chunk_states"],
                        chunk_states_bf16=r["chunk_states_bf16"], chunk=Q, out=go, workspace=wsb)
        ssd.conv1d_silu_bwd(xbc, conv_w, conv_b, g["dx"].view(b, T, di), g["dB"], g["dC"], di, G, N,
                            workspace=wsc)
        ssd.dt_softplus_bwd(dt_raw, dt_bias, g["ddt"], workspace=wsd)
    return step


def make_train_step(cfg, d):
    """One training step of a Mamba-2 block with its projections: in_proj parts
    (z, xBC, dt_raw), the block slice, out_proj, and the backward through all of
    them, each a C-ABI call on preallocated buffers (the GEMMs through ssd_gemm)."""
    import torch
    import selective_state_space_mamba_amd as ssd
    b, T, H, P, N, G, Q = cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.dstate, cfg.ngroups, cfg.chunk
    dm, di, cd, M = cfg.d_model, cfg.d_inner, cfg.conv_dim, cfg.batch * cfg.seqlen
    lib = ssd.load_library()
    u, Wo, go = (to_dev(d[k]) for k in ("u", "W_out", "go"))
    # W_z, W_xbc and W_dt as the row blocks of one in_proj matrix, so that the
    # gradients of z, xBC and dt_raw, written side by side, meet it in one
    # product for du and one for the weight gradients (rows padded with zeros
    # to a multiple of 64, the products' k-tile)
    nin = di + cd + H
    ninp = -(-nin // 64) * 64
    Win = torch.zeros((ninp, dm), dtype=torch.bfloat16, device="cuda")
    Win[:di] = to_dev(d["W_z"])
    Win[di:di + cd] = to_dev(d["W_xbc"])
    Win[di + cd:nin] = to_dev(d["W_dt"])
    Wz, Wx, Wd = Win[:di], Win[di:di + cd], Win[di + cd:nin]
    conv_w, conv_b, dt_bias = to_dev(d["conv_w"]), to_dev(d["conv_b"]), to_dev(d["dt_bias"])
    A_log, D, norm_w = to_dev(d["A_log"]), to_dev(d["D"]), to_dev(d["norm_w"])
    bf = dict(dtype=torch.bfloat16, device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    u8 = dict(dtype=torch.uint8, device="cuda")
    u2, go2 = u.view(M, dm), go.view(M, dm)
    z, xbc, raw = torch.empty((M, di), **bf), torch.empty((M, cd), **bf), torch.empty((M, H), **bf)
    dt = torch.empty((M, H), **bf)
    o = torch.empty((M, dm), **bf)
    f32h = not bf16_history(cfg)
    hist = "chunk_states" if f32h else "chunk_states_bf16"
    fo = {"y": torch.empty((b, T, H, P), **bf), "final_state": torch.empty((b, H, P, N), **f32),
          hist: torch.empty((b, T // Q, H, P, N), **(f32 if f32h else bf))}
    go_ = {"dx": torch.empty((b, T, H, P), **f32), "ddt": torch.empty((b, T, H), **f32),
           "dA_log": torch.empty(H, **f32), "dB": torch.empty((b, T, G, N), **f32),
           "dC": torch.empty((b, T, G, N), **f32), "dD": torch.empty(H, **f32)}
    gact = torch.empty((M, di), **bf)  # the out_proj input gradient, in the activation dtype
    dWo, dWin = (torch.empty(s_, **f32) for s_ in ((dm, di), (ninp, dm)))
    du = torch.empty((M, dm), **f32)
    # [dz | d xBC | d dt_raw | zeros] in bf16, one row per token
    gin = torch.zeros((M, ninp), **bf)
    gz_view, gx_view, gd_view = gin[:, :di].view(b, T, di), gin[:, di:di + cd].view(b, T, cd), gin[:, di + cd:nin]
    prob = ssd._binding.make_problem(fo["y"], to_dev(d["B"]), Q, torch.bfloat16)
    wsf = torch.empty(max(1, ssd.ssd_workspace_bytes(prob, False, f32h)), **u8)
    wsb = torch.empty(max(1, ssd.ssd_workspace_bytes(prob, True, f32h)), **u8)
    wsr = torch.empty(max(1, lib.mamba2_rmsnorm_gated_bwd_workspace_bytes(M, di)), **u8)
    wsc = torch.empty(max(1, lib.mamba2_conv1d_silu_bwd_workspace_bytes(b, T, di, G, N, conv_w.shape[1])), **u8)
    wsd = torch.empty(max(1, lib.ssd_dt_softplus_bwd_workspace_bytes(M, H)), **u8)
    d_dt_bias = torch.empty(H, **f32)

    def step():
        ssd.gemm(u2, Wz, trans_b=True, out=z)
        ssd.gemm(u2, Wx, trans_b=True, out=xbc)
        ssd.gemm(u2, Wd, trans_b=True, out=raw)
        ssd.dt_softplus_fwd(raw, dt_bias, out=dt)
        xs, Bs, Cs = ssd.conv1d_silu_fwd(xbc.view(b, T, cd), conv_w, conv_b, di, G, N)
        xs = xs.view(b, T, H, P)
        dt3 = dt.view(b, T, H)
        r = ssd.ssd_fwd_ex(xs, dt3, A_log, Bs, Cs, D, None, chunk=Q, want_chunk_states=f32h,
                           want_chunk_states_bf16=not f32h, out=fo, workspace=wsf)
        y = r["y"]
        out, inv = ssd.rmsnorm_gated_fwd(y.view(b, T, di), z.view(b, T, di), norm_w, cfg.norm_eps)
        ssd.gemm(out.view(M, di), Wo, trans_b=True, out=o)
        # backward
        ssd.gemm(go2, Wo, out=gact)
        ssd.gemm(go2, out.view(M, di), trans_a=True, out=dWo)
        gy, _, gw = ssd.rmsnorm_gated_bwd(y.view(b, T, di), z.view(b, T, di), norm_w, inv, gact.view(b, T, di),
                                          workspace=wsr, dy_dtype=torch.bfloat16, dz_dtype=torch.bfloat16,
                                          dz_out=gz_view)
        g = ssd.ssd_bwd(xs, dt3, A_log, Bs, Cs, D, gy.view(b, T, H, P), None, chunk_states=r["chunk_states"],
                        chunk_states_bf16=r["chunk_states_bf16"], chunk=Q, out=go_,
                        workspace=wsb, want_d_init_state=False)
        # the gradients of z, xBC and dt_raw come out of their kernels in bf16
        # (the values a cast of the f32 gradients gives), side by side in gin
        ssd.conv1d_silu_bwd(xbc.view(b, T, cd), conv_w, conv_b, g["dx"].view(b, T, di), g["dB"], g["dC"], di, G,
                            N, workspace=wsc, dxbc_dtype=torch.bfloat16, out=gx_view)
        ssd.dt_softplus_bwd(raw, dt_bias, g["ddt"].view(M, H), workspace=wsd, out_dtype=torch.bfloat16,
                            out=(gd_view, d_dt_bias))
        ssd.gemm(gin, Win, out=du)
        ssd.gemm(gin, u2, trans_a=True, out=dWin)
    return step


def train_step_flops(cfg) -> float:
    """Flops of the projection GEMMs in one training step (forward 1x, backward 2x)."""
    dm, di, cd, H = cfg.d_model, cfg.d_inner, cfg.conv_dim, cfg.nheads
    return 3 * 2.0 * cfg.tokens * dm * (di + cd + H + di)


def cpu_baseline(cfg, d, batches: int, min_wall_s: float = 1.0):
    """The oracle on the host over the first `batches` batch rows of the same
    workload: SSD fwd + bwd, and for the block slice the whole chain the GPU
    step runs (dt activation, conv1d + SiLU, SSD, RMSNorm-gated, forward and
    backward)."""
    import numpy as np
    import oracle
    nb = min(cfg.batch, max(1, batches))
    sl = slice(0, nb)
    h0 = None if d.get("h0") is None else d["h0"][sl]
    threads = oracle.default_threads()
    b, T, H, P, G, N = nb, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.ngroups, cfg.dstate

    def run():
        if not cfg.shell:
            args = (d["x"].values[sl], d["dt"].values[sl], d["A_log"], d["B"].values[sl], d["C"].values[sl], d["D"])
            oracle.ssd_fwd(*args, h0, chunk=cfg.chunk, nthreads=threads)
            oracle.ssd_bwd(*args, d["dy"].values[sl], h0, nthreads=threads)
            return
        di = cfg.d_inner
        xbc_v, raw_v, z_v, gout_v = d["xBC"].values[sl], d["dt_raw"].values[sl], d["z"].values[sl], d["gout"].values[sl]
        if cfg.d_model:  # the projections as f64 matrix products
            U = d["u"].values[sl].astype(np.float64)
            WZ, WX, WD, WO = (d[k].values.astype(np.float64) for k in ("W_z", "W_xbc", "W_dt", "W_out"))
            z_v, xbc_v, raw_v = U @ WZ.T, U @ WX.T, U @ WD.T
            gout_v = d["go"].values[sl].astype(np.float64) @ WO
        dt = oracle.dt_softplus_fwd(raw_v, d["dt_bias"])
        _, act = oracle.conv_fwd(xbc_v, d["conv_w"], d["conv_b"])
        x = act[..., :di].reshape(b, T, H, P)
        Bm = act[..., di:di + G * N].reshape(b, T, G, N)
        Cm = act[..., di + G * N:].reshape(b, T, G, N)
        args = (x, dt, d["A_log"], Bm, Cm, d["D"])
        y = oracle.ssd_fwd(*args, h0, chunk=cfg.chunk, nthreads=threads)["y"].reshape(b, T, di)
        out, inv = oracle.rmsnorm_fwd(y, z_v, d["norm_w"], cfg.norm_eps)
        gy, gz, _ = oracle.rmsnorm_bwd(y, z_v, d["norm_w"], inv, gout_v)
        g = oracle.ssd_bwd(*args, gy.reshape(b, T, H, P), h0, nthreads=threads)
        gact = np.concatenate([g["dx"].reshape(b, T, di), g["dB"].reshape(b, T, -1), g["dC"].reshape(b, T, -1)], -1)
        dxbc, _, _ = oracle.conv_bwd(xbc_v, d["conv_w"], d["conv_b"], gact)
        draw, _ = oracle.dt_softplus_bwd(raw_v, d["dt_bias"], g["ddt"])
        if cfg.d_model:
            _ = out.reshape(-1, di) @ WO.T
            gof = d["go"].values[sl].astype(np.float64).reshape(-1, cfg.d_model)
            _ = gof.T @ out.reshape(-1, di)
            Uf = U.reshape(-1, cfg.d_model)
            flat = [gz.reshape(-1, di), dxbc.reshape(-1, cfg.conv_dim), draw.reshape(-1, H)]
            _ = sum(gf @ W for gf, W in zip(flat, (WZ, WX, WD)))
            _ = [gf.T @ Uf for gf in flat]

    # repeat the sample until about a second of wall time (10-30 s of CPU
    # work on a 16-thread host) has been measured
    reps, el = 0, 0.0
    while reps == 0 or el < min_wall_s:
        t0 = time.perf_counter()
        run()
        el += time.perf_counter() - t0
        reps += 1
    what = "SSD fwd+bwd" if not cfg.shell else "dt activation + conv1d/SiLU + SSD + RMSNorm-gated, fwd+bwd"
    if cfg.d_model:
        what += " with the projections as numpy f64 matrix products"
    try:
        avail = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        avail = os.cpu_count() or 1
    return {"value": reps * nb * cfg.seqlen / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "host_cpus": os.cpu_count(), "cpus_available": avail,
            "sample": (f"sequential f64 oracle, {what} on batch rows 0..{nb - 1} of {cfg.batch} "
                       f"({nb * cfg.seqlen} tokens) run {reps} times, {el:.1f} s wall on {threads} threads "
                       f"(the host reports {os.cpu_count()} CPUs, {avail} available to this process; the oracle "
                       "takes at most 16, one GPU's share of the host); tokens/s of that sample")}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="grouped",
                    choices=["tiny", "m130", "grouped", "long", "block", "block_train"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--f32-history", action="store_true",
                    help="keep the saved state history in f32 (default for bf16 problems: bf16, ssd_fwd_ex / ssd_bwd_ex)")
    ap.add_argument("--cpu-batches", type=int, default=0, help="batch rows in the oracle sample (0: workload default)")
    ap.add_argument("--calibrate-copy-mb", type=int, default=0,
                    help="after timing, run a plain device copy of this many MiB (3 times) for counter calibration")
    ap.add_argument("--counter-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the HBM-traffic summary from two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) and exit")
    ap.add_argument("--kernel", default="chunk_bwd_col", help="kernel for --counter-summary")
    ap.add_argument("--mfma-summary", metavar="DIR",
                    help="write the per-kernel MFMA utilisation summary from a rocprofv3 --pmc MfmaUtil "
                         "MfmaFlopsBF16 MfmaFlopsF32 run and exit")
    args = ap.parse_args()
    global F32_HISTORY
    F32_HISTORY = args.f32_history
    if args.mfma_summary:
        write_mfma_summary(args.mfma_summary, args.workload)
        return
    if args.counter_summary:
        write_counter_summary(args.counter_summary[0], args.counter_summary[1], args.kernel, args.workload,
                              args.calibrate_copy_mb)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the SSD path here has no multi-GPU "
              "code; it would shard by batch rows, by groups of heads, or by time with one state exchange "
              "per direction.", file=sys.stderr)
        sys.exit(2)

    import torch
    import selective_state_space_mamba_amd as ssd
    from ssd_inputs import CONFIGS, make_inputs

    cfg = CONFIGS[args.workload]
    log(f"[bench] workload {cfg}")
    d = make_inputs(cfg)
    step = make_step(cfg, d)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} done; timing {args.steps} steps")

    # Per-kernel times: an untimed pass of the same steps with HIP events
    # around every kernel (the events hold the stream up a little between
    # kernels, so they stay out of the timed region).
    kernels = KERNELS_FWD + KERNELS_BWD + (KERNELS_SHELL if cfg.shell else []) + (
        ["gemm"] if cfg.d_model else [])
    ssd.profile_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kms = {}
    for k in kernels:
        ms, n = ssd.profile_kernel_ms(k)
        if n:
            kms[k] = ms / n
    core = {k: v for k, v in kms.items() if k in KERNEL_SOURCES}
    dom = max(core, key=core.get)

    # Timed region: events around the dominant kernel only, whose live
    # average duration gives the roofline figure.
    ssd.profile_enable(True)
    ssd.profile_only(dom)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_dom, n_dom = ssd.profile_kernel_ms(dom)
    ssd.profile_only("")
    ssd.profile_enable(False)
    ms_step = elapsed * 1e3 / args.steps
    value = cfg.tokens * args.steps / elapsed
    log(f"[bench] {ms_step:.3f} ms/step, {value:.4g} tokens/s; {dom} {ms_dom / n_dom:.4f} ms live; "
        "per-kernel ms (profiling pass): " + " ".join(f"{k}={v:.4f}" for k, v in kms.items()))

    t_dom = ms_dom / n_dom * 1e-3
    roofline = roofline_entry(cfg, dom, t_dom)
    t_bwd = sum(v for k, v in kms.items() if k in KERNELS_BWD) * 1e-3
    bwd_alg = backward_algorithmic_bytes(cfg)
    ssd_bwd = {"ms": round(t_bwd * 1e3, 4), "algorithmic_bytes": bwd_alg,
               "achieved": round(bwd_alg / t_bwd / 1e9, 1), "unit": "GB/s",
               "frac": round(bwd_alg / t_bwd / 1e9 / HBM_PEAK_GBS, 4)}

    if args.calibrate_copy_mb > 0:
        nbytes = args.calibrate_copy_mb << 20
        src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on the host")
        cpu = cpu_baseline(cfg, d, args.cpu_batches or (1 if cfg.shell else cfg.batch))

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if cfg.dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": (f"{cfg.name}: b={cfg.batch} T={cfg.seqlen} H={cfg.nheads} P={cfg.headdim} "
                                f"N={cfg.dstate} G={cfg.ngroups} chunk={cfg.chunk} {cfg.dtype}"
                                + (" + conv1d/SiLU + RMSNorm-gated" if cfg.shell else "")
                                + (f" + in/out projections d_model={cfg.d_model}" if cfg.d_model else "")),
                   "global_batch": cfg.batch, "seq_len": cfg.seqlen, "parallelism": "single-gpu",
                   "state_history": "bf16" if bf16_history(cfg) else "f32"},
        "kernel_ms": {k: round(v, 4) for k, v in kms.items()},
        "roofline": roofline,
        "ssd_bwd": ssd_bwd,
        "cpu_baseline": cpu,
    }
    if cfg.d_model and "gemm" in kms:
        # three in_proj products, out_proj, and its two gradient products; the
        # in_proj gradients as one product for du and one for the weights
        n_gemm = 8
        t_g = kms["gemm"] * n_gemm * 1e-3
        line["projections"] = {"ms_per_step": round(t_g * 1e3, 4), "calls": n_gemm,
                               "tflops": round(train_step_flops(cfg) / t_g / 1e12, 1),
                               "peak_tflops": MFMA_PEAK_TFLOPS["bf16"],
                               "library": "rocBLAS gemm_ex" if os.environ.get("SSD_GEMM") == "rocblas" else "hipBLASLt"}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
