#!/usr/bin/env python3
"""Benchmark of the group-wise affine quantized linear hot path on one MI355X.

One step = one pass of the path over one batch at the headline workload
M=4096 tokens, K=N=4608, 4-bit codes, group 64 (square projection of the
4608-wide DiT at 1024x1024): the activation prepass (qlinear_fast_activations:
bf16 x to fp16 with per-row power-of-two scales) followed by the fused
dequant-GEMM on tiled weights (qlinear_forward_ex, FAST mode), i.e. exactly the
kernels qlinear_forward_ex launches for this layer with a workspace. Weights are
quantized by the library's device RTN quantizer and repacked to the tiled
layout during setup, as a loader does once per checkpoint; inputs are seeded
synthetic tensors already resident in HBM when the timed region starts.

Printed: one JSON line with the whole-job throughput (TFLOP/s), the roofline of
the dominant kernel (fused GEMM, timed live with HIP events on its stream), the
other configured workloads and entry points as secondary rows (each with its
roofline fraction), and the CPU oracle timed on this host as a reported
baseline (the headline workload in full, the other workloads on row samples).
"""
from __future__ import annotations

import os
import sys

# the oracle's BLAS uses every core this process may run on; fixed before
# numpy (imported by torch) starts its thread pool
_CORES = len(os.sched_getaffinity(0))
os.environ.setdefault("OPENBLAS_NUM_THREADS", str(_CORES))

import argparse  # noqa: E402
import hashlib  # noqa: E402
import json  # noqa: E402
import subprocess  # noqa: E402
import threading  # noqa: E402
import time  # noqa: E402

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "qlinear TFLOP/s (M=4096,K=N=4608, Q4 g64) + % MFMA peak; GB/s skinny-M"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_F16_TFLOPS = 2500.0      # MI355X dense fp16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
WORKLOAD = dict(name="dit_square_proj_M4096_K4608_N4608_q4_g64", M=4096, K=4608, N=4608, bits=4, wid=6)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm3_fast_q4_M4096_K4608_N4608_traffic.txt")
GEMM_SOURCES = ("gemm3.hip", "gemm3_core.h", "ql_device.h")
SETTLE_S = 0.3                # setup: steps run before the warm-up while the engine clock settles


def log(msg):
    sys.stderr.write(f"[bench] {msg}\n")
    sys.stderr.flush()


def gemm_source_hash() -> str:
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(ROOT, "group_wise_affine_qlinear_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(M, N, K, bits):
    """Codes + scale/bias + bf16 x + fp32 y, each read or written once."""
    return N * K * bits / 8 + 4 * N * K / 64 + 2 * M * K + 4 * M * N


def make_weights(torch, ql, inputs, N, K, bits, wid, copies=1, tiled=False, glu=False):
    """Device-quantized weight sets; tiled=True repacks each set for the GEMM kernels
    (then a set is (tiled_q, tiled_sb, None)); glu=True repacks in GLU order."""
    w = torch.from_numpy(inputs.weights(N, K, wid)).cuda()
    sets = []
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    for _ in range(copies):
        p = torch.empty((N, K * bits // 32), dtype=torch.int32, device="cuda")
        s = torch.empty((N, K // 64), dtype=torch.int16, device="cuda")
        b = torch.empty((N, K // 64), dtype=torch.int16, device="cuda")
        ql.qlinear_quantize_rtn(w, bits, 64, N, K, p, s, b, status)
        if tiled:
            tq, tsb = (ql.qlinear_repack_glu if glu else ql.qlinear_repack)(p, s, b, bits, 64, N, K)
            sets.append((tq, tsb, None))
            del p, s, b
        else:
            sets.append((p, s, b))
    torch.cuda.synchronize()
    if int(status.item()) != 0:
        raise RuntimeError("quantizer reported a range error")
    del w
    return sets


def smi_snapshot():
    """Socket power and clocks from amd-smi (context only; None where the tool
    or a field is unavailable)."""
    try:
        r = subprocess.run(["amd-smi", "metric", "--clock", "--power", "--json"], capture_output=True, text=True,
                           timeout=20)
        d = json.loads(r.stdout[r.stdout.index("{"):])
        g = d["gpu_data"][0]
        clocks = g["clock"]
        gfx = [v["clk"]["value"] for k, v in clocks.items()
               if k.startswith("gfx_") and isinstance(v, dict) and isinstance(v.get("clk"), dict)]
        return {"socket_power_W": g["power"]["socket_power"]["value"],
                "gfx_clk_MHz_mean": round(sum(gfx) / len(gfx)) if gfx else None,
                "mem_clk_MHz": clocks["mem_0"]["clk"]["value"]}
    except Exception:
        return None


def time_calls(torch, fn, iters, warmup, settle_s=0.0):
    """Average per-call time (ms) with HIP events on the current stream, after
    `warmup` calls and then calls for at least `settle_s` seconds while the
    engine clock settles under the load."""
    for _ in range(warmup):
        fn()
    if settle_s > 0:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < settle_s:
            for _ in range(5):
                fn()
            torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(st)
    for _ in range(iters):
        fn()
    e1.record(st)
    e1.synchronize()
    return e0.elapsed_time(e1) / iters


# ------------------------------------------------------------------ secondary cases
#
# Each case sets up its tensors once and returns (call, meta): call() runs the
# measured launch(es) once; meta holds the figures a row reports. GEMM rows
# report TFLOP/s as a fraction of the dense 16-bit MFMA peak (both fp16 and bf16
# are 2.5 PFLOP/s on MI355X); skinny rows report GB/s as a fraction of HBM.
# A call with a workspace runs what automatic dispatch picks there (FAST for
# M > 16: the fp16 prepass and the GEMM, both inside the timed call); the
# spec call qlinear_forward runs with no workspace (for M > 16 the FAST
# GEMM converting x itself, plus its recomputation launch).

def _ws(torch, ql, bits, M, N, K):
    return torch.empty(max(ql.qlinear_workspace_bytes(bits, M, N, K), 16), dtype=torch.uint8, device="cuda")


def case_gemm(torch, ql, inputs, M, N, K, bits, wid, xs="normal", entry="auto_tiled", copies=1, mode=None):
    """entry: auto_tiled / auto_canonical (qlinear_forward_ex with a workspace),
    the benchmark spec (qlinear_forward, canonical, no workspace), split_tiled /
    split_canonical (SPLIT, no workspace), exact_tiled / exact_canonical (EXACT
    with a workspace)."""
    tiled = entry in ("auto_tiled", "split_tiled", "exact_tiled")
    sets = make_weights(torch, ql, inputs, N, K, bits, wid, copies, tiled=tiled)
    x = torch.from_numpy(inputs.activations_bf16(M, K, wid, xs).view("int16")).cuda()
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ws = _ws(torch, ql, bits, M, N, K)
    layout = ql.QL_LAYOUT_TILED if tiled else ql.QL_LAYOUT_CANONICAL
    kw = {}
    if entry.startswith("exact"):
        kw["mode"] = ql.QL_MODE_EXACT
    if entry.startswith("split"):
        kw["mode"] = ql.QL_MODE_SPLIT
    if mode is not None:
        kw["mode"] = mode
    i = [0]

    def call():
        p, s, b = sets[i[0] % copies]
        i[0] += 1
        if entry == "north_star":
            ql.qlinear_forward(x, p, s, b, bits, 64, M, N, K, out)
        else:
            ql.qlinear_forward_ex(x, p, s, b, bits, M, N, K, out, layout=layout,
                                  workspace=None if entry.startswith("split") else ws, **kw)

    return call, {"flop": 2.0 * M * N * K, "weight_copies_rotated": copies}


def case_skinny(torch, ql, inputs, M, N, K, bits, wid, tiled, copies):
    sets = make_weights(torch, ql, inputs, N, K, bits, wid, copies, tiled=tiled)
    x = torch.from_numpy(inputs.activations_bf16(M, K, wid).view("int16")).cuda()
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    layout = ql.QL_LAYOUT_TILED if tiled else ql.QL_LAYOUT_CANONICAL
    i = [0]

    def call():
        p, s, b = sets[i[0] % copies]
        i[0] += 1
        ql.qlinear_forward_ex(x, p, s, b, bits, M, N, K, out, layout=layout, workspace=None)

    return call, {"bytes": algorithmic_bytes(M, N, K, bits), "weight_copies_rotated": copies}


SKINNY_COPIES = 8     # 8 x >= 56 MB of distinct weights > the 256 MB Infinity Cache
COND_COPIES = 4       # 4 x 138 MB of llm_cond_proj weights

# name -> (builder, kwargs, note)
CASES = {
    # the headline shape through the other entry points and numerics
    "north_star_M4096_K4608_N4608_q4": (case_gemm, dict(M=4096, N=4608, K=4608, bits=4, wid=6, entry="north_star"),
                                        "qlinear_forward: canonical weights, no workspace (FAST GEMM converting x)"),
    "split_canonical_M4096_K4608_N4608_q4": (case_gemm, dict(M=4096, N=4608, K=4608, bits=4, wid=6,
                                                              entry="split_canonical"),
                                             "SPLIT GEMM on canonical weights, no workspace"),
    "split_tiled_M4096_K4608_N4608_q4": (case_gemm, dict(M=4096, N=4608, K=4608, bits=4, wid=6, entry="split_tiled"),
                                         "SPLIT GEMM on tiled weights, no workspace"),
    "fast_canonical_M4096_K4608_N4608_q4": (case_gemm, dict(M=4096, N=4608, K=4608, bits=4, wid=6,
                                                             entry="auto_canonical"),
                                            "canonical weights with a workspace: prepass + FAST GEMM on the code rows"),
    "exact_tiled_M4096_K4608_N4608_q4": (case_gemm, dict(M=4096, N=4608, K=4608, bits=4, wid=6, entry="exact_tiled"),
                                         "EXACT: group sums + exact-integer bf16 MFMA GEMM"),
    "exact_canonical_M4096_K4608_N4608_q4": (case_gemm, dict(M=4096, N=4608, K=4608, bits=4, wid=6,
                                                              entry="exact_canonical"),
                                             "EXACT on the canonical code rows"),
    # QKV projection at 1024^2 (outlier channels)
    "qkv_M4608_K4608_N13824_q4": (case_gemm, dict(M=4608, N=13824, K=4608, bits=4, wid=2, xs="outlier"),
                                  "prepass + FAST GEMM, tiled"),
    "qkv_north_star_M4608_K4608_N13824_q4": (case_gemm, dict(M=4608, N=13824, K=4608, bits=4, wid=2, xs="outlier",
                                                              entry="north_star"),
                                             "qlinear_forward (FAST GEMM converting x)"),
    # SwiGLU MLP at 1024^2: gate/up (8-bit and 4-bit) and down (4- and 8-bit)
    "mlp_gateup_M4608_K4608_N24576_q8": (case_gemm, dict(M=4608, N=24576, K=4608, bits=8, wid=3),
                                         "prepass + FAST GEMM, tiled"),
    "mlp_gateup_M4608_K4608_N24576_q4": (case_gemm, dict(M=4608, N=24576, K=4608, bits=4, wid=3),
                                         "prepass + FAST GEMM, tiled"),
    "mlp_down_M4608_K12288_N4608_q4": (case_gemm, dict(M=4608, N=4608, K=12288, bits=4, wid=30),
                                       "prepass + FAST GEMM, tiled"),
    "mlp_down_M4608_K12288_N4608_q8": (case_gemm, dict(M=4608, N=4608, K=12288, bits=8, wid=30),
                                       "prepass + FAST GEMM, tiled"),
    # text conditioning: long K, few tiles
    "llm_cond_proj_M512_K53248_N4608_q4_canonical": (
        case_gemm, dict(M=512, N=4608, K=53248, bits=4, wid=4, xs="slices", entry="auto_canonical", copies=COND_COPIES),
        "canonical weights with a workspace: prepass + FAST GEMM split along K + ordered reduce"),
    "llm_cond_proj_M512_K53248_N4608_q4_tiled": (
        case_gemm, dict(M=512, N=4608, K=53248, bits=4, wid=4, xs="slices", copies=COND_COPIES),
        "tiled, prepass + FAST GEMM split along K + ordered reduce"),
    "llm_cond_proj_M512_K53248_N4608_q4_canonical_exact": (
        case_gemm, dict(M=512, N=4608, K=53248, bits=4, wid=4, xs="slices", entry="exact_canonical",
                        copies=COND_COPIES),
        "EXACT on the canonical code rows, split along K"),
    "llm_cond_proj_M512_K53248_N4608_q4_north_star": (
        case_gemm, dict(M=512, N=4608, K=53248, bits=4, wid=4, xs="slices", entry="north_star", copies=COND_COPIES),
        "qlinear_forward: no workspace, so no K split (FAST GEMM converting x, in row pieces)"),
    # AdaLN / timestep projections (skinny path, HBM-bound)
    "adaln_skinny_M1_K4608_N27648_q4_tiled": (case_skinny, dict(M=1, N=27648, K=4608, bits=4, wid=40, tiled=True,
                                                                copies=SKINNY_COPIES), ""),
    "adaln_skinny_M1_K4608_N27648_q4_canonical": (case_skinny, dict(M=1, N=27648, K=4608, bits=4, wid=40, tiled=False,
                                                                    copies=SKINNY_COPIES), ""),
    "adaln_skinny_M8_K4608_N27648_q4_tiled": (case_skinny, dict(M=8, N=27648, K=4608, bits=4, wid=41, tiled=True,
                                                                copies=SKINNY_COPIES), ""),
    "adaln_skinny_M8_K4608_N27648_q4_canonical": (case_skinny, dict(M=8, N=27648, K=4608, bits=4, wid=41, tiled=False,
                                                                    copies=SKINNY_COPIES), ""),
    "adaln_skinny_M1_K4608_N27648_q8_tiled": (case_skinny, dict(M=1, N=27648, K=4608, bits=8, wid=40, tiled=True,
                                                                copies=SKINNY_COPIES), ""),
    "adaln_skinny_M1_K512_N27648_q4_tiled": (case_skinny, dict(M=1, N=27648, K=512, bits=4, wid=42, tiled=True,
                                                               copies=40),
                                             "the pages' AdaLN width (512) as input: informational"),
    "adaln_skinny_M1_K512_N27648_q8_tiled": (case_skinny, dict(M=1, N=27648, K=512, bits=8, wid=42, tiled=True,
                                                               copies=24),
                                             "8-bit modulation (the mixed plans' width) at the pages' AdaLN width"),
}


CASE_SETTLE_S = 0.2   # calls per case before its timed calls, while the clock settles


def run_case(torch, ql, inputs, name, iters=20, warmup=5):
    builder, kw, note = CASES[name]
    call, meta = builder(torch, ql, inputs, **kw)
    ms = time_calls(torch, call, iters, warmup, CASE_SETTLE_S)
    row = {"path": ql.qlinear_last_path(), "us": round(ms * 1e3, 2)}
    if "flop" in meta:
        tf = meta["flop"] / (ms * 1e-3) / 1e12
        row.update({"TFLOP/s": round(tf, 1), "frac_mfma": round(tf / PEAK_F16_TFLOPS, 4)})
    else:
        gbs = meta["bytes"] / (ms * 1e-3) / 1e9
        row.update({"GB/s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)})
    if meta.get("weight_copies_rotated", 1) > 1:
        row["weight_copies_rotated"] = meta["weight_copies_rotated"]
    if note:
        row["note"] = note
    return row


def fused_epilogue_rows(torch, ql, inputs, rows):
    # SwiGLU MLP gate/up at 1024x1024: plain FAST GEMM (fp32 y, [M, 2F]) against
    # the fused epilogue (bf16 silu(gate) * up, [M, F])
    M, K, N = 4608, 4608, 2 * 12288
    (tq, tsb, _), = make_weights(torch, ql, inputs, N, K, 4, 3, tiled=True, glu=True)
    x = torch.from_numpy(inputs.activations_bf16(M, K, 3).view("int16")).cuda()
    ws = _ws(torch, ql, 4, M, N, K)
    yg = torch.empty((M, N // 2), dtype=torch.bfloat16, device="cuda")
    ms = time_calls(torch, lambda: ql.qlinear_forward_ex(
        x, tq, tsb, None, 4, M, N, K, yg, layout=ql.QL_LAYOUT_TILED, epilogue=ql.QL_EPI_SWIGLU, workspace=ws), 10, 3,
        CASE_SETTLE_S)
    tf = 2 * M * N * K / (ms * 1e-3) / 1e12
    rows["mlp_gateup_M4608_K4608_N24576_q4_swiglu_fused"] = {
        "path": ql.qlinear_last_path(), "us": round(ms * 1e3, 1), "TFLOP/s": round(tf, 1),
        "frac_mfma": round(tf / PEAK_F16_TFLOPS, 4), "out_bytes": M * (N // 2) * 2,
        "note": "prepass + FAST GEMM with silu(gate) * up in the store, bf16 [M, F]"}
    del tq, tsb, x, ws, yg

    # attention-out projection at 1024x1024 (2 samples of 2304 tokens) with the
    # AdaLN gated residual update: GEMM + a separate torch update of the
    # residual stream, against the update fused into the GEMM store
    M, K, N, L = 4608, 4608, 4608, 2304
    (tq, tsb, _), = make_weights(torch, ql, inputs, N, K, 4, 7, tiled=True)
    x = torch.from_numpy(inputs.activations_bf16(M, K, 7).view("int16")).cuda()
    ws = _ws(torch, ql, 4, M, N, K)
    res = torch.from_numpy(inputs.residual_stream(M, N, 7)).cuda()
    gate = torch.from_numpy(inputs.adaln_gate(M // L, N, 7)).cuda()
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")

    def unfused():
        ql.qlinear_forward_ex(x, tq, tsb, None, 4, M, N, K, y, layout=ql.QL_LAYOUT_TILED, workspace=ws)
        res.view(M // L, L, N).addcmul_(gate[:, None, :], y.view(M // L, L, N))

    def fused():
        ql.qlinear_forward_ex(x, tq, tsb, None, 4, M, N, K, res, layout=ql.QL_LAYOUT_TILED, workspace=ws,
                              epilogue=ql.QL_EPI_GATE_RESIDUAL, residual=res, gate=gate, gate_rows=L)

    ms_unf = time_calls(torch, unfused, 20, 5, CASE_SETTLE_S)
    ms_fused = time_calls(torch, fused, 20, 5, CASE_SETTLE_S)
    flop = 2 * M * N * K
    rows["attn_out_M4608_K4608_N4608_q4_gate_unfused"] = {
        "path": "prepass + FAST GEMM + torch addcmul_ on the residual", "us": round(ms_unf * 1e3, 1),
        "TFLOP/s": round(flop / (ms_unf * 1e-3) / 1e12, 1)}
    rows["attn_out_M4608_K4608_N4608_q4_gate_fused"] = {
        "path": ql.qlinear_last_path(), "us": round(ms_fused * 1e3, 1),
        "TFLOP/s": round(flop / (ms_fused * 1e-3) / 1e12, 1),
        "frac_mfma": round(flop / (ms_fused * 1e-3) / 1e12 / PEAK_F16_TFLOPS, 4),
        "note": "residual updated in place: out = residual + gate[sample] * y"}
    log(f"gate/up + SwiGLU {rows['mlp_gateup_M4608_K4608_N24576_q4_swiglu_fused']['us']} us; "
        f"attn-out + gate: unfused {ms_unf*1e3:.1f} us, fused {ms_fused*1e3:.1f} us")


def sweep_rows(torch, ql, inputs, rows):
    # 2048x2048 canvas: per-bit layer sweep, and one pass over the 34 blocks'
    # attention projections (QKV N=13824 then out N=4608) with 34 distinct
    # weight sets per width (every launch streams its weights); fp16
    # activations made once per pass and shared by its 68 projections
    M, K = 16896, 4608
    x = torch.from_numpy(inputs.activations_bf16(M, K, 5).view("int16")).cuda()
    x16, rs = ql.qlinear_fast_activations(x, M, K)
    ws = _ws(torch, ql, 8, M, 13824, K)
    for bits in (2, 3, 4, 8):
        layers = []
        for N in (13824, 4608):
            (p, s, b), = make_weights(torch, ql, inputs, N, K, bits, 5 if N == 4608 else 50)
            sets = [ql.qlinear_repack(p, s, b, bits, 64, N, K) for _ in range(34)]
            del p, s, b
            out = torch.empty((M, N), dtype=torch.float32, device="cuda")
            layers.append((N, sets, out))
            tq, tsb = sets[0]
            ms = time_calls(torch, lambda: ql.qlinear_forward_ex(
                x, tq, tsb, None, bits, M, N, K, out, layout=ql.QL_LAYOUT_TILED, x16=x16, rowscale=rs,
                workspace=ws), 10, 3, CASE_SETTLE_S)
            tf = 2 * M * N * K / (ms * 1e-3) / 1e12
            rows[f"sweep_2048_M{M}_K{K}_N{N}_q{bits}"] = {
                "path": ql.qlinear_last_path(), "us": round(ms * 1e3, 1), "TFLOP/s": round(tf, 1),
                "frac_mfma": round(tf / PEAK_F16_TFLOPS, 4), "note": "FAST GEMM on shared fp16 activations"}

        def one_pass():
            ql.qlinear_fast_activations(x, M, K, x16, rs)
            for i in range(34):
                for N, sets, out in layers:
                    tq, tsb = sets[i]
                    ql.qlinear_forward_ex(x, tq, tsb, None, bits, M, N, K, out, layout=ql.QL_LAYOUT_TILED,
                                          x16=x16, rowscale=rs, workspace=ws)

        ms = time_calls(torch, one_pass, 3, 1)
        flop = 34 * sum(2 * M * N * K for N, _, _ in layers)
        tf = flop / (ms * 1e-3) / 1e12
        rows[f"sweep_2048_34_layer_qkv_out_pass_q{bits}"] = {
            "ms": round(ms, 2), "TFLOP/s": round(tf, 1), "frac_mfma": round(tf / PEAK_F16_TFLOPS, 4),
            "weight_sets": 34,
            "note": "one prepass + 34 x (QKV 16896x4608->13824 + out 16896x4608->4608)"}
        log(f"2048 sweep q{bits}: 34-layer pass {ms:.2f} ms")
        del layers
    del x, x16, rs, ws


def dit_block_rows(torch, ql, inputs, rows):
    # one DiT block at 1024x1024 (4608 tokens) under the mixed-precision plans:
    # modulation (skinny, M=1, 8-bit), QKV, attention-out + gated residual,
    # gate/up + fused SwiGLU (bf16), down (fed by the SwiGLU output) + gated
    # residual, at the plan's bulk width; fp16 activations made per projection
    from group_wise_affine_qlinear_amd import plan as qplan
    M = 4608
    projs = {p.role: p for p in qplan.block_projections("mixed_4_8")}
    wf = {r: torch.from_numpy(inputs.weights(p.N, p.K, 80 + i)).cuda() for i, (r, p) in enumerate(projs.items())}
    x = torch.from_numpy(inputs.activations_bf16(M, 4608, 81).view("int16")).cuda()
    att = torch.from_numpy(inputs.activations_bf16(M, 4608, 82).view("int16")).cuda()
    temb = torch.from_numpy(inputs.activations_bf16(1, qplan.ADALN, 83).view("int16")).cuda()
    res = torch.from_numpy(inputs.residual_stream(M, 4608, 84)).cuda()
    gates = torch.from_numpy(inputs.adaln_gate(2, 4608, 85)).cuda()
    g_attn, g_mlp = gates[0:1].contiguous(), gates[1:2].contiguous()
    qkv = torch.empty((M, 3 * 4608), dtype=torch.bfloat16, device="cuda")
    hmid = torch.empty((M, 12288), dtype=torch.bfloat16, device="cuda")
    mod = torch.empty((1, 6 * 4608), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(ql.qlinear_workspace_bytes(8, M, 2 * 12288, 12288), 16), dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    for policy in ("mixed_3_8", "mixed_4_8"):
        wts = {}
        for p in qplan.block_projections(policy):
            pq = torch.empty((p.N, p.K * p.bits // 32), dtype=torch.int32, device="cuda")
            ps = torch.empty((p.N, p.K // 64), dtype=torch.int16, device="cuda")
            pb = torch.empty((p.N, p.K // 64), dtype=torch.int16, device="cuda")
            ql.qlinear_quantize_rtn(wf[p.role], p.bits, 64, p.N, p.K, pq, ps, pb, status)
            if p.role == "mlp_gate_up":
                tq, tsb = ql.qlinear_repack_glu(pq, ps, pb, p.bits, 64, p.N, p.K)
            else:
                tq, tsb = ql.qlinear_repack(pq, ps, pb, p.bits, 64, p.N, p.K)
            wts[p.role] = (tq, tsb, p)
            del pq, ps, pb
        torch.cuda.synchronize()
        if int(status.item()) != 0:
            raise RuntimeError("quantizer reported a range error")

        def proj(role, xin, out, **kw):
            tq, tsb, p = wts[role]
            ql.qlinear_forward_ex(xin, tq, tsb, None, p.bits, xin.shape[0], p.N, p.K, out,
                                  layout=ql.QL_LAYOUT_TILED, workspace=ws, **kw)

        def block():
            proj("adaln_modulation", temb, mod)
            proj("attn_qkv", x, qkv)
            proj("attn_out", att, res, epilogue=ql.QL_EPI_GATE_RESIDUAL, residual=res, gate=g_attn, gate_rows=M)
            proj("mlp_gate_up", x, hmid, epilogue=ql.QL_EPI_SWIGLU)
            proj("mlp_down", hmid, res, epilogue=ql.QL_EPI_GATE_RESIDUAL, residual=res, gate=g_mlp, gate_rows=M)

        ms = time_calls(torch, block, 10, 3, CASE_SETTLE_S)
        blk = qplan.block_projections(policy)
        flops = sum(2 * (1 if p.role == "adaln_modulation" else M) * p.N * p.K for p in blk)
        tf = flops / (ms * 1e-3) / 1e12
        rows[f"dit_block_1024_{policy}"] = {
            "us": round(ms * 1e3, 1), "TFLOP/s": round(tf, 1), "frac_mfma": round(tf / PEAK_F16_TFLOPS, 4),
            "weight_MB": round(sum(p.storage_bytes for p in blk) / 1e6, 1),
            "bits_per_weight_model": round(qplan.bits_per_weight(qplan.model_plan(policy)), 3),
            "note": "modulation M=1 8-bit skinny; QKV, out+gate, gate/up+SwiGLU, down+gate at the bulk width"}
        log(f"DiT block {policy}: {ms*1e3:.1f} us")
        del wts
    del wf, x, att, temb, res, gates, qkv, hmid, mod, ws


def dense_library_rows(torch, rows):
    # context, not this library's path: the vendor's dense GEMM (torch.matmul,
    # hipBLASLt) on unquantized fp16 and bf16 operands of the same shapes,
    # y = x @ W^T with fp32 accumulation; it reads 16-bit weights (4x the
    # 4-bit codes' bytes) and dequantizes nothing
    for (M, N, K) in ((4096, 4608, 4608), (4608, 13824, 4608)):
        for name, dt in (("fp16", torch.float16), ("bf16", torch.bfloat16)):
            x = torch.randn(M, K, device="cuda", dtype=dt)
            wt = torch.randn(N, K, device="cuda", dtype=dt).t()
            ms = time_calls(torch, lambda: x @ wt, 20, 5, CASE_SETTLE_S)
            tf = 2 * M * N * K / (ms * 1e-3) / 1e12
            rows[f"context_dense_library_{name}_M{M}_K{K}_N{N}"] = {
                "us": round(ms * 1e3, 1), "TFLOP/s": round(tf, 1), "frac_mfma": round(tf / PEAK_F16_TFLOPS, 4),
                "note": f"context only: torch.matmul (hipBLASLt) on dense {name} operands, not the quantized path"}
            log(f"dense library {name} {M}x{K}->{N}: {ms*1e3:.1f} us ({100*tf/PEAK_F16_TFLOPS:.1f}%)")
            del x, wt


def secondary_rows(torch, ql, inputs):
    rows = {}
    for name in CASES:
        rows[name] = run_case(torch, ql, inputs, name)
        r = rows[name]
        rate = f"{r['TFLOP/s']} TFLOP/s ({100 * r['frac_mfma']:.1f}%)" if "TFLOP/s" in r else \
            f"{r['GB/s']} GB/s ({100 * r['frac_hbm']:.1f}%)"
        log(f"{name}: {r['us']} us, {rate}, {r['path']}")
        torch.cuda.empty_cache()
    fused_epilogue_rows(torch, ql, inputs, rows)
    torch.cuda.empty_cache()
    dit_block_rows(torch, ql, inputs, rows)
    torch.cuda.empty_cache()
    sweep_rows(torch, ql, inputs, rows)
    torch.cuda.empty_cache()
    dense_library_rows(torch, rows)
    torch.cuda.empty_cache()
    return rows


# ------------------------------------------------------------------ the oracle on this host

def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [0])
    except Exception:
        return 0


def cpu_baseline(inputs, M, N, K, bits, wid):
    """The oracle as it stands, timed on this host over the full headline workload."""
    import oracle
    w = inputs.weights(N, K, wid)
    q, s16, b16 = oracle.quantize_rtn(w, bits)
    packed = oracle.pack(q, bits)
    x = inputs.activations_bf16(M, K, wid)
    del w, q
    _, t = oracle.timed_forward(x, packed, s16, b16, bits, K)
    tf = 2 * M * N * K / t["total_s"] / 1e12
    return {"value": round(tf, 4), "unit": "TFLOP/s", "cores": _CORES, "kind": "oracle",
            "blas_threads": _blas_threads(), "openblas_num_threads": os.environ.get("OPENBLAS_NUM_THREADS"),
            "sample": f"full workload M={M} K={K} N={N} q{bits}, one run: unpack+dequantize "
                      f"{t['dequant_s']:.2f} s + fp64 GEMM {t['gemm_s']:.2f} s"}


def cpu_oracle_per_config(inputs):
    """The oracle on every configured workload: the whole weight (unpack +
    dequantize) and the fp64 product on a sample of at most 512 rows of x,
    one run each (median of 3 for the tiny and skinny ones); throughput of
    the sample and the full workload's time extrapolated linearly in M."""
    import oracle
    out = {}
    for name, wl in inputs.WORKLOADS.items():
        M, K, N = wl["M"], wl["K"], wl["N"]
        bits = wl["bits"][0]
        m = min(M, 512)
        w = inputs.weights(N, K, wl["id"])
        q, s16, b16 = oracle.quantize_rtn(w, bits)
        packed = oracle.pack(q, bits)
        x = inputs.activations_bf16(m, K, wl["id"], wl["x"])
        del w, q
        reps = 3 if M <= 64 else 1
        runs = sorted((oracle.timed_forward(x, packed, s16, b16, bits, K)[1] for _ in range(reps)),
                      key=lambda t: t["total_s"])
        t = runs[len(runs) // 2]
        full_s = t["dequant_s"] + t["gemm_s"] * M / m
        out[name] = {"bits": bits, "rows_timed": m, "M": M, "dequant_s": round(t["dequant_s"], 3),
                     "gemm_s": round(t["gemm_s"], 3),
                     "sample_TFLOP/s": round(2 * m * N * K / t["total_s"] / 1e12, 4),
                     "full_workload_s_extrapolated": round(full_s, 3)}
        log(f"oracle {name}: {out[name]}")
    return {"cores": _CORES, "blas_threads": _blas_threads(), "workloads": out}


def load_traffic(src_hash):
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha") != src_hash:
        return None
    return rec.get("traffic_bytes_per_launch")


# EXACT-mode GEMM tiles (gemm.hip / gemm2.hip ids) and the shapes the
# automatic table is chosen on: (label, M, N, K, bits, weight id)
SWEEP_TILES = (1, 2, 3, 5, 10, 11)
SWEEP_SHAPES = (
    ("square_M256_K4608_N4608_q4", 256, 4608, 4608, 4, 6),
    ("square_M4096_K4608_N4608_q4", 4096, 4608, 4608, 4, 6),
    ("qkv_M4608_K4608_N13824_q4", 4608, 13824, 4608, 4, 2),
    ("mlp_gateup_M4608_K4608_N24576_q8", 4608, 24576, 4608, 8, 3),
    ("mlp_down_M4608_K12288_N4608_q8", 4608, 4608, 12288, 8, 30),
    ("mlp_down_M4608_K12288_N4608_q4", 4608, 4608, 12288, 4, 30),
    ("llm_cond_proj_M512_K53248_N4608_q4", 512, 4608, 53248, 4, 4),
    ("sweep_2048_M16896_K4608_N13824_q2", 16896, 13824, 4608, 2, 50),
)


def sweep_tiles(torch, ql, inputs):
    """Every EXACT tile on every sweep shape (canonical weights, a workspace,
    the automatic K split), 10 timed calls after 0.1 s of settling; one JSON
    line per shape with the times and the fastest tile, which is what the
    library's EXACT tile table encodes."""
    for label, M, N, K, bits, wid in SWEEP_SHAPES:
        (p, s, b), = make_weights(torch, ql, inputs, N, K, bits, wid)
        x = torch.from_numpy(inputs.activations_bf16(M, K, wid).view("int16")).cuda()
        out = torch.empty((M, N), dtype=torch.float32, device="cuda")
        ws = _ws(torch, ql, bits, M, N, K)
        times = {}
        ql.qlinear_forward_ex(x, p, s, b, bits, M, N, K, out, layout=ql.QL_LAYOUT_CANONICAL, workspace=ws,
                              mode=ql.QL_MODE_EXACT)
        auto_path = ql.qlinear_last_path()
        for tile in SWEEP_TILES:
            def call(tile=tile):
                ql.qlinear_forward_ex(x, p, s, b, bits, M, N, K, out, layout=ql.QL_LAYOUT_CANONICAL,
                                      workspace=ws, mode=ql.QL_MODE_EXACT, tile=tile)
            try:
                call()
            except RuntimeError:
                continue   # the tile cannot serve this shape or width
            times[tile] = round(time_calls(torch, call, 10, 2, 0.1) * 1e3, 1)
        best = min(times, key=times.get)
        print(json.dumps({"sweep": label, "us_by_tile": times, "fastest_tile": best, "auto_path": auto_path}),
              flush=True)
        del p, s, b, x, out, ws
        torch.cuda.empty_cache()


PROFILE_CHOICES = ["none", "step", "copy"] + sorted(CASES)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--profile", choices=PROFILE_CHOICES, default="none",
                    help="short run for rocprofv3: 'step' = the timed step only, 'copy' = a plain copy of known "
                         "size, a secondary case name = that case's launches only")
    ap.add_argument("--profile-calls", type=int, default=40)
    ap.add_argument("--sweep-tiles", action="store_true",
                    help="time every EXACT-mode tile on the configured shapes (one JSON line per shape) and exit")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; the multi-GPU layout is "
                                   "a design note, so --gpus must be 1"}))
        sys.exit(2)

    import torch
    from group_wise_affine_qlinear_amd import inputs
    from group_wise_affine_qlinear_amd import qlinear as ql

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    ql.load_library()

    if args.sweep_tiles:
        sweep_tiles(torch, ql, inputs)
        return
    if args.profile == "copy":
        n = 256 * 1024 * 1024 // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        log(f"copy kernel: {n * 4} bytes read and written per launch, 5 launches")
        return
    if args.profile in CASES:
        # calls while the clock settles (as the timed rows do), then the
        # profiled calls: the last --profile-calls dispatches of the trace
        builder, kw, _ = CASES[args.profile]
        call, _ = builder(torch, ql, inputs, **kw)
        torch.cuda.synchronize()
        t0, n_settle = time.perf_counter(), 0
        while time.perf_counter() - t0 < CASE_SETTLE_S:
            for _ in range(5):
                call()
            n_settle += 5
            torch.cuda.synchronize()
        for _ in range(args.profile_calls):
            call()
        torch.cuda.synchronize()
        log(f"{args.profile}: {n_settle} settling calls, then {args.profile_calls} profiled calls "
            f"({ql.qlinear_last_path()})")
        return

    M, K, N, bits = WORKLOAD["M"], WORKLOAD["K"], WORKLOAD["N"], WORKLOAD["bits"]
    # amd-smi only in the plain run (a profiler's preload would reach the child)
    smi = {"before_setup": smi_snapshot() if args.profile == "none" else None,
           "note": "single amd-smi metric readings, which lag a load of about a second; the engine clock "
                   "during the GEMM (GRBM_GUI_ACTIVE over the traced duration) is in the pipeline profile"}
    log(f"setup {WORKLOAD['name']}")
    (p, s, _), = make_weights(torch, ql, inputs, N, K, bits, WORKLOAD["wid"], tiled=True)
    x = torch.from_numpy(inputs.activations_bf16(M, K, WORKLOAD["wid"]).view("int16")).cuda()
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    x16 = torch.empty((M, K), dtype=torch.float16, device="cuda")
    rowscale = torch.empty((M,), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    steps, warmup = args.steps, args.warmup

    # HIP events around each GEMM launch (the roofline's kernel duration); the
    # prepass time is the step time minus the GEMM time. Events around the
    # prepass too would add a further marker per step to the timed region.
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]

    def step(evs=None):
        ql.qlinear_fast_activations(x, M, K, x16, rowscale, stream=stream)
        if evs:
            evs[0].record(stream)
        ql.qlinear_forward_ex(x, p, s, None, bits, M, N, K, out, layout=ql.QL_LAYOUT_TILED,
                              mode=ql.QL_MODE_FAST, x16=x16, rowscale=rowscale, stream=stream, workspace=None)
        if evs:
            evs[1].record(stream)

    # setup ends with SETTLE_S seconds of steps while the engine clock settles
    # under load (the first tens of steps after setup run up to 15 % slower);
    # then the W untimed warm-up steps and the K timed steps (a profiled run
    # does the same, so the last K dispatches of its trace are the timed ones)
    if args.profile in ("none", "step"):
        t_settle = time.perf_counter()
        while time.perf_counter() - t_settle < SETTLE_S:
            for _ in range(10):
                step()
            torch.cuda.synchronize()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(ev[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    path = ql.qlinear_last_path()
    if args.profile == "step":
        log(f"profiled {steps} steps, path {path}")
        return

    ms_step = (t1 - t0) * 1e3 / steps
    gemm_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
    # the rest of a step: prepass, launches and the event markers
    pre_ms = max(ms_step - gemm_ms, 0.0)
    flop = 2.0 * M * N * K
    value = flop / (ms_step * 1e-3) / 1e12
    achieved = flop / (gemm_ms * 1e-3) / 1e12
    log(f"step {ms_step*1e3:.1f} us (gemm {gemm_ms*1e3:.1f} us, prepass and the rest {pre_ms*1e3:.1f} us) -> {value:.1f} TFLOP/s")
    # distribution of the per-step event times, and a sustained ~1 s loop for
    # clock-throttling context (both after the timed region)
    per_step = sorted(a[1].elapsed_time(b[1]) * 1e3 for a, b in zip(ev[:-1], ev[1:]))   # GEMM end to GEMM end
    gemm_each = sorted(e[0].elapsed_time(e[1]) * 1e3 for e in ev)
    q = lambda v, f: round(v[min(len(v) - 1, int(f * len(v)))], 1) if v else None
    torch.cuda.synchronize()
    # amd-smi sampled from a side thread while the sustained loop runs; the
    # loop lasts at least 1 s and until the sample has returned
    sampler = threading.Thread(target=lambda: smi.__setitem__("during_sustained_loop", smi_snapshot()))
    n_sus, ts0 = 0, time.perf_counter()
    sampler.start()
    while time.perf_counter() - ts0 < 1.0 or (sampler.is_alive() and time.perf_counter() - ts0 < 30.0):
        for _ in range(20):
            step()
        n_sus += 20
        torch.cuda.synchronize()
    sus_ms = (time.perf_counter() - ts0) * 1e3 / n_sus
    sampler.join()
    timing = {"step_us_p10": q(per_step, 0.1), "step_us_median": q(per_step, 0.5), "step_us_p90": q(per_step, 0.9),
              "gemm_us_p10": q(gemm_each, 0.1), "gemm_us_median": q(gemm_each, 0.5),
              "gemm_us_p90": q(gemm_each, 0.9),
              "sustained_1s_step_us": round(sus_ms * 1e3, 1),
              "sustained_1s_TFLOP/s": round(flop / (sus_ms * 1e-3) / 1e12, 1), "sustained_steps": n_sus,
              "settle_s_before_warmup": SETTLE_S}
    log(f"per-step p10/median/p90 {timing['step_us_p10']}/{timing['step_us_median']}/{timing['step_us_p90']} us; "
        f"GEMM median {timing['gemm_us_median']} us; sustained 1 s: {timing['sustained_1s_step_us']} us per step")
    del x16, rowscale, out
    torch.cuda.empty_cache()

    secondary = {} if args.no_secondary else secondary_rows(torch, ql, inputs)
    src_hash = gemm_source_hash()
    traffic = load_traffic(src_hash)

    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD["name"], "M": M, "K": K, "N": N, "bits": bits, "group": 64,
                   "path": path, "mode": "fast", "layout": "tiled", "parallelism": "single-gpu"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_F16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_F16_TFLOPS, 4), "traffic": traffic,
                     "kernel": "fused dequant-GEMM (fp16 MFMA)", "kernel_us": round(gemm_ms * 1e3, 2),
                     "rest_of_step_us": round(pre_ms * 1e3, 2), "kernel_source_sha": src_hash},
        "timing": timing,
        "smi": smi,
        "secondary": secondary,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        rec["cpu_baseline"] = cpu_baseline(inputs, M, N, K, bits, WORKLOAD["wid"])
        rec["cpu_oracle_per_config"] = cpu_oracle_per_config(inputs)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
