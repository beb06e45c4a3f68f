#!/usr/bin/env python3
"""Benchmark of the group-wise affine quantized linear hot path on one MI355X.

One step = one pass of the path over one batch at the headline workload
M=4096 tokens, K=N=4608, 4-bit codes, group 64 (square projection of the
4608-wide DiT at 1024x1024): the activation prepass (qlinear_fast_activations:
bf16 x to fp16 with per-row power-of-two scales) followed by the fused
dequant-GEMM on tiled weights (qlinear_forward_ex, FAST mode), i.e. exactly the
kernels qlinear_forward_ex launches for this layer. Weights are quantized by the
library's device RTN quantizer and repacked to the tiled layout during setup, as
a loader does once per checkpoint; inputs are seeded synthetic tensors already
resident in HBM when the timed region starts.

Printed: one JSON line with the whole-job throughput (TFLOP/s), the roofline of
the dominant kernel (fused GEMM, timed live with HIP events on its stream), the
exact-mode, skinny-M and text-conditioning rows as secondary measurements, and
the CPU oracle timed on this host as a reported baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import subprocess
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "qlinear TFLOP/s (M=4096,K=N=4608, Q4 g64) + % MFMA peak; GB/s skinny-M"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_F16_TFLOPS = 2500.0      # MI355X dense fp16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
WORKLOAD = dict(name="dit_square_proj_M4096_K4608_N4608_q4_g64", M=4096, K=4608, N=4608, bits=4, wid=6)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm3_fast_q4_M4096_K4608_N4608_traffic.txt")


def log(msg):
    sys.stderr.write(f"[bench] {msg}\n")
    sys.stderr.flush()


def gemm_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("gemm3.hip", "ql_device.h"):
        with open(os.path.join(ROOT, "group_wise_affine_qlinear_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(M, N, K, bits):
    return N * K * bits / 8 + 4 * N * K / 64 + 2 * M * K + 4 * M * N


def make_weights(torch, ql, inputs, N, K, bits, wid, copies=1, tiled=False):
    """Device-quantized weight sets; tiled=True repacks each set for the GEMM kernels
    (then a set is (tiled_q, tiled_sb, None))."""
    w = torch.from_numpy(inputs.weights(N, K, wid)).cuda()
    sets = []
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    for _ in range(copies):
        p = torch.empty((N, K * bits // 32), dtype=torch.int32, device="cuda")
        s = torch.empty((N, K // 64), dtype=torch.int16, device="cuda")
        b = torch.empty((N, K // 64), dtype=torch.int16, device="cuda")
        ql.qlinear_quantize_rtn(w, bits, 64, N, K, p, s, b, status)
        if tiled:
            tq, tsb = ql.qlinear_repack(p, s, b, bits, 64, N, K)
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


def time_calls(torch, fn, iters, warmup):
    """Average per-call time (ms) with HIP events on the current stream."""
    for _ in range(warmup):
        fn()
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


def secondary_rows(torch, ql, inputs, exact_sets, x_main):
    rows = {}
    M, K, N, bits = WORKLOAD["M"], WORKLOAD["K"], WORKLOAD["N"], WORKLOAD["bits"]
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    p, s, _ = exact_sets

    def fe():
        ql.qlinear_forward_ex(x_main, p, s, None, bits, M, N, K, out, layout=ql.QL_LAYOUT_TILED,
                              mode=ql.QL_MODE_EXACT)

    ms = time_calls(torch, fe, 20, 5)
    tf = 2 * M * N * K / (ms * 1e-3) / 1e12
    rows[f"exact_mode_M{M}_K{K}_N{N}_q{bits}"] = {
        "path": ql.qlinear_last_path(), "us": round(ms * 1e3, 1), "TFLOP/s": round(tf, 1),
        "frac_mfma_bf16": round(tf / PEAK_BF16_TFLOPS, 4)}
    log(f"exact mode: {ms*1e3:.1f} us, {tf:.0f} TFLOP/s")

    # the plain entry point on canonical weights (EXACT numerics, library-owned workspace)
    (pc, sc, bc), = make_weights(torch, ql, inputs, N, K, bits, WORKLOAD["wid"])

    def fc():
        ql.qlinear_forward(x_main, pc, sc, bc, bits, 64, M, N, K, out)

    ms = time_calls(torch, fc, 20, 5)
    tf = 2 * M * N * K / (ms * 1e-3) / 1e12
    rows[f"canonical_entry_M{M}_K{K}_N{N}_q{bits}"] = {
        "path": ql.qlinear_last_path(), "us": round(ms * 1e3, 1), "TFLOP/s": round(tf, 1),
        "frac_mfma_bf16": round(tf / PEAK_BF16_TFLOPS, 4),
        "note": "qlinear_forward, canonical layout (automatic dispatch: tiled copy in the workspace, exact GEMM)"}
    log(f"canonical qlinear_forward: {ms*1e3:.1f} us, {tf:.0f} TFLOP/s ({ql.qlinear_last_path()})")

    # the same weights with the kernels forced onto the canonical code rows, and FAST numerics
    variants = (
        ("canonical_exact_direct", {"path": ql.QL_PATH_GEMM}, PEAK_BF16_TFLOPS,
         "exact GEMM reading the canonical code rows (forced GEMM path, no copy)"),
        ("canonical_fast", {"mode": ql.QL_MODE_FAST}, PEAK_F16_TFLOPS,
         "prepass + FAST GEMM, automatic dispatch (tiled copy in the workspace)"),
        ("canonical_fast_direct", {"mode": ql.QL_MODE_FAST, "path": ql.QL_PATH_GEMM}, PEAK_F16_TFLOPS,
         "prepass + FAST GEMM reading the canonical code rows (forced GEMM path, no copy)"),
    )
    for name, kw, peak, note in variants:
        def fv(kw=kw):
            ql.qlinear_forward_ex(x_main, pc, sc, bc, bits, M, N, K, out, **kw)

        ms = time_calls(torch, fv, 20, 5)
        tf = 2 * M * N * K / (ms * 1e-3) / 1e12
        rows[f"{name}_M{M}_K{K}_N{N}_q{bits}"] = {
            "path": ql.qlinear_last_path(), "us": round(ms * 1e3, 1), "TFLOP/s": round(tf, 1),
            "frac_mfma": round(tf / peak, 4), "note": note}
        log(f"{name}: {ms*1e3:.1f} us, {tf:.0f} TFLOP/s ({ql.qlinear_last_path()})")
    del out, pc, sc, bc

    K, N = 4608, 27648
    for M, bits, tiled in ((1, 4, False), (1, 4, True), (8, 4, False), (8, 4, True), (1, 8, True), (1, 3, True)):
        copies = 8  # 8 x >= 56 MB of distinct weights > 256 MB Infinity Cache
        sets = make_weights(torch, ql, inputs, N, K, bits, 40 + (M > 1), copies, tiled=tiled)
        x = torch.from_numpy(inputs.activations_bf16(M, K, 40 + (M > 1)).view("int16")).cuda()
        out = torch.empty((M, N), dtype=torch.float32, device="cuda")
        layout = ql.QL_LAYOUT_TILED if tiled else ql.QL_LAYOUT_CANONICAL
        i = [0]

        def fn():
            p, s, b = sets[i[0] % copies]
            i[0] += 1
            ql.qlinear_forward_ex(x, p, s, b, bits, M, N, K, out, layout=layout)

        ms = time_calls(torch, fn, 64, 16)
        by = algorithmic_bytes(M, N, K, bits)
        gbs = by / (ms * 1e-3) / 1e9
        lname = "tiled" if tiled else "canonical"
        rows[f"adaln_skinny_M{M}_K{K}_N{N}_q{bits}_{lname}"] = {
            "path": ql.qlinear_last_path(), "us": round(ms * 1e3, 2), "GB/s": round(gbs, 1),
            "frac_hbm": round(gbs / PEAK_HBM_GBS, 4), "weight_copies_rotated": copies}
        del sets
        log(f"skinny M={M} q{bits} {lname}: {ms*1e3:.1f} us, {gbs:.0f} GB/s")

    # SwiGLU MLP gate/up projection at 1024x1024: plain FAST GEMM (fp32 y, [M, 2F])
    # against the fused epilogue (bf16 silu(gate) * up, [M, F])
    M, K, N = 4608, 4608, 2 * 12288
    w = torch.from_numpy(inputs.weights(N, K, 3)).cuda()
    p = torch.empty((N, K // 8), dtype=torch.int32, device="cuda")
    s = torch.empty((N, K // 64), dtype=torch.int16, device="cuda")
    b = torch.empty((N, K // 64), dtype=torch.int16, device="cuda")
    ql.qlinear_quantize_rtn(w, 4, 64, N, K, p, s, b)
    del w
    tq, tsb = ql.qlinear_repack(p, s, b, 4, 64, N, K)
    gq, gsb = ql.qlinear_repack_glu(p, s, b, 4, 64, N, K)
    del p, s, b
    x = torch.from_numpy(inputs.activations_bf16(M, K, 3).view("int16")).cuda()
    x16, rs = ql.qlinear_fast_activations(x, M, K)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    yg = torch.empty((M, N // 2), dtype=torch.bfloat16, device="cuda")
    ms_plain = time_calls(torch, lambda: ql.qlinear_forward_ex(
        x, tq, tsb, None, 4, M, N, K, y, layout=ql.QL_LAYOUT_TILED, x16=x16, rowscale=rs), 10, 3)
    path_plain = ql.qlinear_last_path()
    ms_glu = time_calls(torch, lambda: ql.qlinear_forward_ex(
        x, gq, gsb, None, 4, M, N, K, yg, layout=ql.QL_LAYOUT_TILED, x16=x16, rowscale=rs,
        epilogue=ql.QL_EPI_SWIGLU), 10, 3)
    tf = 2 * M * N * K / 1e12
    rows["mlp_gateup_M4608_K4608_N24576_q4_fast"] = {
        "path": path_plain, "us": round(ms_plain * 1e3, 1), "TFLOP/s": round(tf / (ms_plain * 1e-3), 1),
        "out_bytes": M * N * 4}
    rows["mlp_gateup_M4608_K4608_N24576_q4_swiglu_fused"] = {
        "path": ql.qlinear_last_path(), "us": round(ms_glu * 1e3, 1), "TFLOP/s": round(tf / (ms_glu * 1e-3), 1),
        "out_bytes": M * (N // 2) * 2}
    log(f"gate/up plain {ms_plain*1e3:.1f} us, fused SwiGLU {ms_glu*1e3:.1f} us")
    del tq, tsb, gq, gsb, x, x16, rs, y, yg

    # attention-out projection at 1024x1024 (2 samples of 2304 tokens) with the
    # AdaLN gated residual update: plain FAST GEMM, GEMM + a separate torch
    # update of the residual stream, and the update fused into the GEMM store
    M, K, N, L = 4608, 4608, 4608, 2304
    w = torch.from_numpy(inputs.weights(N, K, 7)).cuda()
    p = torch.empty((N, K // 8), dtype=torch.int32, device="cuda")
    s = torch.empty((N, K // 64), dtype=torch.int16, device="cuda")
    b = torch.empty((N, K // 64), dtype=torch.int16, device="cuda")
    ql.qlinear_quantize_rtn(w, 4, 64, N, K, p, s, b)
    del w
    tq, tsb = ql.qlinear_repack(p, s, b, 4, 64, N, K)
    del p, s, b
    x = torch.from_numpy(inputs.activations_bf16(M, K, 7).view("int16")).cuda()
    x16, rs = ql.qlinear_fast_activations(x, M, K)
    res = torch.from_numpy(inputs.residual_stream(M, N, 7)).cuda()
    gate = torch.from_numpy(inputs.adaln_gate(M // L, N, 7)).cuda()
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")

    def plain():
        ql.qlinear_forward_ex(x, tq, tsb, None, 4, M, N, K, y, layout=ql.QL_LAYOUT_TILED, x16=x16, rowscale=rs)

    def unfused():
        plain()
        res.view(M // L, L, N).addcmul_(gate[:, None, :], y.view(M // L, L, N))

    def fused():
        ql.qlinear_forward_ex(x, tq, tsb, None, 4, M, N, K, res, layout=ql.QL_LAYOUT_TILED, x16=x16, rowscale=rs,
                              epilogue=ql.QL_EPI_GATE_RESIDUAL, residual=res, gate=gate, gate_rows=L)

    ms_plain = time_calls(torch, plain, 20, 5)
    ms_unf = time_calls(torch, unfused, 20, 5)
    ms_fused = time_calls(torch, fused, 20, 5)
    tf = 2 * M * N * K / 1e12
    rows["attn_out_M4608_K4608_N4608_q4_fast"] = {
        "path": "gemm3 (plain y)", "us": round(ms_plain * 1e3, 1), "TFLOP/s": round(tf / (ms_plain * 1e-3), 1)}
    rows["attn_out_M4608_K4608_N4608_q4_gate_unfused"] = {
        "path": "gemm3 + torch addcmul_ on the residual", "us": round(ms_unf * 1e3, 1),
        "TFLOP/s": round(tf / (ms_unf * 1e-3), 1)}
    rows["attn_out_M4608_K4608_N4608_q4_gate_fused"] = {
        "path": ql.qlinear_last_path(), "us": round(ms_fused * 1e3, 1), "TFLOP/s": round(tf / (ms_fused * 1e-3), 1),
        "note": "residual updated in place: out = residual + gate[sample] * y"}
    log(f"attn-out plain {ms_plain*1e3:.1f} us, unfused gate {ms_unf*1e3:.1f} us, fused gate {ms_fused*1e3:.1f} us")
    del tq, tsb, x, x16, rs, res, gate, y

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
                                  layout=ql.QL_LAYOUT_TILED, **kw)

        def block():
            proj("adaln_modulation", temb, mod)
            proj("attn_qkv", x, qkv)
            proj("attn_out", att, res, epilogue=ql.QL_EPI_GATE_RESIDUAL, residual=res, gate=g_attn, gate_rows=M)
            proj("mlp_gate_up", x, hmid, epilogue=ql.QL_EPI_SWIGLU)
            proj("mlp_down", hmid, res, epilogue=ql.QL_EPI_GATE_RESIDUAL, residual=res, gate=g_mlp, gate_rows=M)

        ms = time_calls(torch, block, 10, 3)
        blk = qplan.block_projections(policy)
        flops = sum(2 * (1 if p.role == "adaln_modulation" else M) * p.N * p.K for p in blk)
        rows[f"dit_block_1024_{policy}"] = {
            "us": round(ms * 1e3, 1), "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 1),
            "weight_MB": round(sum(p.storage_bytes for p in blk) / 1e6, 1),
            "bits_per_weight_model": round(qplan.bits_per_weight(qplan.model_plan(policy)), 3),
            "note": "modulation M=1 8-bit skinny; QKV, out+gate, gate/up+SwiGLU, down+gate at the bulk width"}
        log(f"DiT block {policy}: {ms*1e3:.1f} us")
        del wts
    del wf, x, att, temb, res, gates, qkv, hmid, mod

    # 2048x2048 canvas: per-bit layer sweep, and one pass over the 34 blocks'
    # attention projections (QKV N=13824 then out N=4608) with 34 distinct
    # weight sets per width (every launch streams its weights)
    M, K = 16896, 4608
    x = torch.from_numpy(inputs.activations_bf16(M, K, 5).view("int16")).cuda()
    x16, rs = ql.qlinear_fast_activations(x, M, K)
    for bits in (2, 3, 4, 8):
        layers = []
        for N in (13824, 4608):
            w = torch.from_numpy(inputs.weights(N, K, 5 if N == 4608 else 50)).cuda()
            p = torch.empty((N, K * bits // 32), dtype=torch.int32, device="cuda")
            s = torch.empty((N, K // 64), dtype=torch.int16, device="cuda")
            b = torch.empty((N, K // 64), dtype=torch.int16, device="cuda")
            ql.qlinear_quantize_rtn(w, bits, 64, N, K, p, s, b)
            del w
            sets = [ql.qlinear_repack(p, s, b, bits, 64, N, K) for _ in range(34)]
            del p, s, b
            out = torch.empty((M, N), dtype=torch.float32, device="cuda")
            layers.append((N, sets, out))
            tq, tsb = sets[0]
            ms = time_calls(torch, lambda: ql.qlinear_forward_ex(
                x, tq, tsb, None, bits, M, N, K, out, layout=ql.QL_LAYOUT_TILED, x16=x16, rowscale=rs), 10, 3)
            rows[f"sweep_2048_M{M}_K{K}_N{N}_q{bits}"] = {
                "path": ql.qlinear_last_path(), "us": round(ms * 1e3, 1),
                "TFLOP/s": round(2 * M * N * K / (ms * 1e-3) / 1e12, 1)}

        def one_pass():
            for i in range(34):
                for N, sets, out in layers:
                    tq, tsb = sets[i]
                    ql.qlinear_forward_ex(x, tq, tsb, None, bits, M, N, K, out, layout=ql.QL_LAYOUT_TILED,
                                          x16=x16, rowscale=rs)

        ms = time_calls(torch, one_pass, 3, 1)
        flop = 34 * sum(2 * M * N * K for N, _, _ in layers)
        rows[f"sweep_2048_34_layer_qkv_out_pass_q{bits}"] = {
            "ms": round(ms, 2), "TFLOP/s": round(flop / (ms * 1e-3) / 1e12, 1), "weight_sets": 34,
            "note": "34 x (QKV 16896x4608->13824 + out 16896x4608->4608), shared fp16 activations"}
        log(f"2048 sweep q{bits}: 34-layer pass {ms:.2f} ms")
        del layers
    del x, x16, rs

    M, K, N = 512, 53248, 4608
    copies = 4
    x = torch.from_numpy(inputs.activations_bf16(M, K, 4, "slices").view("int16")).cuda()
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    for tiled in (False, True):
        sets = make_weights(torch, ql, inputs, N, K, 4, 4, copies, tiled=tiled)
        layout = ql.QL_LAYOUT_TILED if tiled else ql.QL_LAYOUT_CANONICAL
        i = [0]

        def fn2():
            p, s, b = sets[i[0] % copies]
            i[0] += 1
            ql.qlinear_forward_ex(x, p, s, b, 4, M, N, K, out, layout=layout)

        ms = time_calls(torch, fn2, 20, 5)
        tf = 2 * M * N * K / (ms * 1e-3) / 1e12
        lname = "tiled" if tiled else "canonical"
        rows[f"llm_cond_proj_M512_K53248_N4608_q4_{lname}"] = {
            "path": ql.qlinear_last_path(), "us": round(ms * 1e3, 1), "TFLOP/s": round(tf, 1),
            "frac_mfma": round(tf / PEAK_BF16_TFLOPS, 4), "weight_copies_rotated": copies}
        log(f"llm_cond_proj {lname}: {ms*1e3:.1f} us, {tf:.0f} TFLOP/s")
        del sets
    del x, out

    # one GPU's share under two-way tensor parallelism at 1024x1024 (M = 4608):
    # column shards (QKV, gate/up: N halved, no exchange) and row shards
    # (attention-out, down: K halved, fp32 partial y for an all-reduce that is
    # not run here)
    M = 4608
    for name, K, N in (("qkv_col_shard", 4608, 6912), ("gateup_col_shard", 4608, 12288),
                       ("attn_out_row_shard", 2304, 4608), ("down_row_shard", 6144, 4608)):
        (p, s, _), = make_weights(torch, ql, inputs, N, K, 4, 8, tiled=True)
        x = torch.from_numpy(inputs.activations_bf16(M, K, 8).view("int16")).cuda()
        out = torch.empty((M, N), dtype=torch.float32, device="cuda")

        def fs():
            ql.qlinear_forward_ex(x, p, s, None, 4, M, N, K, out, layout=ql.QL_LAYOUT_TILED)

        ms = time_calls(torch, fs, 20, 5)
        tf = 2 * M * N * K / (ms * 1e-3) / 1e12
        rows[f"tp2_{name}_M{M}_K{K}_N{N}_q4"] = {
            "path": ql.qlinear_last_path(), "us": round(ms * 1e3, 1), "TFLOP/s": round(tf, 1),
            "frac_mfma": round(tf / PEAK_F16_TFLOPS, 4), "note": "prepass + FAST GEMM on one GPU's shard"}
        log(f"tp2 {name}: {ms*1e3:.1f} us, {tf:.0f} TFLOP/s")
        del p, s, x, out
    return rows


def cpu_baseline(inputs, M, N, K, bits, wid):
    """The oracle as it stands, timed on this host over the full headline workload."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    w = inputs.weights(N, K, wid)
    q, s16, b16 = oracle.quantize_rtn(w, bits)
    packed = oracle.pack(q, bits)
    x = inputs.activations_bf16(M, K, wid)
    del w, q
    _, t = oracle.timed_forward(x, packed, s16, b16, bits, K)
    tf = 2 * M * N * K / t["total_s"] / 1e12
    return {"value": round(tf, 4), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"full workload M={M} K={K} N={N} q{bits}, one run: unpack+dequantize "
                      f"{t['dequant_s']:.2f} s + fp64 GEMM {t['gemm_s']:.2f} s"}


def load_traffic(src_hash):
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha") != src_hash:
        return None
    return rec.get("traffic_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--profile", choices=["none", "step", "copy", "skinny"], default="none",
                    help="short run for rocprofv3: 'step' = the timed step only, 'copy' = a plain copy of known size, 'skinny' = the AdaLN skinny kernel")
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

    if args.profile == "skinny":
        # the skinny path at the AdaLN shape, M=1, tiled 4-bit weights, 8
        # distinct weight copies rotated so every launch streams from HBM
        M, K, N, copies = 1, 4608, 27648, 8
        sets = make_weights(torch, ql, inputs, N, K, 4, 40, copies, tiled=True)
        x = torch.from_numpy(inputs.activations_bf16(M, K, 40).view("int16")).cuda()
        out = torch.empty((M, N), dtype=torch.float32, device="cuda")
        for i in range(16 + 64):
            p, s, _ = sets[i % copies]
            ql.qlinear_forward_ex(x, p, s, None, 4, M, N, K, out, layout=ql.QL_LAYOUT_TILED)
        torch.cuda.synchronize()
        log(f"skinny M=1 K=4608 N=27648 q4 tiled: 80 launches ({ql.qlinear_last_path()})")
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
                              mode=ql.QL_MODE_FAST, x16=x16, rowscale=rowscale, stream=stream)
        if evs:
            evs[1].record(stream)

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
    q = lambda f: round(per_step[min(len(per_step) - 1, int(f * len(per_step)))], 1)
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
    timing = {"step_us_p10": q(0.1), "step_us_median": q(0.5), "step_us_p90": q(0.9),
              "sustained_1s_step_us": round(sus_ms * 1e3, 1),
              "sustained_1s_TFLOP/s": round(flop / (sus_ms * 1e-3) / 1e12, 1), "sustained_steps": n_sus}
    log(f"per-step p10/median/p90 {timing['step_us_p10']}/{timing['step_us_median']}/{timing['step_us_p90']} us; "
        f"sustained 1 s: {timing['sustained_1s_step_us']} us per step")

    secondary = {} if args.no_secondary else secondary_rows(torch, ql, inputs, (p, s, None), x)
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
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
