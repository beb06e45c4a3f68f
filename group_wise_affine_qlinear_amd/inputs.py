"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle checks.

This module draws random numbers and nothing else: it holds none of the
quantized-linear arithmetic (no fitting, packing, dequantizing or products), so
both the library's tests and the CPU oracle can take their inputs from it.

Shapes follow the projection layers of the Ideogram 4 single-stream DiT
(paper notes on jimmysue.github.io, section 2.8 model table and section 2.3
config: model width 4608, MLP width 12288, 13 text-encoder layers of width 4096
concatenated into 53248 features; section 2.1: 4096 image tokens at 1024x1024).

Distributions: weights N(0, 0.02^2) in fp32; activations N(0, 1) in fp32 then
rounded to bf16 (round-half-to-even). Optional structure: a seeded 1% of input
channels scaled by 20 before the bf16 cast (outlier channels), or per-4096-slice
standard deviations drawn from U[0.5, 4] (13 concatenated encoder layers).
AdaLN-gated residual updates: residual stream N(0, 1) in fp32; per-sample gate
values uniform in (-1, 1), the range of a tanh gate.
Every tensor has its own stream: SeedSequence([0, workload_id, role]).
"""
from __future__ import annotations

import numpy as np

ROLE_W = 1
ROLE_X = 2
ROLE_OUTLIER = 3
ROLE_SLICE = 4
ROLE_CODES = 5
ROLE_SCALE = 6
ROLE_BIAS = 7
ROLE_RESIDUAL = 8
ROLE_GATE = 9

# id, M, K, N, bits, x structure
WORKLOADS = {
    "tiny":            dict(id=1, M=64, K=512, N=256, bits=(4,), x="normal"),
    "qkv_1024":        dict(id=2, M=4608, K=4608, N=13824, bits=(4,), x="outlier"),
    "mlp_gateup_1024": dict(id=3, M=4608, K=4608, N=24576, bits=(4, 8), x="normal"),
    "mlp_down_1024":   dict(id=30, M=4608, K=12288, N=4608, bits=(4, 8), x="normal"),
    "llm_cond_proj":   dict(id=4, M=512, K=53248, N=4608, bits=(4,), x="slices"),
    "adaln_m1":        dict(id=40, M=1, K=4608, N=27648, bits=(4,), x="normal"),
    "adaln_m8":        dict(id=41, M=8, K=4608, N=27648, bits=(4,), x="normal"),
    "sweep_2048_n4608":  dict(id=5, M=16896, K=4608, N=4608, bits=(2, 4, 8), x="normal"),
    "sweep_2048_n13824": dict(id=50, M=16896, K=4608, N=13824, bits=(2, 4, 8), x="normal"),
    "square_4096":     dict(id=6, M=4096, K=4608, N=4608, bits=(4,), x="normal"),
}


def rng_for(workload_id: int, role: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([0, int(workload_id), int(role)]))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round-half-to-even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def weights(n: int, k: int, workload_id: int = 0, std: float = 0.02) -> np.ndarray:
    rng = rng_for(workload_id, ROLE_W)
    return (rng.standard_normal((n, k), dtype=np.float32) * np.float32(std)).astype(np.float32)


def activations_f32(m: int, k: int, workload_id: int = 0, structure: str = "normal") -> np.ndarray:
    rng = rng_for(workload_id, ROLE_X)
    x = rng.standard_normal((m, k), dtype=np.float32)
    if structure == "outlier":
        ch = rng_for(workload_id, ROLE_OUTLIER).permutation(k)[: int(0.01 * k)]
        x[:, ch] *= np.float32(20.0)
    elif structure == "slices":
        width = 4096
        nsl = k // width
        stds = rng_for(workload_id, ROLE_SLICE).uniform(0.5, 4.0, size=nsl).astype(np.float32)
        for i in range(nsl):
            x[:, i * width:(i + 1) * width] *= stds[i]
    elif structure != "normal":
        raise ValueError(structure)
    return x


def activations_bf16(m: int, k: int, workload_id: int = 0, structure: str = "normal") -> np.ndarray:
    return f32_to_bf16_bits(activations_f32(m, k, workload_id, structure))


def random_codes(n: int, k: int, bits: int, workload_id: int = 0) -> np.ndarray:
    rng = rng_for(workload_id, ROLE_CODES)
    return rng.integers(0, 1 << bits, size=(n, k), dtype=np.uint8)


def random_f16_bits(n: int, g: int, lo: float, hi: float, workload_id: int = 0, role: int = ROLE_SCALE) -> np.ndarray:
    """Uniform values in [lo, hi) cast to f16 bit patterns (test data only)."""
    rng = rng_for(workload_id, role)
    v = rng.uniform(lo, hi, size=(n, g)).astype(np.float32)
    return v.astype(np.float16).view(np.uint16)


def residual_stream(m: int, n: int, workload_id: int = 0) -> np.ndarray:
    """Residual stream [m, n], N(0, 1) in fp32."""
    return rng_for(workload_id, ROLE_RESIDUAL).standard_normal((m, n), dtype=np.float32)


def adaln_gate(samples: int, n: int, workload_id: int = 0) -> np.ndarray:
    """Per-sample gate rows [samples, n], uniform in (-1, 1) in fp32."""
    return rng_for(workload_id, ROLE_GATE).uniform(-1.0, 1.0, size=(samples, n)).astype(np.float32)


def workload_inputs(name: str, m: int | None = None):
    """(W fp32 [N, K], x bf16 bits [M, K]) for a named workload; M may be overridden."""
    wl = WORKLOADS[name]
    mm = wl["M"] if m is None else m
    w = weights(wl["N"], wl["K"], wl["id"])
    x = activations_bf16(mm, wl["K"], wl["id"], wl["x"])
    return w, x
