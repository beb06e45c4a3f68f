"""Plain, slow, obviously-correct CPU oracle for group-wise affine quantized linear.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py``; never by the library, and it imports
nothing from the library.

What it computes (sources are the pages' titles and sections):

* Format. Each run of 64 consecutive weights along K in one output row shares
  one f16 scale and one f16 bias; this overhead is what adds half a bit to each
  nominal width (Ideogram-4-IQ4_M model card, aimarketly.com, opening section on
  bits per weight). The grid is uniform affine (same card, section on what
  "IQ4" means), and the packed Q4/Q8 tensors use group size 64
  (SceneWorks/ideogram-4-mlx model card, huggingface.co, section "Versions").
  Dequantized weight: W_hat[n, k] = s[n, g] * q[n, k] + b[n, g], g = k // 64.
* Fit. Round-to-nearest from the group's min/max ("candidate 0", the card's
  section on what "IQ4" means; the OrbitQuant W2A4 card's quantization manifest
  names the same int4 RTN group-64 policy).
* Packing. The pages say only "packed". Reading taken: each row's codes form
  one little-endian bit stream along K, code k in stream bits
  [bits*k, bits*k + bits), stream bit i being bit i % 32 of uint32 word
  i // 32. For 2, 4 and 8 bits this puts 32/bits whole codes in each word
  (code k in bits [bits*(k % (32/bits)), +bits) of word k // (32/bits)); for
  3 bits (the 3-bit DiT bulk of the IQ4_M card's previous pack, section
  "Against the pack this replaces"; its layout is not given) a code may
  straddle two words, and every 64-wide group fills exactly 6 words.
* Product. y = x @ W_hat^T, x given as bf16, accumulated in float64.

Readings where the pages are silent (each also listed in the design notes):
min and max order -0 below +0; scale = (max - min) / (2**bits - 1) in fp32; both scale and bias rounded to f16
with round-half-even; q computed from the *stored* f16 scale and bias in fp32
(IEEE subtract and divide), rounded half-to-even, clamped to [0, 2**bits - 1];
a group whose f16 scale is zero gets q = 0; non-finite weights, or a scale or
bias that overflows f16, are rejected.

Every function here is pinned by ``tests/test_oracle.py`` to facts other than
itself (hand-worked examples, exact rational arithmetic, brute force, closed
forms, special cases).

The library's FAST mode is an approximation of the product above that the
pages do not describe; ``forward_fast`` writes out its definition (weights
rounded once to fp16, activations scaled per row by a power of two into
fp16) so the GPU path can be compared with it to fp32-accumulation accuracy,
while ``forward`` remains the reference for the error budget.

SwiGLU (the DiT block's MLP: Ideogram 4 paper notes, section 2.1 pipeline,
section 2.8 table "SwiGLU MLP"; the notes print no formula). Reading taken:
the standard gated form silu(x W_gate^T) * (x W_up^T) with silu(v) =
v / (1 + e^-v), the gate and up weights stacked as rows [gate; up] of one
projection. ``swiglu`` applies it to an exact product in float64.

AdaLN gate (Ideogram 4 paper notes, section 2.1 pipeline: each block takes an
AdaLN scale and gate from the timestep embedding; Ideogram-4-IQ4_M card,
Conversion section: the modulation projection emits a per-layer scale and a
tanh gate whose error multiplies the whole residual stream). Reading taken:
the gate (already through tanh) multiplies a branch's output projection
feature-wise, per sample, before it is added to the residual stream:
out[m, n] = residual[m, n] + gate[m // rows_per_sample, n] * y[m, n].
``gate_residual`` writes that out in float64.

AdaLN scale (the same two passages: the block's input is modulated by a
per-layer scale emitted from the timestep embedding; the pages name a scale
and a gate, no shift, and print no formula). Reading taken: the zero-centred
form, each input channel k of the rows of one sample multiplied by one plus
that sample's scale: x_mod[m, k] = x[m, k] * (1 + scale[m // rows_per_sample, k]).
``adaln_modulate`` writes it out in float64 and ``forward_modulated`` takes
the plain product of the modulated input with the dequantized weights.
"""
from __future__ import annotations

import math
import time

import numpy as np

__all__ = [
    "GROUP", "SUPPORTED_BITS", "check_bits", "codes_per_word", "words_per_row", "bits_per_weight",
    "storage_bytes",
    "f16_bits_to_f32", "f32_to_f16_bits", "bf16_bits_to_f64",
    "quantize_rtn", "pack", "unpack", "dequantize", "gemm_f64", "forward",
    "forward_rows", "error_metrics", "timed_forward",
    "fast_weights_f16", "fast_activations_f16", "forward_fast", "forward_fast_rows", "silu", "swiglu",
    "gate_residual", "adaln_modulate", "forward_modulated",
    "IMATRIX_DELTAS", "quantize_imatrix", "weighted_error",
]

GROUP = 64
SUPPORTED_BITS = (2, 3, 4, 8)


def check_bits(bits: int) -> None:
    if bits not in SUPPORTED_BITS:
        raise ValueError(f"bits must be one of {SUPPORTED_BITS}, got {bits}")


def codes_per_word(bits: int) -> int:
    """Whole codes per uint32 word (widths that divide 32 only)."""
    check_bits(bits)
    if 32 % bits:
        raise ValueError(f"{bits}-bit codes do not tile a 32-bit word")
    return 32 // bits


def words_per_row(bits: int, k: int) -> int:
    """uint32 words of one row's packed codes: k * bits / 32 (k * bits a multiple of 32)."""
    check_bits(bits)
    if (k * bits) % 32:
        raise ValueError("K * bits must be a multiple of 32")
    return k * bits // 32


def bits_per_weight(bits: int, group: int = GROUP) -> float:
    """Nominal width plus one f16 scale and one f16 bias (32 bits) per group.

    Ideogram-4-IQ4_M model card, opening section: the half bit above each
    nominal width is the group overhead of an f16 scale and an f16 bias per 64.
    """
    return bits + 32.0 / group


def storage_bytes(bits: int, n: int, k: int, group: int = GROUP) -> int:
    """Bytes of packed codes + f16 scales + f16 biases for an [n, k] weight."""
    words = n * words_per_row(bits, k)
    groups = n * (k // group)
    return 4 * words + 2 * groups + 2 * groups


# ---------------------------------------------------------------- float helpers

def f16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    """uint16 IEEE half bit patterns -> float32 (exact)."""
    return np.asarray(h, dtype=np.uint16).view(np.float16).astype(np.float32)


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> IEEE half, round-half-to-even (NumPy's conversion), as uint16."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def bf16_bits_to_f64(xb: np.ndarray) -> np.ndarray:
    """uint16 bfloat16 bit patterns -> float64 (exact: bf16 is the top half of fp32)."""
    u = np.asarray(xb, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------- the fit (RTN)

def quantize_rtn(w: np.ndarray, bits: int, group: int = GROUP):
    """Min/max round-to-nearest per (row, 64-wide K group).

    Returns (q uint8 [N, K], s16 uint16 [N, G], b16 uint16 [N, G]) where s16, b16
    are f16 bit patterns. Steps, all in fp32 with IEEE rounding:
      mn, mx  = min, max of the group
      s       = f16((mx - mn) / Q)        Q = 2**bits - 1
      b       = f16(mn)
      q       = clamp(rint_half_even((w - b) / s), 0, Q); q = 0 where s == 0
    Ideogram-4-IQ4_M card, section on what "IQ4" means (min/max candidate,
    round-to-nearest); rounding, tie and division rules are this oracle's
    stated readings.
    """
    w = np.asarray(w, dtype=np.float32)
    if w.ndim != 2:
        raise ValueError("w must be 2-D [N, K]")
    n, k = w.shape
    if group != GROUP:
        raise ValueError("only group size 64 is defined by the pages")
    if k % group != 0:
        raise ValueError("K must be a multiple of the group size")
    if not np.all(np.isfinite(w)):
        raise ValueError("non-finite weight")
    qmax = np.float32(2 ** bits - 1)
    check_bits(bits)
    g = k // group
    wg = w.reshape(n, g, group)
    mn = wg.min(axis=2)
    mx = wg.max(axis=2)
    # min/max order -0 below +0 (IEEE 754-2019 minimum/maximum), so that a
    # group holding both zeros has a well-defined bias sign
    zero_w = wg == 0
    neg0 = (zero_w & np.signbit(wg)).any(axis=2)
    pos0 = (zero_w & ~np.signbit(wg)).any(axis=2)
    mn = np.where(mn == 0, np.where(neg0, np.float32(-0.0), np.float32(0.0)), mn).astype(np.float32)
    mx = np.where(mx == 0, np.where(pos0, np.float32(0.0), np.float32(-0.0)), mx).astype(np.float32)
    s32 = (mx - mn) / qmax                       # fp32 subtract, fp32 divide
    s16 = f32_to_f16_bits(s32)
    b16 = f32_to_f16_bits(mn)
    s_f = f16_bits_to_f32(s16)
    b_f = f16_bits_to_f32(b16)
    if not (np.all(np.isfinite(s_f)) and np.all(np.isfinite(b_f))):
        raise ValueError("scale or bias overflows f16")
    zero = s_f == 0
    safe_s = np.where(zero, np.float32(1), s_f)
    t = (wg - b_f[:, :, None]) / safe_s[:, :, None]   # fp32 subtract, fp32 divide
    q = np.rint(t)                                     # half to even
    q = np.clip(q, 0, qmax)
    q = np.where(zero[:, :, None], np.float32(0), q)
    return q.astype(np.uint8).reshape(n, k), s16, b16


# ------------------------------------------------- importance-weighted fit

# Level-count offsets of the scale search: candidate t starts from codes
# l = rint((w - min) * (Q + d_t) / (max - min)), d_t = (t - 7.5) / 10.
IMATRIX_DELTAS = tuple((t - 7.5) / 10.0 for t in range(16))


def _f32(v):
    return np.float32(v)


def _group_error(w, a, s_f, b_f, q):
    """sum_j a_j * e_j * e_j, e_j = w_j - (s*q_j + b), fp32, j in order; the
    product s*q_j is exact in fp32 (f16 scale, code < 256), so s*q + b rounds once."""
    err = np.zeros(w.shape[:-1], dtype=np.float32)
    for j in range(w.shape[-1]):
        dq = s_f * q[..., j] + b_f
        e = w[..., j] - dq
        err = err + a[..., j] * (e * e)
    return err


def _codes(w, s_f, b_f, qmax):
    """clamp(rint_half_even((w - b) / s), 0, Q) in fp32, 0 where s == 0."""
    zero = s_f == 0
    safe = np.where(zero, np.float32(1), s_f)
    q = np.clip(np.rint((w - b_f[..., None]) / safe[..., None]), 0, qmax).astype(np.float32)
    return np.where(zero[..., None], np.float32(0), q)


def quantize_imatrix(w: np.ndarray, importance: np.ndarray, bits: int, group: int = GROUP):
    """Importance-weighted affine fit per (row, 64-group), same storage as ``quantize_rtn``.

    Objective (Ideogram-4-IQ4_M card, section on what "IQ4" means): an error
    dW_j in input channel j adds dW_j^2 * E[x_j^2] to the output, so each group
    minimises E(s, b) = sum_j E[x_j^2] (w_j - W_hat_j)^2 over its f16 scale and
    bias; the min/max round-to-nearest fit is candidate 0, so the result is
    never worse than RTN by this objective. The pages do not give the other
    candidates; reading taken (this oracle's own search): starting codes l are
    (1) the RTN codes, (2) for each offset d in ``IMATRIX_DELTAS``
    l_j = clamp(rint((w_j - lo) * (Q + d) / (hi - lo)), 0, Q) with [lo, hi] the
    group's [min, max], then (3) the same 16 with [lo, hi] the min and max over
    the channels of nonzero importance (so an outlier in an unweighted channel
    does not set the step). For each, solve the weighted least-squares line
    w ~ s*l + b, round s and b to f16, recompute the codes from the stored s
    and b as RTN does, and keep the candidate with the smallest E (strictly
    smaller: earlier candidates win ties). Candidates whose f16 scale is not a
    positive finite number, or whose bias is not finite, are skipped, as are
    ranges with hi <= lo; a group whose RTN scale is zero keeps RTN.

    Arithmetic: fp32 with one IEEE rounding per operation, no fused
    multiply-add, sums over j = 0..63 in order:
      S0 = sum a_j, S1 = sum a_j*l_j, S2 = sum (a_j*l_j)*l_j,
      T0 = sum a_j*w_j, T1 = sum (a_j*l_j)*w_j,
      D = S0*S2 - S1*S1 (skip unless D > 0),
      s = (S0*T1 - S1*T0) / D, b = (S2*T0 - S1*T1) / D,
      E = sum a_j * (e_j * e_j), e_j = w_j - (s*q_j + b).
    ``importance`` is [K], finite and >= 0. Returns (q uint8 [N, K], s16, b16).
    """
    w = np.asarray(w, dtype=np.float32)
    imp = np.asarray(importance, dtype=np.float32)
    n, k = w.shape
    if imp.shape != (k,):
        raise ValueError("importance must be [K]")
    if not (np.all(np.isfinite(imp)) and np.all(imp >= 0)):
        raise ValueError("importance must be finite and >= 0")
    q0, s16, b16 = quantize_rtn(w, bits, group)
    qmax = np.float32(2 ** bits - 1)
    g = k // group
    wg = w.reshape(n, g, group)
    a = np.broadcast_to(imp.reshape(1, g, group), wg.shape)
    q_best = q0.reshape(n, g, group).astype(np.float32)
    s_best, b_best = s16.copy(), b16.copy()
    err_best = _group_error(wg, a, f16_bits_to_f32(s16), f16_bits_to_f32(b16), q_best)
    live0 = f16_bits_to_f32(s16) != 0
    weighted = a > 0
    ranges = [(wg.min(axis=2), wg.max(axis=2)),
              (np.where(weighted, wg, np.float32(np.inf)).min(axis=2),
               np.where(weighted, wg, np.float32(-np.inf)).max(axis=2))]
    q_rtn = q_best.copy()
    cands = [(None, None)] + [(r, d) for r in range(2) for d in IMATRIX_DELTAS]
    for r, d in cands:
        live = live0.copy()
        if d is None:
            l = q_rtn   # the RTN codes
        else:
            lo, hi = ranges[r]
            live &= hi > lo
            width = np.where(live, hi - lo, np.float32(1))
            lo = np.where(live, lo, np.float32(0))
            inv = (qmax + _f32(d)) / width
            l = np.clip(np.rint((wg - lo[..., None]) * inv[..., None]), 0, qmax).astype(np.float32)
        S0 = np.zeros((n, g), np.float32); S1 = np.zeros((n, g), np.float32); S2 = np.zeros((n, g), np.float32)
        T0 = np.zeros((n, g), np.float32); T1 = np.zeros((n, g), np.float32)
        for j in range(group):
            al = a[..., j] * l[..., j]
            S0 = S0 + a[..., j]
            S1 = S1 + al
            S2 = S2 + al * l[..., j]
            T0 = T0 + a[..., j] * wg[..., j]
            T1 = T1 + al * wg[..., j]
        D = S0 * S2 - S1 * S1
        ok = live & (D > 0)
        safe_d = np.where(ok, D, np.float32(1))
        with np.errstate(over="ignore", invalid="ignore"):
            sc = (S0 * T1 - S1 * T0) / safe_d
            bc = (S2 * T0 - S1 * T1) / safe_d
        sc16, bc16 = f32_to_f16_bits(sc), f32_to_f16_bits(bc)
        sf, bf = f16_bits_to_f32(sc16), f16_bits_to_f32(bc16)
        ok &= np.isfinite(sf) & (sf > 0) & np.isfinite(bf)
        sf = np.where(ok, sf, np.float32(1))
        bf = np.where(ok, bf, np.float32(0))
        qc = _codes(wg, sf, bf, qmax)
        ec = _group_error(wg, a, sf, bf, qc)
        better = ok & (ec < err_best)
        err_best = np.where(better, ec, err_best)
        s_best = np.where(better, sc16, s_best)
        b_best = np.where(better, bc16, b_best)
        q_best = np.where(better[..., None], qc, q_best)
    return q_best.astype(np.uint8).reshape(n, k), s_best.astype(np.uint16), b_best.astype(np.uint16)


def weighted_error(w, importance, q, s16, b16, group: int = GROUP) -> np.ndarray:
    """The fit objective in float64: per (row, group) sum_j E[x_j^2] (w_j - W_hat_j)^2."""
    w = np.asarray(w, dtype=np.float64)
    n, k = w.shape
    wh = dequantize(q, s16, b16, group).astype(np.float64)
    e2 = (w - wh) ** 2 * np.asarray(importance, dtype=np.float64)[None, :]
    return e2.reshape(n, k // group, group).sum(axis=2)


# ---------------------------------------------------------------- packing

_PACK_ROWS = 512   # rows per chunk: bounds the one-byte-per-bit temporaries


def pack(q: np.ndarray, bits: int) -> np.ndarray:
    """q uint8 [N, K] (values < 2**bits) -> uint32 [N, K*bits/32].

    Each row becomes one bit stream: code k contributes its bits, least
    significant first, as stream bits bits*k .. bits*k + bits - 1; the stream
    is then cut into bytes (stream bit i = bit i % 8 of byte i // 8) and the
    bytes into little-endian uint32 words.
    """
    q = np.asarray(q)
    n, k = q.shape
    nw = words_per_row(bits, k)
    if q.size and int(q.max()) >= (1 << bits):
        raise ValueError("code out of range")
    words = np.empty((n, nw), dtype=np.uint32)
    for r0 in range(0, n, _PACK_ROWS):
        qs = q[r0:r0 + _PACK_ROWS].astype(np.uint8)
        code_bits = np.unpackbits(qs[:, :, None], axis=2, bitorder="little")[:, :, :bits]   # [r, k, bits]
        stream = code_bits.reshape(qs.shape[0], k * bits)
        stream_bytes = np.packbits(stream, axis=1, bitorder="little")
        words[r0:r0 + qs.shape[0]] = stream_bytes.view("<u4")
    return words


def unpack(words: np.ndarray, bits: int, k: int) -> np.ndarray:
    """Inverse of ``pack``: uint32 [N, K*bits/32] -> uint8 [N, K]."""
    words = np.asarray(words, dtype=np.uint32)
    n = words.shape[0]
    if words.shape[1] != words_per_row(bits, k):
        raise ValueError("word count does not match K")
    q = np.empty((n, k), dtype=np.uint8)
    for r0 in range(0, n, _PACK_ROWS):
        ws = np.ascontiguousarray(words[r0:r0 + _PACK_ROWS], dtype="<u4")
        stream = np.unpackbits(ws.view(np.uint8), axis=1, bitorder="little")               # [r, k*bits]
        code_bits = stream.reshape(ws.shape[0], k, bits)
        q[r0:r0 + ws.shape[0]] = np.packbits(code_bits, axis=2, bitorder="little")[:, :, 0]
    return q


# ---------------------------------------------------------------- dequantize

def dequantize(q: np.ndarray, s16: np.ndarray, b16: np.ndarray, group: int = GROUP) -> np.ndarray:
    """W_hat = f32(s) * f32(q) + f32(b) in fp32, one group of 64 per (s, b).

    s has at most 11 significant bits and q at most 8, so s*q is exact in fp32
    and the only rounding is the final add: the result is unique.
    """
    q = np.asarray(q)
    n, k = q.shape
    g = k // group
    s = f16_bits_to_f32(s16).reshape(n, g, 1)
    b = f16_bits_to_f32(b16).reshape(n, g, 1)
    qf = q.astype(np.float32).reshape(n, g, group)
    return (s * qf + b).astype(np.float32).reshape(n, k)


# ---------------------------------------------------------------- product

def gemm_f64(x_bf16: np.ndarray, w_hat: np.ndarray) -> np.ndarray:
    """y = f64(x) @ f64(W_hat)^T, float64 accumulation (BLAS dgemm)."""
    x = bf16_bits_to_f64(x_bf16)
    return x @ np.asarray(w_hat, dtype=np.float64).T


def forward(x_bf16, packed, s16, b16, bits, k, group: int = GROUP) -> np.ndarray:
    """Full path: unpack -> dequantize (fp32) -> fp64 GEMM. Returns float64 [M, N]."""
    q = unpack(packed, bits, k)
    w_hat = dequantize(q, s16, b16, group)
    return gemm_f64(x_bf16, w_hat)


def forward_rows(x_bf16, packed, s16, b16, bits, k, rows, cols=None, group: int = GROUP):
    """The same result restricted to selected output rows (and columns)."""
    x_sel = np.asarray(x_bf16)[np.asarray(rows)]
    if cols is not None:
        cols = np.asarray(cols)
        packed, s16, b16 = packed[cols], s16[cols], b16[cols]
    return forward(x_sel, packed, s16, b16, bits, k, group)


def fast_weights_f16(q: np.ndarray, s16: np.ndarray, b16: np.ndarray, group: int = GROUP) -> np.ndarray:
    """FAST-mode weights: s*q + b rounded once to fp16 (nearest, ties to even).

    With s, b in f16 and q < 256 the value s*q + b is exact in float64, so the
    float64 -> float16 conversion is the only rounding.
    """
    q = np.asarray(q)
    n, k = q.shape
    g = k // group
    s = f16_bits_to_f32(s16).astype(np.float64).reshape(n, g, 1)
    b = f16_bits_to_f32(b16).astype(np.float64).reshape(n, g, 1)
    w = s * q.astype(np.float64).reshape(n, g, group) + b
    return w.reshape(n, k).astype(np.float16)


def fast_activations_f16(x_bf16: np.ndarray):
    """FAST-mode activations: each row is scaled by the power of two 2^-e that
    brings its largest magnitude into [2^14, 2^15) (e = floor(log2 max|x|) - 14,
    clamped to [-126, 120]; e = 0 for an all-zero row), then rounded to fp16
    (exact for every scaled magnitude >= 2^-14, i.e. down to 2^-28 of the row's
    largest value). Returns (x16 as float16 [M, K], 2^e as float64 [M])."""
    x = bf16_bits_to_f64(x_bf16)
    m = x.shape[0]
    scale = np.ones(m, dtype=np.float64)
    for r in range(m):
        mx = float(np.max(np.abs(x[r]))) if x.shape[1] else 0.0
        if mx == 0.0:
            e = 0
        elif not math.isfinite(mx):
            e = 120
        else:
            e = min(max(math.frexp(mx)[1] - 1 - 14, -126), 120)   # frexp: mx = f * 2^k, f in [0.5, 1)
        scale[r] = 2.0 ** e
    x16 = (x / scale[:, None]).astype(np.float16)
    return x16, scale


def forward_fast(x_bf16, packed, s16, b16, bits, k, group: int = GROUP) -> np.ndarray:
    """FAST-mode product: 2^e_row * (x16 @ W16^T), accumulated in float64."""
    q = unpack(packed, bits, k)
    w16 = fast_weights_f16(q, s16, b16, group).astype(np.float64)
    x16, scale = fast_activations_f16(x_bf16)
    return scale[:, None] * (x16.astype(np.float64) @ w16.T)


def forward_fast_rows(x_bf16, packed, s16, b16, bits, k, rows, cols=None, group: int = GROUP):
    """``forward_fast`` restricted to selected output rows (and columns): the
    row scales depend only on their row and the fp16 weights only on theirs."""
    x_sel = np.asarray(x_bf16)[np.asarray(rows)]
    if cols is not None:
        cols = np.asarray(cols)
        packed, s16, b16 = packed[cols], s16[cols], b16[cols]
    return forward_fast(x_sel, packed, s16, b16, bits, k, group)


def silu(v) -> np.ndarray:
    """silu(v) = v * sigmoid(v) = v / (1 + exp(-v)), float64; exp overflow for
    v < -709 gives v / inf = -0, the limit."""
    v = np.asarray(v, dtype=np.float64)
    with np.errstate(over="ignore"):
        return v / (1.0 + np.exp(-v))


def swiglu(y: np.ndarray, f: int) -> np.ndarray:
    """Gated output of a stacked [gate; up] product y [M, 2f]: silu(y[:, :f]) * y[:, f:]."""
    y = np.asarray(y, dtype=np.float64)
    assert y.shape[1] == 2 * f
    return silu(y[:, :f]) * y[:, f:]


def gate_residual(y: np.ndarray, residual: np.ndarray, gate: np.ndarray, gate_rows: int) -> np.ndarray:
    """Gated residual update of a branch output y [M, N]: every output row m
    belongs to sample m // gate_rows and adds that sample's gate row times y[m]
    to residual[m]: out = residual + gate[m // gate_rows] * y, in float64."""
    y = np.asarray(y, dtype=np.float64)
    residual = np.asarray(residual, dtype=np.float64)
    gate = np.asarray(gate, dtype=np.float64)
    assert gate_rows >= 1 and y.shape == residual.shape and gate.shape[1] == y.shape[1]
    sample = np.arange(y.shape[0]) // gate_rows
    assert gate.shape[0] > (sample[-1] if len(sample) else -1)
    return residual + gate[sample] * y


def adaln_modulate(x_bf16, scale, rows_per_sample: int) -> np.ndarray:
    """AdaLN scale applied to a bf16 input: row m belongs to sample
    m // rows_per_sample, and x_mod[m, k] = x[m, k] * (1 + scale[sample, k]),
    float64 [M, K]."""
    x = bf16_bits_to_f64(x_bf16)
    scale = np.asarray(scale, dtype=np.float64)
    assert rows_per_sample >= 1 and scale.ndim == 2 and scale.shape[1] == x.shape[1]
    sample = np.arange(x.shape[0]) // rows_per_sample
    assert scale.shape[0] > (sample[-1] if len(sample) else -1)
    return x * (1.0 + scale[sample])


def forward_modulated(x_bf16, scale, rows_per_sample, packed, s16, b16, bits, k, group: int = GROUP):
    """Plain product of the AdaLN-modulated input with the dequantized weights:
    adaln_modulate(x) @ W_hat^T, float64 [M, N]."""
    w_hat = dequantize(unpack(packed, bits, k), s16, b16, group)
    return adaln_modulate(x_bf16, scale, rows_per_sample) @ np.asarray(w_hat, dtype=np.float64).T


def error_metrics(y: np.ndarray, y_ref: np.ndarray) -> dict:
    """relF = ||y - ref||_F / ||ref||_F ; maxabs_over_rms = max|y - ref| / rms(ref)."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    d = y - y_ref
    nref = float(np.linalg.norm(y_ref))
    rms = nref / math.sqrt(max(y_ref.size, 1))
    relf = float(np.linalg.norm(d)) / nref if nref > 0 else float(np.linalg.norm(d))
    mad = float(np.max(np.abs(d))) if d.size else 0.0
    return {"relF": relf, "maxabs_over_rms": (mad / rms) if rms > 0 else mad, "max_abs": mad, "rms": rms}


def timed_forward(x_bf16, packed, s16, b16, bits, k, group: int = GROUP):
    """Oracle forward with the dequantize and GEMM legs timed separately (seconds)."""
    t0 = time.perf_counter()
    q = unpack(packed, bits, k)
    w_hat = dequantize(q, s16, b16, group)
    t1 = time.perf_counter()
    y = gemm_f64(x_bf16, w_hat)
    t2 = time.perf_counter()
    return y, {"dequant_s": t1 - t0, "gemm_s": t2 - t1, "total_s": t2 - t0}
