"""Pins of the CPU oracle to facts other than itself.

Each test states what it checks against: a figure printed on the pages
(tests/golden/page_figures.json), a hand-worked example (tests/golden/
hand_example.json), exact rational arithmetic, brute force or a closed form.
No expected value here comes from the HIP library.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from group_wise_affine_qlinear_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------- independent helpers

def exact_f16_rne(v: Fraction) -> int:
    """Round a rational to IEEE half, half-to-even, returning the bit pattern.

    Written from the IEEE 754 binary16 definition (5 exponent bits, bias 15,
    10 fraction bits, subnormals below 2**-14); shares nothing with NumPy.
    """
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    if a == 0:
        return sign
    e = math.floor(math.log2(a)) if a.numerator and a.denominator else 0
    # fix floor(log2) exactly
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -14)                      # subnormal range shares the 2**-14 exponent
    ulp = Fraction(2) ** (e - 10)
    m = a / ulp                          # significand in units of ulp
    fl = math.floor(m)
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    if fl == 2048:                       # carried into the next binade
        fl = 1024
        e += 1
    if e > 15:
        return sign | 0x7C00             # overflow to inf
    if fl < 1024:                        # subnormal
        return sign | fl
    return sign | ((e + 15) << 10) | (fl - 1024)


def f16_value(bits: int) -> Fraction:
    s = -1 if bits & 0x8000 else 1
    e = (bits >> 10) & 0x1F
    f = bits & 0x3FF
    if e == 0:
        return s * Fraction(f) * Fraction(2) ** -24
    return s * (1 + Fraction(f, 1024)) * Fraction(2) ** (e - 15)


# ----------------------------------------------------------------- bits per weight / sizes

def test_bpw_closed_form_matches_page_overhead():
    fig = _golden("page_figures.json")
    over = fig["group_overhead_bits"]["value"]
    assert fig["group_overhead_bits"]["group"] == oracle.GROUP == fig["group_size"]["value"]
    for b in (2, 3, 4, 8):
        assert oracle.bits_per_weight(b) == b + over
    for (n, k) in [(256, 512), (13824, 4608), (4608, 53248), (3, 64)]:
        for b in (2, 3, 4, 8):
            assert oracle.storage_bytes(b, n, k) * 8 == n * k * (b + over)


def test_page_sizes_follow_from_closed_form():
    fig = _golden("page_figures.json")
    p = fig["quantized_params"]["value"]
    q4 = p * oracle.bits_per_weight(4) / 8 / 1e9
    q8 = p * oracle.bits_per_weight(8) / 8 / 1e9
    bf16 = p * 2 / 1e9
    assert abs(q4 - fig["q4_on_disk_gb"]["value"]) < 0.5       # 14.2 vs ~14
    assert abs(q8 - fig["q8_on_disk_gb"]["value"]) < 0.5       # 26.8 vs ~27
    assert abs(bf16 - fig["bf16_snapshot_gb"]["value"]) < 0.5  # 50.4 vs ~50
    assert abs(q4 / bf16 - fig["q4_download_fraction_vs_bf16"]["value"]) < 0.05


# ----------------------------------------------------------------- packing

def test_pack_hand_words():
    hw = _golden("hand_example.json")["pack_words"]
    for key, bits in (("bits4_codes_1_to_8", 4), ("bits2_codes", 2), ("bits8_codes", 8)):
        codes = np.array([hw[key]["codes"]], dtype=np.uint8)
        word = int(hw[key]["word_hex"], 16)
        packed = oracle.pack(codes, bits)
        assert packed.shape == (1, 1) and int(packed[0, 0]) == word
        assert np.array_equal(oracle.unpack(packed, bits, codes.shape[1]), codes)


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_pack_unpack_round_trip(bits):
    n, k = 7, 256
    q = inputs.random_codes(n, k, bits, workload_id=99)
    assert np.array_equal(oracle.unpack(oracle.pack(q, bits), bits, k), q)
    qmax = (1 << bits) - 1
    for pat in (np.zeros((n, k)), np.full((n, k), qmax), np.tile([0, qmax], (n, k // 2))):
        pat = pat.astype(np.uint8)
        assert np.array_equal(oracle.unpack(oracle.pack(pat, bits), bits, k), pat)
    all_q = oracle.pack(np.full((1, 32), qmax, dtype=np.uint8), bits)
    assert all_q.shape == (1, bits) and np.all(all_q == 0xFFFFFFFF)
    words = np.random.default_rng(5).integers(0, 2**32, size=(n, k * bits // 32), dtype=np.uint64).astype(np.uint32)
    assert np.array_equal(oracle.pack(oracle.unpack(words, bits, k), bits), words)


def test_pack_3bit_hand_words():
    """3-bit bit stream, hand-worked: code k at stream bits 3k .. 3k+2; codes 10
    (bits 30-32) and 21 (bits 63-65) straddle words."""
    def row(**codes):
        q = np.zeros((1, 32), dtype=np.uint8)
        for k, v in codes.items():
            q[0, int(k[1:])] = v
        return q
    cases = [
        (row(c10=7), [0xC0000000, 0x00000001, 0x00000000]),
        (row(c21=5), [0x00000000, 0x80000000, 0x00000002]),
        (row(c0=5, c31=6), [0x00000005, 0x00000000, 0xC0000000]),
        (row(c1=1, c11=3, c22=4), [0x00000008, 0x00000003 << 1, 0x00000004 << 2]),
    ]
    for q, words in cases:
        got = oracle.pack(q, 3)
        assert got.tolist() == [words], (q, [hex(w) for w in got[0]])
        assert np.array_equal(oracle.unpack(got, 3, 32), q)


def test_pack_stream_matches_big_integer():
    """Every width against an independent construction: the row's codes summed
    into one Python integer at bit offsets bits*k, split into 32-bit words."""
    for bits in (2, 3, 4, 8):
        q = inputs.random_codes(5, 192, bits, workload_id=98)
        got = oracle.pack(q, bits)
        for n in range(q.shape[0]):
            v = sum(int(c) << (bits * k) for k, c in enumerate(q[n]))
            words = [(v >> (32 * i)) & 0xFFFFFFFF for i in range(192 * bits // 32)]
            assert got[n].tolist() == words


def test_pack_rejects_out_of_range_code():
    with pytest.raises(ValueError):
        oracle.pack(np.array([[16] + [0] * 7], dtype=np.uint8), 4)


# ----------------------------------------------------------------- f16 / bf16 conversions

def test_f16_rounding_matches_exact_rne():
    vals = [Fraction(1) + Fraction(1, 2048), Fraction(1) + Fraction(3, 2048), Fraction(65504),
            Fraction(1, 2**24), Fraction(3, 2**26), Fraction(5, 2**26), Fraction(-1, 3),
            Fraction(1, 10), Fraction(3, 2) / 15]
    rng = np.random.default_rng(11)
    vals += [Fraction(float(v)) for v in rng.normal(0, 0.05, 400).astype(np.float32)]
    vals += [Fraction(float(v)) for v in rng.uniform(-7e-5, 7e-5, 200).astype(np.float32)]
    for v in vals:
        f32 = np.float32(float(v))
        if Fraction(float(f32)) != v:
            continue  # only values exactly representable in fp32 are fed to the conversion
        got = int(oracle.f32_to_f16_bits(np.array([f32]))[0])
        assert got == exact_f16_rne(v), (v, hex(got), hex(exact_f16_rne(v)))
    # the two ties, by hand: 1 + 2^-11 -> 1.0 (even), 1 + 3*2^-11 -> 1 + 2^-9
    assert int(oracle.f32_to_f16_bits(np.array([1 + 2**-11], np.float32))[0]) == 0x3C00
    assert int(oracle.f32_to_f16_bits(np.array([1 + 3 * 2**-11], np.float32))[0]) == 0x3C02


def test_bf16_decode_known_patterns():
    got = oracle.bf16_bits_to_f64(np.array([0x3F80, 0xC000, 0x4300, 0x0000, 0x8000, 0x0001], dtype=np.uint16))
    assert list(got[:5]) == [1.0, -2.0, 128.0, 0.0, -0.0]
    assert got[5] == 2.0 ** -133


def test_input_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    x = inputs.activations_f32(33, 128, workload_id=7, structure="outlier")
    mine = inputs.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)


# ----------------------------------------------------------------- RTN fit

def test_rtn_hand_example():
    ex = _golden("hand_example.json")["rtn_4bit_group"]
    k = np.arange(64)
    w = (-1 + 0.125 * (k % 16)).astype(np.float32)[None, :]
    q, s16, b16 = oracle.quantize_rtn(w, 4)
    assert int(s16[0, 0]) == int(ex["s16_hex"], 16)
    assert int(b16[0, 0]) == int(ex["b16_hex"], 16)
    assert np.array_equal(q[0], (k % 16).astype(np.uint8))
    words = oracle.pack(q, 4)
    assert [int(v) for v in words[0]] == [int(h, 16) for h in ex["words_hex"]]
    w_hat = oracle.dequantize(q, s16, b16)
    assert np.array_equal(w_hat, w)


def test_rtn_tie_rounds_half_to_even():
    ex = _golden("hand_example.json")["tie_4bit_group"]
    s_f = float(np.float16(0.1))
    assert np.float16(0.1).view(np.uint16) == int(ex["s16_hex"], 16)
    w = np.zeros((1, 64), np.float32)
    w[0, 1] = 1.5
    w[0, 2] = 2.5 * s_f
    w[0, 3] = 3.5 * s_f
    q, s16, b16 = oracle.quantize_rtn(w, 4)
    assert int(s16[0, 0]) == int(ex["s16_hex"], 16) and int(b16[0, 0]) == int(ex["b16_hex"], 16)
    assert list(q[0, :4]) == ex["q_first4"]
    assert not q[0, 4:].any()


def test_constant_group():
    w = np.full((2, 128), 0.3, np.float32)
    w[1, 64:] = -2.75
    q, s16, b16 = oracle.quantize_rtn(w, 4)
    assert not s16.any()
    assert not q.any()
    assert int(b16[0, 0]) == exact_f16_rne(Fraction(float(np.float32(0.3))))
    w_hat = oracle.dequantize(q, s16, b16)
    assert np.array_equal(w_hat[0], np.full(128, float(np.float16(0.3)), np.float32))
    assert np.array_equal(w_hat[1, 64:], np.full(64, -2.75, np.float32))


def test_rtn_rejects_non_finite_and_overflow():
    w = np.zeros((1, 64), np.float32)
    w[0, 5] = np.nan
    with pytest.raises(ValueError):
        oracle.quantize_rtn(w, 4)
    w = np.zeros((1, 64), np.float32)
    w[0, 0] = 1e6   # bias fine (0) but scale 1e6/15 overflows f16
    with pytest.raises(ValueError):
        oracle.quantize_rtn(w, 4)


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_rtn_scale_bias_are_rounded_min_max(bits):
    """s and b equal exact-RNE f16 of (max-min)/Q (fp32 ops) and of min, group by group."""
    w = inputs.weights(6, 256, workload_id=21)
    q, s16, b16 = oracle.quantize_rtn(w, bits)
    qmax = (1 << bits) - 1
    for n in range(w.shape[0]):
        for g in range(w.shape[1] // 64):
            grp = w[n, 64 * g:64 * g + 64]
            mn, mx = np.float32(grp.min()), np.float32(grp.max())
            s32 = np.float32(np.float32(mx - mn) / np.float32(qmax))
            assert int(s16[n, g]) == exact_f16_rne(Fraction(float(s32)))
            assert int(b16[n, g]) == exact_f16_rne(Fraction(float(mn)))
    assert q.max() <= qmax


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_rtn_brute_force_nearest_code(bits):
    """q is the nearest grid point among all 2**bits codes (exact fp64 distances)."""
    w = inputs.weights(16, 512, workload_id=22)
    q, s16, b16 = oracle.quantize_rtn(w, bits)
    s = oracle.f16_bits_to_f32(s16).astype(np.float64).repeat(64, axis=1)
    b = oracle.f16_bits_to_f32(b16).astype(np.float64).repeat(64, axis=1)
    codes = np.arange(1 << bits, dtype=np.float64)
    grid = s[:, :, None] * codes[None, None, :] + b[:, :, None]     # exact in fp64
    d = np.abs(w.astype(np.float64)[:, :, None] - grid)              # exact in fp64
    best = d.min(axis=2)
    chosen = np.take_along_axis(d, q.astype(np.int64)[:, :, None], axis=2)[:, :, 0]
    # the chosen code is optimal up to the fp32 rounding of (w - b) / s
    assert np.all(chosen - best <= 2.0 ** -20 * s)
    # and exactly the argmin wherever the best code is clearly separated
    srt = np.sort(d, axis=2)
    clear = (srt[:, :, 1] - srt[:, :, 0]) > 2.0 ** -18 * s
    assert np.array_equal(q[clear], d.argmin(axis=2)[clear].astype(np.uint8))
    # error bound of round-to-nearest on a uniform grid
    w_hat = oracle.dequantize(q, s16, b16).astype(np.float64)
    assert np.all(np.abs(w - w_hat) <= 0.5 * s + 4 * np.spacing(np.abs(w).astype(np.float32)).astype(np.float64) + 1e-12)


# ----------------------------------------------------------------- dequantize

@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_dequant_equals_exact_then_round(bits):
    """fp32 mul+add equals the exactly computed s*q + b rounded once to fp32."""
    n, k = 32, 256
    q = inputs.random_codes(n, k, bits, workload_id=23)
    s16 = inputs.random_f16_bits(n, k // 64, 1e-4, 0.2, workload_id=23, role=inputs.ROLE_SCALE)
    b16 = inputs.random_f16_bits(n, k // 64, -3.0, 3.0, workload_id=23, role=inputs.ROLE_BIAS)
    got = oracle.dequantize(q, s16, b16)
    s = np.asarray(s16).view(np.float16).astype(np.float64).repeat(64, axis=1)
    b = np.asarray(b16).view(np.float16).astype(np.float64).repeat(64, axis=1)
    exact = s * q.astype(np.float64) + b     # exact in fp64 for these magnitudes
    assert np.array_equal(got, exact.astype(np.float32))
    # spot-check a few against rational arithmetic
    for (i, j) in [(0, 0), (3, 77), (31, 255)]:
        v = f16_value(int(s16[i, j // 64])) * int(q[i, j]) + f16_value(int(b16[i, j // 64]))
        assert Fraction(float(got[i, j])) == Fraction(float(np.float32(float(v))))


# ----------------------------------------------------------------- GEMM

@pytest.mark.parametrize("shape", [(1, 64, 1), (3, 128, 5), (17, 192, 9), (8, 512, 16)])
def test_gemm_brute_force_fsum(shape):
    m, k, n = shape
    x = inputs.activations_bf16(m, k, workload_id=31)
    w = inputs.weights(n, k, workload_id=31)
    q, s16, b16 = oracle.quantize_rtn(w, 4)
    y = oracle.forward(x, oracle.pack(q, 4), s16, b16, 4, k)
    xf = oracle.bf16_bits_to_f64(x)
    w_hat = oracle.dequantize(q, s16, b16).astype(np.float64)
    for i in range(m):
        for j in range(n):
            ref = math.fsum(float(xf[i, t]) * float(w_hat[j, t]) for t in range(k))  # products exact
            assert abs(y[i, j] - ref) <= 1e-12 * max(1.0, math.fsum(abs(float(xf[i, t]) * float(w_hat[j, t])) for t in range(k)))


def test_identity_x_gives_transposed_weights():
    k, n = 128, 24   # M = K != N, so a transposed operand cannot pass
    w = inputs.weights(n, k, workload_id=32)
    q, s16, b16 = oracle.quantize_rtn(w, 4)
    one = 0x3F80
    x = np.zeros((k, k), np.uint16)
    x[np.arange(k), np.arange(k)] = one
    y = oracle.forward(x, oracle.pack(q, 4), s16, b16, 4, k)
    assert y.shape == (k, n)
    assert np.array_equal(y, oracle.dequantize(q, s16, b16).astype(np.float64).T)


def test_zero_and_ones_rows():
    k, n = 256, 10
    w = inputs.weights(n, k, workload_id=33)
    q, s16, b16 = oracle.quantize_rtn(w, 8)
    x = np.zeros((2, k), np.uint16)
    x[1, :] = 0x3F80
    y = oracle.forward(x, oracle.pack(q, 8), s16, b16, 8, k)
    assert not y[0].any()
    w_hat = oracle.dequantize(q, s16, b16)
    for j in range(n):
        assert abs(y[1, j] - math.fsum(float(v) for v in w_hat[j])) <= 1e-12


def test_linearity():
    k, n, m = 256, 12, 5
    w = inputs.weights(n, k, workload_id=34)
    q, s16, b16 = oracle.quantize_rtn(w, 2)
    p = oracle.pack(q, 2)
    x1 = inputs.activations_bf16(m, k, workload_id=34)
    x2 = inputs.activations_bf16(m, k, workload_id=35)
    # x1 + x2 exactly representable? use 2*x1 instead (exact scaling in bf16)
    x1f = oracle.bf16_bits_to_f64(x1)
    two_x1 = inputs.f32_to_bf16_bits((2 * x1f).astype(np.float32))
    y1 = oracle.forward(x1, p, s16, b16, 2, k)
    assert np.allclose(oracle.forward(two_x1, p, s16, b16, 2, k), 2 * y1, rtol=0, atol=1e-12)
    y2 = oracle.forward(x2, p, s16, b16, 2, k)
    xx = np.concatenate([x1, x2])
    assert np.allclose(oracle.forward(xx, p, s16, b16, 2, k), np.concatenate([y1, y2]), rtol=0, atol=1e-12)


def test_error_metrics_closed_form():
    ref = np.ones((4, 4))
    y = ref.copy()
    y[0, 0] += 0.5
    e = oracle.error_metrics(y, ref)
    assert abs(e["relF"] - 0.5 / 4.0) < 1e-15
    assert abs(e["maxabs_over_rms"] - 0.5) < 1e-15


def test_forward_rows_matches_full():
    m, k, n = 9, 128, 11
    x = inputs.activations_bf16(m, k, workload_id=36)
    w = inputs.weights(n, k, workload_id=36)
    q, s16, b16 = oracle.quantize_rtn(w, 4)
    p = oracle.pack(q, 4)
    full = oracle.forward(x, p, s16, b16, 4, k)
    rows, cols = [0, 4, 8], [1, 10]
    sub = oracle.forward_rows(x, p, s16, b16, 4, k, rows, cols)
    assert np.array_equal(sub, full[np.ix_(rows, cols)])


# ----------------------------------------------------------------- planted mistakes

def test_planted_bit_order_mistake_is_caught(monkeypatch):
    """A big-endian nibble order in the oracle's unpack must fail the hand-word pin."""
    real_unpack = oracle.qlinear_oracle.unpack

    def wrong_unpack(words, bits, k):
        q = real_unpack(words, bits, k)
        c = 32 // bits
        return q.reshape(q.shape[0], -1, c)[:, :, ::-1].reshape(q.shape)

    hw = _golden("hand_example.json")["pack_words"]["bits4_codes_1_to_8"]
    word = np.array([[int(hw["word_hex"], 16)]], dtype=np.uint32)
    assert list(wrong_unpack(word, 4, 8)[0]) != hw["codes"]
    assert list(real_unpack(word, 4, 8)[0]) == hw["codes"]


def test_planted_dropped_bias_is_caught():
    """Dequantizing without the bias term must fail the hand example."""
    k = np.arange(64)
    w = (-1 + 0.125 * (k % 16)).astype(np.float32)[None, :]
    q, s16, b16 = oracle.quantize_rtn(w, 4)
    no_bias = oracle.dequantize(q, s16, np.zeros_like(b16))
    assert not np.array_equal(no_bias, w)
    assert np.array_equal(oracle.dequantize(q, s16, b16), w)


# ----------------------------------------------------------------- generators

def test_generators_are_deterministic():
    a = inputs.workload_inputs("tiny")
    b = inputs.workload_inputs("tiny")
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert a[0].shape == (256, 512) and a[1].shape == (64, 512)
    xo = inputs.activations_f32(4, 4608, workload_id=2, structure="outlier")
    big = np.abs(xo).max(axis=0) > 0
    assert big.all()
    xs = inputs.activations_f32(64, 53248, workload_id=4, structure="slices")
    stds = xs.reshape(64, 13, 4096).std(axis=(0, 2))
    assert np.all((stds > 0.4) & (stds < 4.2))


def test_signed_zero_ordering_in_min_max():
    """-0 orders below +0: a group of +-0 gets bias -0 and scale +0."""
    w = np.zeros((2, 64), np.float32)
    w[0, 1::2] = -0.0
    w[1, :] = -0.0
    q, s16, b16 = oracle.quantize_rtn(w, 4)
    assert int(b16[0, 0]) == 0x8000 and int(s16[0, 0]) == 0x0000
    assert int(b16[1, 0]) == 0x8000 and int(s16[1, 0]) == 0x0000
    assert not q.any()


# ----------------------------------------------------------------- FAST-mode definition

def test_fast_weights_single_rounding_matches_exact_rne():
    # every code of several (scale, bias) pairs, including full-mantissa scales
    # whose s*q + b needs more than 11 bits, against exact rational rounding
    rng = np.random.default_rng(5)
    s_bits = [0x3555, 0x2E66, 0x1C01, 0x3BFF] + list(rng.integers(0x1000, 0x3C00, 6))
    b_bits = [0xBC01, 0x3C01, 0x0000, 0xC3FF] + list(rng.integers(0x8400, 0xC000, 6))
    for bits in (2, 4, 8):
        qmax = 2 ** bits - 1
        for sb, bb in zip(s_bits, b_bits):
            q = np.arange(64, dtype=np.int64).reshape(1, 64) % (qmax + 1)
            s16 = np.array([[sb]], np.uint16)
            b16 = np.array([[bb]], np.uint16)
            got = oracle.fast_weights_f16(q, s16, b16).view(np.uint16)[0]
            for k in range(64):
                exact = f16_value(int(sb)) * int(q[0, k]) + f16_value(int(bb))
                assert int(got[k]) == exact_f16_rne(exact), (bits, hex(sb), hex(bb), k)


def test_fast_weights_tie_goes_to_even():
    # s = 0.5, b = 2048: q = 2 gives 2049, halfway between 2048 and 2050 -> 2048
    q = np.array([[2, 6] + [0] * 62])
    s16 = np.array([[0x3800]], np.uint16)  # 0.5
    b16 = np.array([[0x6800]], np.uint16)  # 2048
    w = oracle.fast_weights_f16(q, s16, b16).astype(np.float64)[0]
    assert w[0] == 2048.0 and w[1] == 2052.0   # 2051 is also a tie: 2050 (odd) -> 2052 (even)


def test_fast_equals_exact_when_everything_is_representable():
    rng = np.random.default_rng(8)
    n, k, m = 12, 128, 5
    q = rng.integers(0, 16, (n, k))
    s16 = np.full((n, k // 64), 0x3400, np.uint16)   # 0.25
    b16 = np.full((n, k // 64), 0xC000, np.uint16)   # -2
    packed = oracle.pack(q, 4)
    xb = inputs.f32_to_bf16_bits(rng.integers(-8, 9, (m, k)).astype(np.float32))
    assert np.array_equal(oracle.forward_fast(xb, packed, s16, b16, 4, k),
                          oracle.forward(xb, packed, s16, b16, 4, k))


def test_fast_row_scaling_is_a_power_of_two():
    k = 64
    x = np.zeros((8, k), np.float32)
    x[0, :3] = [65536.0, -3.0, 0.5]     # max 2^16 -> e = 2 (2^16 / 4 = 2^14)
    x[1, 0] = 32768.0                   # exactly 2^15 -> e = 1
    x[2, 0] = 32512.0                   # largest bf16 below 2^15 -> e = 0
    x[3, 0] = -3.0e38                   # near the top of the bf16 range
    x[4, :2] = [3.0, 1.0]               # max 3 = 1.5 * 2^1 -> e = 1 - 14 = -13 (3 * 2^13 = 24576)
    x[5, 0] = 2.0 ** -30                # tiny row -> e = -44, scaled up to 2^14
    # row 6 stays all zero -> e = 0
    x[7, 0] = 2.0 ** -126               # smallest normal fp32: e = -140 clamps to -126
    xb = inputs.f32_to_bf16_bits(x)
    x16, scale = oracle.fast_activations_f16(xb)
    assert list(scale[:3]) == [4.0, 2.0, 1.0]
    assert scale[4] == 2.0 ** -13 and scale[5] == 2.0 ** -44 and scale[6] == 1.0 and scale[7] == 2.0 ** -126
    e3 = int(round(math.log2(scale[3])))
    xmax = float(oracle.bf16_bits_to_f64(xb[3:4, :1])[0, 0])
    assert 16384 <= abs(xmax) * 2.0 ** -e3 < 32768
    # scaled values that are powers of two or small integers stay exact
    assert float(x16[0, 0]) * 4 == 65536.0 and float(x16[0, 1]) * 4 == -3.0 and float(x16[0, 2]) * 4 == 0.5
    assert float(x16[4, 0]) == 24576.0 and float(x16[4, 1]) == 8192.0
    assert float(x16[5, 0]) == 16384.0 and float(x16[7, 0]) == 1.0


def test_fast_activation_subnormals_round_to_nearest():
    # a row whose largest value is 2^14 keeps e = 0, so its small values land
    # in the fp16 subnormal range and round to nearest-even there
    vals = [2.0 ** 14, 2.0 ** -20, 1.5 * 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14 * (1 + 2.0 ** -7)]
    xb = inputs.f32_to_bf16_bits(np.array([vals], np.float32))
    x16, scale = oracle.fast_activations_f16(xb)
    assert scale[0] == 1.0
    for v, got in zip(oracle.bf16_bits_to_f64(xb)[0], x16.view(np.uint16)[0]):
        assert int(got) == exact_f16_rne(Fraction(float(v))), v


def test_fast_tiny_rows_keep_their_accuracy():
    # a row of activations around 1e-9 loses nothing to the fp16 range: its
    # FAST product meets the acceptance bar like a row of unit scale
    rng = np.random.default_rng(15)
    w = (rng.standard_normal((40, 256)) * 0.02).astype(np.float32)
    q, s16, b16 = oracle.quantize_rtn(w, 4)
    packed = oracle.pack(q, 4)
    x = rng.standard_normal((3, 256)).astype(np.float32)
    x[1] *= np.float32(2.0 ** -30)
    x[2] *= np.float32(2.0 ** 20)
    xb = inputs.f32_to_bf16_bits(x)
    fast = oracle.forward_fast(xb, packed, s16, b16, 4, 256)
    exact = oracle.forward(xb, packed, s16, b16, 4, 256)
    for r in range(3):
        e = oracle.error_metrics(fast[r:r + 1], exact[r:r + 1])
        assert e["relF"] < 5e-4, (r, e)


def test_fast_error_budget_on_normal_weights():
    # the FAST mode's only extra rounding is fp16 on W: relative Frobenius error
    # ~2^-11 / sqrt(3) per weight, far inside the 2e-3 acceptance bound
    rng = np.random.default_rng(9)
    w = (rng.standard_normal((64, 512)) * 0.02).astype(np.float32)
    q, s16, b16 = oracle.quantize_rtn(w, 4)
    packed = oracle.pack(q, 4)
    xb = inputs.f32_to_bf16_bits(rng.standard_normal((48, 512)).astype(np.float32))
    e = oracle.error_metrics(oracle.forward_fast(xb, packed, s16, b16, 4, 512),
                             oracle.forward(xb, packed, s16, b16, 4, 512))
    assert 5e-5 < e["relF"] < 5e-4 and e["maxabs_over_rms"] < 3e-3, e


# ---- SwiGLU (stacked gate/up projection) ------------------------------------

def test_silu_closed_forms():
    # sigmoid(ln 3) = 3/4, sigmoid(0) = 1/2, sigmoid(-ln 3) = 1/4
    ln3 = math.log(3.0)
    got = oracle.silu(np.array([0.0, ln3, -ln3, 1000.0, -1000.0]))
    assert got[0] == 0.0
    assert abs(got[1] - 0.75 * ln3) < 1e-15 and abs(got[2] + 0.25 * ln3) < 1e-15
    assert got[3] == 1000.0 and got[4] == 0.0 and math.copysign(1.0, got[4]) < 0


def test_silu_matches_library_logistic():
    from scipy.special import expit
    v = np.linspace(-40, 40, 2001)
    np.testing.assert_allclose(oracle.silu(v), v * expit(v), rtol=1e-14, atol=1e-300)
    # odd part: silu(v) - silu(-v) = v
    np.testing.assert_allclose(oracle.silu(v) - oracle.silu(-v), v, rtol=0, atol=1e-13)


def test_swiglu_pairs_gate_with_up_of_the_same_column():
    y = np.array([[1.0, 2.0, 3.0, 10.0, 20.0, 30.0]])
    got = oracle.swiglu(y, 3)
    expect = np.array([[10.0 / (1 + math.exp(-1.0)), 20.0 * 2 / (1 + math.exp(-2.0)), 30.0 * 3 / (1 + math.exp(-3.0))]])
    np.testing.assert_allclose(got, expect, rtol=1e-15)


def test_forward_fast_rows_is_a_restriction_of_forward_fast():
    rng = np.random.default_rng(12)
    w = (rng.standard_normal((40, 192)) * 0.02).astype(np.float32)
    q, s16, b16 = oracle.quantize_rtn(w, 4)
    packed = oracle.pack(q, 4)
    x = rng.standard_normal((30, 192)).astype(np.float32)
    x[4] *= 1e5
    xb = inputs.f32_to_bf16_bits(x)
    full = oracle.forward_fast(xb, packed, s16, b16, 4, 192)
    rows, cols = np.array([0, 4, 29]), np.array([3, 17, 39])
    assert np.array_equal(oracle.forward_fast_rows(xb, packed, s16, b16, 4, 192, rows, cols), full[rows][:, cols])


def test_swiglu_fast_definition_error_budget():
    # the FAST numerics (fp16 weights) carried through silu(g) * u stay within
    # the FAST budget of relative Frobenius error against the exact product
    rng = np.random.default_rng(13)
    F, K = 64, 512
    w = (rng.standard_normal((2 * F, K)) * 0.02).astype(np.float32)
    q, s16, b16 = oracle.quantize_rtn(w, 4)
    packed = oracle.pack(q, 4)
    xb = inputs.f32_to_bf16_bits(rng.standard_normal((48, K)).astype(np.float32))
    fast = oracle.swiglu(oracle.forward_fast(xb, packed, s16, b16, 4, K), F)
    exact = oracle.swiglu(oracle.forward(xb, packed, s16, b16, 4, K), F)
    e = oracle.error_metrics(fast, exact)
    assert 1e-5 < e["relF"] < 5e-4, e


# ---- AdaLN gated residual update ---------------------------------------------

def test_gate_residual_hand_worked():
    # 3 rows, 2 rows per sample: rows 0 and 1 take gate row 0, row 2 gate row 1
    y = np.array([[1.0, 2.0], [3.0, 4.0], [5.0, 6.0]])
    res = np.array([[10.0, 20.0], [30.0, 40.0], [50.0, 60.0]])
    gate = np.array([[2.0, -1.0], [0.5, 3.0]])
    got = oracle.gate_residual(y, res, gate, 2)
    assert np.array_equal(got, np.array([[12.0, 18.0], [36.0, 36.0], [52.5, 78.0]]))


def test_gate_residual_special_cases():
    rng = np.random.default_rng(14)
    y, res = rng.standard_normal((7, 5)), rng.standard_normal((7, 5))
    # a closed gate leaves the residual stream untouched
    assert np.array_equal(oracle.gate_residual(y, res, np.zeros((4, 5)), 2), res)
    # an open gate on an empty stream is the branch output itself
    assert np.array_equal(oracle.gate_residual(y, np.zeros_like(y), np.ones((1, 5)), 7), y)
    # one sample: every row uses gate row 0, which scales columns
    g = rng.standard_normal((1, 5))
    np.testing.assert_allclose(oracle.gate_residual(y, res, g, 100), res + y @ np.diag(g[0]), rtol=1e-15)
    # per-row gates (one row per sample) equal the elementwise product
    g7 = rng.standard_normal((7, 5))
    np.testing.assert_allclose(oracle.gate_residual(y, res, g7, 1), res + g7 * y, rtol=1e-15)


# ---- AdaLN scale application ----------------------------------------------

def _bf16(vals):
    return inputs.f32_to_bf16_bits(np.asarray(vals, dtype=np.float32))


def test_adaln_modulate_hand_worked():
    # 3 rows of K = 2 (exact in bf16), 2 rows per sample: rows 0, 1 take scale row 0
    x = _bf16([[1.0, 2.0], [-3.0, 0.5], [4.0, -8.0]])
    scale = np.array([[0.5, -0.25], [1.0, -1.5]])
    got = oracle.adaln_modulate(x, scale, 2)
    assert np.array_equal(got, np.array([[1.5, 1.5], [-4.5, 0.375], [8.0, 4.0]]))


def test_adaln_modulate_special_cases():
    x = inputs.activations_bf16(6, 64, 71)
    xf = oracle.bf16_bits_to_f64(x)
    # zero scale is the identity, scale -1 annihilates, scale 1 doubles (exact)
    assert np.array_equal(oracle.adaln_modulate(x, np.zeros((2, 64)), 3), xf)
    assert np.array_equal(oracle.adaln_modulate(x, -np.ones((1, 64)), 6), np.zeros_like(xf))
    assert np.array_equal(oracle.adaln_modulate(x, np.ones((6, 64)), 1), 2.0 * xf)


def test_adaln_forward_brute_force():
    # y[m, n] = sum_k x[m, k] (1 + s[m // r, k]) W[n, k], one term at a time
    rng = np.random.default_rng(72)
    M, N, K, r = 5, 3, 64, 2
    w = inputs.weights(N, K, 73)
    q, s16, b16 = oracle.quantize_rtn(w, 4)
    packed = oracle.pack(q, 4)
    x = inputs.activations_bf16(M, K, 74)
    scale = rng.uniform(-0.9, 0.9, size=(3, K))
    got = oracle.forward_modulated(x, scale, r, packed, s16, b16, 4, K)
    xf = oracle.bf16_bits_to_f64(x)
    wf = oracle.dequantize(q, s16, b16).astype(np.float64)
    for m in range(M):
        for n in range(N):
            ref = math.fsum(xf[m, k] * (1.0 + scale[m // r, k]) * wf[n, k] for k in range(K))
            assert abs(got[m, n] - ref) <= 1e-12 * math.fsum(abs(xf[m, k] * wf[n, k]) * 2 for k in range(K))


def test_adaln_scale_acts_on_input_channels():
    # for one sample, scaling input channel k equals scaling column k of the
    # weights: x_mod @ W^T == x @ (W * (1 + s))^T (N != K, so a scale indexed
    # by output channel would not even broadcast)
    rng = np.random.default_rng(75)
    M, N, K = 4, 5, 128
    w = inputs.weights(N, K, 76)
    q, s16, b16 = oracle.quantize_rtn(w, 8)
    packed = oracle.pack(q, 8)
    x = inputs.activations_bf16(M, K, 77)
    scale = rng.uniform(-1.0, 1.0, size=(1, K))
    got = oracle.forward_modulated(x, scale, M, packed, s16, b16, 8, K)
    wf = oracle.dequantize(q, s16, b16).astype(np.float64)
    ref = oracle.bf16_bits_to_f64(x) @ (wf * (1.0 + scale[0])[None, :]).T
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


# ---- importance-weighted fit (the pages' imatrix objective) ---------------

def _outlier_importance(k, wid):
    x = inputs.activations_f32(64, k, wid, "outlier").astype(np.float64)
    return (x * x).mean(axis=0).astype(np.float32)


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_imatrix_never_worse_than_rtn(bits):
    # candidate 0 is the min/max RTN fit, so the objective never increases
    w = inputs.weights(96, 512, 60 + bits)
    imp = _outlier_importance(512, 60 + bits)
    q, s16, b16 = oracle.quantize_imatrix(w, imp, bits)
    q0, s0, b0 = oracle.quantize_rtn(w, bits)
    e = oracle.weighted_error(w, imp, q, s16, b16)
    e0 = oracle.weighted_error(w, imp, q0, s0, b0)
    assert np.all(e <= e0 * (1 + 1e-6) + 1e-30)
    assert e.sum() < 0.6 * e0.sum()   # and it helps on outlier-channel importance
    assert q.max() <= 2 ** bits - 1


def test_imatrix_keeps_rtn_when_rtn_is_exact():
    # weights exactly on an f16 affine grid: RTN has zero error, every later
    # candidate can at best tie, and ties keep candidate 0
    q = np.tile(np.arange(16, dtype=np.float32), 4)[None, :]
    w = (np.float32(0.125) * q + np.float32(-1.0)).astype(np.float32)
    imp = np.linspace(0.5, 2.0, 64).astype(np.float32)
    got = oracle.quantize_imatrix(w, imp, 4)
    ref = oracle.quantize_rtn(w, 4)
    for a_, b_ in zip(got, ref):
        assert np.array_equal(a_, b_)


def test_imatrix_ignores_an_outlier_in_an_unweighted_channel():
    # 63 weighted values spread over [0, 0.3] and one value 10 whose channel
    # has zero importance: RTN's step (10/15) maps every weighted value to
    # code 0; the fit over the weighted range reproduces them closely
    w = np.concatenate([np.linspace(0, 0.3, 63), [10.0]]).astype(np.float32)[None, :]
    imp = np.ones(64, np.float32)
    imp[63] = 0
    q, s16, b16 = oracle.quantize_imatrix(w, imp, 4)
    q0, s0, b0 = oracle.quantize_rtn(w, 4)
    e = oracle.weighted_error(w, imp, q, s16, b16)[0, 0]
    e0 = oracle.weighted_error(w, imp, q0, s0, b0)[0, 0]
    assert e0 > 1.0 and e < 0.01 * e0
    # the half-step bound of a uniform grid over [0, 0.3] with 15 steps
    wh = oracle.dequantize(q, s16, b16)[0, :63].astype(np.float64)
    assert np.max(np.abs(wh - w[0, :63])) <= 0.3 / 15 / 2 * 1.1


def test_imatrix_is_invariant_to_scaling_importance_by_two():
    # the objective scales by exactly 2 in fp32, so every comparison, and so
    # the chosen fit, is unchanged bit for bit
    w = inputs.weights(32, 256, 64)
    imp = _outlier_importance(256, 64)
    a = oracle.quantize_imatrix(w, imp, 4)
    b = oracle.quantize_imatrix(w, imp * np.float32(2), 4)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_imatrix_rejects_bad_importance():
    w = inputs.weights(4, 64, 65)
    for bad in (np.full(64, -1.0, np.float32), np.full(64, np.nan, np.float32), np.ones(32, np.float32)):
        with pytest.raises(ValueError):
            oracle.quantize_imatrix(w, bad, 4)
