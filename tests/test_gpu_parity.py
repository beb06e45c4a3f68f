"""GPU parity of every libqlinear kernel against the CPU oracle.

Inputs come from the seeded generators; quantization and packing of the test
weights are done by the oracle on the CPU; the library only receives those
bytes. Bit-exact checks: dequantized weights, device quantizer output, identity
and zero inputs. Float outputs: the product's tolerance (relF <= 2e-3,
max|err| <= 1e-2 rms) plus the tighter bound of the exact-integer and split
designs (EXACT and SPLIT numerics; FAST has tests of its own).
"""
import numpy as np
import pytest

import oracle
from group_wise_affine_qlinear_amd import inputs
from group_wise_affine_qlinear_amd import qlinear as ql

from gpu_helpers import (Case, assert_parity, assert_rows, dev, gemv_serves, host_u16, host_u32, run_forward,
                         torch_or_skip)

EXACT_MODES = (ql.QL_MODE_EXACT, ql.QL_MODE_SPLIT)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    t = torch_or_skip()
    ql.load_library()
    return t


# ------------------------------------------------------------------ dequantize / quantize

@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_dequantize_bit_exact(torch, bits):
    c = Case(1, 300, 512, bits, wid=201)
    _, p, s, b = c.device(torch)
    w_out = torch.empty((c.N, c.K), dtype=torch.float32, device="cuda")
    ql.qlinear_dequantize(p, s, b, bits, 64, c.N, c.K, w_out)
    torch.cuda.synchronize()
    ref = oracle.dequantize(c.q, c.s16, c.b16)
    got = w_out.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_device_quantizer_byte_equal(torch, bits):
    w = inputs.weights(257, 1024, workload_id=202)
    # adversarial rows: exact grid, ties, constant, signed zeros, tiny scales
    k = np.arange(1024, dtype=np.float32)
    w[0] = -1 + 0.125 * (k % 16)
    w[1] = 0.0
    w[1, 1::2] = -0.0
    w[2] = 0.3
    w[3] = (k % 64) * 1e-7
    w[4] = (k % 64) * 3e-9
    s01 = np.float32(np.float16(0.1))
    w[5] = 0.0
    w[5, 1] = 1.5
    w[5, 2] = 2.5 * s01
    w[5, 3] = 3.5 * s01
    wd = dev(torch, w)
    N, K = w.shape
    packed = torch.zeros((N, K * bits // 32), dtype=torch.int32, device="cuda")
    s = torch.zeros((N, K // 64), dtype=torch.int16, device="cuda")
    b = torch.zeros((N, K // 64), dtype=torch.int16, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ql.qlinear_quantize_rtn(wd, bits, 64, N, K, packed, s, b, status)
    torch.cuda.synchronize()
    qo, so, bo = oracle.quantize_rtn(w, bits)
    assert int(status.item()) == 0
    assert np.array_equal(host_u16(s), so)
    assert np.array_equal(host_u16(b), bo)
    assert np.array_equal(host_u32(packed), oracle.pack(qo, bits))


def test_device_quantizer_flags_range_error(torch):
    w = np.zeros((2, 64), np.float32)
    w[1, 7] = 1e6
    wd = dev(torch, w)
    packed = torch.zeros((2, 8), dtype=torch.int32, device="cuda")
    s = torch.zeros((2, 1), dtype=torch.int16, device="cuda")
    b = torch.zeros((2, 1), dtype=torch.int16, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ql.qlinear_quantize_rtn(wd, 4, 64, 2, 64, packed, s, b, status)
    torch.cuda.synchronize()
    assert int(status.item()) == ql.QL_ERANGE


# ------------------------------------------------------------------ forward: small cases, all paths

def test_tiny_config_all_paths(torch):
    """M=64, K=512, N=256, 4-bit, seed 0: the tiny workload, full comparison."""
    wl = inputs.WORKLOADS["tiny"]
    w, x = inputs.workload_inputs("tiny")
    c = Case(wl["M"], wl["N"], wl["K"], 4, wid=wl["id"], w=w, x=x)
    ref = c.reference()
    y = run_forward(torch, c, via_ex=False)   # FAST converting x in the GEMM: the acceptance bar
    assert_rows(y.cpu().numpy(), ref, what="qlinear_forward")
    for mode in EXACT_MODES:
        for path in (ql.QL_PATH_GEMM, ql.QL_PATH_SPLITK):
            y = run_forward(torch, c, path=path, mode=mode)
            assert_parity(y.cpu().numpy(), ref, what=f"path {path} {ql.qlinear_last_path()}")


GEMM_SHAPES = [(200, 300, 1024), (129, 129, 192), (17, 40, 64), (384, 256, 512)]


@pytest.mark.parametrize("mode", EXACT_MODES)
@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("shape", GEMM_SHAPES)
def test_gemm_ragged(torch, bits, shape, mode):
    M, N, K = shape
    c = Case(M, N, K, bits, wid=210 + bits)
    ref = c.reference()
    y = run_forward(torch, c, path=ql.QL_PATH_GEMM, mode=mode)
    assert_parity(y.cpu().numpy(), ref, what=ql.qlinear_last_path())
    if K >= 128:
        y = run_forward(torch, c, path=ql.QL_PATH_SPLITK, split_k=3, mode=mode)
        assert_parity(y.cpu().numpy(), ref, what=ql.qlinear_last_path())


@pytest.mark.parametrize("tile", [1, 2, 3, 5, 10, 11])
def test_gemm_every_tile(torch, tile):
    c = Case(300, 520, 640, 4, wid=220, x_structure="outlier")
    ref = c.reference()
    y = run_forward(torch, c, path=ql.QL_PATH_GEMM, tile=tile)
    assert_parity(y.cpu().numpy(), ref, what=ql.qlinear_last_path())


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("M", [1, 3, 8, 9, 16])
def test_skinny_ragged(torch, bits, M):
    c = Case(M, 300, 1536, bits, wid=230 + M)
    ref = c.reference()
    y = run_forward(torch, c, path=ql.QL_PATH_SKINNY)
    # one or two rows on canonical weights run the lane-along-K GEMV of the skinny path
    assert ql.qlinear_last_path().startswith("gemv" if gemv_serves(bits, M, c.K) else "skinny"), ql.qlinear_last_path()
    assert_parity(y.cpu().numpy(), ref, what=ql.qlinear_last_path())


# ------------------------------------------------------------------ exact special cases

def _identity_x(M, K, cols):
    x = np.zeros((M, K), np.uint16)
    x[np.arange(M), cols] = 0x3F80
    return x


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("path", [ql.QL_PATH_GEMM, ql.QL_PATH_SPLITK, ql.QL_PATH_SKINNY])
def test_identity_rows_give_weights_exactly(torch, bits, path):
    K, N = 512, 136
    M = 16 if path == ql.QL_PATH_SKINNY else K
    cols = np.arange(M) if M == K else np.array([0, 1, 63, 64, 100, 127, 128, 200, 255, 256, 300, 383, 384, 450, 510, 511])
    w = inputs.weights(N, K, 240)
    c = Case(M, N, K, bits, wid=240, w=w, x=_identity_x(M, K, cols))
    y = run_forward(torch, c, path=path, split_k=4 if path == ql.QL_PATH_SPLITK else 0,
                    mode=ql.QL_MODE_AUTO if path == ql.QL_PATH_SKINNY else ql.QL_MODE_EXACT).cpu().numpy()
    w_hat = oracle.dequantize(c.q, c.s16, c.b16)
    expect = w_hat[:, cols].T
    if bits == 8:
        assert np.array_equal(y, expect)
    else:
        # with the 128 offset the bias enters as b - 128*s; bit-exact wherever that is exact in fp32
        s = oracle.f16_bits_to_f32(c.s16).astype(np.float64)
        b = oracle.f16_bits_to_f32(c.b16).astype(np.float64)
        exact_b = (b - 128 * s) == (b.astype(np.float32) - np.float32(128) * s.astype(np.float32)).astype(np.float64)
        ok = np.repeat(exact_b, 64, axis=1)[:, cols].T
        assert ok.mean() > 0.99
        assert np.array_equal(y[ok], expect[ok])
        assert np.allclose(y, expect, rtol=2e-7, atol=0)


@pytest.mark.parametrize("path", [ql.QL_PATH_GEMM, ql.QL_PATH_SKINNY])
def test_zero_x_gives_zero(torch, path):
    M = 8 if path == ql.QL_PATH_SKINNY else 100
    c = Case(M, 70, 256, 4, wid=250, x=np.zeros((M, 256), np.uint16))
    y = run_forward(torch, c, path=path).cpu().numpy()
    assert not y.any()


def test_k_zero_and_empty(torch):
    out = torch.full((5, 7), 3.0, dtype=torch.float32, device="cuda")
    x = torch.zeros((5, 0), dtype=torch.int16, device="cuda")
    p = torch.zeros((7, 0), dtype=torch.int32, device="cuda")
    s = torch.zeros((7, 0), dtype=torch.int16, device="cuda")
    ql.qlinear_forward_ex(x, p, s, s, 4, 5, 7, 0, out)
    torch.cuda.synchronize()
    assert not out.cpu().numpy().any()
    out0 = torch.zeros((0, 7), dtype=torch.float32, device="cuda")
    ql.qlinear_forward_ex(torch.zeros((0, 64), dtype=torch.int16, device="cuda"),
                          torch.zeros((7, 8), dtype=torch.int32, device="cuda"),
                          torch.zeros((7, 1), dtype=torch.int16, device="cuda"),
                          torch.zeros((7, 1), dtype=torch.int16, device="cuda"), 4, 0, 7, 64, out0)
    assert ql.qlinear_last_path() == "noop"


@pytest.mark.parametrize("mode", EXACT_MODES)
@pytest.mark.parametrize("path", [ql.QL_PATH_GEMM, ql.QL_PATH_SPLITK, ql.QL_PATH_SKINNY])
def test_bf16_output_within_one_ulp(torch, path, mode):
    M = 12 if path == ql.QL_PATH_SKINNY else 150
    if path == ql.QL_PATH_SKINNY:
        mode = ql.QL_MODE_AUTO
    c = Case(M, 200, 768, 4, wid=260)
    ref = c.reference()
    y = run_forward(torch, c, path=path, out_dtype="bf16", mode=mode)
    got = y.float().cpu().numpy().astype(np.float64)
    ref_bf = oracle.bf16_bits_to_f64(inputs.f32_to_bf16_bits(ref.astype(np.float32)))
    rms = np.sqrt(np.mean(ref ** 2))
    # one bf16 ulp of the value, plus the fp32 design error that can move a near-tie
    assert np.all(np.abs(got - ref_bf) <= np.abs(ref) * 2.0 ** -7 + 1e-5 * rms)


def test_deterministic(torch):
    c = Case(256, 384, 2048, 4, wid=270)
    y1 = run_forward(torch, c, path=ql.QL_PATH_SPLITK, split_k=4).cpu().numpy()
    y2 = run_forward(torch, c, path=ql.QL_PATH_SPLITK, split_k=4).cpu().numpy()
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    c = Case(8, 384, 2048, 4, wid=271)
    y1 = run_forward(torch, c).cpu().numpy()
    y2 = run_forward(torch, c).cpu().numpy()
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))


def test_caller_workspace_and_stream(torch):
    c = Case(300, 256, 1024, 4, wid=280)
    ref = c.reference()
    need = ql.qlinear_workspace_bytes(4, c.M, c.N, c.K)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    x, p, s, b = c.device(torch)
    out = torch.empty((c.M, c.N), dtype=torch.float32, device="cuda")
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        ql.qlinear_forward_ex(x, p, s, b, 4, c.M, c.N, c.K, out, workspace=ws, stream=stream,
                              mode=ql.QL_MODE_EXACT)
    stream.synchronize()
    assert_parity(out.cpu().numpy(), ref)
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(ql.QLinearError) as e:
        ql.qlinear_forward_ex(x, p, s, b, 4, c.M, c.N, c.K, out, workspace=small, mode=ql.QL_MODE_EXACT)
    assert e.value.status == ql.QL_EWORKSPACE


# ------------------------------------------------------------------ degenerate groups and rows

def degenerate_case(M, N, K, bits, wid):
    """Weights with the method's degenerate groups: constant groups (scale 0),
    groups of +0/-0, groups whose range is a few f16 subnormal steps, a row of
    exact grid points and a row spanning +-1e3; activations with an all-zero
    row, a row of large values (2^20 range, scaled per row by the FAST
    prepass) and a row of tiny values."""
    w = inputs.weights(N, K, wid)
    k = np.arange(K, dtype=np.float32)
    w[0] = 0.25                        # constant: scale 0, W_hat = b
    w[1] = 0.0
    w[1, 1::2] = -0.0                  # signed zeros
    w[2] = (k % 64) * np.float32(3e-9)    # range below the smallest normal f16 step
    w[3] = -1 + np.float32(0.125) * (k % 16)  # exact grid points
    w[4] = np.where(k % 2 == 0, 1e3, -1e3).astype(np.float32)
    w[5, :64] = 7.0                    # one constant group in an otherwise normal row
    x = inputs.activations_f32(M, K, wid)
    x[0] = 0.0
    x[1] *= np.float32(2.0 ** 20)
    x[2] *= np.float32(2.0 ** -30)
    return Case(M, N, K, bits, wid=wid, w=w, x=inputs.f32_to_bf16_bits(x))


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_degenerate_groups_every_path(torch, bits):
    """Every numerics mode and path on the degenerate groups and rows, against
    the plain product at the acceptance bar on the whole output and on every
    row at its own scale (rows of x differ in magnitude by 2^50)."""
    c = degenerate_case(40, 96, 256, bits, wid=260 + bits)
    ref = c.reference()
    runs = [dict(path=ql.QL_PATH_GEMM, mode=ql.QL_MODE_EXACT), dict(path=ql.QL_PATH_SPLITK, mode=ql.QL_MODE_EXACT),
            dict(path=ql.QL_PATH_GEMM, mode=ql.QL_MODE_SPLIT), dict(path=ql.QL_PATH_SPLITK, mode=ql.QL_MODE_SPLIT),
            dict(path=ql.QL_PATH_GEMM, mode=ql.QL_MODE_FAST), dict(path=ql.QL_PATH_SPLITK, mode=ql.QL_MODE_FAST),
            dict(path=ql.QL_PATH_SKINNY, m=16),
            dict(path=ql.QL_PATH_GEMM, layout=ql.QL_LAYOUT_TILED, mode=ql.QL_MODE_EXACT),
            dict(path=ql.QL_PATH_GEMM, layout=ql.QL_LAYOUT_TILED, mode=ql.QL_MODE_SPLIT),
            dict(path=ql.QL_PATH_GEMM, layout=ql.QL_LAYOUT_TILED, mode=ql.QL_MODE_FAST),
            dict(path=ql.QL_PATH_SKINNY, layout=ql.QL_LAYOUT_TILED, m=16)]
    xa = np.abs(oracle.bf16_bits_to_f64(c.x))
    wa = np.abs(oracle.dequantize(c.q, c.s16, c.b16).astype(np.float64))
    for kw in runs:
        m = kw.pop("m", c.M)
        cc = c if m == c.M else Case(m, c.N, c.K, bits, wid=0, w=c.w, x=c.x[:m])
        y = run_forward(torch, cc, **kw).cpu().numpy()
        # the zero row of x gives exactly zero
        assert np.all(y[0] == 0.0), ql.qlinear_last_path()
        if kw.get("mode") != ql.QL_MODE_FAST:
            # acceptance bar, row by row: the exact mode's affine fold s*P + (b - 128 s)*sum(x)
            # cancels large terms when a row of x is huge and a weight group spans
            # +-1e3, so its fp32 rounding exceeds the design bound here
            assert_rows(y, ref[:m], what=(ql.qlinear_last_path(), kw))
            continue
        # FAST rounds each weight once to fp16 (2^-11 relative). Its error is
        # bounded relative to sum_k |x||W|, not to |y|: on the column of +-1e3
        # weights (fp16 ulp 0.5) an output that nearly cancels keeps an error
        # of 0.25 * |sum x|, a percent of that output and, next to the row of x
        # scaled by 2^20, ~1.5e-2 of the result's rms (above the max-abs bar;
        # EXACT and SPLIT meet it). The relative Frobenius error of the whole
        # result stays within the bar, and every element obeys the bound of one
        # fp16 rounding per weight plus fp32 accumulation of K terms,
        # (2^-11 + K 2^-24) sum_k |x||W|, which scales with each row.
        assert oracle.error_metrics(y, ref[:m])["relF"] <= 2e-3, ql.qlinear_last_path()
        bound = (2.0 ** -11 + c.K * 2.0 ** -24) * (xa[:m] @ wa.T)
        assert np.all(np.abs(y - ref[:m]) <= bound), ql.qlinear_last_path()
    # FAST also against its written-out model (the large row is scaled by a
    # power of two on the way to fp16, so its products keep their accuracy)
    y = run_forward(torch, c, layout=ql.QL_LAYOUT_TILED, mode=ql.QL_MODE_FAST).cpu().numpy()
    ref_fast = oracle.forward_fast(c.x, c.packed, c.s16, c.b16, bits, c.K)
    assert_parity(y, ref_fast, what=ql.qlinear_last_path())   # fp32 accumulation only: design bound
