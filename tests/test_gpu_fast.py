"""GPU tests of the FAST numerics mode (fp16 dequant-GEMM).

Every case is compared with the oracle's plain fp64 product (``oracle.forward``,
the format's definition) at the acceptance bar, on the whole result and row by
row against each row's own scale, and under the mode's error budget (fp16
half-ulp on the weights). Cases are also compared with the oracle's
written-out model of the mode (``oracle.forward_fast``: weights rounded once
to fp16, rows scaled by a power of two into fp16), where only fp32
accumulation separates the two."""
import numpy as np
import pytest

import oracle
from group_wise_affine_qlinear_amd import inputs, qlinear as ql

from gpu_helpers import (Case, MAXABS_RMS_DESIGN, MAXABS_RMS_TOL, RELF_DESIGN, RELF_TOL, assert_parity, assert_rows,
                         dev, run_forward, torch_or_skip)

pytestmark = pytest.mark.gpu

# error budget of the mode against the exact product: fp16 rounding of W
# (relative ~2^-11/sqrt(3) per weight, 1.7e-4 relative Frobenius on these
# weights) with room for the max over ~1e6 outputs
RELF_FAST = 5e-4
MAXABS_RMS_FAST = 4e-3


@pytest.fixture(scope="module")
def torch():
    t = torch_or_skip()
    ql.load_library()
    return t


def check_fast(y, c):
    y = np.asarray(y, dtype=np.float64)
    assert np.all(np.isfinite(y)), "non-finite output"
    ref_def = oracle.forward_fast(c.x, c.packed, c.s16, c.b16, c.bits, c.K)
    e = oracle.error_metrics(y, ref_def)
    assert e["relF"] <= RELF_DESIGN and e["maxabs_over_rms"] <= MAXABS_RMS_DESIGN, ("vs definition", e)
    ref = c.reference()
    assert_rows(y, ref, what="vs exact, acceptance, row by row")
    e2 = oracle.error_metrics(y, ref)
    assert e2["relF"] <= RELF_FAST and e2["maxabs_over_rms"] <= MAXABS_RMS_FAST, ("vs exact, budget", e2)


FAST_SHAPES = [(520, 390, 320), (300, 520, 640), (17, 40, 64), (256, 256, 512), (777, 1000, 448)]


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("shape", FAST_SHAPES)
def test_fast_parity(torch, shape, bits):
    M, N, K = shape
    c = Case(M, N, K, bits, wid=400 + bits, x_structure="outlier")
    y = run_forward(torch, c, layout=ql.QL_LAYOUT_TILED, mode=ql.QL_MODE_FAST)
    assert ql.qlinear_last_path().startswith("gemm3"), ql.qlinear_last_path()
    check_fast(y.cpu().numpy(), c)


def test_fast_is_auto_choice_with_a_workspace(torch):
    c = Case(64, 256, 256, 4, wid=410)
    run_forward(torch, c, layout=ql.QL_LAYOUT_TILED)
    assert ql.qlinear_last_path().startswith("gemm3")
    run_forward(torch, c)
    assert ql.qlinear_last_path().startswith("gemm3") and ql.qlinear_last_path().endswith("_canonical")
    # no workspace and no fp16 activations: FAST converting x inside the GEMM
    x, p, s, b = c.device(torch)
    out = torch.empty((c.M, c.N), dtype=torch.float32, device="cuda")
    ql.qlinear_forward_ex(x, p, s, b, 4, c.M, c.N, c.K, out, workspace=None)
    assert ql.qlinear_last_path().startswith("gemm3_f16online"), ql.qlinear_last_path()
    run_forward(torch, c, layout=ql.QL_LAYOUT_TILED, mode=ql.QL_MODE_EXACT)
    assert ql.qlinear_last_path().startswith("gemm2")
    c8 = Case(8, 256, 256, 4, wid=411)   # skinny M is always exact
    run_forward(torch, c8, layout=ql.QL_LAYOUT_TILED)
    assert ql.qlinear_last_path().startswith("skinny")


def test_fast_rejects_unsupported_requests(torch):
    with pytest.raises(ql.QLinearError):   # a K split needs two groups at least
        run_forward(torch, Case(64, 256, 64, 4, wid=414), layout=ql.QL_LAYOUT_TILED, mode=ql.QL_MODE_FAST,
                    path=ql.QL_PATH_SPLITK)
    with pytest.raises(ql.QLinearError):   # skinny path
        run_forward(torch, Case(4, 256, 256, 4, wid=413), layout=ql.QL_LAYOUT_TILED, mode=ql.QL_MODE_FAST,
                    path=ql.QL_PATH_SKINNY)


def test_fast_rows_scaled_into_fp16_range(torch):
    M, N, K = 64, 256, 512
    x = inputs.activations_f32(M, K, 420)
    x[3] *= 1.0e5          # |x| up to ~5e5: needs e > 0
    x[7, 100] = 70000.0    # one large value in an otherwise normal row
    x[11] *= 2.0 ** -20    # small row: values in the fp16 subnormal range
    c = Case(M, N, K, 4, wid=420, x=inputs.f32_to_bf16_bits(x))
    y = run_forward(torch, c, layout=ql.QL_LAYOUT_TILED, mode=ql.QL_MODE_FAST).cpu().numpy()
    ref_def = oracle.forward_fast(c.x, c.packed, c.s16, c.b16, 4, K)
    for r in range(M):   # row by row: the rows differ in scale by 10^5
        e = oracle.error_metrics(y[r:r + 1], ref_def[r:r + 1])
        assert e["relF"] <= RELF_DESIGN, (r, e)
    # and against the plain product, each row at its own scale
    assert_rows(y, c.reference(), what="vs exact, row by row")


def test_fast_one_hot_rows_give_fp16_weights_exactly(torch):
    K, N, M = 512, 100, 24
    cols = np.arange(M) * 21 % K
    x = np.zeros((M, K), np.uint16)
    x[np.arange(M), cols] = 0x3F80   # 1.0
    c = Case(M, N, K, 4, wid=430, x=x)
    y = run_forward(torch, c, layout=ql.QL_LAYOUT_TILED, mode=ql.QL_MODE_FAST).cpu().numpy()
    w16 = oracle.fast_weights_f16(c.q, c.s16, c.b16).astype(np.float32)
    assert np.array_equal(y, w16[:, cols].T)
    # against the format's definition: each returned weight lies within the
    # fp16 half-ulp (2^-11 relative, or 2^-25 absolute below 2^-14) of W_hat
    w_hat = oracle.dequantize(c.q, c.s16, c.b16).astype(np.float64)[:, cols].T
    assert np.all(np.abs(y - w_hat) <= np.maximum(np.abs(w_hat) * 2.0 ** -11, 2.0 ** -25))


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_fast_bf16_out_is_rounded_fp32_out(torch, bits):
    c = Case(300, 260, 384, bits, wid=440 + bits)
    y = run_forward(torch, c, layout=ql.QL_LAYOUT_TILED, mode=ql.QL_MODE_FAST).cpu().numpy()
    yb = run_forward(torch, c, layout=ql.QL_LAYOUT_TILED, mode=ql.QL_MODE_FAST, out_dtype="bf16")
    got = yb.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, inputs.f32_to_bf16_bits(y))


# tail pieces and multi-tile blocks with the resident-block count forced small:
# (slots, shape). Tiles are 256 x 256; tail tiles are cut along M into pieces
# of 128, 64 or 32 rows; pieces wholly past M are skipped.
FAST_TAIL_CASES = [
    (4, (520, 1000, 640)),    # 12 tiles over 4 blocks: 3 whole tiles per block, no pieces
    (3, (300, 600, 448)),     # 6 tiles over 3 blocks: 2 whole tiles per block (G=7, odd)
    (9, (600, 1100, 320)),    # 15 tiles, 6 past 9: too many for pieces, whole tiles only
    (5, (520, 1000, 640)),    # 12 tiles: 10 whole, 2 tail tiles x 2 pieces of 128 rows (tile row: 8 rows)
    (4, (300, 600, 448)),     # 6 tiles: 4 whole, 2 tail tiles x 2 pieces (rows 256..299: one partial piece)
    (6, (700, 600, 384)),     # 9 tiles: 6 whole, 3 tail tiles x 2 pieces (rows 512..699)
    (12, (512, 1792, 320)),   # 14 tiles: 12 whole, 2 tail tiles x 4 pieces of 64 rows
    (17, (800, 1280, 320)),   # 20 tiles: 17 whole, 3 tail tiles x 4 pieces (rows 768..799)
    (8, (1030, 512, 256)),    # 10 tiles: 8 whole, 2 tail tiles x 4 pieces (rows 1024..1029)
    (17, (300, 2304, 448)),   # 18 tiles: 17 whole, 1 tail tile x 8 pieces of 32 rows (rows 256..299)
    (9, (256, 2560, 320)),    # 10 tiles: 9 whole, 1 tail tile x 8 pieces
    (33, (768, 3072, 320)),   # 36 tiles: 33 whole, 3 tail tiles x 8 pieces
    (33, (520, 3072, 320)),   # same grid, tail tiles hold rows 512..519 only: 7 of 8 pieces skipped
]


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("slots,shape", FAST_TAIL_CASES)
def test_fast_split_tail(torch, monkeypatch, slots, shape, bits):
    M, N, K = shape
    monkeypatch.setenv("QLINEAR_GEMM_SLOTS", str(slots))
    c = Case(M, N, K, bits, wid=450 + bits)
    y1 = run_forward(torch, c, layout=ql.QL_LAYOUT_TILED, mode=ql.QL_MODE_FAST).cpu().numpy()
    check_fast(y1, c)
    y2 = run_forward(torch, c, layout=ql.QL_LAYOUT_TILED, mode=ql.QL_MODE_FAST).cpu().numpy()
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))


@pytest.mark.parametrize("K", [4608, 8192, 9216])
def test_fast_prepass_row_widths(torch, K):
    # rows held in registers (K <= 8192, two vector counts) and the two-pass
    # conversion for wider rows; one row per scale regime
    M, N = 40, 64
    x = inputs.activations_f32(M, K, 460)
    x[5] *= 3.0e5
    x[9] *= 2.0 ** -18
    c = Case(M, N, K, 4, wid=460, x=inputs.f32_to_bf16_bits(x))
    y = run_forward(torch, c, layout=ql.QL_LAYOUT_TILED, mode=ql.QL_MODE_FAST).cpu().numpy()
    ref_def = oracle.forward_fast(c.x, c.packed, c.s16, c.b16, 4, K)
    for r in range(M):
        e = oracle.error_metrics(y[r:r + 1], ref_def[r:r + 1])
        assert e["relF"] <= RELF_DESIGN, (r, e)
    assert_rows(y, c.reference(), what="vs exact, row by row")


def test_fast_activations_match_definition_bitwise(torch):
    # the standalone prepass: fp16 codes and row scales equal the oracle's
    # definition exactly (both round once, to nearest even)
    M, K = 70, 4608
    x = inputs.activations_f32(M, K, 470)
    x[2] *= 4.0e5
    x[6] *= 2.0 ** -19
    x[9, 17] = -65504.0 * 3
    xb = inputs.f32_to_bf16_bits(x)
    xd = dev(torch, xb)
    x16, rs = ql.qlinear_fast_activations(xd, M, K)
    torch.cuda.synchronize()
    ref16, refscale = oracle.fast_activations_f16(xb)
    assert np.array_equal(x16.cpu().numpy().view(np.uint16), ref16.view(np.uint16))
    assert np.array_equal(rs.cpu().numpy().astype(np.float64), np.asarray(refscale, np.float64))


def test_fast_forward_with_given_activations_is_identical(torch):
    M, N, K = 300, 520, 640
    c = Case(M, N, K, 4, wid=480, x_structure="outlier")
    x, p, s, b = c.device(torch)
    p, s = ql.qlinear_repack(p, s, b, 4, 64, N, K)
    y1 = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    y2 = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    ql.qlinear_forward_ex(x, p, s, None, 4, M, N, K, y1, layout=ql.QL_LAYOUT_TILED, mode=ql.QL_MODE_FAST)
    x16, rs = ql.qlinear_fast_activations(x, M, K)
    ql.qlinear_forward_ex(x, p, s, None, 4, M, N, K, y2, layout=ql.QL_LAYOUT_TILED, mode=ql.QL_MODE_FAST,
                          x16=x16, rowscale=rs)
    torch.cuda.synchronize()
    assert np.array_equal(y1.cpu().numpy().view(np.uint32), y2.cpu().numpy().view(np.uint32))
    check_fast(y2.cpu().numpy(), c)


# K split (grid y) with fp32 partials and the ordered reduction: forced split
# counts, including uneven group ranges, and the automatic split of shapes with
# fewer tiles than CUs
FAST_SPLIT_CASES = [
    ((300, 520, 640), 2),      # G=10: 5+5
    ((300, 520, 640), 3),      # G=10: 4+4+2
    ((777, 300, 1344), 7),     # G=21: 3 x 7
    ((64, 1000, 4608), 0),     # automatic: 4 tiles, G=72
    ((512, 600, 8192), 0),     # automatic: 6 tiles, G=128
]


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("shape,splits", FAST_SPLIT_CASES)
def test_fast_split_k(torch, shape, splits, bits):
    M, N, K = shape
    c = Case(M, N, K, bits, wid=490 + bits, x_structure="outlier")
    path = ql.QL_PATH_SPLITK if splits else ql.QL_PATH_AUTO
    y = run_forward(torch, c, layout=ql.QL_LAYOUT_TILED, mode=ql.QL_MODE_FAST, path=path, split_k=splits)
    lp = ql.qlinear_last_path()
    assert lp.startswith("gemm3") and "_split" in lp, lp
    if splits:
        assert f"_split{len(range(0, K // 64, -(-(K // 64) // splits)))}_" in lp, lp
    check_fast(y.cpu().numpy(), c)
    yb = run_forward(torch, c, layout=ql.QL_LAYOUT_TILED, mode=ql.QL_MODE_FAST, path=path, split_k=splits,
                     out_dtype="bf16")
    got = yb.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, inputs.f32_to_bf16_bits(y.cpu().numpy()))


# canonical weights: the same kernel reads each row's code stream directly, so
# its result equals the tiled run bit for bit (same fp16 weights, same MFMA
# order, same tail pieces and K splits)
CANON_CASES = [(520, 390, 320, 0, 0), (300, 520, 640, 0, 0), (17, 40, 64, 0, 0), (700, 600, 384, 6, 0),
               (300, 2304, 448, 17, 0), (64, 600, 8192, 0, 5)]


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("case", CANON_CASES)
def test_fast_canonical_equals_tiled(torch, monkeypatch, case, bits):
    M, N, K, slots, splits = case
    if slots:
        monkeypatch.setenv("QLINEAR_GEMM_SLOTS", str(slots))
    c = Case(M, N, K, bits, wid=470 + bits, x_structure="outlier")
    path = ql.QL_PATH_SPLITK if splits else ql.QL_PATH_AUTO
    yt = run_forward(torch, c, layout=ql.QL_LAYOUT_TILED, mode=ql.QL_MODE_FAST, path=path, split_k=splits)
    pt = ql.qlinear_last_path()
    yc = run_forward(torch, c, mode=ql.QL_MODE_FAST, path=path, split_k=splits)
    pc = ql.qlinear_last_path()
    assert pc.endswith("_canonical") and pc.replace("_canonical", "_tiled") == pt, (pc, pt)
    assert torch.equal(yc, yt), (pc, (yc - yt).abs().max().item())
    check_fast(yc.cpu().numpy(), c)


def test_fast_canonical_bf16_and_auto_mode(torch):
    c = Case(300, 260, 384, 4, wid=480)
    y = run_forward(torch, c, mode=ql.QL_MODE_FAST).cpu().numpy()
    yb = run_forward(torch, c, mode=ql.QL_MODE_FAST, out_dtype="bf16")
    assert np.array_equal(yb.view(torch.int16).cpu().numpy().view(np.uint16), inputs.f32_to_bf16_bits(y))
    run_forward(torch, c)   # AUTO with a workspace: FAST on canonical weights too
    assert ql.qlinear_last_path().startswith("gemm3"), ql.qlinear_last_path()
