"""GPU tests of FAST numerics without a prepass (a FAST call with no workspace
and no fp16 activations): the GEMM converts the bf16 x to fp16 itself, with
no row scales, and a second launch recomputes with SPLIT numerics every tile
(or row piece) holding a row whose largest magnitude lies above 2^15 or,
nonzero, below 2^-6.

Checks: the oracle's plain fp64 product (``oracle.forward``) at the
acceptance bar, row by row, and under FAST's error budget; bit-identity with
the prepass FAST GEMM wherever the unscaled conversion is exact (every
nonzero |x| >= 2^-17: both then multiply the same fp16 values up to a power
of two per row, in the same order); tiles with an out-of-range row
bit-identical to the SPLIT GEMM's output, the others to FAST's."""
import re

import numpy as np
import pytest

import oracle
from group_wise_affine_qlinear_amd import inputs, qlinear as ql

from gpu_helpers import Case, assert_rows, torch_or_skip

pytestmark = pytest.mark.gpu

# FAST's budget against the exact product (fp16 rounding of W dominates; the
# conversion of x adds at most 2^-24 per value below 2^-17)
RELF_FAST = 5e-4
MAXABS_RMS_FAST = 4e-3


@pytest.fixture(scope="module")
def torch():
    t = torch_or_skip()
    ql.load_library()
    return t


def run_online(torch, c, layout=ql.QL_LAYOUT_CANONICAL, out_dtype="f32"):
    x, p, s, b = c.device(torch)
    if layout == ql.QL_LAYOUT_TILED:
        p, s = ql.qlinear_repack(p, s, b, c.bits, 64, c.N, c.K)
        b = None
    dt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    out = torch.full((c.M, c.N), float("nan"), dtype=dt, device="cuda")
    ql.qlinear_forward_ex(x, p, s, b, c.bits, c.M, c.N, c.K, out, layout=layout, mode=ql.QL_MODE_FAST,
                          workspace=None)
    path = ql.qlinear_last_path()
    torch.cuda.synchronize()
    assert path.startswith("gemm3_f16online"), path
    return out, path


def run_fast_given(torch, c, layout=ql.QL_LAYOUT_CANONICAL):
    """The prepass FAST GEMM on the same grid: the caller's fp16 activations
    from qlinear_fast_activations, no workspace (so no K split)."""
    x, p, s, b = c.device(torch)
    if layout == ql.QL_LAYOUT_TILED:
        p, s = ql.qlinear_repack(p, s, b, c.bits, 64, c.N, c.K)
        b = None
    x16, rs = ql.qlinear_fast_activations(x, c.M, c.K)
    out = torch.full((c.M, c.N), float("nan"), dtype=torch.float32, device="cuda")
    ql.qlinear_forward_ex(x, p, s, b, c.bits, c.M, c.N, c.K, out, layout=layout, mode=ql.QL_MODE_FAST,
                          x16=x16, rowscale=rs, workspace=None)
    path = ql.qlinear_last_path()
    torch.cuda.synchronize()
    assert path.startswith("gemm3_f16_"), path
    return out.cpu().numpy()


def check_online(y, c):
    y = np.asarray(y, dtype=np.float64)
    ref = c.reference()
    assert_rows(y, ref, what="vs exact, acceptance, row by row")
    e = oracle.error_metrics(y, ref)
    assert e["relF"] <= RELF_FAST and e["maxabs_over_rms"] <= MAXABS_RMS_FAST, ("vs exact, budget", e)


def away_from_zero(x_bf16, floor=2.0 ** -10, rows=None):
    """bf16 x with every nonzero magnitude below floor raised to floor (sign
    kept), in the given rows (default: all)."""
    x = (x_bf16.astype(np.uint32) << 16).view(np.float32).copy()
    sel = np.ones(x.shape[0], bool) if rows is None else np.isin(np.arange(x.shape[0]), rows)
    small = (x != 0) & (np.abs(x) < floor) & sel[:, None]
    x = np.where(small, np.copysign(np.float32(floor), x), x).astype(np.float32)
    return inputs.f32_to_bf16_bits(x)


def units(path, M, N):
    """The row ranges [r0, r1) x column blocks [n0, n0 + 256) the launch
    computed as one unit: whole 256 x 256 tiles, and the row pieces of the
    last tail tiles (path ..._tail<T>x<P>_...)."""
    tiles_m, tiles_n = -(-M // 256), -(-N // 256)
    total = tiles_m * tiles_n
    m = re.search(r"_tail(\d+)x(\d+)_", path)
    tail, pieces = (int(m.group(1)), int(m.group(2))) if m else (0, 1)
    out = []
    for t in range(total):
        r0, n0 = (t // tiles_n) * 256, (t % tiles_n) * 256
        if t >= total - tail:
            rows = 256 // pieces
            out += [(r0 + i * rows, min(r0 + (i + 1) * rows, M), n0) for i in range(pieces) if r0 + i * rows < M]
        else:
            out.append((r0, min(r0 + 256, M), n0))
    return out


def flagged_rows(x_bf16):
    mag = (x_bf16 & 0x7FFF).astype(np.uint32)
    mx = mag.max(axis=1)
    return (mx > 0x4700) | ((mx != 0) & (mx < 0x3C80))


ONLINE_SHAPES = [(520, 390, 320), (300, 520, 640), (17, 40, 64), (256, 256, 512), (777, 1000, 448)]


@pytest.mark.parametrize("layout", [ql.QL_LAYOUT_CANONICAL, ql.QL_LAYOUT_TILED])
@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("shape", ONLINE_SHAPES)
def test_online_parity(torch, shape, bits, layout):
    if bits == 3 and layout == ql.QL_LAYOUT_CANONICAL:
        pytest.skip("canonical 3-bit GEMMs run on a tiled copy in a workspace")
    M, N, K = shape
    c = Case(M, N, K, bits, wid=900 + bits, x_structure="outlier")
    y, _ = run_online(torch, c, layout)
    check_online(y.cpu().numpy(), c)


@pytest.mark.parametrize("layout", [ql.QL_LAYOUT_CANONICAL, ql.QL_LAYOUT_TILED])
@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_online_equals_prepass_fast_where_conversion_is_exact(torch, bits, layout):
    if bits == 3 and layout == ql.QL_LAYOUT_CANONICAL:
        pytest.skip("canonical 3-bit GEMMs run on a tiled copy in a workspace")
    M, N, K = 600, 700, 512
    x = away_from_zero(inputs.activations_bf16(M, K, 910 + bits, "outlier"))
    c = Case(M, N, K, bits, wid=910 + bits, x=x)
    y, _ = run_online(torch, c, layout)
    check_online(y.cpu().numpy(), c)
    yf = run_fast_given(torch, c, layout)
    assert np.array_equal(y.cpu().numpy().view(np.uint32), yf.view(np.uint32))


# (slots, shape): whole tiles over few blocks, and tail tiles cut into pieces
ONLINE_GRIDS = [
    (4, (520, 1000, 640)),    # 12 whole tiles, 3 per block
    (5, (520, 1000, 640)),    # 10 whole, 2 tail tiles x 2 pieces of 128 rows
    (12, (512, 1792, 320)),   # 12 whole, 2 tail tiles x 4 pieces of 64 rows
    (17, (300, 2304, 448)),   # 17 whole, 1 tail tile x 8 pieces of 32 rows
    (0, (700, 600, 384)),     # the device's own grid: every tile cut into row pieces
]


@pytest.mark.parametrize("layout", [ql.QL_LAYOUT_CANONICAL, ql.QL_LAYOUT_TILED])
@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("slots,shape", ONLINE_GRIDS)
def test_online_out_of_range_rows_recomputed_with_split(torch, monkeypatch, slots, shape, bits, layout):
    M, N, K = shape
    if slots:
        monkeypatch.setenv("QLINEAR_GEMM_SLOTS", str(slots))
    xf = inputs.activations_f32(M, K, 920 + bits)
    # special rows in the first tile row only, so later tile rows stay in range
    xf[3] *= 1.0e5                  # largest magnitude ~4e5: above 2^15
    xf[40, 7] = 40000.0             # one value above 2^15 in a normal row
    xf[70] *= 2.0 ** -12            # largest ~1e-3: below 2^-6
    xf[100] = 0.0                   # a zero row is in range (exact zeros)
    xf[130] *= 2.0 ** -18           # values in the fp16 subnormal range
    special = [3, 40, 70, 100, 130]
    # other rows: no value below 2^-17, where the unscaled conversion is exact
    x = away_from_zero(inputs.f32_to_bf16_bits(xf), rows=[r for r in range(M) if r not in special])
    rows_bad = flagged_rows(x)
    assert rows_bad[[3, 40, 70, 130]].all() and not rows_bad[100] and rows_bad.sum() == 4
    c = Case(M, N, K, bits, wid=920 + bits, x=x)
    y, path = run_online(torch, c, layout)
    y = y.cpu().numpy()
    check_online(y, c)
    x_, p_, s_, b_ = c.device(torch)
    if layout == ql.QL_LAYOUT_TILED:
        p_, s_ = ql.qlinear_repack(p_, s_, b_, bits, 64, N, K)
        b_ = None
    ys = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    ql.qlinear_forward_ex(x_, p_, s_, b_, bits, M, N, K, ys, layout=layout, mode=ql.QL_MODE_SPLIT, workspace=None)
    assert ql.qlinear_last_path().startswith("gemm4"), ql.qlinear_last_path()
    ys = ys.cpu().numpy()
    yf = run_fast_given(torch, c, layout)
    n_bad = n_good = 0
    for r0, r1, n0 in units(path, M, N):
        n1 = min(n0 + 256, N)
        got = y[r0:r1, n0:n1].view(np.uint32)
        if rows_bad[r0:r1].any():
            assert np.array_equal(got, ys[r0:r1, n0:n1].view(np.uint32)), (r0, n0, "recomputed unit != SPLIT")
            n_bad += 1
        else:
            assert np.array_equal(got, yf[r0:r1, n0:n1].view(np.uint32)), (r0, n0, "in-range unit != FAST")
            n_good += 1
    assert n_bad > 0 and n_good > 0


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_online_bf16_out_is_rounded_fp32_out(torch, bits):
    M, N, K = 300, 260, 384
    xf = inputs.activations_f32(M, K, 930 + bits)
    xf[5] *= 1.0e5   # one recomputed unit: its marker must work for bf16 outputs too
    c = Case(M, N, K, bits, wid=930 + bits, x=inputs.f32_to_bf16_bits(xf))
    y, _ = run_online(torch, c, ql.QL_LAYOUT_TILED)
    yb, _ = run_online(torch, c, ql.QL_LAYOUT_TILED, out_dtype="bf16")
    got = yb.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, inputs.f32_to_bf16_bits(y.cpu().numpy()))


def test_online_repeatable_and_degenerate(torch):
    c = Case(520, 1000, 640, 4, wid=940, x_structure="outlier")
    y1, _ = run_online(torch, c)
    y2, _ = run_online(torch, c)
    assert np.array_equal(y1.cpu().numpy().view(np.uint32), y2.cpu().numpy().view(np.uint32))
    # all-zero x: zero output, no recomputation needed
    z = Case(300, 300, 256, 4, wid=941, x=np.zeros((300, 256), np.uint16))
    yz, _ = run_online(torch, z)
    assert not np.any(yz.cpu().numpy())
