"""GPU parity of the canonical-row GEMV (one or two rows of x, 2-, 4- and
8-bit codes; lanes along K, each wave load one contiguous kilobyte of a row).

The GEMV keeps the skinny path's EXACT numerics (codes as exact bf16 values,
fp32 accumulation, per-chunk scale and bias fold), so it is held to the design
bound of the exact modes against the oracle's plain product, row by row, on
shapes where the chunk count per row is a multiple of 64, leaves a ragged
last lane set, or just reaches 64; bf16 output is one rounding of the fp32
result. The skinny kernel it replaces (QLINEAR_NO_GEMV=1) is held to the same
bound on the same shapes."""
import numpy as np
import pytest

import oracle
from group_wise_affine_qlinear_amd import inputs
from group_wise_affine_qlinear_amd import qlinear as ql

from gpu_helpers import Case, assert_parity, assert_rows, run_forward, torch_or_skip, RELF_DESIGN, MAXABS_RMS_DESIGN

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    t = torch_or_skip()
    ql.load_library()
    return t


# (bits, K): chunks per row C = K*bits/128 of 64, 144 (ragged), 66 (2 lanes in
# the last set), 288 (five sets)
SHAPES = [(4, 2048), (4, 4608), (4, 2112), (8, 1024), (8, 4608), (2, 4096), (2, 4608)]


@pytest.mark.parametrize("bits,K", SHAPES)
@pytest.mark.parametrize("M", [1, 2])
def test_gemv_parity(torch, bits, K, M):
    N = 1000
    c = Case(M, N, K, bits, wid=800 + bits, x_structure="outlier")
    ref = c.reference()
    y = run_forward(torch, c, via_ex=False)
    path = ql.qlinear_last_path()
    if path.startswith("gemv"):
        assert path == f"gemv_b{bits}_m{M}_canonical", path
    else:
        # register budget: two rows of 2-bit codes at this K stay on the skinny kernel
        assert bits == 2 and M == 2, path
    assert_rows(y.cpu().numpy(), ref, RELF_DESIGN, MAXABS_RMS_DESIGN, what=path)
    yb = run_forward(torch, c, via_ex=True, out_dtype="bf16")
    got = yb.float().cpu().numpy().astype(np.float64)
    ref_bf = oracle.bf16_bits_to_f64(inputs.f32_to_bf16_bits(ref.astype(np.float32)))
    rms = np.sqrt(np.mean(ref ** 2))
    assert np.all(np.abs(got - ref_bf) <= np.abs(ref) * 2.0 ** -7 + 1e-4 * rms), path


@pytest.mark.parametrize("bits,K", [(4, 4608), (8, 4608)])
def test_skinny_kernel_on_the_same_shapes(torch, bits, K, monkeypatch):
    monkeypatch.setenv("QLINEAR_NO_GEMV", "1")
    c = Case(1, 700, K, bits, wid=820 + bits)
    y = run_forward(torch, c, via_ex=False)
    assert ql.qlinear_last_path().startswith("skinny"), ql.qlinear_last_path()
    assert_parity(y.cpu().numpy(), c.reference(), what="skinny")


def test_gemv_degenerate_rows(torch):
    """Constant groups, a zero row of x and huge weights through the GEMV."""
    from test_gpu_parity import degenerate_case
    for bits in (2, 4, 8):
        K = 4096  # two rows of 2-bit codes stay within the GEMV's register budget here
        d = degenerate_case(3, 96, K, bits, wid=830 + bits)
        # rows 0-1 (zero row, 2^20 row) as one call of two rows, row 2 (2^-30 row) alone
        for rows in (slice(0, 2), slice(2, 3)):
            x = np.ascontiguousarray(d.x[rows])
            c = Case(x.shape[0], 96, K, bits, wid=830 + bits, w=d.w, x=x)
            y = run_forward(torch, c, via_ex=False).cpu().numpy()
            path = ql.qlinear_last_path()
            assert path.startswith("gemv"), path
            assert_rows(y, c.reference(), what=(bits, rows, path))
            if rows.start == 0:
                assert np.all(y[0] == 0.0)


def test_gemv_full_size_adaln_projection(torch):
    """The AdaLN projection at its full size (M = 1, K = 4608, N = 6 x 4608),
    canonical 4-bit weights, against the plain product on every output."""
    M, K, N = 1, 4608, 6 * 4608
    c = Case(M, N, K, 4, wid=840)
    y = run_forward(torch, c, via_ex=False)
    assert ql.qlinear_last_path() == "gemv_b4_m1_canonical"
    assert_parity(y.cpu().numpy(), c.reference(), what="gemv full size")
