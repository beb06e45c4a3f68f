"""GPU tests of the AdaLN scale fused into the FAST prepass
(``qlinear_fast_activations_adaln``).

End to end, the fused prepass followed by the FAST GEMM on its activations is
compared with the oracle's plain product of the modulated input
(``oracle.forward_modulated``: x * (1 + scale[m // rows]) in float64, times
the dequantized weights) at the acceptance bar, row by row, and within the
FAST budget. The prepass alone is checked against exact properties of the
modulation: a zero scale is the identity (bit-identical to the unmodulated
prepass), a scale of one doubles every value (same fp16 values, row scale
times two), a scale of minus one zeroes the row. The K sizes reach every
prepass kernel (one wave per row with 4, 9 or 16 vectors per lane, and the
block-per-row kernel beyond)."""
import numpy as np
import pytest

import oracle
from group_wise_affine_qlinear_amd import inputs
from group_wise_affine_qlinear_amd import qlinear as ql

from gpu_helpers import Case, assert_rows, dev, torch_or_skip

pytestmark = pytest.mark.gpu

RELF_FAST = 5e-4


@pytest.fixture(scope="module")
def torch():
    t = torch_or_skip()
    ql.load_library()
    return t


def scale_table(samples, K, seed):
    rng = np.random.default_rng(seed)
    s = rng.uniform(-0.9, 0.9, size=(samples, K)).astype(np.float32)
    s[:, 5] = -1.0   # a channel switched off
    s[:, 7] = 3.0    # a channel amplified
    return s


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("M,N,K,rows", [(300, 264, 512, 150), (96, 520, 4608, 1), (257, 136, 8192, 64),
                                        (40, 72, 9216, 7)])
@pytest.mark.parametrize("layout", [ql.QL_LAYOUT_TILED, ql.QL_LAYOUT_CANONICAL])
def test_fused_prepass_then_fast_gemm(torch, bits, M, N, K, rows, layout):
    c = Case(M, N, K, bits, wid=700 + bits, x_structure="outlier")
    samples = -(-M // rows)
    sc = scale_table(samples, K, 701 + K)
    ref = oracle.forward_modulated(c.x, sc.astype(np.float64), rows, c.packed, c.s16, c.b16, bits, K)
    x, p, s, b = c.device(torch)
    x16, rs = ql.qlinear_fast_activations_adaln(x, dev(torch, sc), rows, M, K)
    assert ql.qlinear_last_path() == "fast_activations_adaln"
    if layout == ql.QL_LAYOUT_TILED:
        p, s = ql.qlinear_repack(p, s, b, bits, 64, N, K)
        b = None
    out = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    ql.qlinear_forward_ex(x, p, s, b, bits, M, N, K, out, layout=layout, mode=ql.QL_MODE_FAST, x16=x16,
                          rowscale=rs)
    torch.cuda.synchronize()
    y = out.cpu().numpy()
    what = (bits, M, N, K, rows, ql.qlinear_last_path())
    assert_rows(y, ref, what=what)
    e = oracle.error_metrics(y, ref)
    assert e["relF"] <= RELF_FAST, (what, e)


@pytest.mark.parametrize("K", [512, 4608, 8192, 9216])
def test_modulation_exact_properties(torch, K):
    M = 70
    x = dev(torch, inputs.activations_bf16(M, K, 710, "outlier"))
    x16_0, rs_0 = ql.qlinear_fast_activations(x, M, K)
    z = torch.zeros((2, K), dtype=torch.float32, device="cuda")
    x16_z, rs_z = ql.qlinear_fast_activations_adaln(x, z, 35, M, K)
    o = torch.ones((M, K), dtype=torch.float32, device="cuda")
    x16_o, rs_o = ql.qlinear_fast_activations_adaln(x, o, 1, M, K)
    n = -torch.ones((1, K), dtype=torch.float32, device="cuda")
    x16_n, rs_n = ql.qlinear_fast_activations_adaln(x, n, M, M, K)
    torch.cuda.synchronize()
    # identity: x * (1 + 0) = x exactly
    assert torch.equal(x16_z.view(torch.int16), x16_0.view(torch.int16)) and torch.equal(rs_z, rs_0)
    # doubling: x * 2 is exact, the row exponent moves by one, the fp16 values stay
    assert torch.equal(x16_o.view(torch.int16), x16_0.view(torch.int16)) and torch.equal(rs_o, 2 * rs_0)
    # annihilation: every value becomes a zero, the row scale is one
    assert bool((x16_n.float() == 0).all()) and bool((rs_n == 1).all())


def test_samples_take_their_own_scale_rows(torch):
    """Rows of one sample share a scale row: with a scale of one for sample 1
    and zero for samples 0 and 2, only sample 1's rows double."""
    M, K, rows = 10, 512, 4
    x = dev(torch, inputs.activations_bf16(M, K, 720))
    x16_0, rs_0 = ql.qlinear_fast_activations(x, M, K)
    sc = np.zeros((3, K), np.float32)
    sc[1] = 1.0
    x16, rs = ql.qlinear_fast_activations_adaln(x, dev(torch, sc), rows, M, K)
    torch.cuda.synchronize()
    assert torch.equal(x16.view(torch.int16), x16_0.view(torch.int16))
    want = rs_0.clone()
    want[4:8] *= 2
    assert torch.equal(rs, want)


def test_argument_errors(torch):
    M, K = 8, 128
    x = dev(torch, inputs.activations_bf16(M, K, 730))
    sc = torch.zeros((M, K), dtype=torch.float32, device="cuda")
    lib = ql.load_library()
    x16 = torch.empty((M, K), dtype=torch.float16, device="cuda")
    rs = torch.empty((M,), dtype=torch.float32, device="cuda")
    st = lib.qlinear_fast_activations_adaln(x.data_ptr(), sc.data_ptr() + 4, 1, M, K, x16.data_ptr(),
                                            rs.data_ptr(), None)
    assert st == ql.QL_EALIGN
    st = lib.qlinear_fast_activations_adaln(x.data_ptr(), sc.data_ptr(), 0, M, K, x16.data_ptr(),
                                            rs.data_ptr(), None)
    assert st == ql.QL_EINVAL
