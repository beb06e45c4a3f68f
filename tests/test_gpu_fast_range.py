"""FAST numerics on weights whose dequantized values leave the fp16 range.

FAST rounds each weight to fp16. A column whose bound max(|b|, |b + Q*s|)
over its groups reaches 65504 has its fp16 weights scaled by 2^-c and its
outputs by 2^c (c from that bound, found by the kernel's scan of the tile's
scale and bias words), so results stay finite and accurate. The cases below
put such columns next to normal ones and compare every column, at its own
scale, with the oracle's plain fp64 product at the acceptance bar.
"""
import numpy as np
import pytest

import oracle
from group_wise_affine_qlinear_amd import inputs
from group_wise_affine_qlinear_amd import qlinear as ql

from gpu_helpers import Case, assert_rows, dev, run_forward, torch_or_skip

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    t = torch_or_skip()
    ql.load_library()
    return t


def wide_case(M, N, K, bits, wid):
    """Normal weights except: column 5, group 0 spans [6e4, 1.3e5] (the top of
    the grid is twice the fp16 limit); column 6, group 1 spans [-65504, 6e4];
    column 7 holds b = 6.5e4 with a zero scale (constant group at the limit)."""
    w = inputs.weights(N, K, wid)
    w[5, :64] = np.linspace(6e4, 1.3e5, 64, dtype=np.float32)
    w[6, 64:128] = np.linspace(-65504.0, 6e4, 64, dtype=np.float32)
    w[7, :64] = 65000.0
    return Case(M, N, K, bits, wid=wid, w=w)


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("layout", [ql.QL_LAYOUT_TILED, ql.QL_LAYOUT_CANONICAL])
def test_fast_out_of_fp16_range_columns(torch, bits, layout):
    c = wide_case(300, 296, 512, bits, wid=590 + bits)
    w_hat = oracle.dequantize(c.q, c.s16, c.b16)
    assert np.abs(w_hat[5]).max() > 65504.0          # the case does leave the fp16 range
    ref = c.reference()
    y = run_forward(torch, c, layout=layout, mode=ql.QL_MODE_FAST).cpu().numpy()
    assert ql.qlinear_last_path().startswith("gemm3_f16"), ql.qlinear_last_path()
    assert_rows(y, ref, what=("columns", ql.qlinear_last_path()), axis=1)


def test_fast_out_of_range_auto_and_epilogue(torch):
    """Automatic dispatch on tiled weights (FAST) and the fused gated update
    on the same weights stay finite and on the bar."""
    c = wide_case(260, 288, 384, 4, wid=599)
    ref = c.reference()
    y = run_forward(torch, c, layout=ql.QL_LAYOUT_TILED).cpu().numpy()
    assert ql.qlinear_last_path().startswith("gemm3_f16"), ql.qlinear_last_path()
    assert_rows(y, ref, what="auto", axis=1)
    x, p, s, b = c.device(torch)
    tq, tsb = ql.qlinear_repack(p, s, b, 4, 64, c.N, c.K)
    res = inputs.residual_stream(c.M, c.N, 599)
    gate = inputs.adaln_gate(2, c.N, 599)
    out = dev(torch, res.copy())
    ql.qlinear_forward_ex(x, tq, tsb, None, 4, c.M, c.N, c.K, out, layout=ql.QL_LAYOUT_TILED,
                          epilogue=ql.QL_EPI_GATE_RESIDUAL, residual=out, gate=dev(torch, gate),
                          gate_rows=(c.M + 1) // 2)
    torch.cuda.synchronize()
    expect = oracle.gate_residual(ref, res, gate, (c.M + 1) // 2)
    branch = expect - res.astype(np.float64)
    got_branch = out.cpu().numpy().astype(np.float64) - res.astype(np.float64)
    assert_rows(got_branch, branch, what="gated", axis=1)
