"""GPU tests of the SPLIT numerics (bf16 hi + lo weight terms on bf16 MFMA) and
of the call that allocates nothing (``qlinear_forward``).

SPLIT represents each fp32 weight W = s*q + b (the format's definition, one
rounding) as hi + lo with hi = bf16(W) and lo = bf16(W - hi), both round to
nearest even, so |W - (hi + lo)| <= 2^-16 |W| for every weight: a property
checked directly with one-hot rows of x, which return hi + lo of each weight.
Products are compared with the oracle's plain fp64 product (``oracle.forward``)
at the acceptance bar and at the design bound of the exact modes (relF <=
2e-5, max-abs <= 2e-4 rms): the representation error (<= 2^-16 relative per
weight, ~9e-6 relative Frobenius) plus fp32 accumulation stays inside it.
"""
import numpy as np
import pytest

import oracle
from group_wise_affine_qlinear_amd import inputs
from group_wise_affine_qlinear_amd import qlinear as ql

from gpu_helpers import Case, assert_parity, assert_rows, dev, run_forward, torch_or_skip

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    t = torch_or_skip()
    ql.load_library()
    return t


SPLIT_SHAPES = [(520, 390, 320), (300, 520, 640), (17, 40, 64), (256, 256, 512), (777, 1000, 448)]


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("shape", SPLIT_SHAPES)
@pytest.mark.parametrize("layout", [ql.QL_LAYOUT_CANONICAL, ql.QL_LAYOUT_TILED])
def test_split_parity(torch, shape, bits, layout):
    M, N, K = shape
    c = Case(M, N, K, bits, wid=500 + bits, x_structure="outlier")
    y = run_forward(torch, c, layout=layout, mode=ql.QL_MODE_SPLIT)
    path = ql.qlinear_last_path()
    assert path.startswith("gemm4_bf16x2"), path
    assert_parity(y.cpu().numpy(), c.reference(), what=path)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_north_star_call_on_canonical(torch, bits):
    """qlinear_forward: canonical weights, no workspace: for M > 16 the FAST
    GEMM converting x itself (acceptance bar row by row, FAST budget), the
    skinny kernel or GEMV below (exact-mode bound); SPLIT on request, against
    the plain product at the exact-mode bound."""
    for M in (1, 16, 17, 300):
        c = Case(M, 264, 576, bits, wid=510 + bits)
        ref = c.reference()
        y = run_forward(torch, c, via_ex=False)
        path = ql.qlinear_last_path()
        assert path.startswith(("skinny", "gemv") if M <= 16 else "gemm3_f16online"), path
        assert path.endswith("_canonical"), path
        if M <= 16:
            assert_parity(y.cpu().numpy(), ref, what=path)
            continue
        assert_rows(y.cpu().numpy(), ref, what=path)
        e = oracle.error_metrics(y.cpu().numpy(), ref)
        assert e["relF"] <= 5e-4 and e["maxabs_over_rms"] <= 4e-3, (path, e)
        x, p, s, b = c.device(torch)
        ys = torch.full((M, c.N), float("nan"), dtype=torch.float32, device="cuda")
        ql.qlinear_forward_ex(x, p, s, b, bits, M, c.N, c.K, ys, mode=ql.QL_MODE_SPLIT, workspace=None)
        assert ql.qlinear_last_path().startswith("gemm4_bf16x2"), ql.qlinear_last_path()
        assert_parity(ys.cpu().numpy(), ref, what=ql.qlinear_last_path())


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("slots", [11, 10, 5])
def test_split_row_pieces(torch, bits, slots, monkeypatch):
    """Tail tiles cut along M into 2, 4 or 8 row pieces (resident-block count
    forced small so a small shape has a tail) match whole-tile runs."""
    monkeypatch.setenv("QLINEAR_GEMM_SLOTS", str(slots))
    c = Case(700, 800, 256, bits, wid=520 + bits)
    y = run_forward(torch, c, layout=ql.QL_LAYOUT_TILED, mode=ql.QL_MODE_SPLIT)
    path = ql.qlinear_last_path()
    assert "_tail" in path, path
    assert_parity(y.cpu().numpy(), c.reference(), what=path)


@pytest.mark.parametrize("layout", [ql.QL_LAYOUT_CANONICAL, ql.QL_LAYOUT_TILED])
def test_split_k_split_and_bf16_out(torch, layout):
    c = Case(200, 300, 2048, 4, wid=530)
    ref = c.reference()
    y = run_forward(torch, c, layout=layout, mode=ql.QL_MODE_SPLIT, path=ql.QL_PATH_SPLITK, split_k=5)
    assert "_split" in ql.qlinear_last_path(), ql.qlinear_last_path()
    assert_parity(y.cpu().numpy(), ref, what=ql.qlinear_last_path())
    y2 = run_forward(torch, c, layout=layout, mode=ql.QL_MODE_SPLIT, path=ql.QL_PATH_SPLITK, split_k=5)
    assert np.array_equal(y.cpu().numpy().view(np.uint32), y2.cpu().numpy().view(np.uint32))
    yb = run_forward(torch, c, layout=layout, mode=ql.QL_MODE_SPLIT, out_dtype="bf16")
    got = yb.float().cpu().numpy().astype(np.float64)
    ref_bf = oracle.bf16_bits_to_f64(inputs.f32_to_bf16_bits(ref.astype(np.float32)))
    rms = np.sqrt(np.mean(ref ** 2))
    assert np.all(np.abs(got - ref_bf) <= np.abs(ref) * 2.0 ** -7 + 1e-5 * rms)


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("layout", [ql.QL_LAYOUT_CANONICAL, ql.QL_LAYOUT_TILED])
def test_split_one_hot_rows_bound_every_weight(torch, bits, layout):
    """A one-hot row of x returns hi + lo of each weight of one input channel;
    every weight must lie within 2^-16 of its own magnitude."""
    K, N = 512, 136
    M = K
    x = np.zeros((M, K), np.uint16)
    x[np.arange(M), np.arange(M)] = 0x3F80  # 1.0
    w = inputs.weights(N, K, 540)
    w[3, :64] = 1e3 * np.linspace(-1, 1, 64, dtype=np.float32)  # a wide group
    w[4, 64:128] = 0.5                                            # a constant group
    c = Case(M, N, K, bits, wid=540, w=w, x=x)
    y = run_forward(torch, c, layout=layout, mode=ql.QL_MODE_SPLIT).cpu().numpy().astype(np.float64)
    w_hat = oracle.dequantize(c.q, c.s16, c.b16).astype(np.float64).T  # [K, N]
    assert np.all(np.abs(y - w_hat) <= np.abs(w_hat) * 2.0 ** -16), ql.qlinear_last_path()
    # weights exactly representable as hi + lo (constant group: W = b, an f16) come back exactly
    assert np.array_equal(y[64:128, 4], w_hat[64:128, 4])


def test_split_degenerate_groups_and_rows(torch):
    """The degenerate groups and rows of the exact-mode tests, every row
    against the plain product at the acceptance bar, row by row."""
    from test_gpu_parity import degenerate_case
    for bits in (2, 4, 8):
        c = degenerate_case(40, 96, 256, bits, wid=550 + bits)
        ref = c.reference()
        for layout in (ql.QL_LAYOUT_CANONICAL, ql.QL_LAYOUT_TILED):
            y = run_forward(torch, c, layout=layout, mode=ql.QL_MODE_SPLIT).cpu().numpy()
            assert np.all(y[0] == 0.0)
            assert_rows(y, ref, what=(bits, layout, ql.qlinear_last_path()))


# ------------------------------------------------------------------ the call that allocates nothing

def test_north_star_call_allocates_nothing(torch):
    """A first qlinear_forward at sizes never seen before leaves the device's
    free memory unchanged (the library allocates nothing), for the skinny and
    the GEMM path, on a shape whose automatic plan would split K if a
    workspace were passed."""
    shapes = [(1, 2048, 3072), (333, 1024, 4096), (256, 512, 8192)]
    cases = [Case(M, N, K, 4, wid=560 + i) for i, (M, N, K) in enumerate(shapes)]
    dev_args = [(c.device(torch), torch.empty((c.M, c.N), dtype=torch.float32, device="cuda")) for c in cases]
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    for c, ((x, p, s, b), out) in zip(cases, dev_args):
        ql.qlinear_forward(x, p, s, b, 4, 64, c.M, c.N, c.K, out)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 == free0, (free0, free1)
    for c, (_, out) in zip(cases, dev_args):
        if c.M <= 16:   # skinny kernel / GEMV: the exact-mode bound
            assert_parity(out.cpu().numpy(), c.reference(), what="qlinear_forward")
        else:           # FAST converting x in the GEMM: the acceptance bar, row by row
            assert_rows(out.cpu().numpy(), c.reference(), what="qlinear_forward")


def test_two_streams_concurrently(torch):
    """Two qlinear_forward_ex calls in flight at once on two streams (no
    workspace: the scratch-free plans; and with one workspace each) both
    match the plain product; the library keeps no state the calls share."""
    ca = Case(1000, 1536, 1024, 4, wid=570)
    cb = Case(700, 2048, 768, 8, wid=571)
    da, db = ca.device(torch), cb.device(torch)
    for use_ws in (False, True):
        oa = torch.full((ca.M, ca.N), float("nan"), dtype=torch.float32, device="cuda")
        ob = torch.full((cb.M, cb.N), float("nan"), dtype=torch.float32, device="cuda")
        wa = torch.empty(ql.qlinear_workspace_bytes(4, ca.M, ca.N, ca.K), dtype=torch.uint8, device="cuda")
        wb = torch.empty(ql.qlinear_workspace_bytes(8, cb.M, cb.N, cb.K), dtype=torch.uint8, device="cuda")
        sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
        torch.cuda.synchronize()
        for _ in range(3):
            with torch.cuda.stream(sa):
                ql.qlinear_forward_ex(*da, 4, ca.M, ca.N, ca.K, oa, workspace=wa if use_ws else None, stream=sa)
            with torch.cuda.stream(sb):
                ql.qlinear_forward_ex(*db, 8, cb.M, cb.N, cb.K, ob, workspace=wb if use_ws else None, stream=sb)
        torch.cuda.synchronize()
        # FAST either way (the prepass with a workspace, the in-GEMM conversion
        # without): the acceptance bar, row by row
        assert_rows(oa.cpu().numpy(), ca.reference(), what=("stream a", use_ws))
        assert_rows(ob.cpu().numpy(), cb.reference(), what=("stream b", use_ws))


def test_null_workspace_refusals(torch):
    """Requests that need scratch and bring no workspace are refused before
    any launch, and leave the output untouched."""
    c = Case(64, 128, 256, 4, wid=580)
    x, p, s, b = c.device(torch)
    out = torch.full((c.M, c.N), 7.0, dtype=torch.float32, device="cuda")
    tq, tsb = ql.qlinear_repack(p, s, b, 4, 64, c.N, c.K)
    res = torch.zeros((c.M, c.N), dtype=torch.float32, device="cuda")
    gate = torch.ones((1, c.N), dtype=torch.float32, device="cuda")
    for kw in (dict(mode=ql.QL_MODE_EXACT), dict(path=ql.QL_PATH_SPLITK, split_k=2),
               dict(layout=ql.QL_LAYOUT_TILED, epilogue=ql.QL_EPI_GATE_RESIDUAL, residual=res, gate=gate,
                    gate_rows=c.M)):
        pp, ss, bb = (tq, tsb, None) if kw.get("layout") == ql.QL_LAYOUT_TILED else (p, s, b)
        with pytest.raises(ql.QLinearError) as e:
            ql.qlinear_forward_ex(x, pp, ss, bb, 4, c.M, c.N, c.K, out, workspace=None, **kw)
        assert e.value.status == ql.QL_EWORKSPACE, kw
    c3 = Case(64, 128, 256, 3, wid=581)
    x3, p3, s3, b3 = c3.device(torch)
    with pytest.raises(ql.QLinearError) as e:
        ql.qlinear_forward(x3, p3, s3, b3, 3, 64, c3.M, c3.N, c3.K, out)
    assert e.value.status == ql.QL_EWORKSPACE
    torch.cuda.synchronize()
    assert np.all(out.cpu().numpy() == 7.0)
