"""GPU tests of canonical weights.

The GEMMs read canonical 2/4/8-bit codes directly in every numerics mode (no
per-call copy). FAST and SPLIT run the same kernel on either layout with the
same arithmetic in the same order, so a canonical run equals the run on
weights the caller repacked, bit for bit. Canonical 3-bit codes run every GEMM
on a tiled copy in the workspace (the same bijection as qlinear_repack, so
again equal bit for bit); without a workspace that call is refused."""
import pytest

from group_wise_affine_qlinear_amd import inputs
from group_wise_affine_qlinear_amd import qlinear as ql

from gpu_helpers import Case, assert_parity, assert_rows, run_forward, torch_or_skip

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    t = torch_or_skip()
    ql.load_library()
    return t


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("shape", [(512, 260, 384), (600, 520, 640)])
def test_canonical_runs_directly_and_equals_tiled(torch, bits, shape):
    M, N, K = shape
    c = Case(M, N, K, bits, wid=700 + bits + N)
    ref = c.reference()
    for mode, kname in ((ql.QL_MODE_FAST, "gemm3_f16"), (ql.QL_MODE_SPLIT, "gemm4_bf16x2")):
        y = run_forward(torch, c, mode=mode)
        path = ql.qlinear_last_path()
        assert path.startswith(kname) and path.endswith("_canonical"), path
        yt = run_forward(torch, c, layout=ql.QL_LAYOUT_TILED, mode=mode)
        assert ql.qlinear_last_path() == path.replace("_canonical", "_tiled"), (ql.qlinear_last_path(), path)
        assert torch.equal(y, yt), path
        assert_rows(y.cpu().numpy(), ref, what=path)
    y = run_forward(torch, c, mode=ql.QL_MODE_EXACT)
    assert ql.qlinear_last_path().endswith("_canonical"), ql.qlinear_last_path()
    assert_parity(y.cpu().numpy(), ref, what=ql.qlinear_last_path())
    y1 = run_forward(torch, c, via_ex=False)          # the spec call: no workspace
    assert ql.qlinear_last_path().startswith("gemm3_f16online") and ql.qlinear_last_path().endswith("_canonical")
    assert_rows(y1.cpu().numpy(), ref, what=ql.qlinear_last_path())


@pytest.mark.parametrize("mode", [ql.QL_MODE_EXACT, ql.QL_MODE_FAST, ql.QL_MODE_SPLIT])
def test_3bit_copy_route_equals_caller_repack(torch, mode):
    M, N, K = 600, 520, 640
    c = Case(M, N, K, 3, wid=710)
    y = run_forward(torch, c, mode=mode)
    path = ql.qlinear_last_path()
    assert path.endswith("_tiled_copy"), path
    yt = run_forward(torch, c, layout=ql.QL_LAYOUT_TILED, mode=mode)
    assert ql.qlinear_last_path() == path[:-len("_copy")], (ql.qlinear_last_path(), path)
    assert torch.equal(y, yt)
    assert_rows(y.cpu().numpy(), c.reference(), what=path)


def test_3bit_copy_route_workspace(torch):
    M, N, K, bits = 640, 300, 448, 3
    c = Case(M, N, K, bits, wid=730)
    x, p, s, b = c.device(torch)
    need = ql.qlinear_workspace_bytes(bits, M, N, K)
    assert need >= ql.qlinear_tiled_words(bits, N, K) * 4 + ql.qlinear_tiled_sb_words(N, K) * 4
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    out = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    ql.qlinear_forward_ex(x, p, s, b, bits, M, N, K, out, workspace=ws)
    torch.cuda.synchronize()
    assert ql.qlinear_last_path().endswith("_tiled_copy"), ql.qlinear_last_path()
    assert torch.equal(out, run_forward(torch, c))
    with pytest.raises(ql.QLinearError) as e:
        ql.qlinear_forward_ex(x, p, s, b, bits, M, N, K, out, workspace=ws[:4096])
    assert e.value.status == ql.QL_EWORKSPACE


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_canonical_gate_residual_in_place_equals_tiled(torch, out_dtype):
    """The fused gated update reads canonical weights directly and equals the
    same update on caller-repacked weights, bit for bit."""
    M, N, K, bits = 600, 520, 384, 4
    c = Case(M, N, K, bits, wid=740)
    x, p, s, b = c.device(torch)
    tq, tsb = ql.qlinear_repack(p, s, b, bits, 64, N, K)
    dt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    res0 = torch.from_numpy(inputs.residual_stream(M, N, 741)).cuda().to(dt)
    gate = torch.from_numpy(inputs.adaln_gate(3, N, 741)).cuda()
    yc = res0.clone()
    ql.qlinear_forward_ex(x, p, s, b, bits, M, N, K, yc, epilogue=ql.QL_EPI_GATE_RESIDUAL,
                          residual=yc, gate=gate, gate_rows=200)
    torch.cuda.synchronize()
    pc = ql.qlinear_last_path()
    assert pc.endswith("_gate_canonical"), pc
    yt = res0.clone()
    ql.qlinear_forward_ex(x, tq, tsb, None, bits, M, N, K, yt, layout=ql.QL_LAYOUT_TILED,
                          epilogue=ql.QL_EPI_GATE_RESIDUAL, residual=yt, gate=gate, gate_rows=200)
    torch.cuda.synchronize()
    assert ql.qlinear_last_path() == pc.replace("_canonical", "_tiled"), (ql.qlinear_last_path(), pc)
    assert torch.equal(yc, yt)
