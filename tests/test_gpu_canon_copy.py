"""GPU tests of canonical weights run through a tiled copy.

Under automatic dispatch, canonical 2/4/8-bit weights from 512 rows on (and
3-bit weights on any GEMM path) run on a tiled copy that the repack kernel
writes into the workspace. The copy is the same bijection as qlinear_repack,
so the result equals the run on weights the caller repacked, bit for bit, in
EXACT (the AUTO choice on canonical weights) and FAST mode, and it meets the
exact bound against the oracle. Forced paths, tiles and splits keep the
kernels on the canonical code rows."""
import pytest

from group_wise_affine_qlinear_amd import inputs
from group_wise_affine_qlinear_amd import qlinear as ql

from gpu_helpers import Case, assert_parity, run_forward, torch_or_skip

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    t = torch_or_skip()
    ql.load_library()
    return t


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("shape", [(512, 260, 384), (600, 520, 640)])
def test_copy_route_equals_caller_repack(torch, bits, shape):
    M, N, K = shape
    c = Case(M, N, K, bits, wid=700 + bits + N)
    y = run_forward(torch, c)
    path = ql.qlinear_last_path()
    assert path.startswith("gemm2") and path.endswith("_tiled_copy"), path
    yt = run_forward(torch, c, layout=ql.QL_LAYOUT_TILED, mode=ql.QL_MODE_EXACT)
    assert ql.qlinear_last_path() == path[:-len("_copy")], (ql.qlinear_last_path(), path)
    assert torch.equal(y, yt)
    assert_parity(y.cpu().numpy(), c.reference(), what=path)
    y1 = run_forward(torch, c, via_ex=False)          # the primary entry point takes the same route
    assert ql.qlinear_last_path() == path
    assert torch.equal(y1, y)
    yf = run_forward(torch, c, mode=ql.QL_MODE_FAST)
    pf = ql.qlinear_last_path()
    assert pf.startswith("gemm3") and pf.endswith("_tiled_copy"), pf
    yft = run_forward(torch, c, layout=ql.QL_LAYOUT_TILED, mode=ql.QL_MODE_FAST)
    assert torch.equal(yf, yft)


def test_copy_route_threshold_and_forced_requests(torch):
    run_forward(torch, Case(511, 256, 256, 4, wid=720))
    assert ql.qlinear_last_path().endswith("_canonical"), ql.qlinear_last_path()
    c = Case(512, 256, 256, 4, wid=721)
    ref = c.reference()
    run_forward(torch, c)
    assert ql.qlinear_last_path().endswith("_tiled_copy"), ql.qlinear_last_path()
    for kw in ({"path": ql.QL_PATH_GEMM}, {"path": ql.QL_PATH_SPLITK, "split_k": 2}, {"tile": 10, "path": ql.QL_PATH_GEMM}):
        y = run_forward(torch, c, **kw)
        assert ql.qlinear_last_path().endswith("_canonical"), (kw, ql.qlinear_last_path())
        assert_parity(y.cpu().numpy(), ref, what=(kw, ql.qlinear_last_path()))


def test_copy_route_workspace(torch):
    M, N, K, bits = 640, 300, 448, 4
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
def test_copy_route_gate_residual_in_place(torch, out_dtype):
    """The fused gated update on canonical weights at M >= 512 runs on the copy
    and equals the same update on caller-repacked weights, bit for bit."""
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
    assert pc.endswith("_gate_tiled_copy"), pc
    yt = res0.clone()
    ql.qlinear_forward_ex(x, tq, tsb, None, bits, M, N, K, yt, layout=ql.QL_LAYOUT_TILED,
                          epilogue=ql.QL_EPI_GATE_RESIDUAL, residual=yt, gate=gate, gate_rows=200)
    torch.cuda.synchronize()
    assert ql.qlinear_last_path() == pc[:-len("_copy")], (ql.qlinear_last_path(), pc)
    assert torch.equal(yc, yt)
