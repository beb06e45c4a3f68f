"""GPU test of qlinear_forward_noalloc, the entry point for callers that cannot
allocate: its scratch is a fixed array inside the library instead of a caller
workspace. Called through the C ABI, it must give the output of
qlinear_forward_ex with a caller workspace (same plan, same kernels: bit for
bit) on two calls in a row, the second with a smaller input (the array keeps
the first call's contents), meet the oracle's bar, and refuse a call whose plan
needs more scratch than the array holds before launching anything."""
import ctypes

import numpy as np
import pytest

from group_wise_affine_qlinear_amd import qlinear as ql

from gpu_helpers import Case, assert_rows, torch_or_skip

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    t = torch_or_skip()
    ql.load_library()
    return t


def _args(torch, x, p, s, b, bits, M, N, K, out, layout):
    a = ql.ql_forward_args()
    a.x, a.packed_q, a.scales = x.data_ptr(), p.data_ptr(), s.data_ptr()
    a.biases = b.data_ptr() if b is not None else None
    a.bits, a.group, a.M, a.N, a.K = bits, 64, M, N, K
    a.out, a.out_dtype, a.layout = out.data_ptr(), ql.QL_OUT_F32, layout
    return a


def _run_both(torch, lib, c, layout):
    x, p, s, b = c.device(torch)
    if layout == ql.QL_LAYOUT_TILED:
        p, s = ql.qlinear_repack(p, s, b, c.bits, 64, c.N, c.K)
        b = None
    y_ref = torch.full((c.M, c.N), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(ql.qlinear_workspace_bytes(c.bits, c.M, c.N, c.K), 16), dtype=torch.uint8, device="cuda")
    ql.qlinear_forward_ex(x, p, s, b, c.bits, c.M, c.N, c.K, y_ref, layout=layout, workspace=ws)
    path_ref = ql.qlinear_last_path()
    y = torch.full((c.M, c.N), float("nan"), dtype=torch.float32, device="cuda")
    a = _args(torch, x, p, s, b, c.bits, c.M, c.N, c.K, y, layout)
    stream = torch.cuda.current_stream().cuda_stream
    st = lib.qlinear_forward_noalloc(ctypes.byref(a), stream)
    assert st == ql.QL_OK, ql.qlinear_status_string(st)
    torch.cuda.synchronize()
    assert ql.qlinear_last_path() == path_ref, (ql.qlinear_last_path(), path_ref)
    return y, y_ref


@pytest.mark.parametrize("layout", [ql.QL_LAYOUT_TILED, ql.QL_LAYOUT_CANONICAL])
def test_noalloc_matches_workspace_call_twice(torch, layout):
    lib = ql.load_library()
    assert lib.qlinear_forward_noalloc_max_scratch() == 64 << 20
    # first a larger call (fp16 activations of 8 MiB plus a K split's partials
    # in the array), then a smaller one over the same array
    for shape, wid in (((2048, 1536, 2048), 900), ((600, 520, 640), 901)):
        c = Case(*shape, 4, wid=wid + layout)
        y, y_ref = _run_both(torch, lib, c, layout)
        assert torch.equal(y, y_ref), (shape, layout)
        assert_rows(y.cpu().numpy(), c.reference(), what=("noalloc", shape, layout))


def test_noalloc_k_split_and_exact_mode(torch):
    """A K split (fp32 partials in the array) and EXACT numerics (group sums of
    x in the array), twice, the second call smaller."""
    lib = ql.load_library()
    for shape, wid in (((256, 768, 8192), 910), ((100, 300, 1024), 911)):
        c = Case(*shape, 4, wid=wid)
        x, p, s, b = c.device(torch)
        for mode in (ql.QL_MODE_EXACT, ql.QL_MODE_AUTO):
            y_ref = torch.empty((c.M, c.N), dtype=torch.float32, device="cuda")
            ws = torch.empty(ql.qlinear_workspace_bytes(4, c.M, c.N, c.K), dtype=torch.uint8, device="cuda")
            ql.qlinear_forward_ex(x, p, s, b, 4, c.M, c.N, c.K, y_ref, mode=mode, workspace=ws)
            path_ref = ql.qlinear_last_path()
            y = torch.full((c.M, c.N), float("nan"), dtype=torch.float32, device="cuda")
            a = _args(torch, x, p, s, b, 4, c.M, c.N, c.K, y, ql.QL_LAYOUT_CANONICAL)
            a.mode = mode
            st = lib.qlinear_forward_noalloc(ctypes.byref(a), torch.cuda.current_stream().cuda_stream)
            assert st == ql.QL_OK, ql.qlinear_status_string(st)
            torch.cuda.synchronize()
            assert ql.qlinear_last_path() == path_ref, (ql.qlinear_last_path(), path_ref)
            assert torch.equal(y, y_ref), (shape, mode, path_ref)
            assert_rows(y.cpu().numpy(), c.reference(), what=("noalloc", shape, mode))


def test_noalloc_refuses_plans_beyond_the_array(torch):
    """fp16 activations of 128 MiB do not fit the 64 MiB array: refused before
    any launch, the output untouched; a workspace argument is refused too."""
    lib = ql.load_library()
    M, N, K = 8192, 256, 8192
    x = torch.zeros((M, K), dtype=torch.int16, device="cuda")
    p = torch.zeros((N, K // 8), dtype=torch.int32, device="cuda")
    s = torch.zeros((N, K // 64), dtype=torch.int16, device="cuda")
    out = torch.full((M, N), 5.0, dtype=torch.float32, device="cuda")
    a = _args(torch, x, p, s, s, 4, M, N, K, out, ql.QL_LAYOUT_CANONICAL)
    a.mode = ql.QL_MODE_FAST
    assert lib.qlinear_forward_noalloc(ctypes.byref(a), None) == ql.QL_EWORKSPACE
    a.mode = ql.QL_MODE_AUTO
    a.workspace, a.workspace_bytes = out.data_ptr(), 16
    assert lib.qlinear_forward_noalloc(ctypes.byref(a), None) == ql.QL_EINVAL
    torch.cuda.synchronize()
    assert bool((out == 5.0).all())
