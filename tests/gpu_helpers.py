"""Shared helpers of the GPU parity tests: build a case with the oracle on the
CPU, move its bytes to the device, run the library, compare."""
import numpy as np
import pytest

import oracle
from group_wise_affine_qlinear_amd import inputs
from group_wise_affine_qlinear_amd import qlinear as ql

# Acceptance bar (the product's stated tolerance for bf16-in / fp32-accumulate outputs)
RELF_TOL = 2e-3
MAXABS_RMS_TOL = 1e-2
# Tighter bound implied by the exact-integer design: only fp32 accumulation
# rounding separates the kernels from the fp64 oracle (derivation in the design notes).
RELF_DESIGN = 2e-5
MAXABS_RMS_DESIGN = 2e-4


def gemv_serves(bits, M, K):
    """Whether a canonical-layout call of M rows goes to the lane-along-K GEMV:
    one or two rows, 2/4/8-bit codes, at least 64 16-byte chunks per weight
    row, at most 5 per lane, the lane's slice of x within 96 registers and x
    within 32 KB of LDS."""
    if M < 1 or M > 2 or bits not in (2, 4, 8):
        return False
    chunks = K * bits // 128
    per_lane = -(-chunks // 64)
    return chunks >= 64 and per_lane <= 5 and M * per_lane * (64 // bits) <= 96 and M * K * 2 <= 32768


def torch_or_skip():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def dev(torch, arr):
    arr = np.ascontiguousarray(arr)
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).cuda()
    if arr.dtype == np.uint32:
        return torch.from_numpy(arr.view(np.int32)).cuda()
    return torch.from_numpy(arr).cuda()


def host_u16(t):
    return t.cpu().numpy().view(np.uint16)


def host_u32(t):
    return t.cpu().numpy().view(np.uint32)


class Case:
    """Oracle-side data of one parity case (all produced on the CPU by the oracle)."""

    def __init__(self, M, N, K, bits, wid, x_structure="normal", w=None, x=None):
        self.M, self.N, self.K, self.bits = M, N, K, bits
        self.w = inputs.weights(N, K, wid) if w is None else w
        self.x = inputs.activations_bf16(M, K, wid, x_structure) if x is None else x
        self.q, self.s16, self.b16 = oracle.quantize_rtn(self.w, bits)
        self.packed = oracle.pack(self.q, bits)

    def device(self, torch):
        return (dev(torch, self.x), dev(torch, self.packed), dev(torch, self.s16), dev(torch, self.b16))

    def reference(self, rows=None, cols=None):
        if rows is None and cols is None:
            return oracle.forward(self.x, self.packed, self.s16, self.b16, self.bits, self.K)
        rows = np.arange(self.M) if rows is None else rows
        return oracle.forward_rows(self.x, self.packed, self.s16, self.b16, self.bits, self.K, rows, cols)


def run_forward(torch, case, path=ql.QL_PATH_AUTO, split_k=0, tile=0, out_dtype="f32", via_ex=True,
                layout=ql.QL_LAYOUT_CANONICAL, mode=ql.QL_MODE_AUTO):
    x, p, s, b = case.device(torch)
    if layout == ql.QL_LAYOUT_TILED:
        p, s = ql.qlinear_repack(p, s, b, case.bits, 64, case.N, case.K)
        b = None
    if out_dtype == "f32":
        out = torch.full((case.M, case.N), float("nan"), dtype=torch.float32, device="cuda")
    else:
        out = torch.zeros((case.M, case.N), dtype=torch.bfloat16, device="cuda")
    if via_ex:
        ql.qlinear_forward_ex(x, p, s, b, case.bits, case.M, case.N, case.K, out, path=path,
                              split_k=split_k, tile=tile, layout=layout, mode=mode)
    else:
        ql.qlinear_forward(x, p, s, b, case.bits, 64, case.M, case.N, case.K, out)
    torch.cuda.synchronize()
    return out


def assert_parity(y_gpu, y_ref, design=True, what=""):
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    assert np.all(np.isfinite(y_gpu)), f"{what}: non-finite output"
    e = oracle.error_metrics(y_gpu, y_ref)
    assert e["relF"] <= RELF_TOL and e["maxabs_over_rms"] <= MAXABS_RMS_TOL, (what, e)
    if design:
        assert e["relF"] <= RELF_DESIGN and e["maxabs_over_rms"] <= MAXABS_RMS_DESIGN, (what, e)
    return e


def assert_rows(y_gpu, y_ref, relf=RELF_TOL, maxabs=MAXABS_RMS_TOL, what="", axis=0):
    """Acceptance bar on the whole result and on every row (axis=0) or column
    (axis=1) against that slice's own scale: rows of x, or columns of the
    weights, may differ in magnitude by many orders. A slice whose reference
    is all zero must come back exactly zero."""
    y = np.asarray(y_gpu, dtype=np.float64)
    r = np.asarray(y_ref, dtype=np.float64)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    e = oracle.error_metrics(y, r)
    assert e["relF"] <= relf and e["maxabs_over_rms"] <= maxabs, (what, e)
    if axis == 1:
        y, r = y.T, r.T
    for i in range(r.shape[0]):
        if not np.any(r[i]):
            assert not np.any(y[i]), (what, "zero slice", i)
            continue
        ei = oracle.error_metrics(y[i:i + 1], r[i:i + 1])
        assert ei["relF"] <= relf and ei["maxabs_over_rms"] <= maxabs, (what, "slice", i, ei)
    return e
