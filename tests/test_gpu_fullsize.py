"""GPU parity at the full sizes of the configured workloads, on the full output.

Every workload of ``inputs.WORKLOADS`` runs at its full shape through the
launches the benchmark times and the spec call:
  * ``qlinear_forward`` on canonical weights, no workspace (for M > 16 the
    FAST GEMM converting x itself, against the oracle at the acceptance bar
    row by row and within the FAST budget; below, the skinny kernel or the
    GEMV at the design bound of the exact modes);
  * SPLIT numerics on canonical weights, no workspace, at the design bound;
  * the tiled layout under automatic dispatch with a workspace (FAST GEMM for
    M > 16, the skinny kernel below): against the oracle at the acceptance
    bar, on the whole output and row by row, and within the FAST budget;
  * for the square projection at 1024^2, the benchmark's exact step
    (``qlinear_fast_activations`` then the FAST GEMM on those activations,
    bit-identical to the automatic call) and EXACT on tiled weights.
The oracle quantizes and packs the weights on the CPU and computes the whole
output (fp32 dequantized weights, fp64 product): the largest case (2048^2
sweep, N = 13824) holds about 3 GB of fp64 operands on the host. Weights go to
the device as the oracle's bytes, so the device quantizer is not involved
(it is checked byte for byte elsewhere)."""
import numpy as np
import pytest

import oracle
from group_wise_affine_qlinear_amd import inputs
from group_wise_affine_qlinear_amd import qlinear as ql

from gpu_helpers import MAXABS_RMS_DESIGN, RELF_DESIGN, assert_rows, dev, torch_or_skip

pytestmark = pytest.mark.gpu

# FAST numerics budget against the exact product (fp16 rounding of the weights)
RELF_FAST = 5e-4
MAXABS_RMS_FAST = 4e-3

CASES = [(name, bits) for name, wl in inputs.WORKLOADS.items() for bits in wl["bits"]]


@pytest.fixture(scope="module")
def torch():
    t = torch_or_skip()
    ql.load_library()
    return t


def check(y, ref, relf, maxabs, what):
    e = oracle.error_metrics(y, ref)
    assert e["relF"] <= relf and e["maxabs_over_rms"] <= maxabs, (what, e)
    return e


@pytest.mark.parametrize("name,bits", CASES)
def test_full_size_full_output(torch, name, bits):
    wl = inputs.WORKLOADS[name]
    M, K, N = wl["M"], wl["K"], wl["N"]
    w = inputs.weights(N, K, wl["id"])
    x = inputs.activations_bf16(M, K, wl["id"], wl["x"])
    q, s16, b16 = oracle.quantize_rtn(w, bits)
    packed = oracle.pack(q, bits)
    del w, q
    ref = oracle.forward(x, packed, s16, b16, bits, K)

    xd, pd, sd, bd = dev(torch, x), dev(torch, packed), dev(torch, s16), dev(torch, b16)
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")

    def host(y):
        assert bool(torch.isfinite(y).all()), "non-finite output"
        return y.cpu().numpy()

    # the spec call: canonical weights, no workspace
    out.fill_(float("nan"))
    ql.qlinear_forward(xd, pd, sd, bd, bits, 64, M, N, K, out)
    torch.cuda.synchronize()
    path = ql.qlinear_last_path()
    assert path.startswith(("skinny", "gemv") if M <= 16 else "gemm3_f16online"), path
    y = host(out)
    if M > 16:
        check(y, ref, RELF_FAST, MAXABS_RMS_FAST, ("qlinear_forward, FAST budget", path))
    else:
        check(y, ref, RELF_DESIGN, MAXABS_RMS_DESIGN, ("qlinear_forward", path))
    assert_rows(y, ref, what=("qlinear_forward rows", path))
    if M > 16:
        # SPLIT numerics, no workspace: the exact-mode bound
        out.fill_(float("nan"))
        ql.qlinear_forward_ex(xd, pd, sd, bd, bits, M, N, K, out, mode=ql.QL_MODE_SPLIT, workspace=None)
        torch.cuda.synchronize()
        path = ql.qlinear_last_path()
        assert path.startswith("gemm4_bf16x2"), path
        check(host(out), ref, RELF_DESIGN, MAXABS_RMS_DESIGN, ("split, no workspace", path))

    # tiled layout, automatic dispatch with a workspace
    tq, tsb = ql.qlinear_repack(pd, sd, bd, bits, 64, N, K)
    del pd, sd, bd
    out.fill_(float("nan"))
    ql.qlinear_forward_ex(xd, tq, tsb, None, bits, M, N, K, out, layout=ql.QL_LAYOUT_TILED)
    torch.cuda.synchronize()
    path = ql.qlinear_last_path()
    y = host(out)
    if M > 16:
        assert path.startswith("gemm3"), path
        assert_rows(y, ref, what=("tiled auto, acceptance, rows", path))
        check(y, ref, RELF_FAST, MAXABS_RMS_FAST, ("tiled auto, FAST budget", path))
    else:
        assert path.startswith("skinny"), path
        check(y, ref, RELF_DESIGN, MAXABS_RMS_DESIGN, ("tiled auto", path))

    if name == "square_4096":
        # the benchmark's step: shared fp16 activations, then the FAST GEMM
        x16, rs = ql.qlinear_fast_activations(xd, M, K)
        y2 = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        ql.qlinear_forward_ex(xd, tq, tsb, None, bits, M, N, K, y2, layout=ql.QL_LAYOUT_TILED,
                              mode=ql.QL_MODE_FAST, x16=x16, rowscale=rs)
        torch.cuda.synchronize()
        assert bool(torch.equal(y2, out)), "given activations changed the result"
        # EXACT on tiled weights (the benchmark's exact-mode row)
        out.fill_(float("nan"))
        ql.qlinear_forward_ex(xd, tq, tsb, None, bits, M, N, K, out, layout=ql.QL_LAYOUT_TILED,
                              mode=ql.QL_MODE_EXACT)
        torch.cuda.synchronize()
        check(host(out), ref, RELF_DESIGN, MAXABS_RMS_DESIGN, ("tiled exact", ql.qlinear_last_path()))
