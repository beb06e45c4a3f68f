"""GPU parity at the full sizes of the configured workloads, on sampled outputs.

Every workload of ``inputs.WORKLOADS`` runs at its full shape through the
launches the benchmark times: the canonical entry point (``qlinear_forward``,
EXACT numerics) and the tiled layout with automatic dispatch (FAST numerics
for M > 16, the skinny kernel for M <= 16); the headline square projection
also runs the benchmark's exact sequence (``qlinear_fast_activations`` then
``qlinear_forward_ex`` with the fp16 activations). The oracle, on the CPU,
quantizes and packs the weights and computes a sampled block of outputs (rows
and columns at tile edges, ragged ends and random positions) one by one from
its definition; the GPU result is checked on that block and for finiteness
everywhere."""
import numpy as np
import pytest

import oracle
from group_wise_affine_qlinear_amd import inputs
from group_wise_affine_qlinear_amd import qlinear as ql

from gpu_helpers import MAXABS_RMS_DESIGN, MAXABS_RMS_TOL, RELF_DESIGN, RELF_TOL, dev, torch_or_skip

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


def sample(n, seed, extra=60):
    """Indices at tile edges (multiples of 256 and their neighbours), both ends
    and `extra` seeded random positions, sorted and unique, all < n."""
    edges = [0, 1, 15, 16, 31, 32, 255, 256, 511, 512, n // 2, n - 2, n - 1]
    rng = np.random.default_rng(seed)
    idx = set(i for i in edges if 0 <= i < n)
    idx.update(rng.integers(0, n, size=min(extra, n)).tolist())
    return np.array(sorted(idx), dtype=np.int64)


def check(y_block, ref, relf, maxabs, what):
    e = oracle.error_metrics(y_block, ref)
    assert e["relF"] <= relf and e["maxabs_over_rms"] <= maxabs, (what, e)
    return e


@pytest.mark.parametrize("name,bits", CASES)
def test_full_size_sampled(torch, name, bits):
    wl = inputs.WORKLOADS[name]
    M, K, N = wl["M"], wl["K"], wl["N"]
    w = inputs.weights(N, K, wl["id"])
    x = inputs.activations_bf16(M, K, wl["id"], wl["x"])
    q, s16, b16 = oracle.quantize_rtn(w, bits)
    packed = oracle.pack(q, bits)
    del w, q
    rows, cols = sample(M, 1000 + wl["id"]), sample(N, 2000 + wl["id"])
    ref = oracle.forward_rows(x, packed, s16, b16, bits, K, rows, cols)

    xd, pd, sd, bd = dev(torch, x), dev(torch, packed), dev(torch, s16), dev(torch, b16)
    ri, ci = torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")

    def block(y):
        assert bool(torch.isfinite(y).all()), "non-finite output"
        return y.index_select(0, ri).index_select(1, ci).cpu().numpy()

    # canonical layout, the primary entry point (EXACT numerics)
    out.fill_(float("nan"))
    ql.qlinear_forward(xd, pd, sd, bd, bits, 64, M, N, K, out)
    torch.cuda.synchronize()
    check(block(out), ref, RELF_DESIGN, MAXABS_RMS_DESIGN, ("canonical", ql.qlinear_last_path()))

    # tiled layout, automatic dispatch
    tq, tsb = ql.qlinear_repack(pd, sd, bd, bits, 64, N, K)
    del pd, sd, bd
    out.fill_(float("nan"))
    ql.qlinear_forward_ex(xd, tq, tsb, None, bits, M, N, K, out, layout=ql.QL_LAYOUT_TILED)
    torch.cuda.synchronize()
    path = ql.qlinear_last_path()
    if M > 16:
        assert path.startswith("gemm3"), path
        check(block(out), ref, RELF_TOL, MAXABS_RMS_TOL, ("tiled auto, acceptance", path))
        check(block(out), ref, RELF_FAST, MAXABS_RMS_FAST, ("tiled auto, FAST budget", path))
    else:
        assert path.startswith("skinny"), path
        check(block(out), ref, RELF_DESIGN, MAXABS_RMS_DESIGN, ("tiled auto", path))

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
        check(block(out), ref, RELF_DESIGN, MAXABS_RMS_DESIGN, ("tiled exact", ql.qlinear_last_path()))
