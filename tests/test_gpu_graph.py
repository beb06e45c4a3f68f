"""GPU test: the forward path inside a captured HIP graph.

A serving loop can capture its projections once and replay them. The library
allocates nothing and records no memset, so the sequence below (fp16
activations, the FAST GEMM plain and with both fused epilogues, the exact-mode
GEMM with a K split, the skinny kernel, the FAST GEMM on canonical weights and
the scratch-free SPLIT GEMM of the spec call) is captured on a side
stream and replayed several times, with eager work and synchronizations
between replays; every replay must give the eager results bit for bit."""
import numpy as np
import pytest

from group_wise_affine_qlinear_amd import inputs
from group_wise_affine_qlinear_amd import qlinear as ql

from gpu_helpers import Case, dev, torch_or_skip

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    t = torch_or_skip()
    ql.load_library()
    return t


def test_graph_replays_match_eager(torch):
    M, N, K, bits = 520, 768, 448, 4
    c = Case(M, N, K, bits, wid=700)
    x, p, s, b = c.device(torch)
    tq, tsb = ql.qlinear_repack(p, s, b, bits, 64, N, K)
    gq, gsb = ql.qlinear_repack_glu(p, s, b, bits, 64, N, K)
    cs = Case(8, N, K, bits, wid=701)
    xs = dev(torch, cs.x)
    ws_bytes = max(ql.qlinear_workspace_bytes(bits, M, N, K), 16)
    # the forced 3-way K split needs its fp32 partials beyond the automatic bound
    ws_split = ws_bytes + 3 * M * N * 4 + (K // 64) * 1024 * 4
    ws = [torch.empty(n // 4 + 64, dtype=torch.int32, device="cuda") for n in (ws_bytes, ws_split, ws_bytes)]
    res0 = torch.from_numpy(inputs.residual_stream(M, N, 702)).cuda()
    gate = torch.from_numpy(inputs.adaln_gate(2, N, 702)).cuda()
    x16 = torch.empty((M, K), dtype=torch.float16, device="cuda")
    rs = torch.empty((M,), dtype=torch.float32, device="cuda")
    y_fast = torch.empty((M, N), dtype=torch.float32, device="cuda")
    y_glu = torch.empty((M, N // 2), dtype=torch.bfloat16, device="cuda")
    y_res = torch.empty((M, N), dtype=torch.float32, device="cuda")
    y_exact = torch.empty((M, N), dtype=torch.float32, device="cuda")
    y_skinny = torch.empty((8, N), dtype=torch.float32, device="cuda")
    y_canon = torch.empty((M, N), dtype=torch.float32, device="cuda")
    y_split = torch.empty((M, N), dtype=torch.float32, device="cuda")
    y_online = torch.empty((M, N), dtype=torch.float32, device="cuda")

    def sequence():
        ql.qlinear_fast_activations(x, M, K, x16, rs)
        ql.qlinear_forward_ex(x, tq, tsb, None, bits, M, N, K, y_fast, layout=ql.QL_LAYOUT_TILED,
                              mode=ql.QL_MODE_FAST, x16=x16, rowscale=rs, workspace=ws[0])
        ql.qlinear_forward_ex(x, gq, gsb, None, bits, M, N, K, y_glu, layout=ql.QL_LAYOUT_TILED,
                              x16=x16, rowscale=rs, epilogue=ql.QL_EPI_SWIGLU, workspace=ws[0])
        ql.qlinear_forward_ex(x, tq, tsb, None, bits, M, N, K, y_res, layout=ql.QL_LAYOUT_TILED,
                              x16=x16, rowscale=rs, epilogue=ql.QL_EPI_GATE_RESIDUAL, residual=y_res,
                              gate=gate, gate_rows=260, workspace=ws[0])
        ql.qlinear_forward_ex(x, p, s, b, bits, M, N, K, y_exact, path=ql.QL_PATH_SPLITK, split_k=3,
                              mode=ql.QL_MODE_EXACT, workspace=ws[1])
        ql.qlinear_forward_ex(xs, p, s, b, bits, 8, N, K, y_skinny, workspace=ws[2])
        # canonical weights with a workspace: fp16 prepass into it, FAST GEMM on the code rows
        ql.qlinear_forward_ex(x, p, s, b, bits, M, N, K, y_canon, workspace=ws[0])
        # the spec call's plan (no workspace: FAST converting x in the
        # GEMM, then the recomputation launch) on the capture stream;
        # qlinear_forward itself launches on the default stream
        ql.qlinear_forward_ex(x, p, s, b, bits, M, N, K, y_online, workspace=None)
        ql.qlinear_forward_ex(x, p, s, b, bits, M, N, K, y_split, mode=ql.QL_MODE_SPLIT, workspace=None)

    outs = (y_fast, y_glu, y_res, y_exact, y_skinny, y_canon, y_online, y_split)
    y_res.copy_(res0)
    sequence()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        y_res.copy_(res0)
        sequence()   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=side):
        sequence()
    torch.cuda.synchronize()

    for rep in range(3):
        for o in outs:
            o.fill_(float("nan")) if o.dtype == torch.float32 else o.zero_()
        y_res.copy_(res0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, eager)):
            same = torch.equal(o.view(torch.int16) if o.dtype == torch.bfloat16 else o.view(torch.int32),
                               e.view(torch.int16) if e.dtype == torch.bfloat16 else e.view(torch.int32))
            assert same, (rep, i)
        _ = (torch.randn(256, 256, device="cuda") @ torch.randn(256, 256, device="cuda")).sum().item()
