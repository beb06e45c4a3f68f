"""GPU tests of the tiled weight layout: repack matches the layout definition
(restated here independently of the library), unrepack inverts it bit for bit,
and the forward on tiled weights matches the oracle."""
import numpy as np
import pytest

import oracle
from group_wise_affine_qlinear_amd import inputs, qlinear as ql

from gpu_helpers import Case, assert_parity, dev, host_u16, host_u32, run_forward, torch_or_skip

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    t = torch_or_skip()
    ql.load_library()
    return t


def reference_tiling(q, s16, b16, bits):
    """The tiled layout written out from its definition (include/qlinear.h, layout.hip)."""
    N, K = q.shape
    G, N32, WPG = K // 64, (N + 31) // 32, 2 * bits
    tiled = np.zeros(N32 * G * 32 * WPG, np.uint32)
    sb = np.zeros(N32 * G * 32, np.uint32)
    for st in range(N32):
        for g in range(G):
            base = (st * G + g) * 32 * WPG
            for col in range(32):
                n = st * 32 + col
                if n >= N:
                    continue
                c = q[n, 64 * g:64 * g + 64].astype(np.uint32)
                if bits == 4:
                    for h in range(2):
                        for t in range(4):
                            e = c[32 * h + 8 * t:32 * h + 8 * t + 8]
                            word = sum(int(e[2 * p]) << (4 * p) | int(e[2 * p + 1]) << (16 + 4 * p) for p in range(4))
                            tiled[base + h * 128 + col * 4 + t] = word
                elif bits == 8:
                    for part in range(2):
                        for h in range(2):
                            for t in range(4):
                                e = c[32 * h + 16 * part + 4 * t:32 * h + 16 * part + 4 * t + 4]
                                word = sum(int(e[i]) << (8 * i) for i in range(4))
                                tiled[base + part * 256 + h * 128 + col * 4 + t] = word
                elif bits == 2:
                    for h in range(2):
                        for t in range(2):
                            e = c[32 * h + 16 * t:32 * h + 16 * t + 16]
                            word = sum(int(e[2 * p]) << (2 * p) | int(e[2 * p + 1]) << (16 + 2 * p) for p in range(8))
                            tiled[base + h * 64 + col * 2 + t] = word
                else:
                    # 3-bit: the low two bits as the 2-bit block, then one word
                    # of high bits per (half, column): code 32h + 2P at bit P,
                    # code 32h + 2P + 1 at bit 16 + P
                    for h in range(2):
                        for t in range(2):
                            e = c[32 * h + 16 * t:32 * h + 16 * t + 16] & 3
                            word = sum(int(e[2 * p]) << (2 * p) | int(e[2 * p + 1]) << (16 + 2 * p) for p in range(8))
                            tiled[base + h * 64 + col * 2 + t] = word
                        e = c[32 * h:32 * h + 32] >> 2
                        tiled[base + 128 + h * 32 + col] = sum(int(e[2 * p]) << p | int(e[2 * p + 1]) << (16 + p)
                                                               for p in range(16))
                sb[(st * G + g) * 32 + col] = int(s16[n, g]) | (int(b16[n, g]) << 16)
    return tiled, sb


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_repack_matches_definition_and_round_trips(torch, bits):
    c = Case(1, 70, 256, bits, wid=301)   # 70 rows: a ragged last strip
    _, p, s, b = c.device(torch)
    tq, tsb = ql.qlinear_repack(p, s, b, bits, 64, c.N, c.K)
    torch.cuda.synchronize()
    ref_q, ref_sb = reference_tiling(c.q, c.s16, c.b16, bits)
    assert np.array_equal(host_u32(tq), ref_q)
    assert np.array_equal(host_u32(tsb), ref_sb)
    p2 = torch.zeros_like(p)
    s2 = torch.zeros_like(s)
    b2 = torch.zeros_like(b)
    ql.qlinear_unrepack(tq, tsb, bits, 64, c.N, c.K, p2, s2, b2)
    torch.cuda.synchronize()
    assert np.array_equal(host_u32(p2), c.packed)
    assert np.array_equal(host_u16(s2), c.s16) and np.array_equal(host_u16(b2), c.b16)


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("M", [1, 2, 5, 8, 16])
def test_skinny_tiled_parity(torch, bits, M):
    c = Case(M, 300, 1536, bits, wid=310 + M)
    x, p, s, b = c.device(torch)
    tq, tsb = ql.qlinear_repack(p, s, b, bits, 64, c.N, c.K)
    out = torch.full((M, c.N), float("nan"), dtype=torch.float32, device="cuda")
    ql.qlinear_forward_ex(x, tq, tsb, None, bits, M, c.N, c.K, out, layout=ql.QL_LAYOUT_TILED,
                          path=ql.QL_PATH_SKINNY)
    torch.cuda.synchronize()
    assert "tiled" in ql.qlinear_last_path()
    assert_parity(out.cpu().numpy(), c.reference(), what=ql.qlinear_last_path())


def test_tiled_identity_rows_exact(torch):
    K, N, M = 512, 100, 16
    cols = np.array([0, 1, 63, 64, 100, 127, 128, 200, 255, 256, 300, 383, 384, 450, 510, 511])
    x = np.zeros((M, K), np.uint16)
    x[np.arange(M), cols] = 0x3F80
    c = Case(M, N, K, 8, wid=320, x=x)
    xd, p, s, b = c.device(torch)
    tq, tsb = ql.qlinear_repack(p, s, b, 8, 64, N, K)
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ql.qlinear_forward_ex(xd, tq, tsb, None, 8, M, N, K, out, layout=ql.QL_LAYOUT_TILED)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), oracle.dequantize(c.q, c.s16, c.b16)[:, cols].T)


# Shapes for the 128x64-wave-tile GEMM: several block tiles in M and N with
# ragged edges, odd and even group counts (its K loop runs groups in pairs).
GEMM2_SHAPES = [(520, 390, 320), (200, 300, 1024), (129, 129, 192), (17, 40, 64), (384, 256, 512)]


@pytest.mark.parametrize("layout", [ql.QL_LAYOUT_CANONICAL, ql.QL_LAYOUT_TILED])
@pytest.mark.parametrize("tile", [10, 11])
@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("shape", GEMM2_SHAPES)
def test_gemm2_parity(torch, shape, bits, tile, layout):
    M, N, K = shape
    c = Case(M, N, K, bits, wid=330 + bits, x_structure="outlier")
    ref = c.reference()
    y = run_forward(torch, c, path=ql.QL_PATH_GEMM, tile=tile, layout=layout)
    assert ql.qlinear_last_path().startswith("gemm2"), ql.qlinear_last_path()
    assert_parity(y.cpu().numpy(), ref, what=ql.qlinear_last_path())
    if K >= 192:
        y = run_forward(torch, c, path=ql.QL_PATH_SPLITK, split_k=3, tile=tile, layout=layout)
        assert_parity(y.cpu().numpy(), ref, what=ql.qlinear_last_path())


@pytest.mark.parametrize("layout", [ql.QL_LAYOUT_CANONICAL, ql.QL_LAYOUT_TILED])
@pytest.mark.parametrize("bits", [2, 4, 8])
def test_gemm2_bf16_out(torch, bits, layout):
    c = Case(300, 260, 384, bits, wid=340 + bits)
    ref = run_forward(torch, c, path=ql.QL_PATH_GEMM, tile=10, layout=layout).cpu().numpy()
    y = run_forward(torch, c, path=ql.QL_PATH_GEMM, tile=10, layout=layout, out_dtype="bf16")
    # same accumulation, rounded to nearest-even bf16 at the store
    got = y.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, inputs.f32_to_bf16_bits(ref))


# Split tail: with the resident-block count forced small, the tiles past the
# last full round are cut into K pieces whose partials the last finisher adds.
# (slots, shape) pairs cover 2 and 5 pieces, an uneven last piece, the 8-XCD
# piece placement (8 tail tiles, 16 slots) and both tile heights.
SPLIT_TAIL_CASES = [
    (10, 10, (520, 390, 320)),    # 12 tiles: 10 whole, 2 tail tiles x 5 pieces of 1 group
    (10, 8, (520, 390, 448)),     # 12 tiles: 8 whole, 4 tail tiles x 2 pieces (G=7: 4+3)
    (10, 16, (520, 1000, 640)),   # 24 tiles: 16 whole, 8 tail tiles x 2 pieces, XCD placement
    (11, 6, (300, 260, 576)),     # 128x128 tiles: 9 tiles, 6 whole, 3 tail tiles x 2 pieces
]


@pytest.mark.parametrize("layout", [ql.QL_LAYOUT_CANONICAL, ql.QL_LAYOUT_TILED])
@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("tile,slots,shape", SPLIT_TAIL_CASES)
def test_gemm2_split_tail(torch, monkeypatch, tile, slots, shape, bits, layout):
    M, N, K = shape
    monkeypatch.setenv("QLINEAR_GEMM_SLOTS", str(slots))
    c = Case(M, N, K, bits, wid=350 + bits)
    ref = c.reference()
    y1 = run_forward(torch, c, path=ql.QL_PATH_GEMM, tile=tile, layout=layout)
    assert "_tail" in ql.qlinear_last_path(), ql.qlinear_last_path()
    assert_parity(y1.cpu().numpy(), ref, what=ql.qlinear_last_path())
    # the counters are re-armed and the piece order is fixed: a second call is
    # bit-identical
    y2 = run_forward(torch, c, path=ql.QL_PATH_GEMM, tile=tile, layout=layout)
    assert np.array_equal(y1.cpu().numpy().view(np.uint32), y2.cpu().numpy().view(np.uint32))
    yb = run_forward(torch, c, path=ql.QL_PATH_GEMM, tile=tile, layout=layout, out_dtype="bf16")
    got = yb.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, inputs.f32_to_bf16_bits(y1.cpu().numpy()))
