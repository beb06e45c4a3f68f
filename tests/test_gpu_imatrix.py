"""GPU tests of the device importance-weighted fit (qlinear_quantize_imatrix).

The kernel takes the same fp32 decisions as ``oracle.quantize_imatrix`` (one
rounding per operation, sums in order), so codes, scales and biases must be
byte-equal. Large weights are checked on a sample of rows: the fit of a row
depends only on that row and the importance vector."""
import numpy as np
import pytest

import oracle
from group_wise_affine_qlinear_amd import inputs
from group_wise_affine_qlinear_amd import qlinear as ql

from gpu_helpers import dev, host_u16, host_u32, torch_or_skip

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    t = torch_or_skip()
    ql.load_library()
    return t


def importance(kind, k, wid):
    rng = np.random.default_rng(wid)
    if kind == "outlier":   # E[x^2] of activations with 1% outlier channels
        x = inputs.activations_f32(64, k, wid, "outlier").astype(np.float64)
        return (x * x).mean(axis=0).astype(np.float32)
    if kind == "sparse":    # half of the channels unused
        a = rng.uniform(0.1, 3.0, k).astype(np.float32)
        a[rng.random(k) < 0.5] = 0
        return a
    if kind == "wide":      # importances over eight decades
        return (10.0 ** rng.uniform(-4, 4, k)).astype(np.float32)
    return np.ones(k, np.float32)


def run(torch, w, imp, bits):
    N, K = w.shape
    p = torch.empty((N, K * bits // 32), dtype=torch.int32, device="cuda")
    s = torch.empty((N, K // 64), dtype=torch.int16, device="cuda")
    b = torch.empty((N, K // 64), dtype=torch.int16, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    ql.qlinear_quantize_imatrix(torch.from_numpy(w).cuda(), torch.from_numpy(imp).cuda(), bits, 64, N, K,
                                p, s, b, st)
    torch.cuda.synchronize()
    return host_u32(p), host_u16(s), host_u16(b), int(st.item())


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("kind", ["outlier", "sparse", "wide", "uniform"])
def test_imatrix_byte_equal_to_oracle(torch, bits, kind):
    N, K = 130, 640
    w = inputs.weights(N, K, 600 + bits)
    imp = importance(kind, K, 610 + bits)
    p, s, b, st = run(torch, w, imp, bits)
    assert st == 0
    q, s16, b16 = oracle.quantize_imatrix(w, imp, bits)
    assert np.array_equal(s, s16) and np.array_equal(b, b16)
    assert np.array_equal(p, oracle.pack(q, bits))


@pytest.mark.parametrize("bits", [4, 8])
def test_imatrix_never_worse_than_rtn_on_device(torch, bits):
    N, K = 256, 1024
    w = inputs.weights(N, K, 620 + bits)
    imp = importance("outlier", K, 621)
    p, s, b, st = run(torch, w, imp, bits)
    q = oracle.unpack(p, bits, K)
    q0, s0, b0 = oracle.quantize_rtn(w, bits)
    e = oracle.weighted_error(w, imp, q, s, b)
    e0 = oracle.weighted_error(w, imp, q0, s0, b0)
    assert np.all(e <= e0 * (1 + 1e-6) + 1e-30)
    assert e.sum() < 0.6 * e0.sum()


def test_imatrix_qkv_weight_sampled_rows(torch):
    # the QKV projection weight at full size (13824 x 4608, 4-bit) with
    # outlier-channel importance; 48 rows rechecked by the oracle
    N, K = 13824, 4608
    w = inputs.weights(N, K, 2)
    imp = importance("outlier", K, 2)
    p, s, b, st = run(torch, w, imp, 4)
    assert st == 0
    rows = np.unique(np.concatenate([[0, 1, N - 1], np.random.default_rng(630).integers(0, N, 45)]))
    q, s16, b16 = oracle.quantize_imatrix(w[rows], imp, 4)
    assert np.array_equal(s[rows], s16) and np.array_equal(b[rows], b16)
    assert np.array_equal(p[rows], oracle.pack(q, 4))


def test_imatrix_flags_bad_importance(torch):
    w = inputs.weights(8, 128, 640)
    imp = np.ones(128, np.float32)
    imp[5] = -1.0
    _, _, _, st = run(torch, w, imp, 4)
    assert st == -1   # QL_EINVAL
    imp[5] = np.nan
    _, _, _, st = run(torch, w, imp, 4)
    assert st == -1
