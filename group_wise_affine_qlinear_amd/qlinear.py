"""ctypes binding over libqlinear's C ABI (``include/qlinear.h``).

Argument marshalling only: every step of the product runs in the HIP library.
Device arguments are torch CUDA tensors (PyTorch supplies device memory and the
stream); host helpers take numpy arrays. Each function has the name of the C
entry point it calls. A non-zero status raises ``QLinearError``. The library is
loaded on first use; if it is not built the call fails loudly (there is no
fallback of any kind).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqlinear.so")

QL_OK, QL_EINVAL, QL_EALIGN, QL_EUNSUPPORTED, QL_EWORKSPACE, QL_EHIP, QL_ERANGE = 0, -1, -2, -3, -4, -5, -6
QL_OUT_F32, QL_OUT_BF16 = 0, 1
QL_PATH_AUTO, QL_PATH_SKINNY, QL_PATH_GEMM, QL_PATH_SPLITK = 0, 1, 2, 3
QL_LAYOUT_CANONICAL, QL_LAYOUT_TILED = 0, 1
QL_MODE_AUTO, QL_MODE_EXACT, QL_MODE_FAST, QL_MODE_SPLIT = 0, 1, 2, 3
QL_EPI_NONE, QL_EPI_SWIGLU, QL_EPI_GATE_RESIDUAL = 0, 1, 2

EXPORTED = (
    "qlinear_forward", "qlinear_forward_ex", "qlinear_workspace_bytes", "qlinear_packed_words",
    "qlinear_pack_host", "qlinear_unpack_host", "qlinear_quantize_rtn_host", "qlinear_quantize_rtn",
    "qlinear_dequantize", "qlinear_status_string", "qlinear_last_path", "qlinear_version",
    "qlinear_group_sums", "qlinear_group_sums_ld", "qlinear_tiled_words", "qlinear_tiled_sb_words",
    "qlinear_repack", "qlinear_unrepack", "qlinear_fast_activations", "qlinear_fast_activations_adaln",
    "qlinear_repack_glu",
    "qlinear_unrepack_glu", "qlinear_quantize_imatrix", "qlinear_forward_workspace_bytes",
    "qlinear_forward_noalloc", "qlinear_forward_noalloc_max_scratch",
)


class QLinearError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({qlinear_status_string(status)})")


class ql_forward_args(ctypes.Structure):
    _fields_ = [
        ("x", ctypes.c_void_p),
        ("packed_q", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
        ("biases", ctypes.c_void_p),
        ("bits", ctypes.c_int),
        ("group", ctypes.c_int),
        ("M", ctypes.c_int64),
        ("N", ctypes.c_int64),
        ("K", ctypes.c_int64),
        ("out", ctypes.c_void_p),
        ("out_dtype", ctypes.c_int),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("path", ctypes.c_int),
        ("split_k", ctypes.c_int),
        ("tile", ctypes.c_int),
        ("xsum", ctypes.c_void_p),
        ("ld_xsum", ctypes.c_int64),
        ("layout", ctypes.c_int),
        ("mode", ctypes.c_int),
        ("x16", ctypes.c_void_p),
        ("rowscale", ctypes.c_void_p),
        ("epilogue", ctypes.c_int),
        ("residual", ctypes.c_void_p),
        ("gate", ctypes.c_void_p),
        ("gate_rows", ctypes.c_int64),
    ]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load (once) and return libqlinear with argument types declared."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"libqlinear.so not found at {path}; build it with "
            "`python -m group_wise_affine_qlinear_amd.build` (hipcc, gfx950)")
    # torch ships its own HIP runtime; loading it first makes the library bind
    # to that same runtime, so device pointers and streams from torch are valid
    # in the library's calls (a second runtime instance would not know them)
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    i64, vp, i32, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    sig = {
        "qlinear_forward": ([vp, vp, vp, vp, i32, i32, i64, i64, i64, vp], i32),
        "qlinear_forward_ex": ([ctypes.POINTER(ql_forward_args), vp], i32),
        "qlinear_workspace_bytes": ([i32, i64, i64, i64], sz),
        "qlinear_forward_workspace_bytes": ([ctypes.POINTER(ql_forward_args)], sz),
        "qlinear_forward_noalloc": ([ctypes.POINTER(ql_forward_args), vp], i32),
        "qlinear_forward_noalloc_max_scratch": ([], sz),
        "qlinear_packed_words": ([i32, i64, i64], sz),
        "qlinear_pack_host": ([vp, i32, i64, i64, vp], i32),
        "qlinear_unpack_host": ([vp, i32, i64, i64, vp], i32),
        "qlinear_quantize_rtn_host": ([vp, i32, i32, i64, i64, vp, vp, vp], i32),
        "qlinear_quantize_rtn": ([vp, i32, i32, i64, i64, vp, vp, vp, vp, vp], i32),
        "qlinear_quantize_imatrix": ([vp, vp, i32, i32, i64, i64, vp, vp, vp, vp, vp], i32),
        "qlinear_dequantize": ([vp, vp, vp, i32, i32, i64, i64, vp, vp], i32),
        "qlinear_status_string": ([i32], ctypes.c_char_p),
        "qlinear_last_path": ([ctypes.c_char_p, sz], i32),
        "qlinear_version": ([], i32),
        "qlinear_group_sums": ([vp, i64, i64, vp, i64, vp], i32),
        "qlinear_group_sums_ld": ([i64], i64),
        "qlinear_fast_activations": ([vp, i64, i64, vp, vp, vp], i32),
        "qlinear_fast_activations_adaln": ([vp, vp, i64, i64, i64, vp, vp, vp], i32),
        "qlinear_tiled_words": ([i32, i64, i64], sz),
        "qlinear_tiled_sb_words": ([i64, i64], sz),
        "qlinear_repack": ([vp, vp, vp, i32, i32, i64, i64, vp, vp, vp], i32),
        "qlinear_unrepack": ([vp, vp, i32, i32, i64, i64, vp, vp, vp, vp], i32),
        "qlinear_repack_glu": ([vp, vp, vp, i32, i32, i64, i64, vp, vp, vp], i32),
        "qlinear_unrepack_glu": ([vp, vp, i32, i32, i64, i64, vp, vp, vp, vp], i32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _check(status: int, where: str):
    if status != QL_OK:
        raise QLinearError(status, where)


# ------------------------------------------------------------------ torch helpers

def _torch():
    import torch
    return torch


def _dev_ptr(t, name, dtypes, shape=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


def _stream_handle(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _u16(torch):
    return (torch.int16, torch.uint16, torch.float16, torch.bfloat16)


# ------------------------------------------------------------------ device entry points

def qlinear_forward(x, packed_q, scales, biases, bits, group, M, N, K, out):
    """C ``qlinear_forward``: out[M, N] fp32 = x[M, K] (bf16) @ W_hat^T, default stream."""
    torch = _torch()
    u16 = _u16(torch)
    lib = load_library()
    G = K // group if group else 0
    st = lib.qlinear_forward(
        _dev_ptr(x, "x", u16, (M, K)),
        _dev_ptr(packed_q, "packed_q", (torch.int32, torch.uint32), (N, K * bits // 32)),
        _dev_ptr(scales, "scales", u16, (N, G)),
        _dev_ptr(biases, "biases", u16, (N, G)),
        bits, group, M, N, K,
        _dev_ptr(out, "out", (torch.float32,), (M, N)))
    _check(st, "qlinear_forward")
    return out


# Default of ``qlinear_forward_ex(workspace=...)``: a workspace of
# ``qlinear_workspace_bytes`` taken from torch's caching allocator for the call.
TORCH_WORKSPACE = "torch"


def qlinear_forward_ex(x, packed_q, scales, biases, bits, M, N, K, out, *, group=64,
                       workspace=TORCH_WORKSPACE, stream=None, path=QL_PATH_AUTO, split_k=0, tile=0,
                       xsum=None, layout=QL_LAYOUT_CANONICAL, mode=QL_MODE_AUTO, x16=None,
                       rowscale=None, epilogue=QL_EPI_NONE, residual=None, gate=None, gate_rows=0):
    """C ``qlinear_forward_ex``: explicit stream, workspace, out dtype, layout, numerics mode
    and forced path.

    With ``layout=QL_LAYOUT_TILED``, ``packed_q`` and ``scales`` are the outputs of
    ``qlinear_repack`` (tiled codes, tiled scale|bias words) and ``biases`` is ignored.
    ``mode`` is a ``ql_mode`` (AUTO: FAST for the large-M path; with no workspace and no
    ``x16`` the GEMM converts x to fp16 itself). ``workspace`` is a device tensor the library may use
    as scratch, ``None`` (the call keeps to plans that need none, as the C call with a NULL
    workspace), or by default a tensor of ``qlinear_workspace_bytes`` bytes that torch's caching
    allocator provides on the call's stream (the library itself never allocates);
    ``x16``/``rowscale`` are optional FAST-mode activations from ``qlinear_fast_activations``.
    ``epilogue=QL_EPI_SWIGLU`` takes GLU-ordered tiled weights (``qlinear_repack_glu``) and
    writes ``out`` [M, N/2] = silu(gate) * up. ``epilogue=QL_EPI_GATE_RESIDUAL`` writes
    ``out`` = ``residual`` + ``gate``[m // ``gate_rows``] * y (``residual`` [M, N] of out's
    dtype, may be ``out``; ``gate`` fp32 [ceil(M / gate_rows), N]).
    """
    torch = _torch()
    u16 = _u16(torch)
    lib = load_library()
    G = K // group if group else 0
    a = ql_forward_args()
    a.x = _dev_ptr(x, "x", u16, (M, K))
    a.layout = layout
    if layout == QL_LAYOUT_TILED:
        a.packed_q = _dev_ptr(packed_q, "packed_q", (torch.int32, torch.uint32), (qlinear_tiled_words(bits, N, K),))
        a.scales = _dev_ptr(scales, "scales", (torch.int32, torch.uint32), (qlinear_tiled_sb_words(N, K),))
        a.biases = None
    else:
        a.packed_q = _dev_ptr(packed_q, "packed_q", (torch.int32, torch.uint32), (N, K * bits // 32))
        a.scales = _dev_ptr(scales, "scales", u16, (N, G))
        a.biases = _dev_ptr(biases, "biases", u16, (N, G))
    a.bits, a.group, a.M, a.N, a.K = bits, group, M, N, K
    if out.dtype == torch.float32:
        a.out_dtype = QL_OUT_F32
    elif out.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        a.out_dtype = QL_OUT_BF16
    else:
        raise TypeError("out must be float32 or bfloat16")
    a.epilogue = epilogue
    a.out = _dev_ptr(out, "out", (out.dtype,), (M, N // 2 if epilogue == QL_EPI_SWIGLU else N))
    if isinstance(workspace, str):
        if workspace != TORCH_WORKSPACE:
            raise ValueError(f"workspace must be a device tensor, None or {TORCH_WORKSPACE!r}")
        workspace = None
        nbytes = -1   # sized below, once every field of the call is set
    else:
        nbytes = None
    a.path, a.split_k, a.tile, a.mode = path, split_k, tile, mode
    if xsum is not None:
        a.xsum = _dev_ptr(xsum, "xsum", (torch.float32,))
        a.ld_xsum = xsum.shape[1]
        if xsum.dim() != 2 or xsum.shape[0] != K // group:
            raise ValueError("xsum must be [K/64, ld_xsum]")
    if epilogue == QL_EPI_GATE_RESIDUAL:
        a.gate_rows = gate_rows
        if residual is not None:
            a.residual = _dev_ptr(residual, "residual", (out.dtype,), (M, N))
        if gate is not None and gate_rows >= 1:
            a.gate = _dev_ptr(gate, "gate", (torch.float32,), (-(-M // gate_rows), N))
    if x16 is not None:
        a.x16 = _dev_ptr(x16, "x16", (torch.float16, torch.int16), (M, K))
        a.rowscale = _dev_ptr(rowscale, "rowscale", (torch.float32,), (M,))
    if nbytes == -1:
        nbytes = int(lib.qlinear_forward_workspace_bytes(ctypes.byref(a)))
        if nbytes > 0:
            # allocated on the current stream; a call on another stream marks
            # the tensor in use there so the allocator does not hand it out early
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=x.device)
            if stream is not None and not isinstance(stream, int):
                workspace.record_stream(stream)
    if workspace is not None:
        a.workspace = _dev_ptr(workspace, "workspace", (workspace.dtype,))
        a.workspace_bytes = workspace.numel() * workspace.element_size()
    st = lib.qlinear_forward_ex(ctypes.byref(a), _stream_handle(stream))
    _check(st, "qlinear_forward_ex")
    return out


def qlinear_group_sums_ld(M) -> int:
    return int(load_library().qlinear_group_sums_ld(M))


def qlinear_group_sums(x, M, K, xsum=None, stream=None):
    """C ``qlinear_group_sums``: per-group row sums of x, [K/64, ld] fp32 (allocated if None)."""
    torch = _torch()
    lib = load_library()
    ld = qlinear_group_sums_ld(M)
    if xsum is None:
        xsum = torch.empty((K // 64, ld), dtype=torch.float32, device=x.device)
    st = lib.qlinear_group_sums(_dev_ptr(x, "x", _u16(torch), (M, K)), M, K,
                                _dev_ptr(xsum, "xsum", (torch.float32,)), xsum.shape[1],
                                _stream_handle(stream))
    _check(st, "qlinear_group_sums")
    return xsum


def qlinear_fast_activations(x, M, K, x16=None, rowscale=None, stream=None):
    """C ``qlinear_fast_activations``: fp16 x with per-row power-of-two scales (FAST mode)."""
    torch = _torch()
    lib = load_library()
    if x16 is None:
        x16 = torch.empty((M, K), dtype=torch.float16, device=x.device)
    if rowscale is None:
        rowscale = torch.empty((M,), dtype=torch.float32, device=x.device)
    st = lib.qlinear_fast_activations(_dev_ptr(x, "x", _u16(torch), (M, K)), M, K,
                                      _dev_ptr(x16, "x16", (torch.float16, torch.int16), (M, K)),
                                      _dev_ptr(rowscale, "rowscale", (torch.float32,), (M,)),
                                      _stream_handle(stream))
    _check(st, "qlinear_fast_activations")
    return x16, rowscale


def qlinear_fast_activations_adaln(x, scale, scale_rows, M, K, x16=None, rowscale=None, stream=None):
    """C ``qlinear_fast_activations_adaln``: FAST-mode activations of x * (1 + scale[m // scale_rows])."""
    torch = _torch()
    lib = load_library()
    if x16 is None:
        x16 = torch.empty((M, K), dtype=torch.float16, device=x.device)
    if rowscale is None:
        rowscale = torch.empty((M,), dtype=torch.float32, device=x.device)
    samples = -(-M // scale_rows) if scale_rows > 0 else 0
    st = lib.qlinear_fast_activations_adaln(_dev_ptr(x, "x", _u16(torch), (M, K)),
                                            _dev_ptr(scale, "scale", (torch.float32,), (samples, K)),
                                            scale_rows, M, K,
                                            _dev_ptr(x16, "x16", (torch.float16, torch.int16), (M, K)),
                                            _dev_ptr(rowscale, "rowscale", (torch.float32,), (M,)),
                                            _stream_handle(stream))
    _check(st, "qlinear_fast_activations_adaln")
    return x16, rowscale


def qlinear_tiled_words(bits, N, K) -> int:
    return int(load_library().qlinear_tiled_words(bits, N, K))


def qlinear_tiled_sb_words(N, K) -> int:
    return int(load_library().qlinear_tiled_sb_words(N, K))


def qlinear_repack(packed_q, scales, biases, bits, group, N, K, tiled_q=None, tiled_sb=None, stream=None):
    """C ``qlinear_repack``: canonical -> tiled; returns (tiled_q, tiled_sb) int32 tensors."""
    torch = _torch()
    u16 = _u16(torch)
    lib = load_library()
    dev = packed_q.device
    if tiled_q is None:
        tiled_q = torch.empty(qlinear_tiled_words(bits, N, K), dtype=torch.int32, device=dev)
    if tiled_sb is None:
        tiled_sb = torch.empty(qlinear_tiled_sb_words(N, K), dtype=torch.int32, device=dev)
    st = lib.qlinear_repack(
        _dev_ptr(packed_q, "packed_q", (torch.int32, torch.uint32), (N, K * bits // 32)),
        _dev_ptr(scales, "scales", u16, (N, K // group)),
        _dev_ptr(biases, "biases", u16, (N, K // group)), bits, group, N, K,
        _dev_ptr(tiled_q, "tiled_q", (torch.int32, torch.uint32), (qlinear_tiled_words(bits, N, K),)),
        _dev_ptr(tiled_sb, "tiled_sb", (torch.int32, torch.uint32), (qlinear_tiled_sb_words(N, K),)),
        _stream_handle(stream))
    _check(st, "qlinear_repack")
    return tiled_q, tiled_sb


def qlinear_repack_glu(packed_q, scales, biases, bits, group, N, K, tiled_q=None, tiled_sb=None, stream=None):
    """C ``qlinear_repack_glu``: stacked [gate; up] canonical weight -> tiled GLU order."""
    torch = _torch()
    u16 = _u16(torch)
    lib = load_library()
    dev = packed_q.device
    if tiled_q is None:
        tiled_q = torch.empty(qlinear_tiled_words(bits, N, K), dtype=torch.int32, device=dev)
    if tiled_sb is None:
        tiled_sb = torch.empty(qlinear_tiled_sb_words(N, K), dtype=torch.int32, device=dev)
    st = lib.qlinear_repack_glu(
        _dev_ptr(packed_q, "packed_q", (torch.int32, torch.uint32), (N, K * bits // 32)),
        _dev_ptr(scales, "scales", u16, (N, K // group)),
        _dev_ptr(biases, "biases", u16, (N, K // group)), bits, group, N, K,
        _dev_ptr(tiled_q, "tiled_q", (torch.int32, torch.uint32), (qlinear_tiled_words(bits, N, K),)),
        _dev_ptr(tiled_sb, "tiled_sb", (torch.int32, torch.uint32), (qlinear_tiled_sb_words(N, K),)),
        _stream_handle(stream))
    _check(st, "qlinear_repack_glu")
    return tiled_q, tiled_sb


def qlinear_unrepack_glu(tiled_q, tiled_sb, bits, group, N, K, packed_q, scales, biases, stream=None):
    """C ``qlinear_unrepack_glu``: tiled GLU order -> stacked [gate; up] canonical, into the given tensors."""
    torch = _torch()
    u16 = _u16(torch)
    lib = load_library()
    st = lib.qlinear_unrepack_glu(
        _dev_ptr(tiled_q, "tiled_q", (torch.int32, torch.uint32), (qlinear_tiled_words(bits, N, K),)),
        _dev_ptr(tiled_sb, "tiled_sb", (torch.int32, torch.uint32), (qlinear_tiled_sb_words(N, K),)),
        bits, group, N, K,
        _dev_ptr(packed_q, "packed_q", (torch.int32, torch.uint32), (N, K * bits // 32)),
        _dev_ptr(scales, "scales", u16, (N, K // group)),
        _dev_ptr(biases, "biases", u16, (N, K // group)), _stream_handle(stream))
    _check(st, "qlinear_unrepack_glu")


def qlinear_unrepack(tiled_q, tiled_sb, bits, group, N, K, packed_q, scales, biases, stream=None):
    """C ``qlinear_unrepack``: tiled -> canonical into the given tensors."""
    torch = _torch()
    u16 = _u16(torch)
    lib = load_library()
    st = lib.qlinear_unrepack(
        _dev_ptr(tiled_q, "tiled_q", (torch.int32, torch.uint32), (qlinear_tiled_words(bits, N, K),)),
        _dev_ptr(tiled_sb, "tiled_sb", (torch.int32, torch.uint32), (qlinear_tiled_sb_words(N, K),)),
        bits, group, N, K,
        _dev_ptr(packed_q, "packed_q", (torch.int32, torch.uint32), (N, K * bits // 32)),
        _dev_ptr(scales, "scales", u16, (N, K // group)),
        _dev_ptr(biases, "biases", u16, (N, K // group)),
        _stream_handle(stream))
    _check(st, "qlinear_unrepack")


def qlinear_quantize_rtn(w, bits, group, N, K, packed_q, scales, biases, status=None, stream=None):
    """C ``qlinear_quantize_rtn``: device load-time RTN fit + pack."""
    torch = _torch()
    u16 = _u16(torch)
    lib = load_library()
    st = lib.qlinear_quantize_rtn(
        _dev_ptr(w, "w", (torch.float32,), (N, K)), bits, group, N, K,
        _dev_ptr(packed_q, "packed_q", (torch.int32, torch.uint32), (N, K * bits // 32)),
        _dev_ptr(scales, "scales", u16, (N, K // group)),
        _dev_ptr(biases, "biases", u16, (N, K // group)),
        _dev_ptr(status, "status", (torch.int32,)) if status is not None else None,
        _stream_handle(stream))
    _check(st, "qlinear_quantize_rtn")


def qlinear_quantize_imatrix(w, importance, bits, group, N, K, packed_q, scales, biases, status=None, stream=None):
    """C ``qlinear_quantize_imatrix``: device importance-weighted fit + pack (importance fp32 [K])."""
    torch = _torch()
    u16 = _u16(torch)
    lib = load_library()
    st = lib.qlinear_quantize_imatrix(
        _dev_ptr(w, "w", (torch.float32,), (N, K)),
        _dev_ptr(importance, "importance", (torch.float32,), (K,)), bits, group, N, K,
        _dev_ptr(packed_q, "packed_q", (torch.int32, torch.uint32), (N, K * bits // 32)),
        _dev_ptr(scales, "scales", u16, (N, K // group)),
        _dev_ptr(biases, "biases", u16, (N, K // group)),
        _dev_ptr(status, "status", (torch.int32,)) if status is not None else None,
        _stream_handle(stream))
    _check(st, "qlinear_quantize_imatrix")


def qlinear_dequantize(packed_q, scales, biases, bits, group, N, K, w_out, stream=None):
    """C ``qlinear_dequantize``: W_hat fp32 [N, K]."""
    torch = _torch()
    u16 = _u16(torch)
    lib = load_library()
    st = lib.qlinear_dequantize(
        _dev_ptr(packed_q, "packed_q", (torch.int32, torch.uint32), (N, K * bits // 32)),
        _dev_ptr(scales, "scales", u16, (N, K // group)),
        _dev_ptr(biases, "biases", u16, (N, K // group)),
        bits, group, N, K,
        _dev_ptr(w_out, "w_out", (torch.float32,), (N, K)),
        _stream_handle(stream))
    _check(st, "qlinear_dequantize")
    return w_out


# ------------------------------------------------------------------ host entry points

def qlinear_packed_words(bits, N, K) -> int:
    return int(load_library().qlinear_packed_words(bits, N, K))


def qlinear_workspace_bytes(bits, M, N, K) -> int:
    return int(load_library().qlinear_workspace_bytes(bits, M, N, K))


def qlinear_pack_host(q: np.ndarray, bits: int) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint8)
    n, k = q.shape
    out = np.empty((n, k * bits // 32), dtype=np.uint32)
    _check(load_library().qlinear_pack_host(q.ctypes.data, bits, n, k, out.ctypes.data), "qlinear_pack_host")
    return out


def qlinear_unpack_host(packed: np.ndarray, bits: int, K: int) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint32)
    n = packed.shape[0]
    out = np.empty((n, K), dtype=np.uint8)
    _check(load_library().qlinear_unpack_host(packed.ctypes.data, bits, n, K, out.ctypes.data),
           "qlinear_unpack_host")
    return out


def qlinear_quantize_rtn_host(w: np.ndarray, bits: int, group: int = 64):
    w = np.ascontiguousarray(w, dtype=np.float32)
    n, k = w.shape
    q = np.empty((n, k), dtype=np.uint8)
    g = k // group if group else 0
    s = np.empty((n, g), dtype=np.uint16)
    b = np.empty((n, g), dtype=np.uint16)
    _check(load_library().qlinear_quantize_rtn_host(w.ctypes.data, bits, group, n, k, q.ctypes.data,
                                                    s.ctypes.data, b.ctypes.data), "qlinear_quantize_rtn_host")
    return q, s, b


def qlinear_status_string(status: int) -> str:
    return load_library().qlinear_status_string(status).decode()


def qlinear_last_path() -> str:
    buf = ctypes.create_string_buffer(160)
    _check(load_library().qlinear_last_path(buf, 160), "qlinear_last_path")
    return buf.value.decode()


def qlinear_version() -> int:
    return int(load_library().qlinear_version())
