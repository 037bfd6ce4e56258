"""Python binding of libqmv (the MI355X quantized matrix-vector product).

Argument marshalling only: every function here checks tensor placement and
contiguity, takes device pointers and the current HIP stream from PyTorch, and
calls the C ABI of include/qmv.h with the same name. All computation runs in
the library's HIP kernels (or, for the host codecs, in its C++ code). There is
no fallback: if libqmv.so is not built, every call raises.

Weight tensors are uint8. x / y / affine scales and biases are torch.float32,
torch.float16 or torch.bfloat16 and share one dtype.
"""

from __future__ import annotations

import ctypes
import os
import re

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libqmv.so")
HEADER_PATH = os.path.join(os.path.dirname(PKG_DIR), "include", "qmv.h")

QMV_F32, QMV_F16, QMV_BF16 = 0, 1, 2
QMV_AFFINE, QMV_MXFP4, QMV_NVFP4, QMV_MXFP8 = 0, 1, 2, 3
QMV_SB_E8M0, QMV_SB_F32, QMV_SB_F16 = 4, 5, 6
QMV_EL_E2M1, QMV_EL_E4M3, QMV_EL_E5M2, QMV_EL_INT = 1, 2, 3, 10
FORMATS = {"affine": QMV_AFFINE, "mxfp4": QMV_MXFP4, "nvfp4": QMV_NVFP4, "mxfp8": QMV_MXFP8}

# The symmetric block-scaled formats by their names in the Track-1 table:
# name -> (format family, element code, block), as include/qmv.h lists them.
BLOCK_FORMATS = {
    "mxfp8_e5m2": (QMV_SB_E8M0, QMV_EL_E5M2, 32),
    "nvfp8": (QMV_SB_F32, QMV_EL_E4M3, 16),
    "fp4": (QMV_SB_F32, QMV_EL_E2M1, 32),
    "fp8_e4m3": (QMV_SB_F32, QMV_EL_E4M3, 32),
    "fp8_e5m2": (QMV_SB_F32, QMV_EL_E5M2, 32),
    "nvfp8_f16": (QMV_SB_F16, QMV_EL_E4M3, 16),
    "fp4_f16": (QMV_SB_F16, QMV_EL_E2M1, 32),
    "fp8_e4m3_f16": (QMV_SB_F16, QMV_EL_E4M3, 32),
    "fp8_e5m2_f16": (QMV_SB_F16, QMV_EL_E5M2, 32),
}
for _n in (2, 3, 4, 5, 6, 8):
    BLOCK_FORMATS[f"int{_n}"] = (QMV_SB_F32, QMV_EL_INT + _n, 64)
    BLOCK_FORMATS[f"int{_n}_f16"] = (QMV_SB_F16, QMV_EL_INT + _n, 64)
    BLOCK_FORMATS[f"mxint{_n}"] = (QMV_SB_E8M0, QMV_EL_INT + _n, 32)


def block_format_bits(name: str) -> int:
    """Code width of a block-scaled format's element."""
    el = BLOCK_FORMATS[name][1]
    return 4 if el == QMV_EL_E2M1 else (8 if el <= QMV_EL_E5M2 else el - QMV_EL_INT)
STATUS = {0: "QMV_OK", 1: "QMV_ERR_INVALID_ARGUMENT", 2: "QMV_ERR_UNSUPPORTED",
          3: "QMV_ERR_MISALIGNED", 4: "QMV_ERR_HIP"}


class QmvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class QmvWeights(ctypes.Structure):
    """Mirror of qmv_weights_t."""
    _fields_ = [
        ("format", ctypes.c_int), ("bits", ctypes.c_int), ("group_size", ctypes.c_int),
        ("n_experts", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
        ("w", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("biases", ctypes.c_void_p),
        ("global_scale", ctypes.c_void_p),
    ]


_lib = None


def library_path() -> str:
    return LIB_PATH


def load() -> ctypes.CDLL:
    """Load libqmv.so (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"libqmv.so is not built ({LIB_PATH}); run `python -m bit_matrix_vector_amd.build`")
    # torch first: its HIP runtime is then the one the library binds to, so
    # the streams and device pointers torch hands over belong to the runtime
    # the library calls (loading the library first would bind it to the
    # system runtime and leave two in the process)
    _torch()
    lib = ctypes.CDLL(LIB_PATH)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    sig = {
        "qmv_affine": [vp, i32, i64, i64, i64, vp, vp, vp, vp, i32, i32, vp],
        "qmv_fp_mxfp4": [vp, i32, i64, i64, i64, vp, vp, vp, vp],
        "qmv_fp_nvfp4": [vp, i32, i64, i64, i64, vp, vp, vp, vp, vp],
        "qmv_fp_mxfp8": [vp, i32, i64, i64, i64, vp, vp, vp, vp],
        "qmv_fp_block": [vp, i32, i32, i32, i32, i64, i64, i64, vp, vp, vp, vp],
        "gather_qmv": [vp, i32, ctypes.POINTER(QmvWeights), vp, i64, vp, vp, i64, vp],
        "qmv_pack_codes": [vp, i64, i64, i32, vp],
        "qmv_unpack_codes": [vp, i64, i64, i32, vp],
        "qmv_encode_e4m3": [vp, i64, vp],
        "qmv_unpack_codes_device": [vp, vp, i64, i64, i32, vp],
        "qmv_dequant_device": [vp, i32, ctypes.POINTER(QmvWeights), vp],
        "qmv_moe_gate_up_swiglu": [vp, i32, ctypes.POINTER(QmvWeights),
                                   ctypes.POINTER(QmvWeights), vp, i64, vp, i64, ctypes.c_float,
                                   vp],
        "qmv_moe_down_reduce": [vp, i32, ctypes.POINTER(QmvWeights), vp, i64, vp, vp, i64, vp],
        "qmv_qvm": [vp, i32, ctypes.POINTER(QmvWeights), i64, vp, vp, vp, ctypes.c_size_t],
        "qmv_qvm_noalloc": [vp, i32, ctypes.POINTER(QmvWeights), i64, vp, vp],
        "qmv_qmm": [vp, i32, ctypes.POINTER(QmvWeights), i64, vp, vp, vp, ctypes.c_size_t],
        "qmv_rmsnorm_qmv": [vp, i32, ctypes.POINTER(QmvWeights), i64, vp, vp, ctypes.c_float, vp],
        "gather_qmm": [vp, i32, ctypes.POINTER(QmvWeights), vp, i64, vp, vp, i64, vp],
        "qmv_quantize_affine": [vp, i32, i64, i64, vp, i32, i32, vp, vp, vp],
        "qmv_quantize_mxfp4": [vp, i32, i64, i64, vp, vp, vp],
        "qmv_quantize_mxfp8": [vp, i32, i64, i64, vp, vp, vp],
        "qmv_quantize_nvfp4": [vp, i32, i64, i64, vp, vp, vp, vp],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.qmv_qvm_workspace_bytes.argtypes = [i64, i64, i64]
    lib.qmv_qvm_workspace_bytes.restype = ctypes.c_size_t
    lib.qmv_qvm_noalloc_max_workspace_bytes.argtypes = []
    lib.qmv_qvm_noalloc_max_workspace_bytes.restype = ctypes.c_size_t
    lib.qmv_qmm_workspace_bytes.argtypes = [i64, i64, i64, i32]
    lib.qmv_qmm_workspace_bytes.restype = ctypes.c_size_t
    lib.qmv_packed_row_bytes.argtypes = [i32, i32, i64]
    lib.qmv_packed_row_bytes.restype = i64
    lib.qmv_bench_stream_read.argtypes = [vp, vp, i64, vp, i32]
    lib.qmv_bench_stream_read.restype = ctypes.c_int
    lib.qmv_bench_read_design.argtypes = [vp, vp, i64, vp, i32]
    lib.qmv_bench_read_design.restype = ctypes.c_int
    lib.qmv_bench_copy.argtypes = [vp, vp, vp, i64]
    lib.qmv_bench_copy.restype = ctypes.c_int
    lib.qmv_last_error.argtypes = []
    lib.qmv_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def header_functions() -> list[str]:
    """Names of the functions the headers in include/ declare."""
    inc = os.path.dirname(HEADER_PATH)
    names = set()
    for fn in sorted(os.listdir(inc)):
        if fn.endswith(".h"):
            text = open(os.path.join(inc, fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names.update(re.findall(r"\b(qmv_\w+|gather_qm[vm])\s*\(", text))
    return sorted(names)


def _check(status: int) -> None:
    if status != 0:
        msg = load().qmv_last_error().decode(errors="replace")
        raise QmvError(status, msg)


# ---------------------------------------------------------------------------
# torch marshalling
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    m = {torch.float32: QMV_F32, torch.float16: QMV_F16, torch.bfloat16: QMV_BF16}
    if t.dtype not in m:
        raise TypeError(f"activation dtype must be float32/float16/bfloat16, got {t.dtype}")
    return m[t.dtype]


def _dev(t, name: str, dtype=None):
    torch = _torch()
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _ptr(t):
    return None if t is None or t.numel() == 0 else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _xy(x, N, y):
    torch = _torch()
    x = _dev(x, "x")
    if x.dim() == 1:
        x = x.unsqueeze(0)
    if x.dim() != 2:
        raise ValueError("x must be [B, K]")
    B = x.shape[0]
    if y is None:
        y = torch.empty((B, N), dtype=x.dtype, device=x.device)
    _dev(y, "y", x.dtype)
    if tuple(y.shape) != (B, N):
        raise ValueError(f"y must be [{B}, {N}]")
    return x, y


def qmv_affine(x, w, scales, biases, bits: int, group_size: int, y=None):
    """y[B, N] = x[B, K] . dequant(W)^T for affine codes (see include/qmv.h)."""
    torch = _torch()
    _dev(w, "w", torch.uint8)
    N = w.shape[0]
    x, y = _xy(x, N, y)
    _dev(scales, "scales", x.dtype)
    _dev(biases, "biases", x.dtype)
    _check(load().qmv_affine(_stream(x.device), _dtype_code(x), x.shape[0], x.shape[1], N,
                             _ptr(x), _ptr(w), _ptr(scales), _ptr(biases), bits, group_size,
                             _ptr(y)))
    return y


def qmv_fp_mxfp4(x, w, scales, y=None):
    torch = _torch()
    _dev(w, "w", torch.uint8)
    _dev(scales, "scales", torch.uint8)
    x, y = _xy(x, w.shape[0], y)
    _check(load().qmv_fp_mxfp4(_stream(x.device), _dtype_code(x), x.shape[0], x.shape[1],
                               w.shape[0], _ptr(x), _ptr(w), _ptr(scales), _ptr(y)))
    return y


def qmv_fp_nvfp4(x, w, scales, global_scale=None, y=None):
    """global_scale: a one-element float32 GPU tensor, or None for 1.0."""
    torch = _torch()
    _dev(w, "w", torch.uint8)
    _dev(scales, "scales", torch.uint8)
    _dev(global_scale, "global_scale", torch.float32)
    x, y = _xy(x, w.shape[0], y)
    _check(load().qmv_fp_nvfp4(_stream(x.device), _dtype_code(x), x.shape[0], x.shape[1],
                               w.shape[0], _ptr(x), _ptr(w), _ptr(scales), _ptr(global_scale),
                               _ptr(y)))
    return y


def qmv_fp_mxfp8(x, w, scales, y=None):
    torch = _torch()
    _dev(w, "w", torch.uint8)
    _dev(scales, "scales", torch.uint8)
    x, y = _xy(x, w.shape[0], y)
    _check(load().qmv_fp_mxfp8(_stream(x.device), _dtype_code(x), x.shape[0], x.shape[1],
                               w.shape[0], _ptr(x), _ptr(w), _ptr(scales), _ptr(y)))
    return y


def qmv_fp_block(x, w, scales, fmt: str, y=None):
    """y[B, N] = x . dequant(W)^T for a symmetric block-scaled format named in
    BLOCK_FORMATS; scales are uint8 (E8M0), float32 or float16 by family."""
    torch = _torch()
    code, el, block = BLOCK_FORMATS[fmt]
    _dev(w, "w", torch.uint8)
    want = {QMV_SB_E8M0: torch.uint8, QMV_SB_F32: torch.float32, QMV_SB_F16: torch.float16}[code]
    _dev(scales, "scales", want)
    x, y = _xy(x, w.shape[0], y)
    _check(load().qmv_fp_block(_stream(x.device), _dtype_code(x), code, el, block, x.shape[0],
                               x.shape[1], w.shape[0], _ptr(x), _ptr(w), _ptr(scales), _ptr(y)))
    return y


def make_weights(fmt: str, w, scales, biases=None, *, K: int, bits: int = 4,
                 group_size: int = 32, global_scale=None) -> QmvWeights:
    """qmv_weights_t for expert-stacked (or single, 2-D) weights. The tensors
    must stay alive while the struct is in use. A block-scaled format name
    (BLOCK_FORMATS) fixes the format, element and block itself."""
    torch = _torch()
    _dev(w, "w", torch.uint8)
    n_exp = 1 if w.dim() == 2 else w.shape[0]
    N = w.shape[-2]
    if fmt in BLOCK_FORMATS:
        code, bits, group_size = BLOCK_FORMATS[fmt]
    else:
        code = FORMATS[fmt]
    return QmvWeights(code, bits, group_size, n_exp, N, K,
                      w.data_ptr() if w.numel() else None,
                      scales.data_ptr() if scales is not None and scales.numel() else None,
                      biases.data_ptr() if biases is not None and biases.numel() else None,
                      global_scale.data_ptr() if global_scale is not None else None)


def gather_qmv(x, weights: QmvWeights, lhs_indices, rhs_indices, y=None):
    """y[s] = W[rhs[s]] . x[lhs[s]] (indices: uint32 stored in int32 tensors)."""
    torch = _torch()
    x = _dev(x, "x")
    _dev(lhs_indices, "lhs_indices", torch.int32)
    _dev(rhs_indices, "rhs_indices", torch.int32)
    n_slots = lhs_indices.numel()
    if rhs_indices.numel() != n_slots:
        raise ValueError("lhs_indices and rhs_indices differ in length")
    N = weights.N
    if y is None:
        y = torch.empty((n_slots, N), dtype=x.dtype, device=x.device)
    _dev(y, "y", x.dtype)
    _check(load().gather_qmv(_stream(x.device), _dtype_code(x), ctypes.byref(weights), _ptr(x),
                             x.shape[0], _ptr(lhs_indices), _ptr(rhs_indices), n_slots,
                             _ptr(y)))
    return y


def gather_qmm(x, weights: QmvWeights, lhs_indices, rhs_indices, y=None):
    """y[s] = W[rhs[s]] . x[lhs[s]] for many slots on the matrix cores (bf16 or
    f16; indices: uint32 stored in int32 tensors; sorted rhs is fastest)."""
    torch = _torch()
    x = _dev(x, "x")
    _dev(lhs_indices, "lhs_indices", torch.int32)
    _dev(rhs_indices, "rhs_indices", torch.int32)
    n_slots = lhs_indices.numel()
    if rhs_indices.numel() != n_slots:
        raise ValueError("lhs_indices and rhs_indices differ in length")
    if y is None:
        y = torch.empty((n_slots, weights.N), dtype=x.dtype, device=x.device)
    _dev(y, "y", x.dtype)
    _check(load().gather_qmm(_stream(x.device), _dtype_code(x), ctypes.byref(weights), _ptr(x),
                             x.shape[0], _ptr(lhs_indices), _ptr(rhs_indices), n_slots, _ptr(y)))
    return y


def qmv_unpack_codes_device(packed, K: int, bits: int, codes=None):
    torch = _torch()
    _dev(packed, "packed", torch.uint8)
    rows = packed.shape[0]
    if codes is None:
        codes = torch.empty((rows, K), dtype=torch.uint8, device=packed.device)
    _dev(codes, "codes", torch.uint8)
    _check(load().qmv_unpack_codes_device(_stream(packed.device), _ptr(packed), rows, K, bits,
                                          _ptr(codes)))
    return codes


def qmv_dequant_device(weights: QmvWeights, dtype_code: int, device, out=None):
    torch = _torch()
    if out is None:
        out = torch.empty((weights.N, weights.K), dtype=torch.float32, device=device)
    _dev(out, "out", torch.float32)
    _check(load().qmv_dequant_device(_stream(out.device), dtype_code, ctypes.byref(weights),
                                     _ptr(out)))
    return out


# ---------------------------------------------------------------------------
# qvm
# ---------------------------------------------------------------------------

def qmv_qvm(x, weights: QmvWeights, y=None, workspace=None):
    """y[B, K] = x[B, N] . dequant(W)[N, K] (W one [N, K] matrix). The fp32
    workspace is allocated here unless given (see qmv_qvm_workspace_bytes)."""
    torch = _torch()
    x = _dev(x, "x")
    if x.dim() == 1:
        x = x.unsqueeze(0)
    B = x.shape[0]
    if y is None:
        y = torch.empty((B, weights.K), dtype=x.dtype, device=x.device)
    _dev(y, "y", x.dtype)
    need = int(load().qmv_qvm_workspace_bytes(B, weights.K, weights.N))
    if workspace is None:
        workspace = torch.empty((max(need, 4) // 4,), dtype=torch.float32, device=x.device)
    _check(load().qmv_qvm(_stream(x.device), _dtype_code(x), ctypes.byref(weights), B, _ptr(x),
                          _ptr(y), _ptr(workspace), workspace.numel() * 4))
    return y


def qmv_qvm_noalloc(x, weights: QmvWeights, y):
    """qmv_qvm through the entry point that allocates nothing: the split
    partials go to the library's device scratch (qmv_qvm_noalloc in qmv.h);
    y [B, K] must be given."""
    x = _dev(x, "x")
    if x.dim() == 1:
        x = x.unsqueeze(0)
    _dev(y, "y", x.dtype)
    _check(load().qmv_qvm_noalloc(_stream(x.device), _dtype_code(x), ctypes.byref(weights),
                                  x.shape[0], _ptr(x), _ptr(y)))
    return y


def qmv_rmsnorm_qmv(x, weights: QmvWeights, gamma, eps: float, y=None):
    """y[B, N] = W . RN_T(rmsnorm(x) * gamma), one fused dispatch."""
    torch = _torch()
    x = _dev(x, "x")
    if x.dim() == 1:
        x = x.unsqueeze(0)
    _dev(gamma, "gamma", x.dtype)
    B = x.shape[0]
    if y is None:
        y = torch.empty((B, weights.N), dtype=x.dtype, device=x.device)
    _dev(y, "y", x.dtype)
    _check(load().qmv_rmsnorm_qmv(_stream(x.device), _dtype_code(x), ctypes.byref(weights), B,
                                  _ptr(x), _ptr(gamma), float(eps), _ptr(y)))
    return y


def qmv_qmm(x, weights: QmvWeights, y=None, workspace=None):
    """y[M, N] = x[M, K] . dequant(W)[N, K]^T for any M (bf16 or f16
    activations, matrix cores). The fp32 workspace (qmv_qmm_workspace_bytes,
    often 0) is allocated here unless given."""
    torch = _torch()
    x = _dev(x, "x")
    if x.dim() == 1:
        x = x.unsqueeze(0)
    M = x.shape[0]
    if y is None:
        y = torch.empty((M, weights.N), dtype=x.dtype, device=x.device)
    _dev(y, "y", x.dtype)
    need = int(load().qmv_qmm_workspace_bytes(M, weights.K, weights.N, weights.format))
    if workspace is None and need > 0:
        workspace = torch.empty((need // 4,), dtype=torch.float32, device=x.device)
    ws_ptr = _ptr(workspace) if workspace is not None else None
    ws_bytes = workspace.numel() * 4 if workspace is not None else 0
    _check(load().qmv_qmm(_stream(x.device), _dtype_code(x), ctypes.byref(weights), M, _ptr(x),
                          _ptr(y), ws_ptr, ws_bytes))
    return y


# ---------------------------------------------------------------------------
# fused routed-MoE decode block
# ---------------------------------------------------------------------------

def qmv_moe_gate_up_swiglu(x, gate: QmvWeights, up: QmvWeights, expert_ids, clamp: float = 0.0,
                           mid=None):
    """mid [T * top_k, ffn] = silu(clamp(gate . x)) * clamp(up . x) per routed
    slot; expert_ids: int32 tensor [T, top_k] holding uint32 ids."""
    torch = _torch()
    x = _dev(x, "x")
    _dev(expert_ids, "expert_ids", torch.int32)
    T, k = expert_ids.shape
    if mid is None:
        mid = torch.empty((T * k, gate.N), dtype=x.dtype, device=x.device)
    _dev(mid, "mid", x.dtype)
    _check(load().qmv_moe_gate_up_swiglu(_stream(x.device), _dtype_code(x), ctypes.byref(gate),
                                         ctypes.byref(up), _ptr(x), T, _ptr(expert_ids), k,
                                         float(clamp), _ptr(mid)))
    return mid


def qmv_moe_down_reduce(mid, down: QmvWeights, expert_ids, route_weights, y=None):
    """y [T, hidden] = sum_j route_weights[t, j] * (down[e] . mid[t * top_k + j])."""
    torch = _torch()
    mid = _dev(mid, "mid")
    _dev(expert_ids, "expert_ids", torch.int32)
    _dev(route_weights, "route_weights", torch.float32)
    T, k = expert_ids.shape
    if y is None:
        y = torch.empty((T, down.N), dtype=mid.dtype, device=mid.device)
    _dev(y, "y", mid.dtype)
    _check(load().qmv_moe_down_reduce(_stream(mid.device), _dtype_code(mid), ctypes.byref(down),
                                      _ptr(mid), T, _ptr(expert_ids), _ptr(route_weights), k,
                                      _ptr(y)))
    return y


# ---------------------------------------------------------------------------
# quantize from float (device tensors; outputs allocated here unless given)
# ---------------------------------------------------------------------------

def _qin(w):
    w = _dev(w, "w")
    if w.dim() != 2:
        raise ValueError("w must be [N, K]")
    return w, w.shape[0], w.shape[1]


def qmv_quantize_affine(w, bits: int, group_size: int):
    """Affine codes of w [N, K] (float32/float16/bfloat16): returns (packed
    [N, K*bits/8] uint8, scales [N, K/group_size], biases) with scales and
    biases in w's dtype. See include/qmv.h for the exact rule."""
    torch = _torch()
    w, N, K = _qin(w)
    packed = torch.empty((N, K * bits // 8), dtype=torch.uint8, device=w.device)
    sc = torch.empty((N, K // group_size), dtype=w.dtype, device=w.device)
    bi = torch.empty_like(sc)
    _check(load().qmv_quantize_affine(_stream(w.device), _dtype_code(w), N, K, _ptr(w), bits,
                                      group_size, _ptr(packed), _ptr(sc), _ptr(bi)))
    return packed, sc, bi


def qmv_quantize_mx(w, fmt: str):
    """MXFP4 ('mxfp4') or MXFP8 ('mxfp8') codes of w [N, K]: returns (packed,
    E8M0 scales [N, K/32] uint8)."""
    torch = _torch()
    w, N, K = _qin(w)
    if fmt not in ("mxfp4", "mxfp8"):
        raise ValueError(fmt)
    rb = K // 2 if fmt == "mxfp4" else K
    packed = torch.empty((N, rb), dtype=torch.uint8, device=w.device)
    sc = torch.empty((N, K // 32), dtype=torch.uint8, device=w.device)
    fn = load().qmv_quantize_mxfp4 if fmt == "mxfp4" else load().qmv_quantize_mxfp8
    _check(fn(_stream(w.device), _dtype_code(w), N, K, _ptr(w), _ptr(packed), _ptr(sc)))
    return packed, sc


def qmv_quantize_nvfp4(w):
    """NVFP4 codes of w [N, K]: returns (packed [N, K/2], E4M3 scales [N, K/16]
    uint8, global scale as a one-element float32 tensor)."""
    torch = _torch()
    w, N, K = _qin(w)
    packed = torch.empty((N, K // 2), dtype=torch.uint8, device=w.device)
    sc = torch.empty((N, K // 16), dtype=torch.uint8, device=w.device)
    gs = torch.empty((1,), dtype=torch.float32, device=w.device)
    _check(load().qmv_quantize_nvfp4(_stream(w.device), _dtype_code(w), N, K, _ptr(w),
                                     _ptr(packed), _ptr(sc), _ptr(gs)))
    return packed, sc, gs


# ---------------------------------------------------------------------------
# host codecs (NumPy arrays in host memory)
# ---------------------------------------------------------------------------

def qmv_packed_row_bytes(fmt: str, bits: int, K: int) -> int:
    return int(load().qmv_packed_row_bytes(FORMATS[fmt], bits, K))


def _np_ptr(a):
    return ctypes.c_void_p(a.ctypes.data) if a.size else None


def qmv_pack_codes(codes, bits: int):
    import numpy as np
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    rows, K = codes.shape
    out = np.zeros((rows, K * bits // 8), dtype=np.uint8)
    _check(load().qmv_pack_codes(_np_ptr(codes), rows, K, bits, _np_ptr(out)))
    return out


def qmv_unpack_codes(packed, K: int, bits: int):
    import numpy as np
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    rows = packed.shape[0]
    out = np.zeros((rows, K), dtype=np.uint8)
    _check(load().qmv_unpack_codes(_np_ptr(packed), rows, K, bits, _np_ptr(out)))
    return out


def qmv_encode_e4m3(v):
    import numpy as np
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.zeros(v.shape, dtype=np.uint8)
    _check(load().qmv_encode_e4m3(_np_ptr(v), v.size, _np_ptr(out)))
    return out


__all__ = [
    "qmv_affine", "qmv_fp_mxfp4", "qmv_fp_nvfp4", "qmv_fp_mxfp8", "gather_qmv",
    "make_weights", "qmv_unpack_codes_device", "qmv_dequant_device", "qmv_packed_row_bytes",
    "qmv_pack_codes", "qmv_unpack_codes", "qmv_encode_e4m3", "QmvError", "QmvWeights", "load",
    "header_functions", "library_path",
]
