"""Python binding of libwq.so, the gfx950 W4A16 group-quantized linear.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind include/wq.h.  PyTorch provides device memory and the current
stream.  There is no fallback: if the library is missing, every call raises.

Entry points (the same names as the C ABI, without the ``wq_`` prefix):

* ``quantize_rtn(W, sparse_k)``  split + RTN INT4 group quantization
* ``pack(codes)``                eight codes per 32-bit word
* ``linear(x, packed, scales, zeros)``
* ``linear_sparse(x, packed, scales, zeros, row_ptr, col, val)``
* ``linear_lowrank(x, packed, scales, zeros, L1, L2, row_ptr, col, val)``
  the same plus a rank-r fp16 branch (x . L1^T) . L2^T
* ``quantize_rtn_act_order(W, perm)``, ``linear_act_order(x, perm, ...)``
  act-order layers, kept in the permuted channel order
* ``quantize_act_int8(x, outliers)``, ``linear_w4a8(x, outliers, ...)``
  INT8 activations with fp16 outlier channels on the same INT4 layer
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libwq.so")
GROUP = 128

WQ_OK = 0
STATUS = {0: "WQ_OK", -1: "WQ_ERR_NULL", -2: "WQ_ERR_SHAPE", -3: "WQ_ERR_ALIGN",
          -4: "WQ_ERR_UNSUPPORTED", -5: "WQ_ERR_HIP", -6: "WQ_ERR_WORKSPACE", -7: "WQ_ERR_SCRATCH"}
KERNELS = {"auto": 0, "gemv": 1, "gemm": 2, "gemv_mfma": 3}

# name -> (restype, argtypes) for every symbol declared in include/wq.h
_i64, _i32, _vp, _sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
SIGNATURES = {
    "wq_quantize_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "wq_quantize_rtn": (ctypes.c_int, [_vp, _i64, _i64, _i32, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "wq_quantize_rtn_bits": (ctypes.c_int, [_vp, _i64, _i64, _i32, _i32, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                            _sz, _vp]),
    "wq_pack": (ctypes.c_int, [_vp, _i64, _i64, _vp, _vp]),
    "wq_pack_bits": (ctypes.c_int, [_vp, _i64, _i64, _i32, _vp, _vp]),
    "wq_linear_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "wq_linear": (ctypes.c_int, [_vp, _i64, _i64, _vp, _vp, _vp, _i64, _i32, _vp, _i32, _vp, _sz, _vp]),
    "wq_linear_sparse": (ctypes.c_int, [_vp, _i64, _i64, _vp, _vp, _vp, _i64, _i32, _vp, _vp, _vp, _i64,
                                        _vp, _i32, _vp, _sz, _vp]),
    "wq_linear_sparse_bits": (ctypes.c_int, [_vp, _i64, _i64, _vp, _i32, _vp, _vp, _i64, _i32, _vp, _vp, _vp, _i64,
                                             _vp, _i32, _i32, _vp, _sz, _vp]),
    "wq_linear_sparse_kernel": (ctypes.c_int, [_vp, _i64, _i64, _vp, _vp, _vp, _i64, _i32, _vp, _vp, _vp, _i64,
                                               _vp, _i32, _i32, _vp, _sz, _vp]),
    "wq_linear_lowrank_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64]),
    "wq_linear_lowrank": (ctypes.c_int, [_vp, _i64, _i64, _vp, _vp, _vp, _i64, _i32, _vp, _vp, _vp, _i64,
                                         _vp, _vp, _i64, _vp, _i32, _i32, _vp, _sz, _vp]),
    "wq_quantize_act_order_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "wq_quantize_rtn_act_order": (ctypes.c_int, [_vp, _i64, _i64, _i32, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp,
                                                 _vp, _sz, _vp]),
    "wq_linear_act_order_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "wq_linear_act_order": (ctypes.c_int, [_vp, _i64, _i64, _vp, _vp, _vp, _vp, _i64, _i32, _vp, _vp, _vp, _i64,
                                           _vp, _i32, _i32, _vp, _sz, _vp]),
    "wq_quantize_act_int8": (ctypes.c_int, [_vp, _i64, _i64, _vp, _i64, _vp, _vp, _vp, _vp]),
    "wq_linear_w4a8_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "wq_linear_w4a8": (ctypes.c_int, [_vp, _i64, _i64, _vp, _i64, _vp, _vp, _vp, _i64, _i32, _vp, _i32, _vp, _sz,
                                      _vp]),
    "wq_linear_sparse_noalloc": (ctypes.c_int, [_vp, _i64, _i64, _vp, _vp, _vp, _i64, _i32, _vp, _vp, _vp, _i64,
                                                _vp, _i32, _vp]),
    "wq_auto_kernel": (ctypes.c_int, [_i64, _i64, _i64]),
    "wq_last_hip_error": (ctypes.c_int, []),
    "wq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
}

_lib = None


class WQError(RuntimeError):
    def __init__(self, fn, status, lib):
        msg = lib.wq_status_string(status).decode() if lib is not None else ""
        super().__init__(f"{fn} returned {STATUS.get(status, status)}: {msg}")
        self.status = status


def load():
    """Load libwq.so (built by ``python -m quantized_gemm_rtn_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m quantized_gemm_rtn_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        _lib = lib
    return _lib


def _check(fn, rc):
    if rc != WQ_OK:
        raise WQError(fn, rc, _lib)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _need(t, dtype, name):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def quantize_workspace_bytes(N, K, sparse_k):
    return int(load().wq_quantize_workspace_bytes(N, K, sparse_k))


def quantize_rtn(W, sparse_k: int = 0, group: int = GROUP, workspace=None, bits: int = 4):
    """Dense-and-sparse split and RTN INT4 quantization of ``W`` (float32 [N, K]).

    ``group``: 128, a larger multiple of 128 dividing K, or -1 (one group per
    row); ``bits``: 2 to 4 (codes of fewer bits in the same 4-bit packing). Returns a dict with ``codes`` uint8 [N, K], ``scales``/``zeros``
    float16 [N, K/128] (a coarser group's values repeated in each of its
    128-channel slots), and the sparse part ``row_ptr`` int32 [N+1], ``col``
    int32 [sparse_k], ``val`` float16 [sparse_k]."""
    import torch
    lib = load()
    _need(W, torch.float32, "W")
    N, K = W.shape
    dev = W.device
    # metadata slots per row: one per 64 channels for group 64, else one per 128
    G = K // 64 if group == 64 else K // GROUP
    codes = torch.empty((N, K), dtype=torch.uint8, device=dev)
    scales = torch.empty((N, max(G, 1)), dtype=torch.float16, device=dev)
    zeros = torch.empty((N, max(G, 1)), dtype=torch.float16, device=dev)
    row_ptr = torch.empty(N + 1, dtype=torch.int32, device=dev)
    col = torch.empty(max(sparse_k, 1), dtype=torch.int32, device=dev)
    val = torch.empty(max(sparse_k, 1), dtype=torch.float16, device=dev)
    nbytes = int(lib.wq_quantize_workspace_bytes(N, K, sparse_k))
    if workspace is None and nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    rc = lib.wq_quantize_rtn_bits(_p(W), N, K, group, bits, sparse_k, _p(codes), _p(scales), _p(zeros),
                                  _p(row_ptr), _p(col), _p(val), _p(workspace),
                                  nbytes if workspace is not None else 0, _stream(W))
    _check("wq_quantize_rtn_bits", rc)
    return dict(codes=codes, scales=scales[:, :G], zeros=zeros[:, :G], row_ptr=row_ptr,
                col=col[:sparse_k], val=val[:sparse_k])


def pack(codes, bits: int = 4):
    """Eight INT4 codes per 32-bit word, or (bits = 3) 32 3-bit codes per three
    words (returned as int32 bit patterns, [N, K/8] or [N, 3K/32])."""
    import torch
    lib = load()
    _need(codes, torch.uint8, "codes")
    N, K = codes.shape
    width = K // 8 if bits == 4 else 3 * K // 32
    packed = torch.empty((N, width), dtype=torch.int32, device=codes.device)
    _check("wq_pack_bits", lib.wq_pack_bits(_p(codes), N, K, bits, _p(packed), _stream(codes)))
    return packed


def _layer_format(packed, scales, K, N):
    """(bits, group) of a layer from its tensors' shapes: [N, K/8] words are 4-bit
    codes and [N, 3K/32] 3-bit ones; [N, K/128] metadata is group 128, [N, K/64]
    group 64."""
    if packed.shape[0] != N:
        raise ValueError("inconsistent shapes")
    if packed.shape[1] * 8 == K:
        bits = 4
    elif K % 32 == 0 and packed.shape[1] == 3 * K // 32:
        bits = 3
    else:
        raise ValueError("packed must be [N, K/8] (4-bit) or [N, 3K/32] (3-bit)")
    if tuple(scales.shape) == (N, K // GROUP):
        group = GROUP
    elif tuple(scales.shape) == (N, K // 64):
        group = 64
    else:
        raise ValueError("scales must be [N, K/128] or [N, K/64]")
    return bits, group


def linear_workspace_bytes(M, N, K):
    return int(load().wq_linear_workspace_bytes(M, N, K))


def linear_sparse(x, packed, scales, zeros, row_ptr=None, col=None, val=None, out_dtype=None,
                  kernel: str = "auto", out=None, workspace=None):
    """y = x . dequant(packed, scales, zeros)^T (+ W_sparse x when CSR is given).

    The layer's format follows from the shapes: 4-bit ([N, K/8] words) or 3-bit
    ([N, 3K/32]) codes, one (s, z) per 128 ([N, K/128]) or 64 ([N, K/64]) input
    channels. ``workspace`` (uint8 device tensor of ``linear_workspace_bytes``
    bytes) lets the GEMM split K; when omitted, one is allocated per call."""
    import torch
    lib = load()
    out_dtype = torch.float16 if out_dtype is None else out_dtype
    _need(x, torch.float16, "x")
    _need(packed, torch.int32, "packed")
    _need(scales, torch.float16, "scales")
    _need(zeros, torch.float16, "zeros")
    M, K = x.shape
    N = packed.shape[0]
    bits, group = _layer_format(packed, scales, K, N)
    if zeros.shape != scales.shape:
        raise ValueError("inconsistent shapes")
    nnz = 0
    if row_ptr is not None:
        _need(row_ptr, torch.int32, "row_ptr")
        if row_ptr.numel() != N + 1:
            raise ValueError("row_ptr must have N+1 entries")
        nnz = int(col.numel()) if col is not None else 0
        if nnz:
            _need(col, torch.int32, "col")
            _need(val, torch.float16, "val")
    if out_dtype not in (torch.float16, torch.float32):
        raise TypeError("out_dtype must be float16 or float32")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=x.device)
    else:
        _need(out, out_dtype, "out")
    y_dtype = 1 if out_dtype == torch.float32 else 0
    if workspace is None:
        nbytes = int(lib.wq_linear_workspace_bytes(M, N, K))
        if nbytes:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=x.device)
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib.wq_linear_sparse_bits(_p(x), M, K, _p(packed), bits, _p(scales), _p(zeros), N, group,
                                   _p(row_ptr), _p(col) if nnz else None, _p(val) if nnz else None, nnz,
                                   _p(out), y_dtype, KERNELS[kernel], _p(workspace), wbytes, _stream(x))
    _check("wq_linear_sparse_bits", rc)
    return out


def linear_sparse_noalloc(x, packed, scales, zeros, out, row_ptr=None, col=None, val=None, group: int = GROUP):
    """``linear_sparse`` through ``wq_linear_sparse_noalloc``: no workspace, the
    library's per-GPU scratch instead; ``out`` (float16 or float32 [M, N]) must be
    given, so the call allocates nothing."""
    import torch
    lib = load()
    _need(x, torch.float16, "x")
    _need(packed, torch.int32, "packed")
    _need(scales, torch.float16, "scales")
    _need(zeros, torch.float16, "zeros")
    M, K = x.shape
    N = packed.shape[0]
    if packed.shape[1] * 8 != K or scales.shape != (N, K // group) or zeros.shape != scales.shape:
        raise ValueError("inconsistent shapes")
    if out.dtype not in (torch.float16, torch.float32):
        raise TypeError("out must be float16 or float32")
    _need(out, out.dtype, "out")
    if tuple(out.shape) != (M, N):
        raise ValueError("out must be [M, N]")
    nnz = 0
    if row_ptr is not None:
        _need(row_ptr, torch.int32, "row_ptr")
        if row_ptr.numel() != N + 1:
            raise ValueError("row_ptr must have N+1 entries")
        nnz = int(col.numel()) if col is not None else 0
        if nnz:
            _need(col, torch.int32, "col")
            _need(val, torch.float16, "val")
    rc = lib.wq_linear_sparse_noalloc(_p(x), M, K, _p(packed), _p(scales), _p(zeros), N, group, _p(row_ptr),
                                      _p(col) if nnz else None, _p(val) if nnz else None, nnz, _p(out),
                                      1 if out.dtype == torch.float32 else 0, _stream(x))
    _check("wq_linear_sparse_noalloc", rc)
    return out


def last_hip_error() -> int:
    """hipError_t of this thread's last launch that failed inside the library (0 if none)."""
    return int(load().wq_last_hip_error())


def linear(x, packed, scales, zeros, out_dtype=None, kernel: str = "auto", out=None, workspace=None):
    return linear_sparse(x, packed, scales, zeros, None, None, None, out_dtype, kernel, out, workspace)


def linear_lowrank_workspace_bytes(M, N, K, r):
    return int(load().wq_linear_lowrank_workspace_bytes(M, N, K, r))


def linear_lowrank(x, packed, scales, zeros, L1, L2, row_ptr=None, col=None, val=None, out_dtype=None,
                   kernel: str = "auto", out=None, group: int = GROUP, workspace=None):
    """y = x . dequant(packed, scales, zeros)^T (+ W_sparse x when CSR is given)
    + (x . L1^T) . L2^T, with L1 [r, K] and L2 [N, r] fp16 (r a multiple of 32).

    ``workspace`` (uint8 device tensor of ``linear_lowrank_workspace_bytes``
    bytes) is allocated per call when omitted."""
    import torch
    lib = load()
    out_dtype = torch.float16 if out_dtype is None else out_dtype
    _need(x, torch.float16, "x")
    _need(packed, torch.int32, "packed")
    _need(scales, torch.float16, "scales")
    _need(zeros, torch.float16, "zeros")
    _need(L1, torch.float16, "L1")
    _need(L2, torch.float16, "L2")
    M, K = x.shape
    N = packed.shape[0]
    r = L1.shape[0]
    if packed.shape[1] * 8 != K or scales.shape != (N, K // group) or zeros.shape != scales.shape:
        raise ValueError("inconsistent shapes")
    if L1.shape != (r, K) or L2.shape != (N, r):
        raise ValueError("L1 must be [r, K] and L2 [N, r]")
    nnz = 0
    if row_ptr is not None:
        _need(row_ptr, torch.int32, "row_ptr")
        if row_ptr.numel() != N + 1:
            raise ValueError("row_ptr must have N+1 entries")
        nnz = int(col.numel()) if col is not None else 0
        if nnz:
            _need(col, torch.int32, "col")
            _need(val, torch.float16, "val")
    if out_dtype not in (torch.float16, torch.float32):
        raise TypeError("out_dtype must be float16 or float32")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=x.device)
    else:
        _need(out, out_dtype, "out")
    y_dtype = 1 if out_dtype == torch.float32 else 0
    if workspace is None:
        nbytes = int(lib.wq_linear_lowrank_workspace_bytes(max(M, 1), N, K, r))
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    wbytes = workspace.numel() * workspace.element_size()
    rc = lib.wq_linear_lowrank(_p(x), M, K, _p(packed), _p(scales), _p(zeros), N, group,
                               _p(row_ptr) if nnz else None, _p(col) if nnz else None, _p(val) if nnz else None,
                               nnz, _p(L1), _p(L2), r, _p(out), y_dtype, KERNELS[kernel], _p(workspace), wbytes,
                               _stream(x))
    _check("wq_linear_lowrank", rc)
    return out


def quantize_rtn_act_order(W, perm, sparse_k: int = 0, group: int = GROUP, workspace=None):
    """``quantize_rtn`` of ``W[:, perm]`` (``perm`` int32 [K], a permutation): the
    layer of an act-order quantization, kept in the permuted channel order (its
    CSR columns are positions in that order). Same return value as
    ``quantize_rtn``."""
    import torch
    lib = load()
    _need(W, torch.float32, "W")
    _need(perm, torch.int32, "perm")
    N, K = W.shape
    if perm.numel() != K:
        raise ValueError("perm must have K entries")
    dev = W.device
    G = K // GROUP
    codes = torch.empty((N, K), dtype=torch.uint8, device=dev)
    scales = torch.empty((N, max(G, 1)), dtype=torch.float16, device=dev)
    zeros = torch.empty((N, max(G, 1)), dtype=torch.float16, device=dev)
    row_ptr = torch.empty(N + 1, dtype=torch.int32, device=dev)
    col = torch.empty(max(sparse_k, 1), dtype=torch.int32, device=dev)
    val = torch.empty(max(sparse_k, 1), dtype=torch.float16, device=dev)
    nbytes = int(lib.wq_quantize_act_order_workspace_bytes(N, K, sparse_k))
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    wbytes = workspace.numel() * workspace.element_size()
    rc = lib.wq_quantize_rtn_act_order(_p(W), N, K, group, _p(perm), sparse_k, _p(codes), _p(scales), _p(zeros),
                                       _p(row_ptr), _p(col), _p(val), _p(workspace), wbytes, _stream(W))
    _check("wq_quantize_rtn_act_order", rc)
    return dict(codes=codes, scales=scales[:, :G], zeros=zeros[:, :G], row_ptr=row_ptr,
                col=col[:sparse_k], val=val[:sparse_k])


def linear_act_order_workspace_bytes(M, N, K):
    return int(load().wq_linear_act_order_workspace_bytes(M, N, K))


def linear_act_order(x, perm, packed, scales, zeros, row_ptr=None, col=None, val=None, out_dtype=None,
                     kernel: str = "auto", out=None, group: int = GROUP, workspace=None):
    """y = x . W^T for a layer kept in permuted channel order (``perm`` int32
    [K]; from ``quantize_rtn_act_order``): x, in the original order, has its
    columns gathered through ``perm`` and then meets the layer as in
    ``linear_sparse``."""
    import torch
    lib = load()
    out_dtype = torch.float16 if out_dtype is None else out_dtype
    _need(x, torch.float16, "x")
    _need(perm, torch.int32, "perm")
    _need(packed, torch.int32, "packed")
    _need(scales, torch.float16, "scales")
    _need(zeros, torch.float16, "zeros")
    M, K = x.shape
    N = packed.shape[0]
    if perm.numel() != K or packed.shape[1] * 8 != K or scales.shape != (N, K // group) or \
            zeros.shape != scales.shape:
        raise ValueError("inconsistent shapes")
    nnz = 0
    if row_ptr is not None:
        _need(row_ptr, torch.int32, "row_ptr")
        if row_ptr.numel() != N + 1:
            raise ValueError("row_ptr must have N+1 entries")
        nnz = int(col.numel()) if col is not None else 0
        if nnz:
            _need(col, torch.int32, "col")
            _need(val, torch.float16, "val")
    if out_dtype not in (torch.float16, torch.float32):
        raise TypeError("out_dtype must be float16 or float32")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=x.device)
    else:
        _need(out, out_dtype, "out")
    y_dtype = 1 if out_dtype == torch.float32 else 0
    if workspace is None:
        nbytes = int(lib.wq_linear_act_order_workspace_bytes(max(M, 1), N, K))
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    wbytes = workspace.numel() * workspace.element_size()
    rc = lib.wq_linear_act_order(_p(x), M, K, _p(perm), _p(packed), _p(scales), _p(zeros), N, group,
                                 _p(row_ptr) if row_ptr is not None else None, _p(col) if nnz else None,
                                 _p(val) if nnz else None, nnz, _p(out), y_dtype, KERNELS[kernel], _p(workspace),
                                 wbytes, _stream(x))
    _check("wq_linear_act_order", rc)
    return out


def quantize_act_int8(x, outliers):
    """Per-row INT8 activations with fp16 outlier channels (``outliers`` int32
    [n_out], n_out <= 16): returns ``xq`` int8 [M, K] in the products' byte order,
    ``sx`` float32 [M] and ``xo`` float16 [M, 16]."""
    import torch
    lib = load()
    _need(x, torch.float16, "x")
    _need(outliers, torch.int32, "outliers")
    M, K = x.shape
    xq = torch.empty((M, K), dtype=torch.int8, device=x.device)
    sx = torch.empty(max(M, 1), dtype=torch.float32, device=x.device)
    xo = torch.empty((max(M, 1), 16), dtype=torch.float16, device=x.device)
    n_out = outliers.numel()
    _check("wq_quantize_act_int8", lib.wq_quantize_act_int8(_p(x), M, K, _p(outliers) if n_out else None, n_out,
                                                            _p(xq), _p(sx), _p(xo), _stream(x)))
    return xq, sx[:M], xo[:M]


def linear_w4a8_workspace_bytes(M, N, K):
    return int(load().wq_linear_w4a8_workspace_bytes(M, N, K))


def linear_w4a8(x, outliers, packed, scales, zeros, out_dtype=None, out=None, group: int = GROUP, workspace=None):
    """y = W4A8 product with fp16 outlier channels (``outliers`` int32 [n_out],
    n_out <= 16): the INT8 activations are made per call."""
    import torch
    lib = load()
    out_dtype = torch.float16 if out_dtype is None else out_dtype
    _need(x, torch.float16, "x")
    _need(outliers, torch.int32, "outliers")
    _need(packed, torch.int32, "packed")
    _need(scales, torch.float16, "scales")
    _need(zeros, torch.float16, "zeros")
    M, K = x.shape
    N = packed.shape[0]
    if packed.shape[1] * 8 != K or scales.shape != (N, K // group) or zeros.shape != scales.shape:
        raise ValueError("inconsistent shapes")
    if out_dtype not in (torch.float16, torch.float32):
        raise TypeError("out_dtype must be float16 or float32")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=x.device)
    else:
        _need(out, out_dtype, "out")
    if workspace is None:
        nbytes = int(lib.wq_linear_w4a8_workspace_bytes(max(M, 1), N, K))
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    wbytes = workspace.numel() * workspace.element_size()
    n_out = outliers.numel()
    rc = lib.wq_linear_w4a8(_p(x), M, K, _p(outliers) if n_out else None, n_out, _p(packed), _p(scales), _p(zeros),
                            N, group, _p(out), 1 if out_dtype == torch.float32 else 0, _p(workspace), wbytes,
                            _stream(x))
    _check("wq_linear_w4a8", rc)
    return out


def auto_kernel(M, N, K) -> str:
    k = int(load().wq_auto_kernel(M, N, K))
    return {1: "gemv", 2: "gemm"}[k]
