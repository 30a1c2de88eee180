"""C ABI checks that need no GPU: the library loads, exports every function that
include/wq.h declares, and rejects bad arguments on the host before any HIP call
(the fake device addresses below are never dereferenced)."""
import ctypes
import os
import re

import pytest

import quantized_gemm_rtn_amd as wq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wq.h")

A = ctypes.c_void_p(0x7F0000000000)      # 16-byte aligned fake device address
A2 = ctypes.c_void_p(0x7F0000100000)
A3 = ctypes.c_void_p(0x7F0000200000)
A4 = ctypes.c_void_p(0x7F0000300000)
A5 = ctypes.c_void_p(0x7F0000400000)
MIS = ctypes.c_void_p(0x7F0000000008)    # 8-byte aligned only


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(wq.LIB_PATH):
        import quantized_gemm_rtn_amd.build as b
        b.build()
    return wq.load()


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(wq_[a-z_0-9]+)\s*\(", src)))


def test_header_and_binding_agree(lib):
    names = header_functions()
    assert "wq_quantize_rtn" in names and "wq_pack" in names
    assert "wq_linear" in names and "wq_linear_sparse" in names
    assert sorted(wq.SIGNATURES) == names


def test_every_declared_symbol_is_exported(lib):
    raw = ctypes.CDLL(wq.LIB_PATH)
    for name in header_functions():
        assert hasattr(raw, name), name


def test_status_strings(lib):
    for code in range(-7, 1):
        s = lib.wq_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.wq_status_string(-99).decode() == "unknown status"


def test_auto_kernel(lib):
    """The measured crossover: the decode kernel (1) up to M = 16 everywhere; from
    M = 17 the GEMM (2) on the 70B layer, whose 64 x 256 tiles give every CU a block;
    on smaller layers (64 x 128 tiles) the decode kernel to M = 32, then to M = 48
    where the GEMM splits K fewer than four ways (28 groups), the GEMM above; the
    decode kernel while the tile GEMM's grid has under 128 blocks (group counts that
    are not a multiple of four)."""
    assert lib.wq_auto_kernel(1, 11008, 4096) == 1
    assert lib.wq_auto_kernel(16, 4096, 4096) == 1
    assert lib.wq_auto_kernel(16, 8192, 28672) == 1
    assert lib.wq_auto_kernel(17, 8192, 28672) == 2
    assert lib.wq_auto_kernel(64, 8192, 28672) == 2
    for N, K in [(4096, 4096), (11008, 4096)]:
        assert lib.wq_auto_kernel(32, N, K) == 1
        assert lib.wq_auto_kernel(33, N, K) == 2
        assert lib.wq_auto_kernel(64, N, K) == 2
    assert lib.wq_auto_kernel(48, 8192, 3584) == 1
    assert lib.wq_auto_kernel(49, 8192, 3584) == 2
    assert lib.wq_auto_kernel(40, 300, 3 * 128) == 1      # tile GEMM, 2 blocks
    assert lib.wq_auto_kernel(65, 4096, 4096) == 2
    assert lib.wq_auto_kernel(2048, 14336, 4096) == 2


def test_workspace_sizes(lib):
    assert lib.wq_quantize_workspace_bytes(64, 256, 0) == 0
    b = lib.wq_quantize_workspace_bytes(4096, 4096, 75497)
    assert b >= 4096 * 4096 // 8 + 3 * 4096 * 4 + 2048 * 4
    assert lib.wq_quantize_workspace_bytes(64, 100, 5) == 0      # invalid K
    # the prefill GEMM splits K only when its tile grid cannot fill the GPU; a CSR
    # product of that shape still needs one fp32 partial of y and x transposed
    assert lib.wq_linear_workspace_bytes(2048, 14336, 4096) == 2048 * 14336 * 4 + 4096 * 2048 * 2
    # shapes that only the tile kernel takes (K not a multiple of four groups at
    # M <= 64, an odd number of groups above 128 rows) need nothing unsplit
    assert lib.wq_linear_workspace_bytes(40, 8192, 3 * 128) == 0
    # split-K partials, plus the transposed activations of a product with a CSR term
    ws = lib.wq_linear_workspace_bytes(512, 8192, 28672)
    assert ws >= 2 * 512 * 8192 * 4 + 28672 * 512 * 2
    assert lib.wq_linear_workspace_bytes(0, 8192, 28672) == 0


def linear(lib, x=A, M=1, K=256, packed=A2, scales=A3, zeros=A4, N=64, group=128, row_ptr=None, col=None,
           val=None, nnz=0, y=A5, y_dtype=0, kernel=0):
    return lib.wq_linear_sparse_kernel(x, M, K, packed, scales, zeros, N, group, row_ptr, col, val, nnz, y,
                                       y_dtype, kernel, None, 0, None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), -1), (dict(packed=None), -1), (dict(scales=None), -1), (dict(zeros=None), -1),
    (dict(y=None), -1), (dict(nnz=5, row_ptr=None), -1), (dict(row_ptr=A, nnz=3, col=None, val=A2), -1),
    (dict(row_ptr=A, nnz=3, col=A2, val=None), -1),
    (dict(group=32), -4), (dict(group=256), -4), (dict(y_dtype=2), -4), (dict(kernel=4), -4),
    (dict(M=-1), -2), (dict(N=0), -2), (dict(K=0), -2), (dict(K=100), -2), (dict(K=64), -2),
    (dict(nnz=-1, row_ptr=A), -2), (dict(M=1 << 20, K=4096), -2), (dict(N=1 << 20, K=4096), -2),
    (dict(x=MIS), -3), (dict(packed=MIS), -3), (dict(scales=ctypes.c_void_p(0x7F0000000001)), -3),
    (dict(y=ctypes.c_void_p(0x7F0000000002)), -3),
])
def test_linear_validation(lib, kw, status):
    assert linear(lib, **kw) == status


def test_empty_batch_is_a_no_op(lib):
    """M = 0 computes nothing and accepts NULL activations and output, but the
    weights and the other sizes are still checked (no HIP call either way)."""
    assert linear(lib, M=0, x=None, y=None) == 0
    assert linear(lib, M=0, x=None, y=None, kernel=2) == 0
    assert linear(lib, M=0, x=None, y=None, packed=None) == -1
    assert linear(lib, M=0, x=None, y=None, K=100) == -2
    assert linear(lib, M=1, x=None) == -1


def test_linear_wrappers_validate(lib):
    assert lib.wq_linear(None, 1, 256, A2, A3, A4, 64, 128, A5, 0, None, 0, None) == -1
    assert lib.wq_linear(A, 1, 256, A2, A3, A4, 64, 32, A5, 0, None, 0, None) == -4
    # wq_linear_sparse requires row_ptr
    assert lib.wq_linear_sparse(A, 1, 256, A2, A3, A4, 64, 128, None, None, None, 0, A5, 0, None, 0, None) == -1


def quant(lib, W=A, N=8, K=256, group=128, sparse_k=0, codes=A2, scales=A3, zeros=A4, row_ptr=None, col=None,
          val=None, ws=None, ws_bytes=0):
    return lib.wq_quantize_rtn(W, N, K, group, sparse_k, codes, scales, zeros, row_ptr, col, val, ws, ws_bytes,
                               None)


@pytest.mark.parametrize("kw,status", [
    (dict(W=None), -1), (dict(codes=None), -1), (dict(scales=None), -1), (dict(zeros=None), -1),
    (dict(sparse_k=3), -1), (dict(sparse_k=3, row_ptr=A, col=A, val=None), -1),
    # quantization groups: a multiple of 128 dividing K, or -1 (per row)
    (dict(group=32), -4), (dict(group=192), -4), (dict(group=512), -4), (dict(group=0), -4),
    (dict(group=-2), -4), (dict(K=384, group=256), -4),
    (dict(K=200), -2), (dict(N=0), -2), (dict(sparse_k=-1), -2),
    (dict(sparse_k=8 * 256 + 1, row_ptr=A, col=A, val=A), -2),
    (dict(W=MIS), -3), (dict(codes=MIS), -3),
    (dict(sparse_k=3, row_ptr=A, col=A, val=A), -6),
    (dict(sparse_k=3, row_ptr=A, col=A, val=A, ws=A5, ws_bytes=16), -6),
])
def test_quantize_validation(lib, kw, status):
    assert quant(lib, **kw) == status


def test_pack_validation(lib):
    assert lib.wq_pack(None, 4, 64, A2, None) == -1
    assert lib.wq_pack(A, 4, 12, A2, None) == -2
    assert lib.wq_pack(A, 0, 64, A2, None) == -2
    assert lib.wq_pack(MIS, 4, 64, A2, None) == -3


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(wq, "_lib", None)
    monkeypatch.setattr(wq, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        wq.load()


def lowrank(lib, x=A, M=1, K=256, packed=A2, scales=A3, zeros=A4, N=64, group=128, row_ptr=None, col=None,
            val=None, nnz=0, L1=A5, L2=A, r=32, y=A5, y_dtype=0, kernel=0, ws=None, ws_bytes=0):
    return lib.wq_linear_lowrank(x, M, K, packed, scales, zeros, N, group, row_ptr, col, val, nnz, L1, L2, r, y,
                                 y_dtype, kernel, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(L1=None), -1), (dict(L2=None), -1), (dict(x=None), -1), (dict(nnz=4), -1),
    (dict(r=0), -2), (dict(r=-32), -2), (dict(M=-1), -2),
    (dict(r=16), -4), (dict(r=48), -4), (dict(r=288), -4), (dict(group=64), -4),
    (dict(L1=MIS), -3), (dict(L2=MIS), -3),
    (dict(), -6), (dict(ws=A, ws_bytes=16), -6), (dict(ws=MIS, ws_bytes=1 << 30), -6),
])
def test_lowrank_validation(lib, kw, status):
    assert lowrank(lib, **kw) == status


def test_lowrank_workspace_and_empty_batch(lib):
    # up to 16 rows: t [M, r] fp16 alone (256-byte aligned), on top of the GEMM's own
    assert lib.wq_linear_lowrank_workspace_bytes(1, 11008, 4096, 32) == \
        lib.wq_linear_workspace_bytes(1, 11008, 4096) + 256
    assert lib.wq_linear_lowrank_workspace_bytes(16, 11008, 4096, 256) == \
        lib.wq_linear_workspace_bytes(16, 11008, 4096) + 16 * 256 * 2
    # more rows: t plus the fp32 partials of the down-projection's K chunks
    assert lib.wq_linear_lowrank_workspace_bytes(512, 8192, 28672, 64) >= \
        lib.wq_linear_workspace_bytes(512, 8192, 28672) + 512 * 64 * 2
    for bad in ((1, 64, 256, 16), (1, 64, 256, 0), (0, 64, 256, 32), (1, 64, 100, 32), (1, 64, 256, 512)):
        assert lib.wq_linear_lowrank_workspace_bytes(*bad) == 0
    # an empty batch launches nothing and needs no workspace
    assert lowrank(lib, M=0, x=None, y=None) == 0


# ---------------------------------------------------------------- act-order layers
def quant_ao(lib, W=A, N=8, K=256, group=128, perm=A5, sparse_k=0, codes=A2, scales=A3, zeros=A4, row_ptr=None,
             col=None, val=None, ws=A, ws_bytes=1 << 20):
    return lib.wq_quantize_rtn_act_order(W, N, K, group, perm, sparse_k, codes, scales, zeros, row_ptr, col, val,
                                         ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(perm=None), -1), (dict(W=None), -1), (dict(group=64), -4), (dict(K=200), -2),
    (dict(perm=MIS), -3), (dict(ws=None), -6), (dict(ws_bytes=8 * 256 * 4 - 1), -6), (dict(ws=MIS), -3),
    (dict(sparse_k=3, row_ptr=A, col=A, val=A, ws_bytes=8 * 256 * 4), -6),
])
def test_quantize_act_order_validation(lib, kw, status):
    assert quant_ao(lib, **kw) == status


def lin_ao(lib, x=A, M=1, K=256, perm=A5, N=64, group=128, row_ptr=None, nnz=0, y=A2, kernel=0, ws=A,
           ws_bytes=1 << 20):
    return lib.wq_linear_act_order(x, M, K, perm, A2, A3, A4, N, group, row_ptr, None, None, nnz, y, 0, kernel, ws,
                                   ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(perm=None), -1), (dict(x=None), -1), (dict(nnz=3), -1), (dict(group=256), -4), (dict(kernel=7), -4),
    (dict(K=200), -2), (dict(perm=MIS), -3), (dict(x=MIS), -3),
    (dict(ws=None), -6), (dict(ws_bytes=255), -6), (dict(ws=MIS), -3),
])
def test_linear_act_order_validation(lib, kw, status):
    assert lin_ao(lib, **kw) == status


def test_act_order_workspace_and_empty_batch(lib):
    # the permuted copy (rounded up to 256 bytes) on top of the plain entry point's workspace
    assert lib.wq_quantize_act_order_workspace_bytes(8, 256, 0) == 8 * 256 * 4
    assert lib.wq_quantize_act_order_workspace_bytes(8, 256, 5) == \
        8 * 256 * 4 + lib.wq_quantize_workspace_bytes(8, 256, 5)
    assert lib.wq_linear_act_order_workspace_bytes(1, 11008, 4096) == \
        4096 * 2 + lib.wq_linear_workspace_bytes(1, 11008, 4096)
    assert lib.wq_linear_act_order_workspace_bytes(3, 64, 128) == 768 + lib.wq_linear_workspace_bytes(3, 64, 128)
    for bad in ((0, 64, 256), (1, 0, 256), (1, 64, 100)):
        assert lib.wq_linear_act_order_workspace_bytes(*bad) == 0
    # an empty batch launches nothing and needs no workspace
    assert lin_ao(lib, M=0, x=None, y=None, ws=None, ws_bytes=0) == 0


# ---------------------------------------------------------------- W4A8 with fp16 outlier channels
def lin_w8(lib, x=A, M=4, K=256, outliers=A5, n_out=8, N=64, group=128, y=A2, y_dtype=0, ws=A, ws_bytes=1 << 20):
    return lib.wq_linear_w4a8(x, M, K, outliers, n_out, A2, A3, A4, N, group, y, y_dtype, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(outliers=None), -1), (dict(x=None), -1), (dict(y=None), -1), (dict(n_out=17), -4), (dict(n_out=-1), -4),
    (dict(group=256), -4), (dict(y_dtype=5), -4), (dict(K=200), -2), (dict(N=0), -2), (dict(x=MIS), -3),
    (dict(outliers=ctypes.c_void_p(0x7F0000400002)), -3), (dict(ws=None), -6), (dict(ws_bytes=100), -6),
    (dict(ws=MIS), -3),
])
def test_linear_w4a8_validation(lib, kw, status):
    assert lin_w8(lib, **kw) == status


def test_w4a8_workspace_act_validation_and_empty_batch(lib):
    # xq (M*K int8), s_x, the outlier activations and weights, each rounded up to 256 bytes
    assert lib.wq_linear_w4a8_workspace_bytes(4, 64, 256) == 1024 + 256 + 256 + 64 * 16 * 2
    assert lib.wq_linear_w4a8_workspace_bytes(0, 64, 256) == 0
    assert lin_w8(lib, M=0, x=None, y=None, ws=None, ws_bytes=0) == 0
    assert lin_w8(lib, M=0, x=None, y=None, outliers=None, n_out=0, ws=None, ws_bytes=0) == 0
    act = lib.wq_quantize_act_int8
    assert act(A, 4, 256, None, 2, A2, A3, A4, None) == -1
    assert act(A, 4, 256, A5, 17, A2, A3, A4, None) == -4
    assert act(A, 4, 200, A5, 2, A2, A3, A4, None) == -2
    assert act(A, 4, 256, A5, 2, MIS, A3, A4, None) == -3
    assert act(None, 0, 256, None, 0, None, None, None, None) == 0


def test_quantize_bits_validation(lib):
    q = lib.wq_quantize_rtn_bits
    for bad in (1, 5, 8, 0, -1):
        assert q(A, 8, 256, 128, bad, 0, A2, A3, A4, None, None, None, None, 0, None) == -4
    assert q(None, 8, 256, 128, 3, 0, A2, A3, A4, None, None, None, None, 0, None) == -1
    assert q(A, 8, 200, 128, 3, 0, A2, A3, A4, None, None, None, None, 0, None) == -2


def test_last_hip_error_starts_clear(lib):
    """No launch has failed in this thread: the recorded HIP error is hipSuccess."""
    assert lib.wq_last_hip_error() == 0
    assert wq.last_hip_error() == 0


def test_header_error_contract():
    """The header names the query that returns a failed launch's cause, and does
    not promise that HIP's own error state still holds it (the launchers read it)."""
    src = open(HEADER).read()
    assert "wq_last_hip_error" in src
    assert "hipGetLastError() then holds" not in src
    assert "keeps no state between calls" not in src


def test_no_function_static_state():
    """No mutable function-local statics in the library sources: such caches are
    shared, unsynchronized state between concurrent callers and devices."""
    import glob
    bad = []
    for path in glob.glob(os.path.join(ROOT, "quantized_gemm_rtn_amd", "csrc", "*")):
        for i, line in enumerate(open(path), 1):
            if re.match(r"^\s+static\s+(?!constexpr\b|const\b|_assert|inline\b|hipError_t\b)", line):
                bad.append(f"{os.path.basename(path)}:{i}: {line.strip()}")
    assert not bad, bad


def test_noalloc_validation(lib):
    """wq_linear_sparse_noalloc checks its arguments like wq_linear_sparse and
    rejects, before any HIP call, a product whose split GEMM would need more than
    the scratch it holds per GPU."""
    f = lib.wq_linear_sparse_noalloc
    assert f(None, 1, 256, A2, A3, A4, 64, 128, None, None, None, 0, A5, 0, None) == -1
    assert f(A, 1, 256, A2, A3, A4, 64, 64, None, None, None, 0, A5, 0, None) == -4
    assert f(A, 1, 100, A2, A3, A4, 64, 128, None, None, None, 0, A5, 0, None) == -2
    assert f(MIS, 1, 256, A2, A3, A4, 64, 128, None, None, None, 0, A5, 0, None) == -3
    assert f(None, 0, 256, A2, A3, A4, 64, 128, None, None, None, 0, None, 0, None) == 0   # empty batch
    # 512 x 16384 x 65536 with a CSR term: the split-K partials plus the transposed
    # activations exceed WQ_NOALLOC_SCRATCH_BYTES (96 MiB)
    M, N, K = 512, 16384, 65536
    assert lib.wq_linear_workspace_bytes(M, N, K) > 96 << 20
    assert f(A, M, K, A2, A3, A4, N, 128, A, A2, A3, 10, A5, 0, None) == -7
    # the 70B down-projection at M = 512 with its CSR fits (about 92 MiB)
    assert lib.wq_linear_workspace_bytes(512, 8192, 28672) <= 96 << 20
    # the prefill layer with a CSR term does not split K: one fp32 partial of y and
    # the transposed activations (134 MB) exceed the scratch
    M, N, K = 2048, 14336, 4096
    assert lib.wq_linear_workspace_bytes(M, N, K) == M * N * 4 + K * M * 2
    assert f(A, M, K, A2, A3, A4, N, 128, A, A2, A3, 10, A5, 0, None) == -7
