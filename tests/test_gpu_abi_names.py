"""The four entry points the boundary is named for -- wq_quantize_rtn, wq_pack,
wq_linear and wq_linear_sparse -- called directly through the C ABI (ctypes, no
binding wrapper) on the batched-decode layer (16 x 4096 x 4096 with its CSR) and
the 70B down-projection at M = 64, against the oracle. The products also run with
no workspace and with a workspace one byte short of wq_linear_workspace_bytes:
then the GEMM runs unsplit (and takes the CSR term inside its own tile loop), with
the same results up to rounding order."""
import ctypes

import numpy as np
import pytest

import oracle
import workloads
from gpu_cases import f16_bits_host, oracle_layer, rel_err_all_rows, say, to_dev

pytestmark = pytest.mark.gpu


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _quantize_and_pack(lib, torch, W, sparse_k):
    N, K = W.shape
    Wd = to_dev(W, torch)
    codes = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    scales = torch.empty((N, K // 128), dtype=torch.float16, device="cuda")
    zeros = torch.empty_like(scales)
    row_ptr = torch.empty(N + 1, dtype=torch.int32, device="cuda")
    col = torch.empty(max(sparse_k, 1), dtype=torch.int32, device="cuda")
    val = torch.empty(max(sparse_k, 1), dtype=torch.float16, device="cuda")
    need = lib.wq_quantize_workspace_bytes(N, K, sparse_k)
    ws = torch.empty(need + 256, dtype=torch.uint8, device="cuda")
    args = (_p(Wd), N, K, 128, sparse_k, _p(codes), _p(scales), _p(zeros), _p(row_ptr), _p(col), _p(val))
    if sparse_k:
        # missing or short workspace: refused on the host, nothing launched
        assert lib.wq_quantize_rtn(*args, None, 0, _stream()) == -6
        assert lib.wq_quantize_rtn(*args, _p(ws), need - 1, _stream()) == -6
    assert lib.wq_quantize_rtn(*args, _p(ws), need, _stream()) == 0
    packed = torch.empty((N, K // 8), dtype=torch.int32, device="cuda")
    assert lib.wq_pack(_p(codes), N, K, _p(packed), _stream()) == 0
    torch.cuda.synchronize()
    return dict(codes=codes, scales=scales, zeros=zeros, row_ptr=row_ptr, col=col[:sparse_k], val=val[:sparse_k],
                packed=packed)


def _check_layer(D, L):
    assert np.array_equal(D["codes"].cpu().numpy(), L["q"])
    assert np.array_equal(D["packed"].cpu().numpy().view(np.uint32), L["packed"])
    assert np.array_equal(f16_bits_host(D["scales"]), L["s"].view(np.uint16))
    assert np.array_equal(f16_bits_host(D["zeros"]), L["z"].view(np.uint16))
    assert np.array_equal(D["row_ptr"].cpu().numpy(), L["row_ptr"])
    assert np.array_equal(D["col"].cpu().numpy(), L["col"])
    assert np.array_equal(f16_bits_host(D["val"]), L["val"].view(np.uint16))


def _products(lib, torch, D, x, L, label):
    M, K = x.shape
    N = L["q"].shape[0]
    nnz = int(L["col"].size)
    xd = to_dev(x, torch)
    need = lib.wq_linear_workspace_bytes(M, N, K)
    big = torch.empty(need + 256, dtype=torch.uint8, device="cuda")
    for name, (ws, nbytes) in {"full workspace": (big, need), "no workspace": (None, 0),
                               "one byte short": (big, max(need - 1, 0))}.items():
        for sparse in (False, True):
            y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
            say(f"[abi] {label} M={M} {'wq_linear_sparse' if sparse else 'wq_linear'} {name} (need {need})")
            if sparse:
                rc = lib.wq_linear_sparse(_p(xd), M, K, _p(D["packed"]), _p(D["scales"]), _p(D["zeros"]), N, 128,
                                          _p(D["row_ptr"]), _p(D["col"]), _p(D["val"]), nnz, _p(y), 1, _p(ws),
                                          nbytes, _stream())
            else:
                rc = lib.wq_linear(_p(xd), M, K, _p(D["packed"]), _p(D["scales"]), _p(D["zeros"]), N, 128, _p(y), 1,
                                   _p(ws), nbytes, _stream())
            assert rc == 0, rc
            torch.cuda.synchronize()
            args = (L["row_ptr"], L["col"], L["val"]) if sparse else (None, None, None)
            err = rel_err_all_rows(y, N, lambda rows: oracle.linear_rows(x, L["packed"], L["s"], L["z"], rows, *args))
            say(f"    rel err {err:.3e}")
            assert err <= oracle.TOL, err


def test_named_entry_points_batched_decode(gpu_lib):
    import torch
    lib = gpu_lib.load()
    L = oracle_layer(3)
    D = _quantize_and_pack(lib, torch, L["W"], L["sparse_k"])
    _check_layer(D, L)
    _, x, _ = workloads.make(3)
    _products(lib, torch, D, x, L, "4096x4096")


def test_named_entry_points_70b_down_proj_m64(gpu_lib):
    import torch
    lib = gpu_lib.load()
    L = oracle_layer(5)
    D = _quantize_and_pack(lib, torch, L["W"], L["sparse_k"])
    _check_layer(D, L)
    _, x, _ = workloads.make(5, M=64)
    _products(lib, torch, D, x, L, "8192x28672")
