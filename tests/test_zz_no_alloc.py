"""The no-allocation entry point, wq_linear_sparse_noalloc, against wq_linear_sparse
with a caller-provided workspace: two calls in a row on the library's per-GPU
scratch, the second with a smaller input, each bit-identical to the workspace
call (same kernels, same split plan) and within the oracle tolerance."""
import ctypes

import numpy as np
import pytest

import oracle
import workloads
from gpu_cases import layer_to_dev, say, to_dev

pytestmark = pytest.mark.gpu


def _noalloc(wq, xd, D, out, nnz):
    lib = wq.load()
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    import torch
    M, K = xd.shape
    N = D["packed"].shape[0]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return lib.wq_linear_sparse_noalloc(p(xd), M, K, p(D["packed"]), p(D["scales"]), p(D["zeros"]), N, 128,
                                        p(D["row_ptr"]), p(D["col"]) if nnz else None,
                                        p(D["val"]) if nnz else None, nnz, p(out), 1, stream)


def _with_workspace(wq, xd, D, nnz):
    import torch
    M, K = xd.shape
    N = D["packed"].shape[0]
    ws = torch.empty(max(1, wq.linear_workspace_bytes(M, N, K)), dtype=torch.uint8, device="cuda")
    # garbage in the workspace: its contents on entry must not matter
    ws.fill_(0xA5)
    return wq.linear_sparse(xd, D["packed"], D["scales"], D["zeros"], D["row_ptr"], D["col"] if nnz else None,
                            D["val"] if nnz else None, out_dtype=torch.float32, workspace=ws)


# (M, N, K, nnz per 200 weights): a CSR product whose GEMM splits K with the sparse
# term in the slice sum, then a smaller split one (64 x 256 tiles), then a dense
# split one, a decode-sized one, and a CSR product whose GEMM does not split K (one
# fp32 slice, then the sum with the sparse term)
CASES = [(200, 256, 4096, 1), (40, 96, 2048, 1), (64, 520, 2048, 0), (4, 300, 1024, 1), (300, 2048, 1024, 1)]


def test_noalloc_matches_workspace_entry_point(gpu_lib):
    import torch
    for i, (M, N, K, sp) in enumerate(CASES):
        W = workloads.random_weights(900 + i, N, K)
        L = oracle.quantize_layer(W, N * K // 200 if sp else 0)
        x = workloads.random_x(910 + i, M, K)
        D = layer_to_dev(L, torch)
        xd = to_dev(x, torch)
        nnz = int(L["col"].size)
        say(f"[noalloc] call {i}: M={M} N={N} K={K} nnz={nnz} split_ws={gpu_lib.linear_workspace_bytes(M, N, K)}")
        out = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        rc = _noalloc(gpu_lib, xd, D, out, nnz)
        assert rc == 0, (rc, gpu_lib.last_hip_error())
        ref_ws = _with_workspace(gpu_lib, xd, D, nnz)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_ws), i
        ref = oracle.linear_ref(x, L["q"], L["s"], L["z"], L["row_ptr"], L["col"], L["val"])
        err = oracle.rel_err_inf(out.cpu().numpy(), ref)
        say(f"    rel err {err:.3e}")
        assert err <= oracle.TOL, err


def test_noalloc_binding_fp16(gpu_lib):
    """The binding's wrapper (fp16 output) equals wq_linear_sparse's fp16 output."""
    import torch
    M, N, K = 96, 300, 1024
    W = workloads.random_weights(931, N, K)
    L = oracle.quantize_layer(W, N * K // 200)
    x = workloads.random_x(932, M, K)
    D = layer_to_dev(L, torch)
    xd = to_dev(x, torch)
    out = torch.empty((M, N), dtype=torch.float16, device="cuda")
    gpu_lib.linear_sparse_noalloc(xd, D["packed"], D["scales"], D["zeros"], out, D["row_ptr"], D["col"], D["val"])
    ref = gpu_lib.linear_sparse(xd, D["packed"], D["scales"], D["zeros"], D["row_ptr"], D["col"], D["val"])
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
