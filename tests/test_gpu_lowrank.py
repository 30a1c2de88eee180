"""Parity of the low-rank branch through wq_linear_lowrank with the float64
oracle: y = x . dequant(Wq)^T + W_sparse x + (x . L1^T) . L2^T within
||y - y_ref||_inf <= 5e-3 ||y_ref||_inf, bit-identical fp32 results on the
integer-exact case, on every kernel path (both decode kernels, single and
paired channel tiles, the large-M GEMM split and unsplit, the M <= 64 GEMM, the
tile GEMM for odd group counts) and at full size."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_cases import layer_to_dev, oracle_layer, rel_err_all_rows, say, to_dev

pytestmark = pytest.mark.gpu

TOL = oracle.TOL


def _run(wq, torch, L, D, x, L1, L2, kernel, sparse, out_dtype=None):
    xd = to_dev(x, torch)
    args = (D["row_ptr"], D["col"], D["val"]) if sparse else (None, None, None)
    return wq.linear_lowrank(xd, D["packed"], D["scales"], D["zeros"], to_dev(L1, torch), to_dev(L2, torch), *args,
                             out_dtype=out_dtype, kernel=kernel)


@pytest.mark.parametrize("M,N,K,r,sparse,kernel", [
    (1, 300, 1024, 32, True, "auto"),      # block-staged decode kernel
    (2, 130, 2048, 64, False, "auto"),
    (5, 300, 1536, 96, True, "auto"),      # per-wave staging kernel, rank not a multiple of 128
    (16, 260, 2048, 160, True, "auto"),
    (16, 300, 1024, 32, True, "gemm"),     # M <= 64 GEMM
    (40, 300, 1024, 64, True, "auto"),
    (64, 520, 2048, 32, False, "auto"),
    (100, 300, 1152, 32, True, "auto"),    # tile GEMM (64 < M <= 128)
    (130, 513, 384, 32, False, "auto"),    # tile GEMM (odd number of groups)
    (200, 256, 4096, 32, True, "auto"),    # large-M GEMM, split K, sparse term in the slice sum
    (300, 300, 1152, 64, False, "auto"),
    (70, 300, 1024, 32, True, "gemv"),     # decode kernel forced above its range
    (1100, 130, 2048, 64, True, "auto"),   # tall batch: 64-row down-projection blocks, ragged last block
    (2100, 64, 1024, 32, False, "auto"),   # tall batch, one component tile
])
def test_lowrank_parity(gpu_lib, M, N, K, r, sparse, kernel):
    import torch
    W = workloads.random_weights(M + N + K + r, N, K)
    L = oracle.quantize_layer(W, N * K // 250 if sparse else 0)
    x = workloads.random_x(M + 3 * r, M, K)
    L1, L2 = workloads.lowrank_factors(M + r, r, N, K)
    D = layer_to_dev(L, torch)
    say(f"[lowrank] M={M} N={N} K={K} r={r} sparse={sparse} kernel={kernel}")
    y = _run(gpu_lib, torch, L, D, x, L1, L2, kernel, sparse)
    torch.cuda.synchronize()
    args = (L["row_ptr"], L["col"], L["val"]) if sparse else (None, None, None)
    ref = oracle.linear_ref(x, L["q"], L["s"], L["z"], *args, L1=L1, L2=L2)
    err = oracle.rel_err_inf(y.float().cpu().numpy(), ref)
    say(f"    rel err {err:.3e}")
    assert err <= TOL, err
    # the branch is really there: without it the result is far off
    assert oracle.rel_err_inf(oracle.linear_ref(x, L["q"], L["s"], L["z"], *args), ref) > 10 * TOL


@pytest.mark.parametrize("kernel", ["gemv", "gemm"])
@pytest.mark.parametrize("M,K", [(1, 1024), (2, 4096), (16, 2048), (40, 1024), (200, 4096), (300, 1024)])
def test_lowrank_integer_exact_fp32(gpu_lib, kernel, M, K):
    """Integer codes, zero-points, activations, sparse values and factors with
    power-of-two scales: t = x . L1^T holds integers up to 1024 (exact in fp16)
    and every partial sum is exact in fp32, so y must be bit-identical."""
    import torch
    N, r = 96, 64
    x, q, s, z, rp, col, val = workloads.integer_case(M + K, M, N, K, nnz_per_row=5)
    L1, L2 = workloads.integer_lowrank_factors(M + 1, r, N, K)
    L = dict(q=q, s=s, z=z, packed=oracle.pack(q), row_ptr=rp, col=col, val=val)
    D = layer_to_dev(L, torch)
    say(f"[lowrank exact] kernel={kernel} M={M} K={K}")
    y = _run(gpu_lib, torch, L, D, x, L1, L2, kernel, True, out_dtype=torch.float32)
    ref = oracle.linear_ref(x, q, s, z, rp, col, val, L1=L1, L2=L2)
    assert np.array_equal(y.cpu().numpy().astype(np.float64), ref)


@pytest.mark.parametrize("index,M,K", [(2, 1, None), (5, 8, 3584), (4, 2048, None), (5, 512, None)])
def test_lowrank_full_size_all_outputs(gpu_lib, index, M, K):
    """Rank-32 branches on full-size layers (the decode and prefill layers, the 70B
    down-projection at M = 512 and its K = 3584 shard at M = 8, where each wave
    takes two channel tiles), every output compared."""
    import torch
    L = oracle_layer(index, K=K)
    _, x, _ = workloads.make(index, M=M, K=K)
    N, Kf = L["q"].shape
    L1, L2 = workloads.lowrank_factors(index + M, 32, N, Kf)
    D = layer_to_dev(L, torch)
    sparse = L["sparse_k"] > 0
    say(f"[lowrank full] config {index} M={M} N,K={N},{Kf}")
    y = _run(gpu_lib, torch, L, D, x, L1, L2, "auto", sparse)
    torch.cuda.synchronize()
    args = (L["row_ptr"], L["col"], L["val"]) if sparse else (None, None, None)
    err = rel_err_all_rows(y, N, lambda rows: oracle.linear_rows(x, L["packed"], L["s"], L["z"], rows, *args,
                                                                 L1=L1, L2=L2))
    say(f"    rel err {err:.3e}")
    assert err <= TOL, err


def test_lowrank_deterministic_and_empty(gpu_lib):
    import torch
    M, N, K, r = 200, 256, 4096, 32
    W = workloads.random_weights(91, N, K)
    L = oracle.quantize_layer(W, N * K // 200)
    x = workloads.random_x(92, M, K)
    L1, L2 = workloads.lowrank_factors(93, r, N, K)
    D = layer_to_dev(L, torch)
    a = _run(gpu_lib, torch, L, D, x, L1, L2, "auto", True, out_dtype=torch.float32)
    b = _run(gpu_lib, torch, L, D, x, L1, L2, "auto", True, out_dtype=torch.float32)
    assert torch.equal(a, b)
    e = _run(gpu_lib, torch, L, D, np.zeros((0, K), np.float16), L1, L2, "auto", True)
    torch.cuda.synchronize()
    assert tuple(e.shape) == (0, N)


def test_lowrank_integer_exact_tall_batch(gpu_lib):
    """The 64-row down-projection (600 rows x rank 256: 80 tiles) on the integer
    case: bit-identical fp32 output."""
    import torch
    M, N, K, r = 600, 96, 1024, 256
    x, q, s, z, rp, col, val = workloads.integer_case(M + K, M, N, K, nnz_per_row=5)
    L1, L2 = workloads.integer_lowrank_factors(M + 3, r, N, K)
    L = dict(q=q, s=s, z=z, packed=oracle.pack(q), row_ptr=rp, col=col, val=val)
    D = layer_to_dev(L, torch)
    say(f"[lowrank exact tall] M={M} r={r}")
    y = _run(gpu_lib, torch, L, D, x, L1, L2, "auto", True, out_dtype=torch.float32)
    ref = oracle.linear_ref(x, q, s, z, rp, col, val, L1=L1, L2=L2)
    assert np.array_equal(y.cpu().numpy().astype(np.float64), ref)


@pytest.mark.parametrize("M,N,K,r,sparse,kernel", [
    (1, 300, 1024, 32, True, "gemv"),      # block-staged decode kernel
    (2, 130, 2048, 64, False, "gemv"),
    (1, 200, 12288, 32, True, "gemv"),     # long row (the single-row kernel takes no branch): block-staged
    (5, 300, 1536, 96, True, "gemv"),      # per-wave staging kernel
    (9, 1100, 3584, 256, False, "gemv"),   # rank 256, 28 groups
    (100, 300, 1152, 64, True, "auto"),    # tile GEMM
])
def test_lowrank_consecutive_calls(gpu_lib, M, N, K, r, sparse, kernel):
    """Five calls in a row on the same layer and workspace with new activations
    each time, every one against the oracle: a t left in the workspace by the
    previous call would fail."""
    import torch
    W = workloads.random_weights(7 * M + N + r, N, K)
    L = oracle.quantize_layer(W, N * K // 250 if sparse else 0)
    L1, L2 = workloads.lowrank_factors(M + 5 * r, r, N, K)
    D = layer_to_dev(L, torch)
    L1d, L2d = to_dev(L1, torch), to_dev(L2, torch)
    ws = torch.empty(max(gpu_lib.linear_lowrank_workspace_bytes(M, N, K, r), 1), dtype=torch.uint8, device="cuda")
    args = (L["row_ptr"], L["col"], L["val"]) if sparse else (None, None, None)
    dargs = (D["row_ptr"], D["col"], D["val"]) if sparse else (None, None, None)
    say(f"[lowrank consecutive] M={M} N={N} K={K} r={r} sparse={sparse} kernel={kernel}")
    for call in range(5):
        x = workloads.random_x(1000 + 17 * call + M, M, K)
        y = gpu_lib.linear_lowrank(to_dev(x, torch), D["packed"], D["scales"], D["zeros"], L1d, L2d, *dargs,
                                   kernel=kernel, workspace=ws)
        torch.cuda.synchronize()
        ref = oracle.linear_ref(x, L["q"], L["s"], L["z"], *args, L1=L1, L2=L2)
        err = oracle.rel_err_inf(y.float().cpu().numpy(), ref)
        assert err <= TOL, (call, err)
