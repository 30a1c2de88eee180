"""Parity of the GPU decode GEMV and prefill GEMM (with the fused sparse term)
with the float64 oracle: ||y - y_ref||_inf <= 5e-3 ||y_ref||_inf, bit-identical
fp32 results on the integer-exact case, and run-to-run determinism."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_cases import layer_to_dev, oracle_layer, rel_err_all_rows, run_linear, say, to_dev

pytestmark = pytest.mark.gpu

TOL = oracle.TOL


def _full_check(wq, torch, L, x, kernel, out_dtype=None, sparse=True, label=""):
    D = layer_to_dev(L, torch)
    xd = to_dev(x, torch)
    say(f"[linear] {label} M={x.shape[0]} N,K={L['q'].shape} kernel={kernel}")
    y = run_linear(wq, xd, D, kernel=kernel, out_dtype=out_dtype, sparse=sparse)
    torch.cuda.synchronize()
    if sparse:
        ref = oracle.linear_ref(x, L["q"], L["s"], L["z"], L["row_ptr"], L["col"], L["val"])
    else:
        ref = oracle.linear_ref(x, L["q"], L["s"], L["z"])
    err = oracle.rel_err_inf(y.float().cpu().numpy(), ref)
    say(f"    rel err {err:.3e}")
    assert err <= TOL, err
    return y


@pytest.mark.parametrize("index", [1, 2, 3])
@pytest.mark.parametrize("kernel", ["auto", "gemm"])
def test_small_configs_full(gpu_lib, index, kernel):
    import torch
    L = oracle_layer(index)
    _, x, _ = workloads.make(index)
    _full_check(gpu_lib, torch, L, x, kernel, label=f"config {index}")


def _all_rows_check(wq, torch, L, x, kernel, label):
    """Every output channel of a full-size product against the oracle, computed a
    block of channels at a time."""
    D = layer_to_dev(L, torch)
    xd = to_dev(x, torch)
    N = L["q"].shape[0]
    say(f"[linear] {label} M={x.shape[0]} N,K={L['q'].shape} kernel={kernel} all {N} channels")
    y = run_linear(wq, xd, D, kernel=kernel)
    torch.cuda.synchronize()
    err = rel_err_all_rows(y, N, lambda rows: oracle.linear_rows(x, L["packed"], L["s"], L["z"], rows,
                                                                 L["row_ptr"], L["col"], L["val"]))
    say(f"    rel err {err:.3e}")
    assert err <= TOL, err


def test_config4_prefill_all_outputs(gpu_lib):
    """The prefill layer (2048 x 14336 x 4096, unsplit 128 x 256 tiles with the
    XCD tile order and a partial last round), every output compared."""
    import torch
    L = oracle_layer(4)
    _, x, _ = workloads.make(4)
    _all_rows_check(gpu_lib, torch, L, x, "auto", "config 4")


def test_config4_prefill_with_csr_all_outputs(gpu_lib):
    """The prefill layer with CSR outliers at 0.45 % of its weights (264 241
    entries), as the bench times it: the 128 x 256 GEMM unsplit, writing one fp32
    partial and the transposed activations, then the slice sum with the sparse
    term; every output compared."""
    import torch
    W, x, _ = workloads.make(4)
    N, K = W.shape
    L = oracle.quantize_layer(W, workloads.SPARSE_PPM_DENSE_AND_SPARSE * N * K // 1_000_000)
    del W, L["W_dense"]
    _all_rows_check(gpu_lib, torch, L, x, "auto", "config 4 + CSR")


@pytest.mark.parametrize("M", [1, 8, 64, 512])
def test_config5_sweep_all_outputs(gpu_lib, M):
    import torch
    L = oracle_layer(5)
    _, x, _ = workloads.make(5, M=M)
    _all_rows_check(gpu_lib, torch, L, x, "auto", "config 5")


@pytest.mark.parametrize("M", [1, 512])
def test_config5_shard_all_outputs(gpu_lib, M):
    """One GPU's share of the 70B down-projection split eight ways along K
    (x [M, 3584], W [8192, 3584] with its share of the CSR), in the launch
    configuration the benchmark times."""
    import torch
    L = oracle_layer(5, K=3584)
    _, x, _ = workloads.make(5, M=M, K=3584)
    _all_rows_check(gpu_lib, torch, L, x, "auto", "config 5 shard")


@pytest.mark.parametrize("M", [1, 2, 3, 7, 15, 16, 17, 31, 33, 64, 65, 130])
@pytest.mark.parametrize("kernel", ["gemv", "gemm"])
def test_ragged_shapes(gpu_lib, M, kernel):
    import torch
    N, K = 300, 640
    W = workloads.random_weights(100 + M, N, K)
    L = oracle.quantize_layer(W, 700)
    x = workloads.random_x(200 + M, M, K)
    _full_check(gpu_lib, torch, L, x, kernel, label="ragged")


@pytest.mark.parametrize("N,K,M", [(1, 128, 1), (17, 128, 5), (130, 256, 70), (16, 1152, 16), (257, 384, 129)])
@pytest.mark.parametrize("kernel", ["auto", "gemv", "gemm"])
def test_edge_shapes(gpu_lib, N, K, M, kernel):
    import torch
    W = workloads.random_weights(N * 7 + K, N, K)
    L = oracle.quantize_layer(W, max(1, N * K // 200))
    x = workloads.random_x(M + N, M, K)
    _full_check(gpu_lib, torch, L, x, kernel, label="edge")


@pytest.mark.parametrize("kernel", ["gemv", "gemm"])
@pytest.mark.parametrize("M", [1, 16, 40])
def test_integer_exact_fp32(gpu_lib, kernel, M):
    """Power-of-two scales, integer zero-points, codes, activations and sparse
    values: every partial sum is exact in fp32, so y must be bit-identical."""
    import torch
    N, K = 96, 1024
    x, q, s, z, rp, col, val = workloads.integer_case(3 + M, M, N, K, nnz_per_row=5)
    L = dict(q=q, s=s, z=z, packed=oracle.pack(q), row_ptr=rp, col=col, val=val)
    D = layer_to_dev(L, torch)
    say(f"[exact] kernel={kernel} M={M}")
    y = run_linear(gpu_lib, to_dev(x, torch), D, kernel=kernel, out_dtype=torch.float32)
    ref = oracle.linear_ref(x, q, s, z, rp, col, val)
    assert np.array_equal(y.cpu().numpy().astype(np.float64), ref)


@pytest.mark.parametrize("K", [3584, 1536, 2816, 16896])
@pytest.mark.parametrize("M", [1, 2, 5, 16])
def test_decode_scale_staging_widths(gpu_lib, M, K):
    """Decode kernels whose per-group scales and zero-points are staged as vectors
    of four halves (G = 28, 12), two halves (G = 22) and single halves (G = 132),
    with a ragged N and a CSR term."""
    import torch
    N = 300 if K <= 4096 else 40
    W = workloads.random_weights(K + M, N, K)
    L = oracle.quantize_layer(W, N * K // 300)
    x = workloads.random_x(K + 3 * M, M, K)
    _full_check(gpu_lib, torch, L, x, "gemv", label="staging widths")


@pytest.mark.parametrize("K", [3584, 2816])
@pytest.mark.parametrize("M", [1, 8])
def test_integer_exact_fp32_staging_widths(gpu_lib, M, K):
    """The integer-exact case through the decode kernels at G = 28 and G = 22."""
    import torch
    N = 96
    x, q, s, z, rp, col, val = workloads.integer_case(M + K, M, N, K, nnz_per_row=5)
    L = dict(q=q, s=s, z=z, packed=oracle.pack(q), row_ptr=rp, col=col, val=val)
    D = layer_to_dev(L, torch)
    say(f"[exact staging] M={M} K={K}")
    y = run_linear(gpu_lib, to_dev(x, torch), D, kernel="gemv", out_dtype=torch.float32)
    ref = oracle.linear_ref(x, q, s, z, rp, col, val)
    assert np.array_equal(y.cpu().numpy().astype(np.float64), ref)


@pytest.mark.parametrize("M,N,K", [(17, 300, 1024), (64, 520, 2048), (100, 256, 4096), (128, 1000, 768),
                                   (129, 300, 640), (300, 300, 1152), (257, 513, 384), (200, 256, 4096),
                                   (520, 1000, 2048), (48, 300, 1536)])
def test_dense_large_m(gpu_lib, M, N, K):
    """Dense products (no CSR) above the decode range: ragged M and N, even and odd
    numbers of groups, and single output tiles whose K is split."""
    import torch
    W = workloads.random_weights(3 * M + N, N, K)
    L = oracle.quantize_layer(W, 0)
    x = workloads.random_x(M + 7, M, K)
    _full_check(gpu_lib, torch, L, x, "gemm", sparse=False, label="dense")


@pytest.mark.parametrize("M,N,K", [(40, 300, 1024), (300, 300, 1152), (200, 256, 4096)])
def test_integer_exact_fp32_dense_large_m(gpu_lib, M, N, K):
    """The integer-exact case through the dense kernels above the decode range,
    unsplit and split."""
    import torch
    x, q, s, z, _, _, _ = workloads.integer_case(M + K, M, N, K, nnz_per_row=0)
    L = dict(q=q, s=s, z=z, packed=oracle.pack(q))
    D = layer_to_dev(dict(L, row_ptr=np.zeros(N + 1, np.int32), col=np.zeros(0, np.int32),
                          val=np.zeros(0, np.float16)), torch)
    say(f"[exact dense] M={M} N={N} K={K}")
    y = run_linear(gpu_lib, to_dev(x, torch), D, kernel="gemm", out_dtype=torch.float32, sparse=False)
    ref = oracle.linear_ref(x, q, s, z)
    assert np.array_equal(y.cpu().numpy().astype(np.float64), ref)


@pytest.mark.parametrize("M,N,K", [(17, 300, 2048), (64, 520, 2048), (200, 256, 4096), (300, 300, 2304),
                                   (520, 1000, 2048), (48, 300, 3072)])
def test_sparse_large_m_split(gpu_lib, M, N, K):
    """CSR products whose dense kernel splits K: the sparse term is added in the
    slice sum from transposed activations (one or two 512-row chunks)."""
    import torch
    W = workloads.random_weights(5 * M + N, N, K)
    L = oracle.quantize_layer(W, N * K // 200)
    x = workloads.random_x(M + 11, M, K)
    _full_check(gpu_lib, torch, L, x, "gemm", label="sparse split")


@pytest.mark.parametrize("M,N,K", [(37, 11008, 4096), (5, 8192, 4096), (48, 8192, 3072), (64, 3841, 2048),
                                   (64, 3840, 2048), (130, 16384, 2048), (300, 8192, 2048), (300, 2048, 1024),
                                   (1100, 8192, 1024), (40, 1000, 1024), (40, 8192, 1024)])
def test_sparse_split_wide_layers(gpu_lib, M, N, K):
    """CSR products on layers wide enough (at least 16 column tiles of 64-row tiles,
    32 of 128-row tiles) that the split GEMM writes the transposed activations
    itself, each block a share of every group's channels: ragged M (rows past M
    written as zero), 43 column tiles (shares of 3 channels, the last one partly past
    the group), both tile heights, weight windows of two and four groups, and 3840
    output channels, the widest 64-row layer that still takes the transpose launch;
    and products whose GEMM does not split K (one fp32 slice, then the same sum), on
    wide and narrow layers of both tile heights."""
    import torch
    W = workloads.random_weights(3 * M + N + K, N, K)
    L = oracle.quantize_layer(W, N * K // 200)
    x = workloads.random_x(M + 23, M, K)
    _full_check(gpu_lib, torch, L, x, "gemm", label="sparse split, wide")


@pytest.mark.parametrize("M,N,K", [(40, 96, 4096), (200, 256, 4096), (520, 300, 2048), (37, 11008, 2048),
                                   (300, 8192, 2048), (300, 2048, 1024), (40, 8192, 1024)])
def test_integer_exact_fp32_sparse_split(gpu_lib, M, N, K):
    """The integer-exact case with a CSR term through the split dense kernels."""
    import torch
    x, q, s, z, rp, col, val = workloads.integer_case(M + 2 * K, M, N, K, nnz_per_row=5)
    L = dict(q=q, s=s, z=z, packed=oracle.pack(q), row_ptr=rp, col=col, val=val)
    D = layer_to_dev(L, torch)
    say(f"[exact sparse split] M={M} N={N} K={K}")
    y = run_linear(gpu_lib, to_dev(x, torch), D, kernel="gemm", out_dtype=torch.float32)
    ref = oracle.linear_ref(x, q, s, z, rp, col, val)
    assert np.array_equal(y.cpu().numpy().astype(np.float64), ref)


@pytest.mark.parametrize("kernel", ["gemv", "gemm"])
def test_empty_sparse_equals_dense(gpu_lib, kernel):
    import torch
    L = oracle_layer(1)
    _, x, _ = workloads.make(1)
    D = layer_to_dev(L, torch)
    xd = to_dev(x, torch)
    a = gpu_lib.linear(xd, D["packed"], D["scales"], D["zeros"], kernel=kernel)
    b = gpu_lib.linear_sparse(xd, D["packed"], D["scales"], D["zeros"], D["row_ptr"], D["col"], D["val"],
                              kernel=kernel)
    assert L["sparse_k"] == 0 and torch.equal(a, b)


@pytest.mark.parametrize("kernel", ["gemv", "gemm"])
def test_deterministic(gpu_lib, kernel):
    import torch
    L = oracle_layer(3)
    _, x, _ = workloads.make(3)
    D = layer_to_dev(L, torch)
    xd = to_dev(x, torch)
    a = run_linear(gpu_lib, xd, D, kernel=kernel, out_dtype=torch.float32)
    b = run_linear(gpu_lib, xd, D, kernel=kernel, out_dtype=torch.float32)
    assert torch.equal(a, b)


def test_end_to_end_gpu_pipeline(gpu_lib):
    """GPU quantize -> pack -> linear_sparse against the oracle pipeline."""
    import torch
    L = oracle_layer(3)
    _, x, _ = workloads.make(3)
    out = gpu_lib.quantize_rtn(to_dev(L["W"], torch), sparse_k=L["sparse_k"])
    packed = gpu_lib.pack(out["codes"])
    y = gpu_lib.linear_sparse(to_dev(x, torch), packed, out["scales"], out["zeros"], out["row_ptr"], out["col"],
                              out["val"])
    ref = oracle.linear_ref(x, L["q"], L["s"], L["z"], L["row_ptr"], L["col"], L["val"])
    assert oracle.rel_err_inf(y.float().cpu().numpy(), ref) <= TOL


def test_empty_batch(gpu_lib):
    """M = 0 through the binding: an empty [0, N] result, with and without a CSR."""
    import torch
    L = oracle_layer(1)
    D = layer_to_dev(L, torch)
    x = torch.empty((0, L["q"].shape[1]), dtype=torch.float16, device="cuda")
    for sparse in (False, True):
        y = run_linear(gpu_lib, x, D, sparse=sparse)
        torch.cuda.synchronize()
        assert tuple(y.shape) == (0, L["q"].shape[0])


def test_sparse_split_under_graph_capture(gpu_lib):
    """A CSR product whose GEMM splits K (transpose, split GEMM, slice sum with the
    sparse term) captured in a CUDA graph: every replay equals the eager result,
    with eager calls and synchronizations between the replays."""
    import torch
    M, N, K = 200, 256, 4096
    W = workloads.random_weights(77, N, K)
    L = oracle.quantize_layer(W, N * K // 200)
    x = workloads.random_x(78, M, K)
    D = layer_to_dev(L, torch)
    xd = to_dev(x, torch)
    ws = torch.empty(gpu_lib.linear_workspace_bytes(M, N, K), dtype=torch.uint8, device="cuda")

    def call(out=None):
        return gpu_lib.linear_sparse(xd, D["packed"], D["scales"], D["zeros"], D["row_ptr"], D["col"], D["val"],
                                     out=out, workspace=ws)

    eager = call()
    torch.cuda.synchronize()
    ref = oracle.linear_ref(x, L["q"], L["s"], L["z"], L["row_ptr"], L["col"], L["val"])
    assert oracle.rel_err_inf(eager.float().cpu().numpy(), ref) <= TOL
    out = torch.empty_like(eager)
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        call(out)
    for i in range(4):
        say(f"[graph] replay {i}")
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), i
        again = call()
        torch.cuda.synchronize()
        assert torch.equal(again, eager), i


@pytest.mark.parametrize("N,K", [(300, 12288), (17, 14336), (1000, 16384), (40, 28672), (1, 12288)])
@pytest.mark.parametrize("sparse", [False, True])
def test_single_row_kernel(gpu_lib, N, K, sparse):
    """M = 1 with K a multiple of 2048 from 12288 on runs the single-row kernel
    (whole rows per wave, even and odd chunk counts, ragged N, a CSR term)."""
    import torch
    W = workloads.random_weights(N + K, N, K)
    L = oracle.quantize_layer(W, N * K // 250 if sparse else 0)
    x = workloads.random_x(N + 3 * K, 1, K)
    _full_check(gpu_lib, torch, L, x, "auto", sparse=sparse, label="single row")


@pytest.mark.parametrize("K", [12288, 14336, 28672])
def test_single_row_kernel_integer_exact(gpu_lib, K):
    """The integer-exact case through the single-row kernel: bit-identical fp32."""
    import torch
    N = 70
    x, q, s, z, rp, col, val = workloads.integer_case(K + 9, 1, N, K, nnz_per_row=7)
    L = dict(q=q, s=s, z=z, packed=oracle.pack(q), row_ptr=rp, col=col, val=val)
    D = layer_to_dev(L, torch)
    say(f"[exact single row] K={K}")
    y = run_linear(gpu_lib, to_dev(x, torch), D, kernel="gemv", out_dtype=torch.float32)
    ref = oracle.linear_ref(x, q, s, z, rp, col, val)
    assert np.array_equal(y.cpu().numpy().astype(np.float64), ref)


@pytest.mark.parametrize("M,N,K,kernel", [(1, 101, 4096, "gemv"), (7, 101, 4096, "gemv"), (1, 70, 12288, "gemv"),
                                          (64, 301, 4096, "gemm"), (200, 301, 1024, "gemm")])
@pytest.mark.parametrize("out_dtype", ["f16", "f32"])
def test_output_at_4_byte_offset(gpu_lib, M, N, K, kernel, out_dtype):
    """y 4 bytes past a 16-byte boundary (the least alignment the entry points
    accept) with M * N not a multiple of 4, through the block-staged, per-wave
    staging and single-row decode kernels and the split and large-M GEMMs (with a
    CSR term): right values, and nothing written outside y."""
    import torch
    dt = torch.float16 if out_dtype == "f16" else torch.float32
    off = 4 // dt.itemsize
    W = workloads.random_weights(N + K + M, N, K)
    L = oracle.quantize_layer(W, N * K // 200)
    x = workloads.random_x(M + 2 * N, M, K)
    D = layer_to_dev(L, torch)
    buf = torch.full((M * N + off + 3,), 7.0, dtype=dt, device="cuda")
    y = buf[off:off + M * N].view(M, N)
    say(f"[offset output] M={M} N={N} K={K} kernel={kernel} {out_dtype}")
    gpu_lib.linear_sparse(to_dev(x, torch), D["packed"], D["scales"], D["zeros"], D["row_ptr"], D["col"], D["val"],
                          out_dtype=dt, kernel=kernel, out=y)
    torch.cuda.synchronize()
    assert (buf[:off] == 7.0).all() and (buf[off + M * N:] == 7.0).all()
    ref = oracle.linear_ref(x, L["q"], L["s"], L["z"], L["row_ptr"], L["col"], L["val"])
    err = oracle.rel_err_inf(y.float().cpu().numpy(), ref)
    assert err <= TOL, err
