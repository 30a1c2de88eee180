"""Parity of the other weight formats with the oracle: 3-bit codes in the 3-bit
packing (oracle.pack3) and one (s, z) per 64 input channels, each alone and
together. Codes, metadata and packed words bit-exact; products through the decode
kernels (block-staged at M <= 2, per-wave staging above) and the tile GEMM, with and
without a CSR term, within the tolerance, and bit-identical fp32 on integer-exact
inputs."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_cases import f16_bits_host, oracle_layer, rel_err_all_rows, say, to_dev

pytestmark = pytest.mark.gpu

FORMATS = [(3, 128), (4, 64), (3, 64)]


def _packed(q, bits):
    return oracle.pack3(q) if bits == 3 else oracle.pack(q)


def _dev_layer(torch, L, bits):
    return dict(packed=to_dev(_packed(L["q"], bits), torch), scales=to_dev(L["s"], torch), zeros=to_dev(L["z"], torch),
                row_ptr=to_dev(L["row_ptr"], torch), col=to_dev(L["col"], torch), val=to_dev(L["val"], torch))


def _run(wq, torch, D, x, kernel="auto", sparse=True, out_dtype=None):
    xd = to_dev(x, torch)
    if sparse:
        return wq.linear_sparse(xd, D["packed"], D["scales"], D["zeros"], D["row_ptr"], D["col"], D["val"],
                                kernel=kernel, out_dtype=out_dtype)
    return wq.linear(xd, D["packed"], D["scales"], D["zeros"], kernel=kernel, out_dtype=out_dtype)


@pytest.mark.parametrize("bits,group", FORMATS + [(4, 128)])
@pytest.mark.parametrize("N,K,sk", [(300, 1024, 1500), (97, 3584, 0)])
def test_quantize_and_pack_bit_exact(gpu_lib, bits, group, N, K, sk):
    import torch
    W = workloads.random_weights(N + K + bits + group, N, K)
    L = oracle.quantize_layer(W, sk, group=group, bits=bits)
    say(f"[formats quantize] bits={bits} group={group} N={N} K={K} sparse_k={sk}")
    out = gpu_lib.quantize_rtn(to_dev(W, torch), sparse_k=sk, group=group, bits=bits)
    packed = gpu_lib.pack(out["codes"], bits=bits)
    torch.cuda.synchronize()
    assert tuple(out["scales"].shape) == (N, K // group)
    assert np.array_equal(out["codes"].cpu().numpy(), L["q"])
    assert np.array_equal(f16_bits_host(out["scales"]), L["s"].view(np.uint16))
    assert np.array_equal(f16_bits_host(out["zeros"]), L["z"].view(np.uint16))
    assert np.array_equal(out["col"].cpu().numpy(), L["col"])
    assert np.array_equal(packed.cpu().numpy().view(np.uint32), _packed(L["q"], bits))


def test_pack3_full_decode_layer(gpu_lib):
    """The 7B up-projection quantized to 3 bits: GPU codes and 3-bit words equal the
    oracle's on all 45 M weights (0.375 bytes per weight: 16.9 MB of words)."""
    import torch
    W, _, _ = workloads.make(2)
    L = oracle.quantize_layer(W, 0, bits=3)
    out = gpu_lib.quantize_rtn(to_dev(W, torch), bits=3)
    packed = gpu_lib.pack(out["codes"], bits=3)
    torch.cuda.synchronize()
    p = packed.cpu().numpy().view(np.uint32)
    assert p.nbytes == W.size * 3 // 8
    assert np.array_equal(p, oracle.pack3(L["q"]))


@pytest.mark.parametrize("bits,group", FORMATS)
@pytest.mark.parametrize("M", [1, 2, 3, 8, 16, 17, 64, 130])
@pytest.mark.parametrize("sparse", [False, True])
def test_formats_ragged(gpu_lib, bits, group, M, sparse):
    import torch
    N, K = 300, 640
    W = workloads.random_weights(40 + M + bits, N, K)
    L = oracle.quantize_layer(W, 900 if sparse else 0, group=group, bits=bits)
    x = workloads.random_x(50 + M, M, K)
    D = _dev_layer(torch, L, bits)
    for kernel in ("auto", "gemv", "gemm"):
        say(f"[formats] bits={bits} group={group} M={M} sparse={sparse} kernel={kernel}")
        y = _run(gpu_lib, torch, D, x, kernel, sparse)
        torch.cuda.synchronize()
        args = (L["row_ptr"], L["col"], L["val"]) if sparse else (None, None, None)
        ref = oracle.linear_ref(x, L["q"], L["s"], L["z"], *args, group=group)
        err = oracle.rel_err_inf(y.float().cpu().numpy(), ref)
        assert err <= oracle.TOL, (kernel, err)


@pytest.mark.parametrize("bits,group", FORMATS)
@pytest.mark.parametrize("K", [1024, 3584, 2816, 16896])
@pytest.mark.parametrize("M", [1, 2, 5, 16])
def test_formats_decode_staging(gpu_lib, bits, group, K, M):
    """Decode kernels with (s, z) staged as vectors (K/group a multiple of 8, up to
    256 per row) and by the plain loop (44 or 264 per row with 64-channel groups),
    block-staged activations with (s, z) in registers (K = 1024 is eight groups, so
    staged), ragged N and a CSR term."""
    import torch
    N = 300 if K <= 4096 else 40
    W = workloads.random_weights(K + M + bits + group, N, K)
    L = oracle.quantize_layer(W, N * K // 300, group=group, bits=bits)
    x = workloads.random_x(K + 5 * M, M, K)
    D = _dev_layer(torch, L, bits)
    say(f"[formats staging] bits={bits} group={group} M={M} K={K}")
    y = _run(gpu_lib, torch, D, x, "gemv")
    torch.cuda.synchronize()
    ref = oracle.linear_ref(x, L["q"], L["s"], L["z"], L["row_ptr"], L["col"], L["val"], group=group)
    err = oracle.rel_err_inf(y.float().cpu().numpy(), ref)
    assert err <= oracle.TOL, err


@pytest.mark.parametrize("bits,group", FORMATS)
@pytest.mark.parametrize("M,kernel", [(1, "gemv"), (2, "gemv"), (16, "gemv"), (40, "gemm"), (200, "gemm"),
                                      (16, "gemm"), (40, "gemv")])
def test_formats_integer_exact_fp32(gpu_lib, bits, group, M, kernel):
    """Power-of-two scales, integer zero-points, activations and sparse values,
    codes of `bits` bits: every partial sum is exact in fp32, so y is bit-identical
    (one and two 128-channel tiles per K step, a split and an unsplit GEMM)."""
    import torch
    N, K = 96, 4096 if M == 40 else 1024
    x, q, s, z, rp, col, val = workloads.integer_case(M + bits + group, M, N, K, nnz_per_row=5, group=group)
    if bits == 3:
        q = q & 7
        z = np.minimum(z, 7).astype(np.float16)
    L = dict(q=q, s=s, z=z, row_ptr=rp, col=col, val=val)
    D = _dev_layer(torch, L, bits)
    say(f"[formats exact] bits={bits} group={group} M={M} kernel={kernel}")
    y = _run(gpu_lib, torch, D, x, kernel, out_dtype=torch.float32)
    ref = oracle.linear_ref(x, q, s, z, rp, col, val, group=group)
    assert np.array_equal(y.cpu().numpy().astype(np.float64), ref)


@pytest.mark.parametrize("bits,group", FORMATS)
@pytest.mark.parametrize("index,M", [(2, 1), (3, 16), (5, 8), (4, 2048)])
def test_formats_full_size_all_outputs(gpu_lib, bits, group, index, M):
    """Full-size layers in each format, every output compared: the 7B decode layer,
    the batched decode layer with its CSR, the 70B down-projection at M = 8 with its
    CSR, and the prefill layer (tile GEMM)."""
    import torch
    W, x, cfg = workloads.make(index, M=M)
    N, K = W.shape
    sk = workloads.sparse_k_for(cfg, N, K)
    L = oracle.quantize_layer(W, sk, group=group, bits=bits)
    out = gpu_lib.quantize_rtn(to_dev(W, torch), sparse_k=sk, group=group, bits=bits)
    packed = gpu_lib.pack(out["codes"], bits=bits)
    xd = to_dev(x, torch)
    say(f"[formats full] config {index} M={M} bits={bits} group={group}")
    if sk:
        y = gpu_lib.linear_sparse(xd, packed, out["scales"], out["zeros"], out["row_ptr"], out["col"], out["val"])
    else:
        y = gpu_lib.linear(xd, packed, out["scales"], out["zeros"])
    torch.cuda.synchronize()
    args = (L["row_ptr"], L["col"], L["val"]) if sk else (None, None, None)
    err = rel_err_all_rows(y, N, lambda rows: oracle.linear_rows(x, L["q"], L["s"], L["z"], rows, *args,
                                                                 group=group))
    say(f"    rel err {err:.3e}")
    assert err <= oracle.TOL, err
