"""Bit-exact parity of the GPU split, quantizer and packer with the oracle."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_cases import f16_bits_host, oracle_layer, say, to_dev

pytestmark = pytest.mark.gpu


def _check_layer(wq, torch, L, label):
    W = L["W"]
    sk = L["sparse_k"]
    say(f"[quant] {label}: N,K={W.shape} sparse_k={sk}")
    Wd = to_dev(W, torch)
    out = wq.quantize_rtn(Wd, sparse_k=sk)
    packed = wq.pack(out["codes"])
    torch.cuda.synchronize()
    assert np.array_equal(out["codes"].cpu().numpy(), L["q"]), "codes"
    assert np.array_equal(f16_bits_host(out["scales"]), L["s"].view(np.uint16)), "scales"
    assert np.array_equal(f16_bits_host(out["zeros"]), L["z"].view(np.uint16)), "zeros"
    assert np.array_equal(packed.cpu().numpy().view(np.uint32), L["packed"]), "packed"
    assert np.array_equal(out["row_ptr"].cpu().numpy(), L["row_ptr"]), "row_ptr"
    if sk:
        assert np.array_equal(out["col"].cpu().numpy(), L["col"]), "col"
        assert np.array_equal(f16_bits_host(out["val"]), L["val"].view(np.uint16)), "val"


@pytest.mark.parametrize("index", [1, 2, 3, 4, 5])
def test_configs_bit_exact(gpu_lib, index):
    import torch
    _check_layer(gpu_lib, torch, oracle_layer(index), f"config {index}")


@pytest.mark.parametrize("seed,N,K,sk", [(1, 1, 128, 0), (2, 3, 384, 7), (3, 37, 256, 1), (4, 16, 128, 2048),
                                         (5, 300, 640, 1500), (6, 5, 128, 640)])
def test_small_shapes_bit_exact(gpu_lib, seed, N, K, sk):
    import torch
    W = workloads.random_weights(seed, N, K)
    L = oracle.quantize_layer(W, sk)
    L["W"], L["sparse_k"] = W, sk
    _check_layer(gpu_lib, torch, L, f"seed {seed}")


def test_ties_at_threshold(gpu_lib):
    """Many equal |w| straddle the selection threshold: lower flat index wins."""
    import torch
    rng = np.random.default_rng(77)
    W = (rng.integers(-6, 7, size=(40, 256)) * 0.125).astype(np.float32)
    for sk in (1, 100, 1001, 5000, 40 * 256):
        L = oracle.quantize_layer(W, sk)
        L["W"], L["sparse_k"] = W, sk
        _check_layer(gpu_lib, torch, L, f"ties sk={sk}")


def test_on_grid_and_degenerate_groups(gpu_lib):
    import torch
    rng = np.random.default_rng(9)
    N, G = 6, 3
    e = rng.integers(-14, -1, size=(N, G))
    s16 = ((1 + rng.integers(0, 1024, size=(N, G)) / 1024.0) * 2.0 ** e).astype(np.float16)
    z = rng.integers(0, 16, size=(N, G))
    q = rng.integers(0, 16, size=(N, G, 128))
    q[:, :, 0], q[:, :, 1] = 0, 15
    W = ((q - z[:, :, None]).astype(np.float32) * s16.astype(np.float32)[:, :, None]).reshape(N, -1)
    W[0, :128] = 0.0          # all-zero group
    W[1, 128:256] = 0.5       # constant group
    W[2, :128] = -np.abs(W[2, :128]) - 1.0   # all negative
    L = oracle.quantize_layer(W.astype(np.float32), 0)
    L["W"], L["sparse_k"] = W.astype(np.float32), 0
    _check_layer(gpu_lib, torch, L, "on-grid")
    got = gpu_lib.quantize_rtn(to_dev(W.astype(np.float32), torch))
    assert np.array_equal(got["codes"].cpu().numpy().reshape(N, G, 128)[3:], q[3:].astype(np.uint8))


def test_quantize_is_deterministic(gpu_lib):
    import torch
    L = oracle_layer(3)
    Wd = to_dev(L["W"], torch)
    a = gpu_lib.quantize_rtn(Wd, sparse_k=L["sparse_k"])
    b = gpu_lib.quantize_rtn(Wd, sparse_k=L["sparse_k"])
    for k in a:
        assert torch.equal(a[k], b[k]), k


# ---------------------------------------------------------------- coarser groups
@pytest.mark.parametrize("seed,N,K,group,sk", [
    (31, 37, 1024, 256, 0), (32, 37, 1024, 512, 200), (33, 16, 1024, -1, 0),
    (34, 300, 640, -1, 1500), (35, 5, 384, 384, 0), (36, 64, 3584, 512, 0),
])
def test_coarse_groups_bit_exact(gpu_lib, seed, N, K, group, sk):
    """Groups of 256..K channels (-1: one per row): codes bit-exact against the
    oracle quantizing with that group, and each group's (s, z) repeated over its
    128-channel metadata slots."""
    import torch
    g = K if group == -1 else group
    W = workloads.random_weights(seed, N, K)
    L = oracle.quantize_layer(W, sk, group=g)
    say(f"[quant coarse] N,K={N},{K} group={group} sparse_k={sk}")
    out = gpu_lib.quantize_rtn(to_dev(W, torch), sparse_k=sk, group=group)
    torch.cuda.synchronize()
    assert np.array_equal(out["codes"].cpu().numpy(), L["q"]), "codes"
    rep = g // oracle.GROUP
    assert np.array_equal(f16_bits_host(out["scales"]), np.repeat(L["s"], rep, axis=1).view(np.uint16)), "scales"
    assert np.array_equal(f16_bits_host(out["zeros"]), np.repeat(L["z"], rep, axis=1).view(np.uint16)), "zeros"
    assert np.array_equal(out["row_ptr"].cpu().numpy(), L["row_ptr"]), "row_ptr"
    if sk:
        assert np.array_equal(out["col"].cpu().numpy(), L["col"]), "col"
        assert np.array_equal(f16_bits_host(out["val"]), L["val"].view(np.uint16)), "val"


def test_per_row_groups_full_decode_layer(gpu_lib):
    """One group per row on the 7B up-projection layer [11008, 4096]."""
    import torch
    W, _, _ = workloads.make(2)
    L = oracle.quantize_layer(W, 0, group=W.shape[1])
    out = gpu_lib.quantize_rtn(to_dev(W, torch), group=-1)
    torch.cuda.synchronize()
    assert np.array_equal(out["codes"].cpu().numpy(), L["q"]), "codes"
    assert np.array_equal(f16_bits_host(out["scales"]), np.repeat(L["s"], 32, axis=1).view(np.uint16)), "scales"
    assert np.array_equal(f16_bits_host(out["zeros"]), np.repeat(L["z"], 32, axis=1).view(np.uint16)), "zeros"


@pytest.mark.parametrize("group", [256, -1])
@pytest.mark.parametrize("M", [1, 8, 100])
def test_coarse_group_linear_parity(gpu_lib, group, M):
    """The linear product on coarse-group metadata (GEMV at M = 1, 8, GEMM at
    100, with a CSR) against the oracle dequantizing with the true group."""
    import torch
    N, K, sk = 300, 1024, 600
    g = K if group == -1 else group
    W = workloads.random_weights(41 + M, N, K)
    x = workloads.random_x(42 + M, M, K)
    L = oracle.quantize_layer(W, sk, group=g)
    say(f"[coarse linear] group={group} M={M}")
    out = gpu_lib.quantize_rtn(to_dev(W, torch), sparse_k=sk, group=group)
    packed = gpu_lib.pack(out["codes"])
    y = gpu_lib.linear_sparse(to_dev(x, torch), packed, out["scales"], out["zeros"], out["row_ptr"], out["col"],
                              out["val"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.linear_ref(x, L["q"], L["s"], L["z"], L["row_ptr"], L["col"], L["val"], group=g)
    err = oracle.rel_err_inf(y.cpu().numpy(), ref)
    say(f"    rel err {err:.3e}")
    assert err <= oracle.TOL, err


# ---------------------------------------------------------------- fewer bits
@pytest.mark.parametrize("bits,seed,N,K,group,sk", [(3, 41, 37, 1024, 128, 0), (3, 42, 300, 640, 128, 1500),
                                                    (2, 43, 64, 512, 128, 0), (3, 44, 16, 1024, -1, 100)])
def test_fewer_bits_bit_exact_and_product(gpu_lib, bits, seed, N, K, group, sk):
    """3- and 2-bit codes (in the 4-bit packing) bit-exact against the oracle,
    and the unchanged products (GEMV and GEMM) on them against the oracle."""
    import torch
    g = K if group == -1 else group
    W = workloads.random_weights(seed, N, K)
    L = oracle.quantize_layer(W, sk, group=g, bits=bits)
    say(f"[bits] bits={bits} N,K={N},{K} group={group} sparse_k={sk}")
    out = gpu_lib.quantize_rtn(to_dev(W, torch), sparse_k=sk, group=group, bits=bits)
    packed = gpu_lib.pack(out["codes"])
    torch.cuda.synchronize()
    assert out["codes"].max().item() <= (1 << bits) - 1
    assert np.array_equal(out["codes"].cpu().numpy(), L["q"]), "codes"
    rep = g // oracle.GROUP
    assert np.array_equal(f16_bits_host(out["scales"]), np.repeat(L["s"], rep, axis=1).view(np.uint16)), "scales"
    assert np.array_equal(f16_bits_host(out["zeros"]), np.repeat(L["z"], rep, axis=1).view(np.uint16)), "zeros"
    for M in (1, 100):
        x = workloads.random_x(seed + M, M, K)
        args = (out["row_ptr"], out["col"], out["val"]) if sk else (None, None, None)
        y = gpu_lib.linear_sparse(to_dev(x, torch), packed, out["scales"], out["zeros"], *args,
                                  out_dtype=torch.float32)
        torch.cuda.synchronize()
        rargs = (L["row_ptr"], L["col"], L["val"]) if sk else (None, None, None)
        ref = oracle.linear_ref(x, L["q"], L["s"], L["z"], *rargs, group=g)
        err = oracle.rel_err_inf(y.cpu().numpy(), ref)
        assert err <= oracle.TOL, (M, err)
