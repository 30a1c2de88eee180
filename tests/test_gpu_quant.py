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
