"""Act-order layers through wq_quantize_rtn_act_order and wq_linear_act_order:
the layer in permuted channel order bit-exact against the oracle quantizing
W[:, perm], its dense codes and metadata equal to the oracle's quantization with
scattered groups (a per-channel group index), and the product, fed activations
in the original order, against the oracle in both representations."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_cases import f16_bits_host, say, to_dev

pytestmark = pytest.mark.gpu


def _gidx(perm, group=128):
    g = np.empty(len(perm), np.int64)
    g[perm] = np.arange(len(perm)) // group
    return g


def _check_layer(out, L):
    assert np.array_equal(out["codes"].cpu().numpy(), L["q"]), "codes"
    assert np.array_equal(f16_bits_host(out["scales"]), L["s"].view(np.uint16)), "scales"
    assert np.array_equal(f16_bits_host(out["zeros"]), L["z"].view(np.uint16)), "zeros"
    assert np.array_equal(out["row_ptr"].cpu().numpy(), L["row_ptr"]), "row_ptr"
    if len(L["col"]):
        assert np.array_equal(out["col"].cpu().numpy(), L["col"]), "col"
        assert np.array_equal(f16_bits_host(out["val"]), L["val"].view(np.uint16)), "val"


@pytest.mark.parametrize("seed,N,K,sk", [(1, 37, 1024, 0), (2, 300, 640, 1500), (3, 5, 128, 0), (4, 64, 3584, 300)])
def test_act_order_quantize_bit_exact(gpu_lib, seed, N, K, sk):
    import torch
    W = workloads.random_weights(seed, N, K)
    perm = workloads.channel_permutation(seed + 100, K)
    say(f"[act-order quant] N,K={N},{K} sparse_k={sk}")
    out = gpu_lib.quantize_rtn_act_order(to_dev(W, torch), to_dev(perm, torch), sparse_k=sk)
    torch.cuda.synchronize()
    _check_layer(out, oracle.quantize_layer(W[:, perm], sk))
    if sk == 0:
        # the same layer as quantization with scattered groups, in the original order
        q, s, z = oracle.quantize_rtn_gidx(W, _gidx(perm))
        assert np.array_equal(out["codes"].cpu().numpy(), q[:, perm])
        assert np.array_equal(f16_bits_host(out["scales"]), s.view(np.uint16))
        assert np.array_equal(f16_bits_host(out["zeros"]), z.view(np.uint16))


def test_act_order_quantize_full_decode_layer(gpu_lib):
    import torch
    W, _, _ = workloads.make(2)
    perm = workloads.channel_permutation(7, W.shape[1])
    out = gpu_lib.quantize_rtn_act_order(to_dev(W, torch), to_dev(perm, torch))
    torch.cuda.synchronize()
    q, s, z = oracle.quantize_rtn_gidx(W, _gidx(perm))
    assert np.array_equal(out["codes"].cpu().numpy(), q[:, perm])
    assert np.array_equal(f16_bits_host(out["scales"]), s.view(np.uint16))
    assert np.array_equal(f16_bits_host(out["zeros"]), z.view(np.uint16))


@pytest.mark.parametrize("M,kernel", [(1, "auto"), (5, "auto"), (16, "auto"), (40, "auto"), (200, "auto"),
                                      (8, "gemm"), (70, "gemv")])
@pytest.mark.parametrize("sk", [0, 900])
def test_act_order_linear_parity(gpu_lib, M, kernel, sk):
    import torch
    N, K = 300, 1024
    W = workloads.random_weights(10 + M, N, K)
    x = workloads.random_x(20 + M, M, K)
    perm = workloads.channel_permutation(30 + M, K)
    pd = to_dev(perm, torch)
    say(f"[act-order linear] M={M} kernel={kernel} sparse_k={sk}")
    out = gpu_lib.quantize_rtn_act_order(to_dev(W, torch), pd, sparse_k=sk)
    packed = gpu_lib.pack(out["codes"])
    args = (out["row_ptr"], out["col"], out["val"]) if sk else (None, None, None)
    y = gpu_lib.linear_act_order(to_dev(x, torch), pd, packed, out["scales"], out["zeros"], *args,
                                 out_dtype=torch.float32, kernel=kernel)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    L = oracle.quantize_layer(W[:, perm], sk)
    ref = oracle.linear_ref(x[:, perm], L["q"], L["s"], L["z"],
                            *((L["row_ptr"], L["col"], L["val"]) if sk else (None, None, None)))
    err = oracle.rel_err_inf(y, ref)
    say(f"    rel err {err:.3e}")
    assert err <= oracle.TOL, err
    if sk == 0:
        q, s, z = oracle.quantize_rtn_gidx(W, _gidx(perm))
        assert oracle.rel_err_inf(y, oracle.linear_ref_gidx(x, q, s, z, _gidx(perm))) <= oracle.TOL


@pytest.mark.parametrize("M", [1, 2, 3])
def test_act_order_identity_permutation_is_the_plain_product(gpu_lib, M):
    """Bit for bit, through the decode kernel's two staging paths (M <= 2: the
    block stages all of x; M = 3: per wave and group)."""
    import torch
    N, K = 256, 512
    W = workloads.random_weights(51, N, K)
    x = to_dev(workloads.random_x(52, M, K), torch)
    ident = to_dev(np.arange(K, dtype=np.int32), torch)
    a = gpu_lib.quantize_rtn_act_order(to_dev(W, torch), ident, sparse_k=100)
    b = gpu_lib.quantize_rtn(to_dev(W, torch), sparse_k=100)
    packed = gpu_lib.pack(a["codes"])
    ya = gpu_lib.linear_act_order(x, ident, packed, a["scales"], a["zeros"], a["row_ptr"], a["col"], a["val"],
                                  out_dtype=torch.float32)
    yb = gpu_lib.linear_sparse(x, gpu_lib.pack(b["codes"]), b["scales"], b["zeros"], b["row_ptr"], b["col"],
                               b["val"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(a["codes"], b["codes"]) and torch.equal(ya, yb)
    e = gpu_lib.linear_act_order(x[:0], ident, packed, a["scales"], a["zeros"])
    torch.cuda.synchronize()
    assert tuple(e.shape) == (0, N)


@pytest.mark.parametrize("group", [256, -1])
def test_act_order_with_coarser_groups(gpu_lib, group):
    """Act-order with groups of 256 or one per row: the quantizer's group option
    applies to the permuted channels."""
    import torch
    N, K = 64, 1024
    g = K if group == -1 else group
    W = workloads.random_weights(61, N, K)
    perm = workloads.channel_permutation(62, K)
    out = gpu_lib.quantize_rtn_act_order(to_dev(W, torch), to_dev(perm, torch), group=group)
    torch.cuda.synchronize()
    q, s, z = oracle.quantize_rtn_gidx(W, _gidx(perm, g))
    assert np.array_equal(out["codes"].cpu().numpy(), q[:, perm])
    rep = g // oracle.GROUP
    assert np.array_equal(f16_bits_host(out["scales"]), np.repeat(s, rep, axis=1).view(np.uint16))
    assert np.array_equal(f16_bits_host(out["zeros"]), np.repeat(z, rep, axis=1).view(np.uint16))
