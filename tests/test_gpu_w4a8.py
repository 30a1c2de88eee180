"""W4A8 with fp16 outlier channels through wq_quantize_act_int8 and
wq_linear_w4a8: the INT8 activations, row scales and outlier values bit-exact
against the oracle, the product within the tolerance of the oracle's W4A8 product
(bit-identical on an integer-exact case), at ragged and full sizes."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_cases import f16_bits_host, rel_err_all_rows, say, to_dev

pytestmark = pytest.mark.gpu

# byte order of each 16 channels in the products' INT8 layout
ORDER16 = np.array([0, 2, 4, 6, 1, 3, 5, 7, 8, 10, 12, 14, 9, 11, 13, 15])


def device_order(xq):
    M, K = xq.shape
    return xq.reshape(M, K // 16, 16)[:, :, ORDER16].reshape(M, K)


def _layer(torch, wq, W):
    out = wq.quantize_rtn(to_dev(W, torch))
    return out, wq.pack(out["codes"])


@pytest.mark.parametrize("M,K,n_out", [(1, 4096, 8), (37, 1024, 8), (5, 384, 0), (130, 512, 16), (3, 128, 1)])
def test_act_int8_bit_exact(gpu_lib, M, K, n_out):
    import torch
    _, x, _ = workloads.make(4, M=M, N=64, K=K)
    outliers = np.random.default_rng(M + K).choice(K, n_out, replace=False).astype(np.int32)
    say(f"[act int8] M={M} K={K} n_out={n_out}")
    xq, sx, xo = gpu_lib.quantize_act_int8(to_dev(x, torch), to_dev(outliers, torch))
    torch.cuda.synchronize()
    rq, rs, ro = oracle.quantize_act_int8(x, outliers)
    assert np.array_equal(xq.cpu().numpy(), device_order(rq)), "xq"
    assert np.array_equal(sx.cpu().numpy().view(np.uint32), rs.view(np.uint32)), "s_x"
    pad = np.zeros((M, 16), np.float16)
    pad[:, :n_out] = ro
    assert np.array_equal(f16_bits_host(xo), pad.view(np.uint16)), "xo"


@pytest.mark.parametrize("M,N,K", [(1, 300, 1024), (37, 300, 1024), (128, 256, 512), (200, 130, 384),
                                   (300, 513, 2048)])
def test_w4a8_linear_parity(gpu_lib, M, N, K):
    import torch
    W, x, _ = workloads.make(4, M=M, N=N, K=K)
    outliers = workloads.x_outlier_channels(4, M=M, N=N, K=K)
    say(f"[w4a8] M={M} N={N} K={K} outliers={len(outliers)}")
    out, packed = _layer(torch, gpu_lib, W)
    y = gpu_lib.linear_w4a8(to_dev(x, torch), to_dev(outliers, torch), packed, out["scales"], out["zeros"],
                            out_dtype=torch.float32)
    torch.cuda.synchronize()
    L = oracle.quantize_layer(W)
    ref = oracle.linear_w4a8_ref(x, L["q"], L["s"], L["z"], outliers)
    err = oracle.rel_err_inf(y.cpu().numpy(), ref)
    say(f"    rel err {err:.3e}")
    assert err <= oracle.TOL, err
    # the outlier channels matter: without them in fp16 the result moves well beyond that
    assert oracle.rel_err_inf(oracle.linear_w4a8_ref(x, L["q"], L["s"], L["z"], []), ref) > 2 * oracle.TOL


def test_w4a8_integer_exact_fp32(gpu_lib):
    """Integer activations with a 127 in every row (s_x = 1, xq = x), integer
    outlier values, integer codes and zero-points with power-of-two scales: every
    partial sum is exact, so the fp32 output equals the oracle exactly."""
    import torch
    M, N, K = 40, 96, 512
    rng = np.random.default_rng(5)
    xi = rng.integers(-127, 128, size=(M, K))
    xi[:, 0] = 127
    outliers = np.array([3, 200, 511], np.int32)
    xi[:, outliers] = rng.integers(-60, 61, size=(M, 3))
    x = xi.astype(np.float16)
    q = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    G = K // 128
    s = (2.0 ** rng.integers(-8, -4, size=(N, G))).astype(np.float16)
    z = rng.integers(0, 16, size=(N, G)).astype(np.float16)
    y = gpu_lib.linear_w4a8(to_dev(x, torch), to_dev(outliers, torch), to_dev(oracle.pack(q), torch),
                            to_dev(s, torch), to_dev(z, torch), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().astype(np.float64), oracle.linear_w4a8_ref(x, q, s, z, outliers))


def test_w4a8_full_prefill_all_outputs(gpu_lib):
    """The prefill layer (2048 x 14336 x 4096) with its 8 outlier channels, every
    output compared (the oracle quantizes and multiplies a block of channels at a
    time)."""
    import torch
    W, x, _ = workloads.make(4)
    outliers = workloads.x_outlier_channels(4)
    out, packed = _layer(torch, gpu_lib, W)
    y = gpu_lib.linear_w4a8(to_dev(x, torch), to_dev(outliers, torch), packed, out["scales"], out["zeros"])
    torch.cuda.synchronize()

    def ref_rows(rows):
        L = oracle.quantize_layer(W[rows])
        return oracle.linear_w4a8_ref(x, L["q"], L["s"], L["z"], outliers)

    err = rel_err_all_rows(y, W.shape[0], ref_rows)
    say(f"[w4a8 full] rel err {err:.3e}")
    assert err <= oracle.TOL, err


def test_w4a8_empty_batch_and_determinism(gpu_lib):
    import torch
    W, x, _ = workloads.make(4, M=64, N=256, K=512)
    o = to_dev(workloads.x_outlier_channels(4, M=64, N=256, K=512), torch)
    out, packed = _layer(torch, gpu_lib, W)
    xd = to_dev(x, torch)
    a = gpu_lib.linear_w4a8(xd, o, packed, out["scales"], out["zeros"], out_dtype=torch.float32)
    b = gpu_lib.linear_w4a8(xd, o, packed, out["scales"], out["zeros"], out_dtype=torch.float32)
    e = gpu_lib.linear_w4a8(xd[:0], o, packed, out["scales"], out["zeros"])
    torch.cuda.synchronize()
    assert torch.equal(a, b) and tuple(e.shape) == (0, 256)
