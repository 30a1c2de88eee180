"""A seeded sweep of random shapes and weight formats through the product entry
point, against the float64 oracle: 4-bit codes with 128-channel groups (twice as
often as the others), 3-bit codes, 64-channel groups, both; M from 1 to 200, N from
1 to 700, K from 128 to 28672 (a quarter of the cases single rows, half of those
long enough for the single-row kernel, K a multiple of 2048 up to 32768), CSR terms
from none to about 1 % of the weights, the kernel chosen by M or forced, fp16 or
fp32 output. Each case is printed before it runs, so a failure names its shape."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_cases import say, to_dev

pytestmark = pytest.mark.gpu

FORMATS = [(4, 128), (4, 128), (3, 128), (4, 64), (3, 64)]
MS = [1, 1, 2, 3, 5, 8, 13, 16, 17, 24, 33, 48, 64, 100, 200]
KS = [128, 256, 384, 640, 1024, 1152, 2048, 3584, 4096, 12288, 14336]
KS_LONG = [12288, 14336, 20480, 28672]
CASES = 80


def _case(i):
    rng = np.random.default_rng(9000 + i)
    bits, group = FORMATS[rng.integers(len(FORMATS))]
    M = 1 if rng.random() < 0.25 else int(MS[rng.integers(len(MS))])
    long_row = M == 1 and rng.random() < 0.5
    K = int(KS_LONG[rng.integers(len(KS_LONG))] if long_row else KS[rng.integers(len(KS))])
    n_max = max(1, min(700, 2_000_000 // K))
    N = int(rng.integers(1, n_max + 1))
    sparse_k = 0 if rng.random() < 0.35 else int(rng.integers(1, max(2, N * K // 100)))
    kernel = ["auto", "auto", "gemv", "gemm"][rng.integers(4)]
    f32 = bool(rng.random() < 0.3)
    return bits, group, M, N, K, sparse_k, kernel, f32


@pytest.mark.parametrize("i", range(CASES))
def test_random_shape_against_oracle(gpu_lib, i):
    import torch
    bits, group, M, N, K, sparse_k, kernel, f32 = _case(i)
    say(f"[sweep {i}] bits={bits} group={group} M={M} N={N} K={K} sparse_k={sparse_k} kernel={kernel} f32={f32}")
    W = workloads.random_weights(7000 + i, N, K)
    L = oracle.quantize_layer(W, sparse_k, group=group, bits=bits)
    x = workloads.random_x(8000 + i, M, K)
    packed = oracle.pack3(L["q"]) if bits == 3 else oracle.pack(L["q"])
    xd = to_dev(x, torch)
    dt = torch.float32 if f32 else torch.float16
    if sparse_k:
        y = gpu_lib.linear_sparse(xd, to_dev(packed, torch), to_dev(L["s"], torch), to_dev(L["z"], torch),
                                  to_dev(L["row_ptr"], torch), to_dev(L["col"], torch), to_dev(L["val"], torch),
                                  out_dtype=dt, kernel=kernel)
        ref = oracle.linear_ref(x, L["q"], L["s"], L["z"], L["row_ptr"], L["col"], L["val"], group=group)
    else:
        y = gpu_lib.linear(xd, to_dev(packed, torch), to_dev(L["s"], torch), to_dev(L["z"], torch), out_dtype=dt,
                           kernel=kernel)
        ref = oracle.linear_ref(x, L["q"], L["s"], L["z"], group=group)
    torch.cuda.synchronize()
    err = oracle.rel_err_inf(y.float().cpu().numpy(), ref)
    say(f"    rel err {err:.3e}")
    assert err <= oracle.TOL, err
