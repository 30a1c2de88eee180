"""Per-wave staging decode kernel with each lane's scales and zero-points loaded
into registers per window of four groups (the block stages none): used from M = 3
on when every wave has one or two windows (2048 or 4096 input channels), for 4-bit
codes and for 3-bit codes in the 3-bit packing. Ragged N (a partial 16-channel
tile), M past one 16-row tile, and a CSR term, against the oracle; K = 8192 (four
windows, staged in LDS) alongside."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_cases import say, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("bits", [4, 3])
@pytest.mark.parametrize("K", [2048, 4096, 8192])
@pytest.mark.parametrize("N", [300, 1000])
@pytest.mark.parametrize("M", [3, 8, 16, 20, 33])
def test_decode_sz_in_registers(gpu_lib, bits, K, N, M):
    import torch
    W = workloads.random_weights(7 * K + N + M + bits, N, K)
    L = oracle.quantize_layer(W, N * K // 250, bits=bits)
    x = workloads.random_x(3 * K + M + bits, M, K)
    packed = oracle.pack3(L["q"]) if bits == 3 else oracle.pack(L["q"])
    say(f"[decode sz] bits={bits} K={K} N={N} M={M} nnz={len(L['col'])}")
    y = gpu_lib.linear_sparse(to_dev(x, torch), to_dev(packed, torch), to_dev(L["s"], torch), to_dev(L["z"], torch),
                              to_dev(L["row_ptr"], torch), to_dev(L["col"], torch), to_dev(L["val"], torch),
                              kernel="gemv")
    torch.cuda.synchronize()
    ref = oracle.linear_ref(x, L["q"], L["s"], L["z"], L["row_ptr"], L["col"], L["val"])
    ys = y.float().cpu().numpy()
    assert ys.shape == (M, N) and np.isfinite(ys).all()
    err = oracle.rel_err_inf(ys, ref)
    assert err <= oracle.TOL, err
