"""Shared helpers for the GPU parity tests (imported by test_gpu_*.py).

Expected values always come from the oracle on the CPU; the GPU receives the
same seeded inputs (and, for the linear layer, the oracle's quantized tensors).
"""
import functools
import sys

import numpy as np

import oracle
import workloads


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=None)
def oracle_layer(index, N=None, K=None):
    """Seeded weights of a configuration and their oracle quantization."""
    W, _, cfg = workloads.make(index, M=1, N=N, K=K)
    n, k = W.shape
    sk = workloads.sparse_k_for(cfg, n, k)
    L = oracle.quantize_layer(W, sk)
    L["W"] = W
    L["sparse_k"] = sk
    return L


def to_dev(a, torch):
    """numpy -> device tensor with the dtypes the binding expects."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    if a.dtype == np.float16:
        return torch.from_numpy(a.view(np.int16).copy()).cuda().view(torch.float16)
    return torch.from_numpy(a.copy()).cuda()


def f16_bits_host(t):
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def layer_to_dev(L, torch):
    return dict(packed=to_dev(L["packed"], torch), scales=to_dev(L["s"], torch), zeros=to_dev(L["z"], torch),
                row_ptr=to_dev(L["row_ptr"], torch), col=to_dev(L["col"], torch), val=to_dev(L["val"], torch))


def run_linear(wq, xd, D, kernel="auto", out_dtype=None, sparse=True):
    if sparse:
        return wq.linear_sparse(xd, D["packed"], D["scales"], D["zeros"], D["row_ptr"], D["col"], D["val"],
                                out_dtype=out_dtype, kernel=kernel)
    return wq.linear(xd, D["packed"], D["scales"], D["zeros"], out_dtype=out_dtype, kernel=kernel)


def sample_rows(N, count, seed, tile=128):
    """Output channels to check one by one: at least one in every ``tile``-wide
    column tile (the narrowest tile any product kernel uses), ``count`` more drawn
    at random, and the edges."""
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(N, min(count, N), replace=False).tolist())
    rows |= {0, N - 1, min(15, N - 1), min(16, N - 1)}
    for t0 in range(0, N, tile):
        rows.add(int(rng.integers(t0, min(N, t0 + tile))))
    rows = np.array(sorted(rows))
    assert set((rows // tile).tolist()) == set(range((N + tile - 1) // tile)), "a column tile is not sampled"
    return rows


def rel_err_all_rows(y, N, ref_rows, chunk=1024):
    """max |y - y_ref| / max |y_ref| over EVERY output channel of y [M, N], with the
    oracle's reference computed ``chunk`` channels at a time (``ref_rows(rows)``
    returns float64 [M, len(rows)]), so that memory stays bounded at full size."""
    ys = y.float().cpu().numpy() if hasattr(y, "cpu") else np.asarray(y, np.float64)
    assert np.isfinite(ys).all()
    num = den = 0.0
    seen = np.zeros(N, bool)
    for a in range(0, N, chunk):
        rows = np.arange(a, min(N, a + chunk))
        ref = ref_rows(rows)
        num = max(num, float(np.max(np.abs(ys[:, rows] - ref))))
        den = max(den, float(np.max(np.abs(ref))))
        seen[rows] = True
    assert seen.all(), "an output channel was not compared"
    return num / den if den else num
