"""Pins for the CPU oracle, checked against what the pages and mathematics fix.

None of these tests re-types the oracle's formulas: each checks a property
that a plausible mistake (dropped zero-point, wrong sign, wrong group index,
transposed operand, wrong nibble order, wrong tie-break) would break.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f16_bits(a):
    return np.asarray(a, dtype=np.float16).view(np.uint16)


# ---------------------------------------------------------------- packing
def test_pack_hand_words():
    # codes 0..7 along K land in nibbles 0..7: the word reads 0x76543210
    q = np.arange(8, dtype=np.uint8)[None, :]
    assert oracle.pack(q)[0, 0] == 0x76543210
    q = np.array([[15, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 1]], np.uint8)
    w = oracle.pack(q)
    assert w[0, 0] == 0x0000000F and w[0, 1] == 0x10000000
    q = np.full((2, 8), 0xA, np.uint8)
    q[1] = [1, 2, 3, 4, 5, 6, 7, 8]
    assert list(oracle.pack(q)[:, 0]) == [0xAAAAAAAA, 0x87654321]


def test_pack_roundtrip():
    rng = np.random.default_rng(1)
    q = rng.integers(0, 16, size=(7, 256), dtype=np.uint8)
    p = oracle.pack(q)
    assert p.shape == (7, 32) and p.dtype == np.uint32
    assert np.array_equal(oracle.unpack(p), q)
    # nibble i of word t is code 8t+i, checked with plain integer division
    for n, t, i in [(0, 0, 0), (3, 5, 7), (6, 31, 3)]:
        assert (int(p[n, t]) // 16 ** i) % 16 == q[n, 8 * t + i]


# ---------------------------------------------------------------- quantizer
def _on_grid(seed, N, G, group=128):
    """Weights already on a quantization grid: w = (q - z) * s with s a normal
    fp16, z in [0, 15] and every group holding codes 0 and 15."""
    rng = np.random.default_rng(seed)
    e = rng.integers(-14, -1, size=(N, G))
    m = rng.integers(0, 1024, size=(N, G))
    s16 = ((1.0 + m / 1024.0) * 2.0 ** e).astype(np.float16)
    z = rng.integers(0, 16, size=(N, G))
    q = rng.integers(0, 16, size=(N, G, group))
    for n in range(N):
        for g in range(G):
            a, b = rng.choice(group, 2, replace=False)
            q[n, g, a] = 0
            q[n, g, b] = 15
    s32 = s16.astype(np.float32)
    w = ((q - z[:, :, None]).astype(np.float32) * s32[:, :, None]).astype(np.float32)
    return w.reshape(N, G * group), q.reshape(N, G * group).astype(np.uint8), s16, z


@pytest.mark.parametrize("seed,N,G,group", [(0, 3, 1, 128), (1, 8, 4, 128), (2, 5, 7, 128), (3, 6, 8, 64)])
def test_on_grid_exact_recovery(seed, N, G, group):
    w, q, s16, z = _on_grid(seed, N, G, group)
    # the construction is exact in float32
    assert np.array_equal(((q.reshape(N, G, group) - z[:, :, None]) *
                           s16.astype(np.float64)[:, :, None]).reshape(N, -1), w.astype(np.float64))
    q2, s2, z2 = oracle.quantize_rtn(w, group)
    assert np.array_equal(f16_bits(s2), f16_bits(s16))
    assert np.array_equal(z2.astype(np.int64), z)
    assert np.array_equal(q2, q)


def test_golden_hand_cases():
    with open(os.path.join(GOLDEN, "rtn_hand_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        g = np.full(128, c["fill"], np.float32)
        for k, v in c["entries"].items():
            g[int(k)] = v
        q, s, z = oracle.quantize_rtn(g[None, :])
        assert f16_bits(s)[0, 0] == int(c["scale_bits"], 16), c["name"]
        assert f16_bits(z)[0, 0] == int(c["zero_bits"], 16), c["name"]
        for k in range(128):
            want = c["codes"].get(str(k), c["fill_code"])
            assert q[0, k] == want, (c["name"], k)


def _cfg1_small():
    W, x, cfg = workloads.make(1)
    return W, x


def test_zero_dequantizes_to_exact_zero():
    W, _ = _cfg1_small()
    W = W.copy()
    rng = np.random.default_rng(5)
    W.reshape(-1)[rng.choice(W.size, 4000, replace=False)] = 0.0
    q, s, z = oracle.quantize_rtn(W)
    w_hat = oracle.dequant(q, s, z)
    assert np.all(w_hat[W == 0.0] == 0.0)


def test_group_minimum_gets_code_zero():
    W, _ = _cfg1_small()
    q, s, z = oracle.quantize_rtn(W)
    N, K = W.shape
    G = K // 128
    Wg = W.reshape(N, G, 128)
    qg = q.reshape(N, G, 128)
    amin = Wg.argmin(axis=2)
    for n in range(N):
        for g in range(G):
            zz = int(z[n, g])
            if 0 < zz < 15:
                assert qg[n, g, amin[n, g]] == 0


@pytest.mark.parametrize("group,bits", [(128, 4), (256, 4), (128, 3), (256, 3), (128, 2), (64, 4), (64, 3)])
def test_brute_force_exact_rationals(group, bits):
    """Each code is the nearest grid point in exact arithmetic; the scale is the
    fp16 nearest to range/qmax (qmax = 2^bits - 1) and the zero-point the
    nearest integer to -min/s, with min and max over the group (at 256 channels,
    one group per row)."""
    qmax = (1 << bits) - 1
    W = workloads.random_weights(11, 4, 256, sigma=0.02)
    W[1, 5] *= 20
    W[2, 200] *= -20
    W[3, 0:128] = np.abs(W[3, 0:128])          # an all-positive group (clamped z)
    q, s, z = oracle.quantize_rtn(W, group, bits)
    assert s.shape == (4, 256 // group) and q.max() <= qmax
    near_half = []
    for n in range(W.shape[0]):
        for g in range(256 // group):
            grp = [Fraction(float(v)) for v in W[n, group * g:group * g + group]]
            mn, mx = min(grp), max(grp)
            S = Fraction(float(s[n, g]))
            Z = int(z[n, g])
            # scale: within half an fp16 ulp of the exact range/qmax (plus the
            # float32 rounding of the range and quotient)
            exact = (mx - mn) / qmax
            ulp = Fraction(2) ** (int(np.floor(np.log2(float(S)))) - 10)
            assert abs(S - exact) <= ulp / 2 + exact * Fraction(1, 2 ** 22)
            # zero-point: nearest integer to -mn/S, clamped to [0, 15]
            zc = min(qmax, max(0, round(-mn / S)))
            assert Z == zc
            for k, w in enumerate(grp):
                errs = [abs(w - (c - Z) * S) for c in range(qmax + 1)]
                best = min(errs)
                winners = {c for c in range(qmax + 1) if errs[c] == best}
                qq = int(q[n, group * g + k])
                if qq not in winners:
                    frac = (w / S) - int(w / S)
                    near_half.append((n, g, k, float(frac)))
    assert near_half == []


def test_rounding_error_bound_full_config1():
    W, _ = _cfg1_small()
    q, s, z = oracle.quantize_rtn(W)
    w_hat = oracle.dequant(q, s, z)
    S = np.repeat(s.astype(np.float64), 128, axis=1)
    inner = (q > 0) & (q < 15)
    err = np.abs(w_hat - W.astype(np.float64))
    # RTN: interior codes are within half a step (plus float32 quotient rounding)
    assert np.all(err[inner] <= S[inner] * (0.5 + 2.0 ** -20))
    # outlier-free groups keep every weight within half a step of the grid
    assert np.max(err / S) <= 0.5 + 2.0 ** -20 or np.any(~inner)


# ---------------------------------------------------------------- split
def _tie_heavy(seed, N, K):
    rng = np.random.default_rng(seed)
    W = (rng.integers(-8, 9, size=(N, K)) * 0.25).astype(np.float32)
    return W


@pytest.mark.parametrize("seed,N,K,k", [(0, 4, 16, 5), (1, 6, 24, 17), (2, 3, 40, 1),
                                        (3, 5, 32, 0), (4, 2, 16, 32)])
def test_split_matches_full_stable_sort(seed, N, K, k):
    W = _tie_heavy(seed, N, K)
    Wd, row_ptr, col, val = oracle.split_outliers(W, k)
    flat = W.reshape(-1)
    order = sorted(range(flat.size), key=lambda i: (-abs(float(flat[i])), i))
    chosen = sorted(order[:k])
    got = [int(r) * K + int(c) for r in range(N) for c in col[row_ptr[r]:row_ptr[r + 1]]]
    assert got == chosen
    assert row_ptr[0] == 0 and row_ptr[-1] == k and np.all(np.diff(row_ptr) >= 0)
    for r in range(N):
        seg = col[row_ptr[r]:row_ptr[r + 1]]
        assert np.all(np.diff(seg) > 0)
    assert np.array_equal(val.astype(np.float32), flat[chosen].astype(np.float16).astype(np.float32))
    dense = Wd.reshape(-1)
    assert np.all(dense[chosen] == 0) and not np.any(np.signbit(dense[chosen]))
    rest = np.setdiff1d(np.arange(flat.size), chosen)
    assert np.array_equal(dense[rest], flat[rest])


def test_split_partition_invariants_config3_shape():
    W = workloads.random_weights(3000, 256, 512)
    k = workloads.sparse_k_for(workloads.CONFIGS[3], 256, 512)
    Wd, row_ptr, col, val = oracle.split_outliers(W, k)
    sel = np.zeros(W.shape, bool)
    rows = np.repeat(np.arange(256), np.diff(row_ptr))
    sel[rows, col] = True
    assert sel.sum() == k == 589
    assert np.abs(W[sel]).min() >= np.abs(W[~sel]).max()
    recomposed = Wd.astype(np.float64)
    recomposed[rows, col] += val.astype(np.float64)
    diff = np.abs(recomposed - W)
    assert np.all(diff[~sel] == 0)
    assert np.all(diff[sel] <= np.abs(W[sel]) * 2.0 ** -11)


def test_config_sizes():
    c = workloads.CONFIGS
    assert c[1].n_planted == 1310 and c[2].n_planted == 45088
    assert c[3].sparse_k == 75497 and c[5].sparse_k == 117440
    assert c[1].sparse_k == c[2].sparse_k == c[4].sparse_k == 0


def test_generator_is_seeded():
    W1, x1, _ = workloads.make(1)
    W2, x2, _ = workloads.make(1)
    assert np.array_equal(W1, W2) and np.array_equal(x1.view(np.uint16), x2.view(np.uint16))
    assert W1.dtype == np.float32 and x1.dtype == np.float16
    assert (np.abs(W1) > 0.1).sum() > 900           # the planted x20 outliers (5 sigma otherwise)
    W4, x4, _ = workloads.make(4, M=4, N=8, K=256)
    big = np.flatnonzero(np.abs(x4.astype(np.float32)).max(axis=0) > 10)
    assert 1 <= big.size <= 8


# ---------------------------------------------------------------- linear
def _exact_linear(x, q, s, z, row_ptr, col, val):
    M, K = x.shape
    N = q.shape[0]
    out = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                g = k // 128
                acc += Fraction(float(x[m, k])) * (int(q[n, k]) - int(z[n, g])) * Fraction(float(s[n, g]))
            for e in range(row_ptr[n], row_ptr[n + 1]):
                acc += Fraction(float(val[e])) * Fraction(float(x[m, col[e]]))
            out[m][n] = acc
    return out


def test_linear_brute_force_rationals():
    M, N, K = 3, 5, 256
    W = workloads.random_weights(21, N, K)
    x = workloads.random_x(22, M, K)
    L = oracle.quantize_layer(W, sparse_k=9)
    y = oracle.linear_ref(x, L["packed"], L["s"], L["z"], L["row_ptr"], L["col"], L["val"])
    assert y.shape == (M, N)
    ex = _exact_linear(x, L["q"], L["s"], L["z"], L["row_ptr"], L["col"], L["val"])
    for m in range(M):
        for n in range(N):
            assert abs(y[m, n] - float(ex[m][n])) <= 1e-12 * max(1.0, abs(float(ex[m][n])))


def test_one_hot_x_reads_a_column_of_w_hat():
    N, K = 6, 384
    W = workloads.random_weights(31, N, K)
    q, s, z = oracle.quantize_rtn(W)
    for k in (0, 127, 128, 300):
        x = np.zeros((1, K), np.float16)
        x[0, k] = 1.0
        y = oracle.linear_ref(x, q, s, z)
        g = k // 128
        want = [(int(q[n, k]) - int(z[n, g])) * float(s[n, g]) for n in range(N)]
        assert np.array_equal(y[0], np.array(want))


def test_integer_case_is_exact():
    x, q, s, z, rp, col, val = workloads.integer_case(7, 4, 6, 512, nnz_per_row=3)
    y = oracle.linear_ref(x, oracle.pack(q), s, z, rp, col, val)
    # the same sum in integers: scales are 2^-e, so 16 * y is an integer
    xi = x.astype(np.int64)
    s16 = (s.astype(np.float64) * 16).astype(np.int64)
    W16 = (q.astype(np.int64).reshape(6, 4, 128) - z.astype(np.int64)[:, :, None]) * s16[:, :, None]
    y16 = xi @ W16.reshape(6, 512).T
    for n in range(6):
        for e in range(rp[n], rp[n + 1]):
            y16[:, n] += 16 * int(val[e]) * xi[:, col[e]]
    assert np.array_equal(y * 16, y16.astype(np.float64))


def test_decomposition_and_sparse_two_ways():
    M, N, K = 4, 32, 512
    W = workloads.random_weights(41, N, K)
    x = workloads.random_x(42, M, K)
    L = oracle.quantize_layer(W, sparse_k=60)
    y_full = oracle.linear_ref(x, L["q"], L["s"], L["z"], L["row_ptr"], L["col"], L["val"])
    y_dense = oracle.linear_ref(x, L["q"], L["s"], L["z"])
    # CSR product as a dense matrix built entry by entry
    Wsp = np.zeros((N, K))
    for n in range(N):
        for e in range(L["row_ptr"][n], L["row_ptr"][n + 1]):
            Wsp[n, L["col"][e]] += float(L["val"][e])
    y_sp = x.astype(np.float64) @ Wsp.T
    assert np.allclose(y_full, y_dense + y_sp, rtol=0, atol=1e-12)
    # the decomposition approximates x W^T for the original weights
    y_true = x.astype(np.float64) @ W.astype(np.float64).T
    assert oracle.rel_err_inf(y_full, y_true) < 0.1


def test_nnz_zero_reduces_to_dense():
    W = workloads.random_weights(51, 8, 256)
    x = workloads.random_x(52, 2, 256)
    L = oracle.quantize_layer(W, 0)
    assert L["row_ptr"].tolist() == [0] * 9 and L["col"].size == 0
    y0 = oracle.linear_ref(x, L["q"], L["s"], L["z"], L["row_ptr"], L["col"], L["val"])
    y1 = oracle.linear_ref(x, L["q"], L["s"], L["z"])
    assert np.array_equal(y0, y1)


def test_linear_rows_matches_full():
    M, N, K = 3, 40, 256
    W = workloads.random_weights(61, N, K)
    x = workloads.random_x(62, M, K)
    L = oracle.quantize_layer(W, 25)
    y = oracle.linear_ref(x, L["packed"], L["s"], L["z"], L["row_ptr"], L["col"], L["val"])
    rows = [0, 7, 39, 13]
    ys = oracle.linear_rows(x, L["packed"], L["s"], L["z"], rows, L["row_ptr"], L["col"], L["val"])
    assert np.allclose(ys, y[:, rows], rtol=1e-13, atol=1e-13)


def test_quantization_error_within_tolerance_budget():
    """The fp16 rounding of (q - z) * s that a kernel may take is far below the
    5e-3 parity tolerance: checked on config 1 against the oracle itself."""
    W, x, _ = workloads.make(1)
    L = oracle.quantize_layer(W, 0)
    y = oracle.linear_ref(x, L["q"], L["s"], L["z"])
    w16 = oracle.dequant(L["q"], L["s"], L["z"]).astype(np.float16).astype(np.float64)
    y16 = x.astype(np.float64) @ w16.T
    assert oracle.rel_err_inf(y16, y) < 5e-4


# ---------------------------------------------------------------- low-rank branch


def test_lowrank_brute_force_rationals():
    """(x . L1^T) . L2^T against a triple loop in exact rationals."""
    M, N, K, r = 2, 5, 24, 3
    rng = np.random.default_rng(71)
    x = rng.standard_normal((M, K)).astype(np.float16)
    L1 = rng.standard_normal((r, K)).astype(np.float16)
    L2 = rng.standard_normal((N, r)).astype(np.float16)
    y = oracle.lowrank_term(x, L1, L2)
    assert y.shape == (M, N)
    for m in range(M):
        for n in range(N):
            ex = sum(Fraction(float(L2[n, j])) * sum(Fraction(float(x[m, k])) * Fraction(float(L1[j, k]))
                                                      for k in range(K)) for j in range(r))
            assert abs(y[m, n] - float(ex)) <= 1e-12 * max(1.0, abs(float(ex)))


def test_lowrank_equals_the_dense_product_of_its_factors():
    """In integers, applying the branch as two projections equals multiplying by
    the dense matrix L2 . L1 (a transposed or swapped factor breaks this on
    these non-square shapes)."""
    M, N, K, r = 3, 7, 256, 32
    L1, L2 = workloads.integer_lowrank_factors(72, r, N, K, nnz_per_row=40)
    x = np.random.default_rng(73).integers(-4, 5, size=(M, K)).astype(np.float16)
    W_lr = L2.astype(np.int64) @ L1.astype(np.int64)          # [N, K]
    want = x.astype(np.int64) @ W_lr.T
    assert np.array_equal(oracle.lowrank_term(x, L1, L2), want.astype(np.float64))
    # one-hot activations read a column of L2 . L1
    for k in (0, 5, 255):
        e = np.zeros((1, K), np.float16)
        e[0, k] = 1.0
        assert np.array_equal(oracle.lowrank_term(e, L1, L2)[0], W_lr[:, k].astype(np.float64))


def test_lowrank_in_the_linear_layer():
    """The branch adds to the dense and sparse terms in linear_ref and in
    linear_rows, and rank 0 adds nothing."""
    M, N, K, r = 3, 40, 256, 32
    W = workloads.random_weights(74, N, K)
    x = workloads.random_x(75, M, K)
    L = oracle.quantize_layer(W, 25)
    L1, L2 = workloads.lowrank_factors(76, r, N, K)
    base = oracle.linear_ref(x, L["packed"], L["s"], L["z"], L["row_ptr"], L["col"], L["val"])
    full = oracle.linear_ref(x, L["packed"], L["s"], L["z"], L["row_ptr"], L["col"], L["val"], L1=L1, L2=L2)
    # the branch computed column by column from its definition
    t = [[sum(float(x[m, k]) * float(L1[j, k]) for k in range(K)) for j in range(r)] for m in range(M)]
    for m in range(M):
        for n in (0, 17, 39):
            lr = sum(t[m][j] * float(L2[n, j]) for j in range(r))
            assert abs(full[m, n] - base[m, n] - lr) <= 1e-9 * max(1.0, abs(lr))
    rows = [0, 7, 39, 13]
    ys = oracle.linear_rows(x, L["packed"], L["s"], L["z"], rows, L["row_ptr"], L["col"], L["val"], L1=L1, L2=L2)
    assert np.allclose(ys, full[:, rows], rtol=1e-13, atol=1e-13)
    empty = oracle.lowrank_term(x, np.zeros((0, K), np.float16), np.zeros((N, 0), np.float16))
    assert empty.shape == (M, N) and not empty.any()


# ---------------------------------------------------------------- act-order groups
def _gidx_from_perm(perm, group=128):
    """Channel perm[i] belongs to group i // group (groups are consecutive in the
    permuted order)."""
    g = np.empty(len(perm), np.int64)
    g[np.asarray(perm)] = np.arange(len(perm)) // group
    return g


@pytest.mark.parametrize("group", [128, 256])
def test_gidx_contiguous_groups_reduce_to_plain_groups(group):
    W = workloads.random_weights(81, 7, 512)
    q, s, z = oracle.quantize_rtn_gidx(W, np.arange(512) // group)
    q2, s2, z2 = oracle.quantize_rtn(W, group)
    assert np.array_equal(q, q2) and np.array_equal(s.view(np.uint16), s2.view(np.uint16))
    assert np.array_equal(z.view(np.uint16), z2.view(np.uint16))


def test_gidx_brute_force_exact_rationals():
    """Scattered groups: each group's scale, zero-point and codes follow from the
    min and max over its members, in exact arithmetic."""
    W = workloads.random_weights(82, 3, 256, sigma=0.02)
    W[1, 7] *= 25
    perm = workloads.channel_permutation(83, 256)
    g_idx = _gidx_from_perm(perm)
    q, s, z = oracle.quantize_rtn_gidx(W, g_idx)
    for n in range(3):
        for j in range(2):
            members = [k for k in range(256) if g_idx[k] == j]
            assert len(members) == 128 and members != list(range(128 * j, 128 * j + 128))
            grp = [Fraction(float(W[n, k])) for k in members]
            mn, mx = min(grp), max(grp)
            S, Z = Fraction(float(s[n, j])), int(z[n, j])
            exact = (mx - mn) / 15
            ulp = Fraction(2) ** (int(np.floor(np.log2(float(S)))) - 10)
            assert abs(S - exact) <= ulp / 2 + exact * Fraction(1, 2 ** 22)
            assert Z == min(15, max(0, round(-mn / S)))
            for k, w in zip(members, grp):
                errs = [abs(w - (c - Z) * S) for c in range(16)]
                assert errs[int(q[n, k])] == min(errs)


def test_gidx_product_is_invariant_under_the_channel_permutation():
    """x . w_hat^T with scattered groups equals the product of the permuted
    activations with the layer in permuted (contiguous-group) order."""
    M, N, K = 3, 9, 512
    W = workloads.random_weights(84, N, K)
    x = workloads.random_x(85, M, K)
    perm = workloads.channel_permutation(86, K)
    g_idx = _gidx_from_perm(perm)
    q, s, z = oracle.quantize_rtn_gidx(W, g_idx)
    assert np.array_equal(oracle.dequant_gidx(q, s, z, g_idx)[:, perm], oracle.dequant(q[:, perm], s, z))
    y = oracle.linear_ref_gidx(x, q, s, z, g_idx)
    y2 = oracle.linear_ref(x[:, perm], q[:, perm], s, z)
    assert np.allclose(y, y2, rtol=1e-12, atol=1e-12)
    # and it is not the product with the groups taken as contiguous
    assert not np.allclose(y, oracle.linear_ref(x, q, s, z), rtol=1e-3)


# ---------------------------------------------------------------- W4A8 with fp16 outlier channels
def test_act_int8_exact_grid_values_come_back():
    """Activations already on the INT8 grid of a power-of-two step, with the
    amax at 127 steps, quantize to exactly those integers."""
    rng = np.random.default_rng(91)
    ints = rng.integers(-127, 128, size=(4, 256))
    ints[:, 3] = 127
    x = (ints * 2.0 ** -9).astype(np.float16)
    xq, s, xo = oracle.quantize_act_int8(x, [])
    assert np.all(s == np.float32(2.0 ** -9)) and np.array_equal(xq, ints.astype(np.int8)) and xo.shape == (4, 0)


def test_act_int8_brute_force_rationals():
    """Each INT8 value is the integer nearest to x / s (ties to even) for the
    float32 s = amax / 127 of its row, outliers excluded from the amax."""
    x = workloads.random_x(92, 3, 128)
    outliers = [5, 77]
    x[:, 77] = np.float16(300.0)
    xq, s, xo = oracle.quantize_act_int8(x, outliers)
    for m in range(3):
        amax = max(abs(float(x[m, k])) for k in range(128) if k not in outliers)
        assert s[m] == np.float32(np.float32(amax) / np.float32(127))
        S = Fraction(float(s[m]))
        for k in range(128):
            if k in outliers:
                assert xq[m, k] == 0
                continue
            t = Fraction(float(x[m, k])) / S
            lo = t.numerator // t.denominator
            near = lo if (t - lo < Fraction(1, 2) or (t - lo == Fraction(1, 2) and lo % 2 == 0)) else lo + 1
            # the float32 quotient may round onto a tie or across it only within 2^-24 relative
            if abs(t - lo - Fraction(1, 2)) > abs(t) * Fraction(1, 2 ** 22):
                assert int(xq[m, k]) == max(-127, min(127, near)), (m, k)
    assert np.array_equal(xo, x[:, outliers])


def test_act_int8_outlier_channels_do_not_move_the_scale():
    x = workloads.random_x(93, 2, 256)
    a = oracle.quantize_act_int8(x, [10, 200])
    x2 = x.copy()
    x2[:, 10] = np.float16(-5000.0)
    b = oracle.quantize_act_int8(x2, [10, 200])
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert b[2][0, 0] == np.float16(-5000.0)
    # without the exclusion the scale would follow the outlier
    c = oracle.quantize_act_int8(x2, [200])
    assert np.all(c[1] > 20 * a[1])


def test_w4a8_product_within_the_int8_rounding_bound():
    """|y_w4a8 - y_w4a16| <= s_x / 2 * sum_k |w_hat| per output (each INT8 value
    is within half a step of x / s_x), and outlier channels add no error."""
    M, N, K = 3, 40, 512
    W = workloads.random_weights(94, N, K)
    x = workloads.random_x(95, M, K)
    outliers = [1, 130, 400]
    x[:, outliers] *= np.float16(30)
    q, s, z = oracle.quantize_rtn(W)
    y8 = oracle.linear_w4a8_ref(x, q, s, z, outliers)
    y16 = oracle.linear_ref(x, q, s, z)
    _, sx, _ = oracle.quantize_act_int8(x, outliers)
    W_hat = oracle.dequant(q, s, z)
    bound = sx.astype(np.float64)[:, None] / 2 * np.abs(W_hat).sum(axis=1)[None, :] * (1 + 1e-6)
    assert np.all(np.abs(y8 - y16) <= bound)
    assert np.abs(y8 - y16).max() > 0
    # with every channel an outlier the product is the W4A16 one
    y_all = oracle.linear_w4a8_ref(x, q, s, z, list(range(K)))
    assert np.allclose(y_all, y16, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("bits", [2, 3])
def test_fewer_bits_on_grid_weights_come_back(bits):
    """Weights on a (bits)-bit grid of a power-of-two step, spanning the full code
    range, quantize to exactly those codes and dequantize back exactly."""
    qmax = (1 << bits) - 1
    rng = np.random.default_rng(96 + bits)
    N, K = 6, 256
    codes = rng.integers(0, qmax + 1, size=(N, K))
    codes[:, 0], codes[:, 1] = 0, qmax
    z = rng.integers(0, qmax + 1, size=(N, 1))
    W = ((codes - z) * 2.0 ** -6).astype(np.float32)
    q, s, zz = oracle.quantize_rtn(W, 128, bits)
    assert np.array_equal(q, codes.astype(np.uint8)) and np.all(s == np.float16(2.0 ** -6))
    assert np.array_equal(oracle.dequant(q, s, zz), W.astype(np.float64))


# ---------------------------------------------------------------- 3-bit packing
def _pack3_golden():
    with open(os.path.join(os.path.dirname(__file__), "golden", "pack3_hand_words.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _pack3_golden(), ids=lambda c: c["name"])
def test_pack3_hand_words(case):
    """Words derived by hand from the 3-bit layout, for single codes in each kind
    of slot (a pair's lo and hi half, each word, the split pair 15)."""
    q = np.zeros((1, 32), np.uint8)
    if case["codes"] == "all7":
        q[:] = 7
    else:
        for k, v in case["codes"].items():
            q[0, int(k)] = v
    words = oracle.pack3(q)
    assert [int(w) for w in words[0]] == [int(h, 16) for h in case["words"]], case["name"]
    assert np.array_equal(oracle.unpack3(words), q)


def test_pack3_uses_every_bit_once():
    """Each of the 32 x 3 code bits of a run lands on its own one of the 96 word
    bits: 0.375 bytes per weight with nothing lost or shared."""
    seen = set()
    for k in range(32):
        for b in range(3):
            q = np.zeros((1, 32), np.uint8)
            q[0, k] = 1 << b
            w = oracle.pack3(q)[0]
            bits = [(j, i) for j in range(3) for i in range(32) if (int(w[j]) >> i) & 1]
            assert len(bits) == 1, (k, b, bits)
            seen.add(bits[0])
    assert len(seen) == 96


def test_pack3_roundtrip_and_size():
    rng = np.random.default_rng(33)
    q = rng.integers(0, 8, size=(7, 512)).astype(np.uint8)
    p = oracle.pack3(q)
    assert p.shape == (7, 3 * 512 // 32) and p.dtype == np.uint32
    assert p.nbytes * 8 == q.size * 3
    assert np.array_equal(oracle.unpack3(p), q)
    with pytest.raises(ValueError):
        oracle.pack3(np.full((1, 32), 8, np.uint8))


def test_pack3_differs_from_sequential_bits():
    """The layout is not the plain sequential one (code k at bit 3k of the 96-bit
    run): a mutant that packed sequentially would still round-trip, so the hand
    words above are what pin the layout."""
    q = np.zeros((1, 32), np.uint8)
    q[0, 1] = 1                                   # sequential: bit 3 of word 0
    assert int(oracle.pack3(q)[0, 0]) == 1 << 3   # here: pair 1 lo, i = 1 -> bit 3 too
    q[0, 1], q[0, 5] = 0, 1                       # sequential: bit 15; here: pair 1 hi -> bit 19
    assert int(oracle.pack3(q)[0, 0]) == 1 << 19


def test_group64_is_not_group128():
    """At 64-channel groups each half of a 128-channel group gets its own range:
    the metadata has twice the columns, and a group whose halves differ in range
    gets different scales (a mutant that quantized in 128-channel groups and
    repeated the metadata would fail this)."""
    W = workloads.random_weights(64, 2, 256, sigma=0.02)
    W[0, 0:64] *= 4.0
    q, s, z = oracle.quantize_rtn(W, 64)
    assert s.shape == (2, 4)
    assert float(s[0, 0]) > 2.0 * float(s[0, 1])
    # each 64-channel half equals the quantizer run on that half alone
    for g in range(4):
        qg, sg, zg = oracle.quantize_rtn(W[:, 64 * g:64 * g + 64], 64)
        assert np.array_equal(q[:, 64 * g:64 * g + 64], qg)
        assert np.array_equal(f16_bits(s[:, g:g + 1]), f16_bits(sg))
    # and dequantization at 64 reads the right column
    w_hat = oracle.dequant(q, s, z, 64)
    assert np.allclose(w_hat, W, atol=float(s.astype(np.float64).max()) / 2 + 1e-12)
