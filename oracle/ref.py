"""CPU oracle for the W4A16 group-quantized linear with a sparse outlier term.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the package smoke check and the CPU
baseline leg of the benchmark use it.  It shares no code with the HIP
library (it imports only numpy and the seeded input generator).

What is computed, and where the pages say so
--------------------------------------------
* Dense-and-sparse decomposition: the weight matrix is the sum of a dense
  part that is quantized to a few bits and a sparse part that keeps a small
  fraction of the weights in fp16; the product is split the same way,
  W x = W_dense x + W_sparse x (SqueezeLLM explainer, sections 2.2 and 2.3).
  The sparsity is the count of sparse non-zeros over all weights (section
  2.2).  The pages select the sparse entries with a Hessian-based
  sensitivity; with no model or data, the entries of largest |w| are taken
  instead (ties: lower flat index first).
* Round-to-nearest (RTN) weight-only quantization is the calibration-free
  baseline of weight quantization (AWQ paper, section 2; LLM Compressor
  article, FAQ).  The pages never print its formula.  The reading used
  here: asymmetric INT4 per group of 128 consecutive input channels
  ("W4A16 g128", DeepCompressor README perplexity table), step
  Delta = (max - min) / (2^4 - 1), an integer zero-point, round half to
  even, clamp to [0, 15].
* 4-bit packing: eight codes per 32-bit word so that byte-addressed hardware
  still sees the 4x size cut (AWQ paper, section 1).
* On-the-fly dequantization inside the linear (AWQ paper, section 1):
  w_hat = (q - z) * s, and y = x . w_hat^T + W_sparse x.

Precision
---------
The quantizer (split, range, scale, zero, codes) is evaluated in IEEE
float32 with correctly rounded division and no fused multiply-add, because
its results are integers (codes, zero-points) and fp16 bit patterns that
must be unique; the same float32 definition is what the device kernels
implement.  Dequantization and the linear layer run in float64.

Every function states the readings it takes where the pages are silent.
No function here is "parity unpinned": each is pinned by the CPU tests
(on-grid exact recovery, zero exactness, brute force in exact rationals,
closed forms, full sorts on tiny inputs, hand-worked fixtures).
"""
from __future__ import annotations

import numpy as np

GROUP = 128
QMAX = 15  # 2^4 - 1 for INT4 codes
FP16_MIN_NORMAL = np.float32(2.0 ** -14)


# --------------------------------------------------------------------------
# O1: dense-and-sparse split (SqueezeLLM explainer, sections 2.2-2.3)
# --------------------------------------------------------------------------
def split_outliers(W: np.ndarray, sparse_k: int):
    """Split ``W`` into a dense part and an fp16 CSR sparse part.

    The ``sparse_k`` entries of largest |w| go to the sparse part; entries
    with equal |w| are taken in ascending flat index ``n*K + k``.  The dense
    part is ``W`` with those entries replaced by +0.0, so that
    ``W = W_dense + W_sparse`` holds exactly before the fp16 rounding of the
    sparse values.

    Returns ``(W_dense float32 [N,K], row_ptr int32 [N+1], col int32 [nnz],
    val float16 [nnz])`` with CSR rows = output channels n and columns
    strictly ascending inside a row.
    """
    W = np.asarray(W, dtype=np.float32)
    N, K = W.shape
    total = N * K
    if not 0 <= sparse_k <= total:
        raise ValueError("sparse_k out of range")
    Wd = W.copy()
    if sparse_k == 0:
        return Wd, np.zeros(N + 1, np.int32), np.zeros(0, np.int32), np.zeros(0, np.float16)
    a = np.abs(W).reshape(-1)
    # threshold T = the sparse_k-th largest |w|
    T = np.partition(a, total - sparse_k)[total - sparse_k]
    above = np.flatnonzero(a > T)
    ties = np.flatnonzero(a == T)           # ascending flat index
    need = sparse_k - above.size
    chosen = np.sort(np.concatenate([above, ties[:need]]))
    rows = chosen // K
    cols = chosen % K
    val = W.reshape(-1)[chosen].astype(np.float16)
    Wd.reshape(-1)[chosen] = np.float32(0.0)
    row_ptr = np.zeros(N + 1, np.int64)
    np.add.at(row_ptr, rows + 1, 1)
    row_ptr = np.cumsum(row_ptr).astype(np.int32)
    return Wd, row_ptr, cols.astype(np.int32), val


# --------------------------------------------------------------------------
# O2-O5: RTN group quantizer
# --------------------------------------------------------------------------
def quantize_rtn(Wd: np.ndarray, group: int = GROUP, bits: int = 4):
    """Asymmetric round-to-nearest quantization to ``bits``-bit codes (INT4 by
    default; the SqueezeLLM explainer quantizes to 3 or 4 bits, section 1 and the
    weight-bits option of section 4), one (s, z) per group.  Below, 15 is
    ``qmax = 2^bits - 1``.

    For each row n and group j of ``group`` consecutive input channels:

    * ``mn, mx`` = min and max of the group (zeros left by the split count);
    * ``d = fl32(fl32(mx - mn) / 15)``, floored at 2^-14 (the smallest
      normal fp16) so that a constant group still has a usable step;
    * ``s`` = d rounded to fp16 (nearest even); the codes are computed with
      this stored value, so the stored metadata reproduces them;
    * ``z = clamp(rint(fl32(-mn / s)), 0, 15)``, an integer stored as fp16;
    * ``q = clamp(rint(fl32(w / s)) + z, 0, 15)``.

    ``rint`` is round-half-to-even.  Returns ``(q uint8 [N,K], s float16
    [N,K/group], z float16 [N,K/group])``.
    """
    Wd = np.asarray(Wd, dtype=np.float32)
    N, K = Wd.shape
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    G = K // group
    Wg = Wd.reshape(N, G, group)
    mn = Wg.min(axis=2)
    mx = Wg.max(axis=2)
    rng = (mx - mn).astype(np.float32)
    qmax = (1 << bits) - 1
    d = (rng / np.float32(qmax)).astype(np.float32)
    d = np.maximum(d, FP16_MIN_NORMAL)
    s16 = d.astype(np.float16)
    s = s16.astype(np.float32)
    zf = np.rint((-mn) / s).astype(np.float32)
    z = np.clip(zf, 0, qmax).astype(np.int32)
    t = np.rint(Wg / s[:, :, None]).astype(np.float32)
    q = np.clip(t + z[:, :, None].astype(np.float32), 0, qmax).astype(np.uint8)
    return q.reshape(N, K), s16, z.astype(np.float16)


# --------------------------------------------------------------------------
# O6: packing (AWQ paper, section 1: 4-bit weight packing)
# --------------------------------------------------------------------------
def pack(q: np.ndarray) -> np.ndarray:
    """Eight consecutive codes along K per uint32; code k = 8t + i sits in
    bits [4i, 4i + 4) of word t."""
    q = np.asarray(q, dtype=np.uint8)
    N, K = q.shape
    if K % 8:
        raise ValueError("K must be a multiple of 8")
    q8 = q.reshape(N, K // 8, 8).astype(np.uint32)
    out = np.zeros((N, K // 8), np.uint32)
    for i in range(8):
        out |= q8[:, :, i] << np.uint32(4 * i)
    return out


def unpack(packed: np.ndarray) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint32)
    N, W = packed.shape
    q = np.empty((N, W, 8), np.uint8)
    for i in range(8):
        q[:, :, i] = (packed >> np.uint32(4 * i)) & np.uint32(0xF)
    return q.reshape(N, W * 8)


# 3-bit packing.  The SqueezeLLM explainer stores models of 3 bits per weight
# (section 1; the weight-bits option of sections 4.1 and 5.2), and packing is what
# turns a smaller code into fewer bytes on byte-addressed hardware (AWQ paper,
# section 1); no page gives a 3-bit layout.  The one used here puts every run of
# 32 consecutive codes (k = 32u .. 32u + 31) into three words, 96 bits with none
# wasted.  Within a run, code pair P = 4t + p (t, p = 0..3) is the pair of codes
# lo = 8t + p and hi = 8t + p + 4.  Pairs 0..14 sit five to a word: pair P in word
# P // 5, lo at bits [3i, 3i + 3) and hi at bits [16 + 3i, 16 + 3i + 3) with
# i = P % 5.  Pair 15 (codes 27 and 31) takes the two bits left in each word: bit
# b of code 27 is bit 15 of word b, bit b of code 31 is bit 31 of word b.
def _pairs3():
    """(P, lo offset, hi offset) for the 16 code pairs of a 32-code run."""
    return [(P, 8 * (P // 4) + P % 4, 8 * (P // 4) + P % 4 + 4) for P in range(16)]


def pack3(q: np.ndarray) -> np.ndarray:
    """Codes of at most 3 bits, uint8 [N, K] (K a multiple of 32), packed to uint32
    [N, 3K/32] in the layout described above."""
    q = np.asarray(q, dtype=np.uint8)
    N, K = q.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    if q.size and q.max() > 7:
        raise ValueError("3-bit codes must be at most 7")
    u = q.reshape(N, K // 32, 32).astype(np.uint32)
    out = np.zeros((N, K // 32, 3), np.uint32)
    for P, lo, hi in _pairs3():
        if P < 15:
            w, i = divmod(P, 5)
            out[:, :, w] |= (u[:, :, lo] << np.uint32(3 * i)) | (u[:, :, hi] << np.uint32(16 + 3 * i))
        else:
            for b in range(3):
                out[:, :, b] |= (((u[:, :, lo] >> np.uint32(b)) & np.uint32(1)) << np.uint32(15)) | \
                                (((u[:, :, hi] >> np.uint32(b)) & np.uint32(1)) << np.uint32(31))
    return out.reshape(N, 3 * K // 32)


def unpack3(packed: np.ndarray) -> np.ndarray:
    """Inverse of pack3: uint32 [N, 3K/32] -> uint8 codes [N, K]."""
    packed = np.asarray(packed, dtype=np.uint32)
    N, W = packed.shape
    if W % 3:
        raise ValueError("a 3-bit row holds a multiple of three words")
    w = packed.reshape(N, W // 3, 3)
    q = np.zeros((N, W // 3, 32), np.uint32)
    for P, lo, hi in _pairs3():
        if P < 15:
            j, i = divmod(P, 5)
            q[:, :, lo] = (w[:, :, j] >> np.uint32(3 * i)) & np.uint32(7)
            q[:, :, hi] = (w[:, :, j] >> np.uint32(16 + 3 * i)) & np.uint32(7)
        else:
            for b in range(3):
                q[:, :, lo] |= ((w[:, :, b] >> np.uint32(15)) & np.uint32(1)) << np.uint32(b)
                q[:, :, hi] |= ((w[:, :, b] >> np.uint32(31)) & np.uint32(1)) << np.uint32(b)
    return q.reshape(N, W // 3 * 32).astype(np.uint8)


# --------------------------------------------------------------------------
# O7-O8: dequantization and the linear layer, float64
# --------------------------------------------------------------------------
def dequant(q: np.ndarray, s: np.ndarray, z: np.ndarray, group: int = GROUP) -> np.ndarray:
    """w_hat[n, k] = (q[n, k] - z[n, k // group]) * s[n, k // group] in float64."""
    q = np.asarray(q)
    N, K = q.shape
    G = K // group
    qg = q.reshape(N, G, group).astype(np.float64)
    zf = np.asarray(z).astype(np.float64)[:, :, None]
    sf = np.asarray(s).astype(np.float64)[:, :, None]
    return ((qg - zf) * sf).reshape(N, K)


def sparse_term(x: np.ndarray, row_ptr, col, val, N: int) -> np.ndarray:
    """(W_sparse x)^T for all rows of x: out[m, n] = sum_e val_e * x[m, col_e]
    over the CSR entries e of row n, in float64."""
    x64 = np.asarray(x).astype(np.float64)
    M = x64.shape[0]
    out = np.zeros((M, N), np.float64)
    row_ptr = np.asarray(row_ptr, dtype=np.int64)
    nnz = int(row_ptr[-1]) if row_ptr.size else 0
    if nnz == 0:
        return out
    col = np.asarray(col, dtype=np.int64)[:nnz]
    v = np.asarray(val).astype(np.float64)[:nnz]
    prod = x64[:, col] * v[None, :]           # [M, nnz]
    counts = np.diff(row_ptr)
    nonempty = np.flatnonzero(counts)
    sums = np.add.reduceat(prod, row_ptr[nonempty], axis=1)
    out[:, nonempty] = sums
    return out


# --------------------------------------------------------------------------
# O9: low-rank high-precision branch (DeepCompressor README, SVDQuant section)
# --------------------------------------------------------------------------


def lowrank_term(x, L1, L2) -> np.ndarray:
    """(x . L1^T) . L2^T in float64, for all rows of x.

    The SVDQuant section of the DeepCompressor README moves outliers from the
    activations into the weights and lets a high-precision low-rank branch,
    obtained by SVD, hold the weights' outliers, so that only the residual is
    quantized to 4 bits; run as a separate kernel that branch costs extra
    activation traffic, so the engine fuses it into the low-bit kernel.  The
    pages give neither the rank nor the layout of the factors.  The reading
    here: W = L2 . L1 + R with fp16 factors L1 [r, K] (the down-projection, one
    row per component) and L2 [N, r] (the up-projection), applied to the
    activations as t = x . L1^T and then t . L2^T."""
    x64 = np.asarray(x).astype(np.float64)
    L1 = np.asarray(L1).astype(np.float64)
    L2 = np.asarray(L2).astype(np.float64)
    if L1.shape[0] == 0:
        return np.zeros((x64.shape[0], L2.shape[0]), np.float64)
    return (x64 @ L1.T) @ L2.T


def linear_ref(x, q, s, z, row_ptr=None, col=None, val=None, group: int = GROUP, L1=None, L2=None):
    """y[m, n] = sum_k x[m, k] * w_hat[n, k] + (W_sparse x)[n, m] in float64,
    plus the low-rank branch (x . L1^T . L2^T)[m, n] when the factors are given.

    ``q`` may be the unpacked codes [N, K] (uint8) or the 4-bit packed words
    [N, K/8] (uint32)."""
    q = np.asarray(q)
    if q.dtype == np.uint32:
        q = unpack(q)
    N = q.shape[0]
    W_hat = dequant(q, s, z, group)
    y = np.asarray(x).astype(np.float64) @ W_hat.T
    if row_ptr is not None:
        y += sparse_term(x, row_ptr, col, val, N)
    if L1 is not None:
        y += lowrank_term(x, L1, L2)
    return y


def linear_rows(x, q, s, z, rows, row_ptr=None, col=None, val=None, group: int = GROUP, L1=None, L2=None):
    """The same as ``linear_ref`` restricted to output channels ``rows``
    (used to check full-size outputs one sample at a time)."""
    rows = np.asarray(rows, dtype=np.int64)
    q = np.asarray(q)
    if q.dtype == np.uint32:
        qs = unpack(q[rows])
    else:
        qs = q[rows]
    W_hat = dequant(qs, np.asarray(s)[rows], np.asarray(z)[rows], group)
    x64 = np.asarray(x).astype(np.float64)
    y = x64 @ W_hat.T
    if row_ptr is not None:
        row_ptr = np.asarray(row_ptr, dtype=np.int64)
        col = np.asarray(col, dtype=np.int64)
        v = np.asarray(val).astype(np.float64)
        for j, n in enumerate(rows):
            a, b = row_ptr[n], row_ptr[n + 1]
            if b > a:
                y[:, j] += x64[:, col[a:b]] @ v[a:b]
    if L1 is not None:
        y += lowrank_term(x, L1, np.asarray(L2)[rows])
    return y


# Act-order groups: membership by a per-channel group index
def quantize_rtn_gidx(Wd: np.ndarray, g_idx):
    """RTN quantization with groups given by a per-channel group index.

    The GPTQ-R rows (GPTQ with reordering) of the DeepCompressor README
    perplexity table quantize the input channels in a permuted order, so a group
    is a scattered set of channels: group j = {k : g_idx[k] == j}.  Each group
    is quantized by the definition of ``quantize_rtn`` (min and max over its
    members, then the same s, z and codes), which the membership alone decides:
    the order of the members does not enter.  Returns ``(q uint8 [N,K]`` in the
    original channel order, ``s, z float16 [N,G])``."""
    Wd = np.asarray(Wd, dtype=np.float32)
    g_idx = np.asarray(g_idx)
    N, K = Wd.shape
    if g_idx.shape != (K,):
        raise ValueError("g_idx must have K entries")
    G = int(g_idx.max()) + 1
    q = np.empty((N, K), np.uint8)
    s = np.empty((N, G), np.float16)
    z = np.empty((N, G), np.float16)
    for j in range(G):
        members = np.nonzero(g_idx == j)[0]
        qj, sj, zj = quantize_rtn(Wd[:, members], group=members.size)  # one group
        q[:, members] = qj
        s[:, j] = sj[:, 0]
        z[:, j] = zj[:, 0]
    return q, s, z


def dequant_gidx(q, s, z, g_idx) -> np.ndarray:
    """w_hat[n, k] = (q[n, k] - z[n, g_idx[k]]) * s[n, g_idx[k]] in float64."""
    g_idx = np.asarray(g_idx)
    S = np.asarray(s).astype(np.float64)[:, g_idx]
    Z = np.asarray(z).astype(np.float64)[:, g_idx]
    return (np.asarray(q).astype(np.float64) - Z) * S


def linear_ref_gidx(x, q, s, z, g_idx, row_ptr=None, col=None, val=None) -> np.ndarray:
    """y = x . w_hat^T (+ W_sparse x) in float64 for an act-order layer, all in
    the original channel order."""
    y = np.asarray(x).astype(np.float64) @ dequant_gidx(q, s, z, g_idx).T
    if row_ptr is not None and len(np.asarray(col)):
        y += sparse_term(x, row_ptr, col, val, np.asarray(q).shape[0])
    return y


# W4A8 with fp16 outlier channels
QX = 127


def quantize_act_int8(x, outliers):
    """Per-token INT8 activations with fixed fp16 outlier channels.

    The MixQ news item keeps a few activation channels, the outliers, in high
    precision (they stay the same channels from one decode step to the next) and
    quantizes the rest of each token's activations to INT8 by its absolute
    maximum; the INT8 and the high-precision products are added.  The reading
    here, per row m of x (fp16 values, arithmetic in float32):

    * ``amax`` = max |x[m, k]| over the channels k not in ``outliers``;
    * ``s = fl32(amax / 127)``, or 1 when amax is 0;
    * ``xq[m, k] = clamp(rint(fl32(x[m, k] / s)), -127, 127)`` (half to even),
      and 0 on the outlier channels;
    * ``xo[m, j] = x[m, outliers[j]]`` (fp16, unchanged).

    Returns ``(xq int8 [M,K], s float32 [M], xo float16 [M, n_out])``."""
    x = np.asarray(x, dtype=np.float16)
    outliers = np.asarray(outliers, dtype=np.int64)
    M, K = x.shape
    xf = x.astype(np.float32)
    keep = np.ones(K, bool)
    keep[outliers] = False
    amax = np.abs(xf[:, keep]).max(axis=1) if keep.any() else np.zeros(M, np.float32)
    s = np.where(amax > 0, amax / np.float32(QX), np.float32(1.0)).astype(np.float32)
    xq = np.clip(np.rint(xf / s[:, None]), -QX, QX).astype(np.int8)
    xq[:, ~keep] = 0
    return xq, s, x[:, outliers].copy()


def linear_w4a8_ref(x, q, s, z, outliers, group: int = GROUP) -> np.ndarray:
    """y = s_x[m] * sum_k xq[m, k] * w_hat[n, k] + sum_j xo[m, j] * w_hat[n, outliers[j]]
    in float64: the INT8 channels and the fp16 outlier channels, both against the
    dequantized INT4 weights."""
    xq, sx, xo = quantize_act_int8(x, outliers)
    W_hat = dequant(q, s, z, group)
    y = sx.astype(np.float64)[:, None] * (xq.astype(np.float64) @ W_hat.T)
    if len(np.asarray(outliers)):
        y += xo.astype(np.float64) @ W_hat[:, np.asarray(outliers)].T
    return y


def quantize_layer(W: np.ndarray, sparse_k: int = 0, group: int = GROUP, bits: int = 4):
    """The offline pipeline: split, quantize the dense part, pack (codes of fewer
    than 4 bits go into the same 4-bit packing)."""
    Wd, row_ptr, col, val = split_outliers(W, sparse_k)
    q, s, z = quantize_rtn(Wd, group, bits)
    return dict(W_dense=Wd, q=q, s=s, z=z, packed=pack(q), row_ptr=row_ptr, col=col, val=val)


def rel_err_inf(y, y_ref) -> float:
    """max |y - y_ref| / max |y_ref|, the parity measure for floating outputs."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    den = np.max(np.abs(y_ref)) if y_ref.size else 0.0
    num = np.max(np.abs(y - y_ref)) if y_ref.size else 0.0
    if den == 0.0:
        return float(num)
    return float(num / den)


TOL = 5e-3  # ||y - y_ref||_inf <= TOL * ||y_ref||_inf
