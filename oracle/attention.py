"""fp64 CPU oracle for exact scaled-dot-product attention (forward and backward).

TEST INFRASTRUCTURE ONLY. This module is imported by ``tests/``, by the package's
``smoke()`` check and by the bench's CPU-baseline leg; the library under
``exact_io_aware_46_amd/`` never imports, links or calls it, and it shares no code with
the HIP path (its bf16 widening, masking, softmax and gradients are written here).

What it computes is the plain definition, materialised: the score matrix S and the
probability matrix P are formed in full (per head, per panel of query rows), in float64.

* Standard attention S = Q K^T, P = softmax(S), O = P V, with a mask applied to the
  scores for GPT-style models -- "FlashAttention学习笔记" (amentiraz.github.io),
  section Forward运作流程 / 标准attention计算.
* The softmax is the safe one (row maximum subtracted before exponentiating) -- same
  page, section 标准Safe softmax.
* Order of operations: matmul, scaling, masking, softmax, multiplication by V --
  "高效注意力算法实现 (FlashAttention)" (apxml.com), section FlashAttention：融合算子与
  分块处理 (kernel fusion bullet). FlashAttention returns exactly this output (same page,
  same section, and 优势与影响: exactness).
* The saved softmax statistic used by backward recomputation -- report on
  "FlashAttention：一种基于I/O感知的快速且内存高效的自注意力算法" (fmread.com), section
  算法设计 (backward bullet). Read here as one log-sum-exp per row, natural log.
* Block-sparse attention (same report, 研究亮点 item 3; and the abstract of
  "FlashAttention: Fast and Memory-Efficient Exact Attention with IO-Awareness",
  aha.fim.ai) is read as: a 128x128 table over (query block, key block), nonzero = the
  block's scores are kept, zero = they are masked to -inf.

Readings where the pages are silent (each one is listed with its reasons in the design
notes of the repository):
* scale multiplies Q K^T before masking; the float32 scale is widened exactly;
* causal means key j is allowed for query i iff j <= i (equal lengths);
* key padding (valid length L_b per batch entry) masks keys j >= L_b for every query;
* sliding-window (local) attention, which the deployment page lists as a supported option
  ("IO感知计算如何重塑Transformer内存优化技术格局", bxzpzcl.cn, section 高级功能配置) without
  defining it, is read as a window (left, right) on the key index relative to the query:
  key j is allowed for query i iff i - left <= j <= i + right, a negative bound meaning
  no limit on that side (so (-1, 0) is the causal mask);
* the masks compose by logical AND;
* dropout, which FlashAttention fuses into the kernel ("FlashAttention学习笔记": section
  Kernel融合 lists it among the operations fused into one kernel, and section
  分块计算整体流程 applies it, with the mask, to each block's scores on the way to P̂;
  the report's backward bullet: nothing of size N x N is stored, so the dropout mask is
  regenerated), is read as the usual inverted
  dropout on the attention probabilities: P_drop = P * keep / (1 - p), O = P_drop V, with
  LSE the statistic of the undropped softmax. keep is drawn from a counter-based
  generator so that backward can regenerate it: Philox4x32-10 (Salmon, Moraes, Dror and
  Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011), key (seed low 32 bits,
  seed high 32 bits), counter (j >> 2, i >> 1, b * H + h, offset). One call covers a
  patch of 2 queries x 4 keys: word j & 3 of the output, its low 16 bits for even i and
  its high 16 bits for odd i, is the 16-bit draw r, and the element is kept iff
  r >= floor(p * 2^16) (p resolved to 2^-16; the pages fix no generator, and 16-bit
  draws halve the generator work per element against 32-bit ones). Backward through the
  fixed mask:
  dV = P_drop^T dO, dP = (dO V^T) * keep / (1 - p), D = rowsum(dO * O),
  dS = P * (dP - D);
* FP8 forward. The deployment page says FlashAttention-3 brought FP8 to the forward pass
  on H100 ("IO感知计算如何重塑Transformer内存优化技术格局", section 技术演进时间线) and gives
  no quantisation policy. It is read as follows.
  - Q, K and V arrive as OCP E4M3 codes (1 sign, 4 exponent bits with bias 7,
    3 mantissa bits; subnormals; the all-ones magnitude is NaN; largest finite 448),
    with one float32 descale per tensor: q = descale_q * decode(Q8), likewise k and v.
  - S = scale * q k^T in exact arithmetic, masked as above.
  - In log2 units t = S * log2(e). With m = ceil(max_j t_j) over the row's allowed keys,
    the scaled probabilities P_j = 2^(t_j - m + 6) lie in (0, 64]: the row's largest is in
    (32, 64], so every probability down to 2^-12 of it lies in E4M3's normal range
    (smallest normal 2^-6), and the headroom up to 448 (2^8.8) is left for a one-pass
    kernel whose running reference trails the row maximum.
  - P_j is rounded to E4M3, nearest with ties to even, subnormals included, giving Pq_j.
    l = sum_j P_j is left unrounded.
  - O = descale_v * sum_j Pq_j decode(V8_j) / l, and LSE = ln sum_j exp(S_j).
  - The reference m is an integer, so a kernel whose running reference is any integer (in
    log2 units) quantises the same P, scaled by a power of two. That scaling commutes with
    the rounding wherever both sides are in the normal range.
* a row with no allowed key has O = 0, LSE = -inf and contributes nothing to gradients;
* backward is the derivative of the scalar L = sum(dO * O) with respect to Q, K, V:
  dV = P^T dO, dP = dO V^T, D_i = sum_c dO_ic O_ic, dS = P * (dP - D),
  dQ = scale * dS K, dK = scale * dS^T Q  (textbook softmax calculus; the pages say
  only that backward recomputes P from the saved statistic).

Row panels: to bound memory at long N the query rows of a head are processed in panels.
Every row-local quantity (S row, LSE, P row, O row, D_i, dP row, dS row, dQ row) is
identical to the whole-matrix computation; dK and dV are sums over rows and are
accumulated panel by panel in float64 (only the fp64 summation order differs).
"""
from __future__ import annotations

import numpy as np

MASK_BLOCK = 128
DEFAULT_PANEL = 4096


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def as_f64(x: np.ndarray) -> np.ndarray:
    """Accept either bf16 bit patterns (uint16) or real arrays (numpy float16 for fp16
    inputs, float32, float64); every value is widened exactly."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return widen_bf16(x)
    return x.astype(np.float64)


def allowed(rows: np.ndarray, n_keys: int, causal: bool, blockmask, kv_len_b,
            window=None) -> np.ndarray:
    """Boolean [len(rows), n_keys]: True where query ``rows[r]`` may attend to key j.
    ``window`` is None or (left, right): keys i-left .. i+right, a negative bound = none."""
    rows = np.asarray(rows, dtype=np.int64)
    j = np.arange(n_keys, dtype=np.int64)[None, :]
    i = rows[:, None]
    ok = np.ones((rows.size, n_keys), dtype=bool)
    if causal:
        ok &= j <= i
    if window is not None:
        left, right = int(window[0]), int(window[1])
        if left >= 0:
            ok &= j >= i - left
        if right >= 0:
            ok &= j <= i + right
    if blockmask is not None:
        bm = np.asarray(blockmask) != 0
        ok &= bm[i // MASK_BLOCK, j // MASK_BLOCK]
    if kv_len_b is not None:
        ok &= j < int(kv_len_b)
    return ok


# ------------------------------------------------------------------ dropout

_PHILOX_M = (0xD2511F53, 0xCD9E8D57)  # round multipliers
_PHILOX_W = (0x9E3779B9, 0xBB67AE85)  # key increments (Weyl sequence)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Philox4x32 with 10 rounds on arrays of uint32 counter words and a scalar 2x32-bit key.
    Each round: (hi, lo) of M0*c0 and M1*c2; new counter = (hi1 ^ c1 ^ k0, lo1,
    hi0 ^ c3 ^ k1, lo0); then the key is bumped by the Weyl constants."""
    m = np.uint64(0xFFFFFFFF)
    c = [np.asarray(x, dtype=np.uint64) & m for x in (c0, c1, c2, c3)]
    k0, k1 = np.uint64(k0) & m, np.uint64(k1) & m
    for _ in range(10):
        p0 = np.uint64(_PHILOX_M[0]) * c[0]
        p1 = np.uint64(_PHILOX_M[1]) * c[2]
        c = [((p1 >> np.uint64(32)) ^ c[1] ^ k0) & m, p1 & m,
             ((p0 >> np.uint64(32)) ^ c[3] ^ k1) & m, p0 & m]
        k0 = (k0 + np.uint64(_PHILOX_W[0])) & m
        k1 = (k1 + np.uint64(_PHILOX_W[1])) & m
    return c


def dropout_threshold(p: float) -> int:
    """Elements whose 16-bit draw is below this are dropped: floor(p * 2^16), p being the
    float32 value the kernels receive."""
    pf = float(np.float32(p))
    return int(min(65535.0, np.floor(pf * 65536.0)))


def dropout_keep(rows, n_keys, bh, p, seed, offset):
    """Boolean [len(rows), n_keys]: True where element (i, j) of head bh is kept."""
    rows = np.asarray(rows, dtype=np.int64)
    i = np.broadcast_to(rows[:, None], (rows.size, n_keys))
    j = np.broadcast_to(np.arange(n_keys, dtype=np.int64)[None, :], (rows.size, n_keys))
    words = philox4x32_10(j >> 2, i >> 1, np.full(i.shape, bh), np.full(i.shape, offset),
                          seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    w = np.choose((j & 3).astype(np.int64), words)
    r = (w >> (16 * (i & 1)).astype(np.uint64)) & np.uint64(0xFFFF)
    return r >= np.uint64(dropout_threshold(p))


def _dropout_scale(p: float) -> float:
    return 1.0 / (1.0 - float(np.float32(p)))


def _scores(Qr, K, s, ok):
    """S = s * Q K^T on the given query rows, -inf where not allowed."""
    S = s * (Qr @ K.T)
    S[~ok] = -np.inf
    return S


def _logsumexp_rows(S):
    """Safe log-sum-exp of each row; -inf for a row with no finite entry."""
    m = S.max(axis=1)
    lse = np.full(m.shape, -np.inf)
    live = np.isfinite(m)
    if live.any():
        Sl = S[live]
        lse[live] = m[live] + np.log(np.exp(Sl - m[live][:, None]).sum(axis=1))
    return lse


def _probs(S, lse):
    """P = exp(S - LSE) row by row; rows with LSE = -inf are all zero."""
    P = np.zeros_like(S)
    live = np.isfinite(lse)
    if live.any():
        P[live] = np.exp(S[live] - lse[live][:, None])
    return P


def _scale64(scale: float) -> float:
    return float(np.float32(scale))


def _head_view(x, b, h):
    return as_f64(x[b, h])


def head_forward(Qh, Kh, Vh, scale, causal=False, blockmask=None, kv_len_b=None,
                 rows=None, panel=DEFAULT_PANEL, window=None, dropout=None):
    """One head: returns (O[rows], LSE[rows]) in float64. ``dropout`` is None or
    (p, seed, offset, bh) with bh = b * H + h."""
    N = Kh.shape[0]
    s = _scale64(scale)
    rows = np.arange(Qh.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    O = np.zeros((rows.size, Vh.shape[1]))
    LSE = np.zeros(rows.size)
    for r0 in range(0, rows.size, panel):
        rr = rows[r0:r0 + panel]
        S = _scores(Qh[rr], Kh, s, allowed(rr, N, causal, blockmask, kv_len_b, window))
        lse = _logsumexp_rows(S)
        P = _probs(S, lse)
        if dropout is not None:
            p, seed, offset, bh = dropout
            P = P * dropout_keep(rr, N, bh, p, seed, offset) * _dropout_scale(p)
        O[r0:r0 + rr.size] = P @ Vh
        LSE[r0:r0 + rr.size] = lse
    return O, LSE


def head_backward(Qh, Kh, Vh, dOh, scale, causal=False, blockmask=None, kv_len_b=None,
                  panel=DEFAULT_PANEL, window=None, dropout=None):
    """One head, all rows: returns dict with O, LSE, D, dQ, dK, dV (float64)."""
    N, d = Kh.shape
    s = _scale64(scale)
    out = {k: np.zeros((N, d)) for k in ("O", "dQ", "dK", "dV")}
    out["LSE"] = np.zeros(N)
    out["D"] = np.zeros(N)
    for r0 in range(0, N, panel):
        rr = np.arange(r0, min(N, r0 + panel))
        S = _scores(Qh[rr], Kh, s, allowed(rr, N, causal, blockmask, kv_len_b, window))
        lse = _logsumexp_rows(S)
        P = _probs(S, lse)
        if dropout is None:
            Pd, keep_scale = P, None
        else:
            p, seed, offset, bh = dropout
            keep_scale = dropout_keep(rr, N, bh, p, seed, offset) * _dropout_scale(p)
            Pd = P * keep_scale
        O = Pd @ Vh
        dO = dOh[rr]
        D = (dO * O).sum(axis=1)
        dP = dO @ Vh.T
        if keep_scale is not None:
            dP = dP * keep_scale
        dS = P * (dP - D[:, None])
        out["O"][rr] = O
        out["LSE"][rr] = lse
        out["D"][rr] = D
        out["dQ"][rr] = s * (dS @ Kh)
        out["dK"] += s * (dS.T @ Qh[rr])
        out["dV"] += Pd.T @ dO
    return out


def _kv_len_b(kv_len, b):
    return None if kv_len is None else int(np.asarray(kv_len)[b])


def _head_dropout(dropout, b, h, H):
    return None if dropout is None else (dropout[0], dropout[1], dropout[2], b * H + h)


def forward(q, k, v, scale, causal=False, blockmask=None, kv_len=None, window=None,
            dropout=None):
    """All heads. q, k, v: [B][H][N][d] (bf16 bits or reals). Returns O, LSE (float64)."""
    B, H, N, d = q.shape
    O = np.zeros((B, H, N, d))
    LSE = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            O[b, h], LSE[b, h] = head_forward(_head_view(q, b, h), _head_view(k, b, h),
                                              _head_view(v, b, h), scale, causal, blockmask,
                                              _kv_len_b(kv_len, b), window=window,
                                              dropout=_head_dropout(dropout, b, h, H))
    return O, LSE


def backward(q, k, v, do, scale, causal=False, blockmask=None, kv_len=None, window=None,
             dropout=None):
    """All heads. Returns dict of float64 arrays: O, LSE, D, dQ, dK, dV."""
    B, H, N, d = q.shape
    res = {key: np.zeros((B, H, N, d)) for key in ("O", "dQ", "dK", "dV")}
    res["LSE"] = np.zeros((B, H, N))
    res["D"] = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            r = head_backward(_head_view(q, b, h), _head_view(k, b, h), _head_view(v, b, h),
                              _head_view(do, b, h), scale, causal, blockmask,
                              _kv_len_b(kv_len, b), window=window,
                              dropout=_head_dropout(dropout, b, h, H))
            for key in res:
                res[key][b, h] = r[key]
    return res


def forward_rows(q, k, v, scale, sel, causal=False, blockmask=None, kv_len=None,
                 window=None, dropout=None):
    """Sampled rows: ``sel`` is a sequence of (b, h, i). Returns O [len, d], LSE [len]."""
    H, d = q.shape[1], q.shape[3]
    O = np.zeros((len(sel), d))
    LSE = np.zeros(len(sel))
    for n, (b, h, i) in enumerate(sel):
        o, l = head_forward(_head_view(q, b, h), _head_view(k, b, h), _head_view(v, b, h),
                            scale, causal, blockmask, _kv_len_b(kv_len, b), rows=[i],
                            window=window, dropout=_head_dropout(dropout, b, h, H))
        O[n], LSE[n] = o[0], l[0]
    return O, LSE


def dq_rows(q, k, v, do, scale, sel, causal=False, blockmask=None, kv_len=None,
            window=None, dropout=None):
    """Sampled dQ rows (each row of dQ depends only on its own row of P and dP)."""
    H, N, d = q.shape[1], q.shape[2], q.shape[3]
    s = _scale64(scale)
    out = np.zeros((len(sel), d))
    for n, (b, h, i) in enumerate(sel):
        Qh, Kh, Vh = _head_view(q, b, h), _head_view(k, b, h), _head_view(v, b, h)
        dOi = as_f64(do[b, h, i])[None, :]
        S = _scores(Qh[[i]], Kh, s,
                    allowed([i], N, causal, blockmask, _kv_len_b(kv_len, b), window))
        lse = _logsumexp_rows(S)
        P = _probs(S, lse)
        hd = _head_dropout(dropout, b, h, H)
        ks = 1.0 if hd is None else dropout_keep([i], N, hd[3], hd[0], hd[1], hd[2]) * \
            _dropout_scale(hd[0])
        O = (P * ks) @ Vh
        D = (dOi * O).sum(axis=1)
        dP = (dOi @ Vh.T) * ks
        dS = P * (dP - D[:, None])
        out[n] = (s * (dS @ Kh))[0]
    return out


# --------------------------------------------------------------------- FP8 forward

def _e4m3_table() -> np.ndarray:
    """Value of every E4M3 code 0..255 (OCP: bias 7, subnormals, S.1111.111 = NaN)."""
    vals = np.empty(256)
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e, m = (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            vals[c] = np.nan
        elif e == 0:
            vals[c] = sign * m * 2.0 ** -9          # subnormal: m/8 * 2^-6
        else:
            vals[c] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


E4M3 = _e4m3_table()
E4M3_MAX = 448.0
FP8_P_SHIFT = 6   # log2 of the factor the probabilities are scaled by before rounding


def e4m3_decode(codes) -> np.ndarray:
    """uint8 E4M3 codes -> exact float64 values."""
    return E4M3[np.asarray(codes, dtype=np.uint8)]


def e4m3_round(x) -> np.ndarray:
    """Round float64 values with |x| <= 448 to the nearest E4M3 value, ties to the even
    code (the one whose mantissa's last bit is 0). The grid has spacing 2^-9 below 2^-6
    (subnormals) and 2^(e-3) in binade [2^e, 2^(e+1))."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    assert (a <= E4M3_MAX).all(), "outside the finite E4M3 range"
    # spacing of the grid at a: 2^-9 for a < 2^-6, else 2^(floor(log2 a) - 3)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    q = np.where(a < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.maximum(e, -6) - 3))
    n = a / q                      # exact: q is a power of two
    f = np.floor(n)
    r = n - f
    up = (r > 0.5) | ((r == 0.5) & (np.mod(f, 2) == 1))
    return np.sign(x) * (f + up) * q


def head_forward_fp8(Q8, K8, V8, descale, scale, causal=False, blockmask=None,
                     kv_len_b=None, rows=None, panel=DEFAULT_PANEL, window=None):
    """One head of the FP8 forward: Q8, K8, V8 are uint8 E4M3 codes [N][d], descale is
    (descale_q, descale_k, descale_v) (float32 values). Returns (O[rows], LSE[rows])."""
    dq_, dk_, dv_ = (float(np.float32(x)) for x in descale)
    Qh, Kh = dq_ * e4m3_decode(Q8), dk_ * e4m3_decode(K8)
    Vh = e4m3_decode(V8)
    N = Kh.shape[0]
    s = _scale64(scale)
    rows = np.arange(Qh.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    O = np.zeros((rows.size, Vh.shape[1]))
    LSE = np.zeros(rows.size)
    for r0 in range(0, rows.size, panel):
        rr = rows[r0:r0 + panel]
        S = _scores(Qh[rr], Kh, s, allowed(rr, N, causal, blockmask, kv_len_b, window))
        lse = _logsumexp_rows(S)
        live = np.isfinite(lse)
        t = S * (1.0 / np.log(2.0))
        with np.errstate(invalid="ignore"):
            m = np.ceil(np.where(live, np.max(np.where(np.isfinite(t), t, -np.inf), axis=1), 0))
        P = np.where(np.isfinite(t), np.exp2(t - m[:, None] + FP8_P_SHIFT), 0.0)
        l = P.sum(axis=1)
        Pq = e4m3_round(P)
        num = Pq @ Vh
        O[r0:r0 + rr.size] = np.where(live[:, None], dv_ * num / np.where(live, l, 1.0)[:, None], 0.0)
        LSE[r0:r0 + rr.size] = lse
    return O, LSE


def forward_fp8(q8, k8, v8, descale, scale, causal=False, blockmask=None, kv_len=None,
                window=None):
    """All heads of the FP8 forward. q8, k8, v8: uint8 E4M3 codes [B][H][N][d]."""
    B, H, N, d = q8.shape
    O = np.zeros((B, H, N, d))
    LSE = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            O[b, h], LSE[b, h] = head_forward_fp8(q8[b, h], k8[b, h], v8[b, h], descale, scale,
                                                  causal, blockmask, _kv_len_b(kv_len, b),
                                                  window=window)
    return O, LSE


def forward_fp8_rows(q8, k8, v8, descale, scale, sel, causal=False, blockmask=None,
                     kv_len=None, window=None):
    """Sampled rows of the FP8 forward: ``sel`` is a sequence of (b, h, i)."""
    d = q8.shape[3]
    O = np.zeros((len(sel), d))
    LSE = np.zeros(len(sel))
    for n, (b, h, i) in enumerate(sel):
        o, l = head_forward_fp8(q8[b, h], k8[b, h], v8[b, h], descale, scale, causal,
                                blockmask, _kv_len_b(kv_len, b), rows=[i], window=window)
        O[n], LSE[n] = o[0], l[0]
    return O, LSE


def delta(o, do):
    """D = rowsum(dO * O) over the given arrays (e.g. the bf16 O a kernel wrote)."""
    return (as_f64(o) * as_f64(do)).sum(axis=-1)

