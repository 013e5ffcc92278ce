"""Pins for the fp64 oracle: each test ties it to something other than itself.

* brute force: per-element Python loops with math.fsum / math.exp on tiny shapes,
  including shapes past one 128-wide mask block;
* a library routine: torch CPU float64 softmax attention and autograd gradients;
* closed forms: hand-derived 2x2 example (tests/golden), N = 1, constant V, causal
  row 0, causal with Q = 0 (prefix means, LSE = ln(i+1));
* invariants: rows of P sum to 1 (read through V = I), shift invariance along keys,
  D computed two ways, mask identities (full length == no padding, all-ones block
  table == dense, diagonal block table == independent 128-chunks);
* central finite differences of L = sum(dO * O) for the gradients;
* planted mistakes: perturbed copies of the backward must fail the pins above.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(shape, seed, sd=1.0):
    return sd * np.random.Generator(np.random.PCG64(seed)).standard_normal(shape)


# ---------------------------------------------------------------- brute force

def brute_forward(q, k, v, scale, ok):
    """Per-element loops: q, k, v [N][d] python floats, ok[i][j] booleans."""
    N, d = len(q), len(q[0])
    O = [[0.0] * d for _ in range(N)]
    L = [0.0] * N
    for i in range(N):
        s = {j: scale * math.fsum(q[i][c] * k[j][c] for c in range(d))
             for j in range(N) if ok[i][j]}
        if not s:
            L[i] = -math.inf
            continue
        m = max(s.values())
        z = math.fsum(math.exp(x - m) for x in s.values())
        L[i] = m + math.log(z)
        for c in range(d):
            O[i][c] = math.fsum(math.exp(s[j] - L[i]) * v[j][c] for j in s)
    return np.array(O), np.array(L)


def brute_mask(N, causal, bm, L):
    return [[(not causal or j <= i) and (bm is None or bm[i // 128][j // 128] != 0)
             and (L is None or j < L) for j in range(N)] for i in range(N)]


@pytest.mark.parametrize("N,d,causal,kpad,bm", [
    (1, 3, False, None, None),
    (5, 3, False, None, None),
    (7, 4, True, None, None),
    (6, 2, False, 4, None),
    (6, 2, True, 3, None),
    (6, 2, False, 0, None),
    (200, 2, False, None, [[1, 0], [1, 1]]),
    (200, 2, True, 150, [[1, 1], [0, 1]]),
])
def test_forward_matches_brute_force(N, d, causal, kpad, bm):
    q, k, v = rnd((N, d), 1), rnd((N, d), 2), rnd((N, d), 3)
    scale = 0.7
    bmask = None if bm is None else np.array(bm, dtype=np.uint8)
    O, L = orc.head_forward(q, k, v, scale, causal, bmask, kpad)
    Ob, Lb = brute_forward(q.tolist(), k.tolist(), v.tolist(),
                           float(np.float32(scale)), brute_mask(N, causal, bm, kpad))
    np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-12)
    fin = np.isfinite(Lb)
    assert np.array_equal(np.isfinite(L), fin)
    np.testing.assert_allclose(L[fin], Lb[fin], rtol=0, atol=1e-12)


# ----------------------------------------------------- library routine (torch)

def torch_reference(q, k, v, do, scale, ok):
    import torch
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    bias = torch.zeros(ok.shape, dtype=torch.float64)
    bias[~torch.tensor(ok)] = -math.inf
    S = float(np.float32(scale)) * (tq @ tk.T) + bias
    O = torch.softmax(S, dim=-1) @ tv
    lse = torch.logsumexp(S, dim=-1)
    (O * torch.tensor(do)).sum().backward()
    return O.detach().numpy(), lse.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(), \
        tv.grad.numpy()


@pytest.mark.parametrize("N,d,causal,kpad,bm", [
    (64, 16, False, None, None),
    (97, 32, True, None, None),
    (150, 8, False, 77, None),
    (256, 16, True, None, [[1, 0], [1, 1]]),
    (256, 16, False, 200, [[1, 1], [0, 1]]),
])
def test_matches_torch_float64_autograd(N, d, causal, kpad, bm):
    q, k, v, do = (rnd((N, d), s) for s in (11, 12, 13, 14))
    scale = 1.0 / math.sqrt(d)
    bmask = None if bm is None else np.array(bm, dtype=np.uint8)
    ok = orc.allowed(np.arange(N), N, causal, bmask, kpad)
    assert ok.any(axis=1).all()  # torch's softmax of an all -inf row is NaN
    O, L, dq, dk, dv = torch_reference(q, k, v, do, scale, ok)
    r = orc.head_backward(q, k, v, do, scale, causal, bmask, kpad)
    for a, b in ((r["O"], O), (r["LSE"], L), (r["dQ"], dq), (r["dK"], dk), (r["dV"], dv)):
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-11)


# --------------------------------------------------------------- closed forms

def _golden_value(x):
    if isinstance(x, str):
        table = {"ln3": math.log(3), "ln4": math.log(4), "ln2": math.log(2),
                 "0.75*ln3": 0.75 * math.log(3), "-2*ln3": -2 * math.log(3)}
        return table[x]
    return float(x)


def _golden_array(rows):
    return np.array([[_golden_value(x) for x in r] if isinstance(r, list) else _golden_value(r)
                     for r in rows])


def test_hand_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "hand_example_2x2.json")))
    q, k, v, do = (_golden_array(g[n]) for n in ("q", "k", "v", "do"))
    for case, exp in g["cases"].items():
        r = orc.head_backward(q, k, v, do, g["scale"], causal=(case == "causal"))
        for key, name in (("o", "O"), ("lse", "LSE"), ("dq", "dQ"), ("dk", "dK"), ("dv", "dV")):
            np.testing.assert_allclose(r[name], _golden_array(exp[key]), rtol=0, atol=1e-14,
                                       err_msg=f"{case}/{key}")


def test_single_key_and_query():
    q, k, v, do = (rnd((1, 8), s) for s in (1, 2, 3, 4))
    r = orc.head_backward(q, k, v, do, 0.3)
    np.testing.assert_allclose(r["O"], v, atol=1e-15)
    np.testing.assert_allclose(r["LSE"], [float(np.float32(0.3)) * (q[0] @ k[0])], atol=1e-15)
    np.testing.assert_allclose(r["dQ"], 0, atol=1e-15)
    np.testing.assert_allclose(r["dK"], 0, atol=1e-15)
    np.testing.assert_allclose(r["dV"], do, atol=1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_constant_v_gives_constant_rows(causal):
    N, d = 300, 16
    q, k = rnd((N, d), 5), rnd((N, d), 6)
    row = rnd((d,), 7)
    v = np.tile(row, (N, 1))
    O, _ = orc.head_forward(q, k, v, 0.25, causal)
    np.testing.assert_allclose(O, np.tile(row, (N, 1)), atol=1e-12)


def test_causal_row_zero():
    N, d = 130, 8
    q, k, v = rnd((N, d), 8), rnd((N, d), 9), rnd((N, d), 10)
    O, L = orc.head_forward(q, k, v, 0.5, causal=True)
    np.testing.assert_allclose(O[0], v[0], atol=1e-15)
    np.testing.assert_allclose(L[0], 0.5 * (q[0] @ k[0]), atol=1e-14)


@pytest.mark.parametrize("kpad", [None, 100])
def test_causal_zero_query_prefix_mean(kpad):
    N, d = 260, 8
    q = np.zeros((N, d))
    k, v = rnd((N, d), 15), rnd((N, d), 16)
    O, L = orc.head_forward(q, k, v, 0.125, causal=True, kv_len_b=kpad)
    cnt = np.arange(1, N + 1) if kpad is None else np.minimum(np.arange(1, N + 1), kpad)
    expect = np.cumsum(v, axis=0)[cnt - 1] / cnt[:, None]
    np.testing.assert_allclose(O, expect, atol=1e-12)
    np.testing.assert_allclose(L, np.log(cnt), atol=1e-13)


# ----------------------------------------------------------------- invariants

@pytest.mark.parametrize("causal,kpad,bm", [(False, None, None), (True, None, None),
                                            (False, 90, None), (True, None, [[1, 0], [1, 1]])])
def test_probability_rows_sum_to_one(causal, kpad, bm):
    N = 160
    d = N  # V = identity makes O equal to P
    q, k = rnd((N, d), 20), rnd((N, d), 21)
    bmask = None if bm is None else np.array(bm, dtype=np.uint8)
    P, _ = orc.head_forward(q, k, np.eye(N), 0.1, causal, bmask, kpad)
    ok = orc.allowed(np.arange(N), N, causal, bmask, kpad)
    np.testing.assert_allclose(P.sum(axis=1), 1.0, atol=1e-12)
    assert (P >= 0).all()
    assert (P[~ok] == 0).all()


@pytest.mark.parametrize("causal", [False, True])
def test_shift_invariance_along_keys(causal):
    N, d = 200, 12
    q, k, v = rnd((N, d), 30), rnd((N, d), 31), rnd((N, d), 32)
    u = rnd((d,), 33)
    s = 0.2
    O1, L1 = orc.head_forward(q, k, v, s, causal)
    O2, L2 = orc.head_forward(q, k + u[None, :], v, s, causal)
    np.testing.assert_allclose(O2, O1, atol=1e-12)
    np.testing.assert_allclose(L2 - L1, float(np.float32(s)) * (q @ u), atol=1e-12)


def test_delta_two_ways():
    N, d = 180, 16
    q, k, v, do = (rnd((N, d), s) for s in (40, 41, 42, 43))
    r = orc.head_backward(q, k, v, do, 0.25, causal=True)
    P, _ = orc.head_forward(q, k, np.eye(N), 0.25, causal=True)  # V = I -> P
    dP = do @ v.T
    np.testing.assert_allclose(r["D"], (P * dP).sum(axis=1), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(r["D"], orc.delta(r["O"], do), rtol=1e-12, atol=1e-12)


def test_full_length_padding_is_no_padding():
    N, d = 140, 8
    q, k, v = rnd((N, d), 50), rnd((N, d), 51), rnd((N, d), 52)
    a = orc.head_forward(q, k, v, 0.3, kv_len_b=N)
    b = orc.head_forward(q, k, v, 0.3)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_padding_equals_attention_on_prefix():
    N, d, L = 150, 8, 61
    q, k, v, do = (rnd((N, d), s) for s in (53, 54, 55, 56))
    a = orc.head_backward(q, k, v, do, 0.3, kv_len_b=L)
    # reference: N queries against the first L keys only
    O, Lse = orc.head_forward(q, k[:L], v[:L], 0.3)
    np.testing.assert_allclose(a["O"], O, atol=1e-12)
    np.testing.assert_allclose(a["LSE"], Lse, atol=1e-12)
    assert (a["dK"][L:] == 0).all() and (a["dV"][L:] == 0).all()


def test_all_ones_block_mask_is_dense():
    N, d = 300, 8
    q, k, v = rnd((N, d), 60), rnd((N, d), 61), rnd((N, d), 62)
    bm = np.ones((3, 3), dtype=np.uint8)
    for causal in (False, True):
        a = orc.head_forward(q, k, v, 0.4, causal, bm)
        b = orc.head_forward(q, k, v, 0.4, causal)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_diagonal_block_mask_is_chunked_attention():
    N, d = 300, 8
    q, k, v, do = (rnd((N, d), s) for s in (63, 64, 65, 66))
    bm = np.eye(3, dtype=np.uint8)
    r = orc.head_backward(q, k, v, do, 0.4, blockmask=bm)
    for c0 in range(0, N, 128):
        sl = slice(c0, min(N, c0 + 128))
        rc = orc.head_backward(q[sl], k[sl], v[sl], do[sl], 0.4)
        for key in ("O", "LSE", "dQ", "dK", "dV"):
            np.testing.assert_allclose(r[key][sl], rc[key], atol=1e-12)


def test_fully_masked_rows():
    N, d = 40, 8
    q, k, v, do = (rnd((N, d), s) for s in (70, 71, 72, 73))
    r = orc.head_backward(q, k, v, do, 0.5, kv_len_b=0)
    assert (r["O"] == 0).all() and np.isneginf(r["LSE"]).all()
    for key in ("dQ", "dK", "dV", "D"):
        assert (r[key] == 0).all()
    # a block table that leaves query block 1 with no key block
    N = 200
    q, k, v, do = (rnd((N, d), s) for s in (74, 75, 76, 77))
    bm = np.array([[1, 0], [0, 0]], dtype=np.uint8)
    r = orc.head_backward(q, k, v, do, 0.5, blockmask=bm)
    assert (r["O"][128:] == 0).all() and np.isneginf(r["LSE"][128:]).all()
    assert (r["dQ"][128:] == 0).all() and (r["dK"][128:] == 0).all()


# ----------------------------------------------------------- finite differences

def _loss(q, k, v, do, scale, causal, kpad):
    O, _ = orc.head_forward(q, k, v, scale, causal, None, kpad)
    return float((do * O).sum())


@pytest.mark.parametrize("causal,kpad", [(False, None), (True, None), (False, 9)])
def test_gradients_match_central_differences(causal, kpad):
    N, d = 13, 5
    q, k, v, do = (rnd((N, d), s) for s in (80, 81, 82, 83))
    scale = 0.6
    r = orc.head_backward(q, k, v, do, scale, causal, None, kpad)
    rng = np.random.Generator(np.random.PCG64(84))
    h = 1e-6
    for name, x, g in (("q", q, r["dQ"]), ("k", k, r["dK"]), ("v", v, r["dV"])):
        for _ in range(12):
            i, c = int(rng.integers(N)), int(rng.integers(d))
            xp, xm = x.copy(), x.copy()
            xp[i, c] += h
            xm[i, c] -= h
            args = {"q": q, "k": k, "v": v}
            fp = _loss(*(xp if n == name else args[n] for n in "qkv"), do, scale, causal, kpad)
            fm = _loss(*(xm if n == name else args[n] for n in "qkv"), do, scale, causal, kpad)
            fd = (fp - fm) / (2 * h)
            assert abs(fd - g[i, c]) <= 1e-6 * max(1.0, abs(g[i, c])), (name, i, c, fd, g[i, c])


# ------------------------------------------------------------- sampled entries

def test_sampled_rows_agree_with_full():
    B, H, N, d = 2, 2, 160, 16
    q, k, v, do = (rnd((B, H, N, d), s) for s in (90, 91, 92, 93))
    kv = np.array([160, 97], dtype=np.int32)
    full = orc.backward(q, k, v, do, 0.25, causal=True, kv_len=kv)
    sel = [(0, 1, 0), (1, 0, 5), (1, 1, 159), (0, 0, 128)]
    O, L = orc.forward_rows(q, k, v, 0.25, sel, causal=True, kv_len=kv)
    dq = orc.dq_rows(q, k, v, do, 0.25, sel, causal=True, kv_len=kv)
    for n, (b, h, i) in enumerate(sel):
        np.testing.assert_allclose(O[n], full["O"][b, h, i], atol=1e-13)
        np.testing.assert_allclose(L[n], full["LSE"][b, h, i], atol=1e-13)
        np.testing.assert_allclose(dq[n], full["dQ"][b, h, i], atol=1e-13)


def test_bf16_widening_is_exact():
    bits = np.array([0x3F80, 0xBF80, 0x0000, 0x8000, 0x7F7F, 0x0001, 0x4049], dtype=np.uint16)
    want = [1.0, -1.0, 0.0, -0.0, 3.3895313892515355e38, 9.183549615799121e-41, 3.140625]
    np.testing.assert_array_equal(orc.widen_bf16(bits), want)


# ------------------------------------------------------------ planted mistakes

def _mutant_backward(kind):
    """Copies of the oracle's backward with one plausible mistake each."""
    def run(Qh, Kh, Vh, dOh, scale, causal=False):
        N = Kh.shape[0]
        s = float(np.float32(scale))
        S = s * (Qh @ Kh.T)
        S[~orc.allowed(np.arange(N), N, causal, None, None)] = -np.inf
        m = S.max(axis=1, keepdims=True)
        P = np.exp(S - m)
        P /= P.sum(axis=1, keepdims=True)
        O = P @ Vh
        D = (dOh * O).sum(axis=1)
        dP = dOh @ Vh.T
        dS = P * (dP - D[:, None])
        dQ, dK, dV = s * (dS @ Kh), s * (dS.T @ Qh), P.T @ dOh
        if kind == "drop_delta":
            dS = P * dP
            dQ, dK = s * (dS @ Kh), s * (dS.T @ Qh)
        elif kind == "transposed_dk":
            dK = s * (dS @ Qh)
        elif kind == "missing_scale":
            dQ = dS @ Kh
        elif kind == "dv_not_transposed":
            dV = P @ dOh
        elif kind == "delta_sign":
            dS = P * (dP + D[:, None])
            dQ, dK = s * (dS @ Kh), s * (dS.T @ Qh)
        return {"dQ": dQ, "dK": dK, "dV": dV}
    return run


@pytest.mark.parametrize("kind", ["drop_delta", "transposed_dk", "missing_scale",
                                  "dv_not_transposed", "delta_sign"])
def test_planted_backward_mistakes_are_caught(kind):
    """Each mutant must disagree with the finite-difference gradient somewhere."""
    N, d = 9, 9
    q, k, v, do = (rnd((N, d), s) for s in (100, 101, 102, 103))
    scale = 0.6
    mut = _mutant_backward(kind)(q, k, v, do, scale, causal=True)
    good = _mutant_backward("none")(q, k, v, do, scale, causal=True)
    h = 1e-6
    worst_mut, worst_good = 0.0, 0.0
    for name, x in (("q", q), ("k", k), ("v", v)):
        g_key = {"q": "dQ", "k": "dK", "v": "dV"}[name]
        for i in range(N):
            for c in range(0, d, 4):
                xp, xm = x.copy(), x.copy()
                xp[i, c] += h
                xm[i, c] -= h
                args = {"q": q, "k": k, "v": v}
                fp = _loss(*(xp if n == name else args[n] for n in "qkv"), do, scale, True, None)
                fm = _loss(*(xm if n == name else args[n] for n in "qkv"), do, scale, True, None)
                fd = (fp - fm) / (2 * h)
                worst_mut = max(worst_mut, abs(fd - mut[g_key][i, c]))
                worst_good = max(worst_good, abs(fd - good[g_key][i, c]))
    assert worst_good < 1e-6
    assert worst_mut > 1e-3


def test_planted_forward_mistakes_are_caught():
    """Forward mutants (no max subtraction is harmless; these are not) fail the pins."""
    N, d = 260, 8
    q = np.zeros((N, d))
    k, v = rnd((N, d), 110), rnd((N, d), 111)
    cnt = np.arange(1, N + 1)
    expect = np.cumsum(v, axis=0) / cnt[:, None]
    # causal off by one (j < i instead of j <= i) breaks the prefix-mean closed form
    ok = np.tril(np.ones((N, N), dtype=bool), -1)
    ok[0, 0] = True
    S = np.where(ok, 0.0, -np.inf)
    P = np.exp(S - S.max(axis=1, keepdims=True))
    P /= P.sum(axis=1, keepdims=True)
    assert np.abs(P @ v - expect).max() > 1e-3
    # the real oracle passes it
    O, _ = orc.head_forward(q, k, v, 0.125, causal=True)
    assert np.abs(O - expect).max() < 1e-12


# ------------------------------------------------------------- sliding window
# Reading: key j is allowed for query i iff i - left <= j <= i + right (negative = no
# limit on that side); "IO感知计算如何重塑Transformer内存优化技术格局" (bxzpzcl.cn), section
# 高级功能配置, lists sliding-window attention without defining it.

def brute_window_mask(N, causal, L, left, right):
    rows = []
    for i in range(N):
        row = []
        for j in range(N):
            keep = True
            if causal and j > i:
                keep = False
            if L is not None and j >= L:
                keep = False
            if left >= 0 and i - j > left:
                keep = False
            if right >= 0 and j - i > right:
                keep = False
            row.append(keep)
        rows.append(row)
    return rows


@pytest.mark.parametrize("N,d,causal,kpad,window", [
    (6, 3, False, None, (0, 0)),
    (7, 2, False, None, (2, 0)),
    (7, 2, False, None, (0, 3)),
    (9, 3, False, None, (3, 2)),
    (9, 3, True, None, (3, 2)),
    (8, 2, False, 5, (-1, 2)),
    (8, 2, True, 6, (4, -1)),
    (150, 2, False, None, (40, 70)),
])
def test_window_matches_brute_force(N, d, causal, kpad, window):
    q, k, v = rnd((N, d), 31), rnd((N, d), 32), rnd((N, d), 33)
    scale = 0.8
    O, L = orc.head_forward(q, k, v, scale, causal, None, kpad, window=window)
    Ob, Lb = brute_forward(q.tolist(), k.tolist(), v.tolist(), float(np.float32(scale)),
                           brute_window_mask(N, causal, kpad, *window))
    np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-12)
    fin = np.isfinite(Lb)
    assert np.array_equal(np.isfinite(L), fin)
    np.testing.assert_allclose(L[fin], Lb[fin], rtol=0, atol=1e-12)


def test_window_zero_attends_to_itself():
    # Window (0, 0): each query sees only its own key, so O_i = V_i and
    # LSE_i = scale * q_i . k_i, and dQ = dK = 0 (a single-key softmax is constant).
    N, d = 37, 6
    q, k, v, do = (rnd((N, d), s) for s in (41, 42, 43, 44))
    s = float(np.float32(0.5))
    r = orc.head_backward(q, k, v, do, 0.5, window=(0, 0))
    np.testing.assert_allclose(r["O"], v, atol=1e-14)
    np.testing.assert_allclose(r["LSE"], s * (q * k).sum(axis=1), atol=1e-13)
    np.testing.assert_allclose(r["dV"], do, atol=1e-14)
    assert np.abs(r["dQ"]).max() < 1e-13 and np.abs(r["dK"]).max() < 1e-13


def test_window_identities():
    N, d = 90, 8
    q, k, v, do = (rnd((N, d), s) for s in (51, 52, 53, 54))
    none = orc.head_backward(q, k, v, do, 0.3)
    causal = orc.head_backward(q, k, v, do, 0.3, causal=True)
    for win, ref in (((-1, -1), none), ((N, N), none), ((-1, 0), causal), ((N, 0), causal)):
        r = orc.head_backward(q, k, v, do, 0.3, window=win)
        for key in ("O", "LSE", "dQ", "dK", "dV"):
            np.testing.assert_array_equal(r[key], ref[key])


@pytest.mark.parametrize("left,right", [(5, 3), (0, 7), (11, 0), (4, 4)])
def test_window_rows_are_attention_on_a_key_slice(left, right):
    # Row i with a window is plain (unmasked) softmax attention over the contiguous keys
    # max(0, i-left) .. min(N-1, i+right), computed here with torch on each slice.
    import torch
    N, d = 40, 5
    q, k, v = rnd((N, d), 61), rnd((N, d), 62), rnd((N, d), 63)
    s = float(np.float32(0.9))
    O, L = orc.head_forward(q, k, v, 0.9, window=(left, right))
    for i in range(N):
        lo, hi = max(0, i - left), min(N, i + right + 1)
        S = s * (torch.tensor(q[i]) @ torch.tensor(k[lo:hi]).T)
        np.testing.assert_allclose(O[i], (torch.softmax(S, -1) @ torch.tensor(v[lo:hi])).numpy(),
                                   atol=1e-13)
        np.testing.assert_allclose(L[i], torch.logsumexp(S, -1).item(), atol=1e-13)


def test_window_gradients_match_central_differences():
    N, d, win = 15, 4, (3, 2)
    q, k, v, do = (rnd((N, d), s) for s in (71, 72, 73, 74))
    scale = 0.7
    r = orc.head_backward(q, k, v, do, scale, window=win)

    def loss(qq, kk, vv):
        O, _ = orc.head_forward(qq, kk, vv, scale, window=win)
        return float((do * O).sum())

    rng = np.random.Generator(np.random.PCG64(75))
    h = 1e-6
    for idx, g in ((0, r["dQ"]), (1, r["dK"]), (2, r["dV"])):
        for _ in range(10):
            i, c = int(rng.integers(N)), int(rng.integers(d))
            args_p = [q.copy(), k.copy(), v.copy()]
            args_m = [q.copy(), k.copy(), v.copy()]
            args_p[idx][i, c] += h
            args_m[idx][i, c] -= h
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(fd - g[i, c]) <= 1e-6 * max(1.0, abs(g[i, c])), (idx, i, c)


def test_planted_window_off_by_one_is_caught():
    # A mask that keeps one key too few on the left (j > i - left) must fail the slice pin.
    N, d, left, right = 20, 3, 4, 2
    q, k, v = rnd((N, d), 81), rnd((N, d), 82), rnd((N, d), 83)
    s = float(np.float32(1.0))
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    ok = (j > i - left) & (j <= i + right)
    S = s * (q @ k.T)
    S[~ok] = -np.inf
    P = np.exp(S - S.max(1, keepdims=True))
    O_bad = (P / P.sum(1, keepdims=True)) @ v
    O, _ = orc.head_forward(q, k, v, 1.0, window=(left, right))
    assert np.abs(O_bad - O).max() > 1e-3


def test_f16_inputs_widen_exactly():
    # fp16 tensors reach the oracle as numpy float16 arrays: 1, -2, the largest finite
    # value, the smallest subnormal and pi rounded to binary16.
    bits = np.array([0x3C00, 0xC000, 0x7BFF, 0x0001, 0x4248], dtype=np.uint16)
    want = [1.0, -2.0, 65504.0, 2.0 ** -24, 3.140625]
    np.testing.assert_array_equal(orc.as_f64(bits.view(np.float16)), want)


# ------------------------------------------------------------------ dropout
# Reading (dropout fused, mask regenerated in backward): P_drop = P * keep / (1 - p) with
# keep from Philox4x32-10 (Salmon et al., SC 2011); see the oracle's header.

def test_philox_known_answer_vectors():
    # The generator's published known-answer vectors (counter, key -> output).
    cases = [((0, 0, 0, 0), (0, 0), (0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8)),
             ((0xffffffff,) * 4, (0xffffffff,) * 2,
              (0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd)),
             ((0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344), (0xa4093822, 0x299f31d0),
              (0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1))]
    for c, k, want in cases:
        got = orc.philox4x32_10(*[np.array([x]) for x in c], *k)
        assert [int(w[0]) for w in got] == list(want)


def test_dropout_keep_fraction_and_streams():
    rows = np.arange(256)
    for p in (0.0, 0.25, 0.75):
        keep = orc.dropout_keep(rows, 256, 3, p, 1234, 0)
        n = keep.size
        frac = keep.mean()
        sigma = math.sqrt(p * (1 - p) / n) if 0 < p < 1 else 0.0
        assert abs(frac - (1 - p)) <= 5 * sigma + 1e-12, (p, frac)
    base = orc.dropout_keep(rows, 256, 3, 0.5, 1234, 0)
    for other in (orc.dropout_keep(rows, 256, 4, 0.5, 1234, 0),     # another head
                  orc.dropout_keep(rows, 256, 3, 0.5, 1235, 0),     # another seed
                  orc.dropout_keep(rows, 256, 3, 0.5, 1234, 1),     # another offset
                  orc.dropout_keep(rows, 256, 3, 0.5, 1234 + (1 << 32), 0)):  # seed high word
        diff = (base != other).mean()
        assert abs(diff - 0.5) < 0.02, diff                           # independent streams
    assert orc.dropout_keep(rows, 256, 3, 0.999999, 1234, 0).mean() < 1e-4


def test_dropout_draw_layout_and_threshold_by_hand():
    # Element (i, j) of head bh takes the 16-bit half (low for even i, high for odd i) of
    # output word j % 4 of the call with counter (j // 4, i // 2, bh, offset); it is kept
    # iff that draw r >= floor(p * 2^16). Worked through for single elements with plain
    # integers, and p placed on both sides of the boundary r / 2^16.
    seed, bh, off = 0x0123_4567_89AB_CDEF, 6, 11
    for i, j in ((0, 0), (1, 0), (5, 13), (6, 13), (200, 77), (201, 78), (37, 255)):
        words = orc.philox4x32_10(np.array([j // 4]), np.array([i // 2]), np.array([bh]),
                                  np.array([off]), seed & 0xFFFFFFFF, seed >> 32)
        word = int(words[j % 4][0])
        r = (word >> 16) if i % 2 else (word & 0xFFFF)
        rows = np.array([i])
        # p exactly r / 2^16 (float32 represents it exactly): floor(p 2^16) = r, kept.
        assert orc.dropout_keep(rows, j + 1, bh, r / 65536.0, seed, off)[0, j]
        if r < 65535:   # one step above: threshold r + 1 > r, dropped
            assert not orc.dropout_keep(rows, j + 1, bh, (r + 1) / 65536.0, seed, off)[0, j]


def test_dropout_zero_is_no_dropout():
    N, d = 70, 8
    q, k, v, do = (rnd((N, d), s) for s in (91, 92, 93, 94))
    a = orc.head_backward(q, k, v, do, 0.4, causal=True)
    b = orc.head_backward(q, k, v, do, 0.4, causal=True, dropout=(0.0, 77, 5, 2))
    for key in ("O", "LSE", "dQ", "dK", "dV", "D"):
        np.testing.assert_array_equal(a[key], b[key])


def test_dropout_forward_matches_brute_force():
    N, d, p = 11, 3, 0.3
    q, k, v = rnd((N, d), 95), rnd((N, d), 96), rnd((N, d), 97)
    keep = orc.dropout_keep(np.arange(N), N, 1, p, 99, 7)
    O, L = orc.head_forward(q, k, v, 0.8, dropout=(p, 99, 7, 1))
    s = float(np.float32(0.8))
    rp = 1.0 / (1.0 - float(np.float32(p)))
    for i in range(N):
        sc = [s * math.fsum(q[i][c] * k[j][c] for c in range(d)) for j in range(N)]
        m = max(sc)
        z = math.fsum(math.exp(x - m) for x in sc)
        assert abs(L[i] - (m + math.log(z))) < 1e-12               # LSE ignores dropout
        for c in range(d):
            want = rp * math.fsum(math.exp(sc[j] - m) / z * v[j][c] for j in range(N)
                                  if keep[i, j])
            assert abs(O[i, c] - want) < 1e-12


def test_dropout_gradients_match_central_differences():
    N, d, drop = 14, 4, (0.35, 2024, 3, 5)
    q, k, v, do = (rnd((N, d), s) for s in (101, 102, 103, 104))
    scale = 0.7
    r = orc.head_backward(q, k, v, do, scale, causal=True, dropout=drop)

    def loss(qq, kk, vv):
        O, _ = orc.head_forward(qq, kk, vv, scale, causal=True, dropout=drop)
        return float((do * O).sum())

    rng = np.random.Generator(np.random.PCG64(105))
    h = 1e-6
    for idx, g in ((0, r["dQ"]), (1, r["dK"]), (2, r["dV"])):
        for _ in range(10):
            i, c = int(rng.integers(N)), int(rng.integers(d))
            ap = [q.copy(), k.copy(), v.copy()]
            am = [q.copy(), k.copy(), v.copy()]
            ap[idx][i, c] += h
            am[idx][i, c] -= h
            fd = (loss(*ap) - loss(*am)) / (2 * h)
            assert abs(fd - g[i, c]) <= 1e-6 * max(1.0, abs(g[i, c])), (idx, i, c)


def test_dropout_delta_two_ways():
    # D = rowsum(dO * O) equals sum_j P_drop_ij (dO V^T)_ij.
    N, d, drop = 40, 6, (0.5, 7, 0, 0)
    q, k, v, do = (rnd((N, d), s) for s in (111, 112, 113, 114))
    r = orc.head_backward(q, k, v, do, 0.3, dropout=drop)
    s = float(np.float32(0.3))
    S = s * (q @ k.T)
    P = np.exp(S - S.max(1, keepdims=True))
    P /= P.sum(1, keepdims=True)
    Pd = P * orc.dropout_keep(np.arange(N), N, 0, 0.5, 7, 0) * 2.0
    np.testing.assert_allclose(r["D"], (Pd * (do @ v.T)).sum(1), atol=1e-12)


# ------------------------------------------------------------------ FP8 forward
# Reading: Q, K, V as OCP E4M3 codes with per-tensor descales; the scaled probability
# P = 2^(t - ceil(max t) + 6) is rounded to E4M3 (nearest, ties to even) before P V; l and
# LSE use the unrounded P.

def test_e4m3_decode_matches_torch_and_known_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = orc.e4m3_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[~np.isnan(got)], ref[~np.isnan(ref)])
    known = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
             0x3C: 1.5, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0}
    for c, v in known.items():
        assert orc.e4m3_decode(np.uint8(c)) == v
    assert np.isnan(orc.e4m3_decode(np.uint8(0x7F))) and np.isnan(orc.e4m3_decode(np.uint8(0xFF)))


def test_e4m3_round_matches_torch_nearest_even():
    rng = np.random.Generator(np.random.PCG64(131))
    x = np.concatenate([
        rng.uniform(-448, 448, 20000),
        rng.standard_normal(20000) * 2.0 ** rng.integers(-14, 8, 20000),
    ]).astype(np.float32)
    x = x[np.abs(x) <= 448]
    grid = orc.E4M3[:127]                                  # 0 .. 448
    mids = ((grid[:-1] + grid[1:]) / 2).astype(np.float32)  # exact ties, representable
    x = np.concatenate([x, mids, -mids, grid.astype(np.float32)])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(orc.e4m3_round(x.astype(np.float64)), ref)
    # hand-worked ties: 1 + 1/16 -> 1 (even), 1 + 3/16 -> 1.25, 2^-10 -> 0, 3 * 2^-10 -> 2^-8
    assert list(orc.e4m3_round(np.array([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10]))) == \
        [1.0, 1.25, 0.0, 2.0 ** -8]


def _fp8_codes(shape, seed, sd=1.0):
    rng = np.random.Generator(np.random.PCG64(seed))
    x = (sd * rng.standard_normal(shape)).astype(np.float32)
    return torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_fp8_forward_matches_brute_force():
    N, d = 13, 8
    q8, k8, v8 = _fp8_codes((N, d), 133), _fp8_codes((N, d), 134), _fp8_codes((N, d), 135)
    desc = (0.75, 1.25, 0.5)
    s = float(np.float32(0.6))
    O, L = orc.head_forward_fp8(q8, k8, v8, desc, 0.6, causal=True)
    dec = lambda c: float(torch.tensor([int(c)], dtype=torch.uint8).view(torch.float8_e4m3fn).double())
    for i in range(N):
        sc = [s * math.fsum(0.75 * dec(q8[i, c]) * 1.25 * dec(k8[j, c]) for c in range(d))
              for j in range(i + 1)]
        t = [x / math.log(2.0) for x in sc]
        m = math.ceil(max(t))
        P = [2.0 ** (x - m + 6) for x in t]
        Pq = [float(torch.tensor([p], dtype=torch.float32).to(torch.float8_e4m3fn).double())
              for p in P]
        l = math.fsum(P)
        assert abs(L[i] - ((m - 6) * math.log(2.0) + math.log(l))) < 1e-12
        for c in range(d):
            want = 0.5 * math.fsum(Pq[j] * dec(v8[j, c]) for j in range(i + 1)) / l
            assert abs(O[i, c] - want) < 1e-12, (i, c)


def test_fp8_forward_equal_scores_closed_form():
    # Identical keys: every P_j = p0 = 2^(t0 - ceil t0 + 6), so
    # O = descale_v * (Pq0 / p0) * mean(V).
    N, d = 40, 16
    q8 = _fp8_codes((N, d), 137)
    k8 = np.repeat(_fp8_codes((1, d), 138), N, axis=0)
    v8 = _fp8_codes((N, d), 139)
    desc = (1.0, 0.5, 2.0)
    O, L = orc.head_forward_fp8(q8, k8, v8, desc, 0.3)
    Q, K = orc.e4m3_decode(q8), 0.5 * orc.e4m3_decode(k8)
    t0 = float(np.float32(0.3)) * (Q @ K[0]) / math.log(2.0)
    p0 = 2.0 ** (t0 - np.ceil(t0) + 6)
    ratio = orc.e4m3_round(p0) / p0
    want = 2.0 * ratio[:, None] * orc.e4m3_decode(v8).mean(axis=0)[None, :]
    np.testing.assert_allclose(O, want, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(L, float(np.float32(0.3)) * (Q @ K[0]) + math.log(N), atol=1e-12)


def test_fp8_forward_is_plain_attention_within_the_rounding_of_p():
    # |O_fp8 - O| <= descale_v * (2^-4 sum_j P_j |V_j| + 2^-10 sum_j |V_j|) / l, from
    # |Pq - P| <= max(2^-4 P, 2^-10) for the scaled P = 2^(t - m + 6); LSE is unchanged.
    N, d = 200, 32
    q8, k8, v8 = (_fp8_codes((1, 2, N, d), s) for s in (141, 142, 143))
    desc = (0.9, 1.1, 0.7)
    O, L = orc.forward_fp8(q8, k8, v8, desc, 0.2, causal=True)
    q, k = desc[0] * orc.e4m3_decode(q8), desc[1] * orc.e4m3_decode(k8)
    v = orc.e4m3_decode(v8)
    O0, L0 = orc.forward(q, k, desc[2] * v, 0.2, causal=True)
    np.testing.assert_allclose(L, L0, atol=1e-12)
    Oa, _ = orc.forward(q, k, np.abs(v), 0.2, causal=True)     # sum_j P_j |V_j| / l
    t = np.float32(0.2) * np.einsum("bhid,bhjd->bhij", q, k) / math.log(2.0)
    t = np.where(np.tril(np.ones((N, N), bool)), t, -np.inf)
    m = np.ceil(t.max(-1))
    l = np.exp2(t - m[..., None] + 6).sum(-1)
    csum = np.cumsum(np.abs(v), axis=2)                          # causal sum_j |V_j|
    bound = desc[2] * (2.0 ** -4 * Oa + 2.0 ** -10 * csum / l[..., None])
    assert (np.abs(O - O0) <= bound + 1e-12).all()
    assert np.abs(O - O0).max() > 0                              # the rounding is there


def test_planted_fp8_mistakes_are_caught():
    # Truncation instead of nearest rounding, and a forgotten descale_v, each change the
    # result the brute-force pin fixes. (A floor instead of a ceiling for the reference is
    # no mistake: any power-of-two reference rounds the same in the normal range.)
    N, d = 13, 8
    q8, k8, v8 = _fp8_codes((N, d), 133), _fp8_codes((N, d), 134), _fp8_codes((N, d), 135)
    ref, _ = orc.head_forward_fp8(q8, k8, v8, (0.75, 1.25, 0.5), 0.6, causal=True)
    orig_round, orig_ceil = orc.e4m3_round, np.ceil
    try:
        orc.e4m3_round = lambda x: np.sign(x) * np.floor(np.abs(x) * 8) / 8  # truncation-ish
        bad, _ = orc.head_forward_fp8(q8, k8, v8, (0.75, 1.25, 0.5), 0.6, causal=True)
        assert np.abs(bad - ref).max() > 1e-6
    finally:
        orc.e4m3_round = orig_round
    bad, _ = orc.head_forward_fp8(q8, k8, v8, (0.75, 1.25, 1.0), 0.6, causal=True)
    assert np.abs(bad - ref).max() > 1e-6


def test_planted_fp8_unscaled_probabilities_are_caught():
    # Rounding 2^(t - m) instead of 2^(t - m + 6) changes every probability below 2^-6 of the
    # row maximum (subnormal for the unscaled one, normal for the scaled one): on wide scores
    # the two definitions differ, so the brute-force pin above fixes the shift.
    N, d = 40, 16
    q8, k8, v8 = (_fp8_codes((1, 1, N, d), s, sd=2.0) for s in (145, 146, 147))
    desc = (1.0, 1.0, 0.5)
    ref, _ = orc.forward_fp8(q8, k8, v8, desc, 0.35)
    old = orc.FP8_P_SHIFT
    try:
        orc.FP8_P_SHIFT = 0
        bad, _ = orc.forward_fp8(q8, k8, v8, desc, 0.35)
    finally:
        orc.FP8_P_SHIFT = old
    assert np.abs(bad - ref).max() > 1e-6


@pytest.mark.parametrize("causal,window,kv,bm", [
    (True, None, None, None),
    (False, (50, 10), [300, 170], None),
    (True, None, [300, 99], [[1, 0, 1], [1, 1, 0], [0, 1, 1]]),
])
def test_fp8_rows_equal_the_whole_forward(causal, window, kv, bm):
    # forward_fp8_rows (sampled rows, used at sizes where the whole forward is too slow)
    # returns the rows of forward_fp8, up to the fp64 summation order of a one-row product
    # against a whole-panel one (a few ulp).
    N, d = 300, 32
    B = 1 if kv is None else len(kv)
    q8, k8, v8 = (_fp8_codes((B, 2, N, d), s) for s in (148, 149, 150))
    desc = (0.8, 1.2, 0.6)
    kvn = None if kv is None else np.array(kv, dtype=np.int32)
    bmn = None if bm is None else np.array(bm, dtype=np.uint8)
    O, L = orc.forward_fp8(q8, k8, v8, desc, 0.3, causal, bmn, kvn, window)
    rng = np.random.Generator(np.random.PCG64(151))
    sel = [(int(rng.integers(B)), int(rng.integers(2)), int(rng.integers(N))) for _ in range(12)]
    sel += [(B - 1, 1, N - 1), (0, 0, 0)]
    Or, Lr = orc.forward_fp8_rows(q8, k8, v8, desc, 0.3, sel, causal, bmn, kvn, window)
    idx = tuple(np.array(sel).T)
    np.testing.assert_allclose(Lr, L[idx], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(Or, O[idx], rtol=1e-12, atol=1e-14)
