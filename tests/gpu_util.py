"""Helpers for the GPU parity tests: move seeded bf16 inputs to the device, run libfa
through its C ABI binding, bring results back as float64, and apply the tolerances.

Tolerances (bf16 inputs, fp32 accumulation, fp64 oracle):
  O     max-abs <= 1e-2 and relative L2 <= 5e-3
  LSE   abs <= 1e-3 (and -inf exactly where the oracle has -inf)
  dQ, dK, dV  relative L2 <= 2e-2; where the oracle's whole gradient is zero by
              cancellation (e.g. N = 1: dS = P (dP - D) with dP = D), max-abs <= 1e-4, the
              fp32 rounding left by dP and D being summed in different orders. Exact zeros
              from masking are asserted separately by the mask tests.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import exact_io_aware_46_amd as fa
from exact_io_aware_46_amd import inputs as inp

O_MAX_ABS = 1e-2
O_REL_L2 = 5e-3
LSE_ABS = 1e-3
GRAD_REL_L2 = 2e-2


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray) -> torch.Tensor:
    """bf16 bit patterns (uint16) -> bfloat16 GPU tensor; numpy float16 -> float16 tensor."""
    dt = torch.float16 if x.dtype == np.float16 else torch.bfloat16
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(dt)


def to_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def to_f64(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return inp.bf16_bits_to_f32(to_bits(t)).astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


class Run:
    """Device buffers and results of one libfa forward + backward."""

    def __init__(self, q, k, v, do, scale, causal=False, blockmask=None, kv_len=None,
                 backward=True, window=None, dropout=None):
        self.dq_ = self.dk_ = self.dv_ = None
        self.q, self.k, self.v = to_dev(q), to_dev(k), to_dev(v)
        self.do = to_dev(do) if do is not None else None
        self.bm = None if blockmask is None else torch.from_numpy(
            np.ascontiguousarray(blockmask, dtype=np.uint8)).cuda()
        self.kv = None if kv_len is None else torch.from_numpy(
            np.ascontiguousarray(kv_len, dtype=np.int32)).cuda()
        self.scale, self.causal = scale, causal
        self.o, self.lse = fa.forward(self.q, self.k, self.v, scale, causal, self.bm, self.kv,
                                      window=window, dropout=dropout)
        if backward:
            self.dq_, self.dk_, self.dv_ = fa.backward(self.q, self.k, self.v, self.o, self.lse,
                                                       self.do, scale, causal, self.bm, self.kv,
                                                       window=window, dropout=dropout)
        torch.cuda.synchronize()

    def result(self):
        r = {"O": to_f64(self.o), "LSE": to_f64(self.lse)}
        if self.dq_ is not None:
            r.update(dQ=to_f64(self.dq_), dK=to_f64(self.dk_), dV=to_f64(self.dv_))
        return r


def rel_l2(a, b):
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / nb if nb > 0 else np.linalg.norm(a - b)


def check_o(o, ref, what="", rel_slack=0.0):
    """max |o - ref| <= 1e-2 (+ rel_slack * |ref| elementwise, for stress inputs whose
    outputs exceed the range the 1e-2 bound was set for), and relative L2 <= 5e-3."""
    err = np.abs(o - ref).max() if o.size else 0.0
    bound = O_MAX_ABS + rel_slack * np.abs(ref)
    rl = rel_l2(o, ref)
    assert (np.abs(o - ref) <= bound).all(), f"{what} O max-abs {err:.3e}"
    assert rl <= O_REL_L2, f"{what} O rel-L2 {rl:.3e}"
    return err, rl


def check_lse(lse, ref, what=""):
    ninf = np.isneginf(ref)
    assert np.array_equal(np.isneginf(lse), ninf), f"{what} LSE -inf pattern differs"
    fin = ~ninf
    err = np.abs(lse[fin] - ref[fin]).max() if fin.any() else 0.0
    assert err <= LSE_ABS, f"{what} LSE abs {err:.3e}"
    return err


ZERO_GRAD_ABS = 1e-4


def check_grad(g, ref, name, what=""):
    if (ref == 0).all():
        err = float(np.abs(g).max()) if g.size else 0.0
        assert err <= ZERO_GRAD_ABS, f"{what} {name} should vanish, max-abs {err:.3e}"
        return err
    rl = rel_l2(g, ref)
    assert rl <= GRAD_REL_L2, f"{what} {name} rel-L2 {rl:.3e}"
    return rl


def check_all(res, ref, what="", grads=True, o_rel_slack=0.0):
    out = {}
    out["O"] = check_o(res["O"], ref["O"], what, o_rel_slack)
    out["LSE"] = check_lse(res["LSE"], ref["LSE"], what)
    if grads:
        for name in ("dQ", "dK", "dV"):
            out[name] = check_grad(res[name], ref[name], name, what)
    return out


# ------------------------------------------------------------------ FP8 forward

def run_fp8(q8, k8, v8, scale, descale, causal=False, blockmask=None, kv_len=None,
            window=None):
    """Runs fa_fwd_fp8 on uint8 code arrays; returns (O, LSE) as float64 and the device
    workspace (V transposed)."""
    B, H, N, d = q8.shape
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    q, k, v = dev(q8), dev(k8), dev(v8)
    bm = None if blockmask is None else dev(np.asarray(blockmask, dtype=np.uint8))
    kv = None if kv_len is None else dev(np.asarray(kv_len, dtype=np.int32))
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(fa.fa_fwd_fp8_workspace_bytes(B, H, N, d), dtype=torch.uint8,
                     device="cuda")
    wl, wr = (-1, -1) if window is None else window
    fa.fa_fwd_fp8(q, k, v, o, lse, B, H, N, d, scale, *descale, causal, bm, kv, wl, wr, ws)
    torch.cuda.synchronize()
    return to_f64(o), to_f64(lse), ws


def count_raises(t, ok, tile, thresh, integer):
    """How many times each row's running reference is raised after its first value, under
    the forward kernels' rule: key tiles of ``tile`` keys in order; a tile whose largest
    allowed score exceeds the reference by more than ``thresh`` (log2 units) raises it to
    that score (rounded up if ``integer``). ``t`` [r, N] scores in log2 units, ``ok``
    [r, N] allowed pairs. Used to show that a test's inputs reach the rescaling code."""
    r, N = t.shape
    nt = -(-N // tile)
    tt = np.full((r, nt * tile), -np.inf)
    tt[:, :N] = np.where(ok, t, -np.inf)
    tmax = tt.reshape(r, nt, tile).max(axis=2)
    m = np.full(r, -np.inf)
    cnt = np.zeros(r, dtype=np.int64)
    for j in range(nt):
        mx = tmax[:, j]
        with np.errstate(invalid="ignore"):
            up = mx > m + thresh
        cnt += up & np.isfinite(m)
        m = np.where(up, np.ceil(mx) if integer else mx, m)
    return cnt
