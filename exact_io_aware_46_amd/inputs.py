"""Seeded synthetic inputs for exact attention, shared by the oracle tests, the GPU
parity tests and the bench.

This module holds no attention arithmetic. It only draws random numbers, rounds them
to bfloat16 bit patterns, and builds the masks' *inputs* (key-padding lengths, the
128x128 block table). Everything the method computes lives elsewhere: the fp64 oracle
under ``oracle/`` and the HIP kernels under ``csrc/``. Both read the same bf16 bits.

Workload shapes follow the pages' training workloads only by shape (BERT-large-like,
GPT-2-small-like, long causal, block-sparse); no dataset is read.

Recipe (one ``numpy.random.Generator(PCG64(seed))`` per workload):
  1. draw Q, K, V, dO in that order with ``standard_normal(dtype=float32)``,
     C-order ``[B][H][N][d]``;
  2. round each float32 to bf16 with round-to-nearest-even on the bit pattern (or, for an
     fp16 workload, to IEEE binary16 with numpy's round-to-nearest-even conversion; for an
     FP8 workload, Q, K, V only, each scaled by its own descale = max|x| / 448 and rounded
     to E4M3 codes by torch's float8_e4m3fn conversion);
  3. then, if the workload has one, draw the mask input:
     key padding: ``integers(128, 513, size=B)`` (valid length per sequence);
     block mask:  all diagonal blocks kept, plus a uniform draw without replacement
     of off-diagonal blocks until the kept fraction is ``density``.

Inputs of the largest shapes (billions of elements) are drawn on the device instead, by
``device_normal``: torch's seeded generator, standard normal, directly in the 16-bit type.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

BLOCK = 128  # block-mask granularity in both query and key directions


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even) and return the
    16-bit patterns as uint16. Inputs must be finite (true for every generator here)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def f32_to_f16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to IEEE binary16 (numpy's conversion rounds to nearest even)."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16)


def f32_to_e4m3(x: np.ndarray) -> np.ndarray:
    """Round float32 values (|x| <= 448) to OCP E4M3 codes (uint8), nearest even, with
    torch's float8_e4m3fn conversion."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def quantize_e4m3(x: np.ndarray) -> tuple:
    """Per-tensor FP8 quantisation of float32 values: descale = float32(max|x| / 448)
    (the largest magnitude maps to the largest finite code), codes = E4M3(x / descale).
    Returns (codes, descale)."""
    amax = float(np.abs(x).max())
    descale = float(np.float32(amax / 448.0)) if amax > 0 else 1.0
    y = np.clip(x / np.float32(descale), -448.0, 448.0).astype(np.float32)
    return f32_to_e4m3(y), descale


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32 (used by generators and tests to
    look at inputs; both compute paths do their own widening)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    causal: bool = False
    mask: str = "none"          # "none" | "kpad" | "block"
    density: float = 1.0        # kept fraction of 128x128 blocks for mask == "block"
    seed: int = 0
    window: tuple | None = None  # sliding window (left, right); negative = no limit
    dtype: str = "bf16"          # element type of Q, K, V, dO: "bf16" (uint16 bits), "f16",
                                 # or "fp8" (E4M3 codes with per-tensor descales; forward only)
    dropout: tuple | None = None  # attention dropout (p, seed, offset); None = no dropout

    @property
    def scale(self) -> float:
        """1/sqrt(d) rounded to float32 (the value both sides receive)."""
        return float(np.float32(1.0 / math.sqrt(self.d)))

    def with_n(self, n: int) -> "Workload":
        return dataclasses.replace(self, N=n, name=f"{self.name}_N{n}")


# The workloads, in order: a tiny single head, a GPT-2-small-shaped causal layer, a
# BERT-large-shaped padded layer, a long causal head set, a block-sparse layer, the long
# head set with a sliding window, the long causal head set in fp16, the long causal head
# set with attention dropout, the long causal head set at head dims 96, 32 and 256, and the
# long causal head set in FP8.
WORKLOADS = {
    "single_head_256": Workload("single_head_256", 1, 1, 256, 64, seed=46001),
    "gpt2s_causal_1k": Workload("gpt2s_causal_1k", 8, 12, 1024, 64, causal=True, seed=46002),
    "bertl_kpad_512": Workload("bertl_kpad_512", 16, 16, 512, 64, mask="kpad", seed=46003),
    "long_causal_16k": Workload("long_causal_16k", 1, 16, 16384, 128, causal=True, seed=46004),
    "blocksparse_8k": Workload("blocksparse_8k", 2, 8, 8192, 64, mask="block", density=0.25,
                               seed=46005),
    # Sliding-window (local) causal attention over the long head set: each query sees
    # itself and the 4095 keys before it.
    "sliding_window_16k": Workload("sliding_window_16k", 1, 16, 16384, 128, causal=True,
                                   seed=46006, window=(4095, 0)),
    # The long causal head set in fp16.
    "long_causal_16k_f16": Workload("long_causal_16k_f16", 1, 16, 16384, 128, causal=True,
                                    seed=46007, dtype="f16"),
    # The long causal head set with dropout p = 0.1 on the attention probabilities (the
    # pages fix no rate; 0.1 is the customary attention-dropout rate); the Philox seed is
    # a fixed 64-bit value.
    "long_causal_16k_dropout": Workload("long_causal_16k_dropout", 1, 16, 16384, 128,
                                        causal=True, seed=46008,
                                        dropout=(0.1, 0x5EED_0000_B3D8, 0)),
    # The long causal head set at head dims 96 and 32, which run the 128 and 64 kernels on
    # zero-padded tiles.
    "long_causal_16k_d96": Workload("long_causal_16k_d96", 1, 16, 16384, 96, causal=True,
                                    seed=46009),
    "long_causal_16k_d32": Workload("long_causal_16k_d32", 1, 16, 16384, 32, causal=True,
                                    seed=46010),
    "long_causal_16k_d256": Workload("long_causal_16k_d256", 1, 16, 16384, 256, causal=True,
                                     seed=46012),
    # The long causal head set in FP8 (E4M3 with per-tensor descales; forward only).
    "long_causal_16k_fp8": Workload("long_causal_16k_fp8", 1, 16, 16384, 128, causal=True,
                                    seed=46011, dtype="fp8"),
}
WORKLOAD_ORDER = list(WORKLOADS)


@dataclasses.dataclass
class Inputs:
    """bf16 bit patterns (uint16, [B][H][N][d]) plus optional mask inputs."""
    wl: Workload
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    do: np.ndarray
    kv_len: np.ndarray | None = None      # int32 [B]
    blockmask: np.ndarray | None = None   # uint8 [nb][nb], nb = ceil(N/128)
    descale: tuple | None = None          # fp8: (descale_q, descale_k, descale_v)


def n_blocks(n: int) -> int:
    return (n + BLOCK - 1) // BLOCK


def draw_block_mask(rng: np.random.Generator, n: int, density: float) -> np.ndarray:
    """Diagonal blocks always kept, plus off-diagonal blocks drawn uniformly without
    replacement until round(density * nb^2) blocks are kept in total."""
    nb = n_blocks(n)
    total = int(round(density * nb * nb))
    extra = max(0, total - nb)
    off = np.array([r * nb + c for r in range(nb) for c in range(nb) if r != c], dtype=np.int64)
    mask = np.eye(nb, dtype=np.uint8)
    if extra:
        pick = rng.choice(off.size, size=extra, replace=False)
        mask.reshape(-1)[off[pick]] = 1
    return mask


def make_inputs(wl: Workload, need_do: bool = True) -> Inputs:
    rng = np.random.Generator(np.random.PCG64(wl.seed))
    shape = (wl.B, wl.H, wl.N, wl.d)
    descale = None
    if wl.dtype == "fp8":
        (q, dq), (k, dk), (v, dv) = (quantize_e4m3(rng.standard_normal(shape, dtype=np.float32))
                                     for _ in range(3))
        descale, do = (dq, dk, dv), None
    else:
        cvt = f32_to_f16 if wl.dtype == "f16" else f32_to_bf16_bits
        q = cvt(rng.standard_normal(shape, dtype=np.float32))
        k = cvt(rng.standard_normal(shape, dtype=np.float32))
        v = cvt(rng.standard_normal(shape, dtype=np.float32))
        do = cvt(rng.standard_normal(shape, dtype=np.float32)) if need_do else None
    kv_len = None
    blockmask = None
    if wl.mask == "kpad":
        kv_len = rng.integers(128, 513, size=wl.B).astype(np.int32)
        kv_len = np.minimum(kv_len, wl.N).astype(np.int32)
    elif wl.mask == "block":
        blockmask = draw_block_mask(rng, wl.N, wl.density)
    return Inputs(wl, q, k, v, do, kv_len, blockmask, descale)


def custom_inputs(B: int, H: int, N: int, d: int, seed: int, dist: str = "normal",
                  dtype: str = "bf16") -> tuple:
    """Small ad-hoc shapes for edge-case tests: returns (q, k, v, do) as bf16 bits
    (uint16) or, with ``dtype="f16"``, as numpy float16 arrays.
    ``dist="normal"`` draws all four from N(0,1); ``"wide"`` draws Q and K from N(0, 3^2)
    (scores spread ~9x wider, so the softmax is far from uniform) and V, dO from N(0,1)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    shape = (B, H, N, d)
    out = []
    for i in range(4):
        sd = 3.0 if (dist == "wide" and i < 2) else 1.0
        x = (sd * rng.standard_normal(shape)).astype(np.float32)
        out.append(f32_to_f16(x) if dtype == "f16" else f32_to_bf16_bits(x))
    return tuple(out)


def device_normal(shape, seed: int, dtype: str = "bf16", count: int = 4,
                  device: str = "cuda") -> list:
    """Inputs too large to draw on the host and copy over: ``count`` tensors of standard
    normal values drawn one after another on the device by one torch generator seeded with
    ``seed`` (a stream of its own, unrelated to the numpy streams above), drawn directly in
    bfloat16 or float16. With ``dtype="fp8"`` each is drawn in float32 and quantised per
    tensor as ``quantize_e4m3`` does; the result is then a list of (uint8 codes, descale)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = []
    for _ in range(count):
        if dtype == "fp8":
            x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
            amax = float(x.abs().max())
            descale = float(np.float32(amax / 448.0)) if amax > 0 else 1.0
            x.div_(np.float32(descale)).clamp_(-448.0, 448.0)
            out.append((x.to(torch.float8_e4m3fn).view(torch.uint8), descale))
            del x
        else:
            dt = torch.float16 if dtype == "f16" else torch.bfloat16
            out.append(torch.randn(shape, generator=g, device=device, dtype=dt))
    return out
