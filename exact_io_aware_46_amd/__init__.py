"""libfa: exact, tiled, fused attention for AMD MI355X (gfx950).

Thin Python binding over the C ABI in ``include/fa.h``. Functions with the C names take
torch tensors (device memory owned by the caller) and marshal them to pointers; every
step of the computation runs in the HIP kernels of ``libfa.so``. There is no fallback:
if the library is not built, or a tensor is not on the GPU, the call raises.

    python -m exact_io_aware_46_amd.build   # builds exact_io_aware_46_amd/libfa.so
"""
from __future__ import annotations

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libfa.so")

FA_OK = 0
STATUS_NAMES = {0: "FA_OK", 1: "FA_ERR_NULL", 2: "FA_ERR_SHAPE", 3: "FA_ERR_UNSUPPORTED_D",
                4: "FA_ERR_ALIGN", 5: "FA_ERR_SCALE", 6: "FA_ERR_LAUNCH", 7: "FA_ERR_ALIAS",
                8: "FA_ERR_DROPOUT", 9: "FA_ERR_DTYPE", 10: "FA_ERR_SCRATCH"}
DTYPE_BF16, DTYPE_F16 = 0, 1

_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_U64 = ctypes.c_uint64
_U32 = ctypes.c_uint32

_SIGNATURES = {
    "fa_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P, _P]),
    "fa_fwd_ex": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P, _P, _P]),
    "fa_fwd_window": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P, _P, _I, _I, _P]),
    "fa_bwd_preprocess": (_I, [_P, _P, _P, _I, _I, _I, _I, _P]),
    "fa_bwd_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I]),
    "fa_bwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P, _P, _P]),
    "fa_bwd_ex": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P, _P, _P,
                       _P]),
    "fa_bwd_window": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P, _P,
                           _I, _I, _P, _P]),
    "fa_fwd_f16": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P, _P, _I, _I, _P]),
    "fa_bwd_preprocess_f16": (_I, [_P, _P, _P, _I, _I, _I, _I, _P]),
    "fa_bwd_f16": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P, _P,
                        _I, _I, _P, _P]),
    "fa_fwd_dropout": (_I, [_I, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P, _P, _I, _I, _F,
                            _U64, _U32, _P]),
    "fa_bwd_dropout": (_I, [_I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P,
                            _P, _I, _I, _F, _U64, _U32, _P, _P]),
    "fa_bwd_noalloc": (_I, [_I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P,
                            _P, _I, _I, _F, _U64, _U32, _P]),
    "fa_fwd_fp8_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I]),
    "fa_fwd_fp8": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _F, _F, _F, _I, _P, _P, _I, _I,
                        _P, _P]),
    "fa_strerror": (ctypes.c_char_p, [_I]),
}


class FAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({strerror(status)})")


def lib() -> ctypes.CDLL:
    """Load libfa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m exact_io_aware_46_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


def strerror(status: int) -> str:
    return lib().fa_strerror(int(status)).decode()


# ------------------------------------------------------------- marshalling
#
# Each tensor argument is checked against what the C ABI will read or write through its
# pointer, before the call: of the element type the entry point takes, with exactly the
# number of elements the shape (B, H, N, d) implies (the workspace: at least the bytes
# the library asks for), then on the GPU and contiguous. A raw integer is passed through
# as a device address without checks. Violations raise ValueError and nothing is called.

_DTYPES = None


def _dtypes(kind):
    global _DTYPES
    if _DTYPES is None:
        import torch
        _DTYPES = {"bf16": (torch.bfloat16,), "f16": (torch.float16,),
                   "f32": (torch.float32,), "i32": (torch.int32,),
                   "mask": (torch.uint8, torch.bool),
                   "fp8": (torch.uint8, getattr(torch, "float8_e4m3fn", torch.uint8))}
    return _DTYPES[kind]


class _Args:
    """One call's pointer arguments: ``add`` checks type and size and returns the device
    pointer (None -> NULL); ``ready`` then checks that every tensor is on the GPU and
    contiguous."""

    def __init__(self, B, H, N, d):
        self.B, self.H, self.N, self.d = int(B), int(H), int(N), int(d)
        self.t = self.B * self.H * self.N * self.d     # elements of q, k, v, o, ...
        self.rows = self.B * self.H * self.N           # elements of lse, delta
        self.mask = ((self.N + 127) // 128) ** 2       # elements of the block table
        self._seen = []

    def add(self, t, name, kind=None, numel=None, min_bytes=None):
        if t is None:
            return None
        if isinstance(t, int):
            return t
        if kind is not None and t.dtype not in _dtypes(kind):
            raise ValueError(f"{name} must have dtype "
                             f"{' or '.join(map(str, _dtypes(kind)))}, got {t.dtype}")
        n = t.numel()
        if numel is not None and n != numel:
            raise ValueError(f"{name} has {n} elements, expected {numel}")
        if min_bytes is not None and n * t.element_size() < min_bytes:
            raise ValueError(f"{name} has {n * t.element_size()} bytes, needs {min_bytes}")
        self._seen.append(t)
        return t.data_ptr()

    def ready(self):
        for t in self._seen:
            if not (t.is_cuda and t.is_contiguous()):
                raise ValueError(f"{'a tensor on the host' if not t.is_cuda else 'a non-contiguous tensor'}"
                                 f" (shape {tuple(t.shape)}, {t.dtype}): every tensor must be a "
                                 "contiguous GPU tensor")

    def fwd(self, kind, q, k, v, o, lse):
        return [self.add(q, "q", kind, self.t), self.add(k, "k", kind, self.t),
                self.add(v, "v", kind, self.t), self.add(o, "o", kind, self.t),
                self.add(lse, "lse", "f32", self.rows)]

    def bwd(self, kind, q, k, v, o, lse, dO, dq, dk, dv):
        return [self.add(q, "q", kind, self.t), self.add(k, "k", kind, self.t),
                self.add(v, "v", kind, self.t), self.add(o, "o", kind, self.t),
                self.add(lse, "lse", "f32", self.rows), self.add(dO, "dO", kind, self.t),
                self.add(dq, "dq", kind, self.t), self.add(dk, "dk", kind, self.t),
                self.add(dv, "dv", kind, self.t)]

    def blockmask(self, t):
        return self.add(t, "blockmask", "mask", self.mask)

    def kv_len(self, t):
        return self.add(t, "kv_len", "i32", self.B)

    def workspace(self, t, nbytes):
        return self.add(t, "workspace", None, None, nbytes)


def _stream_ptr(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status, where):
    if status != FA_OK:
        raise FAError(status, where)


def _kind(dtype):
    if dtype == DTYPE_BF16:
        return "bf16"
    if dtype == DTYPE_F16:
        return "f16"
    return None  # the library rejects it (FA_ERR_DTYPE)


def _call(a, name, *args):
    a.ready()
    _check(getattr(lib(), name)(*args), name)


def fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal=0, blockmask=None, stream=None):
    a = _Args(B, H, N, d)
    _call(a, "fa_fwd", *a.fwd("bf16", q, k, v, o, lse), B, H, N, d, float(scale),
          int(bool(causal)), a.blockmask(blockmask), _stream_ptr(stream))


def fa_fwd_ex(q, k, v, o, lse, B, H, N, d, scale, causal=0, blockmask=None, kv_len=None,
              stream=None):
    a = _Args(B, H, N, d)
    _call(a, "fa_fwd_ex", *a.fwd("bf16", q, k, v, o, lse), B, H, N, d, float(scale),
          int(bool(causal)), a.blockmask(blockmask), a.kv_len(kv_len), _stream_ptr(stream))


def fa_fwd_window(q, k, v, o, lse, B, H, N, d, scale, causal=0, blockmask=None, kv_len=None,
                  window_left=-1, window_right=-1, stream=None):
    a = _Args(B, H, N, d)
    _call(a, "fa_fwd_window", *a.fwd("bf16", q, k, v, o, lse), B, H, N, d, float(scale),
          int(bool(causal)), a.blockmask(blockmask), a.kv_len(kv_len), int(window_left),
          int(window_right), _stream_ptr(stream))


def fa_bwd_preprocess(o, dO, delta, B, H, N, d, stream=None):
    a = _Args(B, H, N, d)
    _call(a, "fa_bwd_preprocess", a.add(o, "o", "bf16", a.t), a.add(dO, "dO", "bf16", a.t),
          a.add(delta, "delta", "f32", a.rows), B, H, N, d, _stream_ptr(stream))


def fa_bwd_workspace_bytes(B, H, N, d) -> int:
    return int(lib().fa_bwd_workspace_bytes(B, H, N, d))


def fa_bwd(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale, causal=0, blockmask=None,
           workspace=None, stream=None):
    a = _Args(B, H, N, d)
    _call(a, "fa_bwd", *a.bwd("bf16", q, k, v, o, lse, dO, dq, dk, dv), B, H, N, d,
          float(scale), int(bool(causal)), a.blockmask(blockmask),
          a.workspace(workspace, fa_bwd_workspace_bytes(B, H, N, d)), _stream_ptr(stream))


def fa_bwd_ex(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale, causal=0, blockmask=None,
              kv_len=None, workspace=None, stream=None):
    a = _Args(B, H, N, d)
    _call(a, "fa_bwd_ex", *a.bwd("bf16", q, k, v, o, lse, dO, dq, dk, dv), B, H, N, d,
          float(scale), int(bool(causal)), a.blockmask(blockmask), a.kv_len(kv_len),
          a.workspace(workspace, fa_bwd_workspace_bytes(B, H, N, d)), _stream_ptr(stream))


def fa_bwd_window(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale, causal=0,
                  blockmask=None, kv_len=None, window_left=-1, window_right=-1,
                  workspace=None, stream=None):
    a = _Args(B, H, N, d)
    _call(a, "fa_bwd_window", *a.bwd("bf16", q, k, v, o, lse, dO, dq, dk, dv), B, H, N, d,
          float(scale), int(bool(causal)), a.blockmask(blockmask), a.kv_len(kv_len),
          int(window_left), int(window_right),
          a.workspace(workspace, fa_bwd_workspace_bytes(B, H, N, d)), _stream_ptr(stream))


def fa_fwd_f16(q, k, v, o, lse, B, H, N, d, scale, causal=0, blockmask=None, kv_len=None,
               window_left=-1, window_right=-1, stream=None):
    a = _Args(B, H, N, d)
    _call(a, "fa_fwd_f16", *a.fwd("f16", q, k, v, o, lse), B, H, N, d, float(scale),
          int(bool(causal)), a.blockmask(blockmask), a.kv_len(kv_len), int(window_left),
          int(window_right), _stream_ptr(stream))


def fa_bwd_preprocess_f16(o, dO, delta, B, H, N, d, stream=None):
    a = _Args(B, H, N, d)
    _call(a, "fa_bwd_preprocess_f16", a.add(o, "o", "f16", a.t), a.add(dO, "dO", "f16", a.t),
          a.add(delta, "delta", "f32", a.rows), B, H, N, d, _stream_ptr(stream))


def fa_bwd_f16(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale, causal=0, blockmask=None,
               kv_len=None, window_left=-1, window_right=-1, workspace=None, stream=None):
    a = _Args(B, H, N, d)
    _call(a, "fa_bwd_f16", *a.bwd("f16", q, k, v, o, lse, dO, dq, dk, dv), B, H, N, d,
          float(scale), int(bool(causal)), a.blockmask(blockmask), a.kv_len(kv_len),
          int(window_left), int(window_right),
          a.workspace(workspace, fa_bwd_workspace_bytes(B, H, N, d)), _stream_ptr(stream))


def fa_fwd_dropout(dtype, q, k, v, o, lse, B, H, N, d, scale, causal=0, blockmask=None,
                   kv_len=None, window_left=-1, window_right=-1, dropout_p=0.0, seed=0,
                   offset=0, stream=None):
    a = _Args(B, H, N, d)
    _call(a, "fa_fwd_dropout", int(dtype), *a.fwd(_kind(dtype), q, k, v, o, lse), B, H, N, d,
          float(scale), int(bool(causal)), a.blockmask(blockmask), a.kv_len(kv_len),
          int(window_left), int(window_right), float(dropout_p), int(seed), int(offset),
          _stream_ptr(stream))


def fa_bwd_dropout(dtype, q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale, causal=0,
                   blockmask=None, kv_len=None, window_left=-1, window_right=-1,
                   dropout_p=0.0, seed=0, offset=0, workspace=None, stream=None):
    a = _Args(B, H, N, d)
    _call(a, "fa_bwd_dropout", int(dtype),
          *a.bwd(_kind(dtype), q, k, v, o, lse, dO, dq, dk, dv), B, H, N, d, float(scale),
          int(bool(causal)), a.blockmask(blockmask), a.kv_len(kv_len), int(window_left),
          int(window_right), float(dropout_p), int(seed), int(offset),
          a.workspace(workspace, fa_bwd_workspace_bytes(B, H, N, d)), _stream_ptr(stream))


def fa_bwd_noalloc(dtype, q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale, causal=0,
                   blockmask=None, kv_len=None, window_left=-1, window_right=-1,
                   dropout_p=0.0, seed=0, offset=0, stream=None):
    """fa_bwd_dropout with the library's static device scratch as its workspace."""
    a = _Args(B, H, N, d)
    _call(a, "fa_bwd_noalloc", int(dtype),
          *a.bwd(_kind(dtype), q, k, v, o, lse, dO, dq, dk, dv), B, H, N, d, float(scale),
          int(bool(causal)), a.blockmask(blockmask), a.kv_len(kv_len), int(window_left),
          int(window_right), float(dropout_p), int(seed), int(offset), _stream_ptr(stream))


def fa_fwd_fp8_workspace_bytes(B, H, N, d):
    return int(lib().fa_fwd_fp8_workspace_bytes(B, H, N, d))


def fa_fwd_fp8(q8, k8, v8, o, lse, B, H, N, d, scale, descale_q, descale_k, descale_v,
               causal=0, blockmask=None, kv_len=None, window_left=-1, window_right=-1,
               workspace=None, stream=None):
    a = _Args(B, H, N, d)
    _call(a, "fa_fwd_fp8", a.add(q8, "q", "fp8", a.t), a.add(k8, "k", "fp8", a.t),
          a.add(v8, "v", "fp8", a.t), a.add(o, "o", "bf16", a.t),
          a.add(lse, "lse", "f32", a.rows), B, H, N, d, float(scale), float(descale_q),
          float(descale_k), float(descale_v), int(bool(causal)), a.blockmask(blockmask),
          a.kv_len(kv_len), int(window_left), int(window_right),
          a.workspace(workspace, fa_fwd_fp8_workspace_bytes(B, H, N, d)), _stream_ptr(stream))


# ------------------------------------------------- allocating convenience layer

def _is_f16(t):
    import torch
    if t.dtype == torch.float16:
        return True
    if t.dtype == torch.bfloat16:
        return False
    raise ValueError(f"tensors must be bfloat16 or float16, got {t.dtype}")

def forward(q, k, v, scale, causal=False, blockmask=None, kv_len=None, window=None,
            stream=None, dropout=None):
    """q, k, v: bf16 or fp16 GPU tensors [B, H, N, d] (one type for all). Returns (o, lse)
    newly allocated. ``window`` is None or (left, right) (sliding window, negative = no
    limit); ``dropout`` is None or (p, seed, offset)."""
    import torch
    B, H, N, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    wl, wr = (-1, -1) if window is None else window
    if dropout is not None:
        fa_fwd_dropout(DTYPE_F16 if _is_f16(q) else DTYPE_BF16, q, k, v, o, lse, B, H, N, d,
                       scale, causal, blockmask, kv_len, wl, wr, *dropout, stream=stream)
        return o, lse
    fn = fa_fwd_f16 if _is_f16(q) else fa_fwd_window
    fn(q, k, v, o, lse, B, H, N, d, scale, causal, blockmask, kv_len, wl, wr, stream)
    return o, lse


def backward(q, k, v, o, lse, dO, scale, causal=False, blockmask=None, kv_len=None,
             workspace=None, stream=None, window=None, dropout=None):
    """Returns (dq, dk, dv) newly allocated; allocates the workspace if none is given."""
    import torch
    B, H, N, d = q.shape
    if workspace is None:
        workspace = torch.empty(fa_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8,
                                device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    wl, wr = (-1, -1) if window is None else window
    if dropout is not None:
        fa_bwd_dropout(DTYPE_F16 if _is_f16(q) else DTYPE_BF16, q, k, v, o, lse, dO, dq, dk,
                       dv, B, H, N, d, scale, causal, blockmask, kv_len, wl, wr, *dropout,
                       workspace=workspace, stream=stream)
        return dq, dk, dv
    fn = fa_bwd_f16 if _is_f16(q) else fa_bwd_window
    fn(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale, causal, blockmask, kv_len, wl, wr,
       workspace, stream)
    return dq, dk, dv


def forward_fp8(q8, k8, v8, scale, descale, causal=False, blockmask=None, kv_len=None,
                window=None, stream=None):
    """q8, k8, v8: uint8 GPU tensors [B, H, N, d] of E4M3 codes; descale = (descale_q,
    descale_k, descale_v). Returns (o bf16, lse fp32), newly allocated (plus a transient
    workspace for V transposed)."""
    import torch
    B, H, N, d = q8.shape
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q8.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q8.device)
    ws = torch.empty(max(fa_fwd_fp8_workspace_bytes(B, H, N, d), 1), dtype=torch.uint8,
                     device=q8.device)
    wl, wr = (-1, -1) if window is None else window
    fa_fwd_fp8(q8, k8, v8, o, lse, B, H, N, d, scale, *descale, causal, blockmask, kv_len, wl,
               wr, ws, stream)
    return o, lse
