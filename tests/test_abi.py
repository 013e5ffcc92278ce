"""The C ABI without a GPU: the library loads, exports exactly what include/fa.h
declares, and rejects invalid arguments on the host before any HIP call (so every call
here returns an error code; no call here has valid arguments, none reaches a kernel)."""
import ctypes
import os
import re
import subprocess

import pytest

import exact_io_aware_46_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

# Fake, never-dereferenced device addresses (validation only looks at their values).
A = 0x7F0000000000
T_BYTES = 1 << 30  # spacing that keeps fake buffers disjoint


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_\w+)\s*\(", text)))


def exported_functions():
    out = subprocess.run(["nm", "-D", "--defined-only", fa.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    return sorted(l.split()[-1] for l in out.splitlines() if " T " in l)


@pytest.fixture(scope="module")
def lib():
    return fa.lib()


def test_library_exports_exactly_the_header(lib):
    decl = declared_functions()
    assert decl == ["fa_bwd", "fa_bwd_dropout", "fa_bwd_ex", "fa_bwd_f16",
                    "fa_bwd_noalloc", "fa_bwd_preprocess", "fa_bwd_preprocess_f16",
                    "fa_bwd_window",
                    "fa_bwd_workspace_bytes", "fa_fwd", "fa_fwd_dropout", "fa_fwd_ex",
                    "fa_fwd_f16", "fa_fwd_fp8", "fa_fwd_fp8_workspace_bytes", "fa_fwd_window",
                    "fa_strerror"]
    assert exported_functions() == decl
    for name in decl:
        assert hasattr(lib, name)


def test_strerror(lib):
    for st in range(11):
        assert len(fa.strerror(st)) > 0
    assert fa.strerror(99) == "unknown status"


def ptrs(n):
    return [A + i * T_BYTES for i in range(n)]


def fwd(lib, *, q=None, k=None, v=None, o=None, lse=None, B=1, H=1, N=64, d=64, scale=0.125,
        causal=0, kv=None):
    p = ptrs(5)
    args = [p[0] if q is None else q, p[1] if k is None else k, p[2] if v is None else v,
            p[3] if o is None else o, p[4] if lse is None else lse]
    return lib.fa_fwd_ex(*args, B, H, N, d, scale, causal, None, kv, None)


def test_fwd_null_pointers(lib):
    for name in ("q", "k", "v", "o", "lse"):
        assert fwd(lib, **{name: 0}) == 1


@pytest.mark.parametrize("B,H,N", [(0, 1, 64), (1, 0, 64), (1, 1, 0), (-1, 1, 64),
                                   (1 << 16, 1 << 10, 1 << 10)])
def test_fwd_bad_shape(lib, B, H, N):
    assert fwd(lib, B=B, H=H, N=N) == 2


# The size limits: B*H*N rows and N*d elements per head each at most 2^31 - 1.
@pytest.mark.parametrize("B,H,N,d", [(1, 1, 1 << 24, 128),        # N*d = 2^31
                                     (1, 1, 1 << 23, 256),        # N*d = 2^31
                                     (1 << 7, 1 << 7, 1 << 17, 8),  # B*H*N = 2^31
                                     (3, 5, 143165577, 8)])       # B*H*N = 2^31 + 7
def test_sizes_one_past_the_limits_are_rejected(lib, B, H, N, d):
    assert fwd(lib, B=B, H=H, N=N, d=d) == 2
    assert lib.fa_bwd_workspace_bytes(B, H, N, d) == 0


# Supported: multiples of 8 from 8 to 256.
@pytest.mark.parametrize("d", [0, 4, 20, 100, 260, 264, 512, -64])
def test_fwd_unsupported_head_dim(lib, d):
    assert fwd(lib, d=d) == 3


def test_fwd_misaligned(lib):
    assert fwd(lib, q=A + 8) == 4
    assert fwd(lib, o=A + 3 * T_BYTES + 2) == 4
    assert fwd(lib, lse=A + 4 * T_BYTES + 2) == 4
    assert fwd(lib, kv=A + 6 * T_BYTES + 1) == 4


@pytest.mark.parametrize("scale", [0.0, float("nan"), float("inf"), -float("inf")])
def test_fwd_bad_scale(lib, scale):
    assert fwd(lib, scale=scale) == 5


def test_fwd_alias(lib):
    assert fwd(lib, o=A) == 7                     # o overlaps q
    assert fwd(lib, lse=A + 3 * T_BYTES + 64) == 7  # lse inside o


def bwd(lib, over=None, B=1, H=1, N=64, d=64, scale=0.125, ws_off=0):
    p = ptrs(10)
    p[9] += ws_off
    if over:
        for i, val in over.items():
            p[i] = val
    return lib.fa_bwd_ex(*p[:9], B, H, N, d, scale, 0, None, None, p[9], None)


def test_bwd_errors(lib):
    for i in range(10):
        assert bwd(lib, {i: 0}) == 1
    assert bwd(lib, B=0) == 2
    assert bwd(lib, d=264) == 3
    assert bwd(lib, {0: A + 8}) == 4
    assert bwd(lib, ws_off=16) == 4                  # workspace needs 256-byte alignment
    assert bwd(lib, scale=float("nan")) == 5
    assert bwd(lib, {6: A + 3 * T_BYTES}) == 7       # dq aliases o
    assert bwd(lib, {7: A + 6 * T_BYTES}) == 7       # dk aliases dq
    assert bwd(lib, {9: A + 2 * T_BYTES}) == 7       # workspace aliases v


def test_preprocess_errors(lib):
    assert lib.fa_bwd_preprocess(None, A, A + T_BYTES, 1, 1, 8, 64, None) == 1
    assert lib.fa_bwd_preprocess(A, A + T_BYTES, A + 2 * T_BYTES, 1, 1, 8, 44, None) == 3
    assert lib.fa_bwd_preprocess(A, A + T_BYTES, A + 2, 1, 1, 8, 64, None) == 4
    assert lib.fa_bwd_preprocess(A, A + T_BYTES, A + 4, 1, 1, 8, 64, None) == 7


def test_workspace_bytes_linear_in_n(lib):
    assert fa.fa_bwd_workspace_bytes(0, 1, 1, 64) == 0
    assert fa.fa_bwd_workspace_bytes(1, 1, 1, 100) == 0
    w = [fa.fa_bwd_workspace_bytes(1, 16, n, 128) for n in (2048, 4096, 8192, 16384)]
    assert w[0] == 2 * 16 * 2048 * 4
    assert [x / w[0] for x in w] == [1, 2, 4, 8]


def test_python_binding_rejects_host_tensors():
    import torch
    x = torch.zeros((1, 1, 8, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.fa_fwd(x, x, x, x, torch.zeros((1, 1, 8)), 1, 1, 8, 64, 0.125, stream=0)


def test_window_entry_points_validate_like_the_others(lib):
    # Same host-side checks as fa_fwd_ex / fa_bwd_ex; any window value is accepted.
    p = ptrs(9)
    fwd_args = lambda q, d, scale: (q, p[1], p[2], p[3], p[4], 1, 1, 64, d, scale, 0, None,
                                    None, 3, -1, None)
    assert lib.fa_fwd_window(*fwd_args(None, 64, 0.125)) == 1          # FA_ERR_NULL
    assert lib.fa_fwd_window(*fwd_args(p[0], 260, 0.125)) == 3         # FA_ERR_UNSUPPORTED_D
    assert lib.fa_fwd_window(*fwd_args(p[0], 64, float("nan"))) == 5   # FA_ERR_SCALE
    assert lib.fa_fwd_window(*fwd_args(p[0] + 2, 64, 0.125)) == 4     # FA_ERR_ALIGN
    ws = A + 64 * T_BYTES
    bwd_args = lambda q, N: (q, p[1], p[2], p[3], p[4], p[5], p[6], p[7], p[8], 1, 1, N, 64,
                             0.125, 1, None, None, -1, 7, ws, None)
    assert lib.fa_bwd_window(*bwd_args(None, 64)) == 1                 # FA_ERR_NULL
    assert lib.fa_bwd_window(*bwd_args(p[0], 0)) == 2                  # FA_ERR_SHAPE
    # an output overlapping an input is rejected before any launch
    alias = (p[0], p[1], p[2], p[3], p[4], p[5], p[0], p[7], p[8], 1, 1, 64, 64, 0.125, 0,
             None, None, 5, 5, ws, None)
    assert lib.fa_bwd_window(*alias) == 7                               # FA_ERR_ALIAS


def test_f16_entry_points_validate_like_the_others(lib):
    p = ptrs(9)
    assert lib.fa_fwd_f16(None, p[1], p[2], p[3], p[4], 1, 1, 64, 64, 0.125, 0, None, None,
                          -1, -1, None) == 1                           # FA_ERR_NULL
    assert lib.fa_fwd_f16(p[0], p[1], p[2], p[3], p[4], 1, 1, 64, 12, 0.125, 0, None, None,
                          -1, -1, None) == 3                           # FA_ERR_UNSUPPORTED_D
    assert lib.fa_bwd_preprocess_f16(p[0], p[1], p[2] + 1, 1, 1, 64, 64, None) == 4  # ALIGN
    ws = A + 64 * T_BYTES
    assert lib.fa_bwd_f16(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7], p[8], 1, 1, 64, 64,
                          0.0, 0, None, None, -1, -1, ws, None) == 5     # FA_ERR_SCALE


def test_dropout_entry_points_validate(lib):
    p = ptrs(9)
    fwd = lambda dt, pd: lib.fa_fwd_dropout(dt, p[0], p[1], p[2], p[3], p[4], 1, 1, 64, 64,
                                            0.125, 0, None, None, -1, -1, pd, 7, 0, None)
    assert fwd(0, 1.0) == 8                     # FA_ERR_DROPOUT: p must be < 1
    assert fwd(0, -0.25) == 8
    assert fwd(1, float("nan")) == 8
    assert fwd(2, 0.1) == 9                     # FA_ERR_DTYPE
    ws = A + 64 * T_BYTES
    bwd = lambda dt, pd, q: lib.fa_bwd_dropout(dt, q, p[1], p[2], p[3], p[4], p[5], p[6], p[7],
                                               p[8], 1, 1, 64, 64, 0.125, 0, None, None, -1,
                                               -1, pd, (1 << 40) + 3, 5, ws, None)
    assert bwd(0, 0.1, None) == 1               # FA_ERR_NULL
    assert bwd(5, 0.1, p[0]) == 9
    assert bwd(1, 1.5, p[0]) == 8


def test_fp8_entry_point_validates(lib):
    p = ptrs(5)
    ws = A + 64 * T_BYTES

    def call(q=p[0], N=64, d=128, scale=0.1, desc=(0.01, 0.02, 0.03), o=p[3], w=ws):
        return lib.fa_fwd_fp8(q, p[1], p[2], o, p[4], 1, 2, N, d, scale, *desc, 1, None, None,
                              -1, -1, w, None)
    assert call(q=None) == 1                                   # FA_ERR_NULL
    assert call(w=None) == 1
    assert call(N=0) == 2                                      # FA_ERR_SHAPE
    for d in (32, 96, 72, 256):                                # FP8: 64 and 128 only
        assert call(d=d) == 3
    assert call(scale=0.0) == 5                                # FA_ERR_SCALE
    for desc in ((0.0, 1.0, 1.0), (1.0, -1.0, 1.0), (1.0, 1.0, float("nan")),
                 (float("inf"), 1.0, 1.0)):
        assert call(desc=desc) == 5
    assert call(q=p[0] + 8) == 4                               # FA_ERR_ALIGN
    assert call(w=ws + 16) == 4
    assert call(o=p[0]) == 7                                   # o overlaps q
    assert call(w=p[2]) == 7                                   # workspace overlaps v
    assert fa.fa_fwd_fp8_workspace_bytes(1, 2, 100, 128) == 2 * 128 * 128  # N -> 128
    assert fa.fa_fwd_fp8_workspace_bytes(1, 2, 100, 96) == 0


# ---------------------------------------------- the Python binding's argument checks
# Host tensors are used; dtype and size are checked before the device, so every call
# below raises before anything reaches the library.

def _bf(*shape, dtype=None):
    import torch
    return torch.zeros(shape, dtype=dtype or torch.bfloat16)


def _fwd_py(**over):
    import torch
    B, H, N, d = 2, 1, 200, 64
    a = dict(q=_bf(B, H, N, d), k=_bf(B, H, N, d), v=_bf(B, H, N, d), o=_bf(B, H, N, d),
             lse=torch.zeros((B, H, N)), blockmask=None, kv_len=None)
    a.update(over)
    fa.fa_fwd_window(a["q"], a["k"], a["v"], a["o"], a["lse"], B, H, N, d, 0.125, 1,
                     a["blockmask"], a["kv_len"], -1, -1, stream=0)


@pytest.mark.parametrize("over,msg", [
    ({"kv_len": "int64"}, "dtype"),
    ({"kv_len": "short"}, "elements"),
    ({"blockmask": "small"}, "elements"),
    ({"blockmask": "int32"}, "dtype"),
    ({"k": "longer"}, "elements"),
    ({"v": "f16"}, "dtype"),
    ({"lse": "f64"}, "dtype"),
    ({"o": "short"}, "elements"),
    ({}, "GPU tensor"),
])
def test_python_binding_checks_dtype_and_size(over, msg):
    import torch
    make = {"int64": lambda n: torch.tensor([200, 100]),
            "short": lambda n: torch.zeros(1, dtype=torch.int32) if n == "kv_len"
            else _bf(2, 1, 199, 64),
            "small": lambda n: torch.ones((1, 1), dtype=torch.uint8),
            "int32": lambda n: torch.ones((2, 2), dtype=torch.int32),
            "longer": lambda n: _bf(2, 1, 256, 64),
            "f16": lambda n: _bf(2, 1, 200, 64, dtype=torch.float16),
            "f64": lambda n: torch.zeros((2, 1, 200), dtype=torch.float64)}
    args = {name: make[kind](name) for name, kind in over.items()}
    with pytest.raises(ValueError, match=msg):
        _fwd_py(**args)


def test_python_binding_checks_backward_workspace_and_fp8_types():
    import torch
    B, H, N, d = 1, 2, 64, 128
    t = [_bf(B, H, N, d) for _ in range(8)]
    lse = torch.zeros((B, H, N))
    small = torch.zeros(fa.fa_bwd_workspace_bytes(B, H, N, d) - 1, dtype=torch.uint8)
    with pytest.raises(ValueError, match="bytes"):
        fa.fa_bwd_window(t[0], t[1], t[2], t[3], lse, t[4], t[5], t[6], t[7], B, H, N, d,
                         0.1, 1, None, None, -1, -1, small, stream=0)
    with pytest.raises(ValueError, match="dtype"):   # fp16 tensors through the bf16 entry
        fa.fa_bwd_window(*[x.half() for x in t[:4]], lse, *[x.half() for x in t[4:]], B, H, N,
                         d, 0.1, 1, None, None, -1, -1, small, stream=0)
    q8 = torch.zeros((B, H, N, d), dtype=torch.uint8)
    ws = torch.zeros(fa.fa_fwd_fp8_workspace_bytes(B, H, N, d), dtype=torch.uint8)
    with pytest.raises(ValueError, match="dtype"):   # O of the FP8 forward is bf16
        fa.fa_fwd_fp8(q8, q8, q8, torch.zeros((B, H, N, d)), lse, B, H, N, d, 0.1, 1.0, 1.0,
                      1.0, 1, None, None, -1, -1, ws, stream=0)
    with pytest.raises(ValueError, match="dtype"):
        fa.fa_fwd_fp8(t[0], q8, q8, t[1], lse, B, H, N, d, 0.1, 1.0, 1.0, 1.0, 1, None, None,
                      -1, -1, ws, stream=0)


def test_noalloc_backward_validates_and_rejects_sizes_past_its_scratch(lib):
    # Same checks as fa_bwd_dropout (no workspace argument), then the static scratch limit
    # of 2^22 rows; all before any HIP call.
    p = ptrs(9)

    def call(B=1, H=1, N=64, d=64, dt=0, pd=0.0, q=p[0]):
        return lib.fa_bwd_noalloc(dt, q, p[1], p[2], p[3], p[4], p[5], p[6], p[7], p[8], B, H,
                                  N, d, 0.125, 1, None, None, -1, -1, pd, 0, 0, None)
    assert call(q=None) == 1                     # FA_ERR_NULL
    assert call(N=0) == 2                        # FA_ERR_SHAPE
    assert call(d=12) == 3                       # FA_ERR_UNSUPPORTED_D
    assert call(q=p[0] + 2) == 4                 # FA_ERR_ALIGN
    assert call(pd=1.0) == 8                     # FA_ERR_DROPOUT
    assert call(dt=3) == 9                       # FA_ERR_DTYPE
    assert call(B=2, H=64, N=32769, d=8) == 10   # FA_ERR_SCRATCH: 4,194,432 rows
    assert call(B=1, H=128, N=32769, d=8) == 10
    assert fa.STATUS_NAMES[10] == "FA_ERR_SCRATCH"
