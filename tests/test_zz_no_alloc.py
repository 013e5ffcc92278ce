"""fa_bwd_noalloc (backward with the library's static device scratch as its workspace)
against fa_bwd_dropout (the same kernels with a caller's workspace): two calls in a row,
the second on a smaller problem, every output bitwise equal and within the oracle's
tolerances. Runs alone or after the other GPU tests."""
import numpy as np
import pytest
import torch

import exact_io_aware_46_amd as fa
from exact_io_aware_46_amd import inputs as inp
from oracle import attention as orc
from tests.gpu_util import check_all, say, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _case(B, H, N, d, seed, dtype, causal, kv, drop):
    q, k, v, do = inp.custom_inputs(B, H, N, d, seed=seed, dtype=dtype)
    t = [to_dev(x) for x in (q, k, v, do)]
    kvt = None if kv is None else torch.tensor(kv, dtype=torch.int32, device="cuda")
    code = fa.DTYPE_F16 if dtype == "f16" else fa.DTYPE_BF16
    dr = (0.0, 0, 0) if drop is None else drop
    o, lse = fa.forward(t[0], t[1], t[2], 0.1, causal, None, kvt, dropout=drop)
    grads = {}
    for name in ("dropout", "noalloc"):
        dq, dk, dv = (torch.full_like(t[0], 7.0) for _ in range(3))
        if name == "dropout":
            ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8,
                             device="cuda")
            fa.fa_bwd_dropout(code, t[0], t[1], t[2], o, lse, t[3], dq, dk, dv, B, H, N, d, 0.1,
                              causal, None, kvt, -1, -1, *dr, workspace=ws)
        else:
            fa.fa_bwd_noalloc(code, t[0], t[1], t[2], o, lse, t[3], dq, dk, dv, B, H, N, d, 0.1,
                              causal, None, kvt, -1, -1, *dr)
        torch.cuda.synchronize()
        grads[name] = (dq, dk, dv)
    for a, b in zip(grads["dropout"], grads["noalloc"]):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    ref = orc.backward(q, k, v, do, 0.1, causal, None, kv, dropout=drop)
    res = {"O": to_f64(o), "LSE": to_f64(lse), "dQ": to_f64(grads["noalloc"][0]),
           "dK": to_f64(grads["noalloc"][1]), "dV": to_f64(grads["noalloc"][2])}
    check_all(res, ref, f"noalloc B={B} H={H} N={N} d={d}",
              o_rel_slack=2.0 ** -7 if drop else 0.0)


def test_noalloc_backward_equals_the_workspace_backward_on_two_calls():
    say("[noalloc] call 1: B=2 H=3 N=700 d=128 causal, key padding")
    _case(2, 3, 700, 128, 301, "bf16", True, [700, 431], None)
    say("[noalloc] call 2 (smaller): B=1 H=2 N=129 d=64 fp16, dropout")
    _case(1, 2, 129, 64, 302, "f16", False, None, (0.2, 99, 3))
