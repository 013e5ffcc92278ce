"""The library allocates and clears nothing, so a forward + backward can be captured into a
HIP graph (torch's graph API; the launches go to the capturing stream) and replayed. Every
replay, with eager calls on other data and synchronisations between the replays, must
reproduce the eager outputs bit for bit."""
import numpy as np
import pytest
import torch

import exact_io_aware_46_amd as fa
from exact_io_aware_46_amd import inputs as inp
from tests.gpu_util import say, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d,kv", [(64, None), (128, [300, 171])])
def test_captured_forward_backward_replays_equal_eager(d, kv):
    B = 1 if kv is None else len(kv)
    N, H, scale = 300, 2, 0.11
    q, k, v, do = (to_dev(x) for x in inp.custom_inputs(B, H, N, d, seed=311 + d))
    kvt = None if kv is None else torch.tensor(kv, dtype=torch.int32, device="cuda")
    ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device="cuda")
    o, dq, dk, dv = (torch.empty_like(q) for _ in range(4))
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")

    def step():
        fa.fa_fwd_window(q, k, v, o, lse, B, H, N, d, scale, 1, None, kvt, -1, -1)
        fa.fa_bwd_window(q, k, v, o, lse, do, dq, dk, dv, B, H, N, d, scale, 1, None, kvt,
                         -1, -1, ws)

    say(f"[graph] d={d} kv={kv}: eager reference")
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (o, lse, dq, dk, dv)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    # other eager work on other data between replays
    q2, k2, v2, do2 = (to_dev(x) for x in inp.custom_inputs(B, H, N, d, seed=312 + d))
    for r in range(4):
        for t in (o, lse, dq, dk, dv):
            t.fill_(7.0)
        o2, lse2 = fa.forward(q2, k2, v2, scale, True, None, kvt)
        fa.backward(q2, k2, v2, o2, lse2, do2, scale, True, None, kvt)
        torch.cuda.synchronize()
        say(f"[graph] replay {r}")
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((o, lse, dq, dk, dv), ref):
            it = torch.int16 if a.element_size() == 2 else torch.int32
            assert torch.equal(a.view(it), b.view(it)), f"replay {r} differs"


def test_calls_on_two_streams_at_once_equal_sequential_calls():
    """The library keeps no state between calls: forward + backward of two problems of
    different shapes, each on its own stream (default priority) and running at the same
    time, equal the same calls made one after another, bit for bit."""
    probs = []
    for i, (N, d) in enumerate([(700, 128), (900, 64)]):
        q, k, v, do = (to_dev(x) for x in inp.custom_inputs(1, 4, N, d, seed=331 + i))
        probs.append((q, k, v, do, float(np.float32(d ** -0.5))))

    def run(pr, stream=None):
        q, k, v, do, sc = pr
        o, lse = fa.forward(q, k, v, sc, True, stream=stream)
        ws = torch.empty(fa.fa_bwd_workspace_bytes(*q.shape), dtype=torch.uint8,
                         device="cuda")
        dq, dk, dv = fa.backward(q, k, v, o, lse, do, sc, True, workspace=ws, stream=stream)
        return o, lse, dq, dk, dv

    say("[streams] sequential reference")
    ref = [run(pr) for pr in probs]
    torch.cuda.synchronize()
    say("[streams] two streams at once")
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    outs = []
    for rep in range(3):
        cur = []
        for pr, s in zip(probs, streams):
            with torch.cuda.stream(s):
                cur.append(run(pr, stream=s))
        outs.append(cur)
    for s in streams:
        torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for cur in outs:
        for got, want in zip(cur, ref):
            for a, b in zip(got, want):
                assert torch.equal(a.view(torch.int8), b.view(torch.int8))
