"""The forward and the allocation-free backward (fa_bwd_noalloc) recorded into
a HIP graph and replayed: each replay, with new inputs copied into the
captured buffers between replays (eager work in between), must give the
same bits as the eager calls on those inputs.  The library allocates nothing
and launches only its own kernels on the caller's stream, so the calls can
be captured as they are."""

import numpy as np
import pytest

import seeded_inputs as si
from parity import lib, say, to_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d", [64, 128])
def test_forward_and_noalloc_backward_replay_in_a_graph(d):
    import torch
    fa = lib()
    # 32 heads x 16 query tiles: the persistent grids at d = 64 (forward) and
    # in both backward kernels
    B, H, N = 4, 8, 4000
    scale = 1.0 / np.sqrt(d)
    draws = [si.make_inputs(B, H, N, d, "bf16", 1.0, 9940 + 10 * i + d, backward=True) for i in range(3)]
    dev = [tuple(to_device(x[n][1], "bf16") for n in ("q", "k", "v", "do")) for x in draws]
    q, k, v, do = (torch.empty_like(t) for t in dev[0])
    o, dq, dk, dv = (torch.empty_like(q) for _ in range(4))
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")

    def step():
        fa.fa_fwd(q, k, v, o, lse, scale, True)
        fa.fa_bwd_noalloc(q, k, v, o, lse, do, dq, dk, dv, scale, True)

    for dst, src in zip((q, k, v, do), dev[0]):
        dst.copy_(src)
    step()  # eager first call: the noalloc scratch address and the device's compute-unit count are looked up
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for i, src in enumerate(dev + dev[:1]):
        for dst, s in zip((q, k, v, do), src):
            dst.copy_(s)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (o, lse, dq, dk, dv)]
        step()  # eager on the same inputs
        torch.cuda.synchronize()
        for name, a, b in zip(("o", "lse", "dq", "dk", "dv"), got, (o, lse, dq, dk, dv)):
            if a.dtype == torch.bfloat16:
                a, b = a.view(torch.int16), b.view(torch.int16)
            assert torch.equal(a, b), (name, i)
        say(f"  graph replay {i} d={d}: O, LSE, dQ, dK, dV bitwise equal to the eager calls")
