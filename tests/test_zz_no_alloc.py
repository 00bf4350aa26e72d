"""fa_bwd_noalloc (the backward with the library's static scratch instead of a
caller workspace) against fa_bwd on the same inputs: the same kernels, so the
gradients must be bitwise equal; two calls in a row, the second smaller, so
that left-over scratch contents from the first call cannot leak into it."""

import numpy as np
import pytest

import seeded_inputs as si

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_io_aware_fa2_amd as m
    m.load_library()
    return m


def _run(fa, B, H, N, d, causal, seed):
    import torch
    dev = torch.device("cuda:0")
    inp = si.make_inputs(B, H, N, d, "bf16", 1.0, seed, backward=True)
    q, k, v, do = (torch.from_numpy(inp[n][1].view(np.int16)).view(torch.bfloat16).to(dev)
                   for n in ("q", "k", "v", "do"))
    scale = 1.0 / np.sqrt(d)
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
    ref = fa.bwd(q, k, v, o, lse, do, causal=causal, scale=scale)
    got = tuple(torch.full_like(t, float("nan")) for t in ref)
    fa.fa_bwd_noalloc(q, k, v, o, lse, do, *got, scale, causal)
    torch.cuda.synchronize()
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        assert torch.equal(g.view(torch.int16), r.view(torch.int16)), (name, B, H, N, d, causal)


@pytest.mark.parametrize("d", [64, 128])
def test_noalloc_matches_fa_bwd_two_calls_second_smaller(fa, d):
    print(f"noalloc d={d}: call 1 B=2 H=4 N=1000, call 2 B=1 H=2 N=300", flush=True)
    _run(fa, 2, 4, 1000, d, True, 7001)
    _run(fa, 1, 2, 300, d, True, 7002)
    _run(fa, 1, 3, 257, d, False, 7003)
