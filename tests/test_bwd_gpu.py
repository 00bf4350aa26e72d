"""Backward parity on the GPU: fa_bwd (using the library's own forward O and
LSE, as a training step would) against the float64 oracle's softmax-Jacobian
gradient on the same seeded Q, K, V, dO.  Bound: relative L2 <= 1e-2 for each
of dQ, dK, dV.  Full-size workloads run on the GPU in full; the oracle checks
sampled heads in full."""

import numpy as np
import pytest

import seeded_inputs as si
from oracle import attention_bwd_head
from parity import BWD_REL_L2, gpu_fwd, lib, rel_l2, say, to_device

pytestmark = pytest.mark.gpu


def _run(inp, dtype, causal, scale):
    import torch
    fa = lib()
    q, k, v, o, lse = gpu_fwd(inp, dtype, causal, scale)
    do = to_device(inp["do"][1], dtype)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal, scale)
    torch.cuda.synchronize()
    return dq.float().cpu().numpy(), dk.float().cpu().numpy(), dv.float().cpu().numpy()


def _check_heads(inp, grads, heads, scale, causal, label):
    worst = {"dq": 0.0, "dk": 0.0, "dv": 0.0}
    for (b, h) in heads:
        ref = attention_bwd_head(inp["q"][0][b, h], inp["k"][0][b, h], inp["v"][0][b, h],
                                 inp["do"][0][b, h], scale, causal)
        for name, g, r in zip(("dq", "dk", "dv"), grads, ref):
            assert np.isfinite(g[b, h]).all(), (label, name, b, h)
            if np.linalg.norm(r) == 0.0:
                # e.g. one key: dQ = dK = 0 exactly; only rounding noise may remain
                assert np.abs(g[b, h]).max() <= 1e-5, (label, name, b, h)
                continue
            e = rel_l2(g[b, h], r)
            worst[name] = max(worst[name], e)
    say(f"  {label}: rel-L2 {worst}")
    for name, e in worst.items():
        assert e <= BWD_REL_L2, (label, name, e)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 200, 257, 700])
def test_small_shapes_and_tails(N, causal, d, dtype):
    B, H = 1, 2
    say(f"bwd small B{B} H{H} N{N} d{d} {dtype} causal={causal}")
    inp = si.make_inputs(B, H, N, d, dtype, 1.0, 9000 + N + d, backward=True)
    scale = 1 / np.sqrt(d)
    grads = _run(inp, dtype, causal, scale)
    _check_heads(inp, grads, [(0, 0), (0, 1)], scale, causal, f"N{N} d{d} {dtype} causal={causal}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("scale", [0.0, 1e-35, 2.0])
def test_degenerate_and_large_scales(scale, causal, d):
    # scale 0: uniform attention over the visible keys, dQ = dK = 0 exactly;
    # 1e-35 lies below the smallest scale the dK/dV kernel splits its exponent
    # with (2^-100), where the exponent is -LSE log2 e up to rounding; 2: sharp
    # softmax rows.  bf16 keeps dQ, dK ~ 1e-35 representable.
    N, dtype = 300, "bf16"
    say(f"bwd scale={scale} N{N} d{d} causal={causal}")
    inp = si.make_inputs(1, 2, N, d, dtype, 1.0, 9500 + d + int(causal), backward=True)
    grads = _run(inp, dtype, causal, scale)
    _check_heads(inp, grads, [(0, 0), (0, 1)], scale, causal, f"scale={scale} d{d} causal={causal}")


@pytest.mark.parametrize("name", ["C5", "C5d128", "C5d256"])
def test_c5_full_size_sampled_heads(name):
    w = si.WORKLOADS[name]
    say(f"{name} full size on GPU: {w}")
    inp = si.make_workload_inputs(w)
    grads = _run(inp, w.dtype, w.causal, w.scale)
    _check_heads(inp, grads, [(0, 0), (3, 9), (7, 15)], w.scale, w.causal, name)


def test_backward_deterministic_bitwise():
    import torch
    fa = lib()
    inp = si.make_inputs(2, 2, 900, 128, "bf16", 1.0, 31, backward=True)
    q, k, v, o, lse = gpu_fwd(inp, "bf16", True, 1 / np.sqrt(128))
    do = to_device(inp["do"][1], "bf16")
    a = fa.bwd(q, k, v, o, lse, do, True)
    b = fa.bwd(q, k, v, o, lse, do, True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_gradient_identities_on_gpu():
    """sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i, up to bf16 rounding of the gradients."""
    inp = si.make_inputs(1, 2, 513, 64, "bf16", 1.0, 32, backward=True)
    dq, dk, dv = _run(inp, "bf16", False, 1 / 8)
    do = inp["do"][0].astype(np.float64)
    for h in range(2):
        np.testing.assert_allclose(dk[0, h].sum(axis=0), 0.0, atol=0.05)
        np.testing.assert_allclose(dv[0, h].sum(axis=0), do[0, h].sum(axis=0), atol=0.1)


def test_autograd_function_matches_direct_calls():
    import torch
    fa = lib()
    inp = si.make_inputs(1, 2, 300, 64, "bf16", 1.0, 33, backward=True)
    q, k, v = (to_device(inp[n][1], "bf16").requires_grad_(True) for n in ("q", "k", "v"))
    do = to_device(inp["do"][1], "bf16")
    o = fa.attention(q, k, v, True)
    o.backward(do)
    q2, k2, v2, o2, lse2 = gpu_fwd(inp, "bf16", True, 1 / 8)
    dq, dk, dv = fa.bwd(q2, k2, v2, o2, lse2, do, True)
    assert torch.equal(o.detach(), o2)
    assert torch.equal(q.grad, dq) and torch.equal(k.grad, dk) and torch.equal(v.grad, dv)
