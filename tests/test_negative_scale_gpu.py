"""Parity on the GPU for a negative scale.

softmax(scale * Q K^T) is defined for any finite scale; a negative one gives
the most weight to the keys of smallest q.k.  The kernels take it as |scale|
with the sign bits of one operand of the scores flipped, which is exact
(s q.k = |s| (-q).k, and negating a 16-bit or 8-bit float is exact).  Every
entry point is checked against the float64 oracle at the usual bounds (forward
O max-abs <= 1e-2, mean-abs <= 1e-3, LSE max-abs <= 1e-3; backward relative L2
<= 1e-2), and the square entry points also against the same call with the
queries negated and the scale's magnitude: O and LSE bit for bit; dQ
(negated), dK and dV equal up to a few elements in 10^4 that differ in their
last bits (relative L2 <= 1e-4): the backward takes the scale's sign as is,
and the matrix cores' sums of negated products may round one bit apart from
the negated sums.
"""

import numpy as np
import pytest

import seeded_inputs as si
from oracle import attention_bwd, attention_fwd, kvcache_fwd, varlen_bwd, varlen_fwd
from parity import (BWD_REL_L2, assert_fwd_ok, assert_fwd_ok_peaked, fwd_errors, gpu_fwd, lib, rel_l2, say,
                    to_device)

pytestmark = pytest.mark.gpu


def _grads_ok(grads, ref, label):
    errs = {}
    for name, g, r in zip(("dq", "dk", "dv"), grads, ref):
        gg = g.float().cpu().numpy()
        assert np.isfinite(gg).all(), (label, name)
        errs[name] = rel_l2(gg, r)
    say(f"  {label}: rel-L2 {errs}")
    assert all(e <= BWD_REL_L2 for e in errs.values()), (label, errs)


@pytest.mark.parametrize("dtype,d", [("bf16", 32), ("bf16", 64), ("f16", 64), ("bf16", 96), ("bf16", 128),
                                     ("f16", 128), ("bf16", 256), ("f32", 64), ("f32", 128)])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_negative_scale(causal, dtype, d):
    B, H, N = 1, 2, 300
    scale = -1.0 / np.sqrt(d)
    seed = 12000 + d + int(causal)
    say(f"fwd negative scale N{N} d{d} {dtype} causal={causal} seed={seed}")
    inp = si.make_inputs(B, H, N, d, dtype, 1.0, seed)
    _, _, _, o, lse = gpu_fwd(inp, dtype, causal, scale)
    o_ref, l_ref = attention_fwd(inp["q"][0], inp["k"][0], inp["v"][0], scale, causal)
    assert_fwd_ok(fwd_errors(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref), dtype,
                  f"scale {scale:.4f} d{d} {dtype} causal={causal}")


@pytest.mark.parametrize("d", [32, 64, 96, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_negative_scale(causal, d):
    import torch
    fa = lib()
    B, H, N = 1, 2, 300
    scale = -1.0 / np.sqrt(d)
    seed = 12100 + d + int(causal)
    say(f"bwd negative scale N{N} d{d} causal={causal} seed={seed}")
    inp = si.make_inputs(B, H, N, d, "bf16", 1.0, seed, backward=True)
    q, k, v, do = (to_device(inp[n][1], "bf16") for n in ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v, causal, scale)
    grads = fa.bwd(q, k, v, o, lse, do, causal, scale)
    torch.cuda.synchronize()
    ref = attention_bwd(inp["q"][0], inp["k"][0], inp["v"][0], inp["do"][0], scale, causal)
    _grads_ok(grads, ref, f"d{d} causal={causal}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("scale", [-2.0, -1e-35, -0.0])
def test_backward_degenerate_negative_scales(scale, d):
    # -2: sharp rows; -1e-35: below the 2^-100 floor of the dK/dV kernel's
    # exponent split (dQ, dK ~ 1e-35 stay representable in bf16); -0.0: zero
    import torch
    fa = lib()
    B, H, N = 1, 2, 300
    say(f"bwd scale={scale} N{N} d{d}")
    inp = si.make_inputs(B, H, N, d, "bf16", 1.0, 12200 + d, backward=True)
    q, k, v, do = (to_device(inp[n][1], "bf16") for n in ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v, True, scale)
    grads = fa.bwd(q, k, v, o, lse, do, True, scale)
    torch.cuda.synchronize()
    ref = attention_bwd(inp["q"][0], inp["k"][0], inp["v"][0], inp["do"][0], scale, True)
    if scale == 0.0:
        for name, g in zip(("dq", "dk"), grads[:2]):
            assert np.abs(g.float().cpu().numpy()).max() <= 1e-5, name
        assert rel_l2(grads[2].float().cpu().numpy(), ref[2]) <= BWD_REL_L2
    else:
        _grads_ok(grads, ref, f"scale={scale} d{d}")


# B2 H8 N8100 at d = 64 and d = 128 runs the persistent grids (one workgroup
# per resident slot walking several tiles); N = 700 the one-tile-per-workgroup
# grids; d = 256 the split-key forward and the wide backward.
@pytest.mark.parametrize("B,H,N,d", [(1, 3, 700, 64), (1, 3, 700, 128), (1, 2, 700, 256), (1, 2, 700, 32),
                                     (1, 2, 700, 96), (2, 8, 8100, 64), (2, 8, 8100, 128)])
@pytest.mark.parametrize("causal", [False, True])
def test_negative_scale_equals_negated_queries(B, H, N, d, causal):
    import torch
    fa = lib()
    s = 1.0 / np.sqrt(d)
    say(f"negative scale vs negated queries B{B} H{H} N{N} d{d} causal={causal}")
    inp = si.make_inputs(B, H, N, d, "bf16", 1.0, 12300 + d + N + int(causal), backward=True)
    q, k, v, do = (to_device(inp[n][1], "bf16") for n in ("q", "k", "v", "do"))
    qn = -q
    o1, l1 = fa.fwd(q, k, v, causal, -s)
    o2, l2 = fa.fwd(qn, k, v, causal, s)
    g1 = fa.bwd(q, k, v, o1, l1, do, causal, -s)
    g2 = fa.bwd(qn, k, v, o2, l2, do, causal, s)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "forward"
    pairs = {"dq": (g1[0], -g2[0]), "dk": (g1[1], g2[1]), "dv": (g1[2], g2[2])}
    differ = {n: int((a != b).sum()) for n, (a, b) in pairs.items()}
    rel = {n: rel_l2(a.float().cpu().numpy(), b.float().cpu().numpy().astype(np.float64))
           for n, (a, b) in pairs.items()}
    say(f"  gradients against the negated queries: elements differing {differ} of {q.numel()}, "
        f"relative L2 {rel}")
    assert max(rel.values()) <= 1e-4 and max(differ.values()) <= 1e-4 * q.numel(), (differ, rel)


@pytest.mark.parametrize("d", [64, 128])
def test_fp32_negative_scale_equals_negated_queries_bitwise(d):
    import torch
    fa = lib()
    s = 1.0 / np.sqrt(d)
    inp = si.make_inputs(1, 2, 500, d, "f32", 1.0, 12400 + d)
    q, k, v = (to_device(inp[n][1], "f32") for n in ("q", "k", "v"))
    o1, l1 = fa.fwd(q, k, v, True, -s)
    o2, l2 = fa.fwd(-q, k, v, True, s)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ---------------------------------------------------------------- key/value cache, varlen, FP8

def _kv_check(o, lse, o_ref, lse_ref, label):
    inf_ref = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), inf_ref), label
    fin = ~inf_ref
    assert_fwd_ok(fwd_errors(o[fin], lse[fin], o_ref[fin], lse_ref[fin]), "bf16", label)


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,Nq,Nk,fill", [(2, 3, 1, 1000, 0.3), (3, 2, 5, 777, 0.0), (2, 2, 33, 513, 0.5)])
def test_kvcache_negative_scale(B, H, Nq, Nk, fill, causal, d):
    import torch
    fa = lib()
    seed = 12500 + Nq + Nk + d
    inp = si.make_kvcache_inputs(B, H, Nq, Nk, d, "bf16", 1.0, seed, fill)
    scale = -1.0 / np.sqrt(d)
    say(f"kvcache negative scale B{B} H{H} Nq{Nq} Nk{Nk} d{d} causal={causal} lens={inp['seqlens'].tolist()}")
    q, k, v = (to_device(inp[n][1], "bf16") for n in ("q", "k", "v"))
    lens = torch.from_numpy(inp["seqlens"]).cuda()
    o, lse = fa.fwd_kvcache(q, k, v, lens, causal, scale)
    torch.cuda.synchronize()
    o_ref, l_ref = kvcache_fwd(inp["q"][0], inp["k"][0], inp["v"][0], scale, causal, inp["seqlens"])
    _kv_check(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, f"kvcache Nq{Nq} Nk{Nk} d{d}")


@pytest.mark.parametrize("causal", [False, True])
def test_kvcache_fp8_negative_scale(causal):
    import torch
    fa = lib()
    inp = si.make_kvcache_fp8_inputs(2, 3, 5, 1000, 128, "bf16", 1.0, 12600, 0.3)
    scale = -1.0 / np.sqrt(128)
    say(f"kvcache fp8 negative scale causal={causal} lens={inp['seqlens'].tolist()}")
    q = to_device(inp["q"][1], "bf16")
    k, v = (torch.from_numpy(inp[n][1]).cuda() for n in ("k", "v"))
    lens = torch.from_numpy(inp["seqlens"]).cuda()
    o, lse = fa.fwd_kvcache_fp8(q, k, v, float(inp["k_scale"]), float(inp["v_scale"]), lens, causal, scale)
    torch.cuda.synchronize()
    o_ref, l_ref = kvcache_fwd(inp["q"][0], inp["k"][0], inp["v"][0], scale, causal, inp["seqlens"])
    _kv_check(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, "kvcache fp8")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("same", [False, True])
def test_varlen_negative_scale_fwd_bwd(same, causal, d):
    """Packed sequences: one prefix-sum array (the square kernels) or
    separate query and key counts (the split-key forward, the square
    backward with its own key counts)."""
    import torch
    fa = lib()
    lq = [1, 100, 0, 33, 257]
    lk = lq if same else [50, 100, 7, 33, 300]
    H = 2
    seed = 12700 + d + 2 * int(causal) + int(same)
    inp = si.make_varlen_inputs(lq, lk, H, d, "bf16", 1.0, seed, backward=True)
    scale = -1.0 / np.sqrt(d)
    say(f"varlen negative scale lq={lq} lk={lk} d{d} causal={causal}")
    q, k, v, do = (to_device(inp[n][1], "bf16") for n in ("q", "k", "v", "do"))
    cq = torch.from_numpy(inp["cu_q"]).cuda()
    ck = cq if same else torch.from_numpy(inp["cu_k"]).cuda()
    mq, mk = max(lq), max(lk)
    o, lse = fa.fwd_varlen(q, k, v, cq, ck, mq, mk, causal, scale)
    grads = fa.bwd_varlen(q, k, v, o, lse, do, cq, ck, mq, mk, causal, scale)
    torch.cuda.synchronize()
    o_ref, l_ref = varlen_fwd(inp["q"][0], inp["k"][0], inp["v"][0], inp["cu_q"], inp["cu_k"], scale, causal)
    og, lg = o.float().cpu().numpy(), lse.cpu().numpy()
    _kv_check(og.transpose(1, 0, 2), lg, o_ref.transpose(1, 0, 2), l_ref, f"varlen fwd d{d}")
    ref = varlen_bwd(inp["q"][0], inp["k"][0], inp["v"][0], inp["do"][0], inp["cu_q"], inp["cu_k"], scale, causal)
    for name, g, r in zip(("dq", "dk", "dv"), grads, ref):
        gg = g.float().cpu().numpy()
        assert np.isfinite(gg).all(), name
        e = rel_l2(gg, r) if np.linalg.norm(r) > 0 else float(np.abs(gg).max())
        say(f"  {name} rel-L2 {e:.3e}")
        assert e <= BWD_REL_L2, (name, e)


@pytest.mark.parametrize("gran", ["tensor", "block"])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_forward_negative_scale(causal, gran):
    import torch
    fa = lib()
    N = 700
    inp = si.make_fp8_inputs(1, 2, N, 128, "bf16", 1.0, 12800 + int(causal), gran)
    scale = -1.0 / np.sqrt(128)
    say(f"fp8 negative scale N{N} {gran} causal={causal}")
    t = {n: torch.from_numpy(np.ascontiguousarray(inp[n][1])).cuda() for n in ("q", "k", "v")}
    s = {n: torch.from_numpy(np.ascontiguousarray(inp[n + "_scale"]).reshape(
        -1 if inp[n + "_scale"].size == 1 else inp[n + "_scale"].shape)).cuda() for n in ("q", "k", "v")}
    o, lse = fa.fwd_fp8(t["q"], t["k"], t["v"], s["q"], s["k"], s["v"], gran, causal, scale, torch.bfloat16)
    # the same call on negated codes (sign bit flipped) and the scale's magnitude: bit for bit
    o2, lse2 = fa.fwd_fp8(t["q"] ^ 0x80, t["k"], t["v"], s["q"], s["k"], s["v"], gran, causal, -scale,
                          torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    o_ref, l_ref = attention_fwd(inp["q"][0], inp["k"][0], inp["v"][0], scale, causal)
    assert_fwd_ok_peaked(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, "bf16",
                         f"fp8 {gran} causal={causal}")


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_growing_scores_negative_scale(d, causal):
    """Keys scaled up 6x along the sequence: the row maxima of -|s| q.k grow
    past the first tile's as for a positive scale, so the reference maximum
    is raised (d = 64: re-based tiles; d = 128: the pass redone against exact
    maxima, with the flipped queries).  Against the oracle, and bit for bit
    against the negated queries at |s|."""
    import torch
    fa = lib()
    N = 600
    inp = si.make_inputs(1, 2, N, d, "bf16", 1.0, 12900 + d)
    grow = (1.0 + 5.0 * np.arange(N) / N)[None, None, :, None]
    inp["k"] = si.round_to(inp["k"][0] * grow, "bf16")
    scale = -1 / np.sqrt(d)
    say(f"growing keys negative scale d{d} causal={causal}")
    q, k, v, o, lse = gpu_fwd(inp, "bf16", causal, scale)
    o2, lse2 = fa.fwd(-q, k, v, causal, -scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    o_ref, l_ref = attention_fwd(inp["q"][0], inp["k"][0], inp["v"][0], scale, causal)
    assert_fwd_ok_peaked(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, "bf16",
                         f"growing keys negative scale d{d} causal={causal}")
