"""Parity on the GPU for fa_fwd_fp8 (8-bit E4M3 Q, K, V with float scales,
S = Q K^T on the FP8 matrix cores): against the float64 oracle fed the
dequantised inputs (codes times scales), at the 16-bit forward's bounds (O
max-abs <= 1e-2, mean-abs <= 1e-3; LSE max-abs <= 1e-3), since only the
rounding of the inputs to 8 bits separates the kernel from exact attention.
The error against attention on the 16-bit values the codes came from (the
quantisation error) is printed separately and only sanity-bounded."""

import numpy as np
import pytest

import seeded_inputs as si
from oracle import attention_fwd, attention_fwd_head
from parity import TOL, assert_fwd_ok, assert_fwd_ok_peaked, fwd_errors, lib, say

pytestmark = pytest.mark.gpu


def _up(inp):
    import torch
    dev = "cuda"
    t = {n: torch.from_numpy(np.ascontiguousarray(inp[n][1])).to(dev) for n in ("q", "k", "v")}
    s = {n: torch.from_numpy(np.ascontiguousarray(inp[n + "_scale"]).reshape(-1 if inp[n + "_scale"].size == 1 else
                                                                                 inp[n + "_scale"].shape)).to(dev)
         for n in ("q", "k", "v")}
    return t, s


def _run(inp, gran, causal, scale, out="bf16"):
    import torch
    fa = lib()
    t, s = _up(inp)
    odt = {"bf16": torch.bfloat16, "f16": torch.float16}[out]
    o, lse = fa.fwd_fp8(t["q"], t["k"], t["v"], s["q"], s["k"], s["v"], gran, causal, scale, odt)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("out", ["bf16", "f16"])
@pytest.mark.parametrize("gran", ["tensor", "block"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 255, 257, 1000])
def test_fp8_small_shapes_and_tails(N, causal, gran, out):
    seed = 8100 + N
    inp = si.make_fp8_inputs(1, 2, N, 128, out, 1.0, seed, gran)
    scale = 1.0 / np.sqrt(128)
    say(f"fp8 N{N} causal={causal} {gran} out {out} seed={seed}")
    o, lse = _run(inp, gran, causal, scale, out)
    o_ref, lse_ref = attention_fwd(inp["q"][0], inp["k"][0], inp["v"][0], scale, causal)
    # the dequantised values are no 16-bit values: at one key O is V itself,
    # and its rounding to the output type alone can exceed the mean bound
    assert_fwd_ok_peaked(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, out,
                         f"fp8 N{N} {gran} causal={causal} out {out}")
    # quantisation error: against attention on the 16-bit values the codes came from
    o16, l16 = attention_fwd(inp["q16"][0], inp["k16"][0], inp["v16"][0], scale, causal)
    q = fwd_errors(o.float().cpu().numpy(), lse.cpu().numpy(), o16, l16)
    say(f"    against the 16-bit inputs (quantisation): O max {q['o_max']:.3e} mean {q['o_mean']:.3e} "
        f"LSE max {q['lse_max']:.3e}")
    assert q["o_max"] < 0.5 and q["lse_max"] < 0.5


def test_fp8_block_scales_differ_per_block():
    """Per-block scaling with different block magnitudes (Q rows scaled by 1,
    4, 1/4, 2, 1/2, 3 per 128-row block, K rows by 3, 1/2, 2, 1/4, 4, 1): each
    pair of blocks scales its scores differently, so a scale applied to the
    wrong block shows.  (The scores stay within about 15 in magnitude: the
    FP8 product accumulates its 64 products with less than float32 precision,
    about 2^-13 of the largest partial sum on the MI355X, which at scores of
    50 and more alone reaches LSE errors near 1e-3.)"""
    B, H, N, d = 1, 3, 700, 128
    base = si.make_inputs(B, H, N, d, "bf16", 1.0, 8200)
    blk = np.arange(N) // 128
    fq = np.array([1.0, 4.0, 0.25, 2.0, 0.5, 3.0])[blk][None, None, :, None]
    fk = np.array([3.0, 0.5, 2.0, 0.25, 4.0, 1.0])[blk][None, None, :, None]
    base["q"] = si.round_to(base["q"][0] * fq, "bf16")
    base["k"] = si.round_to(base["k"][0] * fk, "bf16")
    inp = {}
    for nm in ("q", "k", "v"):
        codes, sc, deq = si.quantise_e4m3_scaled(base[nm][0], "block", per_head_only=(nm == "v"))
        inp[nm], inp[nm + "_scale"] = (deq, codes), sc
    scale = 0.02
    for causal in (False, True):
        o, lse = _run(inp, "block", causal, scale)
        o_ref, lse_ref = attention_fwd(inp["q"][0], inp["k"][0], inp["v"][0], scale, causal)
        # scaled-up rows make peaked softmax rows: output rounding allowed for
        assert_fwd_ok_peaked(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, "bf16",
                             f"fp8 varying block scales causal={causal}")


def test_fp8_growing_scores_rerun():
    """Keys growing x1..x6 along the sequence: the reference maximum must be
    raised (the exact-maximum rerun), as in the 16-bit kernel."""
    B, H, N, d = 1, 2, 900, 128
    base = si.make_inputs(B, H, N, d, "bf16", 1.0, 8300)
    base["k"] = si.round_to(base["k"][0] * (1.0 + 5.0 * np.arange(N) / N)[None, None, :, None], "bf16")
    inp = {}
    for nm in ("q", "k", "v"):
        codes, sc, deq = si.quantise_e4m3_scaled(base[nm][0], "block", per_head_only=(nm == "v"))
        inp[nm], inp[nm + "_scale"] = (deq, codes), sc
    scale = 1 / np.sqrt(d)
    for causal in (False, True):
        o, lse = _run(inp, "block", causal, scale)
        o_ref, lse_ref = attention_fwd(inp["q"][0], inp["k"][0], inp["v"][0], scale, causal)
        assert_fwd_ok_peaked(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, "bf16",
                             f"fp8 growing keys causal={causal}")


def test_fp8_bitwise_repeatable():
    import torch
    inp = si.make_fp8_inputs(2, 4, 1500, 128, "bf16", 1.0, 8400, "block")
    o1, l1 = _run(inp, "block", True, 0.088)
    o2, l2 = _run(inp, "block", True, 0.088)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


@pytest.mark.parametrize("name", ["C3f8", "C2f8"])
def test_fp8_workload_full_size_sampled(name):
    """The benchmark's 8-bit workloads at full size, in the launch the
    benchmark times: sampled heads, sampled rows against the oracle."""
    w = si.FP8_WORKLOADS[name]
    inp = si.make_fp8_workload_inputs(w)
    say(f"{name}: B={w.B} H={w.H} N={w.N} d={w.d} {w.granularity} causal={w.causal}")
    o, lse = _run(inp, w.granularity, w.causal, w.scale, w.out_dtype)
    og, lg = o.float().cpu().numpy(), lse.cpu().numpy()
    rng = np.random.default_rng(8500)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, w.N - 1], rng.integers(0, w.N, 40)]))
    for b, h in ((0, 0), (w.B - 1, w.H - 1), (0, w.H // 2)):
        o_ref, l_ref = attention_fwd_head(inp["q"][0][b, h], inp["k"][0][b, h], inp["v"][0][b, h], w.scale,
                                          w.causal, rows=rows)
        assert_fwd_ok(fwd_errors(og[b, h, rows], lg[b, h, rows], o_ref, l_ref), w.out_dtype,
                      f"{name} head ({b},{h}) {len(rows)} rows")
