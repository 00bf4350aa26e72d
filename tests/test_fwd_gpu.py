"""Forward parity on the GPU: the library's fa_fwd against the float64 oracle on
the same seeded inputs.

Small shapes (several tiles and ragged tails, every dtype, d, mask) are compared
element by element on every output.  The full-size workloads run in the same
launch configuration the benchmark times and are compared on sampled outputs
(whole heads, or sampled rows of sampled heads) that the oracle computes one by
one.
"""

import numpy as np
import pytest

import seeded_inputs as si
from oracle import attention_fwd, attention_fwd_head
from parity import TOL, assert_fwd_ok, assert_fwd_ok_peaked, fwd_errors, gpu_fwd, lib, say, to_device

pytestmark = pytest.mark.gpu


def _small(B, H, N, d, dtype, causal, seed, sigma=1.0, scale=None):
    inp = si.make_inputs(B, H, N, d, dtype, sigma, seed)
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    say(f"fwd small B{B} H{H} N{N} d{d} {dtype} causal={causal} seed={seed} scale={scale}")
    q, k, v, o, lse = gpu_fwd(inp, dtype, causal, scale)
    o_ref, lse_ref = attention_fwd(inp["q"][0], inp["k"][0], inp["v"][0], scale, causal)
    err = fwd_errors(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref)
    assert_fwd_ok(err, dtype, f"N{N} d{d} {dtype} causal={causal}")


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 255, 257, 1000])
def test_small_shapes_and_tails(N, causal, d, dtype):
    _small(1, 2, N, d, dtype, causal, seed=7000 + N + d)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
def test_zero_scale(causal, dtype):
    # scale 0: every visible key has the same weight (O is the mean of the
    # visible V rows, LSE the log of their count); masked keys must stay out
    _small(1, 2, 300, 64, dtype, causal, seed=91, scale=0.0)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_several_heads_and_batches(dtype):
    _small(3, 5, 700, 128, dtype, True, seed=77)
    _small(2, 3, 640, 64, dtype, False, seed=78)


def test_c1_tiny_fp32_full():
    w = si.WORKLOADS["C1"]
    inp = si.make_workload_inputs(w)
    say(f"C1 {w}")
    q, k, v, o, lse = gpu_fwd(inp, w.dtype, w.causal, w.scale)
    o_ref, lse_ref = attention_fwd(inp["q"][0], inp["k"][0], inp["v"][0], w.scale, w.causal)
    err = fwd_errors(o.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref)
    assert_fwd_ok(err, "f32", "C1")


def _sampled(w, heads, rows_fn):
    inp = si.make_workload_inputs(w)
    say(f"{w.name} full size on GPU: {w}")
    q, k, v, o, lse = gpu_fwd(inp, w.dtype, w.causal, w.scale)
    og = o.float().cpu().numpy()
    lg = lse.cpu().numpy()
    errs = []
    for (b, hh) in heads:
        rows = rows_fn(w.N)
        o_ref, l_ref = attention_fwd_head(inp["q"][0][b, hh], inp["k"][0][b, hh], inp["v"][0][b, hh],
                                          w.scale, w.causal, rows=rows)
        e = fwd_errors(og[b, hh][rows], lg[b, hh][rows], o_ref, l_ref)
        say(f"  head ({b},{hh}) {len(rows)} rows: {e}")
        errs.append(e)
    agg = dict(o_max=max(e["o_max"] for e in errs), lse_max=max(e["lse_max"] for e in errs),
               o_mean=float(np.mean([e["o_mean"] for e in errs])))
    assert_fwd_ok(agg, w.dtype, w.name)
    assert np.all(np.isfinite(lg)) and np.isfinite(og).all()


def _rows_early_random_late(n, early=512, rand=256, late=64, seed=5):
    rng = np.random.default_rng(seed)
    r = set(range(min(n, early))) | set(rng.integers(0, n, rand).tolist()) | set(range(max(0, n - late), n))
    return np.array(sorted(r))


def test_c2_bf16_noncausal_sampled_heads():
    w = si.WORKLOADS["C2"]
    _sampled(w, [(0, 0), (1, 7), (2, 13), (3, 15)], lambda n: np.arange(n))


def test_c3_bf16_causal_sampled():
    w = si.WORKLOADS["C3"]
    _sampled(w, [(0, 0), (1, 31), (0, 17)], _rows_early_random_late)


def test_c3_d64_bf16_causal_sampled():
    w = si.WORKLOADS["C3d64"]
    _sampled(w, [(0, 3), (1, 30)], _rows_early_random_late)


@pytest.mark.parametrize("name", ["C5", "C5d128", "C5d256"])
def test_c5_forward_full_size_sampled(name):
    # the forward half of the timed step (persistent grid at d = 64; tile
    # pairs and row-major V at d = 256), on its own outputs
    w = si.WORKLOADS[name]
    _sampled(w, [(0, 0), (7, 15), (3, 9)], _rows_early_random_late)


def test_c4_fp16_causal_long_context_sampled():
    w = si.WORKLOADS["C4"]
    _sampled(w, [(0, 0), (0, 31)], lambda n: _rows_early_random_late(n, early=256, rand=128, late=32))


# ------------------------------------------------------------ properties on the GPU

def test_values_all_one_give_exactly_one():
    import torch
    inp = si.make_inputs(1, 2, 333, 128, "bf16", 1.0, 11)
    inp["v"] = si.round_to(np.ones((1, 2, 333, 128), np.float32), "bf16")
    for causal in (False, True):
        q, k, v, o, lse = gpu_fwd(inp, "bf16", causal, 1 / np.sqrt(128))
        assert torch.all(o.float() == 1.0)


def test_deterministic_bitwise():
    import torch
    inp = si.make_inputs(2, 4, 1500, 128, "bf16", 1.0, 12)
    _, _, _, o1, l1 = gpu_fwd(inp, "bf16", True, 1 / np.sqrt(128))
    _, _, _, o2, l2 = gpu_fwd(inp, "bf16", True, 1 / np.sqrt(128))
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


def test_large_scores_stay_finite_and_pick_the_max_key():
    """Queries scaled x30: weights collapse onto the best key; nothing overflows."""
    d = 64
    inp = si.make_inputs(1, 2, 300, d, "bf16", 1.0, 13)
    qv = inp["q"][0] * 30
    inp["q"] = si.round_to(qv, "bf16")
    scale = 1 / np.sqrt(d)
    _, _, _, o, lse = gpu_fwd(inp, "bf16", True, scale)
    og = o.float().cpu().numpy()
    assert np.isfinite(og).all() and np.isfinite(lse.cpu().numpy()).all()
    o_ref, l_ref = attention_fwd(inp["q"][0], inp["k"][0], inp["v"][0], scale, True)
    err = fwd_errors(og, lse.cpu().numpy(), o_ref, l_ref)
    assert_fwd_ok(err, "bf16", "x30 queries")


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_growing_scores_update_the_reference_maximum(d, causal):
    """Keys scaled up 6x along the sequence: later key tiles hold row maxima far
    above the first tile's (by more than the kernels' tile-sum bound allows),
    so the reference maximum must be raised (d = 64: the tile is re-based;
    d = 128, 256: the pass is redone against exact maxima).  Result as the
    oracle."""
    N = 600
    inp = si.make_inputs(1, 2, N, d, "bf16", 1.0, 17 + d)
    grow = (1.0 + 5.0 * np.arange(N) / N)[None, None, :, None]
    inp["k"] = si.round_to(inp["k"][0] * grow, "bf16")
    scale = 1 / np.sqrt(d)
    _, _, _, o, lse = gpu_fwd(inp, "bf16", causal, scale)
    og = o.float().cpu().numpy()
    assert np.isfinite(og).all() and np.isfinite(lse.cpu().numpy()).all()
    o_ref, l_ref = attention_fwd(inp["q"][0], inp["k"][0], inp["v"][0], scale, causal)
    # peaked rows: the bound allows for the bf16 rounding of the output itself
    assert_fwd_ok_peaked(og, lse.cpu().numpy(), o_ref, l_ref, "bf16", f"growing keys d{d} causal={causal}")


def test_growing_scores_take_the_exact_maximum_rerun():
    """The d = 128 kernel redoes a workgroup's pass against exact row maxima
    when a row's tile sum passes its bound: with keys growing x1..x6 along
    the sequence (most rows trigger it) a call must take clearly longer than
    on the same draw without the growth (the rerun costs an extra pass of
    Q K^T plus the whole pass again), while both stay exact."""
    import torch
    fa = lib()
    B, H, N, d = 1, 32, 4096, 128
    inp = si.make_inputs(B, H, N, d, "bf16", 1.0, 4242)
    grow = (1.0 + 5.0 * np.arange(N, dtype=np.float32) / N)[None, None, :, None]
    kg = to_device(si.round_to(inp["k"][0] * grow, "bf16")[1], "bf16")
    q, k, v = (to_device(inp[n][1], "bf16") for n in ("q", "k", "v"))
    o, lse = torch.empty_like(q), torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    scale = 1 / np.sqrt(d)

    def median_ms(kk):
        for _ in range(3):
            fa.fa_fwd(q, kk, v, o, lse, scale, True)
        ts = []
        for _ in range(7):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fa.fa_fwd(q, kk, v, o, lse, scale, True)
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))

    t_plain, t_grow = median_ms(k), median_ms(kg)
    say(f"  d=128 causal B1 H32 N4096: plain {t_plain * 1e3:.0f} us, growing keys {t_grow * 1e3:.0f} us "
        f"(x{t_grow / t_plain:.2f})")
    assert t_grow > 1.3 * t_plain, (t_plain, t_grow)
    # and the rerun result is exact: sampled rows against the oracle
    rows = np.array([0, 1, 63, 64, 1000, 2047, 2048, 4095])
    kk = si.round_to(inp["k"][0] * grow, "bf16")[0]
    for h in (0, 17):
        o_ref, l_ref = attention_fwd_head(inp["q"][0][0, h], kk[0, h], inp["v"][0][0, h], scale, True, rows=rows)
        og = o[0, h, rows].float().cpu().numpy()
        lg = lse[0, h, rows].cpu().numpy()
        assert_fwd_ok_peaked(og, lg, o_ref, l_ref, "bf16", f"growing keys rerun head {h}")


def test_key_shift_invariance_on_gpu():
    """Adding one vector to every key leaves O unchanged (within rounding) and
    shifts LSE_i by scale * q_i . c."""
    d = 64
    inp = si.make_inputs(1, 2, 400, d, "f32", 1.0, 14)
    c = np.linspace(-1, 1, d).astype(np.float32)
    inp2 = dict(inp)
    inp2["k"] = si.round_to(inp["k"][0] + c, "f32")
    scale = 1 / np.sqrt(d)
    _, _, _, o1, l1 = gpu_fwd(inp, "f32", False, scale)
    _, _, _, o2, l2 = gpu_fwd(inp2, "f32", False, scale)
    np.testing.assert_allclose(o2.cpu().numpy(), o1.cpu().numpy(), atol=2e-5)
    shift = scale * (inp["q"][0].astype(np.float64) @ c.astype(np.float64))
    np.testing.assert_allclose(l2.cpu().numpy(), l1.cpu().numpy() + shift, atol=2e-4)


# ------------------------------------------------------------ O(N) device memory (long context)

def test_c4_peak_memory_is_inputs_and_outputs_only():
    """Long-context forward (B=1 H=32 d=128 fp16 causal): peak device memory
    during fa_fwd is exactly Q, K, V, O plus the float32 LSE, i.e. linear in
    N, and the library allocates nothing (free device memory is unchanged
    across the call).  A materialised N x N score matrix would need
    H*N^2*2 bytes (64 GiB at N = 32768)."""
    import torch
    fa = __import__("parity").lib()
    B, H, d = 1, 32, 128
    # one small call first, so that loading the kernel's code is not counted
    x = torch.zeros((1, 1, 256, d), dtype=torch.float16, device="cuda")
    fa.fwd(x, x, x, True)
    torch.cuda.synchronize()
    del x
    peaks = {}
    for N in (8192, 16384, 32768):
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats()
        base = torch.cuda.memory_allocated()
        g = torch.Generator(device="cuda").manual_seed(1004)
        q, k, v = (torch.randn((B, H, N, d), generator=g, device="cuda", dtype=torch.float32)
                   .mul_(0.5).to(torch.float16) for _ in range(3))
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats()
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        free0, _ = torch.cuda.mem_get_info()
        fa.fa_fwd(q, k, v, o, lse, 1.0 / np.sqrt(d), True)
        torch.cuda.synchronize()
        free1, _ = torch.cuda.mem_get_info()
        peak = torch.cuda.max_memory_allocated() - base
        held = torch.cuda.memory_allocated() - base
        expect = 4 * B * H * N * d * 2 + 4 * B * H * N
        nbytes = sum(t.numel() * t.element_size() for t in (q, k, v, o, lse))
        say(f"  N={N}: peak {peak} B, tensors {nbytes} B (Q, K, V, O + LSE = {expect}), "
            f"free device memory before/after fa_fwd {free0}/{free1}")
        assert nbytes == expect
        # nothing beyond the five tensors was ever held; the caching allocator
        # rounds a block below 2 MiB (the 1 MiB LSE at N = 8192) up to 2 MiB
        assert peak == held and 0 <= held - expect < (2 << 20), (N, peak, held, expect)
        assert free1 == free0, "the library allocated device memory"
        assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
        peaks[N] = peak
        del q, k, v, o, lse
    assert peaks[32768] == 2 * peaks[16384]  # linear in N (both sizes are whole 2 MiB blocks)
    assert peaks[32768] == 1_077_936_128
