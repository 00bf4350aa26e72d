"""Parity on the GPU for queries against a key/value cache: the library's
fa_fwd_kvcache against the float64 oracle (oracle/kvcache.py) on the same
seeded inputs.

Small shapes are compared element by element on every output; they cover one
and several 32-query blocks with ragged ends, caches split into many key
ranges (merge kernel) and caches one range covers (direct path), filled
lengths below the query count (empty causal rows), empty caches and caches
whose unfilled rows hold NaN.  The decode workload (B=4 H=32, one query, a
32768-row cache) runs at full size in the launch configuration the benchmark
times and is compared on sampled heads.  Tolerances are those of the
forward: O max-abs <= 1e-2 and mean-abs <= 1e-3, LSE max-abs <= 1e-3.
"""

import numpy as np
import pytest

import seeded_inputs as si
from oracle import kvcache_fwd, kvcache_fwd_head, varlen_fwd
from parity import TOL, lib, say, to_device

pytestmark = pytest.mark.gpu


def _run(inp, dtype, causal, scale, seqlens=True, k_override=None, v_override=None):
    import torch
    fa = lib()
    q = to_device(inp["q"][1], dtype)
    k = to_device(inp["k"][1] if k_override is None else k_override, dtype)
    v = to_device(inp["v"][1] if v_override is None else v_override, dtype)
    lens = torch.from_numpy(inp["seqlens"]).cuda() if seqlens else None
    o, lse = fa.fwd_kvcache(q, k, v, lens, causal, scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


def _check(o, lse, o_ref, lse_ref, dtype, label):
    tol = TOL[dtype]
    inf_ref = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), inf_ref), f"{label}: empty rows differ"
    assert np.all(o[inf_ref] == 0), f"{label}: empty rows must be 0"
    fin = ~inf_ref
    do = np.abs(o.astype(np.float64) - o_ref)
    dl = np.abs(lse[fin].astype(np.float64) - lse_ref[fin])
    o_max, o_mean = float(do.max(initial=0.0)), float(do.mean()) if do.size else 0.0
    l_max = float(dl.max(initial=0.0))
    say(f"  {label}: O max {o_max:.3e} mean {o_mean:.3e}  LSE max {l_max:.3e}  empty rows {int(inf_ref.sum())}")
    assert np.isfinite(o).all() and np.isfinite(lse[fin]).all(), label
    assert o_max <= tol["o_max"] and o_mean <= tol["o_mean"] and l_max <= tol["lse_max"], label


SMALL = [  # B, H, Nq, Nk, min_fill
    (2, 3, 1, 40, 0.5),      # one range covers the cache: direct path
    (2, 3, 1, 1000, 0.3),    # 16 ranges of 64 keys, merged
    (3, 2, 5, 777, 0.0),     # several queries, lengths down to 0 (empty rows)
    (2, 2, 32, 300, 0.05),   # one full query block, lengths below the query count
    (2, 2, 33, 513, 0.5),    # two query blocks, ragged
    (1, 3, 70, 70, 1.0),     # square, several query blocks
    (2, 1, 100, 4097, 0.9),  # long-ish cache, ragged tiles
]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,Nq,Nk,fill", SMALL)
def test_small_shapes(B, H, Nq, Nk, fill, causal, d, dtype):
    seed = 7000 + Nq * 13 + Nk
    inp = si.make_kvcache_inputs(B, H, Nq, Nk, d, dtype, 1.0, seed, fill)
    scale = 1.0 / np.sqrt(d)
    say(f"kvcache B{B} H{H} Nq{Nq} Nk{Nk} d{d} {dtype} causal={causal} seed={seed} lens={inp['seqlens'].tolist()}")
    o, lse = _run(inp, dtype, causal, scale)
    o_ref, lse_ref = kvcache_fwd(inp["q"][0], inp["k"][0], inp["v"][0], scale, causal, inp["seqlens"])
    _check(o, lse, o_ref, lse_ref, dtype, f"Nq{Nq} Nk{Nk} d{d} {dtype} causal={causal}")


@pytest.mark.parametrize("d", [64, 128])
def test_without_lengths_square_equals_the_ordinary_forward(d):
    """seqlens NULL and Nq = Nk: the same outputs as fa_fwd's causal attention
    (both within tolerance of the oracle; they run different kernels)."""
    import torch
    fa = lib()
    inp = si.make_kvcache_inputs(1, 2, 300, 300, d, "bf16", 1.0, 77)
    say(f"kvcache square vs fa_fwd d{d}")
    o, lse = _run(inp, "bf16", True, 1 / np.sqrt(d), seqlens=False)
    q, k, v = (to_device(inp[n][1], "bf16") for n in ("q", "k", "v"))
    o2, lse2 = fa.fwd(q, k, v, True, 1 / np.sqrt(d))
    torch.cuda.synchronize()
    o_ref, lse_ref = kvcache_fwd(inp["q"][0], inp["k"][0], inp["v"][0], 1 / np.sqrt(d), True)
    _check(o, lse, o_ref, lse_ref, "bf16", "kvcache")
    _check(o2.float().cpu().numpy(), lse2.cpu().numpy(), o_ref, lse_ref, "bf16", "fa_fwd")


def test_unfilled_rows_are_never_read():
    """NaN in every cache row at and past the filled length changes nothing."""
    inp = si.make_kvcache_inputs(3, 2, 4, 600, 128, "bf16", 1.0, 78, 0.2)
    lens = inp["seqlens"]
    say(f"kvcache NaN past the filled lengths {lens.tolist()}")
    k, v = inp["k"][1].copy(), inp["v"][1].copy()
    for b, L in enumerate(lens):
        k[b, :, L:] = 0x7FC0  # bf16 NaN
        v[b, :, L:] = 0x7FC0
    for causal in (False, True):
        a = _run(inp, "bf16", causal, 0.09)
        b = _run(inp, "bf16", causal, 0.09, k_override=k, v_override=v)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_deterministic_bitwise():
    inp = si.make_kvcache_inputs(2, 4, 3, 5000, 128, "f16", 1.0, 79)
    a = _run(inp, "f16", True, 0.09)
    b = _run(inp, "f16", True, 0.09)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_large_scores_stay_finite():
    """Queries scaled x30: the running maximum is raised across tiles and
    ranges without overflow."""
    inp = si.make_kvcache_inputs(1, 2, 8, 3000, 64, "bf16", 1.0, 80)
    inp["q"] = si.round_to(inp["q"][0] * 30.0, "bf16")
    o, lse = _run(inp, "bf16", True, 0.125)
    o_ref, lse_ref = kvcache_fwd(inp["q"][0], inp["k"][0], inp["v"][0], 0.125, True, inp["seqlens"])
    _check(o, lse, o_ref, lse_ref, "bf16", "x30 queries")


@pytest.mark.parametrize("name", ["D1", "D1d64"])
def test_decode_workload_full_size_sampled_heads(name):
    """The benchmarked decode step at full size, launch configuration as timed."""
    w = si.KV_WORKLOADS[name]
    say(f"{name} full size on GPU: {w}")
    inp = si.make_kv_workload_inputs(w)
    o, lse = _run(inp, w.dtype, w.causal, w.scale)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    errs = []
    for (b, h) in [(0, 0), (1, 17), (2, 5), (3, 31)]:
        L = int(inp["seqlens"][b])
        o_ref, l_ref = kvcache_fwd_head(inp["q"][0][b, h], inp["k"][0][b, h], inp["v"][0][b, h], w.scale,
                                        w.causal, L)
        _check(o[b, h], lse[b, h], o_ref, l_ref, w.dtype, f"{name} head ({b},{h}) L={L}")


# ------------------------------------------------------------ 8-bit (E4M3) cache

def _run8(inp, dtype, causal, scale, k_codes=None, v_codes=None):
    import torch
    fa = lib()
    q = to_device(inp["q"][1], dtype)
    k = torch.from_numpy(inp["k"][1] if k_codes is None else k_codes).cuda()
    v = torch.from_numpy(inp["v"][1] if v_codes is None else v_codes).cuda()
    lens = torch.from_numpy(inp["seqlens"]).cuda()
    o, lse = fa.fwd_kvcache_fp8(q, k, v, float(inp["k_scale"]), float(inp["v_scale"]), lens, causal, scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,Nq,Nk,fill", [SMALL[0], SMALL[1], SMALL[2], SMALL[4], SMALL[6]])
def test_fp8_cache_small_shapes(B, H, Nq, Nk, fill, causal, d, dtype):
    """Against the oracle on the dequantised cache (k_scale * E4M3 codes): the
    same attention as with a 16-bit cache, to the same tolerances."""
    seed = 8000 + Nq * 13 + Nk
    inp = si.make_kvcache_fp8_inputs(B, H, Nq, Nk, d, dtype, 1.0, seed, fill)
    scale = 1.0 / np.sqrt(d)
    say(f"kvcache fp8 B{B} H{H} Nq{Nq} Nk{Nk} d{d} {dtype} causal={causal} seed={seed} "
        f"k_scale={inp['k_scale']:.4g} v_scale={inp['v_scale']:.4g}")
    o, lse = _run8(inp, dtype, causal, scale)
    o_ref, lse_ref = kvcache_fwd(inp["q"][0], inp["k"][0], inp["v"][0], scale, causal, inp["seqlens"])
    _check(o, lse, o_ref, lse_ref, dtype, f"fp8 Nq{Nq} Nk{Nk} d{d} {dtype} causal={causal}")


def test_fp8_cache_unfilled_rows_are_never_read():
    inp = si.make_kvcache_fp8_inputs(3, 2, 4, 600, 128, "bf16", 1.0, 81, 0.2)
    k, v = inp["k"][1].copy(), inp["v"][1].copy()
    for b, L in enumerate(inp["seqlens"]):
        k[b, :, L:] = 0x7F  # E4M3 NaN
        v[b, :, L:] = 0x7F
    say(f"kvcache fp8 NaN codes past the filled lengths {inp['seqlens'].tolist()}")
    for causal in (False, True):
        a = _run8(inp, "bf16", causal, 0.09)
        b = _run8(inp, "bf16", causal, 0.09, k_codes=k, v_codes=v)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_fp8_decode_workload_full_size_sampled_heads():
    """The benchmarked 8-bit decode step at full size: parity against the
    oracle on the dequantised cache, and (reported separately, as the error
    the quantisation itself adds) the distance to the oracle on the 16-bit
    cache the codes were quantised from."""
    w = si.KV_WORKLOADS["D1f8"]
    say(f"D1f8 full size on GPU: {w}")
    inp = si.make_kv_workload_inputs(w)
    o, lse = _run8(inp, w.dtype, w.causal, w.scale)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    for (b, h) in [(0, 0), (1, 17), (2, 5), (3, 31)]:
        L = int(inp["seqlens"][b])
        o_ref, l_ref = kvcache_fwd_head(inp["q"][0][b, h], inp["k"][0][b, h], inp["v"][0][b, h], w.scale,
                                        w.causal, L)
        _check(o[b, h], lse[b, h], o_ref, l_ref, w.dtype, f"D1f8 head ({b},{h}) L={L}")
        o16, l16 = kvcache_fwd_head(inp["q"][0][b, h], inp["k16"][0][b, h], inp["v16"][0][b, h], w.scale,
                                    w.causal, L)
        qo, ql = float(np.abs(o[b, h] - o16).max()), float(np.abs(lse[b, h] - l16).max())
        say(f"  quantisation error vs the 16-bit cache: O max-abs {qo:.3e}, LSE max-abs {ql:.3e}")
        assert qo < 0.05 and ql < 0.5  # sanity only: E4M3 keeps 3 mantissa bits


# ------------------------------------------------------------ variable-length packed batches

def _run_varlen(inp, dtype, causal, scale, max_q=None, max_k=None, o_init=None):
    import torch
    fa = lib()
    q, k, v = (to_device(inp[n][1], dtype) for n in ("q", "k", "v"))
    cq, ck = (torch.from_numpy(inp[n]).cuda() for n in ("cu_q", "cu_k"))
    mq = int(np.diff(inp["cu_q"]).max()) if max_q is None else max_q
    mk = int(np.diff(inp["cu_k"]).max()) if max_k is None else max_k
    o = torch.zeros_like(q) if o_init is None else to_device(o_init, dtype)
    lse = torch.empty((q.shape[1], q.shape[0]), dtype=torch.float32, device="cuda")
    nb = int(fa.load_library().fa_fwd_varlen_workspace_bytes(len(inp["cu_q"]) - 1, q.shape[1], max(mq, 1),
                                                                max(mk, 1), q.shape[2], fa.dtype_code(q)))
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda") if nb else None
    fa.fa_fwd_varlen(q, k, v, cq, ck, o, lse, ws, max(mq, 1), max(mk, 1), scale, causal)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


VARLEN = [  # query lengths, key lengths
    ([1, 100, 0, 33, 257], [50, 100, 7, 33, 300]),  # decode row, square, empty, ragged, longer cache
    ([64, 5, 200], [16, 500, 40]),                   # more queries than keys (empty causal rows)
    ([1000, 1], [1000, 3000]),                       # one long sequence beside a decode step
]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", range(len(VARLEN)))
def test_varlen_small(case, causal, d, dtype):
    lq, lk = VARLEN[case]
    seed = 9000 + 17 * case + d
    inp = si.make_varlen_inputs(lq, lk, 3, d, dtype, 1.0, seed)
    scale = 1.0 / np.sqrt(d)
    say(f"varlen lq={lq} lk={lk} H3 d{d} {dtype} causal={causal} seed={seed}")
    o, lse = _run_varlen(inp, dtype, causal, scale)
    o_ref, lse_ref = varlen_fwd(inp["q"][0], inp["k"][0], inp["v"][0], inp["cu_q"], inp["cu_k"], scale, causal)
    _check(o.transpose(1, 0, 2), lse, o_ref.transpose(1, 0, 2), lse_ref, dtype,
           f"varlen case {case} d{d} {dtype} causal={causal}")


def test_varlen_equal_lengths_equal_the_ordinary_forward():
    """Equal lengths, packed: the same outputs as fa_fwd on the [B, H, N, d]
    layout of the same values (different kernels, both against the oracle)."""
    import torch
    fa = lib()
    B, H, N, d = 3, 4, 300, 128
    inp = si.make_varlen_inputs([N] * B, [N] * B, H, d, "bf16", 1.0, 91)
    o, lse = _run_varlen(inp, "bf16", True, 1 / np.sqrt(d))
    dense = lambda x: np.ascontiguousarray(x.reshape(B, N, H, d).transpose(0, 2, 1, 3))
    q, k, v = (to_device(dense(inp[n][1]), "bf16") for n in ("q", "k", "v"))
    o2, lse2 = fa.fwd(q, k, v, True, 1 / np.sqrt(d))
    torch.cuda.synchronize()
    o2 = o2.float().cpu().numpy().transpose(0, 2, 1, 3).reshape(B * N, H, d)
    lse2 = lse2.cpu().numpy().transpose(1, 0, 2).reshape(H, B * N)
    o_ref, lse_ref = varlen_fwd(inp["q"][0], inp["k"][0], inp["v"][0], inp["cu_q"], inp["cu_k"], 1 / np.sqrt(d), True)
    t = lambda x: x.transpose(1, 0, 2)
    _check(t(o), lse, t(o_ref), lse_ref, "bf16", "fa_fwd_varlen")
    _check(t(o2), lse2, t(o_ref), lse_ref, "bf16", "fa_fwd on the same values")


def test_varlen_rows_outside_the_sequences_are_left_unchanged():
    inp = si.make_varlen_inputs([10, 20], [30, 20], 2, 64, "bf16", 1.0, 92)
    tq = 30
    inp["cu_q"] = np.array([0, 10, 25], np.int32)  # rows 25..29 belong to no sequence
    sentinel = si.round_to(np.full((tq, 2, 64), 7.0, np.float32), "bf16")[1]
    o, lse = _run_varlen(inp, "bf16", False, 0.125, max_q=20, max_k=30, o_init=sentinel)
    assert np.all(o[25:] == 7.0)
    o_ref, lse_ref = varlen_fwd(inp["q"][0], inp["k"][0], inp["v"][0], inp["cu_q"], inp["cu_k"], 0.125, False)
    _check(o[:25].transpose(1, 0, 2), lse[:, :25], o_ref[:25].transpose(1, 0, 2), lse_ref[:, :25], "bf16",
           "partial cover")


def test_varlen_one_range_per_head_direct_path_sampled():
    """Many long sequences: every head's keys fit one range, so the split
    kernel writes O and LSE itself (no merge); sampled heads against the oracle."""
    fa = lib()
    lq = lk = [4096, 4000, 4096, 3900]
    H, d = 16, 128
    assert fa.load_library().fa_fwd_varlen_workspace_bytes(4, H, 4096, 4096, d, fa.FA_BF16) == 0
    inp = si.make_varlen_inputs(lq, lk, H, d, "bf16", 1.0, 93)
    say("varlen direct path: 4 sequences of ~4096, H16 d128 causal")
    o, lse = _run_varlen(inp, "bf16", True, 1 / np.sqrt(d))
    cu = inp["cu_q"]
    for b, h in [(0, 0), (1, 7), (3, 15)]:
        qs = slice(cu[b], cu[b + 1])
        rows = np.r_[0:256, lq[b] - 128:lq[b]]
        of, lf = kvcache_fwd_head(inp["q"][0][qs, h], inp["k"][0][qs, h], inp["v"][0][qs, h], 1 / np.sqrt(d), True)
        _check(o[qs, h][rows], lse[h, qs][rows], of[rows], lf[rows], "bf16", f"direct path seq {b} head {h}")


def test_varlen_malformed_prefix_sums_stay_in_bounds():
    """Prefix sums that decrease or pass the end are clamped by the kernels
    (no access leaves the tensors); rows only a well-formed sequence covers
    are still exact.  Here sequence 1 has a negative count (skipped) and
    sequence 2 runs past total_q (cut at the end)."""
    lq = [50, 0, 70]
    inp = si.make_varlen_inputs(lq, [60, 10, 80], 2, 128, "bf16", 1.0, 94)
    inp["cu_q"] = np.array([0, 50, 30, 100000], np.int32)  # total_q = 120
    say(f"varlen malformed cu_q {inp['cu_q'].tolist()}")
    o, lse = _run_varlen(inp, "bf16", True, 0.088, max_q=128, max_k=80)
    assert np.isfinite(o).all()
    # rows 0..29 belong to sequence 0 only (sequence 2 starts at row 30)
    of, lf = kvcache_fwd_head(inp["q"][0][0:50, 1], inp["k"][0][0:60, 1], inp["v"][0][0:60, 1], 0.088, True)
    _check(o[0:30, 1], lse[1, 0:30], of[0:30], lf[0:30], "bf16", "sequence 0 rows")
