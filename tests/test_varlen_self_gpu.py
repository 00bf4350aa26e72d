"""Parity on the GPU for fa_fwd_varlen on self-attention batches (one
prefix-sum array passed for both queries and keys), which runs the square
forward kernels on the packed rows in place: against the float64 oracle
(oracle.varlen_fwd) on the same seeded inputs, bit for bit against fa_fwd at
equal lengths, and against the split-key path fa_fwd_varlen takes when the
two prefix-sum arrays are different buffers.  Tolerances are the forward's
(O max-abs <= 1e-2, mean-abs <= 1e-3; LSE max-abs <= 1e-3)."""

import numpy as np
import pytest

import seeded_inputs as si
from oracle import kvcache_fwd_head, varlen_fwd
from parity import TOL, assert_fwd_ok_peaked, lib, say, to_device

pytestmark = pytest.mark.gpu


def _fwd(inp, dtype, causal, scale, max_len=None, same=True, o_init=None):
    import torch
    fa = lib()
    q, k, v = (to_device(inp[n][1], dtype) for n in ("q", "k", "v"))
    cu = torch.from_numpy(inp["cu_q"]).cuda()
    ck = cu if same else cu.clone()
    mx = max(int(np.diff(inp["cu_q"]).max()) if max_len is None else max_len, 1)
    o = torch.zeros_like(q) if o_init is None else to_device(o_init, dtype)
    lse = torch.empty((q.shape[1], q.shape[0]), dtype=torch.float32, device="cuda")
    nb = int(fa.load_library().fa_fwd_varlen_workspace_bytes(len(inp["cu_q"]) - 1, q.shape[1], mx, mx, q.shape[2],
                                                              fa.dtype_code(q)))
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda") if nb else None
    fa.fa_fwd_varlen(q, k, v, cu, ck, o, lse, ws, mx, mx, scale, causal)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


def _check(o, lse, o_ref, lse_ref, dtype, label):
    tol = TOL[dtype]
    assert np.isfinite(o).all() and np.isfinite(lse).all(), label
    do = np.abs(o.astype(np.float64) - o_ref)
    dl = np.abs(lse.astype(np.float64) - lse_ref)
    o_max, o_mean, l_max = float(do.max(initial=0.0)), float(do.mean()) if do.size else 0.0, float(dl.max(initial=0.0))
    say(f"  {label}: O max {o_max:.3e} mean {o_mean:.3e}  LSE max {l_max:.3e}")
    assert o_max <= tol["o_max"] and o_mean <= tol["o_mean"] and l_max <= tol["lse_max"], label


LENGTHS = [
    [1, 100, 0, 33, 257],  # one row, less than a tile, empty, ragged, two tiles
    [64, 5, 600],           # short and several tiles
    [1000, 1],              # one long sequence beside a one-row one
]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [32, 64, 128])  # 32: the split-key kernel serves it
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", range(len(LENGTHS)))
def test_varlen_self_small(case, causal, d, dtype):
    lens = LENGTHS[case]
    seed = 9600 + 11 * case + d
    inp = si.make_varlen_inputs(lens, lens, 3, d, dtype, 1.0, seed)
    scale = 1.0 / np.sqrt(d)
    say(f"varlen self lens={lens} H3 d{d} {dtype} causal={causal} seed={seed}")
    o, lse = _fwd(inp, dtype, causal, scale)
    o_ref, lse_ref = varlen_fwd(inp["q"][0], inp["k"][0], inp["v"][0], inp["cu_q"], inp["cu_k"], scale, causal)
    rows = np.concatenate([np.arange(a, b) for a, b in zip(inp["cu_q"][:-1], inp["cu_q"][1:])])
    _check(o[rows], lse[:, rows], o_ref[rows], lse_ref[:, rows], dtype, f"lens {lens} d{d} {dtype} causal={causal}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_self_equal_lengths_bitwise_equal_fa_fwd(causal, d):
    """Equal lengths: the packed kernels take fa_fwd's tiles in the same
    order (only the row addressing differs), so O and LSE agree bit for bit;
    the split-key path (different prefix-sum buffers) agrees within the
    tolerance, and both match the oracle."""
    import torch
    fa = lib()
    B, H, N = 3, 4, 700
    scale = 1 / np.sqrt(d)
    inp = si.make_varlen_inputs([N] * B, [N] * B, H, d, "bf16", 1.0, 9700 + d + int(causal))
    o, lse = _fwd(inp, "bf16", causal, scale)
    dense = lambda x: np.ascontiguousarray(x.reshape(B, N, H, d).transpose(0, 2, 1, 3))
    q, k, v = (to_device(dense(inp[n][1]), "bf16") for n in ("q", "k", "v"))
    od, lsed = fa.fwd(q, k, v, causal, scale)
    torch.cuda.synchronize()
    od = od.float().cpu().numpy().transpose(0, 2, 1, 3).reshape(B * N, H, d)
    lsed = lsed.cpu().numpy().transpose(1, 0, 2).reshape(H, B * N)
    assert np.array_equal(o, od) and np.array_equal(lse, lsed)
    o2, lse2 = _fwd(inp, "bf16", causal, scale, same=False)
    o_ref, lse_ref = varlen_fwd(inp["q"][0], inp["k"][0], inp["v"][0], inp["cu_q"], inp["cu_k"], scale, causal)
    _check(o, lse, o_ref, lse_ref, "bf16", f"square kernels d{d} causal={causal}")
    _check(o2, lse2, o_ref, lse_ref, "bf16", f"split-key kernel d{d} causal={causal}")


def test_varlen_self_rows_outside_and_max_len_above_lengths():
    """Rows of no sequence keep their contents; a max_len above every length
    only adds workgroups that return at once."""
    inp = si.make_varlen_inputs([10, 20, 5], [10, 20, 5], 2, 128, "bf16", 1.0, 9710)
    inp["cu_q"] = np.array([0, 10, 25], np.int32)  # rows 25..34 belong to no sequence
    sentinel = si.round_to(np.full((35, 2, 128), 7.0, np.float32), "bf16")[1]
    o, lse = _fwd(inp, "bf16", True, 0.088, max_len=600, o_init=sentinel)
    assert np.all(o[25:] == 7.0)
    o_ref, lse_ref = varlen_fwd(inp["q"][0], inp["k"][0], inp["v"][0], inp["cu_q"], inp["cu_q"], 0.088, True)
    _check(o[:25], lse[:, :25], o_ref[:25], lse_ref[:, :25], "bf16", "partial cover, max_len 600")


def test_varlen_self_malformed_prefix_sums_stay_in_bounds():
    """Clamped prefix sums (a negative length, a sequence past the end): no
    access leaves the tensors, and rows only sequence 0 covers are exact."""
    lens = [50, 0, 70]
    inp = si.make_varlen_inputs(lens, lens, 2, 64, "bf16", 1.0, 9720)
    inp["cu_q"] = np.array([0, 50, 30, 100000], np.int32)  # total = 120
    o, lse = _fwd(inp, "bf16", True, 0.125, max_len=128)
    assert np.isfinite(o).all()
    of, lf = kvcache_fwd_head(inp["q"][0][0:50, 1], inp["k"][0][0:50, 1], inp["v"][0][0:50, 1], 0.125, True)
    _check(o[0:30, 1], lse[1, 0:30], of[0:30], lf[0:30], "bf16", "sequence 0 rows 0..29")


def test_varlen_self_prefill_batch_full_size_sampled():
    """The 16-sequence packed batch (lengths uniform in [512, 4096], seed
    1008, H=16, d=128, bf16, causal) the benchmark times; sampled heads of
    two sequences against the oracle."""
    rng = np.random.default_rng(1008)
    lens = rng.integers(512, 4097, size=16).tolist()
    H, d = 16, 128
    scale = 1 / np.sqrt(d)
    inp = si.make_varlen_inputs(lens, lens, H, d, "bf16", 1.0, 1008)
    say(f"varlen self prefill batch lengths {lens}")
    o, lse = _fwd(inp, "bf16", True, scale)
    cu = inp["cu_q"]
    for b, h in [(int(np.argmax(lens)), 3), (5, 12)]:
        rows = slice(int(cu[b]), int(cu[b + 1]))
        of, lf = kvcache_fwd_head(inp["q"][0][rows, h], inp["k"][0][rows, h], inp["v"][0][rows, h], scale, True)
        _check(o[rows, h], lse[h, rows], of, lf, "bf16", f"sequence {b} head {h}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_self_growing_scores(causal, d):
    """Keys scaled up along each sequence (x1 to x6): later key tiles hold row
    maxima far above the first tile's, so the packed kernels must raise their
    reference maximum (d = 64: the tile is re-based; d = 128: the pass is
    redone against exact maxima), as the dense kernels do."""
    lens = [600, 300, 1000, 1]
    seed = 9800 + d + int(causal)
    inp = si.make_varlen_inputs(lens, lens, 2, d, "bf16", 1.0, seed)
    pos = np.concatenate([np.arange(n) / n for n in lens]).astype(np.float32)
    inp["k"] = si.round_to(inp["k"][0] * (1.0 + 5.0 * pos)[:, None, None], "bf16")
    scale = 1.0 / np.sqrt(d)
    say(f"varlen self growing keys lens={lens} H2 d{d} causal={causal} seed={seed}")
    o, lse = _fwd(inp, "bf16", causal, scale)
    o_ref, lse_ref = varlen_fwd(inp["q"][0], inp["k"][0], inp["v"][0], inp["cu_q"], inp["cu_k"], scale, causal)
    # peaked rows: |O| reaches 5.4 here, where bf16 output rounding alone moves an element by up to 0.0156
    assert_fwd_ok_peaked(o, lse, o_ref, lse_ref, "bf16", f"growing keys lens {lens} d{d} causal={causal}")
