"""Backward parity on the GPU for causal self-attention over a packed
variable-length batch: fa_bwd_varlen (fed the library's own fa_fwd_varlen O
and LSE, as a training step would) against the float64 oracle's per-sequence
softmax-Jacobian gradient (oracle.varlen_bwd_causal) on the same seeded Q, K,
V, dO.  Bound: relative L2 <= 1e-2 for each of dQ, dK, dV per sequence and
head, as for fa_bwd.  Lengths cover one row, empty sequences, lengths below,
at and above the 128-row tiles, and ragged tails; the 16-sequence prefill
batch the benchmark times runs in full and is checked on sampled sequences."""

import numpy as np
import pytest

import seeded_inputs as si
from oracle import attention_bwd_head, varlen_bwd_causal
from parity import BWD_REL_L2, lib, rel_l2, say, to_device

pytestmark = pytest.mark.gpu


def _upload(inp, dtype):
    import torch
    q, k, v, do = (to_device(inp[n][1], dtype) for n in ("q", "k", "v", "do"))
    cu = torch.from_numpy(inp["cu_q"]).cuda()
    return q, k, v, do, cu


def _run(inp, dtype, scale, max_len=None, init=None):
    """fa_fwd_varlen (causal) then fa_bwd_varlen; returns dq, dk, dv as float
    [total, H, d] arrays.  `init` pre-fills the gradient buffers."""
    import torch
    fa = lib()
    q, k, v, do, cu = _upload(inp, dtype)
    mx = int(np.diff(inp["cu_q"]).max()) if max_len is None else max_len
    mx = max(mx, 1)
    o, lse = fa.fwd_varlen(q, k, v, cu, cu, mx, mx, True, scale)
    if init is None:
        dq, dk, dv = fa.bwd_varlen(q, k, v, o, lse, do, cu, cu, mx, mx, True, scale)
    else:
        dq, dk, dv = (to_device(init, dtype) for _ in range(3))
        nb = fa.fa_bwd_varlen_workspace_bytes(len(inp["cu_q"]) - 1, q.shape[1], q.shape[0], mx, q.shape[2],
                                              fa.dtype_code(q))
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
        fa.fa_bwd_varlen(q, k, v, o, lse, do, cu, cu, dq, dk, dv, ws, mx, mx, scale, True)
    torch.cuda.synchronize()
    return tuple(g.float().cpu().numpy() for g in (dq, dk, dv))


def _check_seqs(inp, grads, ref, seqs, heads, label):
    cu = inp["cu_q"]
    worst = {"dq": 0.0, "dk": 0.0, "dv": 0.0}
    for b in seqs:
        rows = slice(int(cu[b]), int(cu[b + 1]))
        for h in heads:
            r = ref(b, h) if callable(ref) else tuple(x[rows, h] for x in ref)
            for name, g, rr in zip(("dq", "dk", "dv"), grads, r):
                gg = g[rows, h]
                assert np.isfinite(gg).all(), (label, name, b, h)
                if gg.size == 0:
                    continue
                if np.linalg.norm(rr) == 0.0:
                    # a one-row sequence: dQ = dK = 0 exactly; only rounding noise may remain
                    assert np.abs(gg).max() <= 1e-5, (label, name, b, h)
                    continue
                worst[name] = max(worst[name], rel_l2(gg, rr))
    say(f"  {label}: rel-L2 {worst}")
    for name, e in worst.items():
        assert e <= BWD_REL_L2, (label, name, e)


LENGTHS = [
    [1, 100, 0, 33, 257],  # one row, one tile, empty, ragged, several tiles
    [64, 5, 200],           # below and above a tile
    [1000, 1],              # one long sequence beside a one-row one
]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("case", range(len(LENGTHS)))
def test_varlen_bwd_small(case, d, dtype):
    lens = LENGTHS[case]
    seed = 9300 + 13 * case + d
    H = 3
    inp = si.make_varlen_inputs(lens, lens, H, d, dtype, 1.0, seed, backward=True)
    scale = 1.0 / np.sqrt(d)
    say(f"varlen bwd lens={lens} H{H} d{d} {dtype} seed={seed}")
    grads = _run(inp, dtype, scale)
    ref = varlen_bwd_causal(inp["q"][0], inp["k"][0], inp["v"][0], inp["do"][0], inp["cu_q"], scale)
    _check_seqs(inp, grads, ref, range(len(lens)), range(H), f"lens {lens} d{d} {dtype}")


@pytest.mark.parametrize("d", [64, 128])
def test_varlen_bwd_equal_lengths_bitwise_equal_the_ordinary_backward(d):
    """Equal lengths: the packed kernels take the same tiles in the same
    order as fa_bwd on the [B, H, N, d] layout of the same values (only the
    row addressing differs), so the gradients agree bit for bit."""
    import torch
    fa = lib()
    B, H, N = 3, 4, 300
    scale = 1 / np.sqrt(d)
    inp = si.make_varlen_inputs([N] * B, [N] * B, H, d, "bf16", 1.0, 9400 + d, backward=True)
    q, k, v, do, cu = _upload(inp, "bf16")
    dense = lambda x: x.reshape(B, N, H, d).permute(0, 2, 1, 3).contiguous()
    packed = lambda x: x.permute(0, 2, 1, 3).reshape(B * N, H, d).contiguous()
    qd, kd, vd, dod = (dense(x) for x in (q, k, v, do))
    od, lsed = fa.fwd(qd, kd, vd, True, scale)
    g_dense = fa.bwd(qd, kd, vd, od, lsed, dod, True, scale)
    o = packed(od)
    lse = lsed.permute(1, 0, 2).reshape(H, B * N).contiguous()
    g_var = fa.bwd_varlen(q, k, v, o, lse, do, cu, cu, N, N, True, scale)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), g_var, g_dense):
        assert torch.equal(a, packed(b)), name
    grads = tuple(g.float().cpu().numpy() for g in g_var)
    ref = varlen_bwd_causal(inp["q"][0], inp["k"][0], inp["v"][0], inp["do"][0], inp["cu_q"], scale)
    _check_seqs(inp, grads, ref, range(B), range(H), f"equal lengths d{d}")


def test_varlen_bwd_rows_outside_the_sequences_are_left_unchanged():
    lens = [10, 15]
    inp = si.make_varlen_inputs(lens + [5], lens + [5], 2, 64, "bf16", 1.0, 9410, backward=True)
    inp["cu_q"] = np.array([0, 10, 25], np.int32)  # rows 25..29 belong to no sequence
    sentinel = si.round_to(np.full((30, 2, 64), 7.0, np.float32), "bf16")[1]
    say("varlen bwd partial cover, cu [0, 10, 25] of 30 rows")
    grads = _run(inp, "bf16", 0.125, init=sentinel)
    for g in grads:
        assert np.all(g[25:] == 7.0)
    ref = varlen_bwd_causal(inp["q"][0], inp["k"][0], inp["v"][0], inp["do"][0], inp["cu_q"], 0.125)
    _check_seqs(inp, grads, ref, range(2), range(2), "partial cover")


def test_varlen_bwd_max_len_above_every_length_and_determinism():
    """A max_len larger than every sequence only adds workgroups that find
    their tiles past the sequence and return; repeated calls are bitwise
    identical."""
    lens = [70, 130]
    inp = si.make_varlen_inputs(lens, lens, 2, 128, "bf16", 1.0, 9420, backward=True)
    say("varlen bwd max_len 256 over lengths [70, 130]")
    g1 = _run(inp, "bf16", 0.088, max_len=256)
    g2 = _run(inp, "bf16", 0.088, max_len=256)
    for a, b in zip(g1, g2):
        assert np.array_equal(a, b)
    ref = varlen_bwd_causal(inp["q"][0], inp["k"][0], inp["v"][0], inp["do"][0], inp["cu_q"], 0.088)
    _check_seqs(inp, g1, ref, range(2), range(2), "max_len 256")


def test_varlen_bwd_prefill_batch_full_size_sampled():
    """The 16-sequence packed prefill batch (lengths uniform in [512, 4096],
    seed 1008, H=16, d=128, bf16) the benchmark times, run in full; sampled
    (sequence, head) pairs against the oracle in full."""
    rng = np.random.default_rng(1008)
    lens = rng.integers(512, 4097, size=16).tolist()
    H, d = 16, 128
    scale = 1 / np.sqrt(d)
    inp = si.make_varlen_inputs(lens, lens, H, d, "bf16", 1.0, 1008, backward=True)
    say(f"varlen bwd prefill batch lengths {lens}")
    grads = _run(inp, "bf16", scale)
    cu = inp["cu_q"]

    def ref(b, h):
        rows = slice(int(cu[b]), int(cu[b + 1]))
        return attention_bwd_head(inp["q"][0][rows, h], inp["k"][0][rows, h], inp["v"][0][rows, h],
                                  inp["do"][0][rows, h], scale, True)

    shortest = int(np.argmin(lens))
    _check_seqs(inp, grads, ref, [shortest], [0, 15], "prefill shortest sequence")
    _check_seqs(inp, grads, ref, [5], [7], "prefill sequence 5")


def test_varlen_bwd_malformed_prefix_sums_stay_in_bounds():
    """Prefix sums that decrease or pass the end are clamped (no access
    leaves the tensors).  Sequence 1 has a negative length (skipped) and
    sequence 2 starts at row 30 and is cut at total = 120 rows, so rows
    30..49 are claimed twice; dQ of rows 0..29 involves sequence 0's rows
    0..29 only and stays exact."""
    lens = [50, 0, 70]
    inp = si.make_varlen_inputs(lens, lens, 2, 128, "bf16", 1.0, 9430, backward=True)
    inp["cu_q"] = np.array([0, 50, 30, 100000], np.int32)
    say(f"varlen bwd malformed cu {inp['cu_q'].tolist()}")
    grads = _run(inp, "bf16", 0.088, max_len=128)
    for g in grads:
        assert np.isfinite(g).all()

    def ref(b, h):
        r = attention_bwd_head(inp["q"][0][0:50, h], inp["k"][0][0:50, h], inp["v"][0][0:50, h],
                               inp["do"][0][0:50, h], 0.088, True)
        return tuple(x[:30] for x in r)

    cu_ok = np.array([0, 30], np.int32)
    _check_seqs({"cu_q": cu_ok}, (grads[0], grads[0], grads[0]),
                lambda b, h: (ref(b, h)[0],) * 3, [0], [0, 1], "sequence 0 dQ rows 0..29")


# ---------------------------------------------------------------- unequal counts and the non-causal mask

def _run_general(inp, dtype, scale, causal, same):
    """fa_fwd_varlen then fa_bwd_varlen with query prefix sums cu_q and key
    prefix sums cu_k (`same`: one tensor for both); returns float dq, dk, dv."""
    import torch
    fa = lib()
    q, k, v, do = (to_device(inp[n][1], dtype) for n in ("q", "k", "v", "do"))
    cq = torch.from_numpy(inp["cu_q"]).cuda()
    ck = cq if same else torch.from_numpy(inp["cu_k"]).cuda()
    mq = max(int(np.diff(inp["cu_q"]).max()), 1)
    mk = max(int(np.diff(inp["cu_k"]).max()), 1)
    o, lse = fa.fwd_varlen(q, k, v, cq, ck, mq, mk, causal, scale)
    dq, dk, dv = fa.bwd_varlen(q, k, v, o, lse, do, cq, ck, mq, mk, causal, scale)
    torch.cuda.synchronize()
    return tuple(g.float().cpu().numpy() for g in (dq, dk, dv))


def _check_general(inp, grads, ref, H, label):
    """Per sequence and head, relative L2 of dQ (query rows) and dK, dV (key rows)."""
    cq, ck = inp["cu_q"], inp["cu_k"]
    worst = {"dq": 0.0, "dk": 0.0, "dv": 0.0}
    for b in range(len(cq) - 1):
        for h in range(H):
            for name, g, r, cu in zip(("dq", "dk", "dv"), grads, ref, (cq, ck, ck)):
                rows = slice(int(cu[b]), int(cu[b + 1]))
                gg, rr = g[rows, h], r[rows, h]
                assert np.isfinite(gg).all(), (label, name, b, h)
                if gg.size == 0:
                    continue
                if np.linalg.norm(rr) < 1e-6:
                    # no query sees these keys (or one key only): exact zeros up to rounding noise
                    assert np.abs(gg).max() <= 1e-5, (label, name, b, h)
                    continue
                worst[name] = max(worst[name], rel_l2(gg, rr))
    say(f"  {label}: rel-L2 {worst}")
    for name, e in worst.items():
        assert e <= BWD_REL_L2, (label, name, e)


UNEQUAL = [
    ([5, 300, 1, 200], [40, 100, 7, 200]),    # fewer and more queries than keys, equal counts
    ([130, 0, 64], [257, 9, 1]),              # an empty query sequence, a single key
    ([1000, 33], [600, 700]),                 # several tiles each side, ragged
]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", range(len(UNEQUAL)))
def test_varlen_bwd_unequal_counts(case, causal, d, dtype):
    """Sequences with their own query and key counts (causal: bottom-right
    aligned, so some queries see no key and some keys no query), against the
    oracle's varlen_bwd."""
    from oracle import varlen_bwd
    lq, lk = UNEQUAL[case]
    H = 2
    seed = 9500 + 17 * case + d + int(causal)
    inp = si.make_varlen_inputs(lq, lk, H, d, dtype, 1.0, seed, backward=True)
    scale = 1.0 / np.sqrt(d)
    say(f"varlen bwd unequal lq={lq} lk={lk} H{H} d{d} {dtype} causal={causal} seed={seed}")
    grads = _run_general(inp, dtype, scale, causal, same=False)
    ref = varlen_bwd(inp["q"][0], inp["k"][0], inp["v"][0], inp["do"][0], inp["cu_q"], inp["cu_k"], scale, causal)
    _check_general(inp, grads, ref, H, f"lq {lq} lk {lk} d{d} {dtype} causal={causal}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("case", range(len(LENGTHS)))
def test_varlen_bwd_non_causal_self_attention(case, d):
    """The non-causal mask over packed self-attention sequences (one
    prefix-sum tensor): every query sees its sequence's keys only."""
    from oracle import varlen_bwd
    lens = LENGTHS[case]
    H = 3
    seed = 9600 + 13 * case + d
    inp = si.make_varlen_inputs(lens, lens, H, d, "bf16", 1.0, seed, backward=True)
    scale = 1.0 / np.sqrt(d)
    say(f"varlen bwd non-causal lens={lens} H{H} d{d} seed={seed}")
    grads = _run_general(inp, "bf16", scale, False, same=True)
    ref = varlen_bwd(inp["q"][0], inp["k"][0], inp["v"][0], inp["do"][0], inp["cu_q"], inp["cu_k"], scale, False)
    _check_general(inp, grads, ref, H, f"non-causal lens {lens} d{d}")


@pytest.mark.parametrize("d", [32, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", range(len(UNEQUAL)))
def test_varlen_bwd_unequal_counts_other_head_dims(case, causal, d):
    """d = 32 (the d = 64 kernels with zero columns) and d = 256 (the wide
    kernels) on sequences with their own query and key counts."""
    from oracle import varlen_bwd
    lq, lk = UNEQUAL[case]
    H = 2
    seed = 9540 + 17 * case + d + int(causal)
    inp = si.make_varlen_inputs(lq, lk, H, d, "bf16", 1.0, seed, backward=True)
    scale = 1.0 / np.sqrt(d)
    say(f"varlen bwd unequal lq={lq} lk={lk} H{H} d{d} causal={causal} seed={seed}")
    grads = _run_general(inp, "bf16", scale, causal, same=False)
    ref = varlen_bwd(inp["q"][0], inp["k"][0], inp["v"][0], inp["do"][0], inp["cu_q"], inp["cu_k"], scale, causal)
    _check_general(inp, grads, ref, H, f"lq {lq} lk {lk} d{d} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", range(len(LENGTHS)))
def test_varlen_bwd_self_attention_d96(case, causal):
    """d = 96 (the d = 128 kernels with zero columns) on packed self-attention
    sequences, the route fa_fwd_varlen takes it on."""
    from oracle import varlen_bwd
    lens = LENGTHS[case]
    H = 2
    seed = 9580 + 13 * case + int(causal)
    inp = si.make_varlen_inputs(lens, lens, H, 96, "bf16", 1.0, seed, backward=True)
    scale = 1.0 / np.sqrt(96)
    say(f"varlen bwd self lens={lens} H{H} d96 causal={causal} seed={seed}")
    grads = _run_general(inp, "bf16", scale, causal, same=True)
    ref = varlen_bwd(inp["q"][0], inp["k"][0], inp["v"][0], inp["do"][0], inp["cu_q"], inp["cu_k"], scale, causal)
    _check_general(inp, grads, ref, H, f"self lens {lens} d96 causal={causal}")
