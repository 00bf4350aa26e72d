"""Parity of the persistent grids.  The d = 64 forward (fwd16_pp_kernel) and
the dK/dV and dQ kernels launch one workgroup per resident slot, each walking
its share of the tiles, when the tiles outnumber the slots and the heads split
evenly over the 8 XCDs in whole rounds (the shapes below: more tiles than
the 256 compute units hold, ragged last tiles).  Every output starts as NaN, so a tile that no
workgroup takes shows as NaN; sampled heads (the first, and the last, which
another XCD's workgroups serve) are compared with the float64 oracle at the
usual bounds."""

import numpy as np
import pytest

import seeded_inputs as si
from oracle import attention_bwd_head, attention_fwd_head, varlen_fwd
from parity import BWD_REL_L2, assert_fwd_ok, fwd_errors, lib, rel_l2, say, to_device

pytestmark = pytest.mark.gpu


def _nan_like(t):
    import torch
    return torch.full_like(t, float("nan"))


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_d64_more_tiles_than_slots(causal, dtype):
    import torch
    fa = lib()
    B, H, N, d = 2, 8, 8100, 64  # 16 heads x 32 query tiles of 256 rows, the last ragged
    scale = 1.0 / np.sqrt(d)
    inp = si.make_inputs(B, H, N, d, dtype, 1.0, 9900 + int(causal))
    say(f"persistent fwd B{B} H{H} N{N} d{d} {dtype} causal={causal}")
    q, k, v = (to_device(inp[n][1], dtype) for n in ("q", "k", "v"))
    o = _nan_like(q)
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device="cuda")
    fa.fa_fwd(q, k, v, o, lse, scale, causal)
    torch.cuda.synchronize()
    og, lg = o.float().cpu().numpy(), lse.cpu().numpy()
    assert np.isfinite(og).all() and np.isfinite(lg).all()
    for (b, h) in [(0, 0), (1, 7)]:
        o_ref, l_ref = attention_fwd_head(inp["q"][0][b, h], inp["k"][0][b, h], inp["v"][0][b, h], scale, causal)
        assert_fwd_ok(fwd_errors(og[b, h], lg[b, h], o_ref, l_ref), dtype, f"head ({b},{h})")


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_self_d64_more_tiles_than_slots(causal):
    import torch
    fa = lib()
    lens, H, d = [3000, 4096, 17, 2600], 8, 64  # 32 heads x 16 query tiles, many past short sequences
    scale = 1.0 / np.sqrt(d)
    inp = si.make_varlen_inputs(lens, lens, H, d, "bf16", 1.0, 9910 + int(causal))
    say(f"persistent varlen self lens={lens} H{H} d{d} causal={causal}")
    q, k, v = (to_device(inp[n][1], "bf16") for n in ("q", "k", "v"))
    cu = torch.from_numpy(inp["cu_q"]).cuda()
    o = _nan_like(q)
    lse = torch.full((H, q.shape[0]), float("nan"), dtype=torch.float32, device="cuda")
    fa.fa_fwd_varlen(q, k, v, cu, cu, o, lse, None, max(lens), max(lens), scale, causal)
    torch.cuda.synchronize()
    og, lg = o.float().cpu().numpy(), lse.cpu().numpy()
    assert np.isfinite(og).all() and np.isfinite(lg).all()
    sel = [0, 7]
    o_ref, l_ref = varlen_fwd(inp["q"][0][:, sel], inp["k"][0][:, sel], inp["v"][0][:, sel], inp["cu_q"],
                              inp["cu_k"], scale, causal)
    assert_fwd_ok(fwd_errors(og[:, sel], lg[sel], o_ref, l_ref), "bf16", "heads 0 and 7")


@pytest.mark.parametrize("d", [64, 128])
def test_backward_more_tiles_than_slots(d):
    import torch
    fa = lib()
    # 32 heads x 32 tiles of 128 keys (dK/dV) or 128 query rows (dQ), the last ragged:
    # more than the resident slots (512 at d = 64, 256 at d = 128)
    B, H, N = 4, 8, 4000
    scale = 1.0 / np.sqrt(d)
    inp = si.make_inputs(B, H, N, d, "bf16", 1.0, 9920 + d, backward=True)
    say(f"persistent backward B{B} H{H} N{N} d{d} causal")
    q, k, v = (to_device(inp[n][1], "bf16") for n in ("q", "k", "v"))
    do = to_device(inp["do"][1], "bf16")
    o, lse = fa.fwd(q, k, v, True, scale)
    dq, dk, dv = _nan_like(q), _nan_like(k), _nan_like(v)
    ws = torch.empty(max(fa.fa_bwd_workspace_bytes(B, H, N, d, fa.dtype_code(q)), 16), dtype=torch.uint8,
                     device="cuda")
    fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, ws, scale, True)
    torch.cuda.synchronize()
    grads = [t.float().cpu().numpy() for t in (dq, dk, dv)]
    for g in grads:
        assert np.isfinite(g).all()
    for (b, h) in [(0, 0), (3, 7)]:
        ref = attention_bwd_head(inp["q"][0][b, h], inp["k"][0][b, h], inp["v"][0][b, h], inp["do"][0][b, h],
                                 scale, True)
        errs = [rel_l2(g[b, h], r) for g, r in zip(grads, ref)]
        say(f"  head ({b},{h}): rel-L2 dQ {errs[0]:.2e} dK {errs[1]:.2e} dV {errs[2]:.2e}")
        assert max(errs) <= BWD_REL_L2


@pytest.mark.parametrize("d", [64, 128])
def test_persistent_runs_are_bitwise_repeatable(d):
    """Two calls on a shape that takes the persistent grids (the d = 64
    forward, both backward kernels) give the same bits."""
    import torch
    fa = lib()
    B, H, N = 4, 8, 4000
    inp = si.make_inputs(B, H, N, d, "bf16", 1.0, 9930 + d, backward=True)
    q, k, v, do = (to_device(inp[n][1], "bf16") for n in ("q", "k", "v", "do"))
    o1, l1 = fa.fwd(q, k, v, True)
    o2, l2 = fa.fwd(q, k, v, True)
    g1 = fa.bwd(q, k, v, o1, l1, do, True)
    g2 = fa.bwd(q, k, v, o1, l1, do, True)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    for x, y in zip(g1, g2):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
