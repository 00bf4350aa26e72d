"""Parity on the GPU for the general layouts of the square kernels: head
dimensions 32 and 96 (fa_fwd / fa_bwd run them on the d = 64 / 128 kernels
with the columns past d read as zeros and never stored), and caller strides
(fa_fwd_strided / fa_bwd_strided: [B, N, H, d] tensors, views into a packed
QKV tensor, key/value heads shared by several query heads), against the
float64 oracle on the same seeded inputs at the stated bounds (forward O
max-abs <= 1e-2, mean-abs <= 1e-3, LSE max-abs <= 1e-3; backward relative L2
<= 1e-2), and bit for bit against the contiguous entry points where the same
values are laid out differently."""

import numpy as np
import pytest

import seeded_inputs as si
from oracle import attention_bwd, attention_bwd_head, attention_fwd, attention_fwd_head
from parity import BWD_REL_L2, assert_fwd_ok, fwd_errors, lib, rel_l2, say, to_device

pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------- head dimensions 32 and 96

@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [32, 96])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 255, 257, 1000])
def test_head_dims_32_96_fwd_bwd(N, causal, d, dtype):
    import torch
    fa = lib()
    B, H = 1, 2
    seed = 9900 + N + d
    inp = si.make_inputs(B, H, N, d, dtype, 1.0, seed, backward=True)
    scale = 1.0 / np.sqrt(d)
    say(f"d{d} N{N} {dtype} causal={causal} seed={seed}")
    q, k, v, do = (to_device(inp[n][1], dtype) for n in ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v, causal, scale)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal, scale)
    torch.cuda.synchronize()
    o_ref, l_ref = attention_fwd(inp["q"][0], inp["k"][0], inp["v"][0], scale, causal)
    assert_fwd_ok(fwd_errors(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref), dtype,
                  f"fwd d{d} N{N} causal={causal} {dtype}")
    g_ref = attention_bwd(inp["q"][0], inp["k"][0], inp["v"][0], inp["do"][0], scale, causal)
    errs = {}
    for name, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), g_ref):
        gg = g.float().cpu().numpy()
        assert np.isfinite(gg).all(), name
        if np.linalg.norm(r) < 1e-6:  # N = 1: dQ = dK = 0
            assert np.abs(gg).max() <= 1e-5, name
            continue
        errs[name] = rel_l2(gg, r)
    say(f"  bwd d{d} N{N}: rel-L2 {errs}")
    assert all(e <= BWD_REL_L2 for e in errs.values()), errs


@pytest.mark.parametrize("d", [32, 96])
def test_head_dims_32_96_several_tiles_sampled(d):
    """B=2 H=8 N=2048 causal: many query and key tiles per head; sampled
    heads in full against the oracle."""
    import torch
    fa = lib()
    B, H, N = 2, 8, 2048
    inp = si.make_inputs(B, H, N, d, "bf16", 1.0, 9950 + d, backward=True)
    scale = 1.0 / np.sqrt(d)
    q, k, v, do = (to_device(inp[n][1], "bf16") for n in ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v, True, scale)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, True, scale)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (1, 7)):
        o_ref, l_ref = attention_fwd_head(inp["q"][0][b, h], inp["k"][0][b, h], inp["v"][0][b, h], scale, True)
        assert_fwd_ok(fwd_errors(o[b, h].float().cpu().numpy(), lse[b, h].cpu().numpy(), o_ref, l_ref), "bf16",
                      f"d{d} head ({b},{h})")
        g_ref = attention_bwd_head(inp["q"][0][b, h], inp["k"][0][b, h], inp["v"][0][b, h], inp["do"][0][b, h],
                                   scale, True)
        errs = {n: rel_l2(g[b, h].float().cpu().numpy(), r) for n, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), g_ref)}
        say(f"  d{d} head ({b},{h}) bwd rel-L2 {errs}")
        assert all(e <= BWD_REL_L2 for e in errs.values()), errs


# ---------------------------------------------------------------- caller strides

def _bnhd(t):
    """[B, H, N, d] contiguous -> the same values stored [B, N, H, d], viewed [B, H, N, d]."""
    return t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)


@pytest.mark.parametrize("d", [32, 64, 96, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_strided_bnhd_bitwise_equal_contiguous(sign, causal, d):
    """[B, N, H, d] storage for every tensor: the general layout takes the
    same tiles in the same order as the contiguous call, so O, LSE and the
    gradients agree bit for bit; both against the oracle (positive and
    negative scales)."""
    import torch
    fa = lib()
    B, H, N = 2, 3, 700
    scale = sign / np.sqrt(d)
    inp = si.make_inputs(B, H, N, d, "bf16", 1.0, 9700 + d + int(causal), backward=True)
    q, k, v, do = (to_device(inp[n][1], "bf16") for n in ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v, causal, scale)
    g = fa.bwd(q, k, v, o, lse, do, causal, scale)
    qs, ks, vs, dos = (_bnhd(x) for x in (q, k, v, do))
    os_ = _bnhd(torch.empty_like(q))
    lse_s = torch.empty_like(lse)
    fa.fa_fwd_strided(qs, ks, vs, os_, lse_s, scale, causal)
    gs = tuple(_bnhd(torch.empty_like(q)) for _ in range(3))
    ws = torch.empty(4 * B * H * N, dtype=torch.uint8, device="cuda")
    fa.fa_bwd_strided(qs, ks, vs, os_, lse_s, dos, *gs, ws, scale, causal)
    torch.cuda.synchronize()
    assert torch.equal(os_.contiguous(), o) and torch.equal(lse_s, lse), "forward"
    for name, a, b in zip(("dq", "dk", "dv"), gs, g):
        assert torch.equal(a.contiguous(), b), name
    o_ref, l_ref = attention_fwd(inp["q"][0], inp["k"][0], inp["v"][0], scale, causal)
    assert_fwd_ok(fwd_errors(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref), "bf16", f"[B,N,H,d] d{d}")
    g_ref = attention_bwd(inp["q"][0], inp["k"][0], inp["v"][0], inp["do"][0], scale, causal)
    errs = {n: rel_l2(a.float().cpu().numpy(), r) for n, a, r in zip(("dq", "dk", "dv"), g, g_ref)}
    say(f"  [B,N,H,d] d{d} causal={causal} bwd rel-L2 {errs}")
    assert all(e <= BWD_REL_L2 for e in errs.values()), errs


def test_strided_packed_qkv_views():
    """Q, K, V as views into one packed [B, N, 3, H, d] tensor (row stride
    3 H d) and O, dO, the gradients in [B, N, H, d]: no copies, results as
    the oracle's."""
    import torch
    fa = lib()
    B, H, N, d = 2, 4, 513, 128
    scale = 1.0 / np.sqrt(d)
    inp = si.make_inputs(B, H, N, d, "bf16", 1.0, 9800, backward=True)
    q, k, v, do = (to_device(inp[n][1], "bf16") for n in ("q", "k", "v", "do"))
    qkv = torch.stack([x.permute(0, 2, 1, 3) for x in (q, k, v)], dim=2).contiguous()  # [B, N, 3, H, d]
    qv, kv_, vv = (qkv[:, :, i].permute(0, 2, 1, 3) for i in range(3))
    assert qv.stride(2) == 3 * H * d
    o = _bnhd(torch.empty_like(q))
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    fa.fa_fwd_strided(qv, kv_, vv, o, lse, scale, True)
    grads = tuple(_bnhd(torch.empty_like(q)) for _ in range(3))
    ws = torch.empty(4 * B * H * N, dtype=torch.uint8, device="cuda")
    fa.fa_bwd_strided(qv, kv_, vv, o, lse, _bnhd(do), *grads, ws, scale, True)
    torch.cuda.synchronize()
    o_ref, l_ref = attention_fwd(inp["q"][0], inp["k"][0], inp["v"][0], scale, True)
    assert_fwd_ok(fwd_errors(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref), "bf16", "packed qkv")
    g_ref = attention_bwd(inp["q"][0], inp["k"][0], inp["v"][0], inp["do"][0], scale, True)
    errs = {n: rel_l2(a.float().cpu().numpy(), r) for n, a, r in zip(("dq", "dk", "dv"), grads, g_ref)}
    say(f"  packed qkv bwd rel-L2 {errs}")
    assert all(e <= BWD_REL_L2 for e in errs.values()), errs


def test_strided_shared_kv_heads():
    """Key/value heads shared by groups of query heads through a head stride
    of 0 on the inputs (the forward reads them in place): as the oracle with
    the shared head repeated."""
    import torch
    fa = lib()
    B, H, N, d = 2, 6, 600, 64
    scale = 1.0 / np.sqrt(d)
    inp = si.make_inputs(B, H, N, d, "bf16", 1.0, 9810)
    q = to_device(inp["q"][1], "bf16")
    k1, v1 = (to_device(np.ascontiguousarray(inp[n][1][:, :1]), "bf16") for n in ("k", "v"))  # [B, 1, N, d]
    kx, vx = k1.expand(B, H, N, d), v1.expand(B, H, N, d)
    assert kx.stride(1) == 0
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    for causal in (False, True):
        fa.fa_fwd_strided(q, kx, vx, o, lse, scale, causal)
        torch.cuda.synchronize()
        kr = np.repeat(inp["k"][0][:, :1], H, axis=1)
        vr = np.repeat(inp["v"][0][:, :1], H, axis=1)
        o_ref, l_ref = attention_fwd(inp["q"][0], kr, vr, scale, causal)
        assert_fwd_ok(fwd_errors(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref), "bf16",
                      f"shared kv heads causal={causal}")


# ---------------------------------------------------------------- head dimension 256 (forward)

@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 255, 257, 1000])
def test_head_dim_256_fwd(N, causal, dtype):
    """d = 256 (fa_fwd runs the pipelined kernel at one wavefront per
    SIMD, Q and O in AGPRs, 128-row tiles and 32-key tiles) against the
    oracle."""
    import torch
    fa = lib()
    d = 256
    inp = si.make_inputs(1, 2, N, d, dtype, 1.0, 9990 + N)
    scale = 1.0 / np.sqrt(d)
    say(f"d256 N{N} {dtype} causal={causal}")
    q, k, v = (to_device(inp[n][1], dtype) for n in ("q", "k", "v"))
    o, lse = fa.fwd(q, k, v, causal, scale)
    torch.cuda.synchronize()
    o_ref, l_ref = attention_fwd(inp["q"][0], inp["k"][0], inp["v"][0], scale, causal)
    assert_fwd_ok(fwd_errors(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref), dtype,
                  f"fwd d256 N{N} causal={causal} {dtype}")


def test_head_dim_256_several_tiles_strided_and_varlen():
    """d = 256 at B=2 H=4 N=2048 causal (sampled heads in full), the same
    values through fa_fwd_strided in [B, N, H, d] storage (bit for bit), a
    packed variable-length batch with unequal query and key counts and a
    decode step against a cache split into key ranges, each against the
    oracle."""
    import torch
    from oracle import kvcache_fwd, varlen_fwd
    fa = lib()
    B, H, N, d = 2, 4, 2048, 256
    scale = 1.0 / np.sqrt(d)
    inp = si.make_inputs(B, H, N, d, "bf16", 1.0, 9995)
    q, k, v = (to_device(inp[n][1], "bf16") for n in ("q", "k", "v"))
    o, lse = fa.fwd(q, k, v, True, scale)
    os_ = _bnhd(torch.empty_like(q))
    lse_s = torch.empty_like(lse)
    fa.fa_fwd_strided(_bnhd(q), _bnhd(k), _bnhd(v), os_, lse_s, scale, True)
    torch.cuda.synchronize()
    assert torch.equal(os_.contiguous(), o) and torch.equal(lse_s, lse)
    for b, h in ((0, 0), (1, 3)):
        o_ref, l_ref = attention_fwd_head(inp["q"][0][b, h], inp["k"][0][b, h], inp["v"][0][b, h], scale, True)
        assert_fwd_ok(fwd_errors(o[b, h].float().cpu().numpy(), lse[b, h].cpu().numpy(), o_ref, l_ref), "bf16",
                      f"d256 head ({b},{h})")
    # packed, unequal counts
    lq, lk = [40, 300, 1], [100, 250, 9]
    vl = si.make_varlen_inputs(lq, lk, 2, d, "bf16", 1.0, 9996)
    vq, vk, vv = (to_device(vl[n][1], "bf16") for n in ("q", "k", "v"))
    cq, ck = torch.from_numpy(vl["cu_q"]).cuda(), torch.from_numpy(vl["cu_k"]).cuda()
    for causal in (False, True):
        vo, vlse = fa.fwd_varlen(vq, vk, vv, cq, ck, max(lq), max(lk), causal, scale)
        torch.cuda.synchronize()
        o_ref, l_ref = varlen_fwd(vl["q"][0], vl["k"][0], vl["v"][0], vl["cu_q"], vl["cu_k"], scale, causal)
        fin = np.isfinite(l_ref)
        lg = vlse.cpu().numpy()
        assert np.array_equal(np.isneginf(lg), ~fin), "queries that see no key: LSE = -inf"
        err = fwd_errors(vo.float().cpu().numpy(), np.where(fin, lg, 0), o_ref, np.where(fin, l_ref, 0))
        assert_fwd_ok(err, "bf16", f"d256 varlen causal={causal}")
    # packed self-attention (one prefix-sum array): the square kernel in place
    ls = [300, 1, 129, 700]
    sl = si.make_varlen_inputs(ls, ls, 2, d, "bf16", 1.0, 9998)
    sq, sk, sv = (to_device(sl[n][1], "bf16") for n in ("q", "k", "v"))
    cs = torch.from_numpy(sl["cu_q"]).cuda()
    for causal in (False, True):
        so, slse = fa.fwd_varlen(sq, sk, sv, cs, cs, max(ls), max(ls), causal, scale)
        torch.cuda.synchronize()
        o_ref, l_ref = varlen_fwd(sl["q"][0], sl["k"][0], sl["v"][0], sl["cu_q"], sl["cu_k"], scale, causal)
        assert_fwd_ok(fwd_errors(so.float().cpu().numpy(), slse.cpu().numpy(), o_ref, l_ref), "bf16",
                      f"d256 packed self-attention causal={causal}")
    # decode against a cache (key ranges + merge)
    kv = si.make_kvcache_inputs(2, 2, 1, 3000, d, "bf16", 1.0, 9997, 0.5)
    kq, kk, kvv = (to_device(kv[n][1], "bf16") for n in ("q", "k", "v"))
    lens = torch.from_numpy(kv["seqlens"]).cuda()
    ko, klse = fa.fwd_kvcache(kq, kk, kvv, lens, True, scale)
    torch.cuda.synchronize()
    o_ref, l_ref = kvcache_fwd(kv["q"][0], kv["k"][0], kv["v"][0], scale, True, kv["seqlens"])
    assert_fwd_ok(fwd_errors(ko.float().cpu().numpy(), klse.cpu().numpy(), o_ref, l_ref), "bf16", "d256 decode")



# ---------------------------------------------------------------- head dimension 256 (backward)

@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 255, 257, 1000])
def test_head_dim_256_bwd(N, causal, dtype):
    """d = 256 backward (its own kernels: dK/dV with each 32-key block shared
    by two wavefronts that accumulate one half of the columns each, dQ with
    one wavefront per 32 queries; two tiles per workgroup, tile t and
    nt - 1 - t, so odd tile counts (N = 1, 17, 257) run a middle tile once)."""
    import torch
    fa = lib()
    d = 256
    inp = si.make_inputs(1, 2, N, d, dtype, 1.0, 9980 + N, backward=True)
    scale = 1.0 / np.sqrt(d)
    say(f"d256 bwd N{N} {dtype} causal={causal}")
    q, k, v, do = (to_device(inp[n][1], dtype) for n in ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v, causal, scale)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal, scale)
    torch.cuda.synchronize()
    g_ref = attention_bwd(inp["q"][0], inp["k"][0], inp["v"][0], inp["do"][0], scale, causal)
    errs = {}
    for name, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), g_ref):
        gg = g.float().cpu().numpy()
        assert np.isfinite(gg).all(), name
        if np.linalg.norm(r) < 1e-6:  # N = 1: dQ = dK = 0
            assert np.abs(gg).max() <= 1e-5, name
            continue
        errs[name] = rel_l2(gg, r)
    say(f"  bwd d256 N{N}: rel-L2 {errs}")
    assert all(e <= BWD_REL_L2 for e in errs.values()), errs


@pytest.mark.parametrize("causal", [False, True])
def test_head_dim_256_bwd_deterministic_bitwise(causal):
    """The d = 256 backward twice on the same inputs gives bit-identical dQ,
    dK, dV (no atomics; the halves of P and dS that the two wavefronts of a
    key pair exchange through LDS are written and read in a fixed order), at
    B=1 H=3 N=1100: 18 key tiles and 9 query tiles (an odd count, so one
    workgroup runs its middle tile alone)."""
    import torch
    fa = lib()
    B, H, N, d = 1, 3, 1100, 256
    scale = 1.0 / np.sqrt(d)
    inp = si.make_inputs(B, H, N, d, "bf16", 1.0, 9987, backward=True)
    q, k, v, do = (to_device(inp[n][1], "bf16") for n in ("q", "k", "v", "do"))
    say(f"d256 bwd bitwise repeat N{N} causal={causal}")
    o, lse = fa.fwd(q, k, v, causal, scale)
    g1 = [t.clone() for t in fa.bwd(q, k, v, o, lse, do, causal, scale)]
    g2 = fa.bwd(q, k, v, o, lse, do, causal, scale)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), g1, g2):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), name
    ref = attention_bwd_head(inp["q"][0][0, 1], inp["k"][0][0, 1], inp["v"][0][0, 1], inp["do"][0][0, 1],
                             scale, causal)
    errs = {n: rel_l2(g[0, 1].float().cpu().numpy(), r) for n, g, r in zip(("dq", "dk", "dv"), g1, ref)}
    say(f"  head 1 rel-L2 {errs}")
    assert all(e <= BWD_REL_L2 for e in errs.values()), errs


def test_head_dim_256_bwd_strided_and_varlen():
    """d = 256 backward at B=2 H=4 N=1024 causal through fa_bwd_strided in
    [B, N, H, d] storage (bit for bit against fa_bwd on the same values),
    sampled heads against the oracle, and a packed batch with unequal query
    and key counts (causal and not) against the oracle's varlen_bwd."""
    import torch
    from oracle import varlen_bwd
    fa = lib()
    B, H, N, d = 2, 4, 1024, 256
    scale = 1.0 / np.sqrt(d)
    inp = si.make_inputs(B, H, N, d, "bf16", 1.0, 9985, backward=True)
    q, k, v, do = (to_device(inp[n][1], "bf16") for n in ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v, True, scale)
    g = fa.bwd(q, k, v, o, lse, do, True, scale)
    gs = tuple(_bnhd(torch.empty_like(q)) for _ in range(3))
    ws = torch.empty(4 * B * H * N, dtype=torch.uint8, device="cuda")
    fa.fa_bwd_strided(_bnhd(q), _bnhd(k), _bnhd(v), _bnhd(o), lse, _bnhd(do), *gs, ws, scale, True)
    torch.cuda.synchronize()
    for name, a, bb in zip(("dq", "dk", "dv"), gs, g):
        assert torch.equal(a.contiguous(), bb), name
    for b, h in ((0, 1), (1, 3)):
        g_ref = attention_bwd_head(inp["q"][0][b, h], inp["k"][0][b, h], inp["v"][0][b, h], inp["do"][0][b, h],
                                   scale, True)
        errs = {n: rel_l2(x[b, h].float().cpu().numpy(), r) for n, x, r in zip(("dq", "dk", "dv"), g, g_ref)}
        say(f"  d256 head ({b},{h}) bwd rel-L2 {errs}")
        assert all(e <= BWD_REL_L2 for e in errs.values()), errs
    lq, lk = [40, 300, 1, 0], [100, 250, 9, 5]
    vl = si.make_varlen_inputs(lq, lk, 2, d, "bf16", 1.0, 9986, backward=True)
    vq, vk, vv, vdo = (to_device(vl[n][1], "bf16") for n in ("q", "k", "v", "do"))
    cq, ck = torch.from_numpy(vl["cu_q"]).cuda(), torch.from_numpy(vl["cu_k"]).cuda()
    for causal in (False, True):
        vo, vlse = fa.fwd_varlen(vq, vk, vv, cq, ck, max(lq), max(lk), causal, scale)
        grads = fa.bwd_varlen(vq, vk, vv, vo, vlse, vdo, cq, ck, max(lq), max(lk), causal, scale)
        torch.cuda.synchronize()
        ref = varlen_bwd(vl["q"][0], vl["k"][0], vl["v"][0], vl["do"][0], vl["cu_q"], vl["cu_k"], scale, causal)
        for name, gg, rr, cu in zip(("dq", "dk", "dv"), grads, ref, (vl["cu_q"], vl["cu_k"], vl["cu_k"])):
            gg = gg.float().cpu().numpy()
            assert np.isfinite(gg).all(), name
            for bq in range(len(lq)):
                rows = slice(int(cu[bq]), int(cu[bq + 1]))
                for h in range(2):
                    x, y = gg[rows, h], rr[rows, h]
                    if x.size == 0:
                        continue
                    if np.linalg.norm(y) < 1e-6:
                        assert np.abs(x).max() <= 1e-5, (name, bq, h, causal)
                    else:
                        e = rel_l2(x, y)
                        assert e <= BWD_REL_L2, (name, bq, h, causal, e)
        say(f"  d256 varlen unequal counts causal={causal}: ok")
