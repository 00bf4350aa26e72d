"""The C ABI on the host: the library loads, exports every function include/fa.h
declares, and rejects bad arguments with status codes before touching a device.
No compute call is made here (no GPU is needed)."""

import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

FA_OK, FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_HEADDIM, FA_ERR_DTYPE = 0, 1, 2, 3, 4
FA_ERR_ALIGN, FA_ERR_SCALE, FA_ERR_WORKSPACE, FA_ERR_HIP = 5, 6, 7, 8


@pytest.fixture(scope="module")
def lib():
    import exact_io_aware_fa2_amd as fa
    if not os.path.exists(fa.LIB_PATH):
        from exact_io_aware_fa2_amd._build import build_library
        build_library()
    return fa.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(
        ["fa_abi_version", "fa_status_string", "fa_fwd", "fa_bwd_workspace_bytes", "fa_bwd",
         "fa_bwd_prep", "fa_bwd_dkdv", "fa_bwd_dq", "fa_fwd_kvcache_workspace_bytes",
         "fa_fwd_kvcache", "fa_fwd_kvcache_fp8", "fa_probe_mfma_bf16", "fa_fwd_varlen_workspace_bytes",
         "fa_fwd_varlen", "fa_bwd_varlen_workspace_bytes", "fa_bwd_varlen", "fa_bwd_noalloc_max_rows",
         "fa_bwd_noalloc", "fa_fwd_fp8", "fa_fwd_strided", "fa_bwd_strided"])


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert lib.fa_abi_version() == 10


def test_status_strings(lib):
    for code in range(10):
        s = lib.fa_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.fa_status_string(99).decode() == "unknown status"


# fake, 16-byte aligned addresses: never dereferenced, every call below fails validation
P = [0x10000 * (i + 1) for i in range(12)]


def fwd(lib, q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], B=1, H=2, N=64, d=64, scale=0.125,
        causal=0, dtype=2):
    return lib.fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, None)


def bwd(lib, ws=P[10], wsb=1 << 20, B=1, H=2, N=64, d=64, scale=0.125, dtype=2, **kw):
    a = dict(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], do=P[5], dq=P[6], dk=P[7], dv=P[8])
    a.update(kw)
    return lib.fa_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"], a["dv"],
                      ws, wsb, B, H, N, d, scale, 0, dtype, None)


def test_fwd_argument_errors(lib):
    assert fwd(lib, q=None) == FA_ERR_NULL
    assert fwd(lib, lse=None) == FA_ERR_NULL
    assert fwd(lib, B=0) == FA_ERR_SHAPE
    assert fwd(lib, H=-1) == FA_ERR_SHAPE
    assert fwd(lib, N=0) == FA_ERR_SHAPE
    assert fwd(lib, N=(1 << 22) + 1) == FA_ERR_SHAPE
    assert fwd(lib, B=1 << 20, H=1 << 12) == FA_ERR_SHAPE
    assert fwd(lib, d=80) == FA_ERR_HEADDIM
    assert fwd(lib, d=512) == FA_ERR_HEADDIM
    assert fwd(lib, d=256, dtype=0) == FA_ERR_HEADDIM  # float32: d = 64 or 128
    assert fwd(lib, d=256, N=(1 << 22) - 32) == FA_ERR_SHAPE  # d = 256 rows past 32-bit offsets
    assert fwd(lib, dtype=3) == FA_ERR_DTYPE
    assert fwd(lib, dtype=-1) == FA_ERR_DTYPE
    assert fwd(lib, v=P[2] + 8) == FA_ERR_ALIGN
    assert fwd(lib, lse=P[4] + 4) == FA_ERR_ALIGN
    assert fwd(lib, scale=float("nan")) == FA_ERR_SCALE
    assert fwd(lib, scale=math.inf) == FA_ERR_SCALE
    assert fwd(lib, scale=-math.inf) == FA_ERR_SCALE
    # finite, but |scale| * log2(e) overflows float32 (a negative scale is
    # taken: softmax of scale * QK^T is defined for any finite scale)
    assert fwd(lib, scale=3.0e38) == FA_ERR_SCALE
    assert fwd(lib, scale=-3.0e38) == FA_ERR_SCALE
    assert bwd(lib, scale=3.0e38) == FA_ERR_SCALE
    assert bwd(lib, scale=-3.0e38) == FA_ERR_SCALE


def test_bwd_argument_errors(lib):
    assert bwd(lib, do=None) == FA_ERR_NULL
    assert bwd(lib, dv=None) == FA_ERR_NULL
    assert bwd(lib, N=0) == FA_ERR_SHAPE
    assert bwd(lib, d=80) == FA_ERR_HEADDIM
    assert bwd(lib, dtype=0) == FA_ERR_DTYPE  # the backward takes 16-bit inputs only
    assert bwd(lib, dq=P[6] + 2) == FA_ERR_ALIGN
    assert bwd(lib, scale=float("-inf")) == FA_ERR_SCALE
    assert bwd(lib, ws=None) == FA_ERR_WORKSPACE
    assert bwd(lib, wsb=4 * 2 * 64 - 1) == FA_ERR_WORKSPACE
    assert bwd(lib, ws=P[10] + 4) == FA_ERR_ALIGN


def noalloc(lib, B=1, H=2, N=64, d=64, scale=0.125, dtype=2, **kw):
    a = dict(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], do=P[5], dq=P[6], dk=P[7], dv=P[8])
    a.update(kw)
    return lib.fa_bwd_noalloc(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"], a["dv"],
                              B, H, N, d, scale, 1, dtype, None)


def test_noalloc_argument_errors(lib):
    """fa_bwd_noalloc checks like fa_bwd and refuses sizes beyond its static
    scratch (one float per query row) before any device call."""
    FA_ERR_SCRATCH = 9
    rows = lib.fa_bwd_noalloc_max_rows()
    assert rows == (16 << 20) // 4
    assert noalloc(lib, dv=None) == FA_ERR_NULL
    assert noalloc(lib, N=0) == FA_ERR_SHAPE
    assert noalloc(lib, d=80) == FA_ERR_HEADDIM
    assert noalloc(lib, dtype=0) == FA_ERR_DTYPE
    assert noalloc(lib, lse=P[4] + 4) == FA_ERR_ALIGN
    assert noalloc(lib, scale=math.nan) == FA_ERR_SCALE
    # one row more than the scratch holds (B * H * N = rows + 64)
    assert noalloc(lib, B=rows // 64 + 1, H=1, N=64) == FA_ERR_SCRATCH
    assert noalloc(lib, B=1, H=64, N=rows // 64 + 1) == FA_ERR_SCRATCH


def f8(lib, q=P[0], k=P[1], v=P[2], qs=P[8], ks=P[9], vs=P[10], g=1, o=P[3], lse=P[4], B=1, H=2, N=300, d=128,
       scale=0.088, causal=1, dtype=2):
    return lib.fa_fwd_fp8(q, k, v, qs, ks, vs, g, o, lse, B, H, N, d, scale, causal, dtype, None)


def test_fp8_argument_errors(lib):
    for name in ("q", "k", "v", "qs", "ks", "vs", "o", "lse"):
        assert f8(lib, **{name: None}) == FA_ERR_NULL, name
    assert f8(lib, N=0) == FA_ERR_SHAPE
    assert f8(lib, d=64) == FA_ERR_HEADDIM
    assert f8(lib, d=96) == FA_ERR_HEADDIM
    assert f8(lib, dtype=0) == FA_ERR_DTYPE  # the output is 16-bit
    assert f8(lib, g=2) == FA_ERR_DTYPE      # unknown scale granularity
    assert f8(lib, k=P[1] + 8) == FA_ERR_ALIGN
    assert f8(lib, qs=P[8] + 2) == FA_ERR_ALIGN
    assert f8(lib, scale=-3.0e38) == FA_ERR_SCALE
    assert f8(lib, scale=math.inf) == FA_ERR_SCALE


def test_stage_argument_errors(lib):
    a = dict(B=1, H=2, N=64, d=64)
    ws, wsb = P[10], 1 << 20
    assert lib.fa_bwd_prep(None, P[1], ws, wsb, 1, 2, 64, 64, 2, None) == FA_ERR_NULL
    assert lib.fa_bwd_prep(P[0], P[1], ws, 8, 1, 2, 64, 64, 2, None) == FA_ERR_WORKSPACE
    assert lib.fa_bwd_prep(P[0], P[1], ws, wsb, 1, 2, 64, 80, 2, None) == FA_ERR_HEADDIM
    assert lib.fa_bwd_dkdv(P[0], P[1], P[2], P[3], P[4], ws, wsb, P[5], None,
                           1, 2, 64, 64, 0.1, 1, 2, None) == FA_ERR_NULL
    assert lib.fa_bwd_dkdv(P[0], P[1], P[2], P[3], P[4], ws, wsb, P[5], P[6],
                           1, 2, 64, 64, 0.1, 1, 0, None) == FA_ERR_DTYPE
    assert lib.fa_bwd_dq(P[0], P[1], P[2], P[3], P[4], ws, wsb, P[5] + 2,
                         1, 2, 64, 64, 0.1, 1, 2, None) == FA_ERR_ALIGN
    assert lib.fa_bwd_dq(P[0], P[1], P[2], P[3], P[4], ws, wsb, P[5],
                         1, 2, 64, 64, -math.inf, 1, 2, None) == FA_ERR_SCALE
    assert a


def test_workspace_bytes(lib):
    assert lib.fa_bwd_workspace_bytes(2, 3, 100, 64, 2) == 4 * 2 * 3 * 100
    assert lib.fa_bwd_workspace_bytes(1, 1, 1, 128, 1) == 4
    assert lib.fa_bwd_workspace_bytes(1, 1, 1, 80, 2) == 0
    assert lib.fa_bwd_workspace_bytes(0, 1, 1, 64, 2) == 0
    assert lib.fa_bwd_workspace_bytes(1, 1, 8, 64, 0) == 0


def test_binding_rejects_host_tensors_and_bad_shapes(lib):
    torch = pytest.importorskip("torch")
    import exact_io_aware_fa2_amd as fa
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.fwd(q, q, q)
    with pytest.raises(TypeError):
        fa.dtype_code(torch.zeros(1, dtype=torch.int32))


def test_binding_checks_backward_tensors_before_the_call(lib):
    """Wrong shapes, dtypes or sizes of lse, gradients and the workspace are
    named by the wrappers (before any pointer reaches the library)."""
    torch = pytest.importorskip("torch")
    import exact_io_aware_fa2_amd as fa
    B, H, N, d = 1, 2, 16, 64
    t = lambda *s, dt=torch.bfloat16: torch.zeros(*s, dtype=dt)  # noqa: E731
    q = t(B, H, N, d)
    lse = t(B, H, N, dt=torch.float32)
    ws = torch.zeros(4 * B * H * N, dtype=torch.uint8)
    good = dict(q=q, k=q, v=q, o=q, lse=lse, dout=q, dq=q, dk=q, dv=q, workspace=ws)

    def call(**kw):
        a = dict(good, **kw)
        fa.fa_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dout"], a["dq"], a["dk"], a["dv"],
                  a["workspace"], 0.125, True)

    with pytest.raises(ValueError, match="lse"):
        call(lse=t(B, H, N))  # bf16, not float32
    with pytest.raises(ValueError, match="lse"):
        call(lse=t(B, H, N + 1, dt=torch.float32))
    with pytest.raises(ValueError, match="share shape"):
        call(dv=t(B, H, N, d + 64))
    with pytest.raises(ValueError, match="share shape"):
        call(dout=t(B, H, N, d, dt=torch.float16))
    with pytest.raises(ValueError, match="workspace"):
        call(workspace=torch.zeros(4 * B * H * N - 1, dtype=torch.uint8))
    # the stage wrappers check the same
    with pytest.raises(ValueError, match="share shape"):
        fa.fa_bwd_prep(q, t(B, H, N - 1, d), ws)
    with pytest.raises(ValueError, match="workspace"):
        fa.fa_bwd_prep(q, q, torch.zeros(8, dtype=torch.uint8))
    with pytest.raises(ValueError, match="lse"):
        fa.fa_bwd_dkdv(q, q, q, q, t(B, H, N), ws, q, q, 0.125, True)
    with pytest.raises(ValueError, match="share shape"):
        fa.fa_bwd_dkdv(q, q, q, q, lse, ws, t(B, H, N, 32), q, 0.125, True)
    with pytest.raises(ValueError, match="lse"):
        fa.fa_bwd_dq(q, q, q, q, t(B, 1, N, dt=torch.float32), ws, q, 0.125, True)
    with pytest.raises(ValueError, match="share shape"):
        fa.fa_bwd_dq(q, t(B, H, N, d, dt=torch.float16), q, q, lse, ws, q, 0.125, True)
    # right shapes on the host: refused as host tensors
    with pytest.raises(ValueError, match="GPU"):
        call()


def kv(lib, q=P[0], k=P[1], v=P[2], lens=None, o=P[3], lse=P[4], ws=P[10], wsb=1 << 30, B=2, H=4,
       Nq=1, Nk=4096, d=128, scale=0.088, causal=1, dtype=2):
    return lib.fa_fwd_kvcache(q, k, v, lens, o, lse, ws, wsb, B, H, Nq, Nk, d, scale, causal, dtype, None)


def test_kvcache_argument_errors(lib):
    for name in ("q", "k", "v", "o", "lse"):
        assert kv(lib, **{name: None}) == FA_ERR_NULL, name
    assert kv(lib, Nq=0) == FA_ERR_SHAPE
    assert kv(lib, Nk=0) == FA_ERR_SHAPE
    assert kv(lib, B=0) == FA_ERR_SHAPE
    assert kv(lib, Nk=(1 << 22) + 1) == FA_ERR_SHAPE
    assert kv(lib, Nq=(1 << 22) + 1) == FA_ERR_SHAPE
    assert kv(lib, d=96) == FA_ERR_HEADDIM
    assert kv(lib, dtype=0) == FA_ERR_DTYPE
    assert kv(lib, dtype=7) == FA_ERR_DTYPE
    assert kv(lib, q=P[0] + 8) == FA_ERR_ALIGN
    assert kv(lib, lens=P[9] + 2) == FA_ERR_ALIGN
    assert kv(lib, scale=-3.0e38) == FA_ERR_SCALE
    assert kv(lib, scale=math.nan) == FA_ERR_SCALE
    assert kv(lib, ws=None) == FA_ERR_WORKSPACE
    need = lib.fa_fwd_kvcache_workspace_bytes(2, 4, 1, 4096, 128, 2)
    assert need > 0
    assert kv(lib, wsb=need - 1) == FA_ERR_WORKSPACE
    assert kv(lib, ws=P[10] + 4) == FA_ERR_ALIGN


def test_kvcache_workspace_bytes(lib):
    ws = lib.fa_fwd_kvcache_workspace_bytes
    # a single decode query over a 4096-row cache at B*H = 8 is split into 64 ranges of 64 keys:
    # per range, head and query 128 floats of partial O and 2 log-sum-exps
    assert ws(2, 4, 1, 4096, 128, 2) == 64 * 8 * 1 * 130 * 4
    # B*H = 256 over 32768 keys: ranges double until at most 8192 wavefronts at d = 128
    # (1024 keys, 32 ranges), 16384 at d = 64 (512 keys, 64 ranges)
    assert ws(8, 32, 1, 32768, 128, 1) == 32 * 256 * 130 * 4
    assert ws(8, 32, 1, 32768, 64, 1) == 64 * 256 * 66 * 4
    # one range covers the cache: no workspace (O and LSE are written directly)
    # a 4096-query chunk of one head: 128 query blocks x 64 ranges of 64 keys = 8192 wavefronts
    assert ws(1, 1, 4096, 4096, 64, 2) == 64 * 4096 * 66 * 4
    assert ws(64, 64, 2048, 2048, 128, 2) == 0
    assert ws(2, 4, 1, 4096, 128, 0) == 0  # fp32 is not taken
    assert ws(2, 4, 1, 4096, 32, 2) == 64 * 8 * 34 * 4  # d = 32 is taken by the split-key path
    assert ws(0, 4, 1, 4096, 128, 2) == 0
    assert ws(2, 4, 1, 4096, 96, 2) == 0


def kv8(lib, q=P[0], k=P[1], v=P[2], ks=0.01, vs=0.02, lens=None, o=P[3], lse=P[4], ws=P[10], wsb=1 << 30,
        B=2, H=4, Nq=1, Nk=4096, d=128, scale=0.088, causal=1, dtype=2):
    return lib.fa_fwd_kvcache_fp8(q, k, v, ks, vs, lens, o, lse, ws, wsb, B, H, Nq, Nk, d, scale, causal,
                                  dtype, None)


def test_kvcache_fp8_argument_errors(lib):
    for name in ("q", "k", "v", "o", "lse"):
        assert kv8(lib, **{name: None}) == FA_ERR_NULL, name
    assert kv8(lib, Nk=0) == FA_ERR_SHAPE
    assert kv8(lib, d=96) == FA_ERR_HEADDIM
    assert kv8(lib, d=256) == FA_ERR_HEADDIM
    assert kv(lib, d=96) == FA_ERR_HEADDIM
    assert kv8(lib, dtype=0) == FA_ERR_DTYPE
    assert kv8(lib, k=P[1] + 4) == FA_ERR_ALIGN
    for bad in (0.0, -1.0, math.inf, math.nan):
        assert kv8(lib, ks=bad) == FA_ERR_SCALE
        assert kv8(lib, vs=bad) == FA_ERR_SCALE
    assert kv8(lib, scale=-math.inf) == FA_ERR_SCALE
    # each finite, the exponent factor |scale| * k_scale * log2(e) is not
    assert kv8(lib, scale=1.0e20, ks=1.0e20) == FA_ERR_SCALE
    assert kv8(lib, scale=-1.0e20, ks=1.0e20) == FA_ERR_SCALE
    assert kv(lib, scale=3.0e38) == FA_ERR_SCALE
    assert kv8(lib, ws=None) == FA_ERR_WORKSPACE


def test_probe_argument_errors(lib):
    lib.fa_probe_mfma_bf16.restype = ctypes.c_int64
    lib.fa_probe_mfma_bf16.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
    assert lib.fa_probe_mfma_bf16(0, 10, None) == -FA_ERR_SHAPE
    assert lib.fa_probe_mfma_bf16(10, 0, None) == -FA_ERR_SHAPE
    assert lib.fa_probe_mfma_bf16(1 << 24, 10, None) == -FA_ERR_SHAPE
    # the FLOP count would leave int64
    assert lib.fa_probe_mfma_bf16((1 << 24) - 1, (1 << 31) - 1, None) == -FA_ERR_SHAPE


def vl(lib, q=P[0], k=P[1], v=P[2], cq=P[8], ck=P[9], o=P[3], lse=P[4], ws=P[10], wsb=1 << 30, B=3, H=4,
       tq=300, tk=500, mq=128, mk=256, d=128, scale=0.088, causal=1, dtype=2):
    return lib.fa_fwd_varlen(q, k, v, cq, ck, o, lse, ws, wsb, B, H, tq, tk, mq, mk, d, scale, causal, dtype, None)


def test_varlen_argument_errors(lib):
    for name in ("q", "k", "v", "cq", "ck", "o", "lse"):
        assert vl(lib, **{name: None}) == FA_ERR_NULL, name
    assert vl(lib, B=0) == FA_ERR_SHAPE
    assert vl(lib, tq=0) == FA_ERR_SHAPE
    assert vl(lib, tk=0) == FA_ERR_SHAPE
    assert vl(lib, mq=0) == FA_ERR_SHAPE
    assert vl(lib, mk=(1 << 22) + 1) == FA_ERR_SHAPE
    assert vl(lib, H=64, mk=1 << 17) == FA_ERR_SHAPE  # 2^17 * 64 * 128 * 2 = 2^31 bytes
    assert vl(lib, d=80) == FA_ERR_HEADDIM
    assert vl(lib, dtype=0) == FA_ERR_DTYPE
    assert vl(lib, cq=P[8] + 2) == FA_ERR_ALIGN
    assert vl(lib, o=P[3] + 8) == FA_ERR_ALIGN
    assert vl(lib, scale=-math.nan) == FA_ERR_SCALE
    assert vl(lib, scale=-3.0e38) == FA_ERR_SCALE
    need = lib.fa_fwd_varlen_workspace_bytes(3, 4, 128, 256, 128, 2)
    assert need == lib.fa_fwd_kvcache_workspace_bytes(3, 4, 128, 256, 128, 2) > 0
    assert vl(lib, ws=None) == FA_ERR_WORKSPACE
    assert vl(lib, wsb=need - 1) == FA_ERR_WORKSPACE


def bvl(lib, ptrs=None, cq=P[10], ck=P[10], ws=P[11], wsb=1 << 40, B=3, H=4, tq=300, tk=300, mq=128, mk=128, d=128,
        scale=0.088, causal=1, dtype=2):
    q, k, v, o, lse, do, dq, dk, dv = ptrs if ptrs is not None else P[:9]
    return lib.fa_bwd_varlen(q, k, v, o, lse, do, cq, ck, dq, dk, dv, ws, wsb, B, H, tq, tk, mq, mk, d, scale, causal,
                             dtype, None)


def test_varlen_bwd_argument_errors(lib):
    # every case is rejected before any launch (the pointers are never touched)
    for i in range(9):
        ptrs = list(P[:9])
        ptrs[i] = None
        assert bvl(lib, ptrs) == FA_ERR_NULL, i
    assert bvl(lib, cq=None) == FA_ERR_NULL
    assert bvl(lib, ck=None) == FA_ERR_NULL
    assert bvl(lib, B=0) == FA_ERR_SHAPE
    assert bvl(lib, tq=0) == FA_ERR_SHAPE
    assert bvl(lib, tk=0) == FA_ERR_SHAPE
    assert bvl(lib, tq=1 << 31) == FA_ERR_SHAPE
    assert bvl(lib, mq=0) == FA_ERR_SHAPE
    assert bvl(lib, mk=(1 << 22) + 1) == FA_ERR_SHAPE
    assert bvl(lib, d=80) == FA_ERR_HEADDIM
    assert bvl(lib, d=512) == FA_ERR_HEADDIM
    assert bvl(lib, dtype=0) == FA_ERR_DTYPE
    for i in range(9):
        ptrs = list(P[:9])
        ptrs[i] += 8
        assert bvl(lib, ptrs) == FA_ERR_ALIGN, i
    assert bvl(lib, cq=P[10] + 2) == FA_ERR_ALIGN
    assert bvl(lib, ck=P[9] + 2) == FA_ERR_ALIGN
    assert bvl(lib, scale=float("nan")) == FA_ERR_SCALE
    assert bvl(lib, tq=(1 << 29)) == FA_ERR_SHAPE  # total * H = 2^31
    assert bvl(lib, H=64, mq=(1 << 17) - 512) == FA_ERR_SHAPE  # (2^17) * 64 * 128 * 2 = 2^31 bytes
    assert bvl(lib, H=64, mk=(1 << 17) - 512) == FA_ERR_SHAPE
    need = lib.fa_bwd_varlen_workspace_bytes(3, 4, 300, 128, 128, 2)
    assert need == 4 * 300 * 4
    assert lib.fa_bwd_varlen_workspace_bytes(1, 1, 3, 3, 64, 0) == 0
    assert lib.fa_bwd_varlen_workspace_bytes(1, 1, 3, 3, 80, 2) == 0
    assert lib.fa_bwd_varlen_workspace_bytes(1, 1, 0, 3, 64, 2) == 0
    assert lib.fa_bwd_varlen_workspace_bytes(1, 1, 3, 3, 32, 2) == 4 * 3
    assert bvl(lib, ws=None) == FA_ERR_WORKSPACE
    assert bvl(lib, wsb=need - 1) == FA_ERR_WORKSPACE
    assert bvl(lib, ws=P[11] + 4, wsb=need) == FA_ERR_ALIGN


def _st(n, d=64, bad=None):
    """Strides of n contiguous [1, 2, 64, d] tensors, one entry replaced."""
    st = [2 * 64 * d, 64 * d, d] * n
    if bad is not None:
        st[bad[0]] = bad[1]
    return (ctypes.c_int64 * len(st))(*st)


def test_strided_argument_errors(lib):
    fs = lambda st, d=64, dtype=2, **kw: lib.fa_fwd_strided(  # noqa: E731
        kw.get("q", P[0]), P[1], P[2], P[3], P[4], st, 1, 2, 64, d, 0.125, 1, dtype, None)
    assert fs(None) == FA_ERR_NULL
    assert fs(_st(4), q=None) == FA_ERR_NULL
    assert fs(_st(4), d=80) == FA_ERR_HEADDIM
    assert fs(_st(4), dtype=0) == FA_ERR_DTYPE  # 16-bit only
    assert fs(_st(4, bad=(1, -64))) == FA_ERR_SHAPE    # negative head stride
    assert fs(_st(4, bad=(5, 60))) == FA_ERR_ALIGN     # k's row stride: rows not 16-byte aligned
    assert fs(_st(4, bad=(11, 32))) == FA_ERR_SHAPE    # o's rows overlap (row stride < d)
    assert fs(_st(4, bad=(2, 1 << 24))) == FA_ERR_SHAPE  # q rows past 32-bit offsets
    bs = lambda st, **kw: lib.fa_bwd_strided(  # noqa: E731
        *P[:9], P[10], 1 << 20, st, 1, 2, 64, kw.get("d", 64), 0.125, 1, 2, None)
    assert bs(None) == FA_ERR_NULL
    assert bs(_st(8, bad=(23, 8))) == FA_ERR_SHAPE     # dv rows overlap
    assert bs(_st(8, bad=(14, 4))) == FA_ERR_ALIGN     # dout's row stride
    assert bs(_st(8), d=80) == FA_ERR_HEADDIM


def test_head_dims_taken_by_fwd_and_bwd(lib):
    """d = 32 and 96 are taken by the 16-bit forward and backward (checked
    here by the workspace size function, which makes no device call), not by
    the float32 forward; d = 256 by both 16-bit passes; 80, 16 and 512 by
    neither."""
    for d in (32, 64, 96, 128, 256):
        assert lib.fa_bwd_workspace_bytes(1, 2, 10, d, 2) == 4 * 20, d
    for d in (80, 512, 16):
        assert lib.fa_bwd_workspace_bytes(1, 2, 10, d, 2) == 0, d
        assert bwd(lib, d=d) == FA_ERR_HEADDIM
    assert bwd(lib, d=256, N=(1 << 22) - 32) == FA_ERR_SHAPE  # d = 256 rows past 32-bit offsets
    for d in (80, 16):
        assert fwd(lib, d=d) == FA_ERR_HEADDIM
    assert fwd(lib, d=96, dtype=0) == FA_ERR_HEADDIM
    assert fwd(lib, d=32, dtype=0) == FA_ERR_HEADDIM
    assert kv8(lib, d=256) == FA_ERR_HEADDIM  # the 8-bit cache: d = 32, 64, 128


def test_varlen_self_attention_route_checks_arguments_first(lib):
    # one prefix-sum array for queries and keys selects the square kernels,
    # but only after every argument check (each case below returns before any launch)
    same = dict(cq=P[8], ck=P[8], tq=500, tk=500, mq=256, mk=256)
    assert vl(lib, **same, d=80) == FA_ERR_HEADDIM
    assert vl(lib, **same, dtype=0) == FA_ERR_DTYPE
    assert vl(lib, **same, o=P[3] + 8) == FA_ERR_ALIGN
    assert vl(lib, **same, scale=-math.inf) == FA_ERR_SCALE
    assert vl(lib, **same, q=None) == FA_ERR_NULL
    assert vl(lib, **dict(same, tq=0)) == FA_ERR_SHAPE
