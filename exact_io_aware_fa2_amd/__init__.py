"""Python binding of libfa_mi355x.so, the gfx950 exact-attention library.

Argument marshalling only: every step of attention runs in the library's HIP
kernels.  PyTorch provides device memory and the current HIP stream.  If the
shared library is missing this module raises instead of computing anything
another way.

Raw entry points (same names and argument order as include/fa.h, tensors in
place of pointers):
    fa_fwd(q, k, v, o, lse, scale, causal)
    fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, scale, causal)
    fa_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, scale, causal)  (no workspace)
    fa_bwd_workspace_bytes(B, H, N, d, dtype)
    fa_bwd_prep(o, dout, workspace); fa_bwd_dkdv(...); fa_bwd_dq(...)  (fa_bwd's stages)
    fa_fwd_kvcache(q, k_cache, v_cache, seqlens_k, o, lse, workspace, scale, causal)
    fa_fwd_kvcache_workspace_bytes(B, H, Nq, Nk, d, dtype)
    fa_fwd_kvcache_fp8(q, k_cache, v_cache, k_scale, v_scale, seqlens_k, o, lse, workspace, scale, causal)
    fa_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, o, lse, workspace, max_q, max_k, scale, causal)
    fa_fwd_fp8(q8, k8, v8, q_scale, k_scale, v_scale, granularity, o, lse, scale, causal)
    fa_bwd_varlen(q, k, v, o, lse, dout, cu_seqlens_q, cu_seqlens_k, dq, dk, dv, workspace, max_q, max_k,
                  scale, causal)
    fa_fwd_strided(q, k, v, o, lse, scale, causal)   ([B, H, N, d] views with any strides)
    fa_bwd_strided(q, k, v, o, lse, dout, dq, dk, dv, workspace, scale, causal)
Conveniences that allocate their outputs with torch:
    fwd(q, k, v, causal=False, scale=None) -> (o, lse)
    bwd(q, k, v, o, lse, dout, causal=False, scale=None) -> (dq, dk, dv)
    fwd_kvcache(q, k_cache, v_cache, seqlens_k=None, causal=True, scale=None) -> (o, lse)
    fwd_kvcache_fp8(q, k8, v8, k_scale, v_scale, seqlens_k=None, causal=True, scale=None) -> (o, lse)
    fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_q, max_k, causal=False, scale=None) -> (o, lse)
    fwd_fp8(q8, k8, v8, q_scale, k_scale, v_scale, granularity="block", causal=False, scale=None) -> (o, lse)
    bwd_varlen(q, k, v, o, lse, dout, cu_seqlens_q, cu_seqlens_k=None, max_q=None, max_k=None, causal=True)
    FlashAttention (torch.autograd.Function) and attention(q, k, v, causal, scale)
"""

from __future__ import annotations

import ctypes
import math
import os

LIB_NAME = "libfa_mi355x.so"
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), LIB_NAME)

FA_F32, FA_F16, FA_BF16 = 0, 1, 2
STATUS = {
    0: "FA_OK", 1: "FA_ERR_NULL", 2: "FA_ERR_SHAPE", 3: "FA_ERR_HEADDIM", 4: "FA_ERR_DTYPE",
    5: "FA_ERR_ALIGN", 6: "FA_ERR_SCALE", 7: "FA_ERR_WORKSPACE", 8: "FA_ERR_HIP", 9: "FA_ERR_SCRATCH",
}

_lib = None


class FAError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the shared library (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{LIB_NAME} is not built ({path}); run __graft_entry__.build()")
    # torch ships its own HIP runtime under the same soname as the system's:
    # whichever is loaded first serves the whole process.  Import torch first
    # so that the library's kernels and torch's memory and streams share
    # torch's runtime (loaded the other way round, launches on torch's
    # tensors fail).
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    L = ctypes.CDLL(path)
    vp, i64, f32, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int, ctypes.c_size_t
    L.fa_abi_version.restype = i32
    L.fa_abi_version.argtypes = []
    L.fa_status_string.restype = ctypes.c_char_p
    L.fa_status_string.argtypes = [i32]
    L.fa_fwd.restype = i32
    L.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, f32, i32, i32, vp]
    L.fa_bwd_workspace_bytes.restype = sz
    L.fa_bwd_workspace_bytes.argtypes = [i64, i64, i64, i64, i32]
    L.fa_bwd.restype = i32
    L.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                         i64, i64, i64, i64, f32, i32, i32, vp]
    L.fa_bwd_prep.restype = i32
    L.fa_bwd_prep.argtypes = [vp, vp, vp, sz, i64, i64, i64, i64, i32, vp]
    L.fa_bwd_dkdv.restype = i32
    L.fa_bwd_dkdv.argtypes = [vp, vp, vp, vp, vp, vp, sz, vp, vp, i64, i64, i64, i64, f32, i32, i32, vp]
    L.fa_bwd_dq.restype = i32
    L.fa_bwd_dq.argtypes = [vp, vp, vp, vp, vp, vp, sz, vp, i64, i64, i64, i64, f32, i32, i32, vp]
    L.fa_fwd_kvcache_workspace_bytes.restype = sz
    L.fa_fwd_kvcache_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i32]
    L.fa_fwd_kvcache.restype = i32
    L.fa_fwd_kvcache.argtypes = [vp, vp, vp, vp, vp, vp, vp, sz, i64, i64, i64, i64, i64, f32, i32, i32, vp]
    L.fa_fwd_varlen_workspace_bytes.restype = sz
    L.fa_fwd_varlen_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i32]
    L.fa_fwd_varlen.restype = i32
    L.fa_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, sz, i64, i64, i64, i64, i64, i64, i64, f32, i32,
                                i32, vp]
    L.fa_bwd_varlen_workspace_bytes.restype = sz
    L.fa_bwd_varlen_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i32]
    L.fa_bwd_varlen.restype = i32
    L.fa_bwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i64, i64, i64, i64, i64, i64,
                                i64, f32, i32, i32, vp]
    L.fa_fwd_strided.restype = i32
    L.fa_fwd_strided.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, f32, i32, i32, vp]
    L.fa_bwd_strided.restype = i32
    L.fa_bwd_strided.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, i64, i64, i64, i64, f32, i32, i32, vp]
    L.fa_fwd_fp8.restype = i32
    L.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, vp, i32, vp, vp, i64, i64, i64, i64, f32, i32, i32, vp]
    L.fa_bwd_noalloc_max_rows.restype = sz
    L.fa_bwd_noalloc_max_rows.argtypes = []
    L.fa_bwd_noalloc.restype = i32
    L.fa_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, f32, i32, i32, vp]
    L.fa_probe_mfma_bf16.restype = i64
    L.fa_probe_mfma_bf16.argtypes = [i64, i64, vp]
    L.fa_fwd_kvcache_fp8.restype = i32
    L.fa_fwd_kvcache_fp8.argtypes = [vp, vp, vp, f32, f32, vp, vp, vp, vp, sz, i64, i64, i64, i64, i64, f32, i32,
                                     i32, vp]
    _lib = L
    return L


def _torch():
    import torch
    return torch


def dtype_code(t) -> int:
    torch = _torch()
    m = {torch.float32: FA_F32, torch.float16: FA_F16, torch.bfloat16: FA_BF16}
    if t.dtype not in m:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return m[t.dtype]


def _check(code: int):
    if code != 0:
        msg = load_library().fa_status_string(code).decode()
        raise FAError(code, msg)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(t) -> int:
    torch = _torch()
    return torch.cuda.current_stream(t.device).cuda_stream


def _bhnd(q):
    if q.dim() != 4:
        raise ValueError("expected [B, H, N, d] tensors")
    return tuple(int(x) for x in q.shape)


def _check_tensors(*ts):
    ref = ts[0]
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")
        if t.device != ref.device:
            raise ValueError("all tensors must be on the same device")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")


def _check_like(ref, names, *ts):
    """Every tensor of ts has ref's shape and dtype (names: for the message)."""
    for t in ts:
        if tuple(t.shape) != tuple(ref.shape) or t.dtype != ref.dtype:
            raise ValueError(f"{names} must share shape and dtype")


def _check_f32(t, shape, what: str):
    torch = _torch()
    if tuple(t.shape) != tuple(shape) or t.dtype != torch.float32:
        raise ValueError(f"{what} must be float32 {list(shape)}")


def _check_workspace(workspace, B: int, H: int, N: int):
    """The backward's workspace holds one float32 per query row."""
    nbytes = workspace.numel() * workspace.element_size()
    if nbytes < 4 * B * H * N:
        raise ValueError(f"workspace must hold at least {4 * B * H * N} bytes")


def fa_fwd(q, k, v, o, lse, scale: float, causal: bool) -> None:
    """Enqueue the forward on the current stream of q's device (see include/fa.h)."""
    L = load_library()
    _check_tensors(q, k, v, o, lse)
    B, H, N, d = _bhnd(q)
    for t in (k, v, o):
        if tuple(t.shape) != (B, H, N, d) or t.dtype != q.dtype:
            raise ValueError("q, k, v, o must share shape and dtype")
    torch = _torch()
    if tuple(lse.shape) != (B, H, N) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [B, H, N]")
    _check(L.fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
                    float(scale), int(bool(causal)), dtype_code(q), _stream(q)))


def fa_bwd_workspace_bytes(B: int, H: int, N: int, d: int, dtype: int) -> int:
    return int(load_library().fa_bwd_workspace_bytes(B, H, N, d, dtype))


def fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, scale: float, causal: bool) -> None:
    """Enqueue the backward on the current stream of q's device (see include/fa.h)."""
    L = load_library()
    B, H, N, d = _bhnd(q)
    _check_like(q, "q, k, v, o, dout, dq, dk, dv", k, v, o, dout, dq, dk, dv)
    _check_f32(lse, (B, H, N), "lse")
    _check_workspace(workspace, B, H, N)
    _check_tensors(q, k, v, o, lse, dout, dq, dk, dv, workspace)
    nbytes = workspace.numel() * workspace.element_size()
    _check(L.fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                    _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), nbytes,
                    B, H, N, d, float(scale), int(bool(causal)), dtype_code(q), _stream(q)))


FA_SCALE_TENSOR, FA_SCALE_BLOCK = 0, 1
FP8_BLOCK = 128


def fa_fwd_fp8(q8, k8, v8, q_scale, k_scale, v_scale, granularity: str, o, lse, scale: float,
               causal: bool) -> None:
    """Forward on 8-bit inputs (see include/fa.h): q8, k8, v8 uint8 E4M3 codes
    [B, H, N, d] (d = 128); float32 scales on the device: granularity
    "tensor" one each, "block" q_scale and k_scale [B, H, ceil(N / 128)] and
    v_scale [B, H]; o [B, H, N, d] bf16 or fp16; lse float32 [B, H, N]."""
    L = load_library()
    torch = _torch()
    B, H, N, d = _bhnd(q8)
    for t in (q8, k8, v8):
        if tuple(t.shape) != (B, H, N, d) or t.dtype != torch.uint8:
            raise ValueError("q8, k8, v8 must be uint8 [B, H, N, d] of one shape")
    if tuple(o.shape) != (B, H, N, d) or o.dtype not in (torch.bfloat16, torch.float16):
        raise ValueError("o must be bf16 or fp16 [B, H, N, d]")
    _check_f32(lse, (B, H, N), "lse")
    if granularity == "tensor":
        shapes, g = ((1,), (1,), (1,)), FA_SCALE_TENSOR
    elif granularity == "block":
        nb = (N + FP8_BLOCK - 1) // FP8_BLOCK
        shapes, g = ((B, H, nb), (B, H, nb), (B, H)), FA_SCALE_BLOCK
    else:
        raise ValueError("granularity must be 'tensor' or 'block'")
    for t, shp, nm in zip((q_scale, k_scale, v_scale), shapes, ("q_scale", "k_scale", "v_scale")):
        _check_f32(t, shp, nm)
    _check_tensors(q8, k8, v8, q_scale, k_scale, v_scale, o, lse)
    _check(L.fa_fwd_fp8(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(q_scale), _ptr(k_scale), _ptr(v_scale), g, _ptr(o),
                        _ptr(lse), B, H, N, d, float(scale), int(bool(causal)), dtype_code(o), _stream(q8)))


def fwd_fp8(q8, k8, v8, q_scale, k_scale, v_scale, granularity: str = "block", causal: bool = False,
            scale: float | None = None, out_dtype=None):
    """Allocate O (bf16 unless out_dtype) and LSE and run the 8-bit forward."""
    torch = _torch()
    B, H, N, d = _bhnd(q8)
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16 if out_dtype is None else out_dtype, device=q8.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q8.device)
    fa_fwd_fp8(q8, k8, v8, q_scale, k_scale, v_scale, granularity, o, lse,
               default_scale(d) if scale is None else scale, causal)
    return o, lse


def fa_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, scale: float, causal: bool) -> None:
    """fa_bwd without a workspace: the library's static per-GPU scratch holds
    D_i (B * H * N <= fa_bwd_noalloc_max_rows()); allocates nothing.  Calls
    that overlap in time on one GPU race (see include/fa.h)."""
    L = load_library()
    B, H, N, d = _bhnd(q)
    _check_like(q, "q, k, v, o, dout, dq, dk, dv", k, v, o, dout, dq, dk, dv)
    _check_f32(lse, (B, H, N), "lse")
    _check_tensors(q, k, v, o, lse, dout, dq, dk, dv)
    _check(L.fa_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                            _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, d, float(scale), int(bool(causal)),
                            dtype_code(q), _stream(q)))


def fa_bwd_noalloc_max_rows() -> int:
    return int(load_library().fa_bwd_noalloc_max_rows())


def fa_bwd_prep(o, dout, workspace) -> None:
    """Stage 1 of the backward: workspace[i] = dout_i . o_i (float32)."""
    L = load_library()
    B, H, N, d = _bhnd(o)
    _check_like(o, "o, dout", dout)
    _check_workspace(workspace, B, H, N)
    _check_tensors(o, dout, workspace)
    _check(L.fa_bwd_prep(_ptr(o), _ptr(dout), _ptr(workspace),
                         workspace.numel() * workspace.element_size(), B, H, N, d,
                         dtype_code(o), _stream(o)))


def fa_bwd_dkdv(q, k, v, dout, lse, workspace, dk, dv, scale: float, causal: bool) -> None:
    """Stage 2 of the backward: dK and dV (needs the prepared workspace)."""
    L = load_library()
    B, H, N, d = _bhnd(q)
    _check_like(q, "q, k, v, dout, dk, dv", k, v, dout, dk, dv)
    _check_f32(lse, (B, H, N), "lse")
    _check_workspace(workspace, B, H, N)
    _check_tensors(q, k, v, dout, lse, workspace, dk, dv)
    _check(L.fa_bwd_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse), _ptr(workspace),
                         workspace.numel() * workspace.element_size(), _ptr(dk), _ptr(dv),
                         B, H, N, d, float(scale), int(bool(causal)), dtype_code(q), _stream(q)))


def fa_bwd_dq(q, k, v, dout, lse, workspace, dq, scale: float, causal: bool) -> None:
    """Stage 3 of the backward: dQ (needs the prepared workspace)."""
    L = load_library()
    B, H, N, d = _bhnd(q)
    _check_like(q, "q, k, v, dout, dq", k, v, dout, dq)
    _check_f32(lse, (B, H, N), "lse")
    _check_workspace(workspace, B, H, N)
    _check_tensors(q, k, v, dout, lse, workspace, dq)
    _check(L.fa_bwd_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse), _ptr(workspace),
                       workspace.numel() * workspace.element_size(), _ptr(dq),
                       B, H, N, d, float(scale), int(bool(causal)), dtype_code(q), _stream(q)))


def fa_fwd_kvcache_workspace_bytes(B: int, H: int, Nq: int, Nk: int, d: int, dtype: int) -> int:
    return int(load_library().fa_fwd_kvcache_workspace_bytes(B, H, Nq, Nk, d, dtype))


def fa_fwd_kvcache(q, k_cache, v_cache, seqlens_k, o, lse, workspace, scale: float, causal: bool) -> None:
    """Enqueue queries against a key/value cache on the current stream (see include/fa.h).

    q, o: [B, H, Nq, d]; k_cache, v_cache: [B, H, Nk, d]; seqlens_k: int32 [B]
    on the device or None; lse: float32 [B, H, Nq]; workspace: device bytes or
    None when fa_fwd_kvcache_workspace_bytes() is 0."""
    L = load_library()
    torch = _torch()
    _check_tensors(q, k_cache, v_cache, seqlens_k, o, lse, workspace)
    B, H, Nq, d = _bhnd(q)
    Nk = int(k_cache.shape[2]) if k_cache.dim() == 4 else -1
    if tuple(k_cache.shape) != (B, H, Nk, d) or tuple(v_cache.shape) != (B, H, Nk, d):
        raise ValueError("k_cache and v_cache must be [B, H, Nk, d] with q's B, H and d")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype or o.dtype != q.dtype:
        raise ValueError("q, k_cache, v_cache, o must share dtype")
    if tuple(o.shape) != (B, H, Nq, d):
        raise ValueError("o must be [B, H, Nq, d]")
    if tuple(lse.shape) != (B, H, Nq) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [B, H, Nq]")
    if seqlens_k is not None and (seqlens_k.dtype != torch.int32 or tuple(seqlens_k.shape) != (B,)):
        raise ValueError("seqlens_k must be int32 [B]")
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(L.fa_fwd_kvcache(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens_k), _ptr(o), _ptr(lse),
                            _ptr(workspace), nbytes, B, H, Nq, Nk, d, float(scale), int(bool(causal)),
                            dtype_code(q), _stream(q)))


def fa_fwd_kvcache_fp8(q, k_cache, v_cache, k_scale: float, v_scale: float, seqlens_k, o, lse, workspace,
                       scale: float, causal: bool) -> None:
    """As fa_fwd_kvcache with an 8-bit cache: k_cache, v_cache are uint8 [B, H, Nk, d]
    tensors of OCP E4M3 codes, dequantised as k_scale * code and v_scale * code."""
    L = load_library()
    torch = _torch()
    _check_tensors(q, k_cache, v_cache, seqlens_k, o, lse, workspace)
    B, H, Nq, d = _bhnd(q)
    Nk = int(k_cache.shape[2]) if k_cache.dim() == 4 else -1
    if tuple(k_cache.shape) != (B, H, Nk, d) or tuple(v_cache.shape) != (B, H, Nk, d):
        raise ValueError("k_cache and v_cache must be [B, H, Nk, d] with q's B, H and d")
    if k_cache.dtype != torch.uint8 or v_cache.dtype != torch.uint8:
        raise ValueError("an 8-bit cache holds uint8 E4M3 codes")
    if o.dtype != q.dtype or tuple(o.shape) != (B, H, Nq, d):
        raise ValueError("o must be [B, H, Nq, d] of q's dtype")
    if tuple(lse.shape) != (B, H, Nq) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [B, H, Nq]")
    if seqlens_k is not None and (seqlens_k.dtype != torch.int32 or tuple(seqlens_k.shape) != (B,)):
        raise ValueError("seqlens_k must be int32 [B]")
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(L.fa_fwd_kvcache_fp8(_ptr(q), _ptr(k_cache), _ptr(v_cache), float(k_scale), float(v_scale),
                                _ptr(seqlens_k), _ptr(o), _ptr(lse), _ptr(workspace), nbytes, B, H, Nq, Nk, d,
                                float(scale), int(bool(causal)), dtype_code(q), _stream(q)))


def fwd_kvcache_fp8(q, k_cache, v_cache, k_scale: float, v_scale: float, seqlens_k=None, causal: bool = True,
                    scale: float | None = None, workspace=None):
    """Allocate O, LSE (and the workspace unless given) and run the queries
    against an 8-bit cache. Returns (o, lse)."""
    torch = _torch()
    B, H, Nq, d = _bhnd(q)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if workspace is None:
        nb = fa_fwd_kvcache_workspace_bytes(B, H, Nq, int(k_cache.shape[2]), d, dtype_code(q))
        workspace = torch.empty(nb, dtype=torch.uint8, device=q.device) if nb > 0 else None
    fa_fwd_kvcache_fp8(q, k_cache, v_cache, k_scale, v_scale, seqlens_k, o, lse, workspace,
                       default_scale(d) if scale is None else scale, causal)
    return o, lse


def fwd_kvcache(q, k_cache, v_cache, seqlens_k=None, causal: bool = True, scale: float | None = None,
                workspace=None):
    """Allocate O, LSE (and the workspace unless given) and run the queries
    against the cache. Returns (o, lse)."""
    torch = _torch()
    B, H, Nq, d = _bhnd(q)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if workspace is None:
        nb = fa_fwd_kvcache_workspace_bytes(B, H, Nq, int(k_cache.shape[2]), d, dtype_code(q))
        workspace = torch.empty(nb, dtype=torch.uint8, device=q.device) if nb > 0 else None
    fa_fwd_kvcache(q, k_cache, v_cache, seqlens_k, o, lse, workspace,
                   default_scale(d) if scale is None else scale, causal)
    return o, lse


def fa_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, o, lse, workspace, max_q: int, max_k: int,
                  scale: float, causal: bool) -> None:
    """Enqueue a variable-length packed batch (see include/fa.h): q, o
    [total_q, H, d]; k, v [total_k, H, d]; cu_seqlens_q/k int32 [B + 1] on
    the device; lse float32 [H, total_q]."""
    L = load_library()
    torch = _torch()
    _check_tensors(q, k, v, cu_seqlens_q, cu_seqlens_k, o, lse, workspace)
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("packed tensors are [total, H, d]")
    tq, H, d = (int(x) for x in q.shape)
    tk = int(k.shape[0])
    if tuple(k.shape) != (tk, H, d) or tuple(v.shape) != (tk, H, d) or tuple(o.shape) != (tq, H, d):
        raise ValueError("k, v must be [total_k, H, d] and o [total_q, H, d]")
    if k.dtype != q.dtype or v.dtype != q.dtype or o.dtype != q.dtype:
        raise ValueError("q, k, v, o must share dtype")
    if tuple(lse.shape) != (H, tq) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [H, total_q]")
    B = int(cu_seqlens_q.shape[0]) - 1
    for cu in (cu_seqlens_q, cu_seqlens_k):
        if cu.dtype != torch.int32 or tuple(cu.shape) != (B + 1,):
            raise ValueError("cu_seqlens must be int32 [B + 1]")
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(L.fa_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), _ptr(o), _ptr(lse),
                           _ptr(workspace), nbytes, B, H, tq, tk, int(max_q), int(max_k), d, float(scale),
                           int(bool(causal)), dtype_code(q), _stream(q)))


def fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_q: int, max_k: int, causal: bool = False,
               scale: float | None = None, workspace=None):
    """Allocate O, LSE (and the workspace unless given) and run a packed
    variable-length batch. Returns (o [total_q, H, d], lse [H, total_q]).
    O rows outside every sequence are zero."""
    torch = _torch()
    tq, H, d = (int(x) for x in q.shape)
    B = int(cu_seqlens_q.shape[0]) - 1
    o = torch.zeros_like(q)
    lse = torch.empty((H, tq), dtype=torch.float32, device=q.device)
    if workspace is None:
        nb = int(load_library().fa_fwd_varlen_workspace_bytes(B, H, max_q, max_k, d, dtype_code(q)))
        workspace = torch.empty(nb, dtype=torch.uint8, device=q.device) if nb > 0 else None
    fa_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, o, lse, workspace, max_q, max_k,
                  default_scale(d) if scale is None else scale, causal)
    return o, lse


def fa_bwd_varlen_workspace_bytes(B: int, H: int, total_q: int, max_q: int, d: int, dtype: int) -> int:
    return int(load_library().fa_bwd_varlen_workspace_bytes(B, H, total_q, max_q, d, dtype))


def fa_bwd_varlen(q, k, v, o, lse, dout, cu_seqlens_q, cu_seqlens_k, dq, dk, dv, workspace, max_q: int,
                  max_k: int, scale: float, causal: bool) -> None:
    """Enqueue the backward of a packed variable-length batch (see
    include/fa.h): q, o, dout, dq [total_q, H, d]; k, v, dk, dv [total_k, H,
    d]; lse float32 [H, total_q]; cu_seqlens_q/k int32 [B + 1] on the device
    (the same tensor for self-attention)."""
    L = load_library()
    torch = _torch()
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("packed tensors are [total, H, d]")
    tq, H, d = (int(x) for x in q.shape)
    tk = int(k.shape[0])
    for t in (o, dout, dq):
        if tuple(t.shape) != (tq, H, d) or t.dtype != q.dtype:
            raise ValueError("q, o, dout, dq must be [total_q, H, d] of one dtype")
    for t in (k, v, dk, dv):
        if tuple(t.shape) != (tk, H, d) or t.dtype != q.dtype:
            raise ValueError("k, v, dk, dv must be [total_k, H, d] of q's dtype")
    _check_f32(lse, (H, tq), "lse")
    B = int(cu_seqlens_q.shape[0]) - 1
    for cu in (cu_seqlens_q, cu_seqlens_k):
        if cu.dtype != torch.int32 or tuple(cu.shape) != (B + 1,):
            raise ValueError("cu_seqlens must be int32 [B + 1]")
    _check_tensors(q, k, v, o, lse, dout, cu_seqlens_q, cu_seqlens_k, dq, dk, dv, workspace)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(L.fa_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(cu_seqlens_q),
                           _ptr(cu_seqlens_k), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), nbytes, B, H, tq, tk,
                           int(max_q), int(max_k), d, float(scale), int(bool(causal)), dtype_code(q), _stream(q)))


def bwd_varlen(q, k, v, o, lse, dout, cu_seqlens_q, cu_seqlens_k=None, max_q: int | None = None,
               max_k: int | None = None, causal: bool = True, scale: float | None = None, workspace=None):
    """Allocate dQ, dK, dV (zero rows outside every sequence) and the
    workspace unless given, and run the packed backward (keys share the
    query prefix sums unless cu_seqlens_k is given)."""
    torch = _torch()
    tq, H, d = (int(x) for x in q.shape)
    cu_k = cu_seqlens_q if cu_seqlens_k is None else cu_seqlens_k
    B = int(cu_seqlens_q.shape[0]) - 1
    if max_q is None:
        max_q = max(int((cu_seqlens_q[1:] - cu_seqlens_q[:-1]).max().item()), 1)
    if max_k is None:
        max_k = max_q if cu_seqlens_k is None else max(int((cu_k[1:] - cu_k[:-1]).max().item()), 1)
    dq, dk, dv = torch.zeros_like(q), torch.zeros_like(k), torch.zeros_like(v)
    if workspace is None:
        nb = fa_bwd_varlen_workspace_bytes(B, H, tq, max_q, d, dtype_code(q))
        workspace = torch.empty(max(nb, 16), dtype=torch.uint8, device=q.device)
    fa_bwd_varlen(q, k, v, o, lse, dout, cu_seqlens_q, cu_k, dq, dk, dv, workspace, max_q, max_k,
                  default_scale(d) if scale is None else scale, causal)
    return dq, dk, dv


def _strides_of(*ts):
    """Element strides (batch, head, row) of [B, H, N, d] views whose d
    elements are contiguous, as the flat int64 list the strided entry points
    take."""
    out = []
    for t in ts:
        if t.dim() != 4 or t.stride(3) != 1:
            raise ValueError("strided tensors are [B, H, N, d] views with contiguous d")
        out += [int(t.stride(0)), int(t.stride(1)), int(t.stride(2))]
    return (ctypes.c_int64 * len(out))(*out)


def fa_fwd_strided(q, k, v, o, lse, scale: float, causal: bool) -> None:
    """fa_fwd on [B, H, N, d] views with any strides (contiguous d): e.g.
    [B, N, H, d] tensors transposed, or slices of a packed QKV tensor."""
    L = load_library()
    B, H, N, d = _bhnd(q)
    for t in (k, v, o):
        if tuple(t.shape) != (B, H, N, d) or t.dtype != q.dtype:
            raise ValueError("q, k, v, o must share shape and dtype")
    _check_f32(lse, (B, H, N), "lse")
    if not lse.is_contiguous():
        raise ValueError("lse must be contiguous")
    st = _strides_of(q, k, v, o)
    if not all(t.is_cuda for t in (q, k, v, o, lse)):
        raise ValueError("all tensors must be on the GPU")
    _check(L.fa_fwd_strided(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), st, B, H, N, d, float(scale),
                            int(bool(causal)), dtype_code(q), _stream(q)))


def fa_bwd_strided(q, k, v, o, lse, dout, dq, dk, dv, workspace, scale: float, causal: bool) -> None:
    """fa_bwd on [B, H, N, d] views with any strides (contiguous d)."""
    L = load_library()
    B, H, N, d = _bhnd(q)
    for t in (k, v, o, dout, dq, dk, dv):
        if tuple(t.shape) != (B, H, N, d) or t.dtype != q.dtype:
            raise ValueError("q, k, v, o, dout, dq, dk, dv must share shape and dtype")
    _check_f32(lse, (B, H, N), "lse")
    _check_workspace(workspace, B, H, N)
    if not lse.is_contiguous():
        raise ValueError("lse must be contiguous")
    st = _strides_of(q, k, v, o, dout, dq, dk, dv)
    if not all(t.is_cuda for t in (q, k, v, o, lse, dout, dq, dk, dv, workspace)):
        raise ValueError("all tensors must be on the GPU")
    nbytes = workspace.numel() * workspace.element_size()
    _check(L.fa_bwd_strided(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                            _ptr(workspace), nbytes, st, B, H, N, d, float(scale), int(bool(causal)), dtype_code(q),
                            _stream(q)))


def fa_probe_mfma_bf16(workgroups: int, iters: int) -> int:
    """Enqueue the dense bf16 MFMA probe on the current stream; returns its FLOP count."""
    torch = _torch()
    n = int(load_library().fa_probe_mfma_bf16(workgroups, iters, torch.cuda.current_stream().cuda_stream))
    if n < 0:
        _check(-n)
    return n


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


def fwd(q, k, v, causal: bool = False, scale: float | None = None):
    """Allocate O and LSE and run the forward. Returns (o, lse)."""
    torch = _torch()
    B, H, N, d = _bhnd(q)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    fa_fwd(q, k, v, o, lse, default_scale(d) if scale is None else scale, causal)
    return o, lse


def bwd(q, k, v, o, lse, dout, causal: bool = False, scale: float | None = None, workspace=None):
    """Allocate dQ, dK, dV (and the workspace unless given) and run the backward."""
    torch = _torch()
    B, H, N, d = _bhnd(q)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    if workspace is None:
        nb = fa_bwd_workspace_bytes(B, H, N, d, dtype_code(q))
        workspace = torch.empty(max(nb, 16), dtype=torch.uint8, device=q.device)
    fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace,
           default_scale(d) if scale is None else scale, causal)
    return dq, dk, dv


def _autograd_fn():
    torch = _torch()

    class FlashAttention(torch.autograd.Function):
        """softmax(scale Q K^T [causal]) V with the library's forward and backward."""

        @staticmethod
        def forward(ctx, q, k, v, causal=False, scale=None):
            q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
            s = default_scale(q.shape[-1]) if scale is None else scale
            o, lse = fwd(q, k, v, causal, s)
            ctx.save_for_backward(q, k, v, o, lse)
            ctx.causal, ctx.scale = causal, s
            return o

        @staticmethod
        def backward(ctx, do):
            q, k, v, o, lse = ctx.saved_tensors
            dq, dk, dv = bwd(q, k, v, o, lse, do.contiguous(), ctx.causal, ctx.scale)
            return dq, dk, dv, None, None

    return FlashAttention


def attention(q, k, v, causal: bool = False, scale: float | None = None):
    """Differentiable attention through the library (torch.autograd)."""
    return _autograd_fn().apply(q, k, v, causal, scale)


__all__ = [
    "load_library", "fa_fwd", "fa_bwd", "fa_bwd_workspace_bytes", "fa_bwd_prep", "fa_bwd_dkdv",
    "fa_bwd_dq", "fa_fwd_kvcache", "fa_fwd_kvcache_workspace_bytes", "fa_fwd_kvcache_fp8", "fwd", "bwd",
    "fwd_kvcache", "fwd_kvcache_fp8", "fa_fwd_varlen", "fwd_varlen", "fa_probe_mfma_bf16", "attention",
    "FAError", "FA_F32", "FA_F16", "FA_BF16", "LIB_PATH",
]
