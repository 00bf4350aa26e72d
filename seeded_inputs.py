"""Seeded synthetic inputs shared by the oracle checks and the GPU path.

This module holds no attention arithmetic: it only draws random numbers and
rounds them to the storage dtype.  Both sides (the float64 oracle and the HIP
library) are fed the *same* rounded values, so any difference between them is
the method's own rounding, never the inputs'.

Recipe (identical for every workload):
  * numpy ``default_rng(seed)`` (PCG64);
  * draw Q, K, V and then (for a backward workload) dO, in that order, each as
    float32 ``standard_normal`` of shape [B, H, N, d], multiplied by sigma;
  * round to the storage dtype with round-to-nearest-even (bf16 by bit
    arithmetic on the float32 pattern, fp16 by numpy's IEEE conversion,
    fp32 unchanged).

The named workloads are the five configurations the attention library is
measured on; variants reuse their parent's seed.
"""

from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str  # "f32" | "f16" | "bf16"
    causal: bool
    sigma: float
    seed: int
    backward: bool = False

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))

    def fwd_flop(self) -> float:
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f

    def bwd_flop(self) -> float:
        f = 10.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


@dataclass(frozen=True)
class Fp8Workload:
    """8-bit (E4M3) Q, K, V with float scales: the parent workload's draw
    (same seed, same 16-bit values), quantised per tensor or per block of
    FP8_BLOCK rows of a head (V: per head)."""
    name: str
    B: int
    H: int
    N: int
    d: int
    out_dtype: str  # 16-bit type of O and of the probabilities
    causal: bool
    sigma: float
    seed: int
    granularity: str  # "tensor" | "block"

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))

    def fwd_flop(self) -> float:
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f


WORKLOADS = {
    # tiny forward case: fp32, non-causal
    "C1": Workload("C1", 1, 2, 256, 64, "f32", False, 1.0, 1001),
    # forward bf16 non-causal
    "C2": Workload("C2", 4, 16, 2048, 128, "bf16", False, 1.0, 1002),
    # forward bf16 causal, decoder-pretraining shape (and its d=64 variant)
    "C3": Workload("C3", 2, 32, 8192, 128, "bf16", True, 1.0, 1003),
    "C3d64": Workload("C3d64", 2, 32, 8192, 64, "bf16", True, 1.0, 1003),
    # long-context forward fp16 causal, sigma 0.5
    "C4": Workload("C4", 1, 32, 32768, 128, "f16", True, 0.5, 1004),
    # backward bf16 causal with recompute (and its d=128 variant)
    "C5": Workload("C5", 8, 16, 4096, 64, "bf16", True, 1.0, 1005, backward=True),
    "C5d128": Workload("C5d128", 8, 16, 4096, 128, "bf16", True, 1.0, 1005, backward=True),
    "C5d256": Workload("C5d256", 8, 16, 4096, 256, "bf16", True, 1.0, 1005, backward=True),
}

# the forward on 8-bit inputs: C3's and C2's draws quantised to E4M3 with one
# scale per 128-row block of each head (V: per head), bf16 output
FP8_WORKLOADS = {
    "C3f8": Fp8Workload("C3f8", 2, 32, 8192, 128, "bf16", True, 1.0, 1003, "block"),
    "C2f8": Fp8Workload("C2f8", 4, 16, 2048, 128, "bf16", False, 1.0, 1002, "block"),
}


def round_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = np.isnan(x)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_to(x: np.ndarray, dtype: str):
    """Round float32 values to ``dtype``.

    Returns (values as float32 holding exactly the rounded numbers,
             storage array: uint16 bit patterns for bf16, float16 for f16,
             float32 for f32).
    """
    if dtype == "f32":
        x = np.ascontiguousarray(x, dtype=np.float32)
        return x, x
    if dtype == "f16":
        h = np.ascontiguousarray(x, dtype=np.float32).astype(np.float16)
        return h.astype(np.float32), h
    if dtype == "bf16":
        b = round_bf16_bits(x)
        return bf16_bits_to_f32(b), b
    raise ValueError(f"unknown dtype {dtype!r}")


def make_inputs(B: int, H: int, N: int, d: int, dtype: str, sigma: float, seed: int,
                backward: bool = False):
    """Draw the seeded inputs. Returns a dict name -> (float32 values, storage array)."""
    rng = np.random.default_rng(seed)
    names = ["q", "k", "v"] + (["do"] if backward else [])
    out = {}
    for nm in names:
        x = rng.standard_normal((B, H, N, d), dtype=np.float32)
        if sigma != 1.0:
            x *= np.float32(sigma)
        out[nm] = round_to(x, dtype)
    return out


def make_workload_inputs(w: Workload, backward: bool | None = None):
    return make_inputs(w.B, w.H, w.N, w.d, w.dtype, w.sigma, w.seed,
                       w.backward if backward is None else backward)


# queries against a key/value cache: a decode step of one new token per
# sequence over a 32768-row cache (bf16, causal), filled lengths drawn per
# batch entry between half and all of the capacity
@dataclass(frozen=True)
class KvWorkload:
    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    dtype: str
    causal: bool
    sigma: float
    seed: int
    min_fill: float = 0.5  # filled lengths drawn uniformly in [min_fill * Nk, Nk]
    cache: str = "same"    # "same": K, V in the query dtype; "e4m3": 8-bit cache

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))


KV_WORKLOADS = {
    "D1": KvWorkload("D1", 4, 32, 1, 32768, 128, "bf16", True, 1.0, 1006),
    "D1d64": KvWorkload("D1d64", 4, 32, 1, 32768, 64, "bf16", True, 1.0, 1006),
    # the same decode step with the cache stored as per-tensor scaled E4M3
    "D1f8": KvWorkload("D1f8", 4, 32, 1, 32768, 128, "bf16", True, 1.0, 1006, cache="e4m3"),
}


def make_kvcache_inputs(B: int, H: int, Nq: int, Nk: int, d: int, dtype: str, sigma: float, seed: int,
                        min_fill: float = 0.5):
    """Draw queries, a key/value cache and filled lengths.

    Q [B,H,Nq,d], then K and V [B,H,Nk,d], each float32 standard normal times
    sigma rounded to ``dtype`` (as in make_inputs), then the filled lengths
    seqlens [B] (int32) uniform in [ceil(min_fill * Nk), Nk].
    Returns a dict name -> (float32 values, storage array), plus "seqlens"."""
    rng = np.random.default_rng(seed)
    out = {}
    for nm, n in (("q", Nq), ("k", Nk), ("v", Nk)):
        x = rng.standard_normal((B, H, n, d), dtype=np.float32)
        if sigma != 1.0:
            x *= np.float32(sigma)
        out[nm] = round_to(x, dtype)
    lo = int(np.ceil(min_fill * Nk))
    out["seqlens"] = rng.integers(lo, Nk + 1, size=B).astype(np.int32)
    return out


def make_kv_workload_inputs(w: KvWorkload):
    if w.cache == "e4m3":
        return make_kvcache_fp8_inputs(w.B, w.H, w.Nq, w.Nk, w.d, w.dtype, w.sigma, w.seed, w.min_fill)
    return make_kvcache_inputs(w.B, w.H, w.Nq, w.Nk, w.d, w.dtype, w.sigma, w.seed, w.min_fill)


# ---- 8-bit floating point (OCP E4M3, "fn": no infinities, max 448) for a
# quantised key/value cache.  Only the rounding of drawn values to the
# storage format lives here.

def _e4m3_positive_table() -> np.ndarray:
    """Values of the codes 0x00 .. 0x7E (0x7F is NaN), ascending."""
    codes = np.arange(0x7F)
    e, m = codes >> 3, codes & 7
    return np.where(e == 0, m / 8.0 * 2.0 ** -6, (1 + m / 8.0) * 2.0 ** (e - 7.0))


E4M3_MAX = 448.0


def round_e4m3(x: np.ndarray) -> np.ndarray:
    """float32 -> E4M3 codes (uint8), round to nearest, ties to even, values
    beyond +-448 saturate to +-448, NaN -> 0x7F.

    |x| >= 2^-6 (normal): |x| = f 2^e with f in [0.5, 1); the code is
    8 (e + 6) + rint(16 f) - 8 (3 mantissa bits; a mantissa that rounds up to
    16 carries into the exponent by the same sum).  |x| < 2^-6 (subnormal,
    steps of 2^-9): the code is rint(512 |x|).  rint rounds half to even, and
    the code's last bit is the mantissa's, so ties go to the even code.
    Works in chunks (the arithmetic is exact in float32)."""
    x = np.asarray(x, dtype=np.float32)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    step = 1 << 24
    for i in range(0, flat.size, step):
        xi = flat[i:i + step]
        a = np.minimum(np.abs(xi), np.float32(E4M3_MAX))
        f, e = np.frexp(a)
        normal = 8 * (e.astype(np.int32) + 6) + np.rint(16 * f).astype(np.int32) - 8
        sub = np.rint(a * np.float32(512.0)).astype(np.int32)
        code = np.where(a < np.float32(2.0 ** -6), sub, normal).astype(np.uint8)
        code = np.where(np.signbit(xi) & (code != 0), code | np.uint8(0x80), code)
        out[i:i + step] = np.where(np.isnan(xi), np.uint8(0x7F), code)
    return out.reshape(x.shape)


def e4m3_to_f32(code: np.ndarray) -> np.ndarray:
    """E4M3 codes -> their float32 values (exact)."""
    code = np.asarray(code, dtype=np.uint8)
    tab = np.append(_e4m3_positive_table(), np.nan)
    v = tab[code & 0x7F]
    return np.where(code & 0x80, -v, v).astype(np.float32)


def quantise_e4m3(x: np.ndarray):
    """Per-tensor scaled E4M3 with a power-of-two scale: scale = 2^ceil(log2(
    max|x| / 448)) (1 if x is all zero), codes = round_e4m3(x / scale).
    Returns (codes uint8, scale float32, dequantised float32 values
    scale * e4m3(codes), exact: the scale only shifts exponents)."""
    amax = float(np.max(np.abs(x))) if x.size else 0.0
    scale = np.float32(2.0 ** np.ceil(np.log2(amax / E4M3_MAX)) if amax > 0 else 1.0)
    codes = round_e4m3(np.asarray(x, dtype=np.float32) / scale)
    deq = e4m3_to_f32(codes) * scale
    return codes, scale, deq


def make_kvcache_fp8_inputs(B: int, H: int, Nq: int, Nk: int, d: int, dtype: str, sigma: float, seed: int,
                            min_fill: float = 0.5):
    """As make_kvcache_inputs, with the cache stored as per-tensor scaled E4M3.

    The same draws as make_kvcache_inputs (so the 16-bit and 8-bit caches
    hold the same underlying values); K and V are then quantised with
    quantise_e4m3.  Returns the make_kvcache_inputs dict with "k" and "v"
    replaced by (dequantised float32 values, uint8 codes), the 16-bit cache
    kept as "k16"/"v16", and "k_scale", "v_scale"."""
    out = make_kvcache_inputs(B, H, Nq, Nk, d, dtype, sigma, seed, min_fill)
    out["k16"], out["v16"] = out["k"], out["v"]
    for nm in ("k", "v"):
        codes, sc, deq = quantise_e4m3(out[nm + "16"][0])
        out[nm] = (deq, codes)
        out[nm + "_scale"] = sc
    return out


def make_varlen_inputs(lens_q, lens_k, H: int, d: int, dtype: str, sigma: float, seed: int,
                       backward: bool = False):
    """A packed variable-length batch: Q [sum lens_q, H, d], then K and V
    [sum lens_k, H, d] (and, with backward, dO [sum lens_q, H, d]), drawn and
    rounded as in make_inputs, and the int32 prefix sums cu_q, cu_k [B + 1]."""
    rng = np.random.default_rng(seed)
    tq, tk = int(sum(lens_q)), int(sum(lens_k))
    out = {}
    draws = (("q", tq), ("k", tk), ("v", tk)) + ((("do", tq),) if backward else ())
    for nm, n in draws:
        x = rng.standard_normal((n, H, d), dtype=np.float32)
        if sigma != 1.0:
            x *= np.float32(sigma)
        out[nm] = round_to(x, dtype)
    out["cu_q"] = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    out["cu_k"] = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    return out


# ---- 8-bit Q, K, V with float scales (the 8-bit forward)

FP8_BLOCK = 128  # rows of a head sharing one scale (per-block scaling)


def quantise_e4m3_scaled(x: np.ndarray, granularity: str, per_head_only: bool = False):
    """E4M3 codes with float32 scales for a [B, H, N, d] tensor.

    granularity "tensor": one scale, amax / 448 over the whole tensor;
    "block": one scale per block of FP8_BLOCK rows of each head ([B, H,
    ceil(N / FP8_BLOCK)]), or per head ([B, H]) with per_head_only.  A block
    of zeros gets scale 1.  codes = round_e4m3(x / scale) in float32.
    Returns (codes uint8, scales float32, dequantised float64 values
    scale * e4m3(codes): exact in float64, and what the codes stand for)."""
    x = np.asarray(x, dtype=np.float32)
    B, H, N, d = x.shape
    if granularity == "tensor":
        amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
        sc = np.array([amax / np.float32(E4M3_MAX) if amax > 0 else 1.0], dtype=np.float32)
        rows = np.broadcast_to(sc[0], (B, H, N))
    elif per_head_only:
        amax = np.max(np.abs(x), axis=(2, 3))
        sc = np.where(amax > 0, amax / np.float32(E4M3_MAX), 1.0).astype(np.float32)
        rows = np.broadcast_to(sc[:, :, None], (B, H, N))
    else:
        nb = (N + FP8_BLOCK - 1) // FP8_BLOCK
        pad = np.zeros((B, H, nb * FP8_BLOCK, d), dtype=np.float32)
        pad[:, :, :N] = np.abs(x)
        amax = pad.reshape(B, H, nb, FP8_BLOCK * d).max(axis=3)
        sc = np.where(amax > 0, amax / np.float32(E4M3_MAX), 1.0).astype(np.float32)
        rows = np.repeat(sc, FP8_BLOCK, axis=2)[:, :, :N]
    rows = np.ascontiguousarray(rows, dtype=np.float32)
    codes = round_e4m3(x / rows[..., None])
    deq = e4m3_to_f32(codes).astype(np.float64) * rows[..., None].astype(np.float64)
    return codes, np.ascontiguousarray(sc, dtype=np.float32), deq


def make_fp8_inputs(B: int, H: int, N: int, d: int, out_dtype: str, sigma: float, seed: int, granularity: str):
    """Q, K, V drawn and rounded as make_inputs (the 16-bit inputs, kept as
    "q16", "k16", "v16"), then quantised with quantise_e4m3_scaled: Q and K
    per tensor or per block of FP8_BLOCK rows, V per tensor or per head.
    "q", "k", "v" are (dequantised float64 values, uint8 codes) and
    "q_scale", "k_scale", "v_scale" the float32 scales."""
    base = make_inputs(B, H, N, d, out_dtype, sigma, seed)
    out = {}
    for nm in ("q", "k", "v"):
        out[nm + "16"] = base[nm]
        codes, sc, deq = quantise_e4m3_scaled(base[nm][0], granularity, per_head_only=(nm == "v"))
        out[nm] = (deq, codes)
        out[nm + "_scale"] = sc
    return out


def make_fp8_workload_inputs(w: Fp8Workload):
    return make_fp8_inputs(w.B, w.H, w.N, w.d, w.out_dtype, w.sigma, w.seed, w.granularity)
