#!/usr/bin/env python3
"""Throughput benchmark of the attention library on one MI355X.

One step = the whole hot path over one batch of synthetic input: fa_fwd, then
the three backward stages (fa_bwd_prep, fa_bwd_dkdv, fa_bwd_dq), all through
the C ABI; dQ runs on a second stream beside dK/dV (they are independent),
--serial keeps every stage on one stream.  Per-kernel durations (roofline)
come from a separate pass with the stages in order, each between HIP events.  The default workload is the
fwd+bwd configuration B=8 H=16 N=4096 d=64, bf16, causal, with Q, K, V, dO
drawn as seeded N(0, 1) values (numpy PCG64, seed 1005) rounded to bf16.

Prints ONE JSON line: throughput in TFLOP/s (forward 4*B*H*N^2*d plus
backward 10*B*H*N^2*d, halved for causal), the dominant kernel against the
dense bf16 MFMA peak, and the float64 CPU oracle timed on a bounded sample of
the same workload.

Modes
  (default)             the benchmark above
  --workload D1         a decode step against a key/value cache instead (fa_fwd_kvcache,
                        B=4 H=32, one query, 32768-row cache, d=128): HBM GB/s;
                        D1f8: the same with an 8-bit E4M3 cache (fa_fwd_kvcache_fp8)
  --varlen              fa_fwd_varlen + fa_bwd_varlen on a packed batch of 16 ragged causal sequences
  --fwd-only            fa_fwd alone: time, TFLOP/s and compulsory GB/s per workload
                        (--workload C1,C3,...; --workload short: the short-sequence sweep;
                        --workload C3f8 or C2f8: fa_fwd_fp8 on the 8-bit form of C3's / C2's draw)
  --profile             --warmup + 20 timed steps (stages in order on one stream), no CPU
                        baseline, for rocprofv3 runs;
                        also runs a plain 1 GiB device copy (the calibration
                        kernel for FETCH_SIZE / WRITE_SIZE counters)
  --ingest-pmc F W      turn two rocprofv3 --pmc csv files (FETCH_SIZE, then
                        WRITE_SIZE) into profiles/traffic_<workload>.json
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd+bwd TFLOP/s (bf16, causal/non-causal) and % of MFMA peak, 1 GPU"
PEAK_MFMA_16BIT = 2516.6  # TFLOP/s, MI355X dense bf16/fp16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
PEAK_HBM = 8000.0  # GB/s
COPY_BYTES = 1 << 30  # calibration copy: reads and writes 1 GiB

KERNEL_SOURCES = {
    "kv": ["fa_kvcache.hip", "fa_common.hpp"],
    "fwd": ["fa_fwd.hip", "fa_common.hpp"],
    "prep": ["fa_bwd.hip", "fa_common.hpp"],
    "dkdv": ["fa_bwd.hip", "fa_common.hpp"],
    "dq": ["fa_bwd.hip", "fa_common.hpp"],
    "fwd8": ["fa_fwd_fp8.hip", "fa_common.hpp"],
}
WIDE_SOURCES = ["fa_bwd_wide.hip"]  # the d = 256 dK/dV and dQ kernels
# substrings of the mangled kernel names, as rocprofv3 reports them
KERNEL_SYMBOLS = {"fwd": "fwd16_p", "prep": "bwd_pre_kernel", "dkdv": "bwd_dkdv",
                  "dq": "bwd_dq", "kv": "kv_split", "fwd8": "fwd8_pipe"}


def workload_d(workload: str) -> int:
    """Head dimension of a named workload (0 if it has none by that name)."""
    import seeded_inputs as si
    for table in ("WORKLOADS", "FP8_WORKLOADS", "KV_WORKLOADS"):
        w = getattr(si, table, {}).get(workload)
        if w is not None:
            return int(getattr(w, "d", 0))
    return 0


def src_hash(kernel: str, d: int = 0) -> str:
    """Hash of the sources a kernel is built from (at d = 256 the backward
    stages run the wide kernels)."""
    h = hashlib.sha256()
    srcs = KERNEL_SOURCES[kernel] + (WIDE_SOURCES if d == 256 and kernel in ("dkdv", "dq") else [])
    for f in srcs:
        with open(os.path.join(ROOT, "exact_io_aware_fa2_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def algorithmic(w) -> dict:
    """Algorithmic work per launch of each kernel (FLOP, or bytes for prep).

    fwd:  S = Q K^T and O = P V: 4*B*H*N^2*d FLOP (halved when causal).
    dkdv: S, dP = dO V^T, dV = P^T dO, dK = dS^T Q: 8*B*H*N^2*d (halved).
    dq:   dQ = dS K: 2*B*H*N^2*d (halved).  Its recomputation of S and dP is
          not algorithmic work (the backward's five products are counted once,
          in dkdv and here).
    prep: reads O and dO, writes D: 2*B*H*N*d*s + 4*B*H*N bytes.
    """
    f = w.B * w.H * w.N * w.N * w.d * (0.5 if w.causal else 1.0)
    s = {"bf16": 2, "f16": 2, "f32": 4}[w.dtype]
    return {"fwd": 4 * f, "dkdv": 8 * f, "dq": 2 * f,
            "prep": 2 * w.B * w.H * w.N * w.d * s + 4 * w.B * w.H * w.N}


def traffic_file(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"traffic_{workload}.json")


def load_traffic(workload: str, kernel: str):
    """HBM bytes per launch from the committed counter summary, or None if the
    kernel's sources changed since the counters were taken."""
    p = traffic_file(workload)
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    k = t.get("kernels", {}).get(kernel)
    if not k or k.get("src_sha") != src_hash(kernel, workload_d(workload)):
        return None
    return k["bytes_per_launch"]


def cpu_baseline(w, heads_in, target_s: float):
    """The float64 oracle, as it stands, on whole heads of the workload's own
    draw: heads (b, h) in order, forward then backward, until target_s."""
    from oracle import attention_bwd_head, attention_fwd_head
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"), default=1)
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    q, k, v, do = (heads_in[n] for n in ("q", "k", "v", "do"))
    heads, t_total = 0, 0.0
    while t_total < target_s and heads < q.shape[0]:
        t0 = time.perf_counter()
        attention_fwd_head(q[heads], k[heads], v[heads], w.scale, w.causal)
        attention_bwd_head(q[heads], k[heads], v[heads], do[heads], w.scale, w.causal)
        t_total += time.perf_counter() - t0
        heads += 1
    flop = (4 + 10) * w.N * w.N * w.d * (0.5 if w.causal else 1.0) * heads
    return {"value": round(flop / t_total / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"the first {heads} of the workload's {w.B * w.H} heads in (batch, head) order "
                      f"(the same seeded draw the GPU step uses; N={w.N}, d={w.d}), each once, float64 "
                      f"numpy forward + backward, {t_total:.1f} s; BLAS threads {threads}, "
                      f"host cpus {os.cpu_count()}"}


def measured_mfma_peak() -> dict:
    """Sustained dense bf16 MFMA rate of this device from the library's probe
    (fa_probe_mfma_bf16: register-only v_mfma_f32_32x32x16_bf16 chains, two
    wavefronts per SIMD on 256 compute units), best of 5 timed launches."""
    import torch

    import exact_io_aware_fa2_amd as fa
    wgs, iters = 512, 4096
    fa.fa_probe_mfma_bf16(wgs, iters)
    torch.cuda.synchronize()
    best = 0.0
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        flop = fa.fa_probe_mfma_bf16(wgs, iters)
        e1.record()
        torch.cuda.synchronize()
        best = max(best, flop / (e0.elapsed_time(e1) * 1e-3) / 1e12)
    # 256 CUs x 4096 FLOP per clock (dense bf16): the clock the rate implies
    return {"TFLOP/s": round(best, 1), "frac_of_spec": round(best / PEAK_MFMA_16BIT, 4),
            "implied_clock_GHz": round(best * 1e12 / (256 * 4096) / 1e9, 3),
            "probe": "fa_probe_mfma_bf16, 512 workgroups x 4 wavefronts x 4096 rounds of 4 MFMAs"}


def kv_bytes(w, seqlens) -> float:
    """Compulsory HBM bytes of one call of fa_fwd_kvcache(_fp8): read Q and the
    filled cache rows of K and V once, write O and LSE."""
    s = {"bf16": 2, "f16": 2}[w.dtype]
    sc = 1 if w.cache == "e4m3" else s
    qo = 2 * w.B * w.H * w.Nq * w.d * s + 4 * w.B * w.H * w.Nq
    kv = 2 * w.H * w.d * sc * float(sum(int(x) for x in seqlens))
    return qo + kv


def cpu_baseline_kv(w, inp, target_s: float):
    """The float64 oracle, as it stands, on whole heads of the same decode step."""
    from oracle import kvcache_fwd_head
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"), default=1)
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    heads, t_total, nbytes = 0, 0.0, 0.0
    s = 1 if w.cache == "e4m3" else 2
    while t_total < target_s and heads < w.B * w.H:
        b, h = heads % w.B, heads // w.B
        L = int(inp["seqlens"][b])
        t0 = time.perf_counter()
        kvcache_fwd_head(inp["q"][0][b, h], inp["k"][0][b, h], inp["v"][0][b, h], w.scale, w.causal, L)
        t_total += time.perf_counter() - t0
        nbytes += 2 * L * w.d * s + 2 * w.Nq * w.d * 2 + 4 * w.Nq
        heads += 1
    return {"value": round(nbytes / t_total / 1e9, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{heads} of {w.B * w.H} heads (Nq={w.Nq}, filled lengths of the workload, d={w.d}), "
                      f"float64 numpy, {t_total:.1f} s; BLAS threads {threads}, host cpus {os.cpu_count()}"}


def bench_kvcache(args, w):
    """Decode step against a key/value cache: one fa_fwd_kvcache call (the
    split-key kernel and the merge kernel) per step, HBM-bound."""
    import numpy as np
    import torch

    import exact_io_aware_fa2_amd as fa
    import seeded_inputs as si

    dev = torch.device("cuda:0")
    inp = si.make_kv_workload_inputs(w)

    def up(name):
        a = inp[name][1]
        if w.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    fp8 = w.cache == "e4m3"
    q = up("q")
    if fp8:
        k, v = (torch.from_numpy(inp[n][1]).to(dev) for n in ("k", "v"))
    else:
        k, v = up("k"), up("v")
    lens = torch.from_numpy(inp["seqlens"]).to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)
    nb = fa.fa_fwd_kvcache_workspace_bytes(w.B, w.H, w.Nq, w.Nk, w.d, fa.dtype_code(q))
    ws = torch.empty(nb, dtype=torch.uint8, device=dev) if nb else None

    def step():
        if fp8:
            fa.fa_fwd_kvcache_fp8(q, k, v, float(inp["k_scale"]), float(inp["v_scale"]), lens, o, lse, ws,
                                  w.scale, w.causal)
        else:
            fa.fa_fwd_kvcache(q, k, v, lens, o, lse, ws, w.scale, w.causal)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t_start.record()
    for e0, e1 in evs:
        e0.record()
        step()
        e1.record()
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t_start.elapsed_time(t_end) / args.steps
    ms_call = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    nbytes = kv_bytes(w, inp["seqlens"])
    value = nbytes / (ms_step * 1e-3) / 1e9
    achieved = nbytes / (ms_call * 1e-3) / 1e9
    out = {
        "metric": "attention decode against a KV cache, HBM GB/s (compulsory bytes), 1 GPU",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"{w.dtype}+e4m3" if fp8 else w.dtype,
        "data": f"synthetic: seeded N(0,{w.sigma:g}) Q, K, V (numpy PCG64 seed {w.seed}) rounded to {w.dtype}"
                + (", K and V quantised to E4M3 with power-of-two per-tensor scales" if fp8 else "")
                + f", filled lengths uniform in [{w.min_fill:g} Nk, Nk]",
        "config": {"workload": f"{w.name}: decode B={w.B} H={w.H} Nq={w.Nq} cache Nk={w.Nk} d={w.d} "
                               f"{w.dtype}{' queries, E4M3 cache' if fp8 else ''} "
                               f"{'causal' if w.causal else 'non-causal'}",
                   "B": w.B, "H": w.H, "Nq": w.Nq, "Nk": w.Nk, "d": w.d,
                   "seqlens": [int(x) for x in inp["seqlens"]], "parallelism": "single GPU"},
        "workspace_bytes": nb,
        "wall_s_timed": round(wall, 3),
        "roofline": {"bound": "hbm", "kernel": "kv_split + kv_merge (one call)", "achieved": round(achieved, 1),
                     "peak": PEAK_HBM, "unit": "GB/s", "frac": round(achieved / PEAK_HBM, 4),
                     "traffic": load_traffic(w.name, "kv")},
    }
    if not args.no_cpu_baseline and not args.profile:
        out["cpu_baseline"] = cpu_baseline_kv(w, inp, min(args.cpu_seconds, 10.0))
    if args.profile:
        a = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
    print(json.dumps(out), flush=True)


def bench_fwd_only(args, workloads):
    """fa_fwd alone on each workload: one JSON line each with the median time
    of --steps calls (HIP events, after --warmup), TFLOP/s against the dense
    MFMA peak of the dtype and GB/s of compulsory bytes (Q, K, V read once,
    O and LSE written once) against 8 TB/s."""
    import numpy as np
    import torch

    import exact_io_aware_fa2_amd as fa
    import seeded_inputs as si

    dev = torch.device("cuda:0")
    for w in workloads:
        if isinstance(w, si.Fp8Workload):
            bench_fwd_fp8(args, w)
            continue
        tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[w.dtype]
        inp = si.make_workload_inputs(w, backward=False)
        if args.growing:
            # keys scaled up along the sequence (x1 at key 0 to x6 at the last): the row
            # maxima of later key tiles far exceed the first tile's
            grow = (1.0 + 5.0 * np.arange(w.N, dtype=np.float32) / w.N)[None, None, :, None]
            inp["k"] = si.round_to(inp["k"][0] * grow, w.dtype)

        def up(name):
            a = inp[name][1]
            if w.dtype == "bf16":
                return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
            return torch.from_numpy(a).to(dev)

        q, k, v = up("q"), up("k"), up("v")
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
        for _ in range(args.warmup):
            fa.fa_fwd(q, k, v, o, lse, w.scale, w.causal)
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for e0, e1 in evs:
            e0.record()
            fa.fa_fwd(q, k, v, o, lse, w.scale, w.causal)
            e1.record()
        torch.cuda.synchronize()
        ms = float(np.median([a.elapsed_time(b) for a, b in evs]))
        s = {"bf16": 2, "f16": 2, "f32": 4}[w.dtype]
        nbytes = 4 * w.B * w.H * w.N * w.d * s + 4 * w.B * w.H * w.N
        peak = PEAK_MFMA_16BIT if s == 2 else 157.3
        tf = w.fwd_flop() / (ms * 1e-3) / 1e12
        print(json.dumps({"mode": "forward only", "workload": f"{w.name}: B={w.B} H={w.H} N={w.N} d={w.d} {w.dtype} "
                                                              f"{'causal' if w.causal else 'non-causal'}"
                                                              + (" keys growing x1..x6" if args.growing else ""),
                          "median_us": round(ms * 1e3, 2), "TFLOP/s": round(tf, 1),
                          "frac_mfma_peak": round(tf / peak, 4), "mfma_peak": peak,
                          "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1), "frac_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM, 4),
                          "compulsory_bytes": nbytes, "steps": args.steps}), flush=True)
        del q, k, v, o, lse, inp
    if args.profile:
        # the calibration kernel for FETCH_SIZE / WRITE_SIZE counters
        a = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()


PEAK_MFMA_FP8 = 5033.2  # TFLOP/s, MI355X dense fp8 MFMA (twice the 16-bit rate)


def bench_fwd_fp8(args, w):
    """fa_fwd_fp8 on an 8-bit workload: median of --steps calls.  Half of the
    forward's FLOP (S = Q K^T) run on the FP8 matrix cores, half (O = P V) on
    the 16-bit ones, so the peak of the mix is 2 / (1 / fp8 + 1 / bf16)."""
    import numpy as np
    import torch

    import exact_io_aware_fa2_amd as fa
    import seeded_inputs as si

    dev = torch.device("cuda:0")
    inp = si.make_fp8_workload_inputs(w)
    t = {n: torch.from_numpy(inp[n][1]).to(dev) for n in ("q", "k", "v")}
    sc = {n: torch.from_numpy(inp[n + "_scale"]).to(dev) for n in ("q", "k", "v")}
    odt = {"bf16": torch.bfloat16, "f16": torch.float16}[w.out_dtype]
    o = torch.empty((w.B, w.H, w.N, w.d), dtype=odt, device=dev)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)

    def call():
        fa.fa_fwd_fp8(t["q"], t["k"], t["v"], sc["q"], sc["k"], sc["v"], w.granularity, o, lse, w.scale, w.causal)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for e0, e1 in evs:
        e0.record()
        call()
        e1.record()
    torch.cuda.synchronize()
    ms = float(np.median([a.elapsed_time(b) for a, b in evs]))
    tf = w.fwd_flop() / (ms * 1e-3) / 1e12
    mixed = 2.0 / (1.0 / PEAK_MFMA_FP8 + 1.0 / PEAK_MFMA_16BIT)
    nbytes = 3 * w.B * w.H * w.N * w.d + w.B * w.H * w.N * w.d * 2 + 4 * w.B * w.H * w.N
    print(json.dumps({"mode": "forward only, 8-bit inputs", "workload":
                      f"{w.name}: B={w.B} H={w.H} N={w.N} d={w.d} E4M3 q/k/v, {w.granularity} scales, "
                      f"{w.out_dtype} out, {'causal' if w.causal else 'non-causal'}",
                      "median_us": round(ms * 1e3, 2), "TFLOP/s": round(tf, 1),
                      "frac_mixed_peak": round(tf / mixed, 4), "mixed_peak": round(mixed, 1),
                      "frac_fp8_peak": round(tf / PEAK_MFMA_FP8, 4), "fp8_peak": PEAK_MFMA_FP8,
                      "frac_bf16_peak": round(tf / PEAK_MFMA_16BIT, 4),
                      "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1), "compulsory_bytes": nbytes,
                      "steps": args.steps}), flush=True)
    if args.profile:
        a = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()


def bench_varlen(args):
    """A packed variable-length training batch: 16 causal sequences with
    lengths drawn uniformly in [512, 4096] (seed 1008), H=16, d=128, bf16
    (queries = keys per sequence), through fa_fwd_varlen and fa_bwd_varlen.
    TFLOP/s of the per-sequence causal work, sum_b 2 H L_b^2 d forward and
    2.5 times that backward, median of --steps calls of each."""
    import numpy as np
    import torch

    import exact_io_aware_fa2_amd as fa
    import seeded_inputs as si

    rng = np.random.default_rng(1008)
    lens = rng.integers(512, 4097, size=16).tolist()
    H, d = 16, 128
    scale = 1 / np.sqrt(d)
    inp = si.make_varlen_inputs(lens, lens, H, d, "bf16", 1.0, 1008, backward=True)
    dev = torch.device("cuda:0")
    up = lambda n: torch.from_numpy(inp[n][1].view(np.int16)).view(torch.bfloat16).to(dev)
    q, k, v, do = up("q"), up("k"), up("v"), up("do")
    del inp
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((H, q.shape[0]), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    mx = max(lens)
    lib = fa.load_library()
    nb = int(lib.fa_fwd_varlen_workspace_bytes(len(lens), H, mx, mx, d, fa.FA_BF16))
    ws = torch.empty(nb, dtype=torch.uint8, device=dev) if nb else None
    nbb = int(lib.fa_bwd_varlen_workspace_bytes(len(lens), H, q.shape[0], mx, d, fa.FA_BF16))
    wsb = torch.empty(nbb, dtype=torch.uint8, device=dev)
    fwd = lambda: fa.fa_fwd_varlen(q, k, v, cu, cu, o, lse, ws, mx, mx, scale, True)
    bwd = lambda: fa.fa_bwd_varlen(q, k, v, o, lse, do, cu, cu, dq, dk, dv, wsb, mx, mx, scale, True)

    def timed(call):
        for _ in range(args.warmup):
            call()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for e0, e1 in evs:
            e0.record()
            call()
            e1.record()
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in evs]))

    ms_f = timed(fwd)
    ms_b = timed(bwd)
    flop = sum(2.0 * H * L * L * d for L in lens)
    rate = lambda f, ms: f / (ms * 1e-3) / 1e12
    print(json.dumps({"mode": "varlen training", "workload": f"16 packed sequences, lengths {lens}, H={H} d={d} bf16 causal",
                      "fwd_median_us": round(ms_f * 1e3, 1), "fwd_TFLOP/s": round(rate(flop, ms_f), 1),
                      "bwd_median_us": round(ms_b * 1e3, 1), "bwd_TFLOP/s": round(rate(2.5 * flop, ms_b), 1),
                      "fwd_bwd_TFLOP/s": round(rate(3.5 * flop, ms_f + ms_b), 1),
                      "frac_mfma_peak_fwd_bwd": round(rate(3.5 * flop, ms_f + ms_b) / PEAK_MFMA_16BIT, 4),
                      "workspace_bytes": {"fwd": nb, "bwd": nbb}}), flush=True)


def short_n_workloads():
    """Short sequences, small head dimension: B=16 H=16 d=64 bf16 non-causal,
    N = 128, 256, 512, 1024 (seed 1007); where the forward is closest to the
    HBM roofline (arithmetic intensity ~N/2 FLOP per byte)."""
    import seeded_inputs as si
    return [si.Workload(f"S{n}", 16, 16, n, 64, "bf16", False, 1.0, 1007) for n in (128, 256, 512, 1024)]


def ingest_pmc(fetch_csv: str, write_csv: str, workload: str):
    """Counter summary -> profiles/traffic_<workload>.json.

    Each csv holds one counter per dispatch (KiB).  The plain copy kernel of
    COPY_BYTES in the same run calibrates the counter: factor = true bytes /
    counted bytes (read side from FETCH_SIZE, write side from WRITE_SIZE)."""
    import csv

    def per_kernel(path, counter):
        rows = list(csv.DictReader(open(path)))
        vals = {}
        for r in rows:
            if r.get("Counter_Name") != counter:
                continue
            vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return vals

    fetch = per_kernel(fetch_csv, "FETCH_SIZE")
    write = per_kernel(write_csv, "WRITE_SIZE")

    def find(vals, sym):
        ks = [k for k in vals if sym in k]
        if not ks:
            return None
        xs = [x for k in ks for x in vals[k]]
        return sum(xs) / len(xs)

    copy_sym = [k for k in fetch if "copy" in k.lower() or "elementwise" in k.lower()]
    if not copy_sym:
        raise SystemExit("no copy kernel in the counter file; run bench.py --profile")
    # the largest single copy dispatch is the calibration copy (other, small
    # copies of the same kernel, such as uploads, would skew an average)
    copy_f = max(max(fetch[k]) for k in copy_sym) * 1024
    copy_w = max(max(write[k]) for k in write if k in copy_sym) * 1024
    f_fac, w_fac = COPY_BYTES / copy_f, COPY_BYTES / copy_w
    out = {"workload": workload, "copy_calibration": {"true_bytes": COPY_BYTES,
                                                      "fetch_counted": copy_f,
                                                      "write_counted": copy_w,
                                                      "fetch_factor": f_fac, "write_factor": w_fac},
           "kernels": {}}
    for kern, sym in KERNEL_SYMBOLS.items():
        fv, wv = find(fetch, sym), find(write, sym)
        if fv is None or wv is None:
            continue
        out["kernels"][kern] = {"src_sha": src_hash(kern, workload_d(workload)),
                                "fetch_bytes": fv * 1024 * f_fac, "write_bytes": wv * 1024 * w_fac,
                                "bytes_per_launch": fv * 1024 * f_fac + wv * 1024 * w_fac}
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(traffic_file(workload), "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # The MI355X reaches its steady clock only after ~50 ms of sustained load
    # (kernel durations fall ~25% over that time, then stay); the untimed
    # warm-up covers it so that the timed steps measure the steady state.
    ap.add_argument("--warmup", type=int, default=60)
    ap.add_argument("--workload", default="C5")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile", action="store_true")
    ap.add_argument("--serial", action="store_true",
                    help="time the step with all stages in order on one stream (dQ not beside dK/dV)")
    ap.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--varlen", action="store_true",
                    help="time fa_fwd_varlen and fa_bwd_varlen on a packed batch of 16 ragged causal sequences")
    ap.add_argument("--fwd-only", action="store_true",
                    help="time fa_fwd alone on --workload (any of C1..C5, C3d64, C5d128; comma-separated), "
                         "or on the short-sequence sweep with --workload short")
    ap.add_argument("--growing", action="store_true",
                    help="with --fwd-only: keys scaled by 1 + 5 j / N along the sequence (row maxima "
                         "rise after the first key tile)")
    args = ap.parse_args()

    if args.ingest_pmc:
        ingest_pmc(args.ingest_pmc[0], args.ingest_pmc[1], args.workload)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the library runs on one GPU; use --gpus 1 (on several GPUs, "
                                   "heads would shard across them with no communication)"}))
        sys.exit(2)

    import numpy as np
    import torch

    import exact_io_aware_fa2_amd as fa
    import seeded_inputs as si

    fa.load_library()
    if args.varlen:
        bench_varlen(args)
        return
    if args.fwd_only:
        wls = short_n_workloads() if args.workload == "short" else \
            [si.WORKLOADS[n] if n in si.WORKLOADS else si.FP8_WORKLOADS[n] for n in args.workload.split(",")]
        bench_fwd_only(args, wls)
        return
    if args.workload in si.KV_WORKLOADS:
        bench_kvcache(args, si.KV_WORKLOADS[args.workload])
        return
    w = si.WORKLOADS[args.workload]
    if w.dtype == "f32":
        raise SystemExit("the fwd+bwd step needs a 16-bit workload")
    if args.profile:
        # profiled runs keep the stages on one stream, so that each kernel's
        # traced duration is its own (not shared with a concurrent stage)
        args.steps, args.serial = min(args.steps, 20), True
    dev = torch.device("cuda:0")
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16}[w.dtype]
    inp = si.make_workload_inputs(w, backward=True)

    def up(name):
        a = inp[name][1]
        if w.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    q, k, v, do = up("q"), up("k"), up("v"), up("do")
    # the oracle's sample: the first heads of the same draw (float values, [heads, N, d])
    n_cpu_heads = min(w.B * w.H, 64)
    heads_in = {n: inp[n][0].reshape(w.B * w.H, w.N, w.d)[:n_cpu_heads].copy()
                for n in ("q", "k", "v", "do")}
    del inp
    shape = (w.B, w.H, w.N, w.d)
    o = torch.empty(shape, dtype=tdt, device=dev)
    lse = torch.empty(shape[:3], dtype=torch.float32, device=dev)
    dq, dk, dv = (torch.empty(shape, dtype=tdt, device=dev) for _ in range(3))
    ws = torch.empty(fa.fa_bwd_workspace_bytes(*shape, fa.dtype_code(q)), dtype=torch.uint8, device=dev)
    names = ["fwd", "prep", "dkdv", "dq"]

    def step(evs=None):
        if evs is not None:
            evs[0].record()
        fa.fa_fwd(q, k, v, o, lse, w.scale, w.causal)
        if evs is not None:
            evs[1].record()
        fa.fa_bwd_prep(o, do, ws)
        if evs is not None:
            evs[2].record()
        fa.fa_bwd_dkdv(q, k, v, do, lse, ws, dk, dv, w.scale, w.causal)
        if evs is not None:
            evs[3].record()
        fa.fa_bwd_dq(q, k, v, do, lse, ws, dq, w.scale, w.causal)
        if evs is not None:
            evs[4].record()

    # The two gradient stages after fa_bwd_prep are independent (both read the
    # prepared D vector): dQ runs on a second stream (default priority) beside
    # dK/dV, and the main stream joins it before the step ends.
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()

    def step_overlapped():
        fa.fa_fwd(q, k, v, o, lse, w.scale, w.causal)
        fa.fa_bwd_prep(o, do, ws)
        side.wait_stream(main)
        fa.fa_bwd_dkdv(q, k, v, do, lse, ws, dk, dv, w.scale, w.causal)
        with torch.cuda.stream(side):
            fa.fa_bwd_dq(q, k, v, do, lse, ws, dq, w.scale, w.causal)
        main.wait_stream(side)

    run = step if args.serial else step_overlapped
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()

    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    step_evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    for i in range(args.steps):
        step_evs[i].record()
        run()
    step_evs[args.steps].record()
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t_start.elapsed_time(t_end) / args.steps
    step_ms = [step_evs[i].elapsed_time(step_evs[i + 1]) for i in range(args.steps)]

    # per-kernel durations: the same steps with the stages in order on one
    # stream, each between its own events (these times feed the roofline)
    n_k = max(5, min(args.steps, 20))
    for _ in range(2):
        step()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(n_k)]
    for i in range(n_k):
        step(evs[i])
    torch.cuda.synchronize()
    kern_samples = {n: [e[j].elapsed_time(e[j + 1]) for e in evs] for j, n in enumerate(names)}
    kern_ms = {n: float(np.mean(v)) for n, v in kern_samples.items()}
    # secondary: the same steps with the caches cold, a 512 MiB scrub written
    # before each step (outside the timed region)
    scrub = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    flushed = []
    for i in range(min(args.steps, 10)):
        scrub.fill_(i & 0xFF)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        run()
        e1.record()
        torch.cuda.synchronize()
        flushed.append(e0.elapsed_time(e1))
    del scrub
    ms_flushed = float(np.median(flushed))

    flop_step = w.fwd_flop() + w.bwd_flop()
    value = flop_step / (ms_step * 1e-3) / 1e12
    alg = algorithmic(w)
    per_kernel = {}
    for n in names:
        spread = {"ms_median": round(float(np.median(kern_samples[n])), 4),
                  "ms_min": round(float(np.min(kern_samples[n])), 4)}
        if n == "prep":
            per_kernel[n] = {"ms": round(kern_ms[n], 4), "GB/s": round(alg[n] / kern_ms[n] / 1e6, 1), **spread}
        else:
            tf = alg[n] / (kern_ms[n] * 1e-3) / 1e12
            per_kernel[n] = {"ms": round(kern_ms[n], 4), "TFLOP/s": round(tf, 1),
                             "frac": round(tf / PEAK_MFMA_16BIT, 4), **spread}
    dom = max(["fwd", "dkdv", "dq"], key=lambda n: kern_ms[n])
    achieved = alg[dom] / (kern_ms[dom] * 1e-3) / 1e12
    roof = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2), "peak": PEAK_MFMA_16BIT,
            "unit": "TFLOP/s", "frac": round(achieved / PEAK_MFMA_16BIT, 4),
            "traffic": load_traffic(w.name, dom)}

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_median": round(float(np.median(step_ms)), 4),
        "ms_per_step_min": round(float(np.min(step_ms)), 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": f"synthetic: seeded N(0,{w.sigma:g}) Q, K, V, dO (numpy PCG64 seed {w.seed}) rounded to {w.dtype}",
        "config": {"workload": f"{w.name}: fwd+bwd B={w.B} H={w.H} N={w.N} d={w.d} "
                               f"{w.dtype} {'causal' if w.causal else 'non-causal'}",
                   "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal,
                   "parallelism": "single GPU"},
        "frac_of_peak": round(value / PEAK_MFMA_16BIT, 4),
        "flushed": {"ms_per_step": round(ms_flushed, 4),
                    "value": round(flop_step / (ms_flushed * 1e-3) / 1e12, 2),
                    "note": "median of 10 steps, each after a 512 MiB scrub of the caches"},
        "fwd_tflops": round(w.fwd_flop() / (kern_ms["fwd"] * 1e-3) / 1e12, 1),
        "bwd_tflops": round(w.bwd_flop() / ((kern_ms["prep"] + kern_ms["dkdv"] + kern_ms["dq"]) * 1e-3) / 1e12, 1),
        "kernels": per_kernel,
        "wall_s_timed": round(wall, 3),
        "schedule": "stages in order on one stream" if args.serial else
                    "fwd, prep, then dK/dV and dQ on two streams at once",
        "roofline": roof,
    }
    if not args.profile:
        m = measured_mfma_peak()
        m["frac_of_measured_dominant"] = round(achieved / m["TFLOP/s"], 4)
        out["mfma_peak_measured"] = m
    if not args.no_cpu_baseline and not args.profile:
        out["cpu_baseline"] = cpu_baseline(w, heads_in, args.cpu_seconds)
    if args.profile:
        a = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
