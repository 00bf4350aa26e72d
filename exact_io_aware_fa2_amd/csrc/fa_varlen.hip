// Backward of causal self-attention over a packed variable-length batch.
//
// Packed sequences of different lengths are how the method is used in
// training on real corpora (the pages' drop-in use with the usual attention
// interfaces: "FlashAttention-2 (DE)", "Anwendung und Integration in das
// Ökosystem").  The gradient is computed by the square backward kernels
// (fa_bwd's prep, dK/dV and dQ) on a padded copy of the batch:
// sequence b's rows are copied into [B, H, max_len, d] with zero rows after
// its length L_b, the LSE of those rows set to +infinity, and the gradients
// of the first L_b rows copied back.  This is exact, not an approximation:
//   - causal: a real query i < L_b sees keys j <= i < L_b only, never a
//     padded key, so its scores, probabilities and dQ are the sequence's own;
//   - a padded query has dO = 0 and O = 0, so D = dO.O = 0 and dP = 0, and
//     LSE = +infinity makes its probabilities exp(s - LSE) = 0: dS = P (dP - D)
//     = 0 and its terms in dV = P^T dO and dK = dS^T Q vanish.
// The copies are HBM-bound (16 bytes per thread, coalesced rows).  The
// dK/dV and dQ kernels are given the sequence lengths and skip every tile
// that lies wholly past one, so padding costs only the ragged last tiles.
#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {

// Sequence b's start row and length, clamped into the packed tensor and
// max_len (so malformed prefix sums never move an access out of bounds).
__device__ inline void seq_span(const int32_t* cu, int b, int64_t total, int max_len, int& start, int& len) {
  const int64_t s = min(max((int64_t)cu[b], (int64_t)0), total);
  start = (int)s;
  len = (int)min(max((int64_t)cu[b + 1] - s, (int64_t)0), min((int64_t)max_len, total - s));
}

// Packed [total, H, d] <-> padded [B, H, max_len, d] (16-bit elements), one
// thread per 16 bytes of the padded tensor.  To the padded layout: rows past
// the sequence's length are written as zeros.  Back: only rows within it are
// written.
template <bool TO_PADDED>
__global__ __launch_bounds__(256) void varlen_copy_kernel(const uint16_t* __restrict__ src,
                                                          uint16_t* __restrict__ dst,
                                                          const int32_t* __restrict__ cu, int H, int max_len,
                                                          int d, int64_t total, int64_t n_chunks) {
  const int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (x >= n_chunks) return;
  const int cpr = d / 8;
  const int c = (int)(x % cpr);
  const int64_t row = x / cpr;  // (b h) * max_len + r
  const int r = (int)(row % max_len);
  const int bh = (int)(row / max_len);
  const int b = bh / H, h = bh % H;
  int start, len;
  seq_span(cu, b, total, max_len, start, len);
  const size_t padded = (size_t)row * d + 8 * c;
  const size_t packed = ((size_t)(start + r) * H + h) * d + 8 * c;
  if constexpr (TO_PADDED) {
    *(u32x4_t*)(dst + padded) = r < len ? *(const u32x4_t*)(src + packed) : u32x4_t{0u, 0u, 0u, 0u};
  } else {
    if (r < len) *(u32x4_t*)(dst + packed) = *(const u32x4_t*)(src + padded);
  }
}

// LSE packed [H, total] -> padded [B, H, max_len]; rows past a sequence's
// length get +infinity (their probabilities are then exactly 0).  The thread
// of row 0 of head 0 also records the sequence's clamped length.
__global__ __launch_bounds__(256) void varlen_lse_kernel(const float* __restrict__ src, float* __restrict__ dst,
                                                         int32_t* __restrict__ lens,
                                                         const int32_t* __restrict__ cu, int H, int max_len,
                                                         int64_t total, int64_t n) {
  const int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (x >= n) return;
  const int r = (int)(x % max_len);
  const int bh = (int)(x / max_len);
  const int b = bh / H, h = bh % H;
  int start, len;
  seq_span(cu, b, total, max_len, start, len);
  dst[x] = r < len ? src[(size_t)h * total + start + r] : INFINITY;
  if (r == 0 && h == 0) lens[b] = len;
}

hipError_t launch_bwd_varlen(const VarlenBwdArgs& a) {
  const int64_t rows = (int64_t)a.B * a.H * a.max_len;
  const int64_t chunks = rows * (a.d / 8);
  const dim3 grid_c((unsigned)((chunks + 255) / 256)), grid_l((unsigned)((rows + 255) / 256));
  const void* src_in[5] = {a.q, a.k, a.v, a.o, a.dout};
  for (int t = 0; t < 5; ++t) {
    hipLaunchKernelGGL((varlen_copy_kernel<true>), grid_c, dim3(256), 0, a.stream, (const uint16_t*)src_in[t],
                       (uint16_t*)a.pad[t], a.cu, a.H, a.max_len, a.d, a.total, chunks);
  }
  hipLaunchKernelGGL(varlen_lse_kernel, grid_l, dim3(256), 0, a.stream, a.lse, a.lse_pad, a.lens, a.cu, a.H,
                     a.max_len, a.total, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  BwdArgs b{};
  b.q = a.pad[0];
  b.k = a.pad[1];
  b.v = a.pad[2];
  b.o = a.pad[3];
  b.dout = a.pad[4];
  b.lse = a.lse_pad;
  b.dq = a.pad[5];
  b.dk = a.pad[6];
  b.dv = a.pad[7];
  b.dvec = a.dvec;
  b.BH = a.B * a.H;
  b.N = a.max_len;
  b.d = a.d;
  b.scale = a.scale;
  b.c = a.c;
  b.causal = 1;
  b.dtype = a.dtype;
  b.stream = a.stream;
  b.lens = a.lens;  // skip the tiles past each sequence's length
  b.H = a.H;
  e = launch_bwd(b);
  if (e != hipSuccess) return e;
  void* dst_out[3] = {a.dq, a.dk, a.dv};
  for (int t = 0; t < 3; ++t) {
    hipLaunchKernelGGL((varlen_copy_kernel<false>), grid_c, dim3(256), 0, a.stream, (const uint16_t*)a.pad[5 + t],
                       (uint16_t*)dst_out[t], a.cu, a.H, a.max_len, a.d, a.total, chunks);
  }
  return hipGetLastError();
}

}  // namespace fa
