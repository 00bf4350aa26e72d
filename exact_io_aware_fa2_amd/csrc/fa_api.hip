// C-ABI entry points of libfa_mi355x.so: argument checks, then dispatch to the
// kernel launchers.  Declarations and the contract are in include/fa.h.
#include <float.h>
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "fa.h"
#include "fa_launch.hpp"

namespace fa {

int device_cu_count(hipStream_t stream) {
  constexpr int kDevices = 64;
  static std::atomic<int> cached[kDevices];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (stream && hipStreamGetDevice(stream, &dev) != hipSuccess) return 0;
  if (dev < 0 || dev >= kDevices) return 0;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 0) n = 0;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace fa

namespace {

// One head of one tensor (N x d elements of up to 4 bytes) must stay below
// 2^31 bytes: kernels address within a head with 32-bit byte offsets.
constexpr int64_t kMaxN = int64_t(1) << 22;
constexpr int64_t kMaxWorkgroups = (int64_t(1) << 24) - 1;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shape checks shared by both passes.  Workgroup counts are bounded for the
// smallest query tile any kernel uses (32 rows).
int check_shape(int64_t B, int64_t H, int64_t N, int64_t d) {
  if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
  if (N > kMaxN) return FA_ERR_SHAPE;
  if (B > INT32_MAX / H) return FA_ERR_SHAPE;
  const int64_t bh = B * H;
  if (bh * ((N + 31) / 32) > kMaxWorkgroups) return FA_ERR_SHAPE;
  if (d != 32 && d != 64 && d != 96 && d != 128 && d != 256) return FA_ERR_HEADDIM;
  return FA_OK;
}

// The backward takes the same head dimensions (d = 256 on its own kernels),
// with the rows a 64-row tile reaches past a head's last row within 32-bit
// byte offsets.
int check_shape_bwd(int64_t B, int64_t H, int64_t N, int64_t d) {
  const int st = check_shape(B, H, N, d);
  if (st != FA_OK) return st;
  if (d == 256 && (N + 64) * d * 2 >= (int64_t(1) << 31)) return FA_ERR_SHAPE;
  return FA_OK;
}

fa::KvLayout dense_layout(int64_t H, int64_t Nq, int64_t Nk, int64_t d);

// Head dimensions the square kernels take through the general layout: 32 and
// 96 run on the d = 64 and d = 128 kernels with the columns past d read as
// zeros and never stored.
bool padded_d(int64_t d) { return d == 32 || d == 96; }

// Contiguous [B, H, N, d] tensors and [B, H, N] LSE as a general layout.
fa::GenLayout dense_layout_g(int64_t H, int64_t N, int64_t d) {
  fa::GenLayout g{};
  const fa::Strides s{H * N * d, N * d, d};
  g.q = g.k = g.v = g.o = g.dout = g.dq = g.dk = g.dv = s;
  g.l_sb = H * N;
  g.l_sh = N;
  g.H = (int)H;
  g.dr = (int)d;
  return g;
}

// Packed [total, H, d] tensors (sequence b's rows from cu[b]), LSE [H, total_q].
fa::GenLayout packed_layout_g(int64_t H, int64_t d, const int32_t* cu_q, const int32_t* cu_k, int64_t total_q,
                              int64_t total_k) {
  fa::GenLayout g{};
  const fa::Strides s{0, d, H * d};
  g.q = g.k = g.v = g.o = g.dout = g.dq = g.dk = g.dv = s;
  g.cu_q = cu_q;
  g.cu_k = cu_k;
  g.total_q = total_q;
  g.total_k = total_k;
  g.l_sb = 0;
  g.l_sh = total_q;
  g.H = (int)H;
  g.dr = (int)d;
  return g;
}

// Caller strides (elements; batch, head, row per tensor): non-negative, every
// row start 16-byte aligned (multiples of 8 elements), output rows not
// overlapping (row stride >= d), and the rows a kernel reaches from a head's
// first row (N plus a 512-row prefetch margin) within 32-bit byte offsets.
int check_strides(const int64_t* st, int ntensors, const bool* output, int64_t N, int64_t d) {
  for (int t = 0; t < ntensors; ++t) {
    for (int j = 0; j < 3; ++j) {
      const int64_t x = st[3 * t + j];
      if (x < 0) return FA_ERR_SHAPE;
      if (x % 8) return FA_ERR_ALIGN;
    }
    const int64_t sr = st[3 * t + 2];
    if (sr < d && (output[t] || N > 1)) return FA_ERR_SHAPE;
    if ((N + 512) * sr * 2 >= (int64_t(1) << 31)) return FA_ERR_SHAPE;
  }
  return FA_OK;
}

// The scale must be finite, and so must the factor the kernels use,
// |scale| * log2(e) (it overflows to infinity above about 2.4e38).
int check_scale(float scale) {
  if (!isfinite(scale)) return FA_ERR_SCALE;
  if (!isfinite(fabsf(scale) * fa::kLog2eHost)) return FA_ERR_SCALE;
  return FA_OK;
}

// Factor turning a raw score into log2 units, |scale| * log2(e) (a negative
// scale negates one operand of the scores instead: neg_mask).  The kernels
// mask a score by setting it to -inf before this multiplication, so the factor
// must not be zero: scale = 0 uses the smallest normal float instead, which
// leaves every finite score's contribution at 2^0 = 1 (uniform weights) and
// keeps masked scores at -inf.
float exp2_factor(float scale) {
  const float c = fabsf(scale) * fa::kLog2eHost;
  return c < FLT_MIN ? FLT_MIN : c;
}

// Softmax of s q.k with s < 0 is softmax of |s| (-q).k: the forward kernels,
// which keep a running maximum of the raw scores, flip the sign bits of the
// queries' 16-bit elements under this mask and use |s| for the exponent.
uint32_t neg_mask(float scale) { return scale < 0.0f ? 0x80008000u : 0u; }

// The backward forms P = exp2(q.k c - LSE log2 e) with no maximum: it takes
// the factor with the scale's sign (a negative zero counts as zero).
float exp2_factor_signed(float scale) {
  const float c = exp2_factor(scale);
  return scale < 0.0f ? -c : c;
}

}  // namespace

extern "C" {

int fa_abi_version(void) { return FA_ABI_VERSION; }

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "null pointer argument";
    case FA_ERR_SHAPE: return "invalid shape (B, H, N must be >= 1 and within limits)";
    case FA_ERR_HEADDIM: return "unsupported head dimension for this entry point";
    case FA_ERR_DTYPE: return "unsupported dtype";
    case FA_ERR_ALIGN: return "data pointer not 16-byte aligned";
    case FA_ERR_SCALE: return "scale must be finite (and an 8-bit cache's scales > 0)";
    case FA_ERR_WORKSPACE: return "workspace missing or too small";
    case FA_ERR_HIP: return "HIP runtime error";
    case FA_ERR_SCRATCH: return "sizes exceed the static scratch of fa_bwd_noalloc";
    default: return "unknown status";
  }
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
           int64_t H, int64_t N, int64_t d, float scale, int causal, int dtype, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  int st = check_shape(B, H, N, d);
  if (st != FA_OK) return st;
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
  if (dtype == FA_F32 && d != 64 && d != 128) return FA_ERR_HEADDIM;  // float32: d = 64 or 128
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_ALIGN;
  st = check_scale(scale);
  if (st != FA_OK) return st;
  // d = 256: the rows a workgroup and its prefetch reach from a head's first
  // row stay within 32-bit byte offsets
  if (d == 256 && (N + 64) * d * 2 >= (int64_t(1) << 31)) return FA_ERR_SHAPE;

  fa::FwdArgs a;
  a.general = padded_d(d);
  a.g = dense_layout_g(H, N, d);
  a.g.qneg = neg_mask(scale);
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.BH = (int)(B * H);
  a.N = (int)N;
  a.d = (int)d;
  a.c = exp2_factor(scale);
  a.causal = causal != 0;
  a.dtype = dtype;
  a.stream = (hipStream_t)stream;
  return fa::launch_fwd(a) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d, int dtype) {
  if (check_shape_bwd(B, H, N, d) != FA_OK) return 0;
  if (dtype != FA_F16 && dtype != FA_BF16) return 0;
  return (size_t)(B * H * N) * sizeof(float);
}

}  // extern "C"

namespace {

// Checks shared by the backward entry points; fills `a` on success.  `ptrs`
// lists the data pointers the entry point takes (all required, 16-byte aligned).
int bwd_common(fa::BwdArgs& a, const void* const* ptrs, int nptrs, const void* workspace,
               size_t workspace_bytes, int64_t B, int64_t H, int64_t N, int64_t d, float scale,
               int causal, int dtype, void* stream) {
  for (int i = 0; i < nptrs; ++i)
    if (!ptrs[i]) return FA_ERR_NULL;
  int st = check_shape_bwd(B, H, N, d);
  if (st != FA_OK) return st;
  if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
  for (int i = 0; i < nptrs; ++i)
    if (!aligned16(ptrs[i])) return FA_ERR_ALIGN;
  st = check_scale(scale);
  if (st != FA_OK) return st;
  if (!workspace || workspace_bytes < fa_bwd_workspace_bytes(B, H, N, d, dtype))
    return FA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FA_ERR_ALIGN;
  a = fa::BwdArgs{};
  a.dvec = (float*)workspace;
  a.BH = (int)(B * H);
  a.Nq = a.Nk = (int)N;
  a.d = (int)d;
  a.general = padded_d(d);
  a.g = dense_layout_g(H, N, d);
  a.scale = scale;
  a.c = exp2_factor_signed(scale);
  a.causal = causal != 0;
  a.dtype = dtype;
  a.stream = (hipStream_t)stream;
  return FA_OK;
}

int status_of(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

}  // namespace

extern "C" {

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dout, void* dq, void* dk, void* dv, void* workspace,
           size_t workspace_bytes, int64_t B, int64_t H, int64_t N, int64_t d, float scale,
           int causal, int dtype, void* stream) {
  const void* ptrs[] = {q, k, v, o, lse, dout, dq, dk, dv};
  fa::BwdArgs a;
  const int st = bwd_common(a, ptrs, 9, workspace, workspace_bytes, B, H, N, d, scale, causal,
                            dtype, stream);
  if (st != FA_OK) return st;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  return status_of(fa::launch_bwd(a));
}

int fa_bwd_prep(const void* o, const void* dout, void* workspace, size_t workspace_bytes,
                int64_t B, int64_t H, int64_t N, int64_t d, int dtype, void* stream) {
  const void* ptrs[] = {o, dout};
  fa::BwdArgs a;
  const int st = bwd_common(a, ptrs, 2, workspace, workspace_bytes, B, H, N, d, 0.0f, 0, dtype,
                            stream);
  if (st != FA_OK) return st;
  a.o = o;
  a.dout = dout;
  return status_of(fa::launch_bwd_stage(a, fa::BWD_PREP));
}

int fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                const void* workspace, size_t workspace_bytes, void* dk, void* dv, int64_t B,
                int64_t H, int64_t N, int64_t d, float scale, int causal, int dtype,
                void* stream) {
  const void* ptrs[] = {q, k, v, dout, lse, dk, dv};
  fa::BwdArgs a;
  const int st = bwd_common(a, ptrs, 7, workspace, workspace_bytes, B, H, N, d, scale, causal,
                            dtype, stream);
  if (st != FA_OK) return st;
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = dout;
  a.lse = lse;
  a.dk = dk;
  a.dv = dv;
  return status_of(fa::launch_bwd_stage(a, fa::BWD_DKDV));
}

int fa_bwd_dq(const void* q, const void* k, const void* v, const void* dout, const float* lse,
              const void* workspace, size_t workspace_bytes, void* dq, int64_t B, int64_t H,
              int64_t N, int64_t d, float scale, int causal, int dtype, void* stream) {
  const void* ptrs[] = {q, k, v, dout, lse, dq};
  fa::BwdArgs a;
  const int st = bwd_common(a, ptrs, 6, workspace, workspace_bytes, B, H, N, d, scale, causal,
                            dtype, stream);
  if (st != FA_OK) return st;
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  return status_of(fa::launch_bwd_stage(a, fa::BWD_DQ));
}

}  // extern "C"

namespace {

// Checks of the split-key entry points' sizes: the query and cache lengths
// are bounded like N, the split kernel's workgroup count (four wavefronts
// each) like every other grid; head dimensions 32, 64 and 128.
int check_kv_shape(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d) {
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1) return FA_ERR_SHAPE;
  if (Nq > kMaxN || Nk > kMaxN) return FA_ERR_SHAPE;
  if (B > INT32_MAX / H) return FA_ERR_SHAPE;
  const int64_t bh = B * H;
  if (bh * Nq > INT32_MAX) return FA_ERR_SHAPE;
  const fa::KvPlan p = fa::kv_plan(bh, Nq, Nk, d);
  if ((bh * p.n_qb * p.n_splits + 3) / 4 > kMaxWorkgroups) return FA_ERR_SHAPE;
  if (d != 32 && d != 64 && d != 128 && d != 256) return FA_ERR_HEADDIM;
  return FA_OK;
}

// [B, H, N, d] queries and outputs, [B, H, Nk, d] caches, [B, H, Nq] LSE.
fa::KvLayout dense_layout(int64_t H, int64_t Nq, int64_t Nk, int64_t d) {
  fa::KvLayout l{};
  l.q_sb = l.o_sb = H * Nq * d;
  l.q_sh = l.o_sh = Nq * d;
  l.q_sr = l.o_sr = d;
  l.c_sb = l.v_sb = H * Nk * d;
  l.c_sh = l.v_sh = Nk * d;
  l.c_sr = l.v_sr = d;
  l.l_sb = H * Nq;
  l.l_sh = Nq;
  return l;
}

}  // namespace

extern "C" {

size_t fa_fwd_kvcache_workspace_bytes(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                                      int dtype) {
  if (check_kv_shape(B, H, Nq, Nk, d) != FA_OK) return 0;
  if (dtype != FA_F16 && dtype != FA_BF16) return 0;
  return fa::kv_workspace_bytes(B * H, Nq, Nk, d);
}

int fa_fwd_kvcache(const void* q, const void* k_cache, const void* v_cache, const int32_t* seqlens_k,
                   void* o, float* lse, void* workspace, size_t workspace_bytes, int64_t B, int64_t H,
                   int64_t Nq, int64_t Nk, int64_t d, float scale, int causal, int dtype, void* stream) {
  if (!q || !k_cache || !v_cache || !o || !lse) return FA_ERR_NULL;
  int st = check_kv_shape(B, H, Nq, Nk, d);
  if (st != FA_OK) return st;
  if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_ALIGN;
  if (seqlens_k && (reinterpret_cast<uintptr_t>(seqlens_k) & 3u) != 0) return FA_ERR_ALIGN;
  st = check_scale(scale);
  if (st != FA_OK) return st;
  const size_t need = fa::kv_workspace_bytes(B * H, Nq, Nk, d);
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return FA_ERR_ALIGN;
  }
  fa::KvArgs a;
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.seqlens = seqlens_k;
  a.o = o;
  a.lse = lse;
  a.workspace = need > 0 ? workspace : nullptr;
  a.lay = dense_layout(H, Nq, Nk, d);
  a.lay.qneg = neg_mask(scale);
  a.H = (int)H;
  a.BH = (int)(B * H);
  a.Nq = (int)Nq;
  a.Nk = (int)Nk;
  a.d = (int)d;
  a.c = exp2_factor(scale);
  a.v_scale = 1.0f;
  a.fp8_cache = 0;
  a.causal = causal != 0;
  a.dtype = dtype;
  a.stream = (hipStream_t)stream;
  return status_of(fa::launch_fwd_kvcache(a));
}

int fa_fwd_kvcache_fp8(const void* q, const void* k_cache, const void* v_cache, float k_scale,
                       float v_scale, const int32_t* seqlens_k, void* o, float* lse, void* workspace,
                       size_t workspace_bytes, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                       float scale, int causal, int dtype, void* stream) {
  if (!q || !k_cache || !v_cache || !o || !lse) return FA_ERR_NULL;
  int st = check_kv_shape(B, H, Nq, Nk, d);
  if (st != FA_OK) return st;
  if (d == 256) return FA_ERR_HEADDIM;  // the 8-bit cache: d = 32, 64, 128
  if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_ALIGN;
  if (seqlens_k && (reinterpret_cast<uintptr_t>(seqlens_k) & 3u) != 0) return FA_ERR_ALIGN;
  st = check_scale(scale);
  if (st != FA_OK) return st;
  if (!isfinite(k_scale) || !isfinite(v_scale) || !(k_scale > 0.0f) || !(v_scale > 0.0f)) return FA_ERR_SCALE;
  // the K scale joins the exponent factor: the product must stay finite
  if (!isfinite(scale * k_scale * fa::kLog2eHost)) return FA_ERR_SCALE;
  const size_t need = fa::kv_workspace_bytes(B * H, Nq, Nk, d);
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return FA_ERR_ALIGN;
  }
  fa::KvArgs a;
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.seqlens = seqlens_k;
  a.o = o;
  a.lse = lse;
  a.workspace = need > 0 ? workspace : nullptr;
  a.lay = dense_layout(H, Nq, Nk, d);
  a.lay.qneg = neg_mask(scale);
  a.H = (int)H;
  a.BH = (int)(B * H);
  a.Nq = (int)Nq;
  a.Nk = (int)Nk;
  a.d = (int)d;
  // scores are q . (k_scale * code): the K scale joins the exponent factor
  a.c = exp2_factor(scale * k_scale);
  a.v_scale = v_scale;
  a.fp8_cache = 1;
  a.causal = causal != 0;
  a.dtype = dtype;
  a.stream = (hipStream_t)stream;
  return status_of(fa::launch_fwd_kvcache(a));
}

}  // extern "C"

extern "C" {

int64_t fa_probe_mfma_bf16(int64_t workgroups, int64_t iters, void* stream) {
  if (workgroups < 1 || workgroups > kMaxWorkgroups || iters < 1 || iters > INT32_MAX) return -FA_ERR_SHAPE;
  // the FLOP count (workgroups * iters * 2^19) must fit in int64
  if (workgroups * iters > (INT64_MAX >> 19)) return -FA_ERR_SHAPE;
  if (fa::launch_mfma_peak((int)workgroups, (int)iters, (hipStream_t)stream) != hipSuccess) return -FA_ERR_HIP;
  return workgroups * 4 * iters * 4 * 32768;
}

}  // extern "C"

extern "C" {

size_t fa_fwd_varlen_workspace_bytes(int64_t B, int64_t H, int64_t max_q, int64_t max_k, int64_t d,
                                     int dtype) {
  return fa_fwd_kvcache_workspace_bytes(B, H, max_q, max_k, d, dtype);
}

int fa_fwd_varlen(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                  const int32_t* cu_seqlens_k, void* o, float* lse, void* workspace, size_t workspace_bytes,
                  int64_t B, int64_t H, int64_t total_q, int64_t total_k, int64_t max_q, int64_t max_k,
                  int64_t d, float scale, int causal, int dtype, void* stream) {
  if (!q || !k || !v || !cu_seqlens_q || !cu_seqlens_k || !o || !lse) return FA_ERR_NULL;
  // d = 96: the square kernels only (self-attention below); the split-key kernel takes 32, 64, 128
  int st = check_kv_shape(B, H, max_q, max_k, d == 96 ? 128 : d);
  if (st != FA_OK) return st;
  if (total_q < 1 || total_k < 1 || total_q > INT32_MAX || total_k > INT32_MAX) return FA_ERR_SHAPE;
  // one sequence's rows must stay within 32-bit byte offsets of its first row
  if (max_q * H * d * 2 >= (int64_t(1) << 31) || max_k * H * d * 2 >= (int64_t(1) << 31)) return FA_ERR_SHAPE;
  if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return FA_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(cu_seqlens_q) & 3u) || (reinterpret_cast<uintptr_t>(cu_seqlens_k) & 3u))
    return FA_ERR_ALIGN;
  st = check_scale(scale);
  if (st != FA_OK) return st;
  // Self-attention (one prefix-sum array for queries and keys): the square
  // forward kernels, reading and writing the packed rows in place, when the
  // rows a 256-row tile and its prefetch reach stay within 32-bit byte offsets
  // of a sequence's first row.
  if (cu_seqlens_q == cu_seqlens_k && total_q == total_k && max_q == max_k &&
      (max_q + 512) * H * d * 2 < (int64_t(1) << 31) && total_q * H <= INT32_MAX) {
    fa::FwdArgs f;
    f.q = q;
    f.k = k;
    f.v = v;
    f.o = o;
    f.lse = lse;
    f.BH = (int)(B * H);
    f.N = (int)max_q;
    f.d = (int)d;
    f.c = exp2_factor(scale);
    f.causal = causal != 0;
    f.dtype = dtype;
    f.stream = (hipStream_t)stream;
    f.general = true;
    f.g = packed_layout_g(H, d, cu_seqlens_q, cu_seqlens_k, total_q, total_k);
    f.g.qneg = neg_mask(scale);
    return status_of(fa::launch_fwd(f));
  }
  if (d == 96) return FA_ERR_HEADDIM;
  const size_t need = fa::kv_workspace_bytes(B * H, max_q, max_k, d);
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return FA_ERR_ALIGN;
  }
  fa::KvArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.seqlens = nullptr;
  a.o = o;
  a.lse = lse;
  a.workspace = need > 0 ? workspace : nullptr;
  fa::KvLayout l{};
  l.q_sb = l.o_sb = 0;  // packed [total, H, d]: sequence b starts at row cu[b]
  l.q_sh = l.o_sh = d;
  l.q_sr = l.o_sr = H * d;
  l.c_sb = l.v_sb = 0;
  l.c_sh = l.v_sh = d;
  l.c_sr = l.v_sr = H * d;
  l.l_sb = 0;  // [H, total_q]
  l.l_sh = total_q;
  l.cu_q = cu_seqlens_q;
  l.cu_k = cu_seqlens_k;
  l.total_q = total_q;
  l.total_k = total_k;
  l.qneg = neg_mask(scale);
  a.lay = l;
  a.H = (int)H;
  a.BH = (int)(B * H);
  a.Nq = (int)max_q;
  a.Nk = (int)max_k;
  a.d = (int)d;
  a.c = exp2_factor(scale);
  a.v_scale = 1.0f;
  a.fp8_cache = 0;
  a.causal = causal != 0;
  a.dtype = dtype;
  a.stream = (hipStream_t)stream;
  return status_of(fa::launch_fwd_kvcache(a));
}

}  // extern "C"

extern "C" {

size_t fa_bwd_varlen_workspace_bytes(int64_t B, int64_t H, int64_t total_q, int64_t max_q, int64_t d,
                                     int dtype) {
  if (check_shape_bwd(B, H, max_q, d) != FA_OK) return 0;
  if (total_q < 1 || total_q > INT32_MAX || total_q * H > INT32_MAX) return 0;
  if (dtype != FA_F16 && dtype != FA_BF16) return 0;
  return (size_t)(total_q * H) * sizeof(float);
}

int fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse,
                  const void* dout, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, void* dq, void* dk,
                  void* dv, void* workspace, size_t workspace_bytes, int64_t B, int64_t H, int64_t total_q,
                  int64_t total_k, int64_t max_q, int64_t max_k, int64_t d, float scale, int causal, int dtype,
                  void* stream) {
  const void* ptrs[] = {q, k, v, o, lse, dout, dq, dk, dv};
  for (const void* p : ptrs)
    if (!p) return FA_ERR_NULL;
  if (!cu_seqlens_q || !cu_seqlens_k) return FA_ERR_NULL;
  int st = check_shape_bwd(B, H, max_q, d);
  if (st != FA_OK) return st;
  st = check_shape_bwd(B, H, max_k, d);
  if (st != FA_OK) return st;
  if (total_q < 1 || total_q > INT32_MAX || total_q * H > INT32_MAX) return FA_ERR_SHAPE;
  if (total_k < 1 || total_k > INT32_MAX || total_k * H > INT32_MAX) return FA_ERR_SHAPE;
  // one sequence's rows, and the rows past them a tile and its prefetch
  // reach, stay within 32-bit byte offsets of its first row
  if ((max_q + 512) * H * d * 2 >= (int64_t(1) << 31) || (max_k + 512) * H * d * 2 >= (int64_t(1) << 31))
    return FA_ERR_SHAPE;
  if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
  for (const void* p : ptrs)
    if (!aligned16(p)) return FA_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(cu_seqlens_q) & 3u) || (reinterpret_cast<uintptr_t>(cu_seqlens_k) & 3u))
    return FA_ERR_ALIGN;
  st = check_scale(scale);
  if (st != FA_OK) return st;
  if (!workspace || workspace_bytes < fa_bwd_varlen_workspace_bytes(B, H, total_q, max_q, d, dtype))
    return FA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FA_ERR_ALIGN;

  fa::BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dvec = (float*)workspace;  // D_i, [H, total_q] like the LSE
  a.BH = (int)(B * H);
  a.Nq = (int)max_q;
  a.Nk = (int)max_k;
  a.d = (int)d;
  a.scale = scale;
  a.c = exp2_factor_signed(scale);
  a.causal = causal != 0;
  a.dtype = dtype;
  a.stream = (hipStream_t)stream;
  a.general = true;
  a.g = packed_layout_g(H, d, cu_seqlens_q, cu_seqlens_k, total_q, total_k);
  return status_of(fa::launch_bwd(a));
}

}  // extern "C"

extern "C" {

int fa_fwd_fp8(const void* q8, const void* k8, const void* v8, const float* q_scale, const float* k_scale,
               const float* v_scale, int scale_granularity, void* o, float* lse, int64_t B, int64_t H, int64_t N,
               int64_t d, float scale, int causal, int dtype, void* stream) {
  if (!q8 || !k8 || !v8 || !q_scale || !k_scale || !v_scale || !o || !lse) return FA_ERR_NULL;
  int st = check_shape(B, H, N, d);
  if (st != FA_OK) return st;
  if (d != 128) return FA_ERR_HEADDIM;
  if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
  if (scale_granularity != FA_SCALE_TENSOR && scale_granularity != FA_SCALE_BLOCK) return FA_ERR_DTYPE;
  if (!aligned16(q8) || !aligned16(k8) || !aligned16(v8) || !aligned16(o) || !aligned16(lse)) return FA_ERR_ALIGN;
  const void* sp[] = {q_scale, k_scale, v_scale};
  for (const void* p : sp)
    if (reinterpret_cast<uintptr_t>(p) & 3u) return FA_ERR_ALIGN;
  st = check_scale(scale);
  if (st != FA_OK) return st;
  fa::Fp8Args a;
  a.q = q8;
  a.k = k8;
  a.v = v8;
  a.q_scale = q_scale;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.per_block = scale_granularity == FA_SCALE_BLOCK;
  a.o = o;
  a.lse = lse;
  a.BH = (int)(B * H);
  a.N = (int)N;
  a.d = (int)d;
  a.c = exp2_factor(scale);
  a.qneg = scale < 0.0f;
  a.causal = causal != 0;
  a.dtype = dtype;
  a.stream = (hipStream_t)stream;
  return status_of(fa::launch_fwd_fp8(a));
}

}  // extern "C"

// ------------------------------------------------------------ fa_bwd_noalloc
//
// fa_bwd without a caller workspace, for callers that cannot allocate.  Its
// one scratch array (D_i = dO_i . O_i, one float per query row) is this
// file-scope device array; every GPU holds its own copy at its own address.
// Host code never passes the array's name to a kernel (on the host it is
// only a stand-in symbol): the device address is looked up once per device,
// with that device current, and kept in kScratchPtr.

namespace {

constexpr size_t kScratchBytes = size_t(16) << 20;  // 16 MiB: B * H * N <= 4194304 rows
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, NULL until looked up

// Device address of `scratch` on the device the work runs on (the stream's
// device; the current device for the NULL stream), looked up on the first
// call on that device with it current (the caller's current device is
// restored afterwards).
void* scratch_ptr(hipStream_t stream, int* status) {
  *status = FA_ERR_HIP;
  int cur = -1, dev = -1;
  if (hipGetDevice(&cur) != hipSuccess) return nullptr;
  dev = cur;
  if (stream && hipStreamGetDevice(stream, &dev) != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return nullptr;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return nullptr;
    if (e != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  *status = FA_OK;
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

size_t fa_bwd_noalloc_max_rows(void) { return kScratchBytes / sizeof(float); }

int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t N,
                   int64_t d, float scale, int causal, int dtype, void* stream) {
  const void* ptrs[] = {q, k, v, o, lse, dout, dq, dk, dv};
  for (const void* p : ptrs)
    if (!p) return FA_ERR_NULL;
  int st = check_shape_bwd(B, H, N, d);
  if (st != FA_OK) return st;
  if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
  for (const void* p : ptrs)
    if (!aligned16(p)) return FA_ERR_ALIGN;
  st = check_scale(scale);
  if (st != FA_OK) return st;
  if ((size_t)(B * H * N) * sizeof(float) > kScratchBytes) return FA_ERR_SCRATCH;
  void* ws = scratch_ptr((hipStream_t)stream, &st);
  if (st != FA_OK) return st;
  // the D_i rows are written by the first stage before the others read them:
  // nothing in the scratch has to start at zero
  return fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, ws, kScratchBytes, B, H, N, d, scale, causal, dtype,
                stream);
}

}  // extern "C"

extern "C" {

int fa_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse, const int64_t* strides,
                   int64_t B, int64_t H, int64_t N, int64_t d, float scale, int causal, int dtype, void* stream) {
  if (!q || !k || !v || !o || !lse || !strides) return FA_ERR_NULL;
  int st = check_shape(B, H, N, d);
  if (st != FA_OK) return st;
  if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return FA_ERR_ALIGN;
  const bool out[4] = {false, false, false, true};
  st = check_strides(strides, 4, out, N, d);
  if (st != FA_OK) return st;
  st = check_scale(scale);
  if (st != FA_OK) return st;
  fa::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.BH = (int)(B * H);
  a.N = (int)N;
  a.d = (int)d;
  a.c = exp2_factor(scale);
  a.causal = causal != 0;
  a.dtype = dtype;
  a.stream = (hipStream_t)stream;
  a.general = true;
  a.g = dense_layout_g(H, N, d);
  a.g.qneg = neg_mask(scale);
  fa::Strides* t[4] = {&a.g.q, &a.g.k, &a.g.v, &a.g.o};
  for (int i = 0; i < 4; ++i) *t[i] = fa::Strides{strides[3 * i], strides[3 * i + 1], strides[3 * i + 2]};
  return status_of(fa::launch_fwd(a));
}

int fa_bwd_strided(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                   void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, const int64_t* strides,
                   int64_t B, int64_t H, int64_t N, int64_t d, float scale, int causal, int dtype, void* stream) {
  if (!strides) return FA_ERR_NULL;
  const void* ptrs[] = {q, k, v, o, lse, dout, dq, dk, dv};
  fa::BwdArgs a;
  int st = bwd_common(a, ptrs, 9, workspace, workspace_bytes, B, H, N, d, scale, causal, dtype, stream);
  if (st != FA_OK) return st;
  const bool out[8] = {false, false, false, false, false, true, true, true};
  st = check_strides(strides, 8, out, N, d);
  if (st != FA_OK) return st;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.general = true;
  fa::Strides* t[8] = {&a.g.q, &a.g.k, &a.g.v, &a.g.o, &a.g.dout, &a.g.dq, &a.g.dk, &a.g.dv};
  for (int i = 0; i < 8; ++i) *t[i] = fa::Strides{strides[3 * i], strides[3 * i + 1], strides[3 * i + 2]};
  return status_of(fa::launch_bwd(a));
}

}  // extern "C"
