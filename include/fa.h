/* fa.h - C ABI of the MI355X (gfx950) exact attention library, libfa_mi355x.so.
 *
 * The library computes exact scaled-dot-product attention
 *
 *     O = softmax(scale * Q K^T [+ causal mask]) V,   LSE_i = ln sum_j exp(scale * q_i . k_j)
 *
 * in the tiled, fused, IO-aware way the pages describe: the N x N score and
 * probability matrices are never written to device memory, the row
 * normalisation is accumulated on the fly, only the per-row log-sum-exp is
 * stored, and the backward pass recomputes the scores instead of loading them.
 *   - Exactness (same result as the usual computation up to rounding):
 *     "FlashAttention" lexicon, "Methodische Grundlagen", paragraph
 *     "Exaktheit"; "FlashAttention" glossary, "Wo es verwechselt wird".
 *   - Tiling, fusion, running normalisation, recomputation: "FlashAttention"
 *     lexicon, "Methodische Grundlagen".
 *   - Work split (one head over many compute units; rows split across
 *     wavefronts; few non-matmul operations): "FlashAttention-2 (DE)",
 *     "Technische Architektur und Funktionsprinzipien", items 1-3.
 *   - The mask and the gradient formulas are not on the pages; causal means
 *     key j is visible to query i iff j <= i (top-left aligned, equal query and
 *     key lengths), and the gradient is the chain rule through the softmax.
 *
 * Conventions shared by every entry point (unless its own comment says
 * otherwise: the key/value-cache and variable-length entry points take other
 * layouts and also d = 32, the probe computes nothing)
 *   Layout     q, k, v, o, dout, dq, dk, dv: contiguous row-major [B, H, N, d]
 *              arrays of the element type `dtype` (the *_strided entry points:
 *              any strides).  lse: contiguous [B, H, N] float32.  Head
 *              dimension d: 32, 64, 96, 128 or 256 for 16-bit types (32 and
 *              96 run on the 64 / 128 kernels with the missing columns read
 *              as zeros; the backward runs 256 on kernels of its own); 64
 *              or 128 for float32.
 *   Memory     All data pointers are DEVICE pointers owned by the caller.  The
 *              library allocates no device memory and keeps no pointer after a
 *              call returns.  Every tensor pointer must be 16-byte aligned
 *              (int32 length arrays: 4-byte).
 *   Streams    `stream` is a hipStream_t (NULL = the default stream).  Calls
 *              only enqueue work on it and return; they never synchronise and
 *              never copy to the host.  Concurrent calls on different streams
 *              are safe (the library has no mutable global state).
 *   Numerics   Matrix products multiply in the input precision and accumulate
 *              in float32; outputs have the input type (LSE: float32).  The
 *              probabilities that multiply V are rounded to the input type
 *              (round to nearest even); the float32 path keeps them in float32.
 *   Errors     Return FA_OK (0) or a positive fa_status (the probe: a negated
 *              one).  Arguments are checked
 *              before any device call; on an argument error nothing is
 *              enqueued.  FA_ERR_HIP means the HIP runtime refused the launch
 *              (no device, invalid stream, ...); hipGetLastError() then holds
 *              the runtime's code.  The library never aborts or prints.
 */
#ifndef FA_MI355X_H
#define FA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_ABI_VERSION 10

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = 1,      /* a required pointer is NULL */
  FA_ERR_SHAPE = 2,     /* B, H or N < 1, N > 2^22, or B*H*ceil(N/32) >= 2^24 */
  FA_ERR_HEADDIM = 3,   /* d not taken by this entry point (see each one) */
  FA_ERR_DTYPE = 4,     /* unknown dtype, or a dtype this entry point does not take */
  FA_ERR_ALIGN = 5,     /* a data pointer is not 16-byte aligned */
  FA_ERR_SCALE = 6,     /* scale is NaN or infinite, or |scale| * log2(e) overflows */
  FA_ERR_WORKSPACE = 7, /* workspace NULL or smaller than fa_bwd_workspace_bytes() */
  FA_ERR_HIP = 8,       /* the HIP runtime rejected a launch */
  FA_ERR_SCRATCH = 9    /* fa_bwd_noalloc: the sizes need more than its static scratch */
} fa_status;

typedef enum { FA_F32 = 0, FA_F16 = 1, FA_BF16 = 2 } fa_dtype;

/* Returns FA_ABI_VERSION of the built library. */
int fa_abi_version(void);

/* Static, human-readable name of a status code ("unknown status" otherwise). */
const char* fa_status_string(int status);

/* Forward attention: O = softmax(scale * Q K^T [causal mask]) V and the
 * per-row log-sum-exp, computed tile by tile with a running normalisation and
 * without an N x N array in memory ("FlashAttention" lexicon, "Methodische
 * Grundlagen": tiling and the running normalisation; "FlashAttention-2 (DE)",
 * "Technische Architektur und Funktionsprinzipien": one workgroup per query
 * tile and head, rows split across wavefronts, one normalisation at the end).
 *   q, k, v  [B,H,N,d] inputs of type dtype (FA_F32, FA_F16 or FA_BF16);
 *            d = 32, 64, 96, 128, 256 (FA_F32: 64, 128; at 256 N + 64 <=
 *            2^22).  d = 256 runs the pipelined d = 128 scheme at one
 *            wavefront per SIMD (Q and O in accumulation registers).
 *   o        [B,H,N,d] output, same type.  Fully overwritten.
 *   lse      [B,H,N] float32 output: natural-log log-sum-exp of the scaled
 *            scores of each row over its visible keys.  Fully overwritten.
 *   scale    multiplier of q.k (normally 1/sqrt(d)); any finite value with
 *            |scale| * log2(e) finite (a negative scale weights the keys of
 *            smallest q.k most; 0 gives uniform weights over the visible keys).
 *   causal   0: every key is visible; nonzero: key j visible to query i iff j <= i.
 * The output buffers must not overlap the inputs. */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int64_t B, int64_t H, int64_t N, int64_t d, float scale, int causal,
           int dtype, void* stream);

/* Bytes of device workspace fa_bwd needs for these sizes (4 * B * H * N:
 * one float32 per query row, D_i = dO_i . O_i).  0 for invalid sizes. */
size_t fa_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d, int dtype);

/* Backward attention: gradients of O with respect to Q, K and V, given the
 * upstream gradient dout = dL/dO and the forward's own outputs o and lse.
 * The scores and probabilities are recomputed from q, k and lse instead of
 * being kept from the forward ("FlashAttention" lexicon, "Methodische
 * Grundlagen", "Neuberechnung statt Speicherung"); the result is exact and
 * deterministic ("FlashAttention-2 (DE)", "Leistung und Effizienz").
 *   q, k, v, o, dout  [B,H,N,d] inputs of type dtype (FA_F16 or FA_BF16);
 *                     d = 32, 64, 96, 128 or 256 (N + 64 <= 2^22 at 256).
 *   lse               [B,H,N] float32 from fa_fwd on the same q, k, v.
 *   dq, dk, dv        [B,H,N,d] outputs, same type.  Fully overwritten.
 *   workspace         device scratch of at least fa_bwd_workspace_bytes(),
 *                     owned by the caller, contents need not be initialised.
 * dq/dk/dv are deterministic: repeated calls give bitwise-identical results. */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dout, void* dq, void* dk, void* dv,
           void* workspace, size_t workspace_bytes,
           int64_t B, int64_t H, int64_t N, int64_t d, float scale, int causal,
           int dtype, void* stream);

/* fa_bwd for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same backward, same kernels and bitwise the same results, with no
 * workspace argument.  Its one scratch array (D_i, one float per query row)
 * is a static device array of the library, 16 MiB per GPU, held from the
 * first call on a GPU until the process ends; so B * H * N must be at most
 * fa_bwd_noalloc_max_rows() = 4194304, else FA_ERR_SCRATCH (checked before
 * any device call).  The call allocates nothing: no hipMalloc, hipFree or
 * allocating library routine; its first call on a device looks up that
 * device's copy of the array (hipGetSymbolAddress) once.
 * Every call on one GPU shares that GPU's array and leaves its contents
 * behind: calls that overlap in time on one GPU (different streams, or
 * different threads without ordering) race and may give wrong gradients.
 * Arguments, layout, errors and determinism otherwise as fa_bwd. */
size_t fa_bwd_noalloc_max_rows(void);

int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, void* dq, void* dk, void* dv,
                   int64_t B, int64_t H, int64_t N, int64_t d, float scale, int causal,
                   int dtype, void* stream);

/* The three stages fa_bwd runs, in this order, for callers that schedule or
 * time them separately (same arguments, contract and errors as fa_bwd; each
 * takes only the arrays it reads or writes).
 *   fa_bwd_prep  workspace[b,h,i] = sum_c dout[b,h,i,c] * o[b,h,i,c]   (float32)
 *   fa_bwd_dkdv  dk, dv from q, k, v, dout, lse and the prepared workspace
 *   fa_bwd_dq    dq     from q, k, v, dout, lse and the prepared workspace
 * fa_bwd_dkdv and fa_bwd_dq read the workspace written by fa_bwd_prep and are
 * independent of each other. */
int fa_bwd_prep(const void* o, const void* dout, void* workspace, size_t workspace_bytes,
                int64_t B, int64_t H, int64_t N, int64_t d, int dtype, void* stream);

int fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                const void* workspace, size_t workspace_bytes, void* dk, void* dv,
                int64_t B, int64_t H, int64_t N, int64_t d, float scale, int causal,
                int dtype, void* stream);

int fa_bwd_dq(const void* q, const void* k, const void* v, const void* dout, const float* lse,
              const void* workspace, size_t workspace_bytes, void* dq,
              int64_t B, int64_t H, int64_t N, int64_t d, float scale, int causal,
              int dtype, void* stream);

/* New queries against a key/value cache (inference: decoding one or a few
 * tokens, or a chunk of a prompt, against the keys and values kept from the
 * earlier positions).  The pages place the method in inference and serving
 * next to the block-wise management of that cache ("FlashAttention-2 (DE)",
 * lead paragraph; "FlashAttention" glossary, "Der Engpass ist der Weg zum
 * Speicher, nicht das Rechnen", "Wo es verwechselt wird").  The arithmetic is
 * the same exact attention as fa_fwd with fewer queries than keys:
 *
 *   query i (0 <= i < Nq) of batch entry b sees cache row j iff
 *     j < L_b                               (causal == 0)
 *     j < L_b and j <= i + (L_b - Nq)       (causal != 0: bottom-right aligned,
 *                                            the queries are the last Nq
 *                                            positions of a length-L_b sequence)
 *   with L_b = seqlens_k[b] clamped to [0, Nk], or Nk when seqlens_k is NULL.
 *
 *   q          [B,H,Nq,d] queries, dtype FA_F16 or FA_BF16.
 *   k_cache,   [B,H,Nk,d] caches of capacity Nk rows, same dtype; rows at and
 *   v_cache    past L_b are never read (their contents do not matter).
 *   seqlens_k  DEVICE int32 [B] filled lengths (4-byte aligned), or NULL.
 *   o          [B,H,Nq,d] output, same dtype.  Fully overwritten.
 *   lse        [B,H,Nq] float32 output, natural-log log-sum-exp over the
 *              visible keys.  A query that sees no key (L_b = 0, or causal
 *              with i < Nq - L_b) gets o = 0 and lse = -infinity.
 *   workspace  device scratch of fa_fwd_kvcache_workspace_bytes() bytes
 *              (16-byte aligned), owned by the caller, contents need not be
 *              initialised; may be NULL when that size is 0.  It holds the
 *              partial results of the key ranges the cache is split into.
 *   scale, causal, dtype, stream: as for fa_fwd.  Nq, Nk in [1, 2^22].
 *   d          32, 64, 128 or 256 (fa_fwd_kvcache_fp8: 32, 64, 128).
 * Errors: FA_ERR_NULL (q, k_cache, v_cache, o or lse NULL), FA_ERR_SHAPE,
 * FA_ERR_HEADDIM, FA_ERR_DTYPE (FA_F32 is not taken), FA_ERR_ALIGN,
 * FA_ERR_SCALE, FA_ERR_WORKSPACE (NULL or too small when the size is > 0).
 * Results are bitwise repeatable. */
size_t fa_fwd_kvcache_workspace_bytes(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                                      int dtype);

int fa_fwd_kvcache(const void* q, const void* k_cache, const void* v_cache, const int32_t* seqlens_k,
                   void* o, float* lse, void* workspace, size_t workspace_bytes,
                   int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale, int causal,
                   int dtype, void* stream);

/* fa_fwd_kvcache with the cache stored in 8 bits: k_cache and v_cache hold
 * OCP E4M3 codes (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no
 * infinities, largest value 448; one byte per element, layout [B,H,Nk,d])
 * with one scale per tensor: the cached key row j is k_scale * E4M3(k[j]),
 * the value row v_scale * E4M3(v[j]).  The pages describe 8-bit floating
 * point as a later step of the method's line ("FlashAttention-2 (DE)",
 * "Vergleich mit nachfolgenden Versionen / FlashAttention-3"); here it halves
 * the bytes a decode step reads.  With those dequantised values the result is
 * the same attention as fa_fwd_kvcache computes (the codes convert exactly to
 * the query's 16-bit type); the difference from an unquantised cache is the
 * quantisation of the cache alone.
 *   k_scale, v_scale  finite and > 0, else FA_ERR_SCALE.
 * Every other argument, the workspace size (fa_fwd_kvcache_workspace_bytes
 * with the query's dtype), alignment and error rule is as for
 * fa_fwd_kvcache; dtype is that of q and o (FA_BF16 or FA_F16). */
int fa_fwd_kvcache_fp8(const void* q, const void* k_cache, const void* v_cache, float k_scale,
                       float v_scale, const int32_t* seqlens_k, void* o, float* lse, void* workspace,
                       size_t workspace_bytes, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                       float scale, int causal, int dtype, void* stream);

/* Variable-length packed batch: B sequences of different lengths stored
 * back to back, as training on packed sequences and serving batches of
 * prompts lay them out (the pages' drop-in use with the usual attention
 * interfaces: "FlashAttention-2 (DE)", "Anwendung und Integration in das
 * Ökosystem").  Sequence b owns rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1
 * of q and o, and rows cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1 of k and v;
 * within it, attention is that of fa_fwd_kvcache with Nq = its query count
 * and L = its key count (causal: key j visible to query i iff
 * j <= i + L - Nq, bottom-right aligned; equal lengths give fa_fwd's mask).
 *   q, o          [total_q, H, d] of type dtype (FA_BF16 or FA_F16), packed
 *                 rows; o rows outside every sequence are left unchanged.
 *   k, v          [total_k, H, d], same type.
 *   cu_seqlens_q, DEVICE int32 [B + 1] non-decreasing prefix sums (4-byte
 *   cu_seqlens_k  aligned); entries are clamped to [0, total], a sequence's
 *                 counts to [0, max_q] and [0, max_k], so malformed sums
 *                 never make an access leave the tensors (rows two
 *                 sequences claim then hold unspecified values).
 *   lse           [H, total_q] float32 (natural log; -infinity and o = 0 for
 *                 a query that sees no key).
 *   max_q, max_k  the largest query and key count of any sequence, in
 *                 [1, 2^22]; max * H * d * 2 must stay below 2^31 bytes.
 *   workspace     fa_fwd_varlen_workspace_bytes(B, H, max_q, max_k, d, dtype)
 *                 bytes (16-byte aligned, may be NULL when that is 0).
 * When cu_seqlens_q and cu_seqlens_k are the same pointer (self-attention:
 * equal query and key counts), total_q = total_k, max_q = max_k and
 * (max_q + 512) * H * d * 2 < 2^31, fa_fwd's kernels run on the packed rows
 * in place and the workspace is not used; otherwise the split-key kernels of
 * fa_fwd_kvcache do.  d: 32, 64, 128, 256, and 96 on the self-attention
 * route only.
 * Errors as for fa_fwd_kvcache (FA_ERR_NULL also for NULL prefix sums,
 * FA_ERR_SHAPE for total_q or total_k < 1 or the offset limit). */
size_t fa_fwd_varlen_workspace_bytes(int64_t B, int64_t H, int64_t max_q, int64_t max_k, int64_t d,
                                     int dtype);

int fa_fwd_varlen(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                  const int32_t* cu_seqlens_k, void* o, float* lse, void* workspace, size_t workspace_bytes,
                  int64_t B, int64_t H, int64_t total_q, int64_t total_k, int64_t max_q, int64_t max_k,
                  int64_t d, float scale, int causal, int dtype, void* stream);

/* Backward over a variable-length packed batch: the training side of
 * fa_fwd_varlen's packed layout (the pages' drop-in use with the usual
 * attention interfaces: "FlashAttention-2 (DE)", "Anwendung und Integration
 * in das Ökosystem"; the gradient, recomputed as in fa_bwd: "FlashAttention"
 * lexicon, "Methodische Grundlagen").  Sequence b owns query rows
 * cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 of q, o, dout, dq and key rows
 * cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1 of k, v, dk, dv; within it the mask
 * is fa_fwd_varlen's (causal: key j visible to query i iff j <= i + Lk - Lq,
 * bottom-right aligned; with equal counts the square mask).  fa_bwd's
 * kernels read and write the packed rows in place (row stride H d), one
 * workgroup per head and 128-row tile of max_q (dQ) or max_k (dK, dV), and
 * skip tiles past a sequence's counts.  A key no query sees gets dk = dv = 0,
 * a query that sees no key dq = 0.
 *   q, o, dout    [total_q, H, d] of type dtype (FA_BF16 or FA_F16), packed
 *   k, v          [total_k, H, d]      rows, 16-byte aligned; o and lse are
 *                 fa_fwd_varlen's output for these q, k, v and causal.
 *   lse           [H, total_q] float32 (natural log).
 *   cu_seqlens_q, DEVICE int32 [B + 1] non-decreasing prefix sums (4-byte
 *   cu_seqlens_k  aligned; may be the same pointer), clamped like
 *                 fa_fwd_varlen's (entries to [0, total], counts to
 *                 [0, max]).
 *   dq            [total_q, H, d], dk, dv [total_k, H, d] outputs, same type;
 *                 rows outside every sequence are left unchanged.
 *   max_q, max_k  the largest query / key count of any sequence, in
 *                 [1, 2^22]; (max + 512) * H * d * 2 must stay below 2^31.
 *   d             32, 64, 96 or 128.
 *   workspace     fa_bwd_varlen_workspace_bytes(B, H, total_q, max_q, d,
 *                 dtype) bytes (total_q * H floats: D_i = dO_i . O_i),
 *                 16-byte aligned, contents need not be initialised.
 * Deterministic (fixed reduction order).  Errors: FA_ERR_NULL, FA_ERR_SHAPE
 * (as fa_fwd for B, H, max_q, max_k; totals < 1, total * H > 2^31 - 1, or
 * the offset limit), FA_ERR_HEADDIM, FA_ERR_DTYPE (not FA_BF16 / FA_F16),
 * FA_ERR_ALIGN, FA_ERR_SCALE, FA_ERR_WORKSPACE, FA_ERR_HIP.  The workspace
 * size function returns 0 for arguments the entry point rejects. */
size_t fa_bwd_varlen_workspace_bytes(int64_t B, int64_t H, int64_t total_q, int64_t max_q, int64_t d,
                                     int dtype);

int fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse,
                  const void* dout, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, void* dq, void* dk,
                  void* dv, void* workspace, size_t workspace_bytes, int64_t B, int64_t H, int64_t total_q,
                  int64_t total_k, int64_t max_q, int64_t max_k, int64_t d, float scale, int causal, int dtype,
                  void* stream);

/* Forward and backward with caller strides: any element strides per tensor
 * (batch, head, row; the d elements of a row contiguous), so that [B, N, H, d]
 * tensors, views into a packed QKV tensor [B, N, 3, H, d] and the like are
 * used in place, with no copies (the pages' drop-in use with the usual
 * attention interfaces: "FlashAttention-2 (DE)", "Anwendung und Integration in
 * das Ökosystem").  Same attention, mask, numerics and errors as fa_fwd /
 * fa_bwd (16-bit types only), with:
 *   strides  HOST int64 array, 3 entries per tensor in the order of the
 *            pointers: fa_fwd_strided q, k, v, o (12 entries); fa_bwd_strided
 *            q, k, v, o, dout, dq, dk, dv (24 entries).  Row r of head h of
 *            batch b of a tensor starts at element b*s[0] + h*s[1] + r*s[2].
 *            Every stride must be >= 0 and a multiple of 8 (16-byte aligned
 *            rows: else FA_ERR_ALIGN); an output's row stride >= d; (N + 512)
 *            * row stride * 2 below 2^31 (else FA_ERR_SHAPE).  Inputs may
 *            overlap (a head stride of 0 shares one K/V head among query
 *            heads); outputs must not overlap each other or the inputs.
 *   lse      contiguous [B, H, N] float32 as for fa_fwd; the backward's
 *            workspace as for fa_bwd.
 *   d        32, 64, 96, 128 or 256, as fa_fwd / fa_bwd. */
int fa_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse, const int64_t* strides,
                   int64_t B, int64_t H, int64_t N, int64_t d, float scale, int causal, int dtype, void* stream);

int fa_bwd_strided(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                   void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, const int64_t* strides,
                   int64_t B, int64_t H, int64_t N, int64_t d, float scale, int causal, int dtype, void* stream);

/* Forward attention on 8-bit floating-point inputs.  The pages name 8-bit
 * floating point as the next step of the method's line ("FlashAttention-2
 * (DE)", "Vergleich mit nachfolgenden Versionen / FlashAttention-3"); here Q,
 * K and V are OCP E4M3 codes (1 sign, 4 exponent bits with bias 7, 3
 * mantissa bits, no infinities, largest value 448; one byte per element)
 * with float scales, and S = Q K^T runs on the FP8 matrix cores.
 *   q8, k8, v8  [B,H,N,d] uint8 E4M3 codes, 16-byte aligned; d must be 128.
 *   q_scale,    DEVICE float32 scales (4-byte aligned), all finite and > 0:
 *   k_scale,    FA_SCALE_TENSOR: one float each, element x of a tensor stands
 *   v_scale     for scale * E4M3(x);  FA_SCALE_BLOCK: q_scale and k_scale
 *               [B,H,ceil(N/128)], one per block of 128 rows of a head (row
 *               i of head (b,h) stands for q_scale[b,h,i/128] * E4M3(q8[..])),
 *               v_scale [B,H], one per head.  (Scales cannot be checked by
 *               the host; a non-positive or non-finite one gives unspecified
 *               results.)
 *   o           [B,H,N,d] output of type dtype (FA_BF16 or FA_F16): the
 *               probabilities are rounded to this type and multiply V, whose
 *               codes convert to it exactly.
 *   lse         [B,H,N] float32, natural log, as fa_fwd.
 *   scale, causal, stream, errors: as fa_fwd (FA_ERR_HEADDIM for d != 128,
 *   FA_ERR_DTYPE also for an unknown scale_granularity).
 * With the dequantised values (codes times scales) the result is fa_fwd's
 * exact attention to the 16-bit path's precision: the scores are exact
 * products of the codes accumulated in float32, the scales multiply them in
 * float32; only the rounding of the inputs to 8 bits differs from attention
 * on 16-bit inputs.  Deterministic. */
enum { FA_SCALE_TENSOR = 0, FA_SCALE_BLOCK = 1 };

int fa_fwd_fp8(const void* q8, const void* k8, const void* v8, const float* q_scale, const float* k_scale,
               const float* v_scale, int scale_granularity, void* o, float* lse,
               int64_t B, int64_t H, int64_t N, int64_t d, float scale, int causal,
               int dtype, void* stream);

/* Measurement probe, not part of attention: enqueues a kernel of `workgroups`
 * workgroups (4 wavefronts each) in which every wavefront issues `iters`
 * rounds of four independent dense bf16 matrix products
 * (v_mfma_f32_32x32x16_bf16, 32768 FLOP each) on register operands, reading
 * and writing no memory.  Timed by the caller (events around the call on
 * `stream`), it gives the sustained dense bf16 MFMA rate the attention
 * kernels are compared with beside the published peak.  Returns the FLOP
 * count of the launch (workgroups * 4 * iters * 4 * 32768), or the negated
 * FA_ERR_SHAPE (workgroups not in [1, 2^24 - 1], iters not in
 * [1, 2^31 - 1], or workgroups * iters above 2^44, where the count would
 * leave int64) or FA_ERR_HIP (launch refused). */
int64_t fa_probe_mfma_bf16(int64_t workgroups, int64_t iters, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_H */
