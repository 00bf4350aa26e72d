// Internal interface between the C-ABI entry points (fa_api.hip) and the
// kernel launchers (fa_fwd.hip, fa_bwd.hip).  Arguments arrive here already
// validated: non-null, 16-byte aligned, d one the entry point takes, N >= 1,
// B*H >= 1, finite non-negative scale.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "fa_common.hpp"

namespace fa {

enum Dt { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

constexpr float kLog2eHost = 1.4426950408889634f;

// Compute units of the device that runs `stream` (cached per device; 0 if
// the query fails).
int device_cu_count(hipStream_t stream);

// Grid of a kernel that can walk its tiles persistently (persistent_tile):
// one workgroup per resident slot (per_cu per compute unit) when that is
// fewer than the tiles and the deal comes out even: heads a multiple of 8 and
// every XCD's tiles (nbh / 8 heads of nt tiles) a whole number of rounds of
// its slots / 8 workgroups.  Otherwise one workgroup per tile.
inline uint32_t persistent_grid(int nbh, int nt, int per_cu, hipStream_t stream) {
  const uint32_t total = (uint32_t)nbh * (uint32_t)nt;
  const uint32_t slots = (uint32_t)(device_cu_count(stream) * per_cu);
  if (slots == 0 || slots % 8 != 0 || nbh % 8 != 0 || total <= slots) return total;
  if (((uint32_t)(nbh / 8) * (uint32_t)nt) % (slots / 8) != 0) return total;
  return slots;
}

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int BH;     // batch * heads
  int N;      // sequence length (queries = keys)
  int d;      // head dimension
  float c;    // |scale| * log2(e); a negative scale sets g.qneg
  int causal;
  int dtype;
  hipStream_t stream;
  // General layout (16-bit types only): per-tensor strides, packed
  // self-attention batches (equal query and key counts per sequence, at most
  // N each), head dimensions 32 and 96 (on the 64 / 128 kernels with zero
  // columns); g.dr = d.  false: the dense [BH, N, d] layout.
  bool general = false;
  GenLayout g{};
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* dvec;  // workspace: D_i = dO_i . O_i, one float per query row, at the LSE entry's place
  int BH;
  int Nq;       // queries per sequence (the largest, with prefix sums)
  int Nk;       // keys per sequence (dense: Nk = Nq)
  int d;
  float scale;
  float c;      // scale * log2(e), of the scale's sign (no running maximum in the backward)
  int causal;
  int dtype;
  hipStream_t stream;
  // General layout: per-tensor strides, packed sequences with their own
  // query and key counts (causal aligned bottom right), head dimensions 32
  // and 96 (zero columns on the 64 / 128 kernels); g.dr = d.  false: the
  // dense [BH, N, d] layout.
  bool general = false;
  GenLayout g{};
};

enum BwdStage { BWD_PREP = 0, BWD_DKDV = 1, BWD_DQ = 2 };

// Where the rows of sequence b, head h lie (element offsets): row r of q at
// b q_sb + h q_sh + (start_q(b) + r) q_sr (o likewise with the o strides),
// row j of the keys at b c_sb + h c_sh + (start_k(b) + j) c_sr (values with
// the v strides), and the LSE of query r at b l_sb + h l_sh + start_q(b) + r.  Without prefix sums every sequence
// starts at row 0 and has Nq queries and Nk (or seqlens[b]) cache rows; with
// them, sequence b has rows cu[b] .. cu[b + 1] - 1 of a packed tensor of
// total rows (the kernels clamp both into [0, total]).
struct KvLayout {
  int64_t q_sb, q_sh, q_sr;
  int64_t c_sb, c_sh, c_sr;  // keys
  int64_t l_sb, l_sh;
  int64_t v_sb, v_sh, v_sr;  // values (the keys' strides unless set otherwise)
  int64_t o_sb, o_sh, o_sr;  // output (the queries' strides unless set otherwise)
  const int32_t* cu_q;  // [B + 1] or NULL
  const int32_t* cu_k;  // [B + 1] or NULL
  int64_t total_q, total_k;
  uint32_t qneg = 0;  // 0x80008000: negative scale, the query fragments' signs flipped
};

// Queries against a key/value cache (fa_fwd_kvcache, fa_fwd_varlen).
struct KvArgs {
  const void* q;           // [BH, Nq, d]
  const void* k;           // [BH, Nk, d] cache (capacity Nk rows)
  const void* v;
  const int32_t* seqlens;  // [B] filled rows per batch entry, or NULL (= Nk)
  void* o;                 // [BH, Nq, d]
  float* lse;              // [BH, Nq]
  void* workspace;         // kv_workspace_bytes() bytes (NULL when that is 0)
  KvLayout lay;
  int H;
  int BH;
  int Nq;                  // queries per sequence (the largest, with prefix sums)
  int Nk;                  // cache rows per sequence (the largest, with prefix sums)
  int d;
  float c;                 // |scale| * log2(e) (times the K scale of an 8-bit cache)
  float v_scale;           // multiplies O: the V scale of an 8-bit cache, else 1
  int fp8_cache;           // k, v hold OCP E4M3 codes (1 byte per element)
  int one_range = 0;       // one key range per head (no workspace): the kernel writes O and LSE itself
  int causal;
  int dtype;               // of q and o (FA_BF16 or FA_F16)
  hipStream_t stream;
};

// How the keys are split: every wavefront takes `kps` keys (a power of two,
// >= 64) of one head for one block of 32 queries.  kps doubles from 64 until
// the launch has at most 8192 wavefronts at d = 128 (16384 at d = 64), i.e.
// 32 (64) per compute unit: a decode step over a long cache still spreads
// over the whole chip, while each range moves at least ~128 KB of K and V
// (measured on a B=4 H=32 32768-row decode step: 2x more, shorter ranges
// cost 10-18% at d = 128, 2x fewer changed nothing at d = 64).
struct KvPlan {
  int n_qb;      // 32-query blocks
  int kps;       // keys per range
  int n_splits;  // ranges per head
};

inline KvPlan kv_plan(int64_t BH, int64_t Nq, int64_t Nk, int64_t d) {
  KvPlan p;
  p.n_qb = (int)((Nq + 31) / 32);
  const int64_t max_waves = d >= 256 ? 4096 : d == 128 ? 8192 : 16384;
  int64_t kps = 64;
  while (kps < Nk && BH * p.n_qb * ((Nk + kps - 1) / kps) > max_waves) kps *= 2;
  p.kps = (int)kps;
  p.n_splits = (int)((Nk + kps - 1) / kps);
  return p;
}

// One range covering every key of a head (the square forward at d = 256,
// which takes no workspace).
inline KvPlan kv_plan_one_range(int64_t Nq, int64_t Nk) {
  KvPlan p;
  p.n_qb = (int)((Nq + 31) / 32);
  int64_t kps = 64;
  while (kps < Nk) kps *= 2;
  p.kps = (int)kps;
  p.n_splits = 1;
  return p;
}

// Workspace of the split path: per range, per head and query, d floats of
// partial O then 2 floats of base-2 log-sum-exps.  0 when one range covers
// the cache (the kernel then writes O and LSE directly).
inline size_t kv_workspace_bytes(int64_t BH, int64_t Nq, int64_t Nk, int64_t d) {
  const KvPlan p = kv_plan(BH, Nq, Nk, d);
  if (p.n_splits == 1) return 0;
  return (size_t)p.n_splits * (size_t)BH * (size_t)Nq * (size_t)(d + 2) * sizeof(float);
}

hipError_t launch_fwd_kvcache(const KvArgs& a);


// 8-bit (E4M3) Q, K, V with float scales (fa_fwd_fp8): [BH, N, d] codes;
// per_block: q_scale and k_scale hold one float per 128-row block of each
// head ([BH, ceil(N / 128)]) and v_scale one per head ([BH]); otherwise each
// holds one float for the whole tensor.
struct Fp8Args {
  const void* q;
  const void* k;
  const void* v;
  const float* q_scale;
  const float* k_scale;
  const float* v_scale;
  int per_block;
  void* o;      // [BH, N, d] of dtype
  float* lse;   // [BH, N]
  int BH;
  int N;
  int d;
  float c;      // |scale| * log2(e)
  bool qneg;    // negative scale: the query codes' signs flipped
  int causal;
  int dtype;    // of o and of the probabilities (DT_BF16 or DT_F16)
  hipStream_t stream;
};

hipError_t launch_fwd_fp8(const Fp8Args& a);

// Measurement probe (fa_probe_mfma_bf16): workgroups of 4 wavefronts.
hipError_t launch_mfma_peak(int workgroups, int iters, hipStream_t stream);

hipError_t launch_fwd(const FwdArgs& a);
hipError_t launch_bwd(const BwdArgs& a);                 // all three stages in order
hipError_t launch_bwd_stage(const BwdArgs& a, int stage);  // one stage
hipError_t launch_bwd_wide_stage(const BwdArgs& a, int stage);  // d = 256: dK/dV or dQ

}  // namespace fa
