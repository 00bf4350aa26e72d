// Backward attention for head dimension 256 on gfx950.
//
// The gradient is fa_bwd.hip's (chain rule through the softmax, scores and
// probabilities recomputed from Q, K and the LSE instead of stored:
// "FlashAttention" lexicon, "Methodische Grundlagen", "Neuberechnung statt
// Speicherung"); only the work split differs, because at d = 256 one
// wavefront cannot hold both the B operands of the score products (K and V,
// or Q and dO, over all 256 columns: 128 registers) and the accumulators of
// both gradients (256 registers).  So every 32-key (dK, dV) or 32-query (dQ)
// block is shared by two wavefronts, each accumulating one half of the
// gradient's columns; both compute the block's scores and dP over all 256
// columns (the score products are done twice: 1.5x the algorithmic products
// of the backward).  No software pipeline: each 32-row stage is staged
// through LDS (two buffers, one workgroup barrier per stage) and the matrix
// and vector work of a stage follow each other; one workgroup of four
// wavefronts per compute unit (512 registers per wavefront, the score
// operands and the gradient accumulators in AGPRs, the score products'
// operands read from LDS a few products ahead).
//
// Layouts as in fa_bwd.hip: S (or S^T) accumulator row m of a 32-row block
// holds row perm(m) of the staged tile, so that the transposed LDS reads of
// the gradient products gather rows 4 apart (bank-conflict free), and the
// per-row LSE and D values are staged in the same permuted order.
// General layout (strides per tensor, packed sequences with their own query
// and key counts, bottom-right causal alignment), as the other backward
// kernels' GL variants.
#include <type_traits>

#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {

namespace {

constexpr int WD = 256;                 // head dimension
constexpr int WKS = WD / 16;            // k-steps of the score products
constexpr int WRBL = 2 * (WD + 8);      // LDS row bytes (padded)
constexpr int WBLK = 32 * WRBL;         // one 32-row tile of one tensor in LDS

__device__ inline int wperm(int m) { return (m & 16) | ((m & 3) << 2) | ((m >> 2) & 3); }

// 16-byte chunk i of a 32 x 256 tile (row i / 32, chunk i % 32), loaded by
// 256 threads as 4 chunks each: rows past the range read zeros.
struct TileLoad {
  u32x4_t x[4];
  __device__ inline void load(rsrc_t r, uint32_t rs, int row0, int tid) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = tid + 256 * j;
      x[j] = buf_load16(r, (uint32_t)(row0 + i / 32) * rs + 16 * (i % 32));
    }
  }
  __device__ inline void store(char* lds, int tid) const {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = tid + 256 * j;
      *(u32x4_t*)(lds + (i / 32) * WRBL + 16 * (i % 32)) = x[j];
    }
  }
};

}  // namespace

// dK, dV for d = 256.  Workgroup: 64 keys; wavefront w takes keys
// k0 + 32 (w / 2) and gradient columns 128 (w % 2) .. +127.  Query rows
// stream through LDS in 32-row stages (Q, dO, LSE log2 e, D).
template <class TR, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dkdv_wide_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                          const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                          const float* __restrict__ LSE, const float* __restrict__ Dvec,
                          uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int Nq, int Nk, int n_ktiles,
                          float c, float scale, GenLayout g) {
  constexpr int STG = 2 * WBLK + 2 * 32 * 4;  // Q, dO tiles, then LSE log2 e and D (32 floats each)
  __shared__ __attribute__((aligned(16))) char smem[2 * STG];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int h = lane >> 5;
  const int l32 = lane & 31;
  const int ch = w & 1;  // gradient column half
  using PM = PipeMma<TR, true>;  // K, V (score operands) and dK, dV (accumulators) in AGPRs

  const int bh = blockIdx.x / n_ktiles;
  const int k0 = (blockIdx.x % n_ktiles) * 64;
  const int kw = k0 + 32 * (w >> 1);
  const int b = bh / g.H, hd = bh - b * g.H;
  int sq, Lq, sk, Lk;
  seq_rows(g.cu_q, g.total_q, b, Nq, sq, Lq);
  seq_rows(g.cu_k, g.total_k, b, Nk, sk, Lk);
  if (k0 >= Lk) return;
  const int delta = CAUSAL ? Lk - Lq : 0;
  const TRows tq = tensor_rows(g.q, b, hd, sq, Lq, WD), tdo = tensor_rows(g.dout, b, hd, sq, Lq, WD);
  const TRows tk = tensor_rows(g.k, b, hd, sk, Lk, WD), tv = tensor_rows(g.v, b, hd, sk, Lk, WD);
  const size_t l_off = (size_t)((int64_t)b * g.l_sb + (int64_t)hd * g.l_sh + sq);

  // K and V rows of this wavefront's keys as B operands (column = key), all 256 columns
  u32x4_t kf[WKS], vf[WKS];
  {
    const rsrc_t kres = make_rsrc(K + tk.off, tk.bytes), vres = make_rsrc(V + tv.off, tv.bytes);
    const int key = kw + l32;
#pragma unroll
    for (int ks = 0; ks < WKS; ++ks) {
      kf[ks] = buf_load16(kres, (uint32_t)key * tk.rs + 32 * ks + 16 * h);
      vf[ks] = buf_load16(vres, (uint32_t)key * tv.rs + 32 * ks + 16 * h);
    }
  }
  f32x16_t acc_dk[4], acc_dv[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) acc_dk[db] = acc_dv[db] = zero16();
  PM::copy_wait(acc_dk[0], acc_dk[1], acc_dk[2], acc_dk[3], acc_dv[0], acc_dv[1], acc_dv[2], acc_dv[3]);

  const int i_begin = CAUSAL ? max(0, k0 - delta) : 0;
  const int n_st = (Lq - i_begin + 31) / 32;
  const rsrc_t qres = make_rsrc(Q + tq.off, tq.bytes), ores = make_rsrc(dO + tdo.off, tdo.bytes);
  TileLoad lq_, lo_;
  float lv = 0.0f, dv_ = 0.0f;  // threads 0..31: LSE log2 e and D of row perm(tid)
  auto load_stage = [&](int i0) __attribute__((always_inline)) {
    lq_.load(qres, tq.rs, i0, tid);
    lo_.load(ores, tdo.rs, i0, tid);
    if (tid < 32) {
      const int row = i0 + wperm(tid);
      // rows past the end: +inf makes P = 0 there
      lv = row < Lq ? LSE[l_off + row] * kLog2e : INFINITY;
      dv_ = row < Lq ? Dvec[l_off + row] : 0.0f;
    }
  };
  auto store_stage = [&](char* st) __attribute__((always_inline)) {
    lq_.store(st, tid);
    lo_.store(st + WBLK, tid);
    if (tid < 32) {
      ((float*)(st + 2 * WBLK))[tid] = lv;
      ((float*)(st + 2 * WBLK))[32 + tid] = dv_;
    }
  };
  const uint32_t rbase = (uint32_t)(wperm(l32) * WRBL + 16 * h);
  const int L16 = lane & 15, G = lane >> 4;
  const uint32_t tbase = (uint32_t)((h + 4 * (L16 >> 2)) * WRBL + (16 * (G & 1) + 4 * (L16 & 3)) * 2);

  if (n_st > 0) {
    load_stage(i_begin);
    store_stage(smem);
  }
  __syncthreads();
  for (int s = 0; s < n_st; ++s) {
    char* st = smem + (s & 1) * STG;
    const int i0 = i_begin + 32 * s;
    if (s + 1 < n_st) load_stage(i0 + 32);
    // S = Q K^T, dP = dO V^T (rows: queries perm(m); columns: this wavefront's
    // keys), alternating, each A operand read from LDS four products ahead
    f32x16_t sc, dp;
    mma_pipeline<2 * WKS, 4>([&](int x) { return st + ((x & 1) ? WBLK : 0) + rbase + 32 * (x >> 1); },
                             [&](int x, u32x4_t a) {
                               const int ks = x >> 1;
                               if (x & 1) {
                                 if (ks == 0) dp = PM::mb0(a, vf[0]);
                                 else PM::mb(dp, a, vf[ks]);
                               } else {
                                 if (ks == 0) sc = PM::mb0(a, kf[0]);
                                 else PM::mb(sc, a, kf[ks]);
                               }
                             },
                             [](int) {});
    mfma_wait_v(sc, dp);
    // P = exp2(S c - LSE log2 e), dS = P (dP - D), masked; rounded pairs as B operands
    const float* lvec = (const float*)(st + 2 * WBLK);
    u32x4_t pk[2], dsk[2];
    const int thr = kw - delta - i0 + l32 - h;  // causal: visible iff thr <= qoff(r)
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      float p2[2], ds2[2];
#pragma unroll
      for (int e2 = 0; e2 < 2; ++e2) {
        const int rr = r + e2;
        const int gq = rr / 4, e = rr % 4;
        const int m = 8 * gq + 4 * h + e;  // accumulator row
        float x = fmaf(sc[rr], c, -lvec[m]);
        if (CAUSAL) {
          const int qoff = 16 * (gq / 2) + 4 * e + 2 * (gq % 2);
          x = thr <= qoff ? x : -INFINITY;
        }
        const float p = fast_exp2(x);
        p2[e2] = p;
        ds2[e2] = p * (dp[rr] - lvec[32 + m]);
      }
      pk[r / 8][(r / 2) % 4] = TR::pack2(p2[0], p2[1]);
      dsk[r / 8][(r / 2) % 4] = TR::pack2(ds2[0], ds2[1]);
    }
    // P and dS were written by vector instructions: two wait states before
    // the products read them
    asm volatile("s_nop 1" : "+v"(pk[0]), "+v"(pk[1]), "+v"(dsk[0]), "+v"(dsk[1]));
    // dV^T += dO^T P, dK^T += Q^T dS over this wavefront's 128 columns;
    // product x: k-step t = x / 8, column block db = (x / 2) % 4, dV (x even)
    // or dK (x odd), its transposed A operand read four products ahead
    auto tr_a = [&](int x) __attribute__((always_inline)) -> u32x4_t {
      const char* pq = st + tbase + 16 * (x >> 3) * WRBL + 64 * (4 * ch + ((x >> 1) & 3)) + ((x & 1) ? 0 : WBLK);
      const u32x2_t a0 = lds_read_tr(pq), a1 = lds_read_tr(pq + 2 * WRBL);
      return u32x4_t{a0[0], a0[1], a1[0], a1[1]};
    };
    u32x4_t fr[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) fr[x] = tr_a(x);
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      const u32x4_t a = fr[x % 4];
      if (x + 4 < 16) fr[x % 4] = tr_a(x + 4);
      const int t = x >> 3, db = (x >> 1) & 3;
      if (x & 1) PM::macc(acc_dk[db], a, dsk[t]);
      else PM::macc(acc_dv[db], a, pk[t]);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (s + 1 < n_st) store_stage(smem + ((s + 1) & 1) * STG);
    __syncthreads();
  }

  PM::wait_acc(acc_dk[0], acc_dk[1], acc_dk[2], acc_dk[3], acc_dv[0], acc_dv[1], acc_dv[2], acc_dv[3]);
  // dK (times the scale) and dV, this wavefront's 128 columns of its 32 keys,
  // as whole rows through LDS (the stages are free after the last barrier)
  u32x2_t ok[4][4], ov[4][4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) {
      ok[db][gg] = u32x2_t{TR::pack2(acc_dk[db][4 * gg] * scale, acc_dk[db][4 * gg + 1] * scale),
                           TR::pack2(acc_dk[db][4 * gg + 2] * scale, acc_dk[db][4 * gg + 3] * scale)};
      ov[db][gg] = u32x2_t{TR::pack2(acc_dv[db][4 * gg], acc_dv[db][4 * gg + 1]),
                           TR::pack2(acc_dv[db][4 * gg + 2], acc_dv[db][4 * gg + 3])};
    }
  const int nrows = min(32, Lk - kw);
  const size_t dk_off = (size_t)((int64_t)b * g.dk.sb + (int64_t)hd * g.dk.sh + (int64_t)(sk + kw) * g.dk.sr);
  const size_t dv_off = (size_t)((int64_t)b * g.dv.sb + (int64_t)hd * g.dv.sh + (int64_t)(sk + kw) * g.dv.sr);
  static_assert(8 * kTileRowsBytes<128> <= 2 * STG, "eight 32 x 128 tiles fit the stages");
  store_tile_rows<128>(smem + w * kTileRowsBytes<128>, ok, dK + dk_off + 128 * ch, nrows, lane, (size_t)g.dk.sr);
  store_tile_rows<128>(smem + (4 + w) * kTileRowsBytes<128>, ov, dV + dv_off + 128 * ch, nrows, lane,
                       (size_t)g.dv.sr);
}

// dQ for d = 256.  Workgroup: 64 queries; wavefront w takes queries
// q0 + 32 (w / 2) and gradient columns 128 (w % 2) .. +127.  Key rows (K, V)
// stream through LDS in 32-row stages.
template <class TR, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dq_wide_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                        const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                        const float* __restrict__ LSE, const float* __restrict__ Dvec, uint16_t* __restrict__ dQ,
                        int Nq, int Nk, int n_qtiles, float c, float scale, GenLayout g) {
  constexpr int STG = 2 * WBLK;  // K, V tiles
  __shared__ __attribute__((aligned(16))) char smem[2 * STG];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int h = lane >> 5;
  const int l32 = lane & 31;
  const int ch = w & 1;
  using PM = PipeMma<TR, true>;  // Q, dO (score operands) and dQ (accumulators) in AGPRs

  const int bh = blockIdx.x / n_qtiles;
  int qt = blockIdx.x % n_qtiles;
  if (CAUSAL) qt = n_qtiles - 1 - qt;  // longest rows first
  const int q0 = qt * 64;
  const int qw = q0 + 32 * (w >> 1);
  const int qrow = qw + l32;
  const int b = bh / g.H, hd = bh - b * g.H;
  int sq, Lq, sk, Lk;
  seq_rows(g.cu_q, g.total_q, b, Nq, sq, Lq);
  seq_rows(g.cu_k, g.total_k, b, Nk, sk, Lk);
  if (q0 >= Lq) return;
  const int delta = CAUSAL ? Lk - Lq : 0;
  const TRows tq = tensor_rows(g.q, b, hd, sq, Lq, WD), tdo = tensor_rows(g.dout, b, hd, sq, Lq, WD);
  const TRows tk = tensor_rows(g.k, b, hd, sk, Lk, WD), tv = tensor_rows(g.v, b, hd, sk, Lk, WD);
  const size_t l_off = (size_t)((int64_t)b * g.l_sb + (int64_t)hd * g.l_sh + sq);

  // Q and dO rows of this wavefront's queries as B operands (column = query)
  u32x4_t qf[WKS], of[WKS];
  {
    const rsrc_t qres = make_rsrc(Q + tq.off, tq.bytes), ores = make_rsrc(dO + tdo.off, tdo.bytes);
#pragma unroll
    for (int ks = 0; ks < WKS; ++ks) {
      qf[ks] = buf_load16(qres, (uint32_t)qrow * tq.rs + 32 * ks + 16 * h);
      of[ks] = buf_load16(ores, (uint32_t)qrow * tdo.rs + 32 * ks + 16 * h);
    }
  }
  // rows past the end: P = exp2(-inf) = 0, so dS = 0 there
  const float lq = qrow < Lq ? LSE[l_off + qrow] * kLog2e : INFINITY;
  const float dd = qrow < Lq ? Dvec[l_off + qrow] : 0.0f;
  f32x16_t acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) acc[db] = zero16();
  PM::copy_wait(acc[0], acc[1], acc[2], acc[3]);

  const int kv_end = CAUSAL ? min(Lk, q0 + 64 + delta) : Lk;
  const int n_st = kv_end > 0 ? (kv_end + 31) / 32 : 0;
  const rsrc_t kres = make_rsrc(K + tk.off, tk.bytes), vres = make_rsrc(V + tv.off, tv.bytes);
  TileLoad lk_, lv_;
  const uint32_t rbase = (uint32_t)(wperm(l32) * WRBL + 16 * h);
  const int L16 = lane & 15, G = lane >> 4;
  const uint32_t tbase = (uint32_t)((h + 4 * (L16 >> 2)) * WRBL + (16 * (G & 1) + 4 * (L16 & 3)) * 2);

  if (n_st > 0) {
    lk_.load(kres, tk.rs, 0, tid);
    lv_.load(vres, tv.rs, 0, tid);
    lk_.store(smem, tid);
    lv_.store(smem + WBLK, tid);
  }
  __syncthreads();
  for (int s = 0; s < n_st; ++s) {
    char* st = smem + (s & 1) * STG;
    const int j0 = 32 * s;
    if (s + 1 < n_st) {
      lk_.load(kres, tk.rs, j0 + 32, tid);
      lv_.load(vres, tv.rs, j0 + 32, tid);
    }
    // S^T = K Q^T, dP^T = V dO^T (rows: keys perm(m); columns: this
    // wavefront's queries), alternating, A operands read four products ahead
    f32x16_t sc, dp;
    mma_pipeline<2 * WKS, 4>([&](int x) { return st + ((x & 1) ? WBLK : 0) + rbase + 32 * (x >> 1); },
                             [&](int x, u32x4_t a) {
                               const int ks = x >> 1;
                               if (x & 1) {
                                 if (ks == 0) dp = PM::mb0(a, of[0]);
                                 else PM::mb(dp, a, of[ks]);
                               } else {
                                 if (ks == 0) sc = PM::mb0(a, qf[0]);
                                 else PM::mb(sc, a, qf[ks]);
                               }
                             },
                             [](int) {});
    mfma_wait_v(sc, dp);
    u32x4_t dsk[2];
    const int thr = qrow + delta - j0 - h;  // causal: key j0 + koff(r) visible iff koff(r) <= thr
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      float ds2[2];
#pragma unroll
      for (int e2 = 0; e2 < 2; ++e2) {
        const int rr = r + e2;
        const int gq = rr / 4, e = rr % 4;
        float x = fmaf(sc[rr], c, -lq);
        if (CAUSAL) {
          const int koff = 16 * (gq / 2) + 4 * e + 2 * (gq % 2);
          x = koff <= thr ? x : -INFINITY;
        }
        ds2[e2] = fast_exp2(x) * (dp[rr] - dd);
      }
      dsk[r / 8][(r / 2) % 4] = TR::pack2(ds2[0], ds2[1]);
    }
    // dS was written by vector instructions: two wait states before the
    // products read it
    asm volatile("s_nop 1" : "+v"(dsk[0]), "+v"(dsk[1]));
    // dQ^T += K^T dS^T over this wavefront's 128 columns (keys past the end
    // are zero rows of K: their dS adds nothing); product x: k-step x / 4,
    // column block x % 4, its transposed A operand read four products ahead
    auto tr_a = [&](int x) __attribute__((always_inline)) -> u32x4_t {
      const char* pk = st + tbase + 16 * (x >> 2) * WRBL + 64 * (4 * ch + (x & 3));
      const u32x2_t a0 = lds_read_tr(pk), a1 = lds_read_tr(pk + 2 * WRBL);
      return u32x4_t{a0[0], a0[1], a1[0], a1[1]};
    };
    u32x4_t fr[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) fr[x] = tr_a(x);
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const u32x4_t a = fr[x % 4];
      if (x + 4 < 8) fr[x % 4] = tr_a(x + 4);
      PM::macc(acc[x & 3], a, dsk[x >> 2]);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (s + 1 < n_st) {
      char* nx = smem + ((s + 1) & 1) * STG;
      lk_.store(nx, tid);
      lv_.store(nx + WBLK, tid);
    }
    __syncthreads();
  }

  PM::wait_acc(acc[0], acc[1], acc[2], acc[3]);
  u32x2_t od[4][4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int gg = 0; gg < 4; ++gg)
      od[db][gg] = u32x2_t{TR::pack2(acc[db][4 * gg] * scale, acc[db][4 * gg + 1] * scale),
                           TR::pack2(acc[db][4 * gg + 2] * scale, acc[db][4 * gg + 3] * scale)};
  const size_t dq_off = (size_t)((int64_t)b * g.dq.sb + (int64_t)hd * g.dq.sh + (int64_t)(sq + qw) * g.dq.sr);
  static_assert(4 * kTileRowsBytes<128> <= 2 * STG, "four 32 x 128 tiles fit the stages");
  store_tile_rows<128>(smem + w * kTileRowsBytes<128>, od, dQ + dq_off + 128 * ch, min(32, Lq - qw), lane,
                       (size_t)g.dq.sr);
}

template <class TR, bool CAUSAL>
static hipError_t wide_t(const BwdArgs& a, int stage) {
  if (stage == BWD_DKDV) {
    const int n_ktiles = (a.Nk + 63) / 64;
    hipLaunchKernelGGL((bwd_dkdv_wide_kernel<TR, CAUSAL>), dim3((uint32_t)(n_ktiles * a.BH)), dim3(256), 0,
                       a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                       (const uint16_t*)a.dout, a.lse, a.dvec, (uint16_t*)a.dk, (uint16_t*)a.dv, a.Nq, a.Nk,
                       n_ktiles, a.c, a.scale, a.g);
  } else {
    const int n_qtiles = (a.Nq + 63) / 64;
    hipLaunchKernelGGL((bwd_dq_wide_kernel<TR, CAUSAL>), dim3((uint32_t)(n_qtiles * a.BH)), dim3(256), 0,
                       a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                       (const uint16_t*)a.dout, a.lse, a.dvec, (uint16_t*)a.dq, a.Nq, a.Nk, n_qtiles, a.c,
                       a.scale, a.g);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_wide_stage(const BwdArgs& a, int stage) {
  if (a.dtype == DT_BF16) return a.causal ? wide_t<BF16, true>(a, stage) : wide_t<BF16, false>(a, stage);
  return a.causal ? wide_t<F16, true>(a, stage) : wide_t<F16, false>(a, stage);
}

}  // namespace fa
