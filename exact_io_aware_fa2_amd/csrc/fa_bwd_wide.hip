// Backward attention for head dimension 256 on gfx950.
//
// The gradient is fa_bwd.hip's (chain rule through the softmax, scores and
// probabilities recomputed from Q, K and the LSE instead of stored:
// "FlashAttention" lexicon, "Methodische Grundlagen", "Neuberechnung statt
// Speicherung"); only the work split differs, because at d = 256 one
// wavefront cannot hold the B operands of the score products over all 256
// columns (K and V, or Q and dO: 128 registers) together with the
// accumulators of both dK and dV (256 registers).
// - dK, dV: every 32-key block is shared by two wavefronts, each
//   accumulating one half of the gradients' columns; both compute the
//   block's scores and dP over all 256 columns (those products are done
//   twice).
// - dQ: one gradient, so a wavefront holds its 32 queries' Q and dO operands
//   and all 256 columns of dQ (256 AGPRs), and every score and dP product is
//   done once.
// Both kernels are software-pipelined inside each wavefront: the vector work
// of one 32-row block runs between the matrix products of its neighbours,
// the rows stream through four LDS stage slots with one workgroup barrier
// per block, and one workgroup of four wavefronts runs per compute unit (512
// registers per wavefront, the score operands and the gradient accumulators
// in AGPRs).
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

}  // namespace

// dK, dV for d = 256, software-pipelined inside each wavefront (the scheme
// of fa_bwd.hip's dK/dV kernel, with 32-row stages): a workgroup takes 64
// keys, wavefront w the keys k0 + 32 (w / 2) and the columns 128 (w % 2) ..
// +127 of dK and dV.  Iteration b (query rows i_begin + 32 b .. +31, stage
// slot b % 4) issues
//   matrix: dV^T += dO_{b-1}^T P_{b-1}, dK^T += Q_{b-1}^T dS_{b-1} (8 each,
//           this wavefront's columns), S'_{b+1} = Q_{b+1} K^T - LSE / s and
//           dP_{b+1} = dO_{b+1} V^T - D (16 each, all 256 columns)
//   vector: P_b = exp2(S'_b c), dS_b = P_b (dP_b - D), rounded and packed
// one product after another with the vector work between them (c = s log2 e,
// s the scale; -LSE / s and -D enter as the accumulators' initial values).
// The stage of block b+2 is written to LDS during iteration b from
// registers loaded during iteration b-1; one workgroup barrier per
// iteration.  The first four products of an iteration are dV/dK products
// (slot b-1), so the operand reads issued for them at the end of the
// previous iteration never touch the slot being written.
template <class TR, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dkdv_wpipe_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                           const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                           const float* __restrict__ LSE, const float* __restrict__ Dvec,
                           uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int Nq, int Nk, int n_ktiles,
                           uint32_t total,                           float c, float neg_inv_scale, float scale, GenLayout g) {
  constexpr int NT = 256;
  constexpr int OFF_V = 2 * WBLK;            // -LSE / s (32 floats), then -D (32 floats)
  constexpr int STG = OFF_V + 2 * 32 * 4;    // one stage slot
  constexpr int NCH = 32 * (WD / 8) / NT;    // 16-byte chunks per thread and tensor (4)
  constexpr int NPART = 2 * NCH + 1;         // staging parts: Q chunks, dO chunks, the vectors
  constexpr int NSL = 48;                    // products per iteration
  constexpr int AH = 4;                      // operand reads issued ahead of their product
  constexpr int kW0 = 8, kL0 = 20;           // first staging write, first staging load (product index)
  static_assert(kW0 + NPART <= kL0 && kL0 + NPART <= NSL, "staging fits the iteration");
  static_assert(4 * STG <= 160 * 1024, "four stage slots fit in LDS");
  using PM = PipeMma<TR, true>;  // K, V (score operands) and dK, dV (accumulators) in AGPRs
  __shared__ __attribute__((aligned(16))) char smem[4 * STG];

  auto run_tile = [&](const uint32_t lid) __attribute__((always_inline)) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int h = lane >> 5;
  const int l32 = lane & 31;
  const int ch = w & 1;  // gradient column half
  const float s_out = neg_inv_scale < 0.0f ? -INFINITY : INFINITY;  // initial S of rows past the end

  const int bh = lid / n_ktiles;
  const int k0 = (lid % n_ktiles) * 64;
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
  const int nrows = min(32, Lk - kw);
  const size_t dk_off = (size_t)((int64_t)b * g.dk.sb + (int64_t)hd * g.dk.sh + (int64_t)(sk + kw) * g.dk.sr);
  const size_t dv_off = (size_t)((int64_t)b * g.dv.sb + (int64_t)hd * g.dv.sh + (int64_t)(sk + kw) * g.dv.sr);

  const int i_begin = CAUSAL ? max(0, k0 - delta) : 0;
  const int n_st = (Lq - i_begin + 31) / 32;
  if (n_st <= 0) {
    // no query sees these keys (an empty query sequence): dK = dV = 0
    const u32x4_t z = {0u, 0u, 0u, 0u};
    for (int i = lane; i < 32 * 16; i += 64) {
      const int r = i / 16, cc = i % 16;
      if (r < nrows) {
        *(u32x4_t*)(dK + dk_off + (size_t)r * g.dk.sr + 128 * ch + 8 * cc) = z;
        *(u32x4_t*)(dV + dv_off + (size_t)r * g.dv.sr + 128 * ch + 8 * cc) = z;
      }
    }
    return;
  }

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

  // ---- staging: part j < NCH: chunk tid + 256 j of the Q tile (row
  // (tid + 256 j) / 32, 16-byte column % 32), then the same of dO, then (wave
  // 0) the vectors at position m = lane % 32: row perm(m), -LSE / s for lanes
  // 0..31 and -D for lanes 32..63.
  const rsrc_t qres = make_rsrc(Q + tq.off, tq.bytes), ores = make_rsrc(dO + tdo.off, tdo.bytes);
  u32x4_t sgq[NCH], sgo[NCH];
  float vraw = 0.0f;
  int vrow = 0;
  auto load_part = [&](int i0, int j) __attribute__((always_inline)) {
    if (j < NCH) {
      const int i = tid + NT * j;
      sgq[j] = buf_load16(qres, (uint32_t)(i0 + i / 32) * tq.rs + 16 * (i % 32));
    } else if (j < 2 * NCH) {
      const int i = tid + NT * (j - NCH);
      sgo[j - NCH] = buf_load16(ores, (uint32_t)(i0 + i / 32) * tdo.rs + 16 * (i % 32));
    } else if (w == 0) {
      vrow = i0 + wperm(l32);
      vraw = vrow < Lq ? (h == 0 ? LSE[l_off + vrow] : Dvec[l_off + vrow]) : 0.0f;
    }
  };
  auto store_part = [&](char* st, int j) __attribute__((always_inline)) {
    if (j < NCH) {
      const int i = tid + NT * j;
      *(u32x4_t*)(st + (i / 32) * WRBL + 16 * (i % 32)) = sgq[j];
    } else if (j < 2 * NCH) {
      const int i = tid + NT * (j - NCH);
      *(u32x4_t*)(st + WBLK + (i / 32) * WRBL + 16 * (i % 32)) = sgo[j - NCH];
    } else if (w == 0) {
      // rows past the end: an S of the sign of -1 / s makes S c = -inf (P = 0); D = 0
      const bool in = vrow < Lq;
      ((float*)(st + OFF_V))[lane] = h == 0 ? (in ? vraw * neg_inv_scale : s_out) : (in ? -vraw : 0.0f);
    }
  };
  auto slot = [&](int blk) __attribute__((always_inline)) -> char* { return smem + (blk & 3) * STG; };

  // ---- operands.  Row reads (S, dP): row perm(l32), chunk h (+ 2 ks);
  // transposed reads (dK, dV): as the other backward kernels
  const uint32_t rbase = (uint32_t)(wperm(l32) * WRBL + 16 * h);
  const int L16 = lane & 15, G = lane >> 4;
  const uint32_t tbase = (uint32_t)((h + 4 * (L16 >> 2)) * WRBL + (16 * (G & 1) + 4 * (L16 & 3)) * 2);
  auto row_frag = [&](const char* st, int tensor, int ks) __attribute__((always_inline)) -> u32x4_t {
    return *(const u32x4_t*)(st + tensor * WBLK + rbase + 32 * ks);
  };
  // tensor 0: Q^T (dK), 1: dO^T (dV); k-step t of 16 rows, column block db of this half
  auto tr_frag = [&](const char* st, int tensor, int t, int db) __attribute__((always_inline)) -> u32x4_t {
    const char* p = st + tensor * WBLK + tbase + 16 * t * WRBL + 64 * (4 * ch + db);
    const u32x2_t a0 = lds_read_tr(p), a1 = lds_read_tr(p + 2 * WRBL);
    return u32x4_t{a0[0], a0[1], a1[0], a1[1]};
  };
  // initial values of the S and dP accumulators of a block: -LSE / s, -D of its rows
  auto load_vecs = [&](const char* st, f32x16_t& l, f32x16_t& d) __attribute__((always_inline)) {
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) {
      const float4 l4 = *(const float4*)(st + OFF_V + 32 * gg + 16 * h);
      const float4 d4 = *(const float4*)(st + OFF_V + 128 + 32 * gg + 16 * h);
      l[4 * gg + 0] = l4.x; l[4 * gg + 1] = l4.y; l[4 * gg + 2] = l4.z; l[4 * gg + 3] = l4.w;
      d[4 * gg + 0] = d4.x; d[4 * gg + 1] = d4.y; d[4 * gg + 2] = d4.z; d[4 * gg + 3] = d4.w;
    }
  };
  // product k of an iteration: kind 0: dV (t, db), 1: dK (t, db), 2: S k-step,
  // 3: dP k-step.  Products 0..3: dV/dK of (t, db) = (0, 0), (0, 1); then six
  // groups of [S, dP, S, dP, dV, dK]; then the last four S/dP k-steps.
  struct Prod { int kind, t, db, ks; };
  auto prod = [](int k) constexpr -> Prod {
    if (k < 4) return Prod{k & 1, 0, k >> 1, 0};
    if (k < 40) {
      const int gi = (k - 4) / 6, p = (k - 4) % 6;
      if (p < 4) return Prod{2 + (p & 1), 0, 0, 2 * gi + (p >> 1)};
      const int x = 2 + gi;  // dV/dK pair index 2..7
      return Prod{p - 4, x >> 2, x & 3, 0};
    }
    const int x = k - 40;
    return Prod{2 + (x & 1), 0, 0, 12 + (x >> 1)};
  };
  auto frag = [&](int k, const char* sb1, const char* sb2) __attribute__((always_inline)) -> u32x4_t {
    const Prod p = prod(k);
    if (p.kind == 0) return tr_frag(sb2, 1, p.t, p.db);
    if (p.kind == 1) return tr_frag(sb2, 0, p.t, p.db);
    return row_frag(sb1, p.kind - 2, p.ks);
  };

  f32x16_t sc[2], dp[2];
  u32x4_t pk[2][2], dsk[2][2];  // [set][k-step t]: P and dS rounded, packed in pairs
  u32x4_t fr[AH];

  // ---- one iteration (block bb, PAR = bb % 2)
  auto iteration = [&](auto par_c, int bb) __attribute__((always_inline)) {
    constexpr int PAR = decltype(par_c)::value;
    constexpr int NB = 1 - PAR;
    const char* sb1 = slot(bb + 1);
    const char* sb2 = slot(bb - 1);
    // S_b, dP_b were written by matrix instructions, P and dS of block b-1 by
    // vector instructions: all of them ordered before what reads them next
    mfma_wait_v(sc[PAR], dp[PAR]);
    asm volatile("s_nop 1" : "+v"(pk[NB][0]), "+v"(pk[NB][1]), "+v"(dsk[NB][0]), "+v"(dsk[NB][1]));
    load_vecs(sb1, sc[NB], dp[NB]);
    const int i0 = i_begin + 32 * bb;
    // causal: key kw + l32 is visible to the query of score r iff thr <= qoff(r)
    const int thr = kw - delta - i0 + l32 - h;
    float pe[16], dsv[16];
    auto vwork = [&](int k) __attribute__((always_inline)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (k == 3 * r) {
          float x = sc[PAR][r] * c;
          if constexpr (CAUSAL) {
            const int gq = r / 4, e = r % 4;
            const int qoff = 16 * (gq / 2) + 4 * e + 2 * (gq % 2);
            x = thr <= qoff ? x : -INFINITY;
          }
          pe[r] = fast_exp2(x);
          pin(pe[r]);
        }
        if (k == 3 * r + 1) {
          dsv[r] = pe[r] * dp[PAR][r];  // dp holds dP - D
          pin(dsv[r]);
          if (r & 1) {
            uint32_t p2 = TR::pack2(pe[r - 1], pe[r]), d2 = TR::pack2(dsv[r - 1], dsv[r]);
            pin(p2);
            pin(d2);
            pk[PAR][r / 8][(r / 2) % 4] = p2;
            dsk[PAR][r / 8][(r / 2) % 4] = d2;
          }
        }
      }
      // staging: the stage of block b+2 into its slot, then the loads of block b+3
      if (k >= kW0 && k < kW0 + NPART) store_part(slot(bb + 2), k - kW0);
      if (k >= kL0 && k < kL0 + NPART) load_part(i0 + 96, k - kL0);
    };
    static_for<0, NSL>([&](auto kc) __attribute__((always_inline)) {
      constexpr int k = decltype(kc)::value;
      constexpr Prod p = prod(k);
      const u32x4_t a = fr[k % AH];
      if constexpr (k + AH < NSL) fr[k % AH] = frag(k + AH, sb1, sb2);
      else fr[k % AH] = frag(k + AH - NSL, slot(bb + 2), slot(bb));  // next iteration's dV/dK operands
      if constexpr (p.kind == 0) PM::macc(acc_dv[p.db], a, pk[NB][p.t]);
      else if constexpr (p.kind == 1) PM::macc(acc_dk[p.db], a, dsk[NB][p.t]);
      else if constexpr (p.kind == 2) PM::mb(sc[NB], a, kf[p.ks]);
      else PM::mb(dp[NB], a, vf[p.ks]);
      vwork(k);
      __builtin_amdgcn_sched_barrier(0);
    });
    lds_barrier();
  };

  // ---- prologue: stages 0 and 1 in slots 0 and 1, slot 3 zeroed (block -1:
  // its products multiply it by zero P and dS), block 2 requested; S_0, dP_0;
  // the first operands
#pragma unroll
  for (int j = 0; j < NPART; ++j) load_part(i_begin, j);
#pragma unroll
  for (int j = 0; j < NPART; ++j) store_part(slot(0), j);
#pragma unroll
  for (int j = 0; j < NPART; ++j) load_part(i_begin + 32, j);
#pragma unroll
  for (int j = 0; j < NPART; ++j) store_part(slot(1), j);
  for (int i = tid; i < STG / 16; i += NT) *(u32x4_t*)(slot(3) + 16 * i) = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < NPART; ++j) load_part(i_begin + 64, j);
  lds_barrier();
  PM::copy_wait(acc_dk[0], acc_dk[1], acc_dk[2], acc_dk[3], acc_dv[0], acc_dv[1], acc_dv[2], acc_dv[3]);
  load_vecs(slot(0), sc[0], dp[0]);
  mma_pipeline<2 * WKS, 3>([&](int x) { return slot(0) + ((x & 1) ? WBLK : 0) + rbase + 32 * (x >> 1); },
                           [&](int x, u32x4_t a) {
                             const int ks = x >> 1;
                             if (x & 1) PM::mb(dp[0], a, vf[ks]);
                             else PM::mb(sc[0], a, kf[ks]);
                           },
                           [](int) {});
#pragma unroll
  for (int t = 0; t < 2; ++t) pk[1][t] = dsk[1][t] = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
  for (int x = 0; x < AH; ++x) fr[x] = frag(x, slot(1), slot(3));

  for (int bb = 0; bb < n_st; bb += 2) {
    iteration(std::integral_constant<int, 0>{}, bb);
    if (bb + 1 < n_st) iteration(std::integral_constant<int, 1>{}, bb + 1);
  }

  // ---- the last block's dV, dK products (register set (n_st - 1) % 2)
  auto last = [&](auto par_c) __attribute__((always_inline)) {
    constexpr int PAR = decltype(par_c)::value;
    const char* st = slot(n_st - 1);
    asm volatile("s_nop 1" : "+v"(pk[PAR][0]), "+v"(pk[PAR][1]), "+v"(dsk[PAR][0]), "+v"(dsk[PAR][1]));
    PM::copy_wait(acc_dk[0], acc_dk[1], acc_dk[2], acc_dk[3], acc_dv[0], acc_dv[1], acc_dv[2], acc_dv[3]);
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      PM::macc(acc_dv[x & 3], tr_frag(st, 1, x >> 2, x & 3), pk[PAR][x >> 2]);
      PM::macc(acc_dk[x & 3], tr_frag(st, 0, x >> 2, x & 3), dsk[PAR][x >> 2]);
    }
    // before the two paths join: the compiler may copy the accumulators
    // between registers there, and a copy reads the products' results
    PM::wait_acc(acc_dk[0], acc_dk[1], acc_dk[2], acc_dk[3], acc_dv[0], acc_dv[1], acc_dv[2], acc_dv[3]);
  };
  if (n_st & 1) last(std::integral_constant<int, 0>{});
  else last(std::integral_constant<int, 1>{});

  // dK (times the scale) and dV, this wavefront's 128 columns of its 32 keys,
  // as whole rows through LDS
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
  lds_barrier();  // every wavefront is done with the stage slots
  static_assert(8 * kTileRowsBytes<128> <= 4 * STG, "eight 32 x 128 tiles fit the stage slots");
  store_tile_rows<128>(smem + w * kTileRowsBytes<128>, ok, dK + dk_off + 128 * ch, nrows, lane, (size_t)g.dk.sr);
  store_tile_rows<128>(smem + (4 + w) * kTileRowsBytes<128>, ov, dV + dv_off + 128 * ch, nrows, lane,
                       (size_t)g.dv.sr);
  };
  // a workgroup takes tile t and tile nt - 1 - t of one head (with the causal
  // mask, equal work; the middle tile of an odd count once), and the
  // workgroups of one head run on one XCD and share its L2
  const uint32_t nt = (uint32_t)n_ktiles, npair = (nt + 1) / 2;
  const uint32_t pid = xcd_remap(blockIdx.x, total);
  const uint32_t hh = pid / npair, tt = pid % npair;
  run_tile(hh * nt + tt);
  if (nt - 1 - tt != tt) {
    lds_barrier();
    run_tile(hh * nt + nt - 1 - tt);
  }
}

// dQ for d = 256 with one wavefront per 32 queries: a workgroup takes 128
// queries, wavefront w the queries q0 + 32 w .. +31 and all 256 columns of
// dQ (eight 32 x 32 accumulators in AGPRs beside the Q and dO operands), so
// that every block's scores and dP are computed once.  Iteration b (keys
// 32 b .. +31, stage slot b % 4) issues
//   matrix: dQ^T += K_{b-1}^T dS^T_{b-1} (16), S^T_{b+1} = K_{b+1} Q^T,
//           dP^T_{b+1} = V_{b+1} dO^T - D (16 each)
//   vector: P_b = exp2(S^T_b c - LSE log2 e), dS_b = P_b (dP_b - D), packed
// one product after another with the vector work between them; the K and V
// rows of block b+2 are written to LDS during iteration b from registers
// loaded during iteration b-1; one workgroup barrier per iteration.  The
// first four products of an iteration are dQ products (slot b-1), so the
// operand reads issued for them at the end of the previous iteration never
// touch the slot being written.
template <class TR, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dq_q128_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                        const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                        const float* __restrict__ LSE, const float* __restrict__ Dvec, uint16_t* __restrict__ dQ,
                        int Nq, int Nk, int n_qtiles, uint32_t total, float c, float scale,
                        GenLayout g) {
  constexpr int NT = 256;
  constexpr int STG = 2 * WBLK;              // one stage slot: K, V rows of 32 keys
  constexpr int NCH = 32 * (WD / 8) / NT;    // 16-byte chunks per thread and tensor (4)
  constexpr int NPART = 2 * NCH;             // staging parts: K chunks, V chunks
  constexpr int NSL = 48;                    // products per iteration
  constexpr int AH = 4;                      // operand reads issued ahead of their product
  constexpr int kW0 = 6, kL0 = 20;           // first staging write, first staging load
  static_assert(kW0 + NPART <= kL0 && kL0 + NPART <= NSL, "staging fits the iteration");
  static_assert(4 * STG <= 160 * 1024, "four stage slots fit in LDS");
  using PM = PipeMma<TR, true>;  // Q, dO (score operands) and dQ (accumulators) in AGPRs
  __shared__ __attribute__((aligned(16))) char smem[4 * STG];

  auto run_tile = [&](const uint32_t lid) __attribute__((always_inline)) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int h = lane >> 5;
  const int l32 = lane & 31;

  const int bh = lid / n_qtiles;
  int qt = lid % n_qtiles;
  if (CAUSAL) qt = n_qtiles - 1 - qt;  // longest rows first
  const int q0 = qt * 128;
  const int qw = q0 + 32 * w;
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
  f32x16_t negd;  // initial value of the dP accumulators
#pragma unroll
  for (int i = 0; i < 16; ++i) negd[i] = -dd;
  f32x16_t acc[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) acc[db] = zero16();

  // keys up to the last one visible to the workgroup's last query; the
  // blocks past a wavefront's own last visible key add zeros
  const int kv_end = CAUSAL ? min(Lk, q0 + 128 + delta) : Lk;
  const int n_st = kv_end > 0 ? (kv_end + 31) / 32 : 0;
  if (n_st > 0) {
    const rsrc_t kres = make_rsrc(K + tk.off, tk.bytes), vres = make_rsrc(V + tv.off, tv.bytes);
    // ---- staging: part j < NCH: chunk tid + 256 j of the K tile (row
    // (tid + 256 j) / 32, 16-byte column % 32; rows past the end read
    // zeros), then the same of V
    u32x4_t sgk[NCH], sgv[NCH];
    auto load_part = [&](int j0, int j) __attribute__((always_inline)) {
      const int i = tid + NT * (j % NCH);
      if (j < NCH) sgk[j] = buf_load16(kres, (uint32_t)(j0 + i / 32) * tk.rs + 16 * (i % 32));
      else sgv[j - NCH] = buf_load16(vres, (uint32_t)(j0 + i / 32) * tv.rs + 16 * (i % 32));
    };
    auto store_part = [&](char* st, int j) __attribute__((always_inline)) {
      const int i = tid + NT * (j % NCH);
      if (j < NCH) *(u32x4_t*)(st + (i / 32) * WRBL + 16 * (i % 32)) = sgk[j];
      else *(u32x4_t*)(st + WBLK + (i / 32) * WRBL + 16 * (i % 32)) = sgv[j - NCH];
    };
    auto slot = [&](int blk) __attribute__((always_inline)) -> char* { return smem + (blk & 3) * STG; };

    const uint32_t rbase = (uint32_t)(wperm(l32) * WRBL + 16 * h);
    const int L16 = lane & 15, G = lane >> 4;
    const uint32_t tbase = (uint32_t)((h + 4 * (L16 >> 2)) * WRBL + (16 * (G & 1) + 4 * (L16 & 3)) * 2);
    // A operand of S^T (tensor 0: K) or dP^T (tensor 1: V), k-step ks
    auto row_frag = [&](const char* st, int tensor, int ks) __attribute__((always_inline)) -> u32x4_t {
      return *(const u32x4_t*)(st + tensor * WBLK + rbase + 32 * ks);
    };
    // A operand of dQ^T (K^T): k-step t of 16 keys, column block db
    auto tr_frag = [&](const char* st, int t, int db) __attribute__((always_inline)) -> u32x4_t {
      const char* p = st + tbase + 16 * t * WRBL + 64 * db;
      const u32x2_t a0 = lds_read_tr(p), a1 = lds_read_tr(p + 2 * WRBL);
      return u32x4_t{a0[0], a0[1], a1[0], a1[1]};
    };
    // product k of an iteration: kind 0: dQ (k-step t, column block db), 2:
    // S^T k-step ks, 3: dP^T k-step ks.  Products 0..3: dQ (0, 0..3); then
    // twelve groups [S, dP, dQ] (S, dP k-step g, dQ number g + 4); then the
    // S, dP k-steps 12..15.
    struct Prod { int kind, t, db, ks; };
    auto prod = [](int k) constexpr -> Prod {
      if (k < 4) return Prod{0, 0, k, 0};
      if (k < 40) {
        const int gi = (k - 4) / 3, p = (k - 4) % 3;
        if (p < 2) return Prod{2 + p, 0, 0, gi};
        return Prod{0, (gi + 4) / 8, (gi + 4) % 8, 0};
      }
      const int x = k - 40;
      return Prod{2 + (x & 1), 0, 0, 12 + (x >> 1)};
    };
    auto frag = [&](int k, const char* sb1, const char* sb2) __attribute__((always_inline)) -> u32x4_t {
      const Prod p = prod(k);
      if (p.kind == 0) return tr_frag(sb2, p.t, p.db);
      return row_frag(sb1, p.kind - 2, p.ks);
    };

    f32x16_t sc[2], dp[2];
    u32x4_t dsk[2][2];  // [set][k-step t]: dS rounded, packed in pairs
    u32x4_t fr[AH];

    auto iteration = [&](auto par_c, int bb) __attribute__((always_inline)) {
      constexpr int PAR = decltype(par_c)::value;
      constexpr int NB = 1 - PAR;
      const char* sb1 = slot(bb + 1);
      const char* sb2 = slot(bb - 1);
      mfma_wait_v(sc[PAR], dp[PAR]);
      asm volatile("s_nop 1" : "+v"(dsk[NB][0]), "+v"(dsk[NB][1]));
      const int j0 = 32 * bb;
      const int thr = qrow + delta - j0 - h;  // causal: key j0 + koff(r) visible iff koff(r) <= thr
      float pe[16];
      auto vwork = [&](int k) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if (k == 2 * r) {
            float x = fmaf(sc[PAR][r], c, -lq);
            if constexpr (CAUSAL) {
              const int gq = r / 4, e = r % 4;
              const int koff = 16 * (gq / 2) + 4 * e + 2 * (gq % 2);
              x = koff <= thr ? x : -INFINITY;
            }
            pe[r] = fast_exp2(x) * dp[PAR][r];  // dS (dp holds dP - D)
            pin(pe[r]);
          }
          if (k == 2 * r + 1 && (r & 1)) {
            uint32_t d2 = TR::pack2(pe[r - 1], pe[r]);
            pin(d2);
            dsk[PAR][r / 8][(r / 2) % 4] = d2;
          }
        }
        if (k >= kW0 && k < kW0 + NPART) store_part(slot(bb + 2), k - kW0);
        if (k >= kL0 && k < kL0 + NPART) load_part(j0 + 96, k - kL0);
      };
      static_for<0, NSL>([&](auto kc) __attribute__((always_inline)) {
        constexpr int k = decltype(kc)::value;
        constexpr Prod p = prod(k);
        const u32x4_t a = fr[k % AH];
        if constexpr (k + AH < NSL) fr[k % AH] = frag(k + AH, sb1, sb2);
        else fr[k % AH] = frag(k + AH - NSL, slot(bb + 2), slot(bb));  // next iteration's dQ operands
        if constexpr (p.kind == 0) PM::macc(acc[p.db], a, dsk[NB][p.t]);
        else if constexpr (p.kind == 2) {
          if constexpr (p.ks == 0) sc[NB] = PM::mb0(a, qf[0]);
          else PM::mb(sc[NB], a, qf[p.ks]);
        } else {
          if constexpr (p.ks == 0) dp[NB] = PM::mbc(a, of[0], negd);
          else PM::mb(dp[NB], a, of[p.ks]);
        }
        vwork(k);
        __builtin_amdgcn_sched_barrier(0);
      });
      lds_barrier();
    };

    // ---- prologue: blocks 0 and 1 in slots 0 and 1, slot 3 zeroed (block
    // -1: multiplied by zero dS), block 2 requested; S^T_0, dP^T_0
#pragma unroll
    for (int j = 0; j < NPART; ++j) load_part(0, j);
#pragma unroll
    for (int j = 0; j < NPART; ++j) store_part(slot(0), j);
#pragma unroll
    for (int j = 0; j < NPART; ++j) load_part(32, j);
#pragma unroll
    for (int j = 0; j < NPART; ++j) store_part(slot(1), j);
    for (int i = tid; i < STG / 16; i += NT) *(u32x4_t*)(slot(3) + 16 * i) = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < NPART; ++j) load_part(64, j);
    lds_barrier();
    PM::copy_wait(acc[0], acc[1], acc[2], acc[3], acc[4], acc[5], acc[6], acc[7]);
    mma_pipeline<2 * WKS, 3>([&](int x) { return slot(0) + ((x & 1) ? WBLK : 0) + rbase + 32 * (x >> 1); },
                             [&](int x, u32x4_t a) {
                               const int ks = x >> 1;
                               if (x & 1) {
                                 if (ks == 0) dp[0] = PM::mbc(a, of[0], negd);
                                 else PM::mb(dp[0], a, of[ks]);
                               } else {
                                 if (ks == 0) sc[0] = PM::mb0(a, qf[0]);
                                 else PM::mb(sc[0], a, qf[ks]);
                               }
                             },
                             [](int) {});
#pragma unroll
    for (int t = 0; t < 2; ++t) dsk[1][t] = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int x = 0; x < AH; ++x) fr[x] = frag(x, slot(1), slot(3));

    for (int bb = 0; bb < n_st; bb += 2) {
      iteration(std::integral_constant<int, 0>{}, bb);
      if (bb + 1 < n_st) iteration(std::integral_constant<int, 1>{}, bb + 1);
    }

    // ---- the last block's dQ products (register set (n_st - 1) % 2)
    auto last = [&](auto par_c) __attribute__((always_inline)) {
      constexpr int PAR = decltype(par_c)::value;
      const char* st = slot(n_st - 1);
      asm volatile("s_nop 1" : "+v"(dsk[PAR][0]), "+v"(dsk[PAR][1]));
      PM::copy_wait(acc[0], acc[1], acc[2], acc[3], acc[4], acc[5], acc[6], acc[7]);
#pragma unroll
      for (int x = 0; x < 16; ++x) PM::macc(acc[x & 7], tr_frag(st, x >> 3, x & 7), dsk[PAR][x >> 3]);
      // before the two paths join (the compiler may copy the accumulators there)
      PM::wait_acc(acc[0], acc[1], acc[2], acc[3], acc[4], acc[5], acc[6], acc[7]);
    };
    if (n_st & 1) last(std::integral_constant<int, 0>{});
    else last(std::integral_constant<int, 1>{});
    lds_barrier();  // every wavefront is done with the stage slots
  }

  u32x2_t od[8][4];
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int gg = 0; gg < 4; ++gg)
      od[db][gg] = u32x2_t{TR::pack2(acc[db][4 * gg] * scale, acc[db][4 * gg + 1] * scale),
                           TR::pack2(acc[db][4 * gg + 2] * scale, acc[db][4 * gg + 3] * scale)};
  const size_t dq_off = (size_t)((int64_t)b * g.dq.sb + (int64_t)hd * g.dq.sh + (int64_t)(sq + qw) * g.dq.sr);
  static_assert(4 * kTileRowsBytes<256> <= 4 * STG, "four 32 x 256 tiles fit the stage slots");
  store_tile_rows<256>(smem + w * kTileRowsBytes<256>, od, dQ + dq_off, min(32, Lq - qw), lane, (size_t)g.dq.sr);
  };
  // a workgroup takes tile t and tile nt - 1 - t of one head (with the causal
  // mask, equal work; the middle tile of an odd count once), and the
  // workgroups of one head run on one XCD and share its L2
  const uint32_t nt = (uint32_t)n_qtiles, npair = (nt + 1) / 2;
  const uint32_t pid = xcd_remap(blockIdx.x, total);
  const uint32_t hh = pid / npair, tt = pid % npair;
  run_tile(hh * nt + tt);
  if (nt - 1 - tt != tt) {
    lds_barrier();
    run_tile(hh * nt + nt - 1 - tt);
  }
}

template <class TR, bool CAUSAL>
static hipError_t wide_t(const BwdArgs& a, int stage) {
  if (stage == BWD_DKDV) {
    const int n_ktiles = (a.Nk + 63) / 64;
    const uint32_t total = (uint32_t)(((n_ktiles + 1) / 2) * a.BH);  // workgroups
    // the exponent is (q.k - LSE / s) s log2 e with s the scale, of magnitude
    // at least 2^-100 so that -1 / s stays finite (as fa_bwd.hip's dK/dV)
    const float mag = fmaxf(fabsf(a.scale), 0x1p-100f);
    const float s = a.scale < 0.0f ? -mag : mag;
    hipLaunchKernelGGL((bwd_dkdv_wpipe_kernel<TR, CAUSAL>), dim3(total), dim3(256), 0,
                       a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                       (const uint16_t*)a.dout, a.lse, a.dvec, (uint16_t*)a.dk, (uint16_t*)a.dv, a.Nq, a.Nk,
                       n_ktiles, total, s * kLog2e, -1.0f / s, a.scale, a.g);
  } else {
    const int n_qtiles = (a.Nq + 127) / 128;
    const uint32_t total = (uint32_t)(((n_qtiles + 1) / 2) * a.BH);  // workgroups
    hipLaunchKernelGGL((bwd_dq_q128_kernel<TR, CAUSAL>), dim3(total), dim3(256), 0,
                       a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                       (const uint16_t*)a.dout, a.lse, a.dvec, (uint16_t*)a.dq, a.Nq, a.Nk, n_qtiles, total, a.c,
                       a.scale, a.g);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_wide_stage(const BwdArgs& a, int stage) {
  if (a.dtype == DT_BF16) return a.causal ? wide_t<BF16, true>(a, stage) : wide_t<BF16, false>(a, stage);
  return a.causal ? wide_t<F16, true>(a, stage) : wide_t<F16, false>(a, stage);
}

}  // namespace fa
