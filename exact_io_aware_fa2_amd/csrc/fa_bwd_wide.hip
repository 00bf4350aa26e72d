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
//   accumulating one half of the gradients' columns and computing the scores
//   and dP of one half of each 32-query block (16 x 16 x 32 products); the
//   two exchange their halves of P and dS through LDS.
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
// Layouts: in dQ, as in fa_bwd.hip, S^T accumulator row m of a 32-row block
// holds row perm(m) of the staged tile, so that the transposed LDS reads of
// the gradient products gather rows 4 apart (bank-conflict free); in dK/dV
// row m of a wavefront's 16 x 16 score tile holds staged row half_row(m) of
// its half, so that the P and dS values a lane holds go to consecutive
// positions of the exchange rows.  The per-row LSE and D values are staged
// in the order the accumulators read them.
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

// 16 x 16 x 32 products of the d = 256 dK/dV kernel below (B operand in AGPRs).
typedef float f32x4w_t __attribute__((ext_vector_type(4)));
template <class TR>
__device__ inline void mma16(f32x4w_t& c, u32x4_t a, u32x4_t b) {
  if constexpr (std::is_same_v<TR, BF16>) asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "a"(b));
  else asm("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "a"(b));
}
__device__ inline void mfma_wait4(f32x4w_t& a, f32x4w_t& b, f32x4w_t& c, f32x4w_t& d) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));  // 21 wait states
}
// staged row (0..15 within a half block) of row m of a 16 x 16 score tile:
// the four rows 4 g + i (i = 0..3) a lane holds land on consecutive positions
// of the exchange rows below
__device__ constexpr int half_row(int m) { return ((m >> 2) & 1) + 4 * (m & 3) + 2 * (m >> 3); }

// dK, dV for d = 256 with the scores split between the two wavefronts of a
// pair: a workgroup takes 64 keys, wavefront w the keys k0 + 32 (w / 2) and
// the columns 128 (w % 2) .. +127 of dK and dV (its K and V fragments cover
// all 256 columns, as S and dP need them), and it computes S and dP only
// for the 16 query rows 16 (w % 2) .. +15 of each 32-row block (16 x 16 x 32 products: 32 per block, half the work of the
// full 32 x 32 blocks), and the two wavefronts exchange their halves of P and
// dS (rounded, as the products use them) through LDS.  Iteration b (stage
// slot b % 4) issues
//   matrix: dV^T += dO_{b-1}^T P_{b-1}, dK^T += Q_{b-1}^T dS_{b-1}: first the
//           k-step of the wavefront's own rows (its P, dS read back from the
//           exchange area before the previous barrier), then, between the
//           S, dP products of block b+1, the partner's k-step (read after it)
//   vector: P_b = exp2(S'_b c), dS_b = P_b (dP_b - D) for its 16 rows,
//           written to the exchange area
// with one workgroup barrier per iteration.  Exchange row = key, 32
// positions of 16-bit values (80 bytes with padding), position 16 t + 8 h + j
// for the query the transposed read of the gradient products gives lane
// half h as its j-th value of k-step t.
template <class TR, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dkdv_half_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                          const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                          const float* __restrict__ LSE, const float* __restrict__ Dvec,
                          uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int Nq, int Nk, int n_ktiles,
                          uint32_t total, float c, float neg_inv_scale, float scale, GenLayout g) {
  constexpr int NT = 256;
  constexpr int OFF_V = 2 * WBLK;            // -LSE / s (32 floats), then -D (32 floats)
  constexpr int STG = OFF_V + 2 * 32 * 4;    // one stage slot
  constexpr int NCH = 32 * (WD / 8) / NT;    // 16-byte chunks per thread and tensor (4)
  constexpr int NPART = 2 * NCH + 1;         // staging parts: Q chunks, dO chunks, the vectors
  constexpr int NSL = 48;                    // products per iteration
  constexpr int NF = 32;                     // LDS operands per iteration
  constexpr int AH = 4;                      // operands read ahead of their last use
  constexpr int kW0 = 10, kL0 = 30;          // first staging write, first staging load (product index)
  constexpr int XP = 80;                     // exchange row bytes
  constexpr int XOFF = 4 * STG;              // exchange area: [pair][buffer][P, dS][key][position]
  constexpr int XBUF = 2 * 32 * XP, XPAIR = 2 * XBUF;
  static_assert(kW0 + NPART <= kL0 && kL0 + NPART <= NSL, "staging fits the iteration");
  static_assert(XOFF + 2 * XPAIR <= 160 * 1024, "stage slots and exchange area fit in LDS");
  using PM = PipeMma<TR, true>;  // dK, dV accumulators in AGPRs
  __shared__ __attribute__((aligned(16))) char smem[XOFF + 2 * XPAIR];

  auto run_tile = [&](const uint32_t lid) __attribute__((always_inline)) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int h = lane >> 5;
  const int l32 = lane & 31;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int ch = w & 1;  // gradient column half and query half
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

  // K and V rows of this wavefront's keys as B operands of the 16 x 16 x 32
  // score products: [key half nb][k-step ks], lane: key 16 nb + lane % 16,
  // columns 32 ks + 8 (lane / 16) .. +7
  u32x4_t kf[2][8], vf[2][8];
  {
    const rsrc_t kres = make_rsrc(K + tk.off, tk.bytes), vres = make_rsrc(V + tv.off, tv.bytes);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const int key = kw + 16 * nb + l16;
        kf[nb][ks] = buf_load16(kres, (uint32_t)key * tk.rs + 64 * ks + 16 * g4);
        vf[nb][ks] = buf_load16(vres, (uint32_t)key * tv.rs + 64 * ks + 16 * g4);
      }
  }
  f32x16_t acc_dk[4], acc_dv[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) acc_dk[db] = acc_dv[db] = zero16();

  // ---- staging: part j < NCH: chunk tid + 256 j of the Q tile (row
  // (tid + 256 j) / 32, 16-byte column % 32), then the same of dO, then (wave
  // 0) the vectors at position p = lane % 32 (row 16 (p / 16) + half_row(p %
  // 16)), -LSE / s for lanes 0..31 and -D for lanes 32..63.
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
      vrow = i0 + 16 * (l32 >> 4) + half_row(l32 & 15);
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
  char* const xpair = smem + XOFF + (w >> 1) * XPAIR;
  // exchange addresses: this lane's write (key half nb, P or dS) and its read
  // (k-step t, P or dS) in buffer buf
  auto xw = [&](int buf, int which, int nb) __attribute__((always_inline)) -> char* {
    return xpair + buf * XBUF + which * 32 * XP + (16 * nb + l16) * XP + 2 * (16 * ch + 8 * (g4 & 1) + 4 * (g4 >> 1));
  };
  auto xr = [&](int buf, int which, int t) __attribute__((always_inline)) -> const u32x4_t* {
    return (const u32x4_t*)(xpair + buf * XBUF + which * 32 * XP + l32 * XP + 2 * (16 * t + 8 * h));
  };

  // ---- operands.  Score rows (16 x 16 x 32 A operand): row 16 ch +
  // half_row(lane % 16), columns 32 ks + 8 (lane / 16); transposed reads (dK,
  // dV): as the other backward kernels
  const uint32_t rbase = (uint32_t)((16 * ch + half_row(l16)) * WRBL + 16 * g4);
  const int G = lane >> 4;
  const uint32_t tbase = (uint32_t)((h + 4 * (l16 >> 2)) * WRBL + (16 * (G & 1) + 4 * (l16 & 3)) * 2);
  auto row_frag = [&](const char* st, int tensor, int ks) __attribute__((always_inline)) -> u32x4_t {
    return *(const u32x4_t*)(st + tensor * WBLK + rbase + 64 * ks);
  };
  // tensor 0: Q^T (dK), 1: dO^T (dV); k-step t of 16 rows, column block db of this half
  auto tr_frag = [&](const char* st, int tensor, int t, int db) __attribute__((always_inline)) -> u32x4_t {
    const char* p = st + tensor * WBLK + tbase + 16 * t * WRBL + 64 * (4 * ch + db);
    const u32x2_t a0 = lds_read_tr(p), a1 = lds_read_tr(p + 2 * WRBL);
    return u32x4_t{a0[0], a0[1], a1[0], a1[1]};
  };
  // initial values of this wavefront's S and dP tiles of a block: -LSE / s, -D of its rows
  auto load_vecs = [&](const char* st, f32x4w_t (&l)[2], f32x4w_t (&d)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      l[nb] = *(const f32x4w_t*)(st + OFF_V + 4 * (16 * ch + 4 * g4));
      d[nb] = *(const f32x4w_t*)(st + OFF_V + 128 + 4 * (16 * ch + 4 * g4));
    }
    // the compiler may load once and copy: two wait states before the
    // products that accumulate into them
    asm volatile("s_nop 1" : "+v"(l[0]), "+v"(l[1]), "+v"(d[0]), "+v"(d[1]));
  };
  // LDS operand f of an iteration: 0..7 the own k-step's dV (even) / dK (odd)
  // operands of column block f / 2; then per group gi: Q rows, dO rows (k-step
  // gi of the scores), the partner k-step's gradient operand number gi.
  // Product k: 0..7 own gradient products; then eight groups [S nb 0, dP nb 0,
  // S nb 1, dP nb 1, partner gradient product gi].
  // kind 0 dV, 1 dK (x: own 0 / partner 1 k-step, column block db), 2 S, 3 dP
  // (key half nb); last: the operand's last use
  struct Prod { int kind, f, nb, last, x, db; };
  auto prod = [](int k) constexpr -> Prod {
    if (k < 8) return Prod{k & 1, k, 0, 1, 0, k >> 1};
    const int gi = (k - 8) / 5, p = (k - 8) % 5;
    if (p < 4) return Prod{2 + (p & 1), 8 + 3 * gi + (p & 1), p >> 1, p >> 1, 0, 0};
    return Prod{gi & 1, 8 + 3 * gi + 2, 0, 1, 1, gi >> 1};
  };
  auto frag = [&](int f, const char* sb1, const char* sb2) __attribute__((always_inline)) -> u32x4_t {
    if (f < 8) return tr_frag(sb2, (f & 1) ? 0 : 1, ch, f >> 1);
    const int gi = (f - 8) / 3, r = (f - 8) % 3;
    if (r < 2) return row_frag(sb1, r, gi);
    return tr_frag(sb2, (gi & 1) ? 0 : 1, 1 - ch, gi >> 1);
  };

  f32x4w_t sc[2][2], dp[2][2];  // [register set][key half]
  u32x4_t pko, dso, pkp, dsp;   // P, dS B operands: own k-step, partner k-step
  u32x4_t fr[AH];

  // ---- one iteration (block bb, PAR = bb % 2)
  auto iteration = [&](auto par_c, int bb) __attribute__((always_inline)) {
    constexpr int PAR = decltype(par_c)::value;
    constexpr int NB = 1 - PAR;
    const char* sb1 = slot(bb + 1);
    const char* sb2 = slot(bb - 1);
    mfma_wait4(sc[PAR][0], sc[PAR][1], dp[PAR][0], dp[PAR][1]);  // S_b, dP_b: matrix results
    // the partner's P, dS of block b-1 (written before the last barrier)
    pkp = *xr((bb - 1) & 1, 0, 1 - ch);
    dsp = *xr((bb - 1) & 1, 1, 1 - ch);
    load_vecs(sb1, sc[NB], dp[NB]);
    const int i0 = i_begin + 32 * bb;
    // causal: key kw + 16 nb + lane % 16 is visible to row 4 g + e of the tile
    // iff thr + 16 nb <= 4 e
    const int thr = kw + l16 - delta - i0 - 16 * ch - (g4 & 1) - 2 * (g4 >> 1);
    float pe[8], dsv[8];
    uint32_t pp[2][2], dd[2][2];
    auto vwork = [&](int k) __attribute__((always_inline)) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int nb = e >> 2, r = e & 3;
        if (k == 8 + 2 * e) {
          float x = sc[PAR][nb][r] * c;
          if constexpr (CAUSAL) x = thr + 16 * nb <= 4 * r ? x : -INFINITY;
          pe[e] = fast_exp2(x);
          pin(pe[e]);
        }
        if (k == 9 + 2 * e) {
          dsv[e] = pe[e] * dp[PAR][nb][r];  // dp holds dP - D
          pin(dsv[e]);
          if (r & 1) {
            pp[nb][r >> 1] = TR::pack2(pe[e - 1], pe[e]);
            dd[nb][r >> 1] = TR::pack2(dsv[e - 1], dsv[e]);
            pin(pp[nb][r >> 1]);
            pin(dd[nb][r >> 1]);
          }
        }
      }
      // P_b, dS_b to the exchange area, then this wavefront's own k-step back
      // (the operands of the next iteration's first products)
      if (k >= 26 && k < 30) {
        const int which = (k - 26) >> 1, nb = (k - 26) & 1;
        *(u32x2_t*)xw(bb & 1, which, nb) = which ? u32x2_t{dd[nb][0], dd[nb][1]} : u32x2_t{pp[nb][0], pp[nb][1]};
      }
      if (k == 44) pko = *xr(bb & 1, 0, ch);
      if (k == 45) dso = *xr(bb & 1, 1, ch);
      // staging: the stage of block b+2 into its slot, then the loads of block b+3
      if (k >= kW0 && k < kW0 + NPART) store_part(slot(bb + 2), k - kW0);
      if (k >= kL0 && k < kL0 + NPART) load_part(i0 + 96, k - kL0);
    };
    static_for<0, NSL>([&](auto kc) __attribute__((always_inline)) {
      constexpr int k = decltype(kc)::value;
      constexpr Prod p = prod(k);
      const u32x4_t a = fr[p.f % AH];
      if constexpr (p.last) {
        if constexpr (p.f + AH < NF) fr[p.f % AH] = frag(p.f + AH, sb1, sb2);
        else fr[p.f % AH] = frag(p.f + AH - NF, slot(bb + 2), slot(bb));  // next iteration's first operands
      }
      if constexpr (p.kind == 0) PM::macc(acc_dv[p.db], a, p.x ? pkp : pko);
      else if constexpr (p.kind == 1) PM::macc(acc_dk[p.db], a, p.x ? dsp : dso);
      else if constexpr (p.kind == 2) mma16<TR>(sc[NB][p.nb], a, kf[p.nb][(p.f - 8) / 3]);
      else mma16<TR>(dp[NB][p.nb], a, vf[p.nb][(p.f - 8) / 3]);
      vwork(k);
      __builtin_amdgcn_sched_barrier(0);
    });
    lds_barrier();
  };

  // ---- prologue: stages 0 and 1 in slots 0 and 1, slot 3 and exchange
  // buffer 1 zeroed (block -1: its products multiply zeros), block 2
  // requested; this wavefront's S_0, dP_0; the first operands
#pragma unroll
  for (int j = 0; j < NPART; ++j) load_part(i_begin, j);
#pragma unroll
  for (int j = 0; j < NPART; ++j) store_part(slot(0), j);
#pragma unroll
  for (int j = 0; j < NPART; ++j) load_part(i_begin + 32, j);
#pragma unroll
  for (int j = 0; j < NPART; ++j) store_part(slot(1), j);
  for (int i = tid; i < STG / 16; i += NT) *(u32x4_t*)(slot(3) + 16 * i) = u32x4_t{0u, 0u, 0u, 0u};
  for (int i = tid; i < 2 * XPAIR / 16; i += NT) *(u32x4_t*)(smem + XOFF + 16 * i) = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < NPART; ++j) load_part(i_begin + 64, j);
  lds_barrier();
  PM::copy_wait(acc_dk[0], acc_dk[1], acc_dk[2], acc_dk[3], acc_dv[0], acc_dv[1], acc_dv[2], acc_dv[3]);
  load_vecs(slot(0), sc[0], dp[0]);
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const u32x4_t aq = row_frag(slot(0), 0, ks), ao = row_frag(slot(0), 1, ks);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      mma16<TR>(sc[0][nb], aq, kf[nb][ks]);
      mma16<TR>(dp[0][nb], ao, vf[nb][ks]);
    }
  }
  pko = dso = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
  for (int x = 0; x < AH; ++x) fr[x] = frag(x, slot(1), slot(3));

  for (int bb = 0; bb < n_st; bb += 2) {
    iteration(std::integral_constant<int, 0>{}, bb);
    if (bb + 1 < n_st) iteration(std::integral_constant<int, 1>{}, bb + 1);
  }

  // ---- the last block's dV, dK products: the own k-step from the read-back
  // registers, the partner's from the exchange area (after the last barrier)
  {
    const int bl = n_st - 1;
    const char* st = slot(bl);
    pkp = *xr(bl & 1, 0, 1 - ch);
    dsp = *xr(bl & 1, 1, 1 - ch);
    PM::copy_wait(acc_dk[0], acc_dk[1], acc_dk[2], acc_dk[3], acc_dv[0], acc_dv[1], acc_dv[2], acc_dv[3]);
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const int t = (x >> 2) ? 1 - ch : ch;
      PM::macc(acc_dv[x & 3], tr_frag(st, 1, t, x & 3), (x >> 2) ? pkp : pko);
      PM::macc(acc_dk[x & 3], tr_frag(st, 0, t, x & 3), (x >> 2) ? dsp : dso);
    }
    PM::wait_acc(acc_dk[0], acc_dk[1], acc_dk[2], acc_dk[3], acc_dv[0], acc_dv[1], acc_dv[2], acc_dv[3]);
  }

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
// that every block's scores and dP are computed once; the software pipeline
// of the d = 128 kernels, with 32-row stages in four slots.  Iteration b (keys
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
    hipLaunchKernelGGL((bwd_dkdv_half_kernel<TR, CAUSAL>), dim3(total), dim3(256), 0,
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
