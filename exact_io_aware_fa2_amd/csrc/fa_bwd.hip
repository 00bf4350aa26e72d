// Backward attention kernels for gfx950.
//
// The pages fix only the principle ("FlashAttention" lexicon, "Methodische
// Grundlagen", paragraph "Neuberechnung statt Speicherung"): the score matrix
// is not kept from the forward pass but rebuilt, trading compute for memory
// traffic.  The gradient itself is the chain rule through the softmax:
//
//   P_ij  = exp(scale q_i.k_j - LSE_i)           (rebuilt from Q, K and LSE)
//   dV_j  = sum_i P_ij dO_i
//   dP_ij = dO_i . v_j
//   dS_ij = P_ij (dP_ij - D_i),   D_i = dO_i . O_i   (= sum_j P_ij dP_ij)
//   dQ_i  = scale sum_j dS_ij k_j
//   dK_j  = scale sum_i dS_ij q_i
//
// Three launches on the caller's stream, none of which writes an N x N array:
//   1. bwd_pre:  D_i = dO_i . O_i                       (HBM-bound, fp32 out)
//   2. bwd_dkdv: one workgroup per (128-key tile, batch*head); each
//                wavefront owns 32 keys and keeps K, V, dK, dV in registers
//                while the query tiles stream through LDS.
//   3. bwd_dq:   one workgroup per (query tile, batch*head); each wavefront
//                owns 32 query rows and keeps Q, dO, dQ in registers while the
//                key tiles stream through LDS.
// Splitting dQ from dK/dV recomputes S and dP once more but needs no atomic
// accumulation, so every gradient is bitwise reproducible run to run
// ("FlashAttention-2 (DE)", "Leistung und Effizienz": exact and
// deterministic).
//
// All products use v_mfma_f32_32x32x16 (bf16/fp16 in, fp32 accumulate).  P and
// dS are rounded to the input type (nearest even) before they enter a product.
#include <type_traits>

#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {

// ------------------------------------------------------------------ D_i

// GL: the general layout (strides of O and dO, packed sequences, DR < D
// columns); rows = BH * Nq, row r is query r % Nq of head r / Nq, skipped
// past its sequence's count, and D_i goes where the LSE entry of that row is.
template <class TR, int D, bool GL>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const uint16_t* __restrict__ O,
                                                      const uint16_t* __restrict__ dO,
                                                      float* __restrict__ Dv, int rows, int Nq, GenLayout g) {
  constexpr int KCH = D / 8;            // lanes per row
  constexpr int RPB = 256 / KCH;        // rows per workgroup
  const int tid = threadIdx.x;
  const int row = blockIdx.x * RPB + tid / KCH;
  const int ch = tid % KCH;
  float acc = 0.0f;
  bool real = row < rows;
  size_t o_at = (size_t)row * D, do_at = (size_t)row * D, d_at = (size_t)row;
  if constexpr (GL) {
    const int bh = real ? row / Nq : 0, i = real ? row - bh * Nq : 0;
    const int b = bh / g.H, hd = bh - b * g.H;
    int sq = 0, lq = 0;
    if (real) seq_rows(g.cu_q, g.total_q, b, Nq, sq, lq);
    real = real && i < lq;
    o_at = (size_t)((int64_t)b * g.o.sb + (int64_t)hd * g.o.sh + (int64_t)(sq + i) * g.o.sr);
    do_at = (size_t)((int64_t)b * g.dout.sb + (int64_t)hd * g.dout.sh + (int64_t)(sq + i) * g.dout.sr);
    d_at = (size_t)((int64_t)b * g.l_sb + (int64_t)hd * g.l_sh + sq + i);
  }
  if (real && (!GL || ch < g.dr / 8)) {
    const u32x4_t a = *(const u32x4_t*)(O + o_at + ch * 8);
    const u32x4_t b = *(const u32x4_t*)(dO + do_at + ch * 8);
#pragma unroll
    for (int p = 0; p < 4; ++p) acc = TR::dot2(a[p], b[p], acc);
  }
#pragma unroll
  for (int off = KCH / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (real && ch == 0) Dv[d_at] = acc;
}

// ------------------------------------------------------------------ dK, dV

// dK, dV software-pipelined inside each wavefront: one wavefront per SIMD,
// 4 x 32 keys per workgroup (d = 64 and 128).  Query rows stream through LDS in stages
// of 64 (two blocks of 32); iteration b of a wavefront issues
//   matrix: dV^T += dO_{b-1}^T P_{b-1}, dK^T += Q_{b-1}^T dS_{b-1},
//           S'_{b+1} = Q_{b+1} K^T - LSE / scale, dP_{b+1} = dO_{b+1} V^T - D
//   vector: P_b = exp2(S'_b c), dS_b = P_b (dP_b - D), rounded
// interleaved product by product, so that the matrix core and the vector unit
// of the SIMD work at the same time within the one wavefront (c = scale log2 e;
// -LSE / scale and -D enter as the accumulators' initial values, read from LDS
// two products before the first product that adds to them).  At one wavefront
// per SIMD (d = 128), K, V (operands) and dK, dV (accumulators) stay in AGPRs
// for the whole kernel; at two (d = 64, 256 registers each) all are VGPRs.
//
// LDS stage (four in flight, stage x in slot x % 4): Q and dO tiles with rows
// padded to d + 8 elements, -LSE / scale and -D.  Within every 16 query
// rows the S/dP products take their rows in the order perm(m) = 4 (m % 4) +
// m / 4, so that the four rows a transposed read (lds_read_tr) gathers for
// the dV/dK products lie 4 rows apart: with the padded rows, both the row
// reads (S, dP) and the transposed reads (dV, dK) are free of bank conflicts,
// and no transposed copy of Q or dO is staged.
template <class TR, int D, bool CAUSAL, int OCC, bool GL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
void bwd_dkdv_pipe_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                          const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                          const float* __restrict__ LSE, const float* __restrict__ Dvec,
                          uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int Nq, int Nk, int n_ktiles,
                          uint32_t total, float c, float neg_inv_scale, float scale, GenLayout g) {
  constexpr int NT = 256;
  constexpr int BKV = 128;                  // keys per workgroup
  constexpr int BQ = 64;                    // query rows per stage
  constexpr int KS = D + 8;                 // padded LDS row (elements)
  constexpr int RBL = 2 * KS;               // LDS row bytes
  constexpr uint32_t RB = 2 * D;            // global row bytes
  constexpr int NKS = D / 16;               // k-steps of S and dP
  constexpr int NDB = D / 32;               // 32-column blocks of dK and dV
  constexpr int OFF_O = BQ * RBL;           // stage layout (bytes): Q, dO, then vector w
  constexpr int OFF_L = 2 * BQ * RBL;       // of wave w at OFF_L + 4 BQ w (0: -LSE/scale,
  constexpr int OFF_D = OFF_L + 4 * BQ;     // 1: -D; waves 2, 3 write unread copies)
  constexpr int STG = OFF_L + 16 * BQ;
  constexpr int CPR = D / 8;                // 16-byte chunks per row
  constexpr int ROWSTEP = NT / CPR;         // rows between a thread's staging chunks
  constexpr int NCH = BQ / ROWSTEP;         // staging chunks per thread and tensor
  constexpr int NSL = 4 * NKS;              // products per iteration
  constexpr int AH = OCC == 1 ? 8 : 4;      // operand reads issued ahead of their product
  constexpr int kW0 = NSL / 4;              // first staging write (product index, PAR 1)
  static_assert(kW0 + 2 * (BQ / (NT / (D / 8))) + 1 <= NSL, "staging writes fit the iteration");
  static_assert(2 * NDB == NKS, "S, dV, dK, dP products interleave one to one");
  static_assert(NSL % AH == 0, "operand of product f of an iteration sits in fr[f % AH]");
  static_assert(NSL == 32 || NSL == 16, "vector work schedule below");
  static_assert(OCC * 4 * STG <= 160 * 1024, "four stages per workgroup fit in LDS");
  using PM = PipeMma<TR, OCC == 1>;          // K, V, dK and dV in AGPRs at one wavefront per SIMD
  const float s_out = neg_inv_scale < 0.0f ? -INFINITY : INFINITY;  // initial S of rows past the end

  __shared__ __attribute__((aligned(16))) char smem[4 * STG];

  // one tile: the whole pass from the first load to the last store
  auto run_tile = [&](const uint32_t lid) __attribute__((always_inline)) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int h = lane >> 5;
  const int l32 = lane & 31;

  const int bh = lid / n_ktiles;
  const int kt = lid % n_ktiles;
  const int k0 = kt * BKV;
  const int kw = k0 + 32 * w;               // first key of this wavefront
  const int key = kw + l32;
  // Addressing: dense [BH, N, D] (Nq = Nk), or (GL) the general layout:
  // per-tensor strides, packed sequences with Lq queries and Lk keys (key
  // tiles wholly past Lk skipped), DR < D data columns.  Causal is aligned
  // bottom right: key j is visible to query i iff j <= i + delta, delta =
  // Lk - Lq (0 for equal counts: the square mask).
  int Lq = Nq, Lk = Nk, DR = D, delta = 0;
  size_t q_off, do_off, k_off, v_off, dk_off, dv_off, l_off, dks, dvs;
  uint32_t q_bytes, do_bytes, k_bytes, v_bytes, rsq, rsdo, rsk, rsv;
  if constexpr (GL) {
    const int b = bh / g.H, hd = bh - b * g.H;
    int sq, sk;
    seq_rows(g.cu_q, g.total_q, b, Nq, sq, Lq);
    seq_rows(g.cu_k, g.total_k, b, Nk, sk, Lk);
    DR = g.dr;
    delta = CAUSAL ? Lk - Lq : 0;
    const TRows tq = tensor_rows(g.q, b, hd, sq, Lq, DR), tdo = tensor_rows(g.dout, b, hd, sq, Lq, DR);
    const TRows tk = tensor_rows(g.k, b, hd, sk, Lk, DR), tv = tensor_rows(g.v, b, hd, sk, Lk, DR);
    q_off = tq.off, do_off = tdo.off, k_off = tk.off, v_off = tv.off;
    q_bytes = tq.bytes, do_bytes = tdo.bytes, k_bytes = tk.bytes, v_bytes = tv.bytes;
    rsq = tq.rs, rsdo = tdo.rs, rsk = tk.rs, rsv = tv.rs;
    dk_off = (size_t)((int64_t)b * g.dk.sb + (int64_t)hd * g.dk.sh + (int64_t)sk * g.dk.sr);
    dv_off = (size_t)((int64_t)b * g.dv.sb + (int64_t)hd * g.dv.sh + (int64_t)sk * g.dv.sr);
    dks = (size_t)g.dk.sr, dvs = (size_t)g.dv.sr;
    l_off = (size_t)((int64_t)b * g.l_sb + (int64_t)hd * g.l_sh + sq);
  } else {
    q_off = do_off = k_off = v_off = dk_off = dv_off = (size_t)bh * Nq * D;
    q_bytes = do_bytes = k_bytes = v_bytes = (uint32_t)Nq * RB;
    rsq = rsdo = rsk = rsv = RB;
    dks = dvs = D;
    l_off = (size_t)bh * Nq;
  }
  if (GL && k0 >= Lk) return;

  // K and V rows of this wavefront's keys as B operands (column = key)
  u32x4_t kf[NKS], vf[NKS];
  {
    const rsrc_t kres = make_rsrc(K + k_off, k_bytes);
    const rsrc_t vres = make_rsrc(V + v_off, v_bytes);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const uint32_t pad_k = GL ? col_pad(32 * ks + 16 * h, DR, k_bytes) : 0u;
      const uint32_t pad_v = GL ? col_pad(32 * ks + 16 * h, DR, v_bytes) : 0u;
      kf[ks] = buf_load16(kres, (uint32_t)key * rsk + 16 * h + 32 * ks + pad_k);
      vf[ks] = buf_load16(vres, (uint32_t)key * rsv + 16 * h + 32 * ks + pad_v);
    }
  }
  f32x16_t acc_dk[NDB], acc_dv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    acc_dk[db] = zero16();
    acc_dv[db] = zero16();
  }

  // query row (within its 32-row block) of S/dP row m
  auto perm = [](int m) { return (m & 16) | ((m & 3) << 2) | ((m >> 2) & 3); };
  // row-read fragment of this lane: row perm(l32), chunk h (+ 2 ks)
  const uint32_t rbase = (uint32_t)(perm(l32) * RBL + 16 * h);
  // transposed-read fragment: lane group G = lane / 16 covers columns
  // 16 (G % 2) + 0..15 of rows (h + 2 sec) + 4 e, e = 0..3; lane 4e + i of the
  // group points at columns 4i..4i+3 of row e
  const int L16 = lane & 15, G = lane >> 4;
  const uint32_t tbase = (uint32_t)((h + 4 * (L16 >> 2)) * RBL + (16 * (G & 1) + 4 * (L16 & 3)) * 2);

  // the first query row that sees a key of this tile (causal), and the stages
  const int i_begin = CAUSAL ? max(0, k0 - delta) : 0;
  const int n_st = (Lq - i_begin + BQ - 1) / BQ;
  const int nrows = min(32, Lk - kw);
  const int nch = GL ? DR / 8 : D / 8;
  if (GL && n_st <= 0) {
    // no query sees these keys (an empty query sequence): dK = dV = 0
    const u32x4_t z = {0u, 0u, 0u, 0u};
    for (int i = lane; i < 32 * (D / 8); i += 64) {
      const int r = i / (D / 8), ch = i % (D / 8);
      if (r < nrows && ch < nch) {
        *(u32x4_t*)(dK + dk_off + (size_t)(kw + r) * dks + 8 * ch) = z;
        *(u32x4_t*)(dV + dv_off + (size_t)(kw + r) * dvs + 8 * ch) = z;
      }
    }
    return;
  }

  // ---- staging: chunk i of this thread is row tid / CPR + ROWSTEP i, column
  // chunk tid % CPR, of both Q and dO.  Wave w loads vector w % 2 of the stage
  // (0: -LSE / scale, 1: -D) at positions m = lane: row 32 (m / 32) + perm(m % 32).
  const rsrc_t qres = make_rsrc(Q + q_off, q_bytes);
  const rsrc_t ores = make_rsrc(dO + do_off, do_bytes);
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const bool is_d = (wu & 1) != 0;
  const rsrc_t vres = make_rsrc(is_d ? (const void*)(Dvec + l_off) : (const void*)(LSE + l_off),
                                (uint32_t)Lq * 4);
  const uint32_t g_col = (tid % CPR) * 16;
  const uint32_t gq_off = (uint32_t)(tid / CPR) * rsq + g_col + (GL ? col_pad(g_col, DR, q_bytes) : 0u);
  const uint32_t go_off = (uint32_t)(tid / CPR) * rsdo + g_col + (GL ? col_pad(g_col, DR, do_bytes) : 0u);
  const uint32_t s_off = (uint32_t)(tid / CPR) * RBL + (tid % CPR) * 16;
  const int vrow = (lane & 32) + perm(lane & 31);
  const uint32_t vec_off = OFF_L + 4 * BQ * wu + 4 * lane;
  // The loaded values are only used when they are written to LDS (a whole
  // iteration later), so no wait for the loads stalls the products.  Set 1
  // of the staging registers is used only by the prologue (two stages in
  // flight at once).
  u32x4_t sq[2][NCH], so[2][NCH];
  float vraw[2] = {0.0f, 0.0f};
  int vidx[2] = {0, 0};
  // staging part j < NCH: Q chunk j; j < 2 NCH: dO chunk j - NCH; j = 2 NCH: the vector
  constexpr int NPART = 2 * NCH + 1;
  auto load_part = [&](int i0, int j, int t = 0) __attribute__((always_inline)) {
    if (j < NCH) {
      const uint32_t r = GL ? __builtin_amdgcn_readfirstlane(rsq) : RB;
      sq[t][j] = buf_load16(qres, gq_off + (uint32_t)(i0 + ROWSTEP * j) * r);
    } else if (j < 2 * NCH) {
      const uint32_t r = GL ? __builtin_amdgcn_readfirstlane(rsdo) : RB;
      so[t][j - NCH] = buf_load16(ores, go_off + (uint32_t)(i0 + ROWSTEP * (j - NCH)) * r);
    } else {
      vidx[t] = i0 + vrow;
      vraw[t] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(vres, (uint32_t)vidx[t] * 4, 0, 0));
    }
  };
  auto store_part = [&](uint32_t sb, int j, int t = 0) __attribute__((always_inline)) {
    if (j < NCH) {
      *(u32x4_t*)(smem + sb + s_off + ROWSTEP * j * RBL) = sq[t][j];
    } else if (j < 2 * NCH) {
      *(u32x4_t*)(smem + sb + OFF_O + s_off + ROWSTEP * (j - NCH) * RBL) = so[t][j - NCH];
    } else {
      // rows past the end: an infinite S of the sign of -1 / s (-inf for s > 0,
      // +inf for s < 0) makes S c = -inf, so P = 0; D = 0
      const bool in = vidx[t] < Lq;
      *(float*)(smem + sb + vec_off) = is_d ? (in ? -vraw[t] : 0.0f) : (in ? vraw[t] * neg_inv_scale : s_out);
    }
  };

  // ---- register sets of the pipeline (index: block parity)
  f32x16_t sc[2], dp[2];
  u32x4_t pk[2][2], dsk[2][2];  // [set][k-step t]: P and dS rounded, packed in pairs

  // initial values of the S and dP accumulators (-LSE / scale, -D) of the
  // block in half bb of stage sb
  auto load_vecs = [&](uint32_t sb, int bb, f32x16_t& d, f32x16_t& l) __attribute__((always_inline)) {
    const char* dv = smem + sb + OFF_D + 128 * bb + 16 * h;
    const char* lv = smem + sb + OFF_L + 128 * bb + 16 * h;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float4 d4 = *(const float4*)(dv + 32 * g);
      const float4 l4 = *(const float4*)(lv + 32 * g);
      d[4 * g + 0] = d4.x; d[4 * g + 1] = d4.y; d[4 * g + 2] = d4.z; d[4 * g + 3] = d4.w;
      l[4 * g + 0] = l4.x; l[4 * g + 1] = l4.y; l[4 * g + 2] = l4.z; l[4 * g + 3] = l4.w;
    }
  };
  // A operand of S (tensor 0: Q) or dP (tensor 1: dO) for k-step ks
  auto row_frag = [&](uint32_t sb, int bb, int tensor, int ks) __attribute__((always_inline)) -> u32x4_t {
    return *(const u32x4_t*)(smem + sb + tensor * OFF_O + rbase + bb * 32 * RBL + 32 * ks);
  };
  // A operand of dK^T (tensor 0: Q^T) or dV^T (tensor 1: dO^T) for k-step t, column block db
  auto tr_frag = [&](uint32_t sb, int bb, int tensor, int t, int db) __attribute__((always_inline)) -> u32x4_t {
    const char* p = smem + sb + tensor * OFF_O + tbase + (32 * bb + 16 * t) * RBL + 64 * db;
    const u32x2_t a = lds_read_tr(p), b = lds_read_tr(p + 2 * RBL);
    return u32x4_t{a[0], a[1], b[0], b[1]};
  };
  // operand of product k of an iteration: (dV, dK, S, dP)[k % 4] of index k / 4;
  // sb1: stage of block b+1, sb2: stage of block b-1, nb: their half (1 - b % 2)
  auto frag = [&](int k, uint32_t sb1, uint32_t sb2, int nb) __attribute__((always_inline)) -> u32x4_t {
    const int x = k / 4;
    switch (k % 4) {
      case 0: return tr_frag(sb2, nb, 1, x / NDB, x % NDB);
      case 1: return tr_frag(sb2, nb, 0, x / NDB, x % NDB);
      case 2: return row_frag(sb1, nb, 0, x);
      default: return row_frag(sb1, nb, 1, x);
    }
  };
  u32x4_t fr[AH];  // operands of the next AH products, carried across iterations

  // ---- one iteration.  PAR = b % 2 selects the register sets; q0: first row
  // of block b; (nsb1, nsb2): stages of the next iteration.  PAR 0 requests the
  // stage after next (rows i_ld), PAR 1 writes it to slot sbw.
  auto iteration = [&](auto par_c, auto masked_c, uint32_t sb1, uint32_t sb2, uint32_t nsb1, uint32_t nsb2,
                       int q0, int i_ld, uint32_t sbw) __attribute__((always_inline)) {
    constexpr int PAR = decltype(par_c)::value;
    constexpr bool MASKED = decltype(masked_c)::value;
    constexpr int NB = 1 - PAR;
    // S_b, dP_b were written by matrix instructions, P and dS of block b-1 by
    // vector instructions: all of them ordered before what reads them next
    mfma_wait_v(sc[PAR], dp[PAR]);
    asm volatile("" : "+v"(pk[NB][0]), "+v"(pk[NB][1]), "+v"(dsk[NB][0]), "+v"(dsk[NB][1]));
    load_vecs(sb1, NB, dp[NB], sc[NB]);

    // causal: key kw + l32 is visible to the row of score r iff thr <= qoff(r)
    const int thr = kw - delta - q0 + l32 - h;
    float pe[16], dsv[16];
    auto vwork = [&](int k) __attribute__((always_inline)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        // score r: scale, shift and exp2 at product v0(r), the rest one product later
        constexpr int V0 = NSL / 16;
        const int v0 = V0 * r, v1 = v0 + 1 < NSL ? v0 + 1 : v0;
        if (k == v0) {
          float x = sc[PAR][r] * c;
          if constexpr (MASKED) {
            // score r = 4g + e is S row 8g + 4h + e: query perm(8(g%2) + 4h + e) + 16(g/2)
            const int g = r / 4, e = r % 4;
            const int qoff = 16 * (g / 2) + 4 * e + 2 * (g % 2);
            x = thr <= qoff ? x : -INFINITY;
          }
          pe[r] = fast_exp2(x);
        }
        if (k == v1) {
          dsv[r] = pe[r] * dp[PAR][r];  // dp holds dP - D
          if (r & 1) {
            pk[PAR][r / 8][(r / 2) % 4] = TR::pack2(pe[r - 1], pe[r]);
            dsk[PAR][r / 8][(r / 2) % 4] = TR::pack2(dsv[r - 1], dsv[r]);
          }
        }
      }
      // staging: one load per product from the start of PAR 0, one LDS
      // write per product from kW0 of PAR 1
      if constexpr (PAR == 0) {
        if (k < NPART) load_part(i_ld, k);
      } else {
        if (k >= kW0 && k < kW0 + NPART) store_part(sbw, k - kW0);
      }
    };
    static_for<0, NSL>([&](auto kc) __attribute__((always_inline)) {
      constexpr int k = decltype(kc)::value;
      constexpr int x = k / 4;
      const u32x4_t a = fr[k % AH];
      if constexpr (k + AH < NSL) fr[k % AH] = frag(k + AH, sb1, sb2, NB);
      else fr[k % AH] = frag(k + AH - NSL, nsb1, nsb2, PAR);
      if constexpr (k % 4 == 0) {
        PM::macc(acc_dv[x % NDB], a, pk[NB][x / NDB]);
      } else if constexpr (k % 4 == 1) {
        PM::macc(acc_dk[x % NDB], a, dsk[NB][x / NDB]);
      } else if constexpr (k % 4 == 2) {
        PM::mb(sc[NB], a, kf[x]);
      } else {
        PM::mb(dp[NB], a, vf[x]);
      }
      vwork(k);
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // ---- prologue: stages 0 and 1 in slots 0 and 1, slot 3 zeroed (the first
  // iteration multiplies it by zero P and dS); S_0, dP_0; first operands
#pragma unroll
  for (int j = 0; j < NPART; ++j) load_part(i_begin, j, 0);
#pragma unroll
  for (int j = 0; j < NPART; ++j) load_part(i_begin + BQ, j, 1);
#pragma unroll
  for (int j = 0; j < NPART; ++j) store_part(0, j, 0);
#pragma unroll
  for (int j = 0; j < NPART; ++j) store_part(STG, j, 1);
  for (int i = tid; i < 2 * BQ * RBL / 16; i += NT) *(u32x4_t*)(smem + 3 * STG + 16 * i) = u32x4_t{0u, 0u, 0u, 0u};
  lds_barrier();
  load_vecs(0, 0, dp[0], sc[0]);
  mma_pipeline<2 * NKS, 3>([&](int x) { return smem + ((x & 1) ? OFF_O : 0) + rbase + 32 * (x >> 1); },
                           [&](int x, u32x4_t a) {
                             const int ks = x >> 1;
                             if (x & 1) PM::mb(dp[0], a, vf[ks]);
                             else PM::mb(sc[0], a, kf[ks]);
                           },
                           [](int) {});
#pragma unroll
  for (int t = 0; t < 2; ++t) pk[1][t] = dsk[1][t] = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
  for (int x = 0; x < AH; ++x) fr[x] = frag(x, 0u, 3u * STG, 1);

  // ---- pairs of iterations over the stages.  Causal: the stages with a
  // query that does not see every key of the tile are masked (with the square
  // mask: the first two, each wavefront's diagonal block and those above it).
  auto pair = [&](auto masked_c, int s) __attribute__((always_inline)) {
    const uint32_t b0 = (uint32_t)(s & 3) * STG;
    const uint32_t bp1 = (uint32_t)((s + 1) & 3) * STG;
    const uint32_t bm1 = (uint32_t)((s + 3) & 3) * STG;
    const uint32_t bp2 = (uint32_t)((s + 2) & 3) * STG;
    const int q0 = i_begin + BQ * s;
    iteration(std::integral_constant<int, 0>{}, masked_c, b0, bm1, bp1, b0, q0, q0 + 2 * BQ, 0u);
    iteration(std::integral_constant<int, 1>{}, masked_c, bp1, b0, bp1, b0, q0 + 32, 0, bp2);
    lds_barrier();
  };
  const int n_masked = CAUSAL ? min((k0 + BKV - delta - i_begin + BQ - 1) / BQ, n_st) : 0;
  int s = 0;
  for (; s < n_masked; ++s) pair(std::true_type{}, s);
  for (; s < n_st; ++s) pair(std::false_type{}, s);

  // ---- last block: its dV, dK products (register set 1)
  {
    const uint32_t sb = (uint32_t)((n_st - 1) & 3) * STG;
    asm volatile("" : "+v"(pk[1][0]), "+v"(pk[1][1]), "+v"(dsk[1][0]), "+v"(dsk[1][1]));
    // where the loops join, the accumulators may have been copied between registers
    if constexpr (NDB == 4)
      PM::copy_wait(acc_dk[0], acc_dk[1], acc_dk[2], acc_dk[3], acc_dv[0], acc_dv[1], acc_dv[2], acc_dv[3]);
    else
      PM::copy_wait(acc_dk[0], acc_dk[1], acc_dv[0], acc_dv[1]);
#pragma unroll
    for (int x = 0; x < NKS; ++x) {
      PM::macc(acc_dv[x % NDB], tr_frag(sb, 1, 1, x / NDB, x % NDB), pk[1][x / NDB]);
      PM::macc(acc_dk[x % NDB], tr_frag(sb, 1, 0, x / NDB, x % NDB), dsk[1][x / NDB]);
    }
  }
  if constexpr (NDB == 4)
    PM::wait_acc(acc_dk[0], acc_dk[1], acc_dk[2], acc_dk[3], acc_dv[0], acc_dv[1], acc_dv[2], acc_dv[3]);
  else
    PM::wait_acc(acc_dk[0], acc_dk[1], acc_dv[0], acc_dv[1]);

  // dK, dV rounded and stored as whole rows through LDS: after the last
  // barrier every stage slot but that of the last block is free; dK of
  // wavefront w goes to slot n_st + 1, dV to slot n_st + 2 (32 rows each)
  u32x2_t ok[NDB][4], ov[NDB][4];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      ok[db][g] = u32x2_t{TR::pack2(acc_dk[db][4 * g + 0] * scale, acc_dk[db][4 * g + 1] * scale),
                          TR::pack2(acc_dk[db][4 * g + 2] * scale, acc_dk[db][4 * g + 3] * scale)};
      ov[db][g] = u32x2_t{TR::pack2(acc_dv[db][4 * g + 0], acc_dv[db][4 * g + 1]),
                          TR::pack2(acc_dv[db][4 * g + 2], acc_dv[db][4 * g + 3])};
    }
  static_assert(4 * kTileRowsBytes<D> <= STG, "four wavefronts' rows fit one stage slot");
  store_tile_rows<D>(smem + ((n_st + 1) & 3) * STG + w * kTileRowsBytes<D>, ok,
                     dK + dk_off + (size_t)kw * dks, nrows, lane, dks, nch);
  store_tile_rows<D>(smem + ((n_st + 2) & 3) * STG + w * kTileRowsBytes<D>, ov,
                     dV + dv_off + (size_t)kw * dvs, nrows, lane, dvs, nch);
  };
  for_each_tile(total, (uint32_t)n_ktiles, run_tile);
}

// ------------------------------------------------------------------ dQ

// dQ software-pipelined inside each wavefront: 4 x 32 query rows per
// workgroup, OCC wavefronts per SIMD.  With one (d = 128), Q, dO (B operands)
// and the dQ accumulators stay in AGPRs; with two (d = 64), whose register
// budget is 256 per wavefront, every operand is a VGPR.  Key rows stream
// through LDS in stages of 64 (two blocks of 32), with the layout of
// bwd_dkdv_pipe_kernel (padded rows; S^T row m holds key perm(m) of its 16).
// Iteration b of a wavefront issues
//   matrix: S^T_{b+1} = K_{b+1} Q^T, dP^T_{b+1} = V_{b+1} dO^T - D,
//           dQ^T += K_{b-1}^T dS^T_{b-1}
//   vector: P_b = exp2(S^T_b c - LSE log2 e), dS_b = P_b (dP_b - D), rounded
// interleaved product by product.  Each lane owns one query row, so LSE and D
// are per-lane constants (D enters as the dP accumulators' initial value).
// Keys past the end need no mask: their K and V rows read as zeros, so their
// dS multiplies a zero row of K.
template <class TR, int D, bool CAUSAL, int OCC, bool GL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
void bwd_dq_pipe_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                        const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                        const float* __restrict__ LSE, const float* __restrict__ Dvec,
                        uint16_t* __restrict__ dQ, int Nq, int Nk, int n_qtiles, uint32_t total, float c,
                        float scale, GenLayout g) {
  constexpr int NT = 256;
  constexpr int BR = 128;                   // query rows per workgroup
  constexpr int BC = 64;                    // keys per stage
  constexpr int KS = D + 8;                 // padded LDS row (elements)
  constexpr int RBL = 2 * KS;               // LDS row bytes
  constexpr uint32_t RB = 2 * D;            // global row bytes
  constexpr int NKS = D / 16;               // k-steps of S and dP
  constexpr int NDB = D / 32;               // 32-column blocks of dQ
  constexpr int OFF_V = BC * RBL;           // stage layout (bytes): K, then V
  constexpr int STG = 2 * BC * RBL;
  constexpr int CPR = D / 8;                // 16-byte chunks per row
  constexpr int ROWSTEP = NT / CPR;         // rows between a thread's staging chunks
  constexpr int NCH = BC / ROWSTEP;         // staging chunks per thread and tensor
  constexpr int NPART = 2 * NCH;
  constexpr int NSL = 3 * NKS;              // products per iteration (S, dQ, dP)
  constexpr int AH = NSL % 8 == 0 ? 8 : 6;  // operand reads issued ahead of their product
  constexpr int kW0 = NSL / 4;              // first staging write (product index, PAR 1)
  static_assert(2 * NDB == NKS, "S, dQ, dP products interleave one to one");
  static_assert(NSL % AH == 0, "operand of product f of an iteration sits in fr[f % AH]");
  static_assert(NPART <= NSL && kW0 + NPART <= NSL, "staging fits the iteration");
  static_assert(OCC * 4 * STG <= 160 * 1024, "four stages per workgroup fit in LDS");
  using PM = PipeMma<TR, OCC == 1>;          // Q, dO and dQ in AGPRs at one wavefront per SIMD

  __shared__ __attribute__((aligned(16))) char smem[4 * STG];

  // one tile: the whole pass from the first load to the last store
  auto run_tile = [&](const uint32_t lid) __attribute__((always_inline)) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int h = lane >> 5;
  const int l32 = lane & 31;

  const int bh = lid / n_qtiles;
  int qt = lid % n_qtiles;
  if (CAUSAL) qt = n_qtiles - 1 - qt;       // longest rows first
  const int q0 = qt * BR;
  const int qw = q0 + 32 * w;               // first query row of this wavefront
  const int qrow = qw + l32;
  // Addressing as in the dK/dV kernel: dense [BH, N, D], or (GL) per-tensor
  // strides, packed sequences of Lq queries and Lk keys (query tiles wholly
  // past Lq skipped), DR < D data columns; causal aligned bottom right (key j
  // visible to query i iff j <= i + delta, delta = Lk - Lq).
  int Lq = Nq, Lk = Nk, DR = D, delta = 0;
  size_t q_off, do_off, k_off, v_off, dq_off, l_off, dqs;
  uint32_t q_bytes, do_bytes, k_bytes, v_bytes, rsq, rsdo, rsk, rsv;
  if constexpr (GL) {
    const int b = bh / g.H, hd = bh - b * g.H;
    int sq, sk;
    seq_rows(g.cu_q, g.total_q, b, Nq, sq, Lq);
    seq_rows(g.cu_k, g.total_k, b, Nk, sk, Lk);
    DR = g.dr;
    delta = CAUSAL ? Lk - Lq : 0;
    const TRows tq = tensor_rows(g.q, b, hd, sq, Lq, DR), tdo = tensor_rows(g.dout, b, hd, sq, Lq, DR);
    const TRows tk = tensor_rows(g.k, b, hd, sk, Lk, DR), tv = tensor_rows(g.v, b, hd, sk, Lk, DR);
    q_off = tq.off, do_off = tdo.off, k_off = tk.off, v_off = tv.off;
    q_bytes = tq.bytes, do_bytes = tdo.bytes, k_bytes = tk.bytes, v_bytes = tv.bytes;
    rsq = tq.rs, rsdo = tdo.rs, rsk = tk.rs, rsv = tv.rs;
    dq_off = (size_t)((int64_t)b * g.dq.sb + (int64_t)hd * g.dq.sh + (int64_t)sq * g.dq.sr);
    dqs = (size_t)g.dq.sr;
    l_off = (size_t)((int64_t)b * g.l_sb + (int64_t)hd * g.l_sh + sq);
  } else {
    q_off = do_off = k_off = v_off = dq_off = (size_t)bh * Nq * D;
    q_bytes = do_bytes = k_bytes = v_bytes = (uint32_t)Nq * RB;
    rsq = rsdo = rsk = rsv = RB;
    dqs = D;
    l_off = (size_t)bh * Nq;
  }
  if (GL && q0 >= Lq) return;

  // Q and dO rows of this wavefront's queries as B operands (column = query)
  u32x4_t qf[NKS], of[NKS];
  {
    const rsrc_t qres = make_rsrc(Q + q_off, q_bytes);
    const rsrc_t ores = make_rsrc(dO + do_off, do_bytes);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const uint32_t pad_q = GL ? col_pad(32 * ks + 16 * h, DR, q_bytes) : 0u;
      const uint32_t pad_o = GL ? col_pad(32 * ks + 16 * h, DR, do_bytes) : 0u;
      qf[ks] = buf_load16(qres, (uint32_t)qrow * rsq + 16 * h + 32 * ks + pad_q);
      of[ks] = buf_load16(ores, (uint32_t)qrow * rsdo + 16 * h + 32 * ks + pad_o);
    }
  }
  // rows past the end: P = exp2(-inf) = 0, so dS = 0 there
  const float lq = qrow < Lq ? LSE[l_off + qrow] * kLog2e : INFINITY;
  const float dd = qrow < Lq ? Dvec[l_off + qrow] : 0.0f;
  f32x16_t negd;  // initial value of the dP accumulators
#pragma unroll
  for (int i = 0; i < 16; ++i) negd[i] = -dd;
  f32x16_t acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = zero16();

  // key row (within its 32-key block) of S^T row m
  auto perm = [](int m) { return (m & 16) | ((m & 3) << 2) | ((m >> 2) & 3); };
  const uint32_t rbase = (uint32_t)(perm(l32) * RBL + 16 * h);
  const int L16 = lane & 15, G = lane >> 4;
  const uint32_t tbase = (uint32_t)((h + 4 * (L16 >> 2)) * RBL + (16 * (G & 1) + 4 * (L16 & 3)) * 2);

  // keys visible to the workgroup's last row; none (every row of the tile
  // sees no key: an empty key sequence, or rows before the bottom-right
  // diagonal starts): dQ = 0
  const int kv_end = CAUSAL ? min(Lk, q0 + BR + delta) : Lk;
  const int nch = GL ? DR / 8 : D / 8;
  if (GL && kv_end <= 0) {
    const u32x4_t z = {0u, 0u, 0u, 0u};
    for (int i = lane; i < 32 * (D / 8); i += 64) {
      const int r = i / (D / 8), ch = i % (D / 8);
      if (r < Lq - qw && ch < nch) *(u32x4_t*)(dQ + dq_off + (size_t)(qw + r) * dqs + 8 * ch) = z;
    }
    return;
  }
  const int n_st = (kv_end + BC - 1) / BC;

  // ---- staging: chunk i of this thread is row tid / CPR + ROWSTEP i, column
  // chunk tid % CPR, of both K and V (part j < NCH: K chunk j, else V chunk j - NCH)
  const rsrc_t kres = make_rsrc(K + k_off, k_bytes);
  const rsrc_t vres = make_rsrc(V + v_off, v_bytes);
  const uint32_t g_col = (tid % CPR) * 16;
  const uint32_t gk_off = (uint32_t)(tid / CPR) * rsk + g_col + (GL ? col_pad(g_col, DR, k_bytes) : 0u);
  const uint32_t gv_off = (uint32_t)(tid / CPR) * rsv + g_col + (GL ? col_pad(g_col, DR, v_bytes) : 0u);
  const uint32_t s_off = (uint32_t)(tid / CPR) * RBL + (tid % CPR) * 16;
  // (set 1 of the staging registers: prologue only, two stages in flight)
  u32x4_t sk[2][NCH], sv[2][NCH];
  auto load_part = [&](int j0, int j, int t = 0) __attribute__((always_inline)) {
    if (j < NCH) {
      const uint32_t r = GL ? __builtin_amdgcn_readfirstlane(rsk) : RB;
      sk[t][j] = buf_load16(kres, gk_off + (uint32_t)(j0 + ROWSTEP * j) * r);
    } else {
      const uint32_t r = GL ? __builtin_amdgcn_readfirstlane(rsv) : RB;
      sv[t][j - NCH] = buf_load16(vres, gv_off + (uint32_t)(j0 + ROWSTEP * (j - NCH)) * r);
    }
  };
  auto store_part = [&](uint32_t sb, int j, int t = 0) __attribute__((always_inline)) {
    if (j < NCH) *(u32x4_t*)(smem + sb + s_off + ROWSTEP * j * RBL) = sk[t][j];
    else *(u32x4_t*)(smem + sb + OFF_V + s_off + ROWSTEP * (j - NCH) * RBL) = sv[t][j - NCH];
  };

  // ---- register sets of the pipeline (index: block parity)
  f32x16_t sc[2], dp[2];
  u32x4_t dsk[2][2];  // [set][k-step t]: dS rounded, packed in pairs

  // A operand of S^T (tensor 0: K) or dP^T (tensor 1: V) for k-step ks
  auto row_frag = [&](uint32_t sb, int bb, int tensor, int ks) __attribute__((always_inline)) -> u32x4_t {
    return *(const u32x4_t*)(smem + sb + tensor * OFF_V + rbase + bb * 32 * RBL + 32 * ks);
  };
  // A operand of dQ^T (K^T) for k-step t, column block db
  auto tr_frag = [&](uint32_t sb, int bb, int t, int db) __attribute__((always_inline)) -> u32x4_t {
    const char* p = smem + sb + tbase + (32 * bb + 16 * t) * RBL + 64 * db;
    const u32x2_t a = lds_read_tr(p), b = lds_read_tr(p + 2 * RBL);
    return u32x4_t{a[0], a[1], b[0], b[1]};
  };
  // operand of product k of an iteration: (S, dQ, dP)[k % 3] of index k / 3;
  // sb1: stage of block b+1, sb2: stage of block b-1, nb: their half (1 - b % 2)
  auto frag = [&](int k, uint32_t sb1, uint32_t sb2, int nb) __attribute__((always_inline)) -> u32x4_t {
    const int x = k / 3;
    switch (k % 3) {
      case 0: return row_frag(sb1, nb, 0, x);
      case 1: return tr_frag(sb2, nb, x / NDB, x % NDB);
      default: return row_frag(sb1, nb, 1, x);
    }
  };
  u32x4_t fr[AH];  // operands of the next AH products, carried across iterations

  // ---- one iteration.  PAR = b % 2 selects the register sets; j0: first key
  // of block b; (nsb1, nsb2): stages of the next iteration.  PAR 0 requests the
  // stage after next (keys j_ld), PAR 1 writes it to slot sbw.
  auto iteration = [&](auto par_c, auto masked_c, uint32_t sb1, uint32_t sb2, uint32_t nsb1, uint32_t nsb2,
                       int j0, int j_ld, uint32_t sbw) __attribute__((always_inline)) {
    constexpr int PAR = decltype(par_c)::value;
    constexpr bool MASKED = decltype(masked_c)::value;
    constexpr int NB = 1 - PAR;
    // S_b, dP_b were written by matrix instructions, dS of block b-1 by vector
    // instructions: all of them ordered before what reads them next
    mfma_wait_v(sc[PAR], dp[PAR]);
    asm volatile("" : "+v"(dsk[NB][0]), "+v"(dsk[NB][1]));

    // causal: key j0 + koff(r) is visible to this lane's row iff koff(r) <= thr
    const int thr = qrow + delta - j0 - h;
    float pe[16], dsv[16];
    auto vwork = [&](int k) __attribute__((always_inline)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        // score r: scale, shift and exp2 at product v0(r), the rest one later
        const int v0 = r * NSL / 16, v1 = v0 + 1 < NSL ? v0 + 1 : v0;
        if (k == v0) {
          float x = fmaf(sc[PAR][r], c, -lq);
          if constexpr (MASKED) {
            // score r = 4g + e is S^T row 8g + 4h + e: key perm(8(g%2) + 4h + e) + 16(g/2)
            const int g = r / 4, e = r % 4;
            const int koff = 16 * (g / 2) + 4 * e + 2 * (g % 2);
            x = koff <= thr ? x : -INFINITY;
          }
          pe[r] = fast_exp2(x);
        }
        if (k == v1) {
          dsv[r] = pe[r] * dp[PAR][r];  // dp holds dP - D
          if (r & 1) dsk[PAR][r / 8][(r / 2) % 4] = TR::pack2(dsv[r - 1], dsv[r]);
        }
      }
      if constexpr (PAR == 0) {
        if (k < NPART) load_part(j_ld, k);
      } else {
        if (k >= kW0 && k < kW0 + NPART) store_part(sbw, k - kW0);
      }
    };
    static_for<0, NSL>([&](auto kc) __attribute__((always_inline)) {
      constexpr int k = decltype(kc)::value;
      constexpr int x = k / 3;
      const u32x4_t a = fr[k % AH];
      if constexpr (k + AH < NSL) fr[k % AH] = frag(k + AH, sb1, sb2, NB);
      else fr[k % AH] = frag(k + AH - NSL, nsb1, nsb2, PAR);
      if constexpr (k % 3 == 0) {
        if constexpr (x == 0) sc[NB] = PM::mb0(a, qf[0]);
        else PM::mb(sc[NB], a, qf[x]);
      } else if constexpr (k % 3 == 1) {
        PM::macc(acc[x % NDB], a, dsk[NB][x / NDB]);
      } else {
        if constexpr (x == 0) dp[NB] = PM::mbc(a, of[0], negd);
        else PM::mb(dp[NB], a, of[x]);
      }
      vwork(k);
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // ---- prologue: stages 0 and 1 in slots 0 and 1, slot 3 zeroed (the first
  // iteration multiplies it by zero dS); S_0, dP_0; first operands
#pragma unroll
  for (int j = 0; j < NPART; ++j) load_part(0, j, 0);
#pragma unroll
  for (int j = 0; j < NPART; ++j) load_part(BC, j, 1);
#pragma unroll
  for (int j = 0; j < NPART; ++j) store_part(0, j, 0);
#pragma unroll
  for (int j = 0; j < NPART; ++j) store_part(STG, j, 1);
  for (int i = tid; i < STG / 16; i += NT) *(u32x4_t*)(smem + 3 * STG + 16 * i) = u32x4_t{0u, 0u, 0u, 0u};
  lds_barrier();
  mma_pipeline<2 * NKS, 3>([&](int x) { return smem + ((x & 1) ? OFF_V : 0) + rbase + 32 * (x >> 1); },
                           [&](int x, u32x4_t a) {
                             const int ks = x >> 1;
                             if (x & 1) {
                               if (ks == 0) dp[0] = PM::mbc(a, of[0], negd);
                               else PM::mb(dp[0], a, of[ks]);
                             } else if (ks == 0) {
                               sc[0] = PM::mb0(a, qf[0]);
                             } else {
                               PM::mb(sc[0], a, qf[ks]);
                             }
                           },
                           [](int) {});
#pragma unroll
  for (int t = 0; t < 2; ++t) dsk[1][t] = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
  for (int x = 0; x < AH; ++x) fr[x] = frag(x, 0u, 3u * STG, 1);

  // ---- pairs of iterations over the stages.  Causal: the stages with a key
  // that some row of the workgroup does not see are masked (with the square
  // mask: the last two, each wavefront's diagonal block and the fully masked
  // blocks past it).
  auto pair = [&](auto masked_c, int s) __attribute__((always_inline)) {
    const uint32_t b0 = (uint32_t)(s & 3) * STG;
    const uint32_t bp1 = (uint32_t)((s + 1) & 3) * STG;
    const uint32_t bm1 = (uint32_t)((s + 3) & 3) * STG;
    const uint32_t bp2 = (uint32_t)((s + 2) & 3) * STG;
    const int j0 = BC * s;
    iteration(std::integral_constant<int, 0>{}, masked_c, b0, bm1, bp1, b0, j0, j0 + 2 * BC, bp2);
    iteration(std::integral_constant<int, 1>{}, masked_c, bp1, b0, bp1, b0, j0 + 32, 0, bp2);
    lds_barrier();
  };
  const int n_open = CAUSAL ? min(max(q0 + delta + 1, 0) / BC, n_st) : n_st;
  int s = 0;
  for (; s < n_open; ++s) pair(std::false_type{}, s);
  for (; s < n_st; ++s) pair(std::true_type{}, s);

  // ---- last block: its dQ products (register set 1)
  {
    const uint32_t sb = (uint32_t)((n_st - 1) & 3) * STG;
    asm volatile("" : "+v"(dsk[1][0]), "+v"(dsk[1][1]));
#pragma unroll
    for (int x = 0; x < NKS; ++x) PM::macc(acc[x % NDB], tr_frag(sb, 1, x / NDB, x % NDB), dsk[1][x / NDB]);
  }
  if constexpr (NDB == 4) PM::wait_acc(acc[0], acc[1], acc[2], acc[3]);
  else PM::wait_acc(acc[0], acc[1]);

  u32x2_t od[NDB][4];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      od[db][g] = u32x2_t{TR::pack2(acc[db][4 * g + 0] * scale, acc[db][4 * g + 1] * scale),
                          TR::pack2(acc[db][4 * g + 2] * scale, acc[db][4 * g + 3] * scale)};
  // dQ stored as whole rows through LDS: after the last barrier every stage
  // slot but that of the last block is free
  static_assert(4 * kTileRowsBytes<D> <= STG, "four wavefronts' rows fit one stage slot");
  store_tile_rows<D>(smem + ((n_st + 1) & 3) * STG + w * kTileRowsBytes<D>, od,
                     dQ + dq_off + (size_t)qw * dqs, min(32, Lq - qw), lane, dqs, nch);
  };
  for_each_tile(total, (uint32_t)n_qtiles, run_tile);
}

// ------------------------------------------------------------------ launch

template <class TR, int D>
static hipError_t prep_t(const BwdArgs& a) {
  constexpr int RPB = 256 / (D / 8);
  const int rows = a.BH * a.Nq;
  if (a.general)
    hipLaunchKernelGGL((bwd_pre_kernel<TR, D, true>), dim3((rows + RPB - 1) / RPB), dim3(256), 0, a.stream,
                       (const uint16_t*)a.o, (const uint16_t*)a.dout, a.dvec, rows, a.Nq, a.g);
  else
    hipLaunchKernelGGL((bwd_pre_kernel<TR, D, false>), dim3((rows + RPB - 1) / RPB), dim3(256), 0, a.stream,
                       (const uint16_t*)a.o, (const uint16_t*)a.dout, a.dvec, rows, a.Nq, a.g);
  return hipGetLastError();
}

template <class TR, int D, bool CAUSAL, bool GL>
static void dkdv_launch(const BwdArgs& a) {
  const int n_ktiles = (a.Nk + 127) / 128;
  const uint32_t total = (uint32_t)(n_ktiles * a.BH);
  // The kernel forms the exponent as (q.k - LSE / s) * s log2 e with s the
  // scale (of either sign: no running maximum is taken here).  Below 2^-100
  // in magnitude (scale 0 included) it takes s = +-2^-100 there, so that
  // -1 / s stays finite: q.k then vanishes beside LSE / s in float and the
  // exponent is -LSE log2 e, its value at scale 0 (dK is still multiplied by
  // the true scale).
  const float mag = fmaxf(fabsf(a.scale), 0x1p-100f);
  const float s = a.scale < 0.0f ? -mag : mag;
  // persistent (one workgroup per resident slot) when the tiles deal out evenly
  const uint32_t grid = persistent_grid(a.BH, n_ktiles, D == 128 ? 1 : 2, a.stream);
  hipLaunchKernelGGL((bwd_dkdv_pipe_kernel<TR, D, CAUSAL, D == 128 ? 1 : 2, GL>), dim3(grid), dim3(256), 0,
                     a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                     (const uint16_t*)a.dout, a.lse, a.dvec, (uint16_t*)a.dk, (uint16_t*)a.dv,
                     a.Nq, a.Nk, n_ktiles, total, s * kLog2e, -1.0f / s, a.scale, a.g);
}

template <class TR, int D, bool CAUSAL>
static hipError_t dkdv_t(const BwdArgs& a) {
  if (a.general) dkdv_launch<TR, D, CAUSAL, true>(a);
  else dkdv_launch<TR, D, CAUSAL, false>(a);
  return hipGetLastError();
}

// dQ: the pipelined kernel, one wavefront per SIMD at d = 128 and two at d = 64
template <class TR, int D, bool CAUSAL, bool GL>
static void dq_launch(const BwdArgs& a) {
  const int n_qtiles = (a.Nq + 127) / 128;
  const uint32_t total = (uint32_t)(n_qtiles * a.BH);
  // persistent (one workgroup per resident slot) when the tiles deal out evenly
  const uint32_t grid = persistent_grid(a.BH, n_qtiles, D == 128 ? 1 : 2, a.stream);
  hipLaunchKernelGGL((bwd_dq_pipe_kernel<TR, D, CAUSAL, D == 128 ? 1 : 2, GL>), dim3(grid), dim3(256), 0,
                     a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                     (const uint16_t*)a.dout, a.lse, a.dvec, (uint16_t*)a.dq, a.Nq, a.Nk, n_qtiles, total,
                     a.c, a.scale, a.g);
}

template <class TR, int D, bool CAUSAL>
static hipError_t dq_t(const BwdArgs& a) {
  if (a.general) dq_launch<TR, D, CAUSAL, true>(a);
  else dq_launch<TR, D, CAUSAL, false>(a);
  return hipGetLastError();
}

// the kernels' width: d = 128 and 96 (general layout, zero columns) on the
// d = 128 kernels, d = 64 and 32 on the d = 64 kernels
template <class TR>
static hipError_t stage_t(const BwdArgs& a, int stage) {
  if (a.d == 256) {  // the wide kernels (fa_bwd_wide.hip), always in the general layout
    if (stage != BWD_PREP) return launch_bwd_wide_stage(a, stage);
    const int rows = a.BH * a.Nq;
    hipLaunchKernelGGL((bwd_pre_kernel<TR, 256, true>), dim3((rows + 7) / 8), dim3(256), 0, a.stream,
                       (const uint16_t*)a.o, (const uint16_t*)a.dout, a.dvec, rows, a.Nq, a.g);
    return hipGetLastError();
  }
  const bool d128 = a.d > 64;
  switch (stage) {
    case BWD_PREP: return d128 ? prep_t<TR, 128>(a) : prep_t<TR, 64>(a);
    case BWD_DKDV:
      if (d128) return a.causal ? dkdv_t<TR, 128, true>(a) : dkdv_t<TR, 128, false>(a);
      return a.causal ? dkdv_t<TR, 64, true>(a) : dkdv_t<TR, 64, false>(a);
    default:
      if (d128) return a.causal ? dq_t<TR, 128, true>(a) : dq_t<TR, 128, false>(a);
      return a.causal ? dq_t<TR, 64, true>(a) : dq_t<TR, 64, false>(a);
  }
}

hipError_t launch_bwd_stage(const BwdArgs& a, int stage) {
  return a.dtype == DT_BF16 ? stage_t<BF16>(a, stage) : stage_t<F16>(a, stage);
}

hipError_t launch_bwd(const BwdArgs& a) {
  for (int st : {BWD_PREP, BWD_DKDV, BWD_DQ}) {
    const hipError_t e = launch_bwd_stage(a, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace fa
