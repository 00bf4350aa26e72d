// Forward attention kernels for gfx950: O = softmax(scale * Q K^T [causal]) V,
// plus the per-row log-sum-exp, computed tiled and fused in one pass.
//
// The method ("FlashAttention" lexicon, "Methodische Grundlagen"): Q, K, V are
// cut into blocks that fit on-chip memory; similarity, normalisation and
// weighting run in one pass with no intermediate in HBM; the row normaliser
// is accumulated as the keys stream by and earlier partial results are
// corrected when a larger score appears; only the log-sum-exp per row is kept
// for the backward pass.  The work split follows "FlashAttention-2 (DE)",
// "Technische Architektur", items 1-3: few non-matmul operations, one head
// spread over many compute units (one workgroup per query tile and head), and
// query rows split across wavefronts so each wavefront normalises its own
// rows without exchanging partial results through shared memory.
//
// gfx950 mapping (16-bit inputs):
//   * workgroup = 8 wavefronts (two per SIMD) x 32 query rows; grid = query
//     tiles x (batch * heads), XCD-grouped, heaviest causal tiles first.
//   * each wavefront computes S^T = K Q^T with v_mfma_f32_32x32x16: the
//     accumulator then holds, per lane, one query row (lane % 32) and 16 keys,
//     so row reductions are in-lane plus one exchange between half-waves,
//     and the probabilities are already in the B-operand layout of
//     O^T += V^T P^T (they never leave registers).
//   * K and V tiles are staged HBM -> registers -> LDS with coalesced loads
//     while earlier tiles are consumed; K row-major (padded rows), V in an
//     interleaved, bank-swizzled layout that is one 16-byte read per product.
//   * softmax in the exp2 domain with scale*log2(e) folded into one FMA and a
//     single normalisation at the end.  Two kernels: fwd16_pipe_kernel (d =
//     128) software-pipelines matrix and vector work inside each wavefront
//     against a fixed reference maximum; fwd16_pp_kernel (d = 64) alternates
//     whole matrix and vector phases between the two wavefronts of a SIMD;
//     both against a reference maximum fixed by the first key tile.
//   * causal: key tiles above a workgroup's diagonal are never loaded or
//     multiplied; only tiles crossing the diagonal are masked.
#include <type_traits>

#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {

// Row of a 32-key block that accumulator row m of S^T reads at d = 256:
// inside each 16 keys, row 4 (m mod 4) + (m / 4) mod 4, so that the keys of
// the probabilities one lane holds for a 16-key step are the rows a
// transposed read of V gives it.
__device__ constexpr int key_perm(int m) { return (m & 16) | ((m & 3) << 2) | ((m >> 2) & 3); }

// Reference maximum of both 16-bit kernels: fixed by the first tile, and
// changed only when the sum of a row's probabilities over one key tile
// exceeds this bound (the pipelined kernel then redoes its pass against exact
// row maxima, the ping-pong kernel re-bases that tile); no single
// probability, nor a packed fp16 value, can exceed it.  The final
// normalisation uses the same reference for numerator and denominator.
constexpr float kSumMax = 32768.0f;

// 16-bit forward, software-pipelined (used for d = 128).  Two wavefronts
// per SIMD (8 per workgroup), each owning QB = 1 block of 32 query rows.  Key
// tiles of BC keys are processed as a software pipeline inside each
// wavefront; iteration j issues
//   matrix cores:  S_{j+1} = K_{j+1} Q^T   and   O += V_{j-1}^T P_{j-1}
//   vector ALU:    softmax of S_j -> P_j
// interleaved instruction by instruction (the two kinds of work are
// independent within an iteration), plus the staging of later tiles.  Two
// such wavefronts share each SIMD, so one's matrix instructions run under the
// other's vector work.  One workgroup barrier per iteration hands the LDS
// buffers over.
//
// Softmax: against a reference maximum m_run fixed by the first tile (its
// exact row maximum), every score is read once (scale, shift, exp2, pack,
// sum).  If a row's tile sum ever exceeds kSumMax its probabilities may be out
// of range: the wavefront raises a flag and the workgroup redoes the whole
// pass against exact row maxima computed directly from Q and K (every
// probability is then at most 1).  So the steady state never re-bases O.
//
// Staging (all threads): iteration j writes K_{j+2} and V_j to LDS from
// registers loaded during iteration j-1, then requests K_{j+3} and V_{j+1}
// (d = 256: from registers loaded during iteration j-2, then requests K_{j+4}
// and V_{j+2} into the same registers).  Iteration j reads K_{j+1} and
// V_{j-1}, so two buffers of each suffice.
//
// LDS layouts (per buffer):
//   K: row-major, rows padded to D + 8 elements, so 16 consecutive rows read
//      at one 16-byte column fall in distinct banks and every fragment address
//      is a fixed offset from one base.
//   V: [key/16][h][d][8]: the 16-byte unit (s, h, c) holds column c of keys
//      16s + 4h + {0,1,2,3} and 16s + 8 + 4h + {0,1,2,3}, exactly the eight
//      values lane (c % 32, h) needs for one O^T += V^T P^T instruction.
//      Within a row (s, h) column c sits at slot c ^ ((c >> 3) & 3), so the
//      staging writes (lanes CW columns apart) and the fragment reads (lanes
//      on consecutive columns) both hit distinct banks.
//
// d = 256 stages V row-major like K instead (rows padded to D + 8) and reads
// its product operand with two transposed reads, K operand rows in the order
// key_perm.
//
// d <= 128: all matrix operands and accumulators live in VGPRs (the MfmaAsm
// forms), two wavefronts per SIMD.  d = 256: one wavefront per SIMD (4 per
// workgroup, 128 rows), with the Q fragments (B operands of S) and the O
// accumulators in AGPRs (PipeMma with AG), 32-key tiles, and two query tiles
// per workgroup (total = workgroups: one per tile at d <= 128, where a second
// tile adds spills, one per pair of tiles at d = 256).
template <class TR, int D, int BC, int QB, bool CAUSAL, bool GL>
__global__ __launch_bounds__(D > 128 ? 256 : 512 / QB)
__attribute__((amdgpu_waves_per_eu(D > 128 ? 1 : 3 - QB, D > 128 ? 1 : 3 - QB)))
void fwd16_pipe_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                  const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                  float* __restrict__ LSE, int N, int n_qtiles, uint32_t total, float c, GenLayout g) {
  // QB: 32-row query blocks per wavefront (2: one wavefront per SIMD, 1: two;
  // d = 256: 1 at one wavefront per SIMD)
  constexpr bool AG = D > 128;          // Q and O in AGPRs
  using PM = PipeMma<TR, AG>;
  constexpr int NT = AG ? 256 : 512 / QB;  // threads per workgroup
  constexpr int NW = NT / 64;           // wavefronts per workgroup
  constexpr int BR = NW * 32 * QB;      // query rows per workgroup (256; 128 at d = 256)
  constexpr int KS = D + 8;             // padded K row (elements)
  constexpr int NKB = BC / 32;          // 32-key blocks per tile
  constexpr int NDB = D / 32;           // 32-column blocks of the output
  constexpr int NKS = D / 16;           // k-steps of S over d
  constexpr int NSS = BC / 16;          // k-steps of O over the keys of a tile
  constexpr int NQF = NKB * NKS;        // K fragments per tile
  constexpr int NVF = NSS * NDB;        // V fragments per tile
  constexpr int NS = QB * (NQF + NVF);  // matrix instructions per iteration
  constexpr int KCH = D / 8;            // 16-byte chunks per row
  constexpr int NKC = BC * KCH / NT;    // K chunks staged per thread
  constexpr int CW = BC * D / (8 * NT); // V columns staged per thread (8 keys each)
  constexpr int NCG = D / CW;           // V column groups
  constexpr uint32_t RB = D * 2;        // bytes per row
  static_assert(NQF == NVF, "the two products alternate one to one");
  static_assert(NKC >= 1 && (CW == 2 || CW == 4), "staging split over all threads");
  constexpr int NBLK = QB * NKB;        // 32x32 score blocks per wavefront and tile
  constexpr int NPAIR = NBLK * 8;       // packed probability pairs per lane and tile
  // staging inside an iteration (step = one matrix instruction)
  constexpr int kStg0 = 2;              // staging writes every other step from here
  constexpr int kLoad = kStg0 + 2 * (NKC + CW);  // then the loads of later tiles
  static_assert(kLoad < NS, "schedule fits one iteration");

  __shared__ __attribute__((aligned(16))) uint16_t sK[2][BC * KS];
  // d = 256: V row-major like K (rows padded to D + 8), its product operands
  // read transposed; d <= 128: the interleaved layout below
  constexpr int VSR = AG ? D + 8 : D;
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][BC * VSR];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int h = lane >> 5;
  const int l32 = lane & 31;

  // d = 256: tile t and tile nt - 1 - t of one head (equal work with the
  // causal mask; the middle tile of an odd count once); d <= 128: one tile.
  // The workgroups of one head run on one XCD.
  constexpr int NTILE = D > 128 ? 2 : 1;
  for (int it = 0; it < NTILE; ++it) {
  uint32_t lid;
  if constexpr (D > 128) {
    const uint32_t nt = (uint32_t)n_qtiles, npair = (nt + 1) / 2;
    const uint32_t pid = xcd_remap(blockIdx.x, total);
    const uint32_t hh = pid / npair, tt = pid % npair;
    if (it == 1) {
      if (nt - 1 - tt == tt) break;
      lds_barrier();
    }
    lid = hh * nt + (it == 0 ? tt : nt - 1 - tt);
  } else {
    lid = xcd_remap(blockIdx.x, total);
  }
  const int bh = lid / n_qtiles;
  int qt = lid % n_qtiles;
  if (CAUSAL) qt = n_qtiles - 1 - qt;  // heaviest tiles first
  const int q0 = qt * BR;
  // Addressing: dense [BH, N, D], or (GL) the general layout: per-tensor
  // strides, a packed self-attention batch (head bh's Nb rows, its sequence;
  // tiles wholly past them skipped), and data with DR < D columns (columns
  // past DR read zeros and are not stored).
  int Nb = N, DR = D;
  size_t q_off, k_off, v_off, o_off, l_off, os;
  uint32_t q_bytes, k_bytes, v_bytes, rsq, rsk, rsv;
  if constexpr (GL) {
    const int b = bh / g.H, hd = bh - b * g.H;
    int sq, sk, nq, nk;
    seq_rows(g.cu_q, g.total_q, b, N, sq, nq);
    seq_rows(g.cu_k, g.total_k, b, N, sk, nk);
    Nb = min(nq, nk);  // self-attention: equal counts (malformed sums: the smaller)
    DR = g.dr;
    const TRows tq = tensor_rows(g.q, b, hd, sq, Nb, DR), tk = tensor_rows(g.k, b, hd, sk, Nb, DR);
    const TRows tv = tensor_rows(g.v, b, hd, sk, Nb, DR), to = tensor_rows(g.o, b, hd, sq, Nb, DR);
    q_off = tq.off, k_off = tk.off, v_off = tv.off, o_off = to.off;
    q_bytes = tq.bytes, k_bytes = tk.bytes, v_bytes = tv.bytes;
    rsq = tq.rs, rsk = tk.rs, rsv = tv.rs;
    os = (size_t)g.o.sr;
    l_off = (size_t)((int64_t)b * g.l_sb + (int64_t)hd * g.l_sh + sq);
  } else {
    q_off = k_off = v_off = o_off = (size_t)bh * N * D;
    q_bytes = k_bytes = v_bytes = (uint32_t)N * RB;
    rsq = rsk = rsv = RB;
    os = D;
    l_off = (size_t)bh * N;
  }
  if (GL && q0 >= Nb) continue;
  // the row strides as the staging loads use them: re-read per use in the
  // general layout, so that the per-row offsets are not kept live across the loop
  auto row_stride_k = [&]() __attribute__((always_inline)) -> uint32_t {
    if constexpr (GL) return __builtin_amdgcn_readfirstlane(rsk);
    return RB;
  };
  auto row_stride_v = [&]() __attribute__((always_inline)) -> uint32_t {
    if constexpr (GL) return __builtin_amdgcn_readfirstlane(rsv);
    return RB;
  };
  const int qw = q0 + 32 * QB * w;  // first query row of this wavefront

  // Q rows as the B operand of S^T = K Q^T, loaded once (rows past the end
  // read zeros; their results are never stored); their signs are flipped for
  // a negative scale once they have arrived (first pass's prologue).
  u32x4_t qf[QB][NKS];
  {
    const rsrc_t qres = make_rsrc(Q + q_off, q_bytes);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        qf[qb][ks] = buf_load16(qres, (uint32_t)(qw + 32 * qb + l32) * rsq + 32 * ks + 16 * h +
                                          (GL ? col_pad(32 * ks + 16 * h, DR, q_bytes) : 0u));
  }

  const int kv_end = CAUSAL ? min(Nb, q0 + BR) : Nb;
  const int n_tiles = (kv_end + BC - 1) / BC;

  // ---- staging.  Rows past the end of the sequence read zeros (their scores
  // are masked, their values multiplied by zero probabilities).
  const rsrc_t kres = make_rsrc(K + k_off, k_bytes);
  const rsrc_t vres = make_rsrc(V + v_off, v_bytes);
  // Staging register sets.  Two at d = 256, where one wavefront per SIMD
  // leaves no partner to run while a wavefront waits: each iteration then
  // writes data loaded two iterations earlier, so a load has two
  // iterations, not one, to arrive.
  constexpr int NSET = AG ? 2 : 1;
  u32x4_t stk[NSET][NKC];
  uint32_t stv[NSET][8][CW / 2];
  u32x4_t stvr[AG ? NSET : 1][AG ? NKC : 1];  // d = 256: V chunks as K's
  const uint32_t voffr = (uint32_t)(tid / KCH) * rsv + (tid % KCH) * 16 +
                         (GL ? col_pad((tid % KCH) * 16, DR, v_bytes) : 0u);
  // K: chunk tid + NT r -> row (tid / KCH) + (NT / KCH) r, 16-byte column tid % KCH
  const uint32_t koff = (uint32_t)(tid / KCH) * rsk + (tid % KCH) * 16 +
                        (GL ? col_pad((tid % KCH) * 16, DR, k_bytes) : 0u);
  const int kst = (tid / KCH) * KS + (tid % KCH) * 8;
  // V: unit tid -> (16-key step vs, half vh, column group vc); 8 rows x CW columns
  const int vc = tid % NCG;
  const int vh = (tid / NCG) & 1;
  const int vs = tid / (2 * NCG);
  const uint32_t voff = (uint32_t)(16 * vs + 4 * vh) * rsv + vc * CW * 2 +
                        (GL ? col_pad(vc * CW * 2, DR, v_bytes) : 0u);
  const int vrow = (2 * vs + vh) * D * 8;
  const int vsw = (CW * vc) ^ ((CW * vc >> 3) & 3);  // swizzled slot of column CW vc (+ cc: xor)

  auto load_k = [&](int tile, int set = 0) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < NKC; ++r)
      stk[set][r] = buf_load16(kres, koff + (uint32_t)(tile * BC + (NT / KCH) * r) * row_stride_k());
  };
  auto load_v = [&](int tile, int set = 0) __attribute__((always_inline)) {
    if constexpr (AG) {
#pragma unroll
      for (int r = 0; r < NKC; ++r)
        stvr[set][r] = buf_load16(vres, voffr + (uint32_t)(tile * BC + (NT / KCH) * r) * row_stride_v());
      return;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t off = voff + (uint32_t)(tile * BC + 8 * (k / 4) + (k % 4)) * row_stride_v();
      if constexpr (CW == 4) {
        const u32x2_t x = buf_load8(vres, off);
        stv[set][k][0] = x[0];
        stv[set][k][1] = x[1];
      } else {
        stv[set][k][0] = __builtin_amdgcn_raw_buffer_load_b32(vres, off, 0, 0);
      }
    }
  };
  // staging write number i (0 <= i < NKC + CW) into buffer b, from register set `set`
  auto store_part = [&](int i, int b, int set = 0) __attribute__((always_inline)) {
    if (i < NKC) {
      *(u32x4_t*)(&sK[b][kst + i * (NT / KCH) * KS]) = stk[set][i];
    } else if constexpr (AG) {
      *(u32x4_t*)(&sV[b][(tid / KCH + (i - NKC) * (NT / KCH)) * VSR + (tid % KCH) * 8]) = stvr[set][i - NKC];
    } else {
      const int cc = i - NKC;  // column within the group
      uint32_t o[4];
#pragma unroll
      for (int kp = 0; kp < 4; ++kp) {
        const uint32_t x0 = stv[set][2 * kp][cc / 2], x1 = stv[set][2 * kp + 1][cc / 2];
        o[kp] = (cc & 1) ? pack_hi(x0, x1) : pack_lo(x0, x1);
      }
      *(u32x4_t*)(&sV[b][vrow + 8 * (vsw ^ cc)]) = u32x4_t{o[0], o[1], o[2], o[3]};
    }
  };

  // ---- per-lane state
  // element offset of this lane's K fragment; d = 256: row key_perm(l32), so
  // that the keys of the probabilities a lane holds for a 16-key step are
  // the rows a transposed V read gives it (4 apart: bank-conflict free)
  const int kfrag = (AG ? key_perm(l32) : l32) * KS + 8 * h;
  const int vfrag = (h * D + (l32 ^ ((l32 >> 3) & 3))) * 8;  // this lane's V fragment
  f32x16_t acc[QB][NDB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[qb][db] = zero16();
  f32x16_t sA[QB][NKB], sB[QB][NKB];      // scores of two consecutive tiles
  // packed probabilities of two tiles: [qb][kb][t] is the B operand of the
  // O product for the keys 32 kb + 16 t + ...
  u32x4_t pA[QB][NKB][2], pB[QB][NKB][2];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) pB[qb][kb][0] = pB[qb][kb][1] = u32x4_t{0u, 0u, 0u, 0u};
  float m_run[QB], lsum[QB][NKB], ltsum[QB][NKB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) lsum[qb][kb] = ltsum[qb][kb] = 0.0f;
  }

  // fragment addresses: QK fragment i -> (kb, ks); PV fragment i -> (k-step, db)
  auto kaddr = [&](int b, int i) -> const uint16_t* {
    return sK[b] + kfrag + 32 * (i % NKB) * KS + 16 * (i / NKB);
  };
  auto vaddr = [&](int b, int i) -> const uint16_t* {
    return sV[b] + vfrag + (2 * (i / NDB) * D + 32 * (i % NDB)) * 8;
  };
  // PV operand i of buffer b (k-step i / NDB, column block i % NDB)
  const int vtr = (h + 4 * ((lane & 15) >> 2)) * VSR + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  auto vread = [&](int b, int i) __attribute__((always_inline)) -> u32x4_t {
    if constexpr (AG) {
      const uint16_t* p = sV[b] + vtr + 16 * (i / NDB) * VSR + 32 * (i % NDB);
      const u32x2_t a0 = lds_read_tr(p), a1 = lds_read_tr(p + 2 * VSR);
      return u32x4_t{a0[0], a0[1], a1[0], a1[1]};
    }
    return *(const u32x4_t*)vaddr(b, i);
  };
  auto pfrag = [&](const u32x4_t (&p)[QB][NKB][2], int qb, int ss) -> u32x4_t { return p[qb][ss / 2][ss % 2]; };
  // All score blocks of one register set, or all O accumulators, as operands
  // of a hazard wait (matrix result -> vector access).
  auto wait_scores = [&](f32x16_t (&sc)[QB][NKB]) __attribute__((always_inline)) {
    f32x16_t* x = &sc[0][0];  // QB * NKB blocks
    static_assert(QB * NKB == 1 || QB * NKB == 2 || QB * NKB == 4, "operand list below");
    if constexpr (QB * NKB == 1) mfma_wait_v(x[0]);
    else if constexpr (QB * NKB == 2) mfma_wait_v(x[0], x[1]);
    else mfma_wait_v(x[0], x[1], x[2], x[3]);
  };
  auto wait_acc = [&]() __attribute__((always_inline)) {
    f32x16_t* x = &acc[0][0];  // QB * NDB blocks
    static_assert(QB * NDB == 2 || QB * NDB == 4 || QB * NDB == 8, "operand list below");
    if constexpr (QB * NDB == 2) PM::wait_acc(x[0], x[1]);
    else if constexpr (QB * NDB == 4) PM::wait_acc(x[0], x[1], x[2], x[3]);
    else PM::wait_acc(x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]);
  };

  bool rerun = false;
  bool exact = false;  // second pass: m_run holds exact row maxima
  // ---- one pipelined iteration.  PAR = j & 1 selects register sets and
  // buffers; MASKED tiles (crossing the causal diagonal or the end of the
  // sequence) mask scores as they are read.
  auto iteration = [&](auto par, auto masked, int j) __attribute__((always_inline)) {
    constexpr int PAR = decltype(par)::value;
    constexpr bool MASKED = decltype(masked)::value;
    f32x16_t(&s_cur)[QB][NKB] = PAR ? sB : sA;
    f32x16_t(&s_next)[QB][NKB] = PAR ? sA : sB;
    u32x4_t(&p_prev)[QB][NKB][2] = PAR ? pA : pB;
    u32x4_t(&p_cur)[QB][NKB][2] = PAR ? pB : pA;
    constexpr int RD = 1 - PAR;  // buffers read: K_{j+1}, V_{j-1}
    constexpr int WR = PAR;      // buffers written: K_{j+2}, V_j
    const int j0 = j * BC;
    wait_scores(s_cur);  // S_j was produced by matrix instructions

    // score r of block (qb, kb), -inf where masked: its key j0 + 4h + off(kb, r)
    // is hidden iff off >= lim[qb], the first hidden key of the row (the end of
    // the sequence, or causally the key after the row's own) less j0 + 4h --
    // one compare per score against a value of this iteration
    int lim[QB];
    if constexpr (MASKED) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        lim[qb] = (CAUSAL ? min(Nb, qw + 32 * qb + l32 + 1) : Nb) - j0 - (AG ? h : 4 * h);
    }
    auto score = [&](int qb, int kb, int r) __attribute__((always_inline)) -> float {
      const float x = s_cur[qb][kb][r];
      // key of score r less j0 and the lane's part (4 h; d = 256: h)
      const int koff = AG ? 16 * (r / 8) + 4 * (r % 4) + 2 * ((r / 4) & 1) : 8 * (r / 4) + (r % 4);
      if constexpr (MASKED) return 32 * kb + koff >= lim[qb] ? -INFINITY : x;
      return x;
    };

    // Softmax of S_j against the reference maximum m_run, as a software
    // pipeline over the steps: pair i of scores (two adjacent values of one
    // block) enters at step i * NS / NPAIR and advances one stage per step,
    //   stage 0: scale and shift (fma)    stage 1: exp2
    //   stage 2: pack, fp32 sums          stage 3: 16-bit sums, keep P
    // so the instructions of one step never depend on each other.  No row
    // maximum is searched here: a row whose tile sum exceeds kSumMax (its
    // maximum grew a lot since the first tile) raises `rerun` below.
    if (j == 0 && !exact) {
      // first tile: its exact row maximum (over both half-waves) is the
      // reference; finite, as key 0 is visible to every row
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; r += 2) mx = max3f(mx, score(qb, kb, r), score(qb, kb, r + 1));
        const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, mx),
                                                         __builtin_bit_cast(uint32_t, mx), false, false);
        m_run[qb] = __builtin_elementwise_maximum(__builtin_bit_cast(float, (uint32_t)sw[0]),
                                                  __builtin_bit_cast(float, (uint32_t)sw[1])) * c;
      }
    }
    float tl[QB][NKB], tlt[QB][NKB];
    float mneg[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) mneg[qb] = -m_run[qb];
    float ta[NPAIR][2], te[NPAIR][2];
    uint32_t tp[NPAIR];
    auto stage = [&](int i, int k) __attribute__((always_inline)) {
      const int b = i % NBLK, rp = i / NBLK;
      const int qb = b / NKB, kb = b % NKB;
      if (k == 0) {
        ta[i][0] = fmaf(score(qb, kb, 2 * rp), c, mneg[qb]);
        ta[i][1] = fmaf(score(qb, kb, 2 * rp + 1), c, mneg[qb]);
      } else if (k == 1) {
        te[i][0] = fast_exp2(ta[i][0]);
        te[i][1] = fast_exp2(ta[i][1]);
      } else if (k == 2) {
        tp[i] = TR::pack2(te[i][0], te[i][1]);
        tl[qb][kb] = rp == 0 ? te[i][0] + te[i][1] : tl[qb][kb] + (te[i][0] + te[i][1]);
      } else {
        tlt[qb][kb] = TR::sum2(tp[i], rp == 0 ? 0.0f : tlt[qb][kb]);
        pin(tp[i]);
        p_cur[qb][kb][rp / 4][rp % 4] = tp[i];
        if (rp == 7) {
          pin(tl[qb][kb]);
          pin(tlt[qb][kb]);
        }
      }
    };
    auto valu = [&](int st) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < NPAIR; ++i)
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (i * NS / NPAIR + k == st) stage(i, k);
      // staging: writes of K_{j+2} and V_j, then requests for K_{j+3}, V_{j+1}
      if constexpr (NSET == 1) {
        if (st == kStg0) wait_vmem();
        if (st >= kStg0 && st < kLoad && (st - kStg0) % 2 == 0) store_part((st - kStg0) / 2, WR);
        if (st == kLoad) {
          load_k(j + 3);
          load_v(j + 1);
        }
      } else {
        // set PAR holds K_{j+2} and V_j (loaded two iterations ago; the
        // compiler waits for exactly those loads) and then receives K_{j+4},
        // V_{j+2}
        if (st >= kStg0 && st < kLoad && (st - kStg0) % 2 == 0) store_part((st - kStg0) / 2, WR, PAR);
        if (st == kLoad) {
          load_k(j + 4, PAR);
          load_v(j + 2, PAR);
        }
      }
    };

    // matrix instructions: fragment f (even: V fragment of O += V^T P, odd:
    // K fragment of S) feeds QB products; operand reads run kAhead fragments
    // ahead (at d = 256, 8 ahead measured no faster).  Steps past NS only
    // finish the softmax pipeline.
    constexpr int kAhead = 3;
    constexpr int NF = NQF + NVF;
    auto is_pv = [](int f) { return (f & 1) == 0; };
    auto fidx = [](int f) { return f >> 1; };
    auto faddr = [&](int f) -> const uint16_t* {
      return is_pv(f) ? vaddr(RD, fidx(f)) : kaddr(RD, fidx(f));
    };
    auto fread = [&](int f) __attribute__((always_inline)) -> u32x4_t {
      if (is_pv(f)) return vread(RD, fidx(f));
      return *(const u32x4_t*)kaddr(RD, fidx(f));
    };
    u32x4_t fr[kAhead];
#pragma unroll
    for (int x = 0; x < kAhead; ++x) fr[x] = fread(x);
    static_for<0, NS + 3>([&](auto stc) __attribute__((always_inline)) {
      constexpr int st = decltype(stc)::value;
      if constexpr (st < NS) {
        constexpr int f = st / QB, qb = st % QB;
        const u32x4_t a = fr[f % kAhead];
        if constexpr (qb == QB - 1 && f + kAhead < NF) fr[f % kAhead] = fread(f + kAhead);
        constexpr int i = fidx(f);
        if constexpr (is_pv(f)) {
          constexpr int ss = i / NDB, db = i % NDB;
          PM::macc(acc[qb][db], a, pfrag(p_prev, qb, ss));
        } else {
          constexpr int kb = i % NKB, ks = i / NKB;
          if constexpr (ks == 0) s_next[qb][kb] = PM::mb0(a, qf[qb][ks]);
          else PM::mb(s_next[qb][kb], a, qf[qb][ks]);
        }
      }
      valu(st);
      __builtin_amdgcn_sched_barrier(0);
    });

    // Tile row sums over both half-waves (the swap leaves the two halves'
    // values in the two results, in some order, in every lane).
    bool big = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float t = tl[qb][0];
#pragma unroll
      for (int kb = 1; kb < NKB; ++kb) t += tl[qb][kb];
      const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, t),
                                                       __builtin_bit_cast(uint32_t, t), false, false);
      t = __builtin_bit_cast(float, (uint32_t)sw[0]) + __builtin_bit_cast(float, (uint32_t)sw[1]);
      big |= !(t <= kSumMax);
    }
    rerun |= big;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        lsum[qb][kb] += tl[qb][kb];
        ltsum[qb][kb] += tlt[qb][kb];
      }
    lds_barrier();
  };
  // ---- one pass over the keys
  auto run_pass = [&]() __attribute__((always_inline)) {
    // ---- prologue: K_0, K_1 in LDS, V buffer 1 zeroed (iteration 0 multiplies
    // it by the zero probabilities pB), S_0 computed, K_2 and V_0 requested.
    if constexpr (AG) {
      for (int i = tid; i < BC * VSR / 8; i += NT) *(u32x4_t*)(&sV[1][8 * i]) = u32x4_t{0u, 0u, 0u, 0u};
    } else {
  #pragma unroll
      for (int i = 0; i < CW; ++i) *(u32x4_t*)(&sV[1][(tid + NT * i) * 8]) = u32x4_t{0u, 0u, 0u, 0u};
    }
    load_k(0);
    wait_vmem();  // Q fragments and K_0
    if (!exact) {
  #pragma unroll
      for (int qb = 0; qb < QB; ++qb)
  #pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          qf[qb][ks] = sign_flip(qf[qb][ks], g.qneg);
          PM::operand_wait(qf[qb][ks]);
        }
    }
  #pragma unroll
    for (int i = 0; i < NKC; ++i) store_part(i, 0);
    load_k(1);
    wait_vmem();
  #pragma unroll
    for (int i = 0; i < NKC; ++i) store_part(i, 1);
    lds_barrier();
    mma_pipeline<NQF, 3>([&](int i) { return kaddr(0, i); },
                         [&](int i, u32x4_t a) {
                           const int kb = i % NKB, ks = i / NKB;
  #pragma unroll
                           for (int qb = 0; qb < QB; ++qb) {
                             if (ks == 0) sA[qb][kb] = PM::mb0(a, qf[qb][ks]);
                             else PM::mb(sA[qb][kb], a, qf[qb][ks]);
                           }
                         },
                         [](int) {});
    load_k(2);
    load_v(0);
    if constexpr (NSET == 2) {
      load_k(3, 1);
      load_v(1, 1);
    }
    lds_barrier();  // every wave is done with K_0 before iteration 0 overwrites it

    // Tiles are processed in pairs (the two register sets), over an even number
    // of tiles: a padding tile past the last one is fully masked (its keys lie
    // past the end of the sequence or, causally, past every row of this
    // workgroup) and contributes nothing.  The leading tiles whose keys are all
    // visible to every row of this wavefront run without masking; the rest
    // (the causal diagonal, the ragged end) mask scores as they are read.
    const int n_iter = (n_tiles + 1) & ~1;
    int n_open = Nb / BC;
    if (CAUSAL) n_open = min(n_open, (qw + 1) / BC);
    n_open = __builtin_amdgcn_readfirstlane(min(n_open, n_tiles) & ~1);
    int j = 0;
    for (; j < n_open; j += 2) {
      iteration(std::integral_constant<int, 0>{}, std::false_type{}, j);
      iteration(std::integral_constant<int, 1>{}, std::false_type{}, j + 1);
    }
    for (; j < n_iter; j += 2) {
      iteration(std::integral_constant<int, 0>{}, std::true_type{}, j);
      iteration(std::integral_constant<int, 1>{}, std::true_type{}, j + 1);
    }

    // last tile (odd index): O += V^T P from register set B and V buffer 1
    if constexpr (AG) {
#pragma unroll
      for (int i = 0; i < NVF; ++i) {
        const u32x4_t a = vread(1, i);
        const int ss = i / NDB, db = i % NDB;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) PM::macc(acc[qb][db], a, pfrag(pB, qb, ss));
      }
    } else {
      mma_pipeline<NVF, 3>([&](int i) { return vaddr(1, i); },
                           [&](int i, u32x4_t a) {
                             const int ss = i / NDB, db = i % NDB;
    #pragma unroll
                             for (int qb = 0; qb < QB; ++qb) PM::macc(acc[qb][db], a, pfrag(pB, qb, ss));
                           },
                           [](int) {});
    }
  };

  // Did a row of this workgroup need a new reference maximum?  (Rare: only
  // when a row maximum grows by about log2(kSumMax / BC) or more after its
  // first tile.)  Then every wavefront computes its rows' exact maxima
  // directly from Q and K, and the pass is redone against them.
  __shared__ int s_rerun[NW];
  for (;;) {
    run_pass();
    if (exact) break;
    if (lane == 0) s_rerun[w] = __builtin_amdgcn_ballot_w64(rerun) != 0;
    lds_barrier();
    bool any = false;
#pragma unroll
    for (int i = 0; i < NW; ++i) any |= s_rerun[i] != 0;
    if (!any) break;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int row = qw + 32 * qb + l32;
      const int kend = CAUSAL ? min(Nb, qw + 32 * qb + 32) : Nb;
      float mx = -INFINITY;
      for (int k0 = 0; k0 < kend; k0 += 32) {
        const uint32_t ko = (uint32_t)(k0 + l32) * rsk + 16 * h;
        auto kpad = [&](int ks) -> uint32_t { return GL ? col_pad(32 * ks + 16 * h, DR, k_bytes) : 0u; };
        f32x16_t sc = PM::mb0(buf_load16(kres, ko + kpad(0)), qf[qb][0]);
#pragma unroll
        for (int ks = 1; ks < NKS; ++ks) PM::mb(sc, buf_load16(kres, ko + 32 * ks + kpad(ks)), qf[qb][ks]);
        mfma_wait_v(sc);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 8 * (r / 4) + 4 * h + (r % 4);
          if (!(key >= Nb || (CAUSAL && key > row))) mx = __builtin_elementwise_maximum(mx, sc[r]);
        }
      }
      mx = __builtin_elementwise_maximum(mx, swap_halves(mx));
      m_run[qb] = mx * c;
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[qb][db] = zero16();
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        lsum[qb][kb] = ltsum[qb][kb] = 0.0f;
        pB[qb][kb][0] = pB[qb][kb][1] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
    exact = true;
  }
  wait_acc();

  // epilogue: normalise once, store O and LSE
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float l = 0.0f, lt = 0.0f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      l += lsum[qb][kb];
      lt += ltsum[qb][kb];
    }
    l += swap_halves(l);
    lt += swap_halves(lt);
    const float inv = 1.0f / lt;
    const int qrow = qw + 32 * qb + l32;
    u32x2_t ov[NDB][4];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        ov[db][g] = u32x2_t{TR::pack2(acc[qb][db][4 * g + 0] * inv, acc[qb][db][4 * g + 1] * inv),
                            TR::pack2(acc[qb][db][4 * g + 2] * inv, acc[qb][db][4 * g + 3] * inv)};
    // O stored as whole rows through LDS: waves 0..NW/2-1 use the K buffers,
    // the others the V buffers (every wavefront is past its last LDS read:
    // barrier below, before the first write)
    static_assert(QB == 1 && (NW / 2) * kTileRowsBytes<D> <= (int)sizeof(sK) &&
                      (NW / 2) * kTileRowsBytes<D> <= (int)sizeof(sV), "rows fit the tile buffers");
    if (qb == 0) lds_barrier();
    store_tile_rows<D>((w < NW / 2 ? (char*)sK : (char*)sV) + (w % (NW / 2)) * kTileRowsBytes<D>, ov,
                       O + o_off + (size_t)(qw + 32 * qb) * os, min(32, Nb - (qw + 32 * qb)), lane, os,
                       GL ? DR / 8 : D / 8);
    if (qrow < Nb && h == 0) LSE[l_off + qrow] = (m_run[qb] + __log2f(l)) * kLn2;
  }
  }
}

// 16-bit forward, phase ping-pong (used for d = 64).  8 wavefronts, two per
// SIMD, each owning 32 query rows.
// Every wavefront alternates two phases per key tile j:
//   M-phase j: S_j = K_j Q^T  and  O += V_{j-1}^T P_{j-1}   (matrix cores)
//   V-phase j: online softmax of S_j -> P_j                (vector ALU)
// Waves 4..7 run one phase behind waves 0..3, so on every SIMD one wave is in
// its M-phase while the other is in its V-phase, and the two kinds of work
// overlap.  A workgroup barrier separates phases ("slots").
//
// Staging: waves 0..3 stage K tiles, waves 4..7 stage V tiles.  A wave issues
// the global loads of tile j+2 in its V-phase j (a few instructions) and writes
// that tile to LDS in its next M-phase, between matrix instructions, where the
// vector ALU is otherwise idle.  K is double-buffered, V triple-buffered (the
// trailing waves still read V_{j-1} while V_{j+1} is written).
//
// LDS layouts (per buffer):
//   K: row-major, rows padded to D + 8 elements, so 16 consecutive rows read
//      at one 16-byte column fall in distinct banks and every fragment address
//      is a fixed offset from one base.
//   V: [key/16][h][d][8]: the 16-byte unit (s, h, c) holds column c of keys
//      16s + 4h + {0,1,2,3} and 16s + 8 + 4h + {0,1,2,3}, exactly the eight
//      values lane (c % 32, h) needs for one O^T += V^T P^T instruction.
//      Column c sits at slot c ^ ((c >> 3) & 3) of its row (bank-conflict-
//      free staging writes and fragment reads).
template <class TR, int D, int BC, bool CAUSAL, bool GL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd16_pp_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                  const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                  float* __restrict__ LSE, int N, int n_qtiles, uint32_t total, float c, GenLayout g) {
  constexpr int NW = 8;                     // wavefronts per workgroup
  constexpr int BR = 32 * NW;               // query rows per workgroup
  constexpr int KCH = D / 8;                // 16-byte chunks per row
  constexpr int KS = D + 8;                 // padded K row (elements)
  constexpr int NKB = BC / 32;              // 32-key blocks per tile
  constexpr int NDB = D / 32;               // 32-column blocks of the output
  constexpr int NKS = D / 16;               // MFMA k-steps over d
  constexpr int NQK = NKS * NKB;            // S MFMAs per tile
  constexpr int NPV = NKB * 2 * NDB;        // O MFMAs per tile
  static_assert(BC * KCH == 1024 && (BC / 16) * 2 * (D / 4) == 256,
                "one K chunk set and one V unit per staging thread");
  static_assert(NQK == NPV, "matrix phase interleaves the two products one to one");

  __shared__ __attribute__((aligned(16))) uint16_t sK[2][BC * KS];
  __shared__ __attribute__((aligned(16))) uint16_t sV[3][BC * D];

  // one tile: the whole pass from the first load to the last store
  auto run_tile = [&](const uint32_t lid) __attribute__((always_inline)) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int grp = w >> 2;          // 0: leading group (stages K), 1: trailing group (stages V)
  const int st = tid & 255;        // staging index within the group
  const int h = lane >> 5;
  const int l32 = lane & 31;

  const int bh = lid / n_qtiles;
  int qt = lid % n_qtiles;
  if (CAUSAL) qt = n_qtiles - 1 - qt;  // heaviest tiles first
  const int q0 = qt * BR;
  constexpr uint32_t RB = D * 2;   // bytes per row
  // Addressing: dense [BH, N, D], or (GL) the general layout (per-tensor
  // strides, a packed self-attention batch with tiles wholly past the
  // sequence skipped, DR < D data columns), as in fwd16_pipe_kernel.
  int Nb = N, DR = D;
  size_t q_off, k_off, v_off, o_off, l_off, os;
  uint32_t q_bytes, k_bytes, v_bytes, rsq, rsk, rsv;
  if constexpr (GL) {
    const int b = bh / g.H, hd = bh - b * g.H;
    int sq, sk, nq, nk;
    seq_rows(g.cu_q, g.total_q, b, N, sq, nq);
    seq_rows(g.cu_k, g.total_k, b, N, sk, nk);
    Nb = min(nq, nk);
    DR = g.dr;
    const TRows tq = tensor_rows(g.q, b, hd, sq, Nb, DR), tk = tensor_rows(g.k, b, hd, sk, Nb, DR);
    const TRows tv = tensor_rows(g.v, b, hd, sk, Nb, DR), to = tensor_rows(g.o, b, hd, sq, Nb, DR);
    q_off = tq.off, k_off = tk.off, v_off = tv.off, o_off = to.off;
    q_bytes = tq.bytes, k_bytes = tk.bytes, v_bytes = tv.bytes;
    rsq = tq.rs, rsk = tk.rs, rsv = tv.rs;
    os = (size_t)g.o.sr;
    l_off = (size_t)((int64_t)b * g.l_sb + (int64_t)hd * g.l_sh + sq);
  } else {
    q_off = k_off = v_off = o_off = (size_t)bh * N * D;
    q_bytes = k_bytes = v_bytes = (uint32_t)N * RB;
    rsq = rsk = rsv = RB;
    os = D;
    l_off = (size_t)bh * N;
  }
  if (GL && q0 >= Nb) return;
  const int qw = q0 + 32 * w;      // first query row of this wavefront
  const int qrow = qw + l32;

  // Q rows as the B operand of S^T = K Q^T, loaded once (rows past the end
  // read zeros; their results are never stored); signs flipped for a negative
  // scale (the products here are compiler builtins, which keep the wait
  // states after that vector write themselves).
  u32x4_t qf[NKS];
  {
    const rsrc_t qres = make_rsrc(Q + q_off, q_bytes);
    const uint32_t qoff = (uint32_t)qrow * rsq + 16 * h;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      qf[ks] = sign_flip(buf_load16(qres, qoff + 32 * ks + (GL ? col_pad(32 * ks + 16 * h, DR, q_bytes) : 0u)),
                         g.qneg);
  }

  f32x16_t acc_o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc_o[db] = zero16();
  f32x16_t s[NKB];
  uint32_t pt[NKB][8];
  float m_run = -INFINITY, l_run = 0.0f, lt_run = 0.0f;

  const int kv_end = CAUSAL ? min(Nb, q0 + BR) : Nb;
  const int n_tiles = (kv_end + BC - 1) / BC;
  const int wave_end = CAUSAL ? min(Nb, qw + 32) : Nb;
  const int wave_tiles = (wave_end + BC - 1) / BC;

  // ---- staging: 4 x 16 bytes per thread in both roles.  Rows past the end of
  // the sequence read zeros (their scores are masked to -inf, so they add 0).
  // One resource per tensor: each is uniform across the wave (SGPRs); a
  // resource selected by the (per-lane) group index would not be.
  const rsrc_t kres = make_rsrc(K + k_off, k_bytes);
  const rsrc_t vres = make_rsrc(V + v_off, v_bytes);
  u32x4_t stg[4];
  // K role: chunk ci = st + 256 r -> row ci / KCH, 16-byte column ci % KCH
  const uint32_t koff = (uint32_t)(st / KCH) * rsk + (st % KCH) * 16 +
                        (GL ? col_pad((st % KCH) * 16, DR, k_bytes) : 0u);
  const int kst = (st / KCH) * KS + (st % KCH) * 8;
  // V role: unit st -> (16-key step vs, half vh, 4-column chunk vc); 8 rows x 8 bytes
  const int vc = st % (D / 4);
  const int vh = (st / (D / 4)) & 1;
  const int vs = st / (D / 2);
  const uint32_t voff = (uint32_t)(16 * vs + 4 * vh) * rsv + vc * 8 + (GL ? col_pad(vc * 8, DR, v_bytes) : 0u);
  const int vst = ((2 * vs + vh) * D + 4 * vc) * 8;
  const int vsw = (vc >> 1) & 3;  // slot swizzle of this thread's four columns

  auto load_tile = [&](int j0) {
    if (grp == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) stg[r] = buf_load16(kres, koff + (uint32_t)(j0 + (256 / KCH) * r) * rsk);
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const u32x2_t x = buf_load8(vres, voff + (uint32_t)(j0 + 8 * (k / 4) + (k % 4)) * rsv);
        stg[k / 2][2 * (k % 2) + 0] = x[0];
        stg[k / 2][2 * (k % 2) + 1] = x[1];
      }
    }
  };
  auto store_k = [&](int buf) {
#pragma unroll
    for (int r = 0; r < 4; ++r) *(u32x4_t*)(&sK[buf][kst + r * (256 / KCH) * KS]) = stg[r];
  };
  auto store_v = [&](int buf) {
    // stg[kp] = {row 2kp cols (0,1), row 2kp cols (2,3), row 2kp+1 cols (0,1), row 2kp+1 cols (2,3)}
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      uint32_t o[4];
#pragma unroll
      for (int kp = 0; kp < 4; ++kp) {
        const uint32_t a = stg[kp][cc / 2], b = stg[kp][2 + cc / 2];
        o[kp] = (cc & 1) ? pack_hi(a, b) : pack_lo(a, b);
      }
      *(u32x4_t*)(&sV[buf][vst + 8 * (cc ^ vsw)]) = u32x4_t{o[0], o[1], o[2], o[3]};
    }
  };
  auto store_tile = [&](int j) {  // tile j into its buffer
    if (grp == 0) store_k(j & 1);
    else store_v(j % 3);
  };

  // ---- matrix products
  const int kfrag = l32 * KS + 8 * h;  // element offset of this lane's K fragment
  const int vfrag = (h * D + (l32 ^ ((l32 >> 3) & 3))) * 8;  // this lane's V fragment
  auto qk_step = [&](const uint16_t* kb_, int i) {  // i-th of NQK: ks = i / NKB, kb = i % NKB
    const int ks = i / NKB, kb = i % NKB;
    const u32x4_t kf = *(const u32x4_t*)(kb_ + 32 * kb * KS + 16 * ks);
    // the first k-step starts from a zero accumulator (inline constant: no
    // vector instructions to clear the score registers)
    s[kb] = TR::mfma(kf, qf[ks], ks == 0 ? zero16() : s[kb]);
  };
  auto pv_step = [&](const uint16_t* vb_, int i) {  // i-th of NPV: (kb, t) = i / NDB, db = i % NDB
    const int kt = i / NDB, db = i % NDB;
    const int kb = kt / 2, t = kt % 2;
    const u32x4_t pf = u32x4_t{pt[kb][4 * t + 0], pt[kb][4 * t + 1], pt[kb][4 * t + 2], pt[kb][4 * t + 3]};
    const u32x4_t vf = *(const u32x4_t*)(vb_ + ((2 * kt) * D + 32 * db) * 8);
    acc_o[db] = TR::mfma(vf, pf, acc_o[db]);
  };

  // ---- prologue: tile 0 in LDS, tile 1 requested
  load_tile(0);
  if (grp == 0) store_k(0);
  else store_v(0);
  wait_vmem();  // Q fragments and tile 0 resident before the loop
  if (n_tiles > 1) load_tile(BC);
  lds_barrier();

  const int n_slots = 2 * n_tiles + 2;
  for (int slot = 0; slot < n_slots; ++slot) {
    const int ph = slot - grp;  // this wave's own phase counter
    if (ph >= 0 && (ph & 1) == 0) {
      // ---------------- M-phase j: write tile j+1, S_j = K_j Q^T, O += V_{j-1}^T P_{j-1}
      __builtin_amdgcn_s_setprio(1);
      const int j = ph >> 1;
      const bool stage = j + 1 < n_tiles;
      const bool do_qk = j < wave_tiles;
      const bool do_pv = j >= 1 && j - 1 < wave_tiles;
      const uint16_t* kb_ = sK[j & 1] + kfrag;
      const uint16_t* vb_ = sV[(j + 2) % 3] + vfrag;  // V_{j-1}
      if (do_qk && do_pv) {
        // Steady state, written as an explicit software pipeline: the products
        // alternate S and O steps, each operand is read from LDS kAhead steps
        // before its product, and the staging writes (with the V packing) sit
        // between products.  sched_barrier keeps the compiler from regrouping
        // the reads next to their uses.  The staging write is unconditional:
        // past the last tile it rewrites a buffer no product reads again.
        constexpr int NST = NQK + NPV;  // steps: even = S (QK), odd = O (PV)
        constexpr int kAhead = 4;
        auto frag_addr = [&](int step) -> const uint16_t* {
          const int i = step >> 1;
          if (step & 1) {
            const int kt = i / NDB, db = i % NDB;
            return vb_ + ((2 * kt) * D + 32 * db) * 8;
          }
          const int ks = i / NKB, kb = i % NKB;
          return kb_ + 32 * kb * KS + 16 * ks;
        };
        auto fused = [&](auto role) {
          constexpr int R = decltype(role)::value;
          u32x4_t fr[kAhead];
#pragma unroll
          for (int x = 0; x < kAhead; ++x) fr[x] = *(const u32x4_t*)frag_addr(x);
#pragma unroll
          for (int stp = 0; stp < NST; ++stp) {
            const u32x4_t a = fr[stp % kAhead];
            if (stp + kAhead < NST) fr[stp % kAhead] = *(const u32x4_t*)frag_addr(stp + kAhead);
            const int i = stp >> 1;
            if (stp & 1) {
              const int kt = i / NDB, db = i % NDB;
              const int kb = kt / 2, t = kt % 2;
              const u32x4_t pf = u32x4_t{pt[kb][4 * t + 0], pt[kb][4 * t + 1], pt[kb][4 * t + 2],
                                         pt[kb][4 * t + 3]};
              acc_o[db] = TR::mfma(a, pf, acc_o[db]);
            } else {
              const int ks = i / NKB, kb = i % NKB;
              s[kb] = TR::mfma(a, qf[ks], ks == 0 ? zero16() : s[kb]);
            }
            // staging: one 16-byte LDS write every 8 steps
            if (stp % 8 == 3) {
              const int cc = stp / 8;
              if constexpr (R == 0) {
                *(u32x4_t*)(&sK[(j + 1) & 1][kst + cc * (256 / KCH) * KS]) = stg[cc];
              } else {
                uint32_t o[4];
#pragma unroll
                for (int kp = 0; kp < 4; ++kp) {
                  const uint32_t x0 = stg[kp][cc / 2], x1 = stg[kp][2 + cc / 2];
                  o[kp] = (cc & 1) ? pack_hi(x0, x1) : pack_lo(x0, x1);
                }
                *(u32x4_t*)(&sV[(j + 1) % 3][vst + 8 * (cc ^ vsw)]) = u32x4_t{o[0], o[1], o[2], o[3]};
              }
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        };
        if (grp == 0) fused(std::integral_constant<int, 0>{});
        else fused(std::integral_constant<int, 1>{});
      } else {
        if (stage) store_tile(j + 1);
        if (do_qk) {
#pragma unroll
          for (int i = 0; i < NQK; ++i) qk_step(kb_, i);
        }
        if (do_pv) {
#pragma unroll
          for (int i = 0; i < NPV; ++i) pv_step(vb_, i);
        }
      }
      __builtin_amdgcn_s_setprio(0);
    } else if (ph >= 0) {
      // ---------------- V-phase j: request tile j+2, softmax of S_j
      const int j = (ph - 1) >> 1;
      if (j + 2 < n_tiles) load_tile((j + 2) * BC);
      if (j < wave_tiles) {
        const int j0 = j * BC;
        if (wave_uniform((CAUSAL && j0 + BC - 1 > qw) || j0 + BC > Nb)) {
          // key j0 + 4h + off is hidden iff off >= lim (one compare per score)
          const int lim = (CAUSAL ? min(Nb, qrow + 1) : Nb) - j0 - 4 * h;
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (32 * kb + 8 * (r / 4) + (r % 4) >= lim) s[kb][r] = -INFINITY;
        }
        // probabilities against the reference maximum m_run
        float lsum, ltsum;
        auto softmax = [&]() __attribute__((always_inline)) {
          const float mneg = -m_run;
          lsum = 0.0f;
          ltsum = 0.0f;
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
              const float p0 = fast_exp2(fmaf(s[kb][r], c, mneg));
              const float p1 = fast_exp2(fmaf(s[kb][r + 1], c, mneg));
              lsum += p0 + p1;
              const uint32_t pk = TR::pack2(p0, p1);
              ltsum = TR::sum2(pk, ltsum);
              pt[kb][r / 2] = pk;
            }
        };
        // The reference is the first tile's row maximum and is raised only
        // when a tile's row sum exceeds kSumMax (a maximum grew by about
        // log2(kSumMax / BC) or more): then, for this tile, the row maxima are
        // searched, O and the sums re-based and the probabilities recomputed.
        bool rebase = j == 0;
        if (!rebase) {
          softmax();
          rebase = wave_uniform(__builtin_amdgcn_ballot_w64(!(lsum + swap_halves(lsum) <= kSumMax)) != 0);
        }
        if (rebase) {
          float mx = -INFINITY;
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; r += 2) mx = max3f(mx, s[kb][r], s[kb][r + 1]);
          const float mnew = __builtin_elementwise_maximum(m_run, __builtin_elementwise_maximum(mx, swap_halves(mx)) * c);
          const float alpha = fast_exp2(m_run - mnew);  // 0 on the first tile
          m_run = mnew;
          l_run *= alpha;
          lt_run *= alpha;
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc_o[db][r] *= alpha;
          softmax();
        }
        l_run += lsum;
        lt_run += ltsum;
      }
    }
    lds_barrier();
  }

  // epilogue: normalise once, store O and LSE
  const float lt = lt_run + swap_halves(lt_run);
  const float l = l_run + swap_halves(l_run);
  const float inv = 1.0f / lt;
  u32x2_t ov[NDB][4];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      ov[db][g] = u32x2_t{TR::pack2(acc_o[db][4 * g + 0] * inv, acc_o[db][4 * g + 1] * inv),
                          TR::pack2(acc_o[db][4 * g + 2] * inv, acc_o[db][4 * g + 3] * inv)};
  // O stored as whole rows through LDS (the K buffers; the loop ended with a barrier)
  static_assert(8 * kTileRowsBytes<D> <= (int)sizeof(sK), "rows of all wavefronts fit the K buffers");
  store_tile_rows<D>((char*)sK + w * kTileRowsBytes<D>, ov, O + o_off + (size_t)qw * os, min(32, Nb - qw), lane, os,
                     GL ? DR / 8 : D / 8);
  if (qrow < Nb && h == 0) LSE[l_off + qrow] = (m_run + __log2f(l)) * kLn2;
  };
  for_each_tile(total, (uint32_t)n_qtiles, run_tile);
}

// fp32 inputs: same scheme with v_mfma_f32_32x32x2_f32 and unrounded fp32
// probabilities; one block of 32 query rows per wavefront, 32-key tiles.
// qsign = -1 for a negative scale (the query rows negated, c = |scale| log2 e).
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void fwd32_kernel(const float* __restrict__ Q,
                                                    const float* __restrict__ K,
                                                    const float* __restrict__ V,
                                                    float* __restrict__ O, float* __restrict__ LSE,
                                                    int N, int n_qtiles, uint32_t total, float c,
                                                    float qsign) {
  constexpr int BC = 32;
  constexpr int BR = 128;
  constexpr int KP = D + 1;  // padded K row (conflict-free column reads)
  constexpr int NDB = D / 32;
  __shared__ float sK[BC * KP];
  __shared__ __attribute__((aligned(16))) float sV[BC * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int h = lane >> 5;
  const int l32 = lane & 31;

  const uint32_t lid = xcd_remap(blockIdx.x, total);
  const int bh = lid / n_qtiles;
  int qt = lid % n_qtiles;
  if (CAUSAL) qt = n_qtiles - 1 - qt;
  const int q0 = qt * BR;
  const size_t head_off = (size_t)bh * N * D;
  const int qw = q0 + 32 * w;
  const int qrow = qw + l32;

  float qf[D / 2];
#pragma unroll
  for (int ks = 0; ks < D / 2; ++ks)
    qf[ks] = (qrow < N) ? qsign * Q[head_off + (size_t)qrow * D + 2 * ks + h] : 0.0f;

  f32x16_t acc_o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc_o[db] = zero16();
  float m_run = -INFINITY, l_run = 0.0f;

  const int kv_end = CAUSAL ? min(N, q0 + BR) : N;
  const int n_tiles = (kv_end + BC - 1) / BC;
  const int wave_last = CAUSAL ? min(N, qw + 32) : N;
  const int wave_tiles = (wave_last + BC - 1) / BC;

  // staging: 16-byte chunks x = tid + 256 i of the tile (row x / (D / 4),
  // columns 4 (x % (D / 4)) + 0..3), loaded one tile ahead into registers so
  // the next tile's loads are in flight while this one is computed; rows past
  // the end are zeros
  constexpr int NST = BC * D / 4 / 256;
  float4 kst[NST], vst[NST];
  auto load_tile = [&](int j0) {
#pragma unroll
    for (int i = 0; i < NST; ++i) {
      const int x = tid + 256 * i, row = x / (D / 4), col = 4 * (x % (D / 4));
      const bool ok = j0 + row < N;
      const size_t off = head_off + (size_t)(j0 + row) * D + col;
      kst[i] = ok ? *(const float4*)(K + off) : float4{0.0f, 0.0f, 0.0f, 0.0f};
      vst[i] = ok ? *(const float4*)(V + off) : float4{0.0f, 0.0f, 0.0f, 0.0f};
    }
  };
  load_tile(0);
  for (int jt = 0; jt < n_tiles; ++jt) {
    const int j0 = jt * BC;
    __syncthreads();  // every wave is done with the previous tile
#pragma unroll
    for (int i = 0; i < NST; ++i) {
      const int x = tid + 256 * i, row = x / (D / 4), col = 4 * (x % (D / 4));
      float* kd = sK + row * KP + col;  // padded rows: not 16-byte aligned
      kd[0] = kst[i].x;
      kd[1] = kst[i].y;
      kd[2] = kst[i].z;
      kd[3] = kst[i].w;
      *(float4*)(sV + row * D + col) = vst[i];
    }
    if (jt + 1 < n_tiles) load_tile(j0 + BC);
    __syncthreads();
    if (jt >= wave_tiles) continue;

    f32x16_t s = zero16();
#pragma unroll
    for (int ks = 0; ks < D / 2; ++ks) s = mfma_f32(sK[l32 * KP + 2 * ks + h], qf[ks], s);

#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = j0 + 8 * (r / 4) + 4 * h + (r % 4);
      if (key >= N || (CAUSAL && key > qrow)) s[r] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = fmaxf(mx, swap_halves(mx));
    const float mnew = fmaxf(m_run, mx * c);
    const float alpha = fast_exp2(m_run - mnew);
    m_run = mnew;
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_o[db][r] *= alpha;
    float p[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      p[r] = fast_exp2(fmaf(s[r], c, -mnew));
      l_run += p[r];
    }
    // O^T += V^T P^T: k-step r pairs key 8(r/4)+(r%4) (h = 0) with key 8(r/4)+4+(r%4) (h = 1)
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 8 * (r / 4) + 4 * h + (r % 4);
        acc_o[db] = mfma_f32(sV[key * D + 32 * db + l32], p[r], acc_o[db]);
      }
  }

  const float l = l_run + swap_halves(l_run);
  const float inv = 1.0f / l;
  if (qrow < N) {
    float* orow = O + head_off + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) orow[32 * db + 8 * (r / 4) + 4 * h + (r % 4)] = acc_o[db][r] * inv;
    if (h == 0) LSE[(size_t)bh * N + qrow] = (m_run + __log2f(l)) * kLn2;
  }
}

// ------------------------------------------------------------------ launch

// d = 128 (and d = 96 in the general layout): 256 rows and 64-key tiles per
// workgroup of 8 wavefronts; d = 256: 128 rows and 32-key tiles per workgroup
// of 4 (one wavefront per SIMD).
template <class TR, int D, bool CAUSAL, bool GL>
static void launch_pipe_gl(const FwdArgs& a) {
  constexpr int BR = D > 128 ? 128 : 256;
  constexpr int BC = D > 128 ? 32 : 64;
  const int n_qtiles = (a.N + BR - 1) / BR;
  const uint32_t total = (uint32_t)((D > 128 ? (n_qtiles + 1) / 2 : n_qtiles) * a.BH);  // workgroups
  hipLaunchKernelGGL((fwd16_pipe_kernel<TR, D, BC, 1, CAUSAL, GL>), dim3(total), dim3(D > 128 ? 256 : 512), 0,
                     a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                     (uint16_t*)a.o, a.lse, a.N, n_qtiles, total, a.c, a.g);
}

template <class TR, bool CAUSAL, bool GL>
static void launch_pp_gl(const FwdArgs& a) {  // d = 64 (and d = 32 in the general layout)
  constexpr int BR = 256;
  const int n_qtiles = (a.N + BR - 1) / BR;
  const uint32_t total = (uint32_t)(n_qtiles * a.BH);
  // persistent: one resident workgroup per compute unit (86 KB of LDS)
  const uint32_t grid = persistent_grid(a.BH, n_qtiles, 1, a.stream);
  hipLaunchKernelGGL((fwd16_pp_kernel<TR, 64, 128, CAUSAL, GL>), dim3(grid), dim3(512), 0, a.stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                     (uint16_t*)a.o, a.lse, a.N, n_qtiles, total, a.c, a.g);
}

template <class TR, bool CAUSAL>
static hipError_t launch_pipe(const FwdArgs& a) {
  if (a.d > 128) {
    if (a.general) launch_pipe_gl<TR, 256, CAUSAL, true>(a);
    else launch_pipe_gl<TR, 256, CAUSAL, false>(a);
  } else {
    if (a.general) launch_pipe_gl<TR, 128, CAUSAL, true>(a);
    else launch_pipe_gl<TR, 128, CAUSAL, false>(a);
  }
  return hipGetLastError();
}

template <class TR, bool CAUSAL>
static hipError_t launch_pp(const FwdArgs& a) {
  if (a.general) launch_pp_gl<TR, CAUSAL, true>(a);
  else launch_pp_gl<TR, CAUSAL, false>(a);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
static hipError_t launch32(const FwdArgs& a) {
  const int n_qtiles = (a.N + 127) / 128;
  const uint32_t total = (uint32_t)(n_qtiles * a.BH);
  hipLaunchKernelGGL((fwd32_kernel<D, CAUSAL>), dim3(total), dim3(256), 0, a.stream,
                     (const float*)a.q, (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse,
                     a.N, n_qtiles, total, a.c, a.g.qneg ? -1.0f : 1.0f);
  return hipGetLastError();
}

template <class TR>
static hipError_t dispatch16(const FwdArgs& a) {
  // the kernel's width: d = 256 and 128 (and 96: general layout, zero
  // columns) on the pipelined kernel, d = 64 and 32 on the d = 64 kernel
  if (a.d > 64) return a.causal ? launch_pipe<TR, true>(a) : launch_pipe<TR, false>(a);
  return a.causal ? launch_pp<TR, true>(a) : launch_pp<TR, false>(a);
}

hipError_t launch_fwd(const FwdArgs& a) {
  if (a.general && a.dtype != DT_BF16 && a.dtype != DT_F16) return hipErrorInvalidValue;  // 16-bit only
  switch (a.dtype) {
    case DT_BF16: return dispatch16<BF16>(a);
    case DT_F16: return dispatch16<F16>(a);
    default:
      if (a.d == 128) return a.causal ? launch32<128, true>(a) : launch32<128, false>(a);
      return a.causal ? launch32<64, true>(a) : launch32<64, false>(a);
  }
}

}  // namespace fa
