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
//   * workgroup = 4 wavefronts x QB blocks of 32 query rows; grid = query
//     tiles x (batch * heads), XCD-grouped, heaviest causal tiles first.
//   * each wavefront computes S^T = K Q^T with v_mfma_f32_32x32x16: the
//     accumulator then holds, per lane, one query row (lane % 32) and 16 keys,
//     so row max / row sum are in-lane plus one exchange between half-waves,
//     and the probabilities are already in the B-operand layout of
//     O^T += V^T P^T (they never leave registers).
//   * K and V tiles of 64 keys are staged HBM -> registers -> LDS with 16-byte
//     coalesced loads, double buffered (the next tile is in flight while the
//     current one is consumed).  K is stored row-major with an XOR swizzle of
//     its 16-byte chunks; V is stored as groups of 4 keys per column
//     ([key/4][d][4]) so the V^T operand is two 8-byte LDS reads per lane.
//   * softmax in the exp2 domain with scale*log2(e) folded into one FMA; the
//     output is rescaled only when a row maximum grows by more than kTau (in
//     log2 units), and normalised once at the end (deferred rescaling).
//   * causal: key tiles above the diagonal are never loaded or multiplied;
//     only tiles crossing the diagonal are masked.
#include <type_traits>

#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {

// A row maximum is only re-based when it grows by more than kTau (log2 units).
// Between re-bases probabilities are bounded by 2^kTau, which bf16/fp16 and
// the fp32 accumulators hold without loss of relative precision; the final
// normalisation uses the same reference maximum for numerator and
// denominator, so the result is unchanged mathematically.
constexpr float kTau = 8.0f;

// 16-bit forward.  8 wavefronts, two per SIMD, each owning 32 query rows.
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
template <class TR, int D, int BC, bool CAUSAL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd16_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                  const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                  float* __restrict__ LSE, int N, int n_qtiles, uint32_t total, float c) {
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

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int grp = w >> 2;          // 0: leading group (stages K), 1: trailing group (stages V)
  const int st = tid & 255;        // staging index within the group
  const int h = lane >> 5;
  const int l32 = lane & 31;

  const uint32_t lid = xcd_remap(blockIdx.x, total);
  const int bh = lid / n_qtiles;
  int qt = lid % n_qtiles;
  if (CAUSAL) qt = n_qtiles - 1 - qt;  // heaviest tiles first
  const int q0 = qt * BR;
  const size_t head_off = (size_t)bh * N * D;
  constexpr uint32_t RB = D * 2;   // bytes per row
  const uint32_t head_bytes = (uint32_t)N * RB;
  const int qw = q0 + 32 * w;      // first query row of this wavefront
  const int qrow = qw + l32;

  // Q rows as the B operand of S^T = K Q^T, loaded once (rows past the end
  // read zeros; their results are never stored).
  u32x4_t qf[NKS];
  {
    const rsrc_t qres = make_rsrc(Q + head_off, head_bytes);
    const uint32_t qoff = (uint32_t)qrow * RB + 16 * h;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[ks] = buf_load16(qres, qoff + 32 * ks);
  }

  f32x16_t acc_o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc_o[db] = zero16();
  f32x16_t s[NKB];
  uint32_t pt[NKB][8];
  float m_run = -INFINITY, l_run = 0.0f, lt_run = 0.0f;

  const int kv_end = CAUSAL ? min(N, q0 + BR) : N;
  const int n_tiles = (kv_end + BC - 1) / BC;
  const int wave_end = CAUSAL ? min(N, qw + 32) : N;
  const int wave_tiles = (wave_end + BC - 1) / BC;

  // ---- staging: 4 x 16 bytes per thread in both roles.  Rows past the end of
  // the sequence read zeros (their scores are masked to -inf, so they add 0).
  // One resource per tensor: each is uniform across the wave (SGPRs); a
  // resource selected by the (per-lane) group index would not be.
  const rsrc_t kres = make_rsrc(K + head_off, head_bytes);
  const rsrc_t vres = make_rsrc(V + head_off, head_bytes);
  u32x4_t stg[4];
  // K role: chunk ci = st + 256 r -> row ci / KCH, 16-byte column ci % KCH
  const uint32_t koff = (uint32_t)(st / KCH) * RB + (st % KCH) * 16;
  const int kst = (st / KCH) * KS + (st % KCH) * 8;
  // V role: unit st -> (16-key step vs, half vh, 4-column chunk vc); 8 rows x 8 bytes
  const int vc = st % (D / 4);
  const int vh = (st / (D / 4)) & 1;
  const int vs = st / (D / 2);
  const uint32_t voff = (uint32_t)(16 * vs + 4 * vh) * RB + vc * 8;
  const int vst = ((2 * vs + vh) * D + 4 * vc) * 8;

  auto load_tile = [&](int j0) {
    if (grp == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) stg[r] = buf_load16(kres, koff + (uint32_t)(j0 + (256 / KCH) * r) * RB);
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const u32x2_t x = buf_load8(vres, voff + (uint32_t)(j0 + 8 * (k / 4) + (k % 4)) * RB);
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
      *(u32x4_t*)(&sV[buf][vst + 8 * cc]) = u32x4_t{o[0], o[1], o[2], o[3]};
    }
  };
  auto store_tile = [&](int j) {  // tile j into its buffer
    if (grp == 0) store_k(j & 1);
    else store_v(j % 3);
  };

  // ---- matrix products
  const int kfrag = l32 * KS + 8 * h;  // element offset of this lane's K fragment
  const int vfrag = (h * D + l32) * 8;  // element offset of this lane's V fragment
  auto qk_step = [&](const uint16_t* kb_, int i) {  // i-th of NQK: ks = i / NKB, kb = i % NKB
    const int ks = i / NKB, kb = i % NKB;
    const u32x4_t kf = *(const u32x4_t*)(kb_ + 32 * kb * KS + 16 * ks);
    s[kb] = TR::mfma(kf, qf[ks], s[kb]);
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
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) s[kb] = zero16();
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
              s[kb] = TR::mfma(a, qf[ks], s[kb]);
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
                *(u32x4_t*)(&sV[(j + 1) % 3][vst + 8 * cc]) = u32x4_t{o[0], o[1], o[2], o[3]};
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
        if (wave_uniform((CAUSAL && j0 + BC - 1 > qw) || j0 + BC > N)) {
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = j0 + 32 * kb + 8 * (r / 4) + 4 * h + (r % 4);
              if (key >= N || (CAUSAL && key > qrow)) s[kb][r] = -INFINITY;
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
        mx = fmaxf(mx, swap_halves(mx));
        const float mnew = mx * c;
        if (mnew > m_run + kTau) {
          const float alpha = fast_exp2(m_run - mnew);
          m_run = mnew;
          l_run *= alpha;
          lt_run *= alpha;
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc_o[db][r] *= alpha;
        }
        const float mneg = -m_run;
        float lsum = 0.0f, ltsum = 0.0f;
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
  if (qrow < N) {
    uint16_t* orow = O + head_off + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = 32 * db + 8 * g + 4 * h;
        const uint32_t w0 = TR::pack2(acc_o[db][4 * g + 0] * inv, acc_o[db][4 * g + 1] * inv);
        const uint32_t w1 = TR::pack2(acc_o[db][4 * g + 2] * inv, acc_o[db][4 * g + 3] * inv);
        *(u32x2_t*)(orow + col) = u32x2_t{w0, w1};
      }
    if (h == 0) LSE[(size_t)bh * N + qrow] = (m_run + __log2f(l)) * kLn2;
  }
}

// fp32 inputs: same scheme with v_mfma_f32_32x32x2_f32 and unrounded fp32
// probabilities; one block of 32 query rows per wavefront, 32-key tiles.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void fwd32_kernel(const float* __restrict__ Q,
                                                    const float* __restrict__ K,
                                                    const float* __restrict__ V,
                                                    float* __restrict__ O, float* __restrict__ LSE,
                                                    int N, int n_qtiles, uint32_t total, float c) {
  constexpr int BC = 32;
  constexpr int BR = 128;
  constexpr int KP = D + 1;  // padded K row (conflict-free column reads)
  constexpr int NDB = D / 32;
  __shared__ float sK[BC * KP];
  __shared__ float sV[BC * D];

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
    qf[ks] = (qrow < N) ? Q[head_off + (size_t)qrow * D + 2 * ks + h] : 0.0f;

  f32x16_t acc_o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc_o[db] = zero16();
  float m_run = -INFINITY, l_run = 0.0f;

  const int kv_end = CAUSAL ? min(N, q0 + BR) : N;
  const int n_tiles = (kv_end + BC - 1) / BC;
  const int wave_last = CAUSAL ? min(N, qw + 32) : N;
  const int wave_tiles = (wave_last + BC - 1) / BC;

  for (int jt = 0; jt < n_tiles; ++jt) {
    const int j0 = jt * BC;
    __syncthreads();
    for (int x = tid; x < BC * D; x += 256) {
      const int row = x / D, col = x % D;
      const bool ok = j0 + row < N;
      sK[row * KP + col] = ok ? K[head_off + (size_t)(j0 + row) * D + col] : 0.0f;
      sV[row * D + col] = ok ? V[head_off + (size_t)(j0 + row) * D + col] : 0.0f;
    }
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

template <class TR, int D, int BC, bool CAUSAL>
static hipError_t launch16(const FwdArgs& a) {
  constexpr int BR = 256;
  const int n_qtiles = (a.N + BR - 1) / BR;
  const uint32_t total = (uint32_t)(n_qtiles * a.BH);
  hipLaunchKernelGGL((fwd16_kernel<TR, D, BC, CAUSAL>), dim3(total), dim3(512), 0, a.stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                     (uint16_t*)a.o, a.lse, a.N, n_qtiles, total, a.c);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
static hipError_t launch32(const FwdArgs& a) {
  const int n_qtiles = (a.N + 127) / 128;
  const uint32_t total = (uint32_t)(n_qtiles * a.BH);
  hipLaunchKernelGGL((fwd32_kernel<D, CAUSAL>), dim3(total), dim3(256), 0, a.stream,
                     (const float*)a.q, (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse,
                     a.N, n_qtiles, total, a.c);
  return hipGetLastError();
}

template <class TR>
static hipError_t dispatch16(const FwdArgs& a) {
  if (a.d == 128) return a.causal ? launch16<TR, 128, 64, true>(a) : launch16<TR, 128, 64, false>(a);
  return a.causal ? launch16<TR, 64, 128, true>(a) : launch16<TR, 64, 128, false>(a);
}

hipError_t launch_fwd(const FwdArgs& a) {
  switch (a.dtype) {
    case DT_BF16: return dispatch16<BF16>(a);
    case DT_F16: return dispatch16<F16>(a);
    default:
      if (a.d == 128) return a.causal ? launch32<128, true>(a) : launch32<128, false>(a);
      return a.causal ? launch32<64, true>(a) : launch32<64, false>(a);
  }
}

}  // namespace fa
