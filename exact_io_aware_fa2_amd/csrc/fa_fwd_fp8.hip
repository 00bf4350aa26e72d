// Forward attention with 8-bit (OCP E4M3) Q, K and V for gfx950: the scores
// S = Q K^T are products of 8-bit operands on the FP8 matrix cores
// (v_mfma_scale_f32_32x32x64_f8f6f4, twice the dense rate of the 16-bit
// products), everything after them is the 16-bit kernel's arithmetic.
//
// The pages name 8-bit floating point as the next step of the method's line
// ("FlashAttention-2 (DE)", "Vergleich mit nachfolgenden Versionen /
// FlashAttention-3": FP8 for more speed on newer hardware); they give no
// format and no scaling scheme.  Here:
//   * Q, K, V are E4M3 codes (1 byte per element, [B, H, N, d]) with float
//     scales: the value of element x of a tensor is scale * E4M3(x).  Q and K
//     have one scale per 128-row block of a head (per-block scaling) or one
//     per tensor; V one per head or one per tensor.
//   * S^T = K8 Q8^T on the FP8 matrix cores in float32 (a product of two
//     E4M3 values is exact in float32); the Q and K scales multiply the
//     exponent factor, so each key tile's scores take c = scale * log2(e) *
//     sq * sk once per tile, not per score.
//   * P~ = RNE(P) in the 16-bit output type, O^T += V^T P~^T on the 16-bit
//     matrix cores, with the V codes converted exactly to that type as they
//     are written to LDS (every E4M3 value is a bf16 and an fp16 value); V's
//     scale multiplies O once at the end.
// So with the dequantised values the result is exact attention to the
// 16-bit kernels' precision: only the rounding of the inputs to 8 bits
// separates it from attention on 16-bit inputs.
//
// Work split and pipeline: those of the d = 128 16-bit kernel (fa_fwd.hip,
// fwd16_pipe_kernel): 8 wavefronts (two per SIMD) x 32 query rows, key tiles
// of 64 staged through LDS two ahead, one workgroup barrier per tile, the
// softmax of tile j interleaved with the products of tiles j+1 (S) and j-1
// (O), against a reference maximum fixed by the first tile with an exact
// rerun when a row's tile sum exceeds 2^15.  Per tile a wavefront issues 4
// FP8 products (S) and 16 16-bit products (O) in the order S, O, O, O, O, ...
#include <float.h>

#include <type_traits>

#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {

typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));

// 8-bit products, all operands in VGPRs (as TR::mma): c += A B and a fresh
// A B, for OCP E4M3 A and B (format fields 0), block scales 2^0 (E8M0 code
// 127 in `one`).  The result needs the same hazard wait before vector reads
// as the 16-bit products (mfma_wait_v: 21 wait states, the 16-pass product
// needs 20).
__device__ __forceinline__ void mma8(f32x16_t& c, const i32x8_t& a, const i32x8_t& b, int one) {
  asm("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %3 op_sel_hi:[0,0,0]"
      : "+v"(c)
      : "v"(a), "v"(b), "v"(one));
}
__device__ __forceinline__ f32x16_t mma8_0(const i32x8_t& a, const i32x8_t& b, int one) {
  f32x16_t c;
  asm("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, 0, %3, %3 op_sel_hi:[0,0,0]"
      : "=&v"(c)
      : "v"(a), "v"(b), "v"(one));
  return c;
}

__device__ __forceinline__ i32x8_t cat8(u32x4_t a, u32x4_t b) {
  return i32x8_t{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
}

constexpr float kSumMax8 = 32768.0f;

// Scale block of Q and K rows (per-block scaling).
constexpr int kFp8Block = 128;

template <class TR, int D, bool CAUSAL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd8_pipe_kernel(const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K,
                      const uint8_t* __restrict__ V, const float* __restrict__ q_scale,
                      const float* __restrict__ k_scale, const float* __restrict__ v_scale, int per_block,
                      uint16_t* __restrict__ O, float* __restrict__ LSE, int N, int n_qtiles, uint32_t total,
                      float c, uint32_t qneg) {
  constexpr int NT = 512;                // threads per workgroup
  constexpr int NW = NT / 64;            // wavefronts per workgroup
  constexpr int BC = 64;                 // keys per tile
  constexpr int BR = NW * 32;            // query rows per workgroup (256)
  constexpr int KS8 = D + 16;            // padded K row in LDS (bytes): 16 rows of a read in distinct banks
  constexpr int NKB = BC / 32;           // 32-key blocks per tile
  constexpr int NDB = D / 32;            // 32-column blocks of the output
  constexpr int NK8 = D / 64;            // k-steps of the 8-bit S product over d
  constexpr int NSS = BC / 16;           // k-steps of O over the keys of a tile
  constexpr int NQF = NKB * NK8;         // 8-bit S products per tile
  constexpr int NVF = NSS * NDB;         // 16-bit O products per tile
  constexpr int NS = NQF + NVF;          // matrix instructions per iteration
  constexpr int GAP = NS / NQF;          // an S product every GAP steps
  constexpr int KCH = D / 16;            // 16-byte chunks per K8 row
  constexpr int NKC = BC * KCH / NT;     // K chunks staged per thread
  constexpr int CW = BC * D / (8 * NT);  // V columns staged per thread (8 keys each)
  constexpr int NCG = D / CW;            // V column groups
  constexpr uint32_t RB = D;             // bytes per 8-bit row
  static_assert(NS % NQF == 0 && NKC == 1 && CW == 2, "schedule and staging below are for d = 128");
  constexpr int NBLK = NKB;              // 32x32 score blocks per wavefront and tile
  constexpr int NPAIR = NBLK * 8;        // packed probability pairs per lane and tile
  constexpr int kStg0 = 2;               // staging writes every other step from here
  constexpr int kLoad = kStg0 + 2 * (NKC + CW);
  static_assert(kLoad < NS, "schedule fits one iteration");

  // LDS: two K tiles (8-bit rows) and two V tiles (16-bit, interleaved); the
  // epilogue reuses the whole space for the output rows of all wavefronts
  constexpr int kLdsK = 2 * BC * KS8, kLdsV = 2 * BC * D * 2;
  constexpr int kLdsO = NW * kTileRowsBytes<D>;
  constexpr int kLds = kLdsK + kLdsV > kLdsO ? kLdsK + kLdsV : kLdsO;
  __shared__ __attribute__((aligned(16))) char smem[kLds];
  uint8_t(*sK)[BC * KS8] = (uint8_t(*)[BC * KS8])smem;
  uint16_t(*sV)[BC * D] = (uint16_t(*)[BC * D])(smem + kLdsK);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int h = lane >> 5;
  const int l32 = lane & 31;
  // E8M0 2^0, the block scales of the 8-bit products: set once, far ahead of
  // every product that reads it (the opaque asm keeps the compiler from
  // rematerialising it next to a product)
  int one = 127;
  asm volatile("" : "+v"(one));

  const uint32_t lid = xcd_remap(blockIdx.x, total);
  const int bh = lid / n_qtiles;
  int qt = lid % n_qtiles;
  if (CAUSAL) qt = n_qtiles - 1 - qt;  // heaviest tiles first
  const int q0 = qt * BR;
  const size_t head_off = (size_t)bh * N * D;  // elements (= bytes of the 8-bit tensors)
  const uint32_t head_bytes = (uint32_t)N * RB;
  const int qw = q0 + 32 * w;  // first query row of this wavefront

  // scales: block index of a row (per-block), or entry 0 (per-tensor)
  const int nblk = (N + kFp8Block - 1) / kFp8Block;
  const size_t sbase = per_block ? (size_t)bh * nblk : 0;
  auto kscale = [&](int key0) __attribute__((always_inline)) -> float {
    return k_scale[per_block ? sbase + (size_t)(min(key0, N - 1) / kFp8Block) : 0];
  };
  const float sq = q_scale[per_block ? sbase + (size_t)(min(qw, N - 1) / kFp8Block) : 0];
  const float sv = v_scale[per_block ? (size_t)bh : 0];
  const float cq = c * sq;
  // exponent factor of the key tile starting at key0 (never 0: a masked
  // score is -inf before the multiplication)
  auto ctile = [&](int key0) __attribute__((always_inline)) -> float {
    return fmaxf(cq * kscale(key0), FLT_MIN);
  };

  // Q rows as the B operand of S^T = K Q^T: 32 bytes of d per lane and k-step
  // (bytes 64 ks + 32 h .. +31), loaded once; rows past the end read zeros.
  // A negative scale flips the codes' sign bits (qneg = 0x80808080) once
  // they have arrived (first pass's prologue): the scores are |scale| (-q).k,
  // c = |scale| log2 e.
  i32x8_t qf[NK8];
  {
    const rsrc_t qres = make_rsrc(Q + head_off, head_bytes);
#pragma unroll
    for (int ks = 0; ks < NK8; ++ks) {
      const uint32_t off = (uint32_t)(qw + l32) * RB + 64 * ks + 32 * h;
      qf[ks] = cat8(buf_load16(qres, off), buf_load16(qres, off + 16));
    }
  }

  const int kv_end = CAUSAL ? min(N, q0 + BR) : N;
  const int n_tiles = (kv_end + BC - 1) / BC;

  // ---- staging.  Rows past the end read zeros (their scores are masked,
  // their values multiplied by zero probabilities).
  const rsrc_t kres = make_rsrc(K + head_off, head_bytes);
  const rsrc_t vres = make_rsrc(V + head_off, head_bytes);
  u32x4_t stk;
  uint32_t stv[8], stvc[8];  // V: two codes of 8 rows, and the same as 16-bit pairs
  // K: chunk tid -> row tid / KCH, 16-byte column tid % KCH
  const uint32_t koff = (uint32_t)(tid / KCH) * RB + (tid % KCH) * 16;
  const int kst = (tid / KCH) * KS8 + (tid % KCH) * 16;
  // V: unit tid -> (16-key step vs, half vh, column group vc): 8 rows x 2 columns
  const int vc = tid % NCG;
  const int vh = (tid / NCG) & 1;
  const int vs = tid / (2 * NCG);
  const uint32_t voff = (uint32_t)(16 * vs + 4 * vh) * RB + vc * CW;
  const int vrow = (2 * vs + vh) * D * 8;
  const int vsw = (CW * vc) ^ ((CW * vc >> 3) & 3);  // swizzled slot of column CW vc (+ cc: xor)

  auto load_k = [&](int tile) { stk = buf_load16(kres, koff + (uint32_t)(tile * BC) * RB); };
  auto load_v = [&](int tile) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t off = voff + (uint32_t)(tile * BC + 8 * (k / 4) + (k % 4)) * RB;
      stv[k] = __builtin_amdgcn_raw_buffer_load_b16(vres, off, 0, 0);
    }
  };
  // staging write number i (0: the K chunk; 1, 2: V columns) into buffer b
  auto store_part = [&](int i, int b) __attribute__((always_inline)) {
    if (i < NKC) {
      *(u32x4_t*)(&sK[b][kst]) = stk;
    } else {
      const int cc = i - NKC;  // column within the group
      if (cc == 0) {
        // two codes of each row -> a packed 16-bit pair (columns 2 vc, 2 vc + 1)
#pragma unroll
        for (int k = 0; k < 8; ++k) stvc[k] = TR::from_e4m3(stv[k], false);
      }
      uint32_t o[4];
#pragma unroll
      for (int kp = 0; kp < 4; ++kp) {
        const uint32_t x0 = stvc[2 * kp], x1 = stvc[2 * kp + 1];
        o[kp] = (cc & 1) ? pack_hi(x0, x1) : pack_lo(x0, x1);
      }
      *(u32x4_t*)(&sV[b][vrow + 8 * (vsw ^ cc)]) = u32x4_t{o[0], o[1], o[2], o[3]};
    }
  };

  // ---- per-lane state
  const int kfrag = l32 * KS8 + 32 * h;  // byte offset of this lane's K fragment
  const int vfrag = (h * D + (l32 ^ ((l32 >> 3) & 3))) * 8;  // this lane's V fragment
  f32x16_t acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = zero16();
  f32x16_t sA[NKB], sB[NKB];  // scores of two consecutive tiles
  u32x4_t pA[NKB][2], pB[NKB][2];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) pB[kb][0] = pB[kb][1] = u32x4_t{0u, 0u, 0u, 0u};
  float m_run = -INFINITY, lsum[NKB], ltsum[NKB];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) lsum[kb] = ltsum[kb] = 0.0f;

  // S product i of a tile -> (kb, k-step) = (i % NKB, i / NKB); O product i -> (k-step, db)
  auto kaddr = [&](int b, int i) -> const uint8_t* { return sK[b] + kfrag + 32 * (i % NKB) * KS8 + 64 * (i / NKB); };
  auto vaddr = [&](int b, int i) -> const uint16_t* {
    return sV[b] + vfrag + (2 * (i / NDB) * D + 32 * (i % NDB)) * 8;
  };
  auto kfr = [&](int b, int i) __attribute__((always_inline)) -> i32x8_t {
    const uint8_t* p = kaddr(b, i);
    return cat8(*(const u32x4_t*)p, *(const u32x4_t*)(p + 16));
  };
  auto wait_acc = [&]() __attribute__((always_inline)) { mfma_wait_v(acc[0], acc[1], acc[2], acc[3]); };

  bool rerun = false;
  bool exact = false;  // second pass: m_run holds exact row maxima
  float ct_next = ctile(0);
  // ---- one pipelined iteration (see fwd16_pipe_kernel): PAR = j & 1 selects
  // register sets and buffers; MASKED tiles mask scores as they are read
  auto iteration = [&](auto par, auto masked, int j) __attribute__((always_inline)) {
    constexpr int PAR = decltype(par)::value;
    constexpr bool MASKED = decltype(masked)::value;
    f32x16_t(&s_cur)[NKB] = PAR ? sB : sA;
    f32x16_t(&s_next)[NKB] = PAR ? sA : sB;
    u32x4_t(&p_prev)[NKB][2] = PAR ? pA : pB;
    u32x4_t(&p_cur)[NKB][2] = PAR ? pB : pA;
    constexpr int RD = 1 - PAR;  // buffers read: K_{j+1}, V_{j-1}
    constexpr int WR = PAR;      // buffers written: K_{j+2}, V_j
    const int j0 = j * BC;
    const float ct = ct_next;    // exponent factor of tile j
    ct_next = ctile(j0 + BC);
    mfma_wait_v(s_cur[0], s_cur[1]);  // S_j was produced by matrix instructions

    auto score = [&](int kb, int r) __attribute__((always_inline)) -> float {
      const float x = s_cur[kb][r];
      if constexpr (MASKED) {
        const int key = j0 + 32 * kb + 8 * (r / 4) + 4 * h + (r % 4);
        return (key >= N || (CAUSAL && key > qw + l32)) ? -INFINITY : x;
      }
      return x;
    };
    if (j == 0 && !exact) {
      // first tile: its exact row maximum (both half-waves) is the reference
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) mx = max3f(mx, score(kb, r), score(kb, r + 1));
      const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, mx),
                                                       __builtin_bit_cast(uint32_t, mx), false, false);
      m_run = __builtin_elementwise_maximum(__builtin_bit_cast(float, (uint32_t)sw[0]),
                                            __builtin_bit_cast(float, (uint32_t)sw[1])) * ct;
    }
    float tl[NKB], tlt[NKB];
    const float mneg = -m_run;
    float ta[NPAIR][2], te[NPAIR][2];
    uint32_t tp[NPAIR];
    auto stage = [&](int i, int k) __attribute__((always_inline)) {
      const int kb = i % NBLK, rp = i / NBLK;
      if (k == 0) {
        ta[i][0] = fmaf(score(kb, 2 * rp), ct, mneg);
        ta[i][1] = fmaf(score(kb, 2 * rp + 1), ct, mneg);
      } else if (k == 1) {
        te[i][0] = fast_exp2(ta[i][0]);
        te[i][1] = fast_exp2(ta[i][1]);
      } else if (k == 2) {
        tp[i] = TR::pack2(te[i][0], te[i][1]);
        tl[kb] = rp == 0 ? te[i][0] + te[i][1] : tl[kb] + (te[i][0] + te[i][1]);
      } else {
        tlt[kb] = TR::sum2(tp[i], rp == 0 ? 0.0f : tlt[kb]);
        pin(tp[i]);
        p_cur[kb][rp / 4][rp % 4] = tp[i];
        if (rp == 7) {
          pin(tl[kb]);
          pin(tlt[kb]);
        }
      }
    };
    auto valu = [&](int st) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < NPAIR; ++i)
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (i * NS / NPAIR + k == st) stage(i, k);
      if (st == kStg0) wait_vmem();
      if (st >= kStg0 && st < kLoad && (st - kStg0) % 2 == 0) store_part((st - kStg0) / 2, WR);
      if (st == kLoad) {
        load_k(j + 3);
        load_v(j + 1);
      }
    };

    // matrix steps: step st is S product st / GAP when st % GAP == 0, else O
    // product st - st / GAP - 1; O operands are read kAhead O products ahead,
    // the next S operand right after the S product before it
    constexpr int kAhead = 3;
    u32x4_t fr[kAhead];
#pragma unroll
    for (int x = 0; x < kAhead; ++x) fr[x] = *(const u32x4_t*)vaddr(RD, x);
    i32x8_t kq = kfr(RD, 0);
    static_for<0, NS + 3>([&](auto stc) __attribute__((always_inline)) {
      constexpr int st = decltype(stc)::value;
      if constexpr (st < NS) {
        if constexpr (st % GAP == 0) {
          constexpr int i = st / GAP;
          constexpr int kb = i % NKB, ks = i / NKB;
          const i32x8_t a = kq;
          if constexpr (i + 1 < NQF) kq = kfr(RD, i + 1);
          if constexpr (ks == 0) s_next[kb] = mma8_0(a, qf[ks], one);
          else mma8(s_next[kb], a, qf[ks], one);
        } else {
          constexpr int i = st - st / GAP - 1;
          const u32x4_t a = fr[i % kAhead];
          if constexpr (i + kAhead < NVF) fr[i % kAhead] = *(const u32x4_t*)vaddr(RD, i + kAhead);
          constexpr int ss = i / NDB, db = i % NDB;
          TR::mma(acc[db], a, p_prev[ss / 2][ss % 2]);
        }
      }
      valu(st);
      __builtin_amdgcn_sched_barrier(0);
    });

    // tile row sums over both half-waves; a sum past the bound asks for the rerun
    float t = tl[0];
#pragma unroll
    for (int kb = 1; kb < NKB; ++kb) t += tl[kb];
    const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, t),
                                                     __builtin_bit_cast(uint32_t, t), false, false);
    t = __builtin_bit_cast(float, (uint32_t)sw[0]) + __builtin_bit_cast(float, (uint32_t)sw[1]);
    rerun |= !(t <= kSumMax8);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      lsum[kb] += tl[kb];
      ltsum[kb] += tlt[kb];
    }
    lds_barrier();
  };

  auto run_pass = [&]() __attribute__((always_inline)) {
    // prologue: K_0, K_1 in LDS, V buffer 1 zeroed (iteration 0 multiplies it
    // by the zero probabilities pB), S_0 computed, K_2 and V_0 requested
#pragma unroll
    for (int i = 0; i < CW; ++i) *(u32x4_t*)(&sV[1][(tid + NT * i) * 8]) = u32x4_t{0u, 0u, 0u, 0u};
    load_k(0);
    wait_vmem();  // Q fragments and K_0
    if (!exact) {
#pragma unroll
      for (int ks = 0; ks < NK8; ++ks) {
        qf[ks] ^= (int32_t)qneg;
        asm volatile("s_nop 1" : "+v"(qf[ks]));  // vector write -> inline-asm product read
      }
    }
    store_part(0, 0);
    load_k(1);
    wait_vmem();
    store_part(0, 1);
    lds_barrier();
#pragma unroll
    for (int i = 0; i < NQF; ++i) {
      const int kb = i % NKB, ks = i / NKB;
      const i32x8_t a = kfr(0, i);
      if (ks == 0) sA[kb] = mma8_0(a, qf[ks], one);
      else mma8(sA[kb], a, qf[ks], one);
    }
    load_k(2);
    load_v(0);
    ct_next = ctile(0);
    lds_barrier();  // every wave is done with K_0 before iteration 0 overwrites it

    const int n_iter = (n_tiles + 1) & ~1;
    int n_open = N / BC;
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
    mma_pipeline<NVF, 3>([&](int i) { return vaddr(1, i); },
                         [&](int i, u32x4_t a) { TR::mma(acc[i % NDB], a, pB[(i / NDB) / 2][(i / NDB) % 2]); },
                         [](int) {});
  };

  // A row whose tile sum passed the bound: every wavefront computes its rows'
  // exact maxima directly from Q and K and the pass is redone against them.
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
    const int row = qw + l32;
    const int kend = CAUSAL ? min(N, qw + 32) : N;
    float mx = -INFINITY;
    for (int k0 = 0; k0 < kend; k0 += 32) {
      const uint32_t ko = (uint32_t)(k0 + l32) * RB + 32 * h;
      f32x16_t sc = mma8_0(cat8(buf_load16(kres, ko), buf_load16(kres, ko + 16)), qf[0], one);
#pragma unroll
      for (int ks = 1; ks < NK8; ++ks)
        mma8(sc, cat8(buf_load16(kres, ko + 64 * ks), buf_load16(kres, ko + 64 * ks + 16)), qf[ks], one);
      mfma_wait_v(sc);
      const float ck = ctile(k0);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + 8 * (r / 4) + 4 * h + (r % 4);
        if (!(key >= N || (CAUSAL && key > row))) mx = __builtin_elementwise_maximum(mx, sc[r] * ck);
      }
    }
    m_run = __builtin_elementwise_maximum(mx, swap_halves(mx));
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = zero16();
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      lsum[kb] = ltsum[kb] = 0.0f;
      pB[kb][0] = pB[kb][1] = u32x4_t{0u, 0u, 0u, 0u};
    }
    exact = true;
  }
  wait_acc();

  // epilogue: normalise once (times V's scale), store O and LSE
  float l = 0.0f, lt = 0.0f;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    l += lsum[kb];
    lt += ltsum[kb];
  }
  l += swap_halves(l);
  lt += swap_halves(lt);
  const float inv = sv / lt;
  const int qrow = qw + l32;
  u32x2_t ov[NDB][4];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      ov[db][g] = u32x2_t{TR::pack2(acc[db][4 * g + 0] * inv, acc[db][4 * g + 1] * inv),
                          TR::pack2(acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv)};
  // O stored as whole rows through LDS (the whole space: every wavefront is
  // past its last LDS read after the barrier below)
  lds_barrier();
  store_tile_rows<D>(smem + w * kTileRowsBytes<D>, ov, O + head_off + (size_t)qw * D, min(32, N - qw), lane);
  if (qrow < N && h == 0) LSE[(size_t)bh * N + qrow] = (m_run + __log2f(l)) * kLn2;
}

template <class TR, bool CAUSAL>
static hipError_t launch8(const Fp8Args& a) {
  constexpr int BR = 256;
  const int n_qtiles = (a.N + BR - 1) / BR;
  const uint32_t total = (uint32_t)(n_qtiles * a.BH);
  hipLaunchKernelGGL((fwd8_pipe_kernel<TR, 128, CAUSAL>), dim3(total), dim3(512), 0, a.stream,
                     (const uint8_t*)a.q, (const uint8_t*)a.k, (const uint8_t*)a.v, a.q_scale, a.k_scale,
                     a.v_scale, a.per_block, (uint16_t*)a.o, a.lse, a.N, n_qtiles, total, a.c,
                     a.qneg ? 0x80808080u : 0u);
  return hipGetLastError();
}

hipError_t launch_fwd_fp8(const Fp8Args& a) {
  if (a.dtype == DT_BF16) return a.causal ? launch8<BF16, true>(a) : launch8<BF16, false>(a);
  return a.causal ? launch8<F16, true>(a) : launch8<F16, false>(a);
}

}  // namespace fa
