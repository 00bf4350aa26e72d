// Shared device helpers for the gfx950 (CDNA4) attention kernels.
//
// Everything here is written for one target: 64-lane wavefronts, the
// v_mfma_f32_32x32x16_{bf16,f16} and v_mfma_f32_32x32x2_f32 matrix
// instructions, and 16-byte LDS/global accesses.
//
// MFMA 32x32 register layouts used throughout (lane l = 0..63, h = l / 32):
//   A operand (M x K):  lane l holds row m = l % 32 and a set of K elements
//                       that depends only on h (8 for bf16/f16, 1 for f32).
//   B operand (K x N):  lane l holds column n = l % 32 and the K elements of
//                       the same set as the A operand of the same lane.
//   C/D (M x N), 16 fp32 values per lane, value r:
//                       row m = 8 * (r / 4) + 4 * h + (r % 4), column n = l % 32.
// Only the output layout is relied on exactly.  For the operands the kernels
// only rely on "the same (h, element index) names the same K position in A
// and in B", so the order of the contraction index inside an instruction is a
// free relabelling (a permutation of the summation).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 16-bit element traits: bf16 and fp16 share every kernel; they differ only in
// the MFMA opcode, the fp32 -> 16-bit packing and the 2-wide dot product.
struct BF16 {
  __device__ static inline f32x16_t mfma(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  // Two fp32 values -> packed pair, round to nearest even (v_cvt_pk_bf16_f32).
  __device__ static inline uint32_t pack2(float lo, float hi) {
    bf16x2_t r;
    r[0] = (__bf16)lo;
    r[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, r);
  }
  // acc + x.lo + x.hi for a packed pair (v_dot2c_f32_bf16 against (1, 1)).
  __device__ static inline float sum2(uint32_t x, float acc) {
    const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, x), one, acc, false);
  }
  // acc + a.lo*b.lo + a.hi*b.hi
  __device__ static inline float dot2(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), acc, false);
  }
  // All-VGPR forms (see MfmaAsm below): c += A B, and a fresh A B.
  __device__ static inline void mma(f32x16_t& c, u32x4_t a, u32x4_t b) {
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
  }
  __device__ static inline f32x16_t mma0(u32x4_t a, u32x4_t b) {
    f32x16_t c;
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
    return c;
  }
  // Mixed classes: B operand in AGPRs (VGPR accumulator), or accumulator in
  // AGPRs (VGPR operands).
  __device__ static inline void mma_vva(f32x16_t& c, u32x4_t a, u32x4_t b) {
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "a"(b));
  }
  __device__ static inline f32x16_t mma0_vva(u32x4_t a, u32x4_t b) {
    f32x16_t c;
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "a"(b));
    return c;
  }
  __device__ static inline void mma_avv(f32x16_t& c, u32x4_t a, u32x4_t b) {
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
  }
  // A B + c into fresh VGPRs, c (VGPRs) left unchanged
  __device__ static inline f32x16_t mma_c(u32x4_t a, u32x4_t b, const f32x16_t& c) {
    f32x16_t d;
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %3" : "=&v"(d) : "v"(a), "v"(b), "v"(c));
    return d;
  }
  __device__ static inline f32x16_t mma_c_vva(u32x4_t a, u32x4_t b, const f32x16_t& c) {
    f32x16_t d;
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %3" : "=&v"(d) : "v"(a), "a"(b), "v"(c));
    return d;
  }
  // Two OCP E4M3 codes (bytes 0, 1 of x, or 2, 3 with hi) -> packed pair,
  // exact (v_cvt_scalef32_pk_bf16_fp8 with scale 1).
  __device__ static inline uint32_t from_e4m3(uint32_t x, bool hi) {
    return __builtin_bit_cast(uint32_t, hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, true)
                                           : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, false));
  }
};

struct F16 {
  __device__ static inline f32x16_t mfma(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
  __device__ static inline uint32_t pack2(float lo, float hi) {
    f16x2_t r;
    r[0] = (_Float16)lo;
    r[1] = (_Float16)hi;
    return __builtin_bit_cast(uint32_t, r);
  }
  __device__ static inline float sum2(uint32_t x, float acc) {
    const f16x2_t one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, x), one, acc, false);
  }
  __device__ static inline float dot2(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b),
                                  acc, false);
  }
  // All-VGPR forms (see MfmaAsm below): c += A B, and a fresh A B.
  __device__ static inline void mma(f32x16_t& c, u32x4_t a, u32x4_t b) {
    asm("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
  }
  __device__ static inline f32x16_t mma0(u32x4_t a, u32x4_t b) {
    f32x16_t c;
    asm("v_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
    return c;
  }
  __device__ static inline void mma_vva(f32x16_t& c, u32x4_t a, u32x4_t b) {
    asm("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "a"(b));
  }
  __device__ static inline f32x16_t mma0_vva(u32x4_t a, u32x4_t b) {
    f32x16_t c;
    asm("v_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "a"(b));
    return c;
  }
  __device__ static inline void mma_avv(f32x16_t& c, u32x4_t a, u32x4_t b) {
    asm("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
  }
  // A B + c into fresh VGPRs, c (VGPRs) left unchanged
  __device__ static inline f32x16_t mma_c(u32x4_t a, u32x4_t b, const f32x16_t& c) {
    f32x16_t d;
    asm("v_mfma_f32_32x32x16_f16 %0, %1, %2, %3" : "=&v"(d) : "v"(a), "v"(b), "v"(c));
    return d;
  }
  __device__ static inline f32x16_t mma_c_vva(u32x4_t a, u32x4_t b, const f32x16_t& c) {
    f32x16_t d;
    asm("v_mfma_f32_32x32x16_f16 %0, %1, %2, %3" : "=&v"(d) : "v"(a), "a"(b), "v"(c));
    return d;
  }
  // Two OCP E4M3 codes -> packed fp16 pair, exact (v_cvt_scalef32_pk_f16_fp8, scale 1).
  __device__ static inline uint32_t from_e4m3(uint32_t x, bool hi) {
    return __builtin_bit_cast(uint32_t, hi ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, true)
                                           : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, false));
  }
};

// MfmaAsm: TR::mma / TR::mma0 keep every operand and the result in VGPRs.
// The compiler's own MFMA selection places accumulators in AGPRs whenever a
// kernel needs many registers, which splits the register budget in halves
// and costs copies for every vector access; with these forms a kernel can
// use all of its registers as VGPRs (MFMA issue overlaps other waves' vector
// work equally well with VGPR accumulators).  The compiler's hazard tracking
// does not look inside inline assembly, so a kernel using these forms must
// itself separate a matrix instruction's result from any vector-ALU access to
// it by the required wait states: mfma_wait_v below, placed between the last
// product and the first vector access of its result, with the result as
// operands so that no access moves above the wait.  Back-to-back
// accumulation into the same registers needs no wait states.
#define FA_MFMA_WAIT "s_nop 7\n\ts_nop 7\n\ts_nop 4"
__device__ __forceinline__ void mfma_wait_v(f32x16_t& a) { asm volatile(FA_MFMA_WAIT : "+v"(a)); }
__device__ __forceinline__ void mfma_wait_v(f32x16_t& a, f32x16_t& b) {
  asm volatile(FA_MFMA_WAIT : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void mfma_wait_v(f32x16_t& a, f32x16_t& b, f32x16_t& c, f32x16_t& d) {
  asm volatile(FA_MFMA_WAIT : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
}
__device__ __forceinline__ void mfma_wait_v(f32x16_t& a, f32x16_t& b, f32x16_t& c, f32x16_t& d,
                                            f32x16_t& e, f32x16_t& f, f32x16_t& g, f32x16_t& h) {
  asm volatile(FA_MFMA_WAIT : "+v"(a), "+v"(b), "+v"(c), "+v"(d), "+v"(e), "+v"(f), "+v"(g), "+v"(h));
}
// The same for accumulators held in AGPRs (before v_accvgpr_read).
__device__ __forceinline__ void mfma_wait_a(f32x16_t& a, f32x16_t& b) {
  asm volatile(FA_MFMA_WAIT : "+a"(a), "+a"(b));
}
__device__ __forceinline__ void mfma_wait_a(f32x16_t& a, f32x16_t& b, f32x16_t& c, f32x16_t& d) {
  asm volatile(FA_MFMA_WAIT : "+a"(a), "+a"(b), "+a"(c), "+a"(d));
}
__device__ __forceinline__ void mfma_wait_a(f32x16_t& a, f32x16_t& b, f32x16_t& c, f32x16_t& d,
                                            f32x16_t& e, f32x16_t& f, f32x16_t& g, f32x16_t& h) {
  asm volatile(FA_MFMA_WAIT : "+a"(a), "+a"(b), "+a"(c), "+a"(d), "+a"(e), "+a"(f), "+a"(g), "+a"(h));
}
#undef FA_MFMA_WAIT

// The other direction: a vector-ALU write of a VGPR needs two wait states
// before a matrix instruction reads it, which the compiler does not count
// for the inline-assembly products either.  valu_to_mfma_wait follows such a
// write of an operand (the value as its operand: the write stays above it,
// every read below).  Operands that arrive by loads need none.
__device__ __forceinline__ void valu_to_mfma_wait(u32x4_t& x) { asm volatile("s_nop 1" : "+v"(x)); }

// Products of the software-pipelined kernels.  With AG (one wavefront per
// SIMD, 512 registers) the B operands of mb* and the accumulators of macc
// stay in AGPRs; without (two wavefronts per SIMD, 256 registers each) every
// operand is a VGPR.  wait_acc: the wait states before vector reads of macc
// accumulators.
template <class TR, bool AG>
struct PipeMma {
  __device__ static inline f32x16_t mb0(u32x4_t a, u32x4_t b) {
    if constexpr (AG) return TR::mma0_vva(a, b); else return TR::mma0(a, b);
  }
  __device__ static inline void mb(f32x16_t& c, u32x4_t a, u32x4_t b) {
    if constexpr (AG) TR::mma_vva(c, a, b); else TR::mma(c, a, b);
  }
  __device__ static inline f32x16_t mbc(u32x4_t a, u32x4_t b, const f32x16_t& c) {
    if constexpr (AG) return TR::mma_c_vva(a, b, c); else return TR::mma_c(a, b, c);
  }
  __device__ static inline void macc(f32x16_t& c, u32x4_t a, u32x4_t b) {
    if constexpr (AG) TR::mma_avv(c, a, b); else TR::mma(c, a, b);
  }
  __device__ static inline void wait_acc(f32x16_t& a, f32x16_t& b) {
    if constexpr (AG) mfma_wait_a(a, b); else mfma_wait_v(a, b);
  }
  __device__ static inline void wait_acc(f32x16_t& a, f32x16_t& b, f32x16_t& c, f32x16_t& d) {
    if constexpr (AG) mfma_wait_a(a, b, c, d); else mfma_wait_v(a, b, c, d);
  }
  __device__ static inline void wait_acc(f32x16_t& a, f32x16_t& b, f32x16_t& c, f32x16_t& d,
                                         f32x16_t& e, f32x16_t& f, f32x16_t& g, f32x16_t& h) {
    if constexpr (AG) mfma_wait_a(a, b, c, d, e, f, g, h); else mfma_wait_v(a, b, c, d, e, f, g, h);
  }
  // Two wait states between a vector write of an mb* B operand (in AGPRs
  // with AG) and the products that read it (see valu_to_mfma_wait).
  __device__ static inline void operand_wait(u32x4_t& x) {
    if constexpr (AG) asm volatile("s_nop 1" : "+a"(x));
    else asm volatile("s_nop 1" : "+v"(x));
  }
  // Two wait states between vector writes of macc accumulators (register
  // copies the compiler places where control flow joins) and products that
  // read them next.
  __device__ static inline void copy_wait(f32x16_t& a, f32x16_t& b, f32x16_t& c, f32x16_t& d) {
    if constexpr (AG) asm volatile("s_nop 1" : "+a"(a), "+a"(b), "+a"(c), "+a"(d));
    else asm volatile("s_nop 1" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
  }
  __device__ static inline void copy_wait(f32x16_t& a, f32x16_t& b, f32x16_t& c, f32x16_t& d,
                                          f32x16_t& e, f32x16_t& f, f32x16_t& g, f32x16_t& h) {
    if constexpr (AG) asm volatile("s_nop 1" : "+a"(a), "+a"(b), "+a"(c), "+a"(d), "+a"(e), "+a"(f), "+a"(g), "+a"(h));
    else asm volatile("s_nop 1" : "+v"(a), "+v"(b), "+v"(c), "+v"(d), "+v"(e), "+v"(f), "+v"(g), "+v"(h));
  }
};

// Four 16-bit elements from LDS, transposed across each group of 16 lanes
// (ds_read_b64_tr_b16): with lane j of a group pointing at 4 consecutive
// elements E[j][0..3], lane i of the group receives E[4 * e + i / 4][i % 4]
// for e = 0..3.  So if lanes 4e..4e+3 point at row R_e, columns C + 0..15 in
// steps of 4, lane i receives column C + i of rows R_0..R_3.
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
__device__ inline u32x2_t lds_read_tr(const void* p) {
  return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)p));
}

__device__ inline f32x16_t mfma_f32(float a, float b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__device__ inline f32x16_t zero16() {
  f32x16_t z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.0f;
  return z;
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Value held by lane (l ^ 32): the other half-wave.
__device__ inline float swap_halves(float x) { return __shfl_xor(x, 32, 64); }

// Workgroup index -> logical tile index, so that the workgroups the hardware
// places on one XCD (consecutive dispatch ids go round-robin over the 8 XCDs)
// receive one contiguous range of logical tiles.  Tiles of the same head then
// run on the same XCD and share its L2 for the K/V stream.  A bijection on
// [0, total) for any total.
__device__ inline uint32_t xcd_remap(uint32_t pid, uint32_t total) {
  const uint32_t nx = 8;
  const uint32_t x = pid % nx, slot = pid / nx;
  const uint32_t base = total / nx, rem = total % nx;
  return x * base + (x < rem ? x : rem) + slot;
}

// Tile of round r for workgroup b of a persistent grid of G workgroups
// (G < total, G and nbh multiples of 8).  Tiles are numbered head * nt + t,
// t = 0 the heaviest with the causal mask.  Workgroup b runs on XCD b % 8 and
// takes tiles of the heads congruent to b modulo 8 only.  Within an XCD the
// tiles are taken head by head, G / 8 per round, so the workgroups of one
// XCD work on a few heads at a time and those heads' K/V stay in its L2
// (dealt in the other order, every tile of a round belongs to another head
// and K/V is fetched again per tile).  Rounds alternate direction: with
// whole heads per round, a workgroup's tile t in one round is followed by
// about nt - 1 - t in the next, which evens out the causal costs.  Every
// tile is dealt exactly once; returns nbh * nt when round r has none left
// for b (then none of the later rounds has one either).
__device__ inline uint32_t persistent_tile(uint32_t b, uint32_t G, uint32_t r, uint32_t nbh, uint32_t nt) {
  const uint32_t x = b % 8, j = b / 8, gx = G / 8, nhx = nbh / 8;
  const uint32_t p = r * gx + ((r & 1) ? gx - 1 - j : j);
  if (p >= nhx * nt) return nbh * nt;
  const uint32_t hi = p / nt, t = p - hi * nt;
  return (x + 8 * hi) * nt + t;
}

// Runs run_tile(tile) for the tiles of this workgroup: its own (grid =
// total; XCD-grouped numbering), or, in a persistent grid of fewer
// workgroups than tiles, its share by persistent_tile, one after another
// with a barrier between them that hands the LDS buffers on.  The persistent
// grid spares the launch of a workgroup into a compute unit another has just
// left, which leaves the unit idle for microseconds.  Tiles are independent:
// no workgroup waits for another.
template <class F>
__device__ inline void for_each_tile(uint32_t total, uint32_t nt, F&& run_tile);

// Raw buffer access: 32-bit byte offsets from a per-head base, with the
// hardware range check (an access at or past `bytes` reads zeros).  The whole
// offset goes in the VGPR operand so the range check covers it.
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ inline rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ inline u32x4_t buf_load16(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ inline u32x2_t buf_load8(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
}

// Barrier for LDS hand-off between wavefronts: waits for this wave's LDS
// accesses only, so global loads issued for the next tile stay in flight.
__device__ inline void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <class F>
__device__ inline void for_each_tile(uint32_t total, uint32_t nt, F&& run_tile) {
  const bool pers = gridDim.x < total;
  const uint32_t nbh = total / nt;
  const uint32_t rounds = pers ? (nbh / 8 * nt + gridDim.x / 8 - 1) / (gridDim.x / 8) : 1u;
  for (uint32_t r = 0; r < rounds; ++r) {
    const uint32_t lid = pers ? persistent_tile(blockIdx.x, gridDim.x, r, nbh, nt) : xcd_remap(blockIdx.x, total);
    if (lid >= total) break;
    if (r > 0) lds_barrier();
    run_tile(lid);
  }
}

// A straight-line run of NST matrix products, each taking its A operand from
// LDS: operand k is read AHEAD products before its use, and `extra(k)` (LDS
// staging writes and the like) runs after product k.  The scheduling barrier
// after each product stops the compiler from regrouping the reads next to
// their uses, so AHEAD reads stay in flight behind the matrix core.
template <int NST, int AHEAD, class Addr, class Mma, class Extra>
__device__ inline void mma_pipeline(Addr addr, Mma mma, Extra extra) {
  u32x4_t fr[AHEAD];
#pragma unroll
  for (int x = 0; x < AHEAD; ++x) fr[x] = *(const u32x4_t*)addr(x);
#pragma unroll
  for (int k = 0; k < NST; ++k) {
    const u32x4_t a = fr[k % AHEAD];
    if (k + AHEAD < NST) fr[k % AHEAD] = *(const u32x4_t*)addr(k + AHEAD);
    mma(k, a);
    extra(k);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// f(integral_constant<int, I>) for I = B .. E-1, expanded at compile time (a
// long straight-line schedule that a loop unroller might refuse to expand).
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Materialise x here: an empty asm that "modifies" x keeps the computation of x
// from being sunk past later branches towards its first use.
__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(uint32_t& x) { asm volatile("" : "+v"(x)); }

// max(a, b, c) without NaN canonicalisation of the inputs (v_maximum3_f32).
__device__ __forceinline__ float max3f(float a, float b, float c) {
  return __builtin_elementwise_maximum(a, __builtin_elementwise_maximum(b, c));
}

// A condition the same in every lane of the wave, made visibly uniform so the
// compiler branches on it instead of predicating every guarded instruction.
__device__ inline bool wave_uniform(bool x) { return __builtin_amdgcn_readfirstlane((int)x) != 0; }

// A wavefront's 32 x D output tile held in the layout of a transposed
// product's accumulators (lane l owns row l % 32; v[db][g] holds its columns
// 32 db + 8 g + 4 h + 0..3 as two packed pairs) is stored through LDS, so
// that each store instruction writes whole rows (16 bytes per lane,
// 64 / (D / 8) rows per instruction) instead of 8-byte pieces of 32 rows.
// lds: this wavefront's scratch, 32 rows of 2 D bytes, 16-byte chunk c of
// row r at chunk position c ^ (r % (D / 8)); rows at and past nrows, and
// 16-byte chunks at and past nch, are not stored; row r goes to dst + r *
// row_stride (elements).
template <int D>
__device__ inline void store_tile_rows(char* lds, const u32x2_t (&v)[D / 32][4], uint16_t* dst, int nrows,
                                       int lane, size_t row_stride = D, int nch = D / 8) {
  constexpr int RS = 2 * D;
  constexpr int CPR = D / 8;     // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;  // rows per store instruction
  const int h = lane >> 5, l32 = lane & 31;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *(u32x2_t*)(lds + l32 * RS + ((4 * db + g) ^ (l32 % CPR)) * 16 + 8 * h) = v[db][g];
  // the rows read below were written by other lanes of this wavefront
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int r = RPI * i + lane / CPR, ch = lane % CPR;
    const u32x4_t x = *(const u32x4_t*)(lds + r * RS + (ch ^ (r % CPR)) * 16);
    if (r < nrows && ch < nch) *(u32x4_t*)(dst + (size_t)r * row_stride + 8 * ch) = x;
  }
}
// ---- general layouts: any element strides per tensor (batch, head, row;
// the head dimension contiguous), packed variable-length batches, and head
// dimensions below the kernel's D.
//
// Tensor t's row r of sequence b, head h starts at element
//   b * t.sb + h * t.sh + (start(b) + r) * t.sr,
// start(b) = cu[b] for a packed batch (whose tensors have sb = 0), else 0.
// LSE and D_i entry (b, h, r) is at b * l_sb + h * l_sh + start_q(b) + r.
// Columns at and past dr (a head dimension below the kernel's D) read as
// zeros and are not stored, so the kernel's products over D columns are the
// products over dr.
struct Strides {
  int64_t sb, sh, sr;
};
struct GenLayout {
  Strides q, k, v, o, dout, dq, dk, dv;
  const int32_t* cu_q;  // [B + 1] query-side prefix sums, or NULL
  const int32_t* cu_k;  // [B + 1] key-side prefix sums, or NULL
  int64_t total_q, total_k;  // rows of the packed tensors (prefix sums clamped into [0, total])
  int64_t l_sb, l_sh;
  int H;
  int dr;
  uint32_t qneg;  // forward kernels: 0x80008000 for a negative scale (sign_flip of the queries), else 0
};

// First row and row count of sequence b's queries (or keys): prefix sums
// clamped into [0, total] and the count to [0, nmax]; without prefix sums
// rows 0 .. nmax - 1.
__device__ inline void seq_rows(const int32_t* __restrict__ cu, int64_t total, int b, int nmax, int& start,
                                int& count) {
  if (cu) {
    const int64_t s0 = min(max((int64_t)cu[b], (int64_t)0), total);
    start = (int)s0;
    count = (int)min(max((int64_t)cu[b + 1] - s0, (int64_t)0), min((int64_t)nmax, total - s0));
  } else {
    start = 0;
    count = nmax;
  }
}

// One tensor's rows of one (sequence, head): element offset of row 0, row
// stride in bytes (16-bit elements), and the buffer range in bytes, which
// ends right after the last real row's dr columns (rows from `count` on read
// zeros).
struct TRows {
  size_t off;
  uint32_t rs;
  uint32_t bytes;
};
__device__ inline TRows tensor_rows(const Strides& t, int b, int h, int start, int count, int dr) {
  TRows r;
  r.off = (size_t)((int64_t)b * t.sb + (int64_t)h * t.sh + (int64_t)start * t.sr);
  r.rs = (uint32_t)(t.sr * 2);
  r.bytes = count > 0 ? (uint32_t)(count - 1) * r.rs + 2u * (uint32_t)dr : 0u;
  return r;
}

// Offset added to a load whose 16-bit columns start at byte `cb` of a row:
// past the data's dr columns it moves the load past the buffer range, so it
// reads zeros (bytes < 2^31 and row offsets < 2^31 keep the sum in 32 bits).
__device__ inline uint32_t col_pad(uint32_t cb, int dr, uint32_t bytes) { return cb >= 2u * (uint32_t)dr ? bytes : 0u; }

// A negative scale s enters the forward kernels as |s| with the queries
// negated, since s q.k = |s| (-q).k: the query fragments' 16-bit elements
// have their sign bits flipped (m = 0x80008000), or are left alone (m = 0).
// The exponent factor and every running maximum then see |s|, as for s >= 0.
__device__ inline u32x4_t sign_flip(u32x4_t x, uint32_t m) { return x ^ m; }

// Where the rows of head bh lie.  Dense [BH, N, D]: rows of D elements from
// bh N D, vectors (LSE, D_i) from bh N, all N rows real.  Packed (VL): head
// h of sequence b = bh / H owns rows cu[b] .. cu[b + 1] - 1 of [total, H, D]
// (row stride H D, vectors [H, total] from h total + cu[b]), clamped into
// [0, total] and to N rows, so malformed prefix sums never move an access out
// of the tensors.  `bytes` ends right after the last real row: buffer loads
// of rows from Nb on read zeros, as past the end of a dense head.
struct HeadRows {
  size_t off;       // element offset of row 0
  size_t vec;       // element offset of vector entry 0
  uint32_t rs;      // row stride (bytes)
  uint32_t bytes;   // buffer range from row 0
  int Nb;           // real rows
};

template <int D, bool VL>
__device__ inline HeadRows head_rows(int bh, int N, const int32_t* __restrict__ cu, int H, int total) {
  HeadRows r;
  if constexpr (VL) {
    const int b = bh / H, hd = bh - b * H;
    const int64_t s0 = min(max((int64_t)cu[b], (int64_t)0), (int64_t)total);
    r.Nb = (int)min(max((int64_t)cu[b + 1] - s0, (int64_t)0), min((int64_t)N, (int64_t)total - s0));
    r.off = ((size_t)s0 * H + hd) * D;
    r.vec = (size_t)hd * total + s0;
    r.rs = (uint32_t)H * (2 * D);
    r.bytes = r.Nb > 0 ? (uint32_t)(r.Nb - 1) * r.rs + 2 * D : 0u;
  } else {
    r.Nb = N;
    r.off = (size_t)bh * N * D;
    r.vec = (size_t)bh * N;
    r.rs = 2 * D;
    r.bytes = (uint32_t)N * (2 * D);
  }
  return r;
}

// bytes of LDS scratch per wavefront for store_tile_rows
template <int D>
constexpr int kTileRowsBytes = 32 * 2 * D;

// Wait until every vector-memory load issued so far has returned.
__device__ inline void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// (a.lo, b.lo) and (a.hi, b.hi) as packed pairs, one v_perm_b32 each.
__device__ inline uint32_t pack_lo(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ inline uint32_t pack_hi(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

// Scheduling hints (instruction classes for __builtin_amdgcn_sched_group_barrier).
constexpr int kSchedVALU = 0x002, kSchedMFMA = 0x008, kSchedDSRead = 0x100, kSchedDSWrite = 0x200;

}  // namespace fa
