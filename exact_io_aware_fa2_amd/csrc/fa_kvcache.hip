// Attention of a few new queries against a key/value cache, for gfx950.
//
// The pages name inference beside training as what the method speeds up
// ("FlashAttention-2 (DE)", lead paragraph; "Das Attention-Problem in
// Transformern": Falcon-40B inference) and place it in model serving next to
// the block-wise management of the key/value cache ("FlashAttention"
// glossary, "Der Engpass ist der Weg zum Speicher, nicht das Rechnen" and
// "Wo es verwechselt wird"; related terms "KV Cache", "Memory-Bound").  The
// computation is the same exact attention with Nq new queries (usually 1) and
// a cache of capacity Nk rows, of which the first L = seqlens[b] are filled:
// query i sees key j iff j < L and, causal, j <= i + L - Nq (the queries are
// the last Nq positions of the sequence: the mask is aligned bottom right).
//
// With few queries the work per key is tiny and the cache has to be read once
// from HBM, so the bound is HBM bandwidth, not the matrix cores.  To spread
// one head's cache over many compute units the keys are split into ranges
// ("split-KV"): every wavefront takes one range of `kps` keys and one block of
// 32 queries, runs the tiled online softmax over its range, and writes a
// partial result (O normalised within the range, and two log-sum-exps in base
// 2).  A second kernel merges the ranges of each query with the identity the
// online softmax itself rests on ("FlashAttention" lexicon, "Methodische
// Grundlagen", "Fortlaufende Normierung"):
//     LSE = log2 sum_s 2^{LSE_s},   O = sum_s 2^{LSE_s - LSE} O_s.
// When one range covers every key the first kernel writes O and LSE itself.
//
// Per 32-key tile a wavefront loads K and V rows with coalesced 16-byte loads
// (each instruction reads whole rows), writes them to its own LDS rows,
// computes S^T = K Q^T with the A operands read back row-wise, and
// O^T += V^T P~^T with V read back transposed (ds_read_b64_tr_b16).  Loading
// the A operands of K straight from memory (32 rows touched per instruction)
// measured 5-10% slower.  With few query blocks (decoding) the four
// wavefronts of a workgroup are independent, each staging its own tiles (no
// workgroup barrier); consecutive wavefronts take consecutive ranges (no
// reuse between them, so no XCD grouping).  With four or more query blocks
// per head (prefill, packed batches) a workgroup's wavefronts take four
// consecutive blocks of one range and stage each tile once for all four
// (GRP below; 12% faster on a packed prefill batch).
#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {

// Key (within its 32-key tile) that A-operand row m of S^T = K Q^T holds: m
// with bits 2 and 3 exchanged.  Accumulator value r of lane half h is S^T row
// 8 (r / 4) + 4 h + r % 4, i.e. key 16 (r / 8) + 8 h + r % 8, so the eight
// scores r = 8 t .. 8 t + 7 a lane feeds into P~ V k-step t are eight
// consecutive keys 16 t + 8 h + 0..7 -- the eight rows one pair of transposed
// LDS reads returns for the V^T operand.
__device__ inline int kv_tile_key(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

// F8: the cache holds OCP E4M3 codes (one byte per element) with per-tensor
// scales; K's scale is folded into c by the launcher, V's multiplies the
// output (v_scale, 1 for a 16-bit cache).  The codes are converted to the
// query's 16-bit type (exactly: every E4M3 value is a bf16 and an fp16 value)
// as they are written to LDS, so the products and everything after them are
// those of the 16-bit cache.
//
// GRP (many queries, 16-bit cache): a workgroup takes four consecutive query
// blocks of one (head, key range) instead of four independent ones, and its
// wavefronts stage each K and V tile once for all four (every thread loads
// and writes a quarter of it, two LDS buffers, one workgroup barrier per
// tile), instead of each wavefront staging its own copy.
template <class TR, int D, bool CAUSAL, bool DIRECT, bool F8, bool GRP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D > 128 ? 1 : 2))) void kv_split_kernel(
    const uint16_t* __restrict__ Q, const void* __restrict__ K, const void* __restrict__ V,
    const int32_t* __restrict__ seqlens, uint16_t* __restrict__ O, float* __restrict__ LSE,
    float* __restrict__ part_o, float* __restrict__ part_l, KvLayout lay, int H, int BH, int Nq, int Nk,
    int n_qb, int n_splits, int kps, uint32_t n_waves, float c, float v_scale) {
  constexpr int NKS = D / 16;          // k-steps of S^T = K Q^T
  constexpr int NDB = D / 32;          // 32-row blocks of O^T
  constexpr uint32_t RBC = F8 ? D : 2 * D;  // bytes of one cache row's d elements
  constexpr int RS = 2 * D + 64;       // LDS row bytes of the V tile: a stride of 16 (mod 64)
                                       // dwords puts the 4 rows of a transposed read in 4 bank groups
  constexpr int RSK = 2 * D + 16;      // LDS row bytes of the K tile: a stride of 4 (mod 64) dwords
                                       // puts the 16 rows of a row-wise operand read in 16 bank groups
  constexpr int VCH = (int)RBC / 16;   // 16-byte chunks per cache row
  constexpr int NVL = 32 * VCH / 64;   // chunks per lane per tile and tensor
  constexpr int EPC = F8 ? 16 : 8;     // elements per chunk
  static_assert(32 * RS >= kTileRowsBytes<D>, "the output tile fits the V rows");
  static_assert(!(GRP && F8), "shared staging is for the 16-bit cache");
  constexpr int BUF = 32 * (RS + RSK);  // one tile of V rows, then K rows
  static_assert(!GRP || 2 * BUF >= 4 * kTileRowsBytes<D>, "four output tiles fit the two buffers");
  __shared__ __attribute__((aligned(16))) char smem[(GRP ? 2 : 4) * BUF];

  const int lane = threadIdx.x & 63;
  // wave-uniform values are made visibly uniform (readfirstlane), so that the
  // buffer resources built from them live in scalar registers
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int h = lane >> 5;
  const int l32 = lane & 31;
  // wavefront -> (head, key range, query block), query block fastest
  int qb, split, bh;
  if constexpr (GRP) {
    const uint32_t n_qg = ((uint32_t)n_qb + 3) / 4;  // groups of four query blocks
    const uint32_t g = blockIdx.x;
    qb = (int)(4 * (g % n_qg)) + w;
    split = (int)((g / n_qg) % (uint32_t)n_splits);
    bh = (int)(g / (n_qg * (uint32_t)n_splits));
  } else {
    const uint32_t wid = 4 * blockIdx.x + (uint32_t)w;
    if (wid >= n_waves) return;
    qb = (int)(wid % (uint32_t)n_qb);
    split = (int)((wid / (uint32_t)n_qb) % (uint32_t)n_splits);
    bh = (int)(wid / ((uint32_t)n_qb * (uint32_t)n_splits));
  }
  const int b = bh / H, hd = bh % H;
  // this sequence's queries (start qs, count Lq) and cache rows (start ks0, count L)
  int qs = 0, Lq = Nq, ks0 = 0, L;
  if (lay.cu_q) {
    qs = (int)min(max((int64_t)lay.cu_q[b], (int64_t)0), lay.total_q);
    Lq = (int)min(max((int64_t)lay.cu_q[b + 1] - qs, (int64_t)0), min((int64_t)Nq, lay.total_q - qs));
  }
  if (lay.cu_k) {
    ks0 = (int)min(max((int64_t)lay.cu_k[b], (int64_t)0), lay.total_k);
    L = (int)min(max((int64_t)lay.cu_k[b + 1] - ks0, (int64_t)0), min((int64_t)Nk, lay.total_k - ks0));
  } else {
    L = seqlens ? min(max(seqlens[b], 0), Nk) : Nk;
  }
  qs = __builtin_amdgcn_readfirstlane(qs);
  Lq = __builtin_amdgcn_readfirstlane(Lq);
  ks0 = __builtin_amdgcn_readfirstlane(ks0);
  L = __builtin_amdgcn_readfirstlane(L);
  const int q0 = 32 * qb;
  // no query of this sequence in this block (GRP: in the workgroup's four
  // blocks; a wavefront of a later, empty block still stages and waits)
  if ((GRP ? q0 - 32 * w : q0) >= Lq) return;
  char* lds = smem + w * BUF;  // (per wavefront) V rows, then K rows
  char* ldk = lds + 32 * RS;

  const int qi = q0 + l32;  // this lane's query (rows past Lq read as zeros, never stored)
  // last visible key of this lane's query, and of the block's last real query
  const int lim = CAUSAL ? min(L - 1, qi + L - Lq) : L - 1;
  const int q_last = GRP ? q0 - 32 * w + 127 : q0 + 31;  // last query of the block (GRP: group)
  const int lim_blk = CAUSAL ? min(L - 1, min(q_last, Lq - 1) + L - Lq) : L - 1;
  const int kb = split * kps;
  const int ke = min(kb + kps, lim_blk + 1);

  // Q rows of this block as B operands (column = query); their signs are
  // flipped for a negative scale in the first tile, once the K rows (loaded
  // after them) have arrived
  const uint32_t rsq = (uint32_t)lay.q_sr * 2;             // bytes between query rows
  const uint32_t rsc = (uint32_t)lay.c_sr * (F8 ? 1 : 2);  // bytes between cache rows
  const size_t q_head = (size_t)(b * lay.q_sb + hd * lay.q_sh + qs * lay.q_sr);  // elements
  const size_t o_head = (size_t)(b * lay.o_sb + hd * lay.o_sh + qs * lay.o_sr);  // elements
  u32x4_t qf[NKS];
  {
    const rsrc_t qres = make_rsrc(Q + q_head, Lq > 0 ? (uint32_t)(Lq - 1) * rsq + 2 * D : 0u);
    const uint32_t off = (uint32_t)qi * rsq + 16 * h;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[ks] = buf_load16(qres, off + 32 * ks);
  }
  // the cache of this head up to the filled length: rows at and past L read as zeros
  const size_t cache_head = (size_t)(b * lay.c_sb + hd * lay.c_sh + ks0 * lay.c_sr) * (F8 ? 1 : 2);  // bytes
  const size_t v_head = (size_t)(b * lay.v_sb + hd * lay.v_sh + ks0 * lay.v_sr) * (F8 ? 1 : 2);     // bytes
  const uint32_t rsv = (uint32_t)lay.v_sr * (F8 ? 1 : 2);  // bytes between value rows
  const uint32_t cache_bytes = L > 0 ? (uint32_t)(L - 1) * rsc + RBC : 0u;
  const uint32_t v_bytes = L > 0 ? (uint32_t)(L - 1) * rsv + RBC : 0u;
  const rsrc_t kres = make_rsrc((const char*)K + cache_head, cache_bytes);
  const rsrc_t vres = make_rsrc((const char*)V + v_head, v_bytes);
  const int k_row = kv_tile_key(l32) * RSK + 16 * h;  // A operand of K: row read from LDS
  // transposed-read address of this lane: group G = lane / 16 reads columns
  // 16 (G % 2) + 0..15 of rows 8 h + 0..3 (and + 4), lane 4 e + i of the group
  // pointing at columns 4 i .. 4 i + 3 of row e
  const int L16 = lane & 15, G = lane >> 4;
  const int tr_base = (8 * h + (L16 >> 2)) * RS + (16 * (G & 1) + 4 * (L16 & 3)) * 2;

  float m = -INFINITY;     // running reference maximum (base-2 units), the same in both halves
  float l = 0.0f, lt = 0.0f;  // this lane's partial sums of P and of the rounded P~
  f32x16_t acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = zero16();

  // K and V are loaded one tile ahead: the loads of tile i + 1 go into the
  // registers tile i has just written to LDS (K right after its K rows are in
  // LDS, V right after its V rows), so one tile's loads are in flight while a
  // tile is computed.  (Two tiles ahead -- in the registers of one 16-bit
  // tile for the 8-bit cache, or at a wavefront per SIMD less for the 16-bit
  // cache at d = 64 -- measured no faster, and the 8-bit cache then fetched
  // 5% more than its compulsory bytes.)  The loads are issued for every tile
  // (the last one reloads itself, an L2 hit), so that the wait counts are the
  // same on every path and no wait for one tile's data also waits for the
  // next tile's.  Chunk i of a thread is 16-byte chunk x % VCH of row
  // x / VCH of the tile (VCH chunks per cache row), x = 64 i + lane for a
  // wavefront's own staging, x = 256 i + thread for the workgroup's (GRP).
  constexpr int NCH = GRP ? 32 * VCH / 256 : NVL;  // chunks per thread and tensor
  static_assert(NCH >= 1, "every thread stages at least one chunk");
  const int tid_s = GRP ? (int)threadIdx.x : lane;
  constexpr int CST = GRP ? 256 : 64;
  u32x4_t kc[NCH], vv[NCH];
  auto load_k = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int ch = CST * i + tid_s;
      kc[i] = buf_load16(kres, (uint32_t)(k0 + ch / VCH) * rsc + 16 * (ch % VCH));
    }
  };
  auto load_v = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int ch = CST * i + tid_s;
      vv[i] = buf_load16(vres, (uint32_t)(k0 + ch / VCH) * rsv + 16 * (ch % VCH));
    }
  };
  // chunk x (16 bytes of a cache row) -> its row's LDS position: as is, or
  // as 16 E4M3 codes converted to 32 bytes of the 16-bit type
  auto put = [&](char* dst, u32x4_t x) __attribute__((always_inline)) {
    if constexpr (F8) {
      u32x4_t a, b;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        a[2 * j] = TR::from_e4m3(x[j], false);
        a[2 * j + 1] = TR::from_e4m3(x[j], true);
        b[2 * j] = TR::from_e4m3(x[2 + j], false);
        b[2 * j + 1] = TR::from_e4m3(x[2 + j], true);
      }
      *(u32x4_t*)dst = a;
      *(u32x4_t*)(dst + 16) = b;
    } else {
      *(u32x4_t*)dst = x;
    }
  };
  // keys of this range visible to this lane's query
  const int lim_r = min(lim, ke - 1);
  if (kb < ke) {
    // K before V: the wait for a tile's K leaves its V in flight, on entry as
    // on the back edge
    load_k(kb);
    __builtin_amdgcn_sched_barrier(0);
    load_v(kb);
  }
  auto wave_sync = []() __attribute__((always_inline)) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  };

  // one 32-key tile starting at key k0, staged in bv (V rows) and bk (K rows);
  // the staging registers then receive the tile starting at key kn
  auto tile = [&](char* bv, char* bk, int k0, int kn, bool first) __attribute__((always_inline)) {
    // K rows -> LDS.  Own staging: the previous tile's operand reads are done
    // (they fed its S products, which come before its V writes and their
    // fence).  GRP: this buffer was last read two tiles ago, before the
    // previous tile's barrier.
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int ch = CST * i + tid_s;
      put(bk + (ch / VCH) * RSK + 2 * EPC * (ch % VCH), kc[i]);
    }
    if (first) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) qf[ks] = sign_flip(qf[ks], lay.qneg);
    }
    load_k(kn);
    if constexpr (GRP) {
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int ch = CST * i + tid_s;
        put(bv + (ch / VCH) * RS + 2 * EPC * (ch % VCH), vv[i]);
      }
      load_v(kn);
      lds_barrier();  // the whole tile is in LDS
    } else {
      wave_sync();
    }
    u32x4_t kf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) kf[ks] = *(const u32x4_t*)(bk + k_row + 32 * ks);
    f32x16_t s = zero16();
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) s = TR::mfma(kf[ks], qf[ks], s);

    // scores in base-2 units, masked; tile maximum of the query over both halves
    float x[16];
    float mt = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = k0 + 16 * (r / 8) + 8 * h + (r % 8);
      x[r] = key <= lim_r ? s[r] * c : -INFINITY;
      mt = fmaxf(mt, x[r]);
    }
    mt = fmaxf(mt, swap_halves(mt));
    const float mn = fmaxf(m, mt);
    const float mu = mn == -INFINITY ? 0.0f : mn;  // no visible key yet: every weight is 0
    const float alpha = fast_exp2(m - mu);
    if (__any(alpha != 1.0f)) {
      l *= alpha;
      lt *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
    }
    m = mn;
    u32x4_t pk[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p0 = fast_exp2(x[8 * t + 2 * j] - mu), p1 = fast_exp2(x[8 * t + 2 * j + 1] - mu);
        l += p0 + p1;
        pk[t][j] = TR::pack2(p0, p1);
        lt = TR::sum2(pk[t][j], lt);
      }

    if constexpr (!GRP) {
      // V rows -> this wavefront's LDS (after the previous tile's reads)
      wave_sync();
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int ch = CST * i + tid_s;
        put(bv + (ch / VCH) * RS + 2 * EPC * (ch % VCH), vv[i]);
      }
      load_v(kn);
      wave_sync();
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const char* p = bv + tr_base + 16 * t * RS + 64 * db;
        const u32x2_t a = lds_read_tr(p), b2 = lds_read_tr(p + 4 * RS);
        acc[db] = TR::mfma(u32x4_t{a[0], a[1], b2[0], b2[1]}, pk[t], acc[db]);
      }
  };
  int it = 0;
  for (int k0 = kb; k0 < ke; k0 += 32, ++it) {
    const int kn = k0 + 32 < ke ? k0 + 32 : k0;
    if constexpr (GRP) {
      char* bv = smem + (it & 1) * BUF;
      tile(bv, bv + 32 * RS, k0, kn, it == 0);
    } else {
      tile(lds, ldk, k0, kn, it == 0);
    }
  }
  l += swap_halves(l);
  lt += swap_halves(lt);
  const bool empty = m == -INFINITY;  // no visible key for this query in this range
  const float inv = empty ? 0.0f : v_scale / lt;

  if constexpr (DIRECT) {
    u32x2_t ov[NDB][4];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        ov[db][g] = u32x2_t{TR::pack2(acc[db][4 * g + 0] * inv, acc[db][4 * g + 1] * inv),
                            TR::pack2(acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv)};
    if constexpr (GRP) {
      lds_barrier();  // every wavefront is done with the tiles; slice w of the buffers is its own
      store_tile_rows<D>(smem + w * kTileRowsBytes<D>, ov, O + o_head + (size_t)q0 * lay.o_sr, min(32, Lq - q0),
                         lane, (size_t)lay.o_sr);
    } else {
      wave_sync();
      store_tile_rows<D>(lds, ov, O + o_head + (size_t)q0 * lay.o_sr, min(32, Lq - q0), lane, (size_t)lay.o_sr);
    }
    if (h == 0 && qi < Lq)
      LSE[b * lay.l_sb + hd * lay.l_sh + qs + qi] = empty ? -INFINITY : (m + __log2f(l)) * kLn2;
  } else {
    if (qi < Lq) {
      const size_t rec = ((size_t)split * BH + bh) * Nq + qi;
      float* po = part_o + rec * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *(float4*)(po + 32 * db + 8 * g + 4 * h) =
              float4{acc[db][4 * g] * inv, acc[db][4 * g + 1] * inv, acc[db][4 * g + 2] * inv,
                     acc[db][4 * g + 3] * inv};
      if (h == 0)
        *(float2*)(part_l + 2 * rec) =
            empty ? float2{-INFINITY, -INFINITY} : float2{m + __log2f(lt), m + __log2f(l)};
    }
  }
}

// One wavefront per query row: combine the key ranges' partial results.
// part_l holds per range (log2 of the range's sum of rounded weights P~, log2
// of its sum of P), both including the range's reference maximum; part_o the
// range's O normalised by its own sum of P~.  O is normalised by the total
// sum of P~ (the weights that multiplied V), LSE uses the total sum of P.
// Lane s computes the weight of range s (s = lane, lane + 64, ...); the loop
// over the ranges' O rows then takes each weight from its lane, so no load
// waits for another (an empty range has weight 0 and an all-zero row).
template <class TR, int D>
__global__ __launch_bounds__(256) void kv_merge_kernel(const float* __restrict__ part_o,
                                                       const float* __restrict__ part_l,
                                                       uint16_t* __restrict__ O, float* __restrict__ LSE,
                                                       KvLayout lay, int H, int Nq, int rows, int n_splits) {
  constexpr int PER = D >= 64 ? D / 64 : 1;  // columns per lane
  constexpr int UNR = 16;                    // ranges whose rows are loaded before their use
  const int lane = threadIdx.x & 63;
  const int row = (int)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  if (row >= rows) return;
  // row = (batch * H + head) * Nq + query; queries past the sequence's own
  // count have no partial results and no output
  const int bh = row / Nq, qi = row % Nq, b = bh / H, hd = bh % H;
  int qs = 0, Lq = Nq;
  if (lay.cu_q) {
    qs = (int)min(max((int64_t)lay.cu_q[b], (int64_t)0), lay.total_q);
    Lq = (int)min(max((int64_t)lay.cu_q[b + 1] - qs, (int64_t)0), min((int64_t)Nq, lay.total_q - qs));
  }
  if (qi >= __builtin_amdgcn_readfirstlane(Lq)) return;
  float mt = -INFINITY, ml = -INFINITY;
  for (int s = lane; s < n_splits; s += 64) {
    const float2 v = *(const float2*)(part_l + 2 * ((size_t)s * rows + row));
    mt = fmaxf(mt, v.x);
    ml = fmaxf(ml, v.y);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    mt = fmaxf(mt, __shfl_xor(mt, off, 64));
    ml = fmaxf(ml, __shfl_xor(ml, off, 64));
  }
  const bool empty = mt == -INFINITY;
  float acc[PER];
#pragma unroll
  for (int p = 0; p < PER; ++p) acc[p] = 0.0f;
  float ws = 0.0f, ls = 0.0f;
  if (!empty) {
    for (int s0 = 0; s0 < n_splits; s0 += 64) {
      // weight of range s0 + lane (0 past the last range or for an empty range)
      float wt = 0.0f;
      if (s0 + lane < n_splits) {
        const float2 v = *(const float2*)(part_l + 2 * ((size_t)(s0 + lane) * rows + row));
        wt = fast_exp2(v.x - mt);
        ws += wt;
        ls += fast_exp2(v.y - ml);
      }
      const int ns = min(64, n_splits - s0);
      for (int j0 = 0; j0 < ns; j0 += UNR) {
        float x[UNR][PER];
#pragma unroll
        for (int j = 0; j < UNR; ++j) {
          const int s = s0 + min(j0 + j, ns - 1);  // clamped: a repeated row gets weight 0 below
          const float* po = part_o + ((size_t)s * rows + row) * D + min(PER * lane, D - PER);
#pragma unroll
          for (int p = 0; p < PER; ++p) x[j][p] = po[p];
        }
#pragma unroll
        for (int j = 0; j < UNR; ++j) {
          const float wj = __shfl(wt, j0 + j, 64);
          const float wu = j0 + j < ns ? wj : 0.0f;
#pragma unroll
          for (int p = 0; p < PER; ++p) acc[p] += wu * x[j][p];
        }
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      ws += __shfl_xor(ws, off, 64);
      ls += __shfl_xor(ls, off, 64);
    }
  }
  const float inv = empty ? 0.0f : 1.0f / ws;
  uint16_t* orow = O + (size_t)(b * lay.o_sb + hd * lay.o_sh + (qs + qi) * lay.o_sr) + PER * lane;
  if constexpr (PER == 4) {
    *(u32x2_t*)orow = u32x2_t{TR::pack2(acc[0] * inv, acc[1] * inv), TR::pack2(acc[2] * inv, acc[3] * inv)};
  } else if constexpr (PER == 2) {
    *(uint32_t*)orow = TR::pack2(acc[0] * inv, acc[1] * inv);
  } else if (PER * lane < D) {  // d = 32: lanes 32..63 hold no column
    *orow = (uint16_t)(TR::pack2(acc[0] * inv, 0.0f) & 0xFFFFu);
  }
  if (lane == 0) LSE[b * lay.l_sb + hd * lay.l_sh + qs + qi] = empty ? -INFINITY : (ml + __log2f(ls)) * kLn2;
}

// ------------------------------------------------------------------ launch

template <class TR, int D, bool CAUSAL, bool F8, bool GRP>
static hipError_t launch_split(const KvArgs& a, const KvPlan& p, bool direct, float* part_o, float* part_l) {
  const uint32_t n_waves = (uint32_t)((int64_t)a.BH * p.n_qb * p.n_splits);
  const uint32_t n_wg = GRP ? (uint32_t)((int64_t)a.BH * p.n_splits * ((p.n_qb + 3) / 4)) : (n_waves + 3) / 4;
  if (direct)
    hipLaunchKernelGGL((kv_split_kernel<TR, D, CAUSAL, true, F8, GRP>), dim3(n_wg), dim3(256), 0, a.stream,
                       (const uint16_t*)a.q, a.k, a.v, a.seqlens, (uint16_t*)a.o, a.lse, nullptr, nullptr, a.lay,
                       a.H, a.BH, a.Nq, a.Nk, p.n_qb, p.n_splits, p.kps, n_waves, a.c, a.v_scale);
  else
    hipLaunchKernelGGL((kv_split_kernel<TR, D, CAUSAL, false, F8, GRP>), dim3(n_wg), dim3(256), 0, a.stream,
                       (const uint16_t*)a.q, a.k, a.v, a.seqlens, nullptr, nullptr, part_o, part_l, a.lay, a.H,
                       a.BH, a.Nq, a.Nk, p.n_qb, p.n_splits, p.kps, n_waves, a.c, a.v_scale);
  return hipGetLastError();
}

// Many query blocks per head (prefill, packed batches) and a 16-bit cache:
// workgroups of four query blocks share each staged tile (GRP); few query
// blocks (decode) or an 8-bit cache: independent wavefronts.
template <class TR, int D, bool CAUSAL, bool F8>
static hipError_t launch_kv(const KvArgs& a, const KvPlan& p) {
  float* part_o = (float*)a.workspace;
  float* part_l = part_o ? part_o + (size_t)p.n_splits * a.BH * a.Nq * D : nullptr;
  const bool direct = p.n_splits == 1;
  hipError_t e;
  if constexpr (!F8 && D >= 64) {  // (at d = 32 a tile is fewer chunks than threads)
    e = p.n_qb >= 4 ? launch_split<TR, D, CAUSAL, false, true>(a, p, direct, part_o, part_l)
                    : launch_split<TR, D, CAUSAL, false, false>(a, p, direct, part_o, part_l);
  } else {
    e = launch_split<TR, D, CAUSAL, F8, false>(a, p, direct, part_o, part_l);
  }
  if (e != hipSuccess || direct) return e;
  const int rows = a.BH * a.Nq;
  hipLaunchKernelGGL((kv_merge_kernel<TR, D>), dim3((rows + 3) / 4), dim3(256), 0, a.stream, part_o, part_l,
                     (uint16_t*)a.o, a.lse, a.lay, a.H, a.Nq, rows, p.n_splits);
  return hipGetLastError();
}

template <class TR, bool F8>
static hipError_t dispatch_kv(const KvArgs& a, const KvPlan& p) {
  if constexpr (!F8) {
    if (a.d == 256) return a.causal ? launch_kv<TR, 256, true, F8>(a, p) : launch_kv<TR, 256, false, F8>(a, p);
  }
  if (a.d == 128) return a.causal ? launch_kv<TR, 128, true, F8>(a, p) : launch_kv<TR, 128, false, F8>(a, p);
  if (a.d == 64) return a.causal ? launch_kv<TR, 64, true, F8>(a, p) : launch_kv<TR, 64, false, F8>(a, p);
  return a.causal ? launch_kv<TR, 32, true, F8>(a, p) : launch_kv<TR, 32, false, F8>(a, p);
}

hipError_t launch_fwd_kvcache(const KvArgs& a) {
  const KvPlan p = a.one_range ? kv_plan_one_range(a.Nq, a.Nk) : kv_plan(a.BH, a.Nq, a.Nk, a.d);
  if (a.fp8_cache && a.d == 256) return hipErrorInvalidValue;
  if (a.fp8_cache) return a.dtype == DT_BF16 ? dispatch_kv<BF16, true>(a, p) : dispatch_kv<F16, true>(a, p);
  return a.dtype == DT_BF16 ? dispatch_kv<BF16, false>(a, p) : dispatch_kv<F16, false>(a, p);
}

}  // namespace fa
