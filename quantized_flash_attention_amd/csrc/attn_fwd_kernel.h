// INT8-QK / BF16-PV flash attention forward for gfx950 (CDNA4): the kernel
// template and its launch helpers, instantiated by attn_fwd_inst_*.hip.
//
// Method: FastVideo API docs, "minimax_h3_sparse_int8" (int8 QK with per-token
// scales and fp32 accumulation, BF16 PV, tile-64 block mask with a validity
// vector masking partial key tiles, 64-query tiles so no blocks are added, one
// V scale per (head, channel) applied once in the epilogue); comfy-kitchen
// issue #177 (an additive per-key bias [1,1,1,K] shared by heads and queries:
// it is loaded once per key tile and folded into the score scaling, so its
// stride-0 broadcast costs one key vector per tile); FlyDSL PR #886 (LSE from
// the log2-domain running max: m*ln2 + ln(l), -inf for fully masked rows, one
// writer per row).
//
// Work decomposition
//   block  = BM = 128 query rows of one (b,h), 4 waves. Block-sparse blocks
//            hold two 64-query tiles (the unit of the tile mask) and walk
//            the union of their key-tile lists.
//   wave   = 32 query rows. The wave computes S^T = K8 Q8^T with
//            v_mfma_i32_32x32x32_i8 (A = K rows from LDS, B = Q codes kept in
//            VGPRs for the whole key loop), so each lane ends up owning one
//            query row (lane % 32) and 16 of the 32 keys of a block: row max
//            and row sum need a single exchange with lane ^ 32.
//   PV     = O^T += V^T P^T with v_mfma_f32_32x32x16_{bf16,f16}: P^T comes
//            straight from the lane's own score registers, V^T is read from
//            the row-major LDS V tile with ds_read_b64_tr_b16 (4 keys of one
//            channel per lane), and O^T leaves each lane holding 16 channels
//            of its own query row per 32-channel block, so the online-softmax
//            rescale is a per-lane scalar.
//   keys   = 64 per tile. K8/V tiles and the raw key terms go global -> LDS
//            by buffer loads that write LDS directly, into a 3-stage ring
//            (copies run two tiles ahead of the MFMAs).
//   grid   = 1-D, remapped so that the blocks one XCD runs cover whole heads
//            (consecutive block ids are dealt round-robin to the 8 XCDs);
//            blocks sharing K/V then share that XCD's L2. Causal calls order
//            the blocks by walk length instead (causal_order).
#pragma once

#include "qfa_internal.h"

#include <float.h>

#include <type_traits>

namespace qfa {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Lazy rescaling: the running reference max only moves when a row's max
// exceeds it by more than this (log2 units), so p <= 2^8 between rescales.
constexpr float kRescaleSlack = 8.0f;

constexpr int BN = 64;  // keys per tile

// The int32 score accumulators start at the bit pattern of 1.5*2^23, so the
// MFMA leaves bits(1.5*2^23) + S: read as fp32 that is exactly 1.5*2^23 + S
// (|S| <= 128*127^2 < 2^22). Then S*ks = fma(x, ks, -1.5*2^23*ks), one
// instruction instead of a convert and a multiply; the rounding of the
// per-key constant adds at most 0.75*ks (under one unit of S) to S*ks.
constexpr int kMagicBits = 0x4B400000;
constexpr float kMagic = 12582912.0f;

template <int D>
struct Tile {
  static constexpr int kStride = D + 16;        // bytes per K8 row in LDS
  static constexpr int vStride = 2 * D + 64;    // bytes per V row in LDS
  static constexpr int kBytes = BN * kStride;
  static constexpr int vBytes = BN * vStride;
};

__device__ __forceinline__ int xcd_remap(int L, int total) {
  const int per = total / 8, rem = total % 8;
  const int xcd = L % 8, slot = L / 8;
  return xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
}

// Causal launches: dispatch index k -> work index L. Work is numbered by
// query-tile rank (longest walk first), then (head, split) unit. Blocks k and
// k + ncu start on the same CU, so the second round of ncu blocks runs in
// reverse (in groups of 8, keeping k mod 8): each CU then pairs a long walk
// with a short one. Block k runs on XCD k mod 8, so when the unit count is a
// multiple of 8 a unit's blocks share one XCD (L mod 8 = unit mod 8);
// otherwise the units rotate over the XCDs. (Padding the unit count to a
// multiple of 8 would pin the padding to whole XCDs: with 4 units, XCDs 4..7
// would get nothing but empty blocks.) Any order is correct; this one
// balances the first two rounds, and later blocks take freed slots longest
// first.
__device__ __forceinline__ int causal_order(int k, int total, int ncu) {
  if (ncu % 8 != 0 || k < ncu || k >= 2 * ncu) return k;
  const int m = min(total, 2 * ncu) - ncu;   // blocks of the second round
  const int j = k - ncu;
  return m % 8 == 0 ? ncu + (m / 8 - 1 - j / 8) * 8 + j % 8 : ncu + (m - 1 - j);
}

__device__ __forceinline__ float load_bias(const void* p, int dtype, int64_t idx) {
  if (dtype == FP32) return ((const float*)p)[idx];
  const uint32_t h = ((const uint16_t*)p)[idx];
  return dtype == BF16 ? bf16_bits_to_float(h) : half_bits_to_float(h);
}

// Dense calls walk the key tiles that cover up to 4 key segments, segment
// after segment. Tile `it` of that walk and the bounds [slo, shi) of its
// segment; everything here is wave-uniform and lives in SGPRs.
__device__ __forceinline__ void seg_at(const AttnArgs& a, int it, int& tile, int& slo, int& shi) {
  int t0 = a.seg_t0[0], base = 0;
  slo = a.seg_lo[0];
  shi = a.seg_hi[0];
#pragma unroll
  for (int g = 1; g < 4; ++g) {
    const bool past = it >= a.seg_cum[g];
    t0 = past ? a.seg_t0[g] : t0;
    slo = past ? a.seg_lo[g] : slo;
    shi = past ? a.seg_hi[g] : shi;
    base = past ? a.seg_cum[g] : base;
  }
  tile = t0 + it - base;
}

__device__ __forceinline__ float max3(float a, float b, float c) { return fmaxf(a, fmaxf(b, c)); }

// max of 32 values as a tree of v_max3
__device__ __forceinline__ float max32(const float (&t)[2][16]) {
  float a[11];
#pragma unroll
  for (int k = 0; k < 10; ++k) {
    const int i = 3 * k, j = 3 * k + 1, l = 3 * k + 2;
    a[k] = max3(t[i / 16][i % 16], t[j / 16][j % 16], t[l / 16][l % 16]);
  }
  a[10] = fmaxf(t[1][14], t[1][15]);
  const float b0 = max3(a[0], a[1], a[2]), b1 = max3(a[3], a[4], a[5]), b2 = max3(a[6], a[7], a[8]);
  const float b3 = fmaxf(a[9], a[10]);
  return fmaxf(max3(b0, b1, b2), b3);
}

__device__ __forceinline__ float xmax32(float x) {
  // max with the partner lane (lane ^ 32): v_permlane32_swap hands each lane
  // the value of the other half-wave
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}

__device__ __forceinline__ float xsum32(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// ---- LDS tiles ------------------------------------------------------------
// Tiles are copied from global memory straight into LDS (buffer loads with
// the LDS destination: each load instruction writes 64 lanes x 16 bytes,
// lane after lane, from a wave-uniform LDS base). Rows are therefore stored
// unpadded, and bank conflicts of the operand reads are avoided by XOR-ing
// the 16-byte chunk index with a function of the row:
//  K rows (R = D bytes of int8 codes, or 2D bytes of bf16/fp16 for the
//    unquantized path; R/16 chunks): the MFMA A-operand read hands 16 lanes
//    16 rows of one chunk; chunk ^= (row / (256/R)) mod (R/16) puts them on
//    16 different 16-byte bank groups.
//  V rows (2D bytes, D/8 chunks): ds_read_b64_tr_b16 hands a 16-lane group
//    4 consecutive rows of one 32-byte window; chunk ^= (row mod 4) *
//    (D/32) moves the 4 windows apart.
template <int R>
__device__ __forceinline__ int k_chunk_pos(int row, int chunk) {
  constexpr int kChunks = R / 16, kRowsPer256 = 256 / R;
  return chunk ^ ((row / kRowsPer256) & (kChunks - 1));
}
template <int D>
__device__ __forceinline__ int v_chunk_pos(int row, int chunk) {
  return chunk ^ ((row & 3) * (D / 32));
}

typedef unsigned v4u __attribute__((ext_vector_type(4)));

// Buffer descriptor of `bytes` bytes at `base` (raw addressing, range-checked:
// a lane whose offset is at or past the size reads zero).
__device__ __forceinline__ v4u buf_desc(const void* base, int64_t bytes) {
  const uint64_t p = (uint64_t)base;
  const unsigned n = bytes <= 0 ? 0u : (bytes >= 0x7fffffff ? 0x7fffffffu : (unsigned)bytes);
  return v4u{(unsigned)p, (unsigned)(p >> 32) & 0xffffu, n, 0x00020000u};
}

// Same for a size known to be below 2^31 bytes: no clamping, so the
// descriptor costs a handful of scalar instructions.
// The values are wave-uniform; readfirstlane states it for the compiler,
// which otherwise may keep a copy of them in VGPRs.
__device__ __forceinline__ v4u buf_desc32(const void* base, int bytes) {
  const uint64_t p = (uint64_t)base;
  return v4u{(unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)p),
             (unsigned)__builtin_amdgcn_readfirstlane((int)((p >> 32) & 0xffffu)),
             (unsigned)__builtin_amdgcn_readfirstlane(bytes), 0x00020000u};
}

// LDS byte address of a shared-memory location.
template <typename T>
__device__ __forceinline__ unsigned lds_addr(const T* p) {
  return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) T*)p;
}

// Global -> LDS copy of one lane-linear block: lane l's SIZE bytes (16, 4,
// or 2 or 1 zero-extended to 4) land at lds + l*max(SIZE,4). Written as inline
// assembly so that the compiler neither waits on these copies before
// unrelated LDS reads nor counts them: every wait for them is explicit
// (wait_vmcnt / stage_barrier), and the loop issues no other vector-memory
// instruction, so those waits count exactly these copies.
// M0 is reserved to the compiler, which warns about clobbering it; the
// kernels of this file make no other use of M0, so nothing is live in it
// across these statements.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <int SIZE>
__device__ __forceinline__ void lds_copy(unsigned lds, int voff, v4u desc) {
  if constexpr (SIZE == 16)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(lds), "v"(voff), "s"(desc) : "memory", "m0");
  else if constexpr (SIZE == 4)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                 :: "s"(lds), "v"(voff), "s"(desc) : "memory", "m0");
  else if constexpr (SIZE == 2)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_ushort %1, %2, 0 offen lds"
                 :: "s"(lds), "v"(voff), "s"(desc) : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_ubyte %1, %2, 0 offen lds"
                 :: "s"(lds), "v"(voff), "s"(desc) : "memory", "m0");
}
#pragma clang diagnostic pop

// Per-key terms of one tile: sc[0] key scale ks, sc[1] = -kMagic*ks (turns
// the biased accumulator into S*ks with one FMA; for an excluded key ks = 0
// and sc[1] = -inf, so its score comes out -inf), sc[2] log2-domain bias
// term bias*log2(e) (biased calls only), sc[3] the -kMagic*ks / -inf terms
// of the second query tile of a block-sparse block. Wave 0 copies the key
// scales into raw[0] and derives sc[0], sc[1] (and sc[3]); wave 1 copies the
// bias values into raw[1] and derives sc[2].
struct KeyTerms {
  float sc[4][BN];
  uint32_t raw[2][BN];
};

// At most N vector-memory operations (copies) of this wave outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}
// All LDS operations of this wave done, at most N vector-memory operations
// (and LDS copies) of this wave outstanding, then the workgroup barrier. The
// asm memory clobber keeps the compiler from moving memory accesses across
// it; the (at most N) LDS copies still in flight target stages nobody reads before the
// next barrier.
// sched_barrier(0) on both sides keeps the compiler from moving any
// instruction (arithmetic included) across the barrier.
template <int N>
__device__ __forceinline__ void stage_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" :: "n"(N) : "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Epilogue of one lane's query row: O = O_acc / l * v_scale (RNE to the
// output type) and, for LSE instances, LSE = (m + log2 l) ln 2 + sm_scale*qmu
// (-inf for a row with no attended key, whose O is 0).
template <int D, bool LSE>
__device__ __forceinline__ void store_rows(const AttnArgs& a, const v16f (&o)[D / 32], const float (&lsum)[4],
                                           float m_run, int b, int h, int hk, int q, int64_t qrow, bool qvalid,
                                           int hl) {
  const float l_tot = xsum32((lsum[0] + lsum[1]) + (lsum[2] + lsum[3]));
  if (!qvalid) return;
  const float inv_l = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  const int64_t obase = (int64_t)b * a.o_sb + (int64_t)h * a.o_sh + (int64_t)q * a.o_ss;
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = 32 * c + 8 * g + 4 * hl;
      float vals[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) vals[r] = o[c][4 * g + r] * inv_l;
      if (a.v_scale) {
        const float4 vs = *(const float4*)(a.v_scale + (int64_t)hk * D + d0);   // the V head's scale
        vals[0] *= vs.x; vals[1] *= vs.y; vals[2] *= vs.z; vals[3] *= vs.w;
      }
      if (a.out_dtype == FP32) {
        *(float4*)((float*)a.out + obase + d0) = make_float4(vals[0], vals[1], vals[2], vals[3]);
      } else if (a.out_dtype == BF16) {
        const uint32_t w0 = float_to_bf16_bits(vals[0]) | (float_to_bf16_bits(vals[1]) << 16);
        const uint32_t w1 = float_to_bf16_bits(vals[2]) | (float_to_bf16_bits(vals[3]) << 16);
        *(uint2*)((uint16_t*)a.out + obase + d0) = make_uint2(w0, w1);
      } else {
        const uint32_t w0 = float_to_half_bits(vals[0]) | (float_to_half_bits(vals[1]) << 16);
        const uint32_t w1 = float_to_half_bits(vals[2]) | (float_to_half_bits(vals[3]) << 16);
        *(uint2*)((uint16_t*)a.out + obase + d0) = make_uint2(w0, w1);
      }
    }
  }
  if (LSE && hl == 0) {
    float L = -INFINITY;
    if (l_tot > 0.0f) {
      L = (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
      if (a.qmu) L += a.sm_scale * a.qmu[qrow];
    }
    a.lse[qrow] = L;
  }
}

// LSE is a compile-time trait: the LSE store exists only in the instances
// that return it, so the plain kernels carry no runtime branch for it.
//
// Software pipeline, per 64-key tile j (one barrier per tile). LDS holds
// three stages of K8, V and key terms; at the start of iteration j, K(j+1),
// V(j), the key terms of tile j and the raw terms of tile j+1 are in LDS,
// S(j) is in registers, and the copies of K(j+2) and V(j+1) are in flight.
//   A  dequantize S(j) while the int8 MFMAs of S(j+1) = K8(j+1) Q8^T run;
//      start the copies of K(j+3), V(j+2) and the raw terms of tile j+2;
//      write the key terms of tile j+1 (raw values copied during tile
//      j-1); row max; lazy rescale.
//   B  p = exp2(t - m) one 16-key chunk at a time, packed to V's type, row
//      sum, and the bf16 MFMAs O^T += V^T P^T of that chunk.
//   C  wait for this wave's copies of K(j+2), V(j+1) and the raw terms of
//      tile j+2; barrier.
// Copies past the end of the tile list use empty buffer ranges and write
// zeros, and the MFMAs of a tile past the end run on those zeros, so the
// loop body has no branch besides the rescale.
//
// DUMP instances (dense, whole key range) stop after the int8 MFMAs: they
// store each tile's int32 scores S = Q8 K8^T into `out` (int32 [B,H,Sq,Sk])
// through the same copies, LDS layout, MFMA and seeded accumulators, and
// skip V, the key terms and the softmax. They exist to check those scores
// bit for bit.
//
// CAUSAL instances (dense, one segment [0, Sk), Sq == Sk) stop each block's
// walk at the tile holding its last row's key; the (at most two) tiles that
// cross the block's diagonal run in a loop of their own that sets the scores
// of keys past the row to -inf, so the main loop is the plain one. Blocks
// run heaviest first.
//
// QB instances compute Q K^T on the unquantized bf16/fp16 Q and K (the type
// of V) with the bf16/fp16 MFMA, accumulating from 0 in fp32; the key terms
// are then ks = 1 and 0/-inf, the row factor sm_scale*log2(e), and the rest
// of the tile is the same code. Their K tiles take 2D bytes per row: at
// D = 128 a 3-stage ring (101 KB) would hold one block per CU, whose
// register budget the compiler then fills with AGPRs copied to VGPRs on
// every tile, so these instances use 2 stages (67 KB, two blocks per CU):
// tile j copies K(j+2), V(j+1) and the raw terms of tile j+2, and ends
// waiting for all of them (one tile of lead instead of two).
//
// BIAS2D instances (dense, int8 QK) add a materialised per-(query, key) bias
// or bool keep mask [B|1,H|1,Q,K]: each lane loads its row's 32 values of the
// tile (8 loads of 16 bytes, 4 keys each) at the start of the tile and adds
// them after the dequantization, in natural-log units.
//
// Occupancy: two blocks per CU (two waves per SIMD) everywhere; at D = 64
// the LDS ring (40.5 KB) and most instances (154-167 VGPRs) allow three. The
// causal D = 64 instances need 172-199 VGPRs for their peeled diagonal loop
// unbounded; bounded to three waves per SIMD they fit 168 (a few bytes of
// scratch outside the loops) and run 6-8 % faster. BIAS2D instances at D = 64
// (208-213 VGPRs) stay at two.
template <int D, int VT, int NW, bool SPARSE, bool HAS_BIAS, bool LSE, bool DUMP = false, bool CAUSAL = false,
          bool QB = false, bool BIAS2D = false>
__global__ __launch_bounds__(NW * 64, (D == 64 && CAUSAL && !BIAS2D) ? 3 : 2) void attn_fwd_kernel(AttnArgs a,
                                                                                                  int qtiles,
                                                                                                  int total_blocks) {
  constexpr int BM = 32 * NW;
  constexpr int KC = D / 32;                     // 32-channel blocks of O
  constexpr int NSTG = (QB && D == 128) ? 2 : 3; // LDS stages
  constexpr int KROW = QB ? 2 * D : D;           // bytes per K row in LDS
  constexpr int QSTEPS = QB ? D / 16 : D / 32;   // QK MFMA k-steps (16 bytes of Q per lane each)
  constexpr int K_BYTES = BN * KROW, V_BYTES = BN * 2 * D;
  constexpr int KI = K_BYTES / 1024, VI = V_BYTES / 1024;   // 1 KB copy instructions per tile
  constexpr int KI_W = KI / NW, VI_W = VI / NW;            // ... per wave
  constexpr int K_ROWS_I = 1024 / KROW, V_ROWS_I = 1024 / (2 * D);   // rows per copy instruction
  constexpr int N_COPY_W = KI_W + (DUMP ? 0 : VI_W);      // copy instructions per wave per tile
  static_assert(KI % NW == 0 && VI % NW == 0, "copy split");
  typedef typename std::conditional<VT == BF16, v8bf, v8h>::type pvec;

  __shared__ __attribute__((aligned(1024))) unsigned char kbuf[NSTG][K_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char vbuf[NSTG][V_BYTES];
  __shared__ __attribute__((aligned(16))) KeyTerms kt[NSTG];

  // work unit = (head, split); a split-K call cuts each walk into ns ranges
  const int ns = (SPARSE || DUMP) ? 1 : a.nsplit;
  int bh, qt, split;
  if constexpr (CAUSAL) {
    const int L = causal_order((int)blockIdx.x, total_blocks, a.ncu);
    const int units = total_blocks / qtiles;
    const int unit = L % units;
    qt = qtiles - 1 - L / units;
    bh = unit / ns;
    split = unit % ns;
  } else {
    const int bid = xcd_remap((int)blockIdx.x, total_blocks);
    const int unit = bid / qtiles;
    bh = unit / ns;
    split = unit % ns;
    qt = bid % qtiles;
  }
  const int b = bh / a.H, h = bh % a.H;
  const int tid = threadIdx.x, lane = tid % 64;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int hl = lane / 32;          // k-group of this lane in the MFMA operands
  // key-term row of this wave's additive terms (block-sparse: per query tile)
  const int nks_row = (SPARSE && wave >= 2) ? 3 : 1;
  const int q = qt * BM + wave * 32 + (lane % 32);
  const bool qvalid = q < a.Sq;
  const int64_t qrow = (int64_t)bh * a.Sq + q;

  // ---- tile lists (scalar loads: the lists are read-only here) ----
  // A block-sparse block covers the query tiles 2qt (waves 0, 1) and 2qt+1
  // (waves 2, 3) and walks the union of their key-tile lists, so the two
  // share every K8/V copy; a tile only one of them attends carries -inf
  // terms for the other.
  const __attribute__((address_space(4))) int32_t* list_a = nullptr;
  const __attribute__((address_space(4))) int32_t* list_b = nullptr;
  int ntk = 0, n_tiles, na = 0, nb = 0, ia = 0, ib = 0;
  int it0 = 0;   // walk position of this block's first tile (split-K: its range start)
  if constexpr (SPARSE) {
    ntk = a.Sk / BN;
    const int qa = 2 * qt, qb = 2 * qt + 1;
    const __attribute__((address_space(4))) int32_t* cnt = (const __attribute__((address_space(4))) int32_t*)a.count;
    list_a = (const __attribute__((address_space(4))) int32_t*)(a.index + ((int64_t)bh * ntk + qa) * ntk);
    list_b = qb < ntk ? list_a + ntk : list_a;
    na = min(max(cnt[(int64_t)bh * ntk + qa], 0), ntk);
    nb = qb < ntk ? min(max(cnt[(int64_t)bh * ntk + qb], 0), ntk) : 0;
    n_tiles = INT32_MAX;   // the length of the union, known once the walk reaches its end
  } else {
    n_tiles = a.seg_ntiles;
    if constexpr (CAUSAL) n_tiles = min(n_tiles, (min(a.Sk, qt * BM + BM) + BN - 1) / BN);
    // split-K: walk positions [it0, n_tiles) of the whole walk (ns * walk < 2^31)
    it0 = split * n_tiles / ns;
    n_tiles = (split + 1) * n_tiles / ns;
  }
  const __attribute__((address_space(4))) int32_t* vbs = (const __attribute__((address_space(4))) int32_t*)a.vbs;
  // The key tiles of this block in loop order, one per call: the tile, the
  // key range [lo, hi) attended inside it, and `valid`: 0 past the end of
  // the walk, else bit 0 set, plus (block-sparse) bit 1 when query tile 2qt
  // attends it and bit 2 when 2qt+1 does. Dense calls step a cursor and read
  // the segment tables only when a segment ends. Block-sparse calls merge
  // the two ascending lists (entries are clamped into [0, ntk); lists that
  // are not strictly ascending give unspecified results but stay in bounds,
  // and the walk ends after at most na + nb steps). Wave-uniform throughout.
  int cur_it = it0 - 1, cur_tile = -1, cur_slo = 0, cur_shi = 0;
  auto next_tile = [&](int& tile, int& lo, int& hi, int& valid) __attribute__((always_inline)) {
    ++cur_it;
    if constexpr (SPARSE) {
      const int ta = ia < na ? min(max(list_a[ia], 0), ntk - 1) : INT32_MAX;
      const int tb = ib < nb ? min(max(list_b[ib], 0), ntk - 1) : INT32_MAX;
      const int t = min(ta, tb);
      if (t == INT32_MAX) {
        n_tiles = min(n_tiles, cur_it);
        tile = 0;
        lo = hi = 0;
        valid = 0;
      } else {
        valid = 1 | (ta == t ? 2 : 0) | (tb == t ? 4 : 0);
        ia += ta == t ? 1 : 0;
        ib += tb == t ? 1 : 0;
        tile = t;
        lo = t * BN;
        hi = lo + (vbs ? min(max(vbs[t], 0), BN) : BN);
      }
    } else {
      valid = cur_it < n_tiles ? 1 : 0;
      ++cur_tile;
      if (cur_tile * BN >= cur_shi) seg_at(a, cur_it, cur_tile, cur_slo, cur_shi);
      tile = cur_tile;
      lo = max(cur_slo, cur_tile * BN);
      hi = valid ? min(cur_shi, cur_tile * BN + BN) : lo;
    }
  };

  // ---- Q codes (QB: Q values) of this lane's row: kept in VGPRs for the
  // whole key loop; 16 bytes per QK k-step ----
  v4i qreg[QSTEPS];
  const uint16_t* qsrc = QB ? (const uint16_t*)a.qf + ((int64_t)b * a.q_sb + (int64_t)h * a.q_sh + (int64_t)q * a.q_ss)
                            : nullptr;
#pragma unroll
  for (int c = 0; c < QSTEPS; ++c) {
    if (!qvalid) qreg[c] = v4i{0, 0, 0, 0};
    else if (QB) qreg[c] = *(const v4i*)(qsrc + 16 * c + 8 * hl);
    else qreg[c] = *(const v4i*)(a.q8 + qrow * D + 32 * c + 16 * hl);
  }
  // row factor of the log2-domain logits; kept above zero so that an
  // excluded key (-inf) stays -inf when scaled (a zero row's logits are 0
  // either way)
  const float crow = DUMP ? 1.0f
                          : (QB ? a.sm_scale * kLog2e
                                : fmaxf(qvalid ? a.qs[qrow] * (a.sm_scale * kLog2e) : 0.0f, 1e-30f));

  // ---- per-(b,h) sources; every copy and load is range-checked. K8, key
  // scales and V come from the K/V head of this query head (grouped-query
  // calls share one among H / Hkv consecutive query heads) ----
  const int hk = h / (a.H / a.Hkv);
  const int64_t bhk = (int64_t)b * a.Hkv + hk;
  const unsigned char* kbase =
      QB ? (const unsigned char*)a.kf + ((int64_t)b * a.k_sb + (int64_t)hk * a.k_sh) * 2
         : (const unsigned char*)(a.k8 + bhk * a.Sk * D);
  const int k_row = QB ? (int)(a.k_ss * 2) : D;   // source bytes per K row (below 2^25, checked by the caller)
  const unsigned char* vbase = (const unsigned char*)a.v + ((int64_t)b * a.v_sb + (int64_t)hk * a.v_sh) * 2;
  const int v_row = (int)(a.v_ss * 2);   // below 2^25 (checked by the caller)
  const float* ksbase = QB ? nullptr : a.ks + bhk * a.Sk;
  const int64_t bias_off = (int64_t)b * a.bias_sb + (int64_t)h * a.bias_sh;
  const int bias_esz = a.bias_dtype == FP32 ? 4 : 2;
  // BIAS2D: one buffer descriptor over this wave's 32 rows of the bias (rows
  // past Sq read zero); the lane's row starts b2_row bytes in; the
  // natural-log row factor qs*sm_scale. A buffer load returns zero for every
  // dword not wholly inside the range, so the range ends at the dword that
  // holds the last row's key Sk - 1 (4-byte aligned, as rows start on
  // 16-byte boundaries, so it never leaves the page of a valid byte); the
  // bytes of keys past Sk are forced out in the tile that holds them
  const int b2_esz = a.bias_dtype == FP32 ? 4 : (a.bias_dtype == BOOL ? 1 : 2);
  v4u b2_desc = {0u, 0u, 0u, 0u};
  int b2_row = 0;
  float crow_nat = 0.0f;
  if constexpr (BIAS2D) {
    const int q0 = qt * BM + wave * 32;
    const int nrow = max(0, min(32, a.Sq - q0));
    const int64_t tail = ((int64_t)a.Sk * b2_esz + 3) & ~(int64_t)3;
    b2_desc = buf_desc32((const unsigned char*)a.bias + (bias_off + (int64_t)q0 * a.bias_sq) * b2_esz,
                         nrow > 0 ? (int)((int64_t)(nrow - 1) * a.bias_sq * b2_esz + tail) : 0);
    b2_row = (lane % 32) * (int)a.bias_sq * b2_esz;   // below 2^31 (checked by the caller)
    crow_nat = fmaxf(qvalid ? a.qs[qrow] * a.sm_scale : 0.0f, 1e-30f);
  }
  // unbiased instances take a [1,1,1,K] keep mask (bool bytes) through the
  // key terms: a masked key is excluded like a segment edge, at no per-score cost
  const int keep_mask = (!HAS_BIAS && !BIAS2D && !SPARSE && !DUMP && a.bias != nullptr) ? 1 : 0;

  // per-lane source offsets of this wave's copy instructions (tile-relative)
  int k_src[KI_W], v_src[VI_W];
#pragma unroll
  for (int i = 0; i < KI_W; ++i) {
    const int ins = wave + i * NW;
    const int row = ins * K_ROWS_I + lane / (KROW / 16), pos = lane % (KROW / 16);
    // LDS chunk `pos` of this row holds source chunk c with k_chunk_pos(row, c) == pos
    k_src[i] = row * k_row + k_chunk_pos<KROW>(row, pos) * 16;
  }
#pragma unroll
  for (int i = 0; i < VI_W; ++i) {
    const int ins = wave + i * NW;
    const int row = ins * V_ROWS_I + lane / (D / 8), pos = lane % (D / 8);
    v_src[i] = row * v_row + v_chunk_pos<D>(row, pos) * 16;
  }

  // K8 / V rows of a tile into a stage (zeros when `valid` is false; rows
  // past Sk read zero). The descriptor covers the tile's rows only, so its
  // size is a 32-bit scalar computation.
  auto copy_k = [&](int stage, int tile, int valid) __attribute__((always_inline)) {
    const int key0 = tile * BN;
    const int rows = valid ? min(BN, a.Sk - key0) : 0;
    const v4u d = buf_desc32(kbase + (int64_t)key0 * k_row, rows > 0 ? (rows - 1) * k_row + KROW : 0);
#pragma unroll
    for (int i = 0; i < KI_W; ++i) lds_copy<16>(lds_addr(&kbuf[stage][(wave + i * NW) * 1024]), k_src[i], d);
  };
  // V rows past the tile's walked range (past a segment's end, pad keys of
  // block-sparse tiles, rows past Sk) read zero: the range ends at row hi and
  // an out-of-range lane of a copy writes zeros to LDS, so a non-finite V row
  // of such a key never meets its zero weight in the PV product. (Rows before
  // lo, where a segment starts inside the tile, are read.)
  auto copy_v = [&](int stage, int tile, int hi, int valid) __attribute__((always_inline)) {
    if constexpr (DUMP) return;
    const int key0 = tile * BN;
    const int rows = valid ? hi - key0 : 0;
    const v4u d = buf_desc32(vbase + (int64_t)key0 * v_row, rows > 0 ? (rows - 1) * v_row + 2 * D : 0);
#pragma unroll
    for (int i = 0; i < VI_W; ++i) lds_copy<16>(lds_addr(&vbuf[stage][(wave + i * NW) * 1024]), v_src[i], d);
  };
  // raw key terms of a tile: wave 0 copies the key scales of keys
  // key0 + lane, wave 1 the bias values, or (unbiased kernel with a keep
  // mask) the mask bytes (range [lo, hi): keys outside it read zero and are
  // excluded when the terms are derived)
  auto copy_terms = [&](int stage, int tile, int lo, int hi, int valid) __attribute__((always_inline)) {
    if constexpr (DUMP) return;
    const int nk = valid ? hi - lo : 0;
    const int rel = tile * BN + lane - lo;   // negative offsets wrap and read as out of range
    if (wave == 0) {
      if (!QB) lds_copy<4>(lds_addr(&kt[stage].raw[0][0]), rel * 4, buf_desc32(ksbase + lo, nk * 4));
    } else if (HAS_BIAS && wave == 1) {
      const v4u d = buf_desc32((const unsigned char*)a.bias + (bias_off + lo) * bias_esz, nk * bias_esz);
      if (bias_esz == 4) lds_copy<4>(lds_addr(&kt[stage].raw[1][0]), rel * 4, d);
      else lds_copy<2>(lds_addr(&kt[stage].raw[1][0]), rel * 2, d);
    } else if (!HAS_BIAS && keep_mask && wave == 1) {
      lds_copy<1>(lds_addr(&kt[stage].raw[1][0]), rel, buf_desc32((const unsigned char*)a.bias + bias_off + lo, nk));
    }
  };
  // derive the terms of a tile from its copied raw values (the calling
  // wave's own copy must have landed)
  // (block-sparse: sc[1] holds the terms of query tile 2qt, sc[3] those of
  // 2qt+1, which differ in the tiles only one of them attends)
  auto derive_terms = [&](int stage, int tile, int lo, int hi, int flags) __attribute__((always_inline)) {
    if constexpr (DUMP) return;
    const int key = tile * BN + lane;
    const bool in = key >= lo && key < hi;
    if (wave == 0) {
      // QB: unscaled fp32 scores, ks = 1 and no accumulator seed
      const float ks = QB ? 1.0f : (in ? __uint_as_float(kt[stage].raw[0][lane]) : 0.0f);
      const float seed = QB ? 0.0f : -kMagic * ks;
      kt[stage].sc[0][lane] = ks;
      // an excluded key dequantizes to fma(x, ks, -inf) = -inf; a keep mask
      // (copied by wave 1) excludes its zero entries the same way
      const bool keep = HAS_BIAS || !keep_mask || kt[stage].raw[1][lane] != 0u;
      const bool in_a = in && keep && (!SPARSE || (flags & 2));
      kt[stage].sc[1][lane] = in_a ? seed : -INFINITY;
      if (SPARSE) kt[stage].sc[3][lane] = in && (flags & 4) ? seed : -INFINITY;
    } else if (HAS_BIAS && wave == 1) {
      const uint32_t r = kt[stage].raw[1][lane];
      const float bias = a.bias_dtype == FP32 ? __uint_as_float(r)
                                              : (a.bias_dtype == BF16 ? bf16_bits_to_float(r) : half_bits_to_float(r));
      kt[stage].sc[2][lane] = bias * kLog2e;
    }
  };

  // ---- online softmax state (log2 domain) ----
  v16f o[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) o[c] = v16f{};
  float m_run = -INFINITY;
  float lsum[4] = {0.0f, 0.0f, 0.0f, 0.0f};

  // operand addressing
  const int grp = lane / 16, sl = lane % 16;
  const int tr_row = 4 * hl + sl / 4;                     // ds_read_b64_tr_b16 source row (+ tile row base)
  const int tr_byte = 2 * (16 * (grp % 2) + 4 * (sl % 4));  // ... and byte inside a 64-byte channel block

  // S^T = K8 Q8^T of one 32-key block; accumulators start at kMagicBits
  // (QB: S^T = K Q^T in fp32 from 0, its bits held in the same registers)
  v16i s[2];
  auto qk_block = [&](int stage, int blk) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s[blk][r] = QB ? 0 : kMagicBits;
    const int row = 32 * blk + lane % 32;
#pragma unroll
    for (int c = 0; c < QSTEPS; ++c) {
      const v4i kv = *(const v4i*)(&kbuf[stage][row * KROW + k_chunk_pos<KROW>(row, 2 * c + hl) * 16]);
      if constexpr (!QB) {
        s[blk] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kv, qreg[c], s[blk], 0, 0, 0);
      } else if constexpr (VT == BF16) {
        s[blk] = __builtin_bit_cast(v16i, __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(v8bf, kv), __builtin_bit_cast(v8bf, qreg[c]), __builtin_bit_cast(v16f, s[blk]), 0, 0, 0));
      } else {
        s[blk] = __builtin_bit_cast(v16i, __builtin_amdgcn_mfma_f32_32x32x16_f16(
            __builtin_bit_cast(v8h, kv), __builtin_bit_cast(v8h, qreg[c]), __builtin_bit_cast(v16f, s[blk]), 0, 0, 0));
      }
    }
  };

  // ---- prologue: K(0), K(1), V(0), the terms of tile 0 and the raw terms of
  // tile 1 in LDS; S(0) ----
  int t0c;              // tile of the current iteration
  int t1, l1, h1, v1;   // tiles iter+1 and iter+2 of the loop below
  int t2, l2, h2, v2;   // (v: inside the walk)
  {
    int t0, l0, h0, v0;
    next_tile(t0, l0, h0, v0);
    t0c = t0;
    next_tile(t1, l1, h1, v1);
    copy_terms(0, t0, l0, h0, v0);
    copy_terms(1, t1, l1, h1, v1);
    copy_k(0, t0, v0);
    copy_v(0, t0, h0, v0);
    copy_k(1, t1, v1);
    wait_vmcnt<0>();
    // the keep-mask bytes wave 0 folds in were copied by wave 1
    if (keep_mask) stage_barrier<0>();
    derive_terms(0, t0, l0, h0, v0);
    stage_barrier<0>();
    qk_block(0, 0);
    qk_block(0, 1);
    // every wave's reads of K(0) are done before stage 0 is refilled
    stage_barrier<0>();
    next_tile(t2, l2, h2, v2);
    if constexpr (NSTG == 3) {
      copy_k(2, t2, v2);
      copy_v(1, t1, h1, v1);
    }
  }

  // One tile. Excluded keys (segment edges, pad keys of block-sparse tiles)
  // carry -inf in their key terms, so every tile runs the same code.
  // `diag` (a literal at each call): the tile may hold keys past some row
  auto tile_body = [&](int iter, int st0, int st1, int st2, bool diag) __attribute__((always_inline)) {
    // st0 = iter % NSTG, st1 = (iter + 1) % NSTG, st2 = (iter + 2) % NSTG
    const KeyTerms& tc = kt[st0];
    // BIAS2D: this tile's 32 bias values of the lane's row, 4 keys per load
    // (keys 32 blk + 8 g + 4 hl + [0, 4) for load blk*4 + g), issued before
    // the tile's copies; each block's four are waited for and added right
    // after that block's dequantization (asm keeps the compiler from
    // draining every copy before their first use)
    v4u braw[8];
    if constexpr (BIAS2D) {
      const int kb = b2_row + (t0c * BN + 4 * hl) * b2_esz;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int off = kb + (32 * (i / 4) + 8 * (i % 4)) * b2_esz;
        asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen" : "=v"(braw[i]) : "v"(off), "s"(b2_desc) : "memory");
      }
    }
    int t3, l3, h3, v3;
    next_tile(t3, l3, h3, v3);
    copy_terms(st2, t2, l2, h2, v2);
    // terms of tile iter+1 from the raw values copied during the previous
    // tile (first read after this tile's barrier)
    derive_terms(st1, t1, l1, h1, v1);

    if constexpr (DUMP) {
      // S(iter) out (int32 [B,H,Sq,Sk]), S(iter+1) MFMAs, K copy, barrier;
      // the walk of a score dump is the single segment [0, Sk), unsplit
      const int tile = iter, lo = iter * BN, hi = min(a.Sk, lo + BN);
      int32_t* srow = (int32_t*)a.out + qrow * a.Sk;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = tile * BN + 32 * blk + 8 * g + 4 * hl + r;
            if (qvalid && key >= lo && key < hi) srow[key] = s[blk][4 * g + r] - kMagicBits;
          }
        qk_block(st1, blk);
      }
      copy_k(st0, t3, v3);
      wait_vmcnt<N_COPY_W>();
      stage_barrier<N_COPY_W>();
      t1 = t2;
      v1 = v2;
      t2 = t3;
      v2 = v3;
      return;
    }

    // ===== A: dequantize S(iter); S(iter+1) MFMAs; copies; row max =====
    // unbiased: t = S*ks, crow is applied in the exponent; biased:
    // t = S*ks*crow + lb (excluded keys: -inf either way)
    float t[2][16];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int kk = 32 * blk + 8 * g + 4 * hl;
        const float4 kv = *(const float4*)(&tc.sc[0][kk]);
        const float4 nv = *(const float4*)(&tc.sc[nks_row][kk]);
        const float kvs[4] = {kv.x, kv.y, kv.z, kv.w};
        const float nvs[4] = {nv.x, nv.y, nv.z, nv.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) t[blk][4 * g + r] = fmaf(__int_as_float(s[blk][4 * g + r]), kvs[r], nvs[r]);
        if (HAS_BIAS) {
          const float4 bv = *(const float4*)(&tc.sc[2][kk]);
          const float bvs[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) t[blk][4 * g + r] = fmaf(t[blk][4 * g + r], crow, bvs[r]);
        }
      }
      if constexpr (BIAS2D) {
        // block 0: at most loads 4..7 and the key-scale copy of wave 0 are
        // newer; block 1: at most this tile's K copies. The registers are
        // operands of the wait, so no read of them moves above it.
        if (blk == 0) {
          asm volatile("s_waitcnt vmcnt(4)" : "+v"(braw[0]), "+v"(braw[1]), "+v"(braw[2]), "+v"(braw[3]) :: "memory");
        } else {
          asm volatile("s_waitcnt vmcnt(%4)" : "+v"(braw[4]), "+v"(braw[5]), "+v"(braw[6]), "+v"(braw[7])
                       : "n"(KI_W) : "memory");
        }
        // t = S*ks*qs*sm_scale + bias (natural log; excluded keys stay -inf)
        auto apply = [&](auto decode) __attribute__((always_inline)) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            float bv[4];
            decode(braw[4 * blk + g], bv);
#pragma unroll
            for (int r = 0; r < 4; ++r) t[blk][4 * g + r] = fmaf(t[blk][4 * g + r], crow_nat, bv[r]);
          }
        };
        if (a.bias_dtype == FP32) {
          apply([](const v4u& w, float (&bv)[4]) {
            bv[0] = __uint_as_float(w.x); bv[1] = __uint_as_float(w.y);
            bv[2] = __uint_as_float(w.z); bv[3] = __uint_as_float(w.w);
          });
        } else if (a.bias_dtype == BOOL) {
          apply([](const v4u& w, float (&bv)[4]) {
#pragma unroll
            for (int r = 0; r < 4; ++r) bv[r] = ((w.x >> (8 * r)) & 0xffu) ? 0.0f : -INFINITY;
          });
        } else if (a.bias_dtype == BF16) {
          apply([](const v4u& w, float (&bv)[4]) {
            bv[0] = bf16_bits_to_float(w.x & 0xffffu); bv[1] = bf16_bits_to_float(w.x >> 16);
            bv[2] = bf16_bits_to_float(w.y & 0xffffu); bv[3] = bf16_bits_to_float(w.y >> 16);
          });
        } else {
          apply([](const v4u& w, float (&bv)[4]) {
            bv[0] = half_bits_to_float(w.x & 0xffffu); bv[1] = half_bits_to_float(w.x >> 16);
            bv[2] = half_bits_to_float(w.y & 0xffffu); bv[3] = half_bits_to_float(w.y >> 16);
          });
        }
      }
      qk_block(st1, blk);   // the score registers of this block are free again
      if (blk == 0) {
        if constexpr (NSTG == 3) copy_k(st0, t3, v3);   // K(iter+3) over K(iter)
        else copy_k(st0, t2, v2);                       // K(iter+2) over K(iter)
      }
    }
    if constexpr (NSTG == 3) copy_v(st2, t2, h2, v2);       // V(iter+2) over V(iter-1)
    else copy_v(st1, t1, h1, v1);                           // V(iter+1) over V(iter-1)
    if constexpr (BIAS2D) {
      // keys past Sk (only in the tile that holds key Sk - 1) read row
      // padding or the next row: excluded by their key terms, but a NaN or
      // +inf there would make fma(-inf, c, bias) NaN. A bool byte decodes
      // to 0 or -inf, so the keep-mask form needs nothing.
      const int key0 = t0c * BN;
      if (key0 + BN > a.Sk && a.bias_dtype != BOOL) {
        const int lim = a.Sk - 1 - key0;   // last key of the row, tile-relative
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (32 * blk + 8 * g + 4 * hl + r > lim) t[blk][4 * g + r] = -INFINITY;
      }
    }
    if (CAUSAL && diag) {
      // the walk is the single segment [0, Sk), so tile it0 + iter holds keys
      // (it0 + iter)*BN + [0, BN); only waves whose first row lies before the
      // tile's last key see a key past their row
      const int key0 = (it0 + iter) * BN;
      if (qt * BM + wave * 32 < key0 + BN - 1) {
        const int lim = q - key0;   // last attended key of this row, tile-relative
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (32 * blk + 8 * g + 4 * hl + r > lim) t[blk][4 * g + r] = -INFINITY;
      }
    }
    // crow > 0, so max(u)*crow = max(u*crow) (also for -inf); BIAS2D: t is
    // in natural-log units
    const float mx = HAS_BIAS ? xmax32(max32(t)) : xmax32(max32(t)) * (BIAS2D ? kLog2e : crow);

    // ---- lazy rescale: only when a row max passes the reference by the slack ----
    if (__builtin_expect(__any(mx > m_run + kRescaleSlack), 0)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int i = 0; i < 4; ++i) lsum[i] *= alpha;
#pragma unroll
      for (int c = 0; c < KC; ++c) o[c] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == -INFINITY) ? 0.0f : m_run;

    // ===== B: p = exp2(t - m) chunk by chunk, row sum, PV MFMAs =====
    const unsigned char* vcur = vbuf[st0];
#pragma unroll
    for (int chunk = 0; chunk < 4; ++chunk) {
      const int blk = chunk / 2, m = chunk % 2;
      uint32_t pw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x0, x1;
        if (HAS_BIAS) {
          x0 = t[blk][8 * m + 2 * e] - m_use;
          x1 = t[blk][8 * m + 2 * e + 1] - m_use;
        } else if (BIAS2D) {
          x0 = fmaf(t[blk][8 * m + 2 * e], kLog2e, -m_use);
          x1 = fmaf(t[blk][8 * m + 2 * e + 1], kLog2e, -m_use);
        } else {
          x0 = fmaf(t[blk][8 * m + 2 * e], crow, -m_use);
          x1 = fmaf(t[blk][8 * m + 2 * e + 1], crow, -m_use);
        }
        const float p0 = __builtin_amdgcn_exp2f(x0);
        const float p1 = __builtin_amdgcn_exp2f(x1);
        if constexpr (VT == BF16) {
          const v2bf pair = {(__bf16)p0, (__bf16)p1};
          pw[e] = __builtin_bit_cast(uint32_t, pair);
          // with an LSE the row sum takes the fp32 values (a sum of rounded
          // p would carry up to 2^-9 relative error into the LSE when one key
          // dominates); without one it sums the rounded weights PV uses, so
          // the output is their exact weighted mean
          if (LSE) lsum[e] += p0 + p1;
          else lsum[e] = __builtin_amdgcn_fdot2_f32_bf16(pair, v2bf{(__bf16)1.0f, (__bf16)1.0f}, lsum[e], false);
        } else {
          const v2h pair = {(_Float16)p0, (_Float16)p1};
          pw[e] = __builtin_bit_cast(uint32_t, pair);
          if (LSE) lsum[e] += p0 + p1;
          else lsum[e] = __builtin_amdgcn_fdot2(pair, v2h{(_Float16)1.0f, (_Float16)1.0f}, lsum[e], false);
        }
      }
      const pvec pb = __builtin_bit_cast(pvec, pw);
      const int row0 = 32 * blk + 16 * m + tr_row;   // and row0 + 8
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        const int byte = 64 * c + tr_byte;
        const int a0 = row0 * (2 * D) + v_chunk_pos<D>(row0, byte / 16) * 16 + byte % 16;
        const int a1 = (row0 + 8) * (2 * D) + v_chunk_pos<D>(row0 + 8, byte / 16) * 16 + byte % 16;
        const v4s lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(vcur + a0));
        const v4s hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(vcur + a1));
        const v4s both[2] = {lo4, hi4};
        if constexpr (VT == BF16) {
          const v8bf av = __builtin_bit_cast(v8bf, both);
          o[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb, o[c], 0, 0, 0);
        } else {
          const v8h av = __builtin_bit_cast(v8h, both);
          o[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, pb, o[c], 0, 0, 0);
        }
      }
    }

    // ===== C: this wave's copies older than this tile's K/V copies are done
    // (2 stages: all of them); barrier =====
    constexpr int kLag = NSTG == 3 ? N_COPY_W : 0;
    wait_vmcnt<kLag>();
    stage_barrier<kLag>();
    t0c = t1;
    t1 = t2;
    l1 = l2;
    h1 = h2;
    v1 = v2;
    t2 = t3;
    l2 = l3;
    h2 = h3;
    v2 = v3;
  };

  // causal: tiles [0, n_plain) hold no key past the block's first row and
  // run the plain body; the (at most two) tiles across the diagonal run a
  // copy with the mask, so the main loop carries none of its code. Other
  // instances test n_tiles itself on every pass: a block-sparse walk sets
  // it (from INT32_MAX) only when its lists run out.
  // (loop counts are relative to it0; n_tiles is a walk position)
  const int n_plain = CAUSAL ? max(0, min(n_tiles, (qt * BM + 1) / BN) - it0) : 0;
  int st0 = 0, st1 = 1, st2 = 2 % NSTG;
  auto rotate = [&]() __attribute__((always_inline)) {
    const int tmp = st0;
    st0 = st1;
    st1 = NSTG == 3 ? st2 : tmp;
    st2 = NSTG == 3 ? tmp : st0;
  };
  int iter = 0;
  for (; iter < (CAUSAL ? n_plain : n_tiles - it0); ++iter) {
    tile_body(iter, st0, st1, st2, false);
    rotate();
  }
  if constexpr (CAUSAL) {
    for (; iter < n_tiles - it0; ++iter) {
      tile_body(iter, st0, st1, st2, true);
      rotate();
    }
  }
  // drain this wave's remaining copies (they target stages nobody reads)
  wait_vmcnt<0>();

  if constexpr (!DUMP) {
    if (LSE && ns > 1) {
      // split-K partial: normalised fp32 O and its LSE into this split's slice
      const int64_t rows = (int64_t)a.B * a.H * a.Sq;
      AttnArgs p = a;
      p.out = a.part_o + split * rows * D;
      p.out_dtype = FP32;
      p.o_sb = (int64_t)a.H * a.Sq * D;
      p.o_sh = (int64_t)a.Sq * D;
      p.o_ss = D;
      p.lse = a.part_lse + split * rows;
      store_rows<D, LSE>(p, o, lsum, m_run, b, h, hk, q, qrow, qvalid, hl);
    } else {
      store_rows<D, LSE>(a, o, lsum, m_run, b, h, hk, q, qrow, qvalid, hl);
    }
  }
}


template <int D, int VT, bool QB>
hipError_t launch_d_vt(const AttnArgs& a, hipStream_t s) {
  const bool sparse = a.index != nullptr;
  const int qtiles = (a.Sq + 127) / 128;   // 128 query rows (two 64-query tiles) per block
  const int ns = sparse ? 1 : a.nsplit;    // split-K ranges per walk (dense calls)
  const int total = qtiles * a.B * a.H * ns;
  if (total == 0) return hipSuccess;
  // split partials always carry their LSE
  const bool lse = a.lse != nullptr || ns > 1;
  constexpr bool F = false, T = true;
  if (debug_enabled()) {
    const bool bias2d = !QB && !sparse && a.bias && a.bias_sq != 0;
    const bool keyterm_bias = !sparse && !bias2d && a.bias && a.bias_dtype != BOOL;
    const bool keep = !sparse && !bias2d && a.bias && a.bias_dtype == BOOL;
    debug_log("attn_fwd_kernel<D=%d, V=%s, sparse=%d, bias=%d, lse=%d, causal=%d, qk=%s, bias2d=%d> keep_mask=%d "
              "grid %d x 256 (query blocks %d, B*H %d, splits %d) Sq %d Sk %d segments %d out %s",
              D, VT == BF16 ? "bf16" : "fp16", (int)sparse, (int)keyterm_bias, (int)lse, a.causal, QB ? "bf16/fp16" : "int8",
              (int)bias2d, (int)keep, total, qtiles, a.B * a.H, ns, a.Sq, a.Sk, a.nseg,
              a.out_dtype == FP32 ? "fp32" : (a.out_dtype == BF16 ? "bf16" : "fp16"));
  }
  if (!QB && !sparse && a.bias && a.bias_sq != 0) {
    // materialised [B|1,H|1,Q,K] bias or keep mask
    if (a.causal) {
      if (lse) attn_fwd_kernel<D, VT, 4, F, F, T, F, T, F, T><<<total, 256, 0, s>>>(a, qtiles, total);
      else attn_fwd_kernel<D, VT, 4, F, F, F, F, T, F, T><<<total, 256, 0, s>>>(a, qtiles, total);
    } else {
      if (lse) attn_fwd_kernel<D, VT, 4, F, F, T, F, F, F, T><<<total, 256, 0, s>>>(a, qtiles, total);
      else attn_fwd_kernel<D, VT, 4, F, F, F, F, F, F, T><<<total, 256, 0, s>>>(a, qtiles, total);
    }
  } else if (sparse) {
    if (lse) attn_fwd_kernel<D, VT, 4, T, F, T, F, F, QB><<<total, 256, 0, s>>>(a, qtiles, total);
    else attn_fwd_kernel<D, VT, 4, T, F, F, F, F, QB><<<total, 256, 0, s>>>(a, qtiles, total);
  } else if (a.causal) {
    // a keep mask (bool bias) runs in the unbiased instance (block order: causal_order)
    if (a.bias && a.bias_dtype != BOOL) {
      if (lse) attn_fwd_kernel<D, VT, 4, F, T, T, F, T, QB><<<total, 256, 0, s>>>(a, qtiles, total);
      else attn_fwd_kernel<D, VT, 4, F, T, F, F, T, QB><<<total, 256, 0, s>>>(a, qtiles, total);
    } else {
      if (lse) attn_fwd_kernel<D, VT, 4, F, F, T, F, T, QB><<<total, 256, 0, s>>>(a, qtiles, total);
      else attn_fwd_kernel<D, VT, 4, F, F, F, F, T, QB><<<total, 256, 0, s>>>(a, qtiles, total);
    }
  } else if (a.bias && a.bias_dtype != BOOL) {
    if (lse) attn_fwd_kernel<D, VT, 4, F, T, T, F, F, QB><<<total, 256, 0, s>>>(a, qtiles, total);
    else attn_fwd_kernel<D, VT, 4, F, T, F, F, F, QB><<<total, 256, 0, s>>>(a, qtiles, total);
  } else {
    if (lse) attn_fwd_kernel<D, VT, 4, F, F, T, F, F, QB><<<total, 256, 0, s>>>(a, qtiles, total);
    else attn_fwd_kernel<D, VT, 4, F, F, F, F, F, QB><<<total, 256, 0, s>>>(a, qtiles, total);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || ns == 1) return e;
  CombineArgs c{a.B, a.H, a.Sq, D, ns, a.part_o, a.part_lse, a.out, a.out_dtype, a.o_sb, a.o_sh, a.o_ss, a.lse};
  return launch_split_combine(c, s);
}

template <int D, int VT>
hipError_t launch_d_vt(const AttnArgs& a, hipStream_t s) {
  return a.qf ? launch_d_vt<D, VT, true>(a, s) : launch_d_vt<D, VT, false>(a, s);
}

template <int D>
hipError_t launch_qk_dump_d(const AttnArgs& a, hipStream_t s) {
  const int qtiles = (a.Sq + 127) / 128;
  const int total = qtiles * a.B * a.H;
  if (total == 0) return hipSuccess;
  debug_log("attn_fwd_kernel<D=%d, score dump> grid %d x 256 Sq %d Sk %d", D, total, a.Sq, a.Sk);
  attn_fwd_kernel<D, BF16, 4, false, false, false, true><<<total, 256, 0, s>>>(a, qtiles, total);
  return hipGetLastError();
}

}  // namespace
}  // namespace qfa
