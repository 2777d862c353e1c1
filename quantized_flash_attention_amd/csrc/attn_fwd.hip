// INT8-QK / BF16-PV flash attention forward for gfx950 (CDNA4).
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
//   block  = BM = 32*NW query rows of one (b,h); NW = 4 dense, 2 block-sparse
//            (a 64-query tile, the unit of the tile mask).
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
//   keys   = 64 per tile. K8/V tiles are staged global -> VGPR (prefetch of
//            the next tile while the current one is computed) -> LDS.
//   grid   = 1-D, remapped so that the blocks one XCD runs cover whole heads
//            (consecutive block ids are dealt round-robin to the 8 XCDs);
//            blocks sharing K/V then share that XCD's L2.
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

__device__ __forceinline__ float load_bias(const void* p, int dtype, int64_t idx) {
  if (dtype == FP32) return ((const float*)p)[idx];
  const uint32_t h = ((const uint16_t*)p)[idx];
  return dtype == BF16 ? bf16_bits_to_float(h) : half_bits_to_float(h);
}

// Key-tile iteration: either the tiles covering up to 4 key segments, or the
// key-tile list of this query tile (block-sparse). Every field is uniform
// across the block; plain scalars (no arrays) keep them in SGPRs.
struct TileIter {
  int n;                                  // number of tiles
  int t0_0, t0_1, t0_2, t0_3;             // first tile of each segment
  int n_0, n_1, n_2;                      // tiles of segments 0..2 (segment 3 takes the rest)
  int lo_0, lo_1, lo_2, lo_3, hi_0, hi_1, hi_2, hi_3;
  const int32_t* list;                    // sparse: key tiles
  const int32_t* vbs;                     // sparse: valid counts (nullable)
  int ntiles_k;                           // sparse: number of key tiles

  // tile index and the valid key range [lo, hi) inside it (absolute keys).
  // A listed tile outside [0, ntiles_k) is treated as an empty tile.
  __device__ __forceinline__ void get(int it, int& tile, int& lo, int& hi) const {
    if (list) {
      tile = __builtin_amdgcn_readfirstlane(list[it]);
      if (tile < 0 || tile >= ntiles_k) {
        tile = 0;
        lo = hi = 0;
        return;
      }
      lo = tile * BN;
      hi = lo + (vbs ? min(max(__builtin_amdgcn_readfirstlane(vbs[tile]), 0), BN) : BN);
      return;
    }
    int t0, slo, shi;
    if (it < n_0) {
      t0 = t0_0; slo = lo_0; shi = hi_0;
    } else if ((it -= n_0) < n_1) {
      t0 = t0_1; slo = lo_1; shi = hi_1;
    } else if ((it -= n_1) < n_2) {
      t0 = t0_2; slo = lo_2; shi = hi_2;
    } else {
      it -= n_2;
      t0 = t0_3; slo = lo_3; shi = hi_3;
    }
    tile = t0 + it;
    lo = max(slo, tile * BN);
    hi = min(shi, tile * BN + BN);
  }
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes <= 0 ? 0 : (bytes >= 0x7fffffff ? 0x7fffffff : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

// 16-byte load through a buffer resource; offsets at or past the resource's
// size read as zero (hardware range check), so tile tails need no branches.
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
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

template <int D>
struct Smem {
  unsigned char k[BN * Tile<D>::kStride];
  unsigned char v[BN * Tile<D>::vStride];
  float ks[BN];   // key scales
  float nks[BN];  // -kMagic * ks: turns the biased accumulator into S*ks with one FMA
  float lb[BN];   // log2-domain additive term per key: bias*log2(e), or -inf for an excluded key
};

// LSE is a compile-time trait: the LSE store exists only in the instances
// that return it, so the plain kernels carry no runtime branch for it.
template <int D, int VT, int NW, bool SPARSE, bool HAS_BIAS, bool LSE>
__global__ __launch_bounds__(NW * 64, 2) void attn_fwd_kernel(AttnArgs a, int qtiles, int total_blocks) {
  constexpr int BM = 32 * NW;
  constexpr int NT = NW * 64;
  constexpr int KC = D / 32;                       // int8 MFMA k-steps / 32-channel blocks
  constexpr int K_CHUNKS = BN * D / 16;            // 16-byte chunks in a K8 tile
  constexpr int V_CHUNKS = BN * D * 2 / 16;        // 16-byte chunks in a V tile
  constexpr int K_PER_T = K_CHUNKS / NT;
  constexpr int V_PER_T = V_CHUNKS / NT;
  static_assert(K_CHUNKS % NT == 0 && V_CHUNKS % NT == 0, "tile split");
  using T = Tile<D>;
  typedef typename std::conditional<VT == BF16, v8bf, v8h>::type pvec;

  // two stages: tile i is computed from one while tile i+1 is written to the other
  __shared__ __attribute__((aligned(16))) Smem<D> sm[2];

  const int bid = xcd_remap((int)blockIdx.x, total_blocks);
  const int bh = bid / qtiles, qt = bid % qtiles;
  const int b = bh / a.H, h = bh % a.H;
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int hl = lane / 32;          // k-group of this lane in the MFMA operands
  const int q = qt * BM + wave * 32 + (lane % 32);
  const bool qvalid = q < a.Sq;
  const int64_t qrow = (int64_t)bh * a.Sq + q;

  // ---- tile list ----
  TileIter it{};
  if (SPARSE) {
    const int T = a.Sk / BN;
    it.list = a.index + ((int64_t)bh * T + qt) * T;
    it.vbs = a.vbs;
    it.ntiles_k = T;
    it.n = min(max(__builtin_amdgcn_readfirstlane(a.count[(int64_t)bh * T + qt]), 0), T);
  } else {
    // segments beyond nseg are empty; the host passes at least one
    auto seg = [&](int g, int& t0, int& n, int& lo, int& hi) {
      lo = g < a.nseg ? a.seg_lo[g] : 0;
      hi = g < a.nseg ? a.seg_hi[g] : 0;
      t0 = lo / BN;
      n = hi > lo ? (hi + BN - 1) / BN - t0 : 0;
    };
    int n3;
    seg(0, it.t0_0, it.n_0, it.lo_0, it.hi_0);
    seg(1, it.t0_1, it.n_1, it.lo_1, it.hi_1);
    seg(2, it.t0_2, it.n_2, it.lo_2, it.hi_2);
    seg(3, it.t0_3, n3, it.lo_3, it.hi_3);
    it.n = it.n_0 + it.n_1 + it.n_2 + n3;
  }

  // ---- Q codes for this lane's row: kept in VGPRs for the whole key loop ----
  v4i qreg[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    if (qvalid) qreg[c] = *(const v4i*)(a.q8 + qrow * D + 32 * c + 16 * hl);
    else qreg[c] = v4i{0, 0, 0, 0};
  }
  const float crow = qvalid ? a.qs[qrow] * (a.sm_scale * kLog2e) : 0.0f;

  // ---- per-(b,h) sources; every tile load is a range-checked buffer load ----
  const unsigned char* kbase = (const unsigned char*)(a.k8 + (int64_t)bh * a.Sk * D);
  const int64_t k_bytes = (int64_t)a.Sk * D;
  const unsigned char* vbase = (const unsigned char*)a.v + ((int64_t)b * a.v_sb + (int64_t)h * a.v_sh) * 2;
  const int64_t v_bytes = a.Sk > 0 ? ((int64_t)(a.Sk - 1) * a.v_ss + D) * 2 : 0;
  const int v_row = (int)(a.v_ss * 2);
  const float* ksbase = a.ks + (int64_t)bh * a.Sk;
  const int64_t bias_off = (int64_t)b * a.bias_sb + (int64_t)h * a.bias_sh;

  // per-thread constant offsets inside a tile
  int k_off[K_PER_T], v_off[V_PER_T], k_lds[K_PER_T], v_lds[V_PER_T];
#pragma unroll
  for (int i = 0; i < K_PER_T; ++i) {
    const int c = tid + i * NT, row = c / (D / 16), col = c % (D / 16);
    k_off[i] = row * D + col * 16;
    k_lds[i] = row * T::kStride + col * 16;
  }
#pragma unroll
  for (int i = 0; i < V_PER_T; ++i) {
    const int c = tid + i * NT, row = c / (D / 8), col = c % (D / 8);
    v_off[i] = row * v_row + col * 16;
    v_lds[i] = row * T::vStride + col * 16;
  }

  // ---- staging registers for one tile ----
  uint4 kreg[K_PER_T], vreg[V_PER_T];
  float ksreg = 0.0f, lbreg = 0.0f;

  auto gload = [&](int tile, int lo, int hi) {
    const int key0 = __builtin_amdgcn_readfirstlane(tile * BN);
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(kbase + (int64_t)key0 * D, k_bytes - (int64_t)key0 * D);
    const __amdgpu_buffer_rsrc_t vr =
        make_rsrc(vbase + (int64_t)key0 * v_row, v_bytes - (int64_t)key0 * v_row);
#pragma unroll
    for (int i = 0; i < K_PER_T; ++i) kreg[i] = bload16(kr, k_off[i]);
#pragma unroll
    for (int i = 0; i < V_PER_T; ++i) vreg[i] = bload16(vr, v_off[i]);
    if (tid < BN) {
      const int key = key0 + tid;
      const bool in = key >= lo && key < hi;   // [lo, hi) lies inside [0, Sk)
      ksreg = in ? ksbase[key] : 0.0f;
      float lbv = 0.0f;
      if (HAS_BIAS && in) lbv = load_bias(a.bias, a.bias_dtype, bias_off + key) * kLog2e;
      lbreg = in ? lbv : -INFINITY;
    }
  };
  auto lstore = [&](Smem<D>& s) {
#pragma unroll
    for (int i = 0; i < K_PER_T; ++i) *(uint4*)(s.k + k_lds[i]) = kreg[i];
#pragma unroll
    for (int i = 0; i < V_PER_T; ++i) *(uint4*)(s.v + v_lds[i]) = vreg[i];
    if (tid < BN) {
      s.ks[tid] = ksreg;
      s.nks[tid] = -kMagic * ksreg;
      s.lb[tid] = lbreg;
    }
  };

  // ---- online softmax state (log2 domain) ----
  v16f o[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) o[c] = v16f{};
  float m_run = -INFINITY;
  float lsum[4] = {0.0f, 0.0f, 0.0f, 0.0f};

  // ds_read_b64_tr_b16 source addressing (per 16-lane group): lane s of the
  // group reads 4 channels at (key0 + s/4, dbase + 4*(s%4)); the hardware
  // hands lane i of the group the 4 keys of channel dbase + i.
  const int grp = lane / 16, sl = lane % 16;
  const int tr_row = 4 * hl + sl / 4;
  const int tr_col = 16 * (grp % 2) + 4 * (sl % 4);

  if (it.n > 0) {
    int tile, lo, hi;
    it.get(0, tile, lo, hi);
    gload(tile, lo, hi);
    lstore(sm[0]);
    __syncthreads();
  }

  // one key tile per iteration: tile `iter` is in `cur`; tile iter+1 is
  // fetched meanwhile and written to `nxt`
  for (int iter = 0; iter < it.n; ++iter) {
    Smem<D>& cur = sm[iter & 1];
    Smem<D>& nxt = sm[(iter + 1) & 1];
    int tile, lo, hi;
    it.get(iter, tile, lo, hi);
    // unmasked tile without bias: scores need no additive term
    const bool plain = !HAS_BIAS && lo == tile * BN && hi == tile * BN + BN;
    const bool more = iter + 1 < it.n;
    if (more) {
      int t2, l2, h2;
      it.get(iter + 1, t2, l2, h2);
      gload(t2, l2, h2);
    }

    // ---- S^T = K8 Q8^T: two 32-key blocks, accumulators biased by kMagicBits ----
    v16i s[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[blk][r] = kMagicBits;
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        const v4i kv = *(const v4i*)(cur.k + (32 * blk + (lane % 32)) * T::kStride + 32 * c + 16 * hl);
        s[blk] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kv, qreg[c], s[blk], 0, 0, 0);
      }
    }

    // ---- dequantize: u = S*ks; plain tiles keep u, the others take t = u*c + lb ----
    float t[2][16];
    float mx;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int kk = 32 * blk + 8 * g + 4 * hl;
        const float4 kv = *(const float4*)(cur.ks + kk);
        const float4 nv = *(const float4*)(cur.nks + kk);
        const float kvs[4] = {kv.x, kv.y, kv.z, kv.w};
        const float nvs[4] = {nv.x, nv.y, nv.z, nv.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) t[blk][4 * g + r] = fmaf(__int_as_float(s[blk][4 * g + r]), kvs[r], nvs[r]);
      }
    if (plain) {
      mx = xmax32(max32(t)) * crow;     // crow >= 0, so max(u)*c = max(u*c)
    } else {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float4 bv = *(const float4*)(cur.lb + 32 * blk + 8 * g + 4 * hl);
          const float bvs[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) t[blk][4 * g + r] = fmaf(t[blk][4 * g + r], crow, bvs[r]);
        }
      mx = xmax32(max32(t));
    }

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
    // plain tiles hold u and need t = u*c; the others already hold t
    const float tscale = plain ? crow : 1.0f;

    // ---- p = exp2(t - m) as packed P^T operands, fp32 row sum, PV ----
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        // the row sum takes the fp32 values: a sum of bf16-rounded p would
        // carry up to 2^-9 relative error into the LSE when one key dominates
        uint32_t pw[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(t[blk][8 * m + 2 * e], tscale, -m_use));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(t[blk][8 * m + 2 * e + 1], tscale, -m_use));
          lsum[e] += p0 + p1;
          if constexpr (VT == BF16) {
            const v2bf pair = {(__bf16)p0, (__bf16)p1};
            pw[e] = __builtin_bit_cast(uint32_t, pair);
          } else {
            const v2h pair = {(_Float16)p0, (_Float16)p1};
            pw[e] = __builtin_bit_cast(uint32_t, pair);
          }
        }
        const pvec pb = __builtin_bit_cast(pvec, pw);
        const int krow = 32 * blk + 16 * m + tr_row;
#pragma unroll
        for (int c = 0; c < KC; ++c) {
          const unsigned char* p0 = cur.v + krow * T::vStride + (32 * c + tr_col) * 2;
          const v4s lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)p0);
          const v4s hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4s*)(p0 + 8 * T::vStride));
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
    }

    if (more) lstore(nxt);
    __syncthreads();
  }

  // ---- epilogue: O = O_acc / l * v_scale, LSE ----
  const float l_tot = xsum32((lsum[0] + lsum[1]) + (lsum[2] + lsum[3]));
  if (!qvalid) return;
  const float inv_l = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  const int64_t obase = (int64_t)b * a.o_sb + (int64_t)h * a.o_sh + (int64_t)q * a.o_ss;
#pragma unroll
  for (int c = 0; c < KC; ++c) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = 32 * c + 8 * g + 4 * hl;
      float vals[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) vals[r] = o[c][4 * g + r] * inv_l;
      if (a.v_scale) {
        const float4 vs = *(const float4*)(a.v_scale + (int64_t)h * D + d0);
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

template <int D, int VT>
hipError_t launch_d_vt(const AttnArgs& a, hipStream_t s) {
  const bool sparse = a.index != nullptr;
  const int NW = sparse ? 2 : 4;
  const int BM = 32 * NW;
  const int qtiles = (a.Sq + BM - 1) / BM;
  const int total = qtiles * a.B * a.H;
  if (total == 0) return hipSuccess;
  if (sparse) {
    if (a.lse) attn_fwd_kernel<D, VT, 2, true, false, true><<<total, 128, 0, s>>>(a, qtiles, total);
    else attn_fwd_kernel<D, VT, 2, true, false, false><<<total, 128, 0, s>>>(a, qtiles, total);
  } else if (a.bias) {
    if (a.lse) attn_fwd_kernel<D, VT, 4, false, true, true><<<total, 256, 0, s>>>(a, qtiles, total);
    else attn_fwd_kernel<D, VT, 4, false, true, false><<<total, 256, 0, s>>>(a, qtiles, total);
  } else {
    if (a.lse) attn_fwd_kernel<D, VT, 4, false, false, true><<<total, 256, 0, s>>>(a, qtiles, total);
    else attn_fwd_kernel<D, VT, 4, false, false, false><<<total, 256, 0, s>>>(a, qtiles, total);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(const AttnArgs& a, hipStream_t s) {
  if (a.D == 128) return a.v_dtype == BF16 ? launch_d_vt<128, BF16>(a, s) : launch_d_vt<128, FP16>(a, s);
  return a.v_dtype == BF16 ? launch_d_vt<64, BF16>(a, s) : launch_d_vt<64, FP16>(a, s);
}

}  // namespace qfa
