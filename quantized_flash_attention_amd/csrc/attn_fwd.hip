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

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Lazy rescaling: the running reference max only moves when a row's max
// exceeds it by more than this (log2 units), so p <= 2^8 between rescales.
constexpr float kRescaleSlack = 8.0f;

constexpr int BN = 64;  // keys per tile

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
// key-tile list of this query tile (block-sparse).
struct TileIter {
  int n;               // number of tiles
  int seg_t0[4], seg_n[4], seg_lo[4], seg_hi[4];
  int nseg;
  const int32_t* list; // sparse: key tiles
  const int32_t* vbs;  // sparse: valid counts (nullable)
  int ntiles_k;        // sparse: number of key tiles

  // tile index and the valid key range [lo, hi) inside it (absolute keys).
  // A listed tile outside [0, ntiles_k) is treated as an empty tile.
  __device__ __forceinline__ void get(int it, int& tile, int& lo, int& hi) const {
    if (list) {
      tile = list[it];
      if (tile < 0 || tile >= ntiles_k) {
        tile = 0;
        lo = hi = 0;
        return;
      }
      lo = tile * BN;
      hi = lo + (vbs ? min(max(vbs[tile], 0), BN) : BN);
      return;
    }
    int g = 0;
    while (g + 1 < nseg && it >= seg_n[g]) { it -= seg_n[g]; ++g; }
    tile = seg_t0[g] + it;
    lo = max(seg_lo[g], tile * BN);
    hi = min(seg_hi[g], tile * BN + BN);
  }
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

  __shared__ __attribute__((aligned(16))) unsigned char k_lds[T::kBytes];
  __shared__ __attribute__((aligned(16))) unsigned char v_lds[T::vBytes];
  __shared__ __attribute__((aligned(16))) float ks_lds[BN];
  __shared__ __attribute__((aligned(16))) float lb_lds[BN];

  const int bid = xcd_remap((int)blockIdx.x, total_blocks);
  const int bh = bid / qtiles, qt = bid % qtiles;
  const int b = bh / a.H, h = bh % a.H;
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int hl = lane / 32;          // k-group of this lane in the MFMA operands
  const int q = qt * BM + wave * 32 + (lane % 32);
  const bool qvalid = q < a.Sq;
  const int64_t qrow = (int64_t)bh * a.Sq + q;

  // ---- tile list ----
  TileIter it;
  it.list = nullptr;
  it.vbs = nullptr;
  it.nseg = 0;
  it.ntiles_k = 0;
  if (SPARSE) {
    const int T = a.Sk / BN;
    it.list = a.index + ((int64_t)bh * T + qt) * T;
    it.vbs = a.vbs;
    it.ntiles_k = T;
    it.n = min(max(a.count[(int64_t)bh * T + qt], 0), T);
  } else {
    it.nseg = a.nseg;
    it.n = 0;
    for (int g = 0; g < 4; ++g) {
      if (g < a.nseg) {
        const int t0 = a.seg_lo[g] / BN, t1 = (a.seg_hi[g] + BN - 1) / BN;
        it.seg_t0[g] = t0;
        it.seg_n[g] = a.seg_hi[g] > a.seg_lo[g] ? t1 - t0 : 0;
        it.seg_lo[g] = a.seg_lo[g];
        it.seg_hi[g] = a.seg_hi[g];
        it.n += it.seg_n[g];
      } else {
        it.seg_t0[g] = it.seg_n[g] = it.seg_lo[g] = it.seg_hi[g] = 0;
      }
    }
  }

  // ---- Q codes for this lane's row: kept in VGPRs for the whole key loop ----
  v4i qreg[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    if (qvalid) qreg[c] = *(const v4i*)(a.q8 + qrow * D + 32 * c + 16 * hl);
    else qreg[c] = v4i{0, 0, 0, 0};
  }
  const float crow = qvalid ? a.qs[qrow] * (a.sm_scale * kLog2e) : 0.0f;

  const int8_t* kbase = a.k8 + (int64_t)bh * a.Sk * D;
  const float* ksbase = a.ks + (int64_t)bh * a.Sk;
  const uint16_t* vbase = (const uint16_t*)a.v + (int64_t)b * a.v_sb + (int64_t)h * a.v_sh;
  const int64_t bias_off = (int64_t)b * a.bias_sb + (int64_t)h * a.bias_sh;

  // ---- staging registers for one tile ----
  uint4 kreg[K_PER_T], vreg[V_PER_T];
  float ksreg = 0.0f, lbreg = 0.0f;

  auto gload = [&](int tile) {
    const int key0 = tile * BN;
#pragma unroll
    for (int i = 0; i < K_PER_T; ++i) {
      const int c = tid + i * NT;
      const int row = c / (D / 16), col = c % (D / 16);
      const int key = key0 + row;
      kreg[i] = key < a.Sk ? *(const uint4*)(kbase + (int64_t)key * D + col * 16) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < V_PER_T; ++i) {
      const int c = tid + i * NT;
      const int row = c / (D / 8), col = c % (D / 8);
      const int key = key0 + row;
      vreg[i] = key < a.Sk ? *(const uint4*)(vbase + (int64_t)key * a.v_ss + col * 8) : make_uint4(0, 0, 0, 0);
    }
    if (tid < BN) {
      const int key = key0 + tid;
      ksreg = key < a.Sk ? ksbase[key] : 0.0f;
      if (HAS_BIAS) lbreg = key < a.Sk ? load_bias(a.bias, a.bias_dtype, bias_off + key) * kLog2e : 0.0f;
    }
  };
  auto lstore = [&]() {
#pragma unroll
    for (int i = 0; i < K_PER_T; ++i) {
      const int c = tid + i * NT;
      const int row = c / (D / 16), col = c % (D / 16);
      *(uint4*)(k_lds + row * T::kStride + col * 16) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < V_PER_T; ++i) {
      const int c = tid + i * NT;
      const int row = c / (D / 8), col = c % (D / 8);
      *(uint4*)(v_lds + row * T::vStride + col * 16) = vreg[i];
    }
    if (tid < BN) {
      ks_lds[tid] = ksreg;
      if (HAS_BIAS) lb_lds[tid] = lbreg;
    }
  };

  // ---- online softmax state (log2 domain) ----
  v16f o[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) o[c] = v16f{};
  float m_run = -INFINITY, l_run = 0.0f;

  // ds_read_b64_tr_b16 source addressing (per 16-lane group): lane s of the
  // group reads 4 channels at (key0 + s/4, dbase + 4*(s%4)); the hardware
  // hands lane i of the group the 4 keys of channel dbase + i.
  const int grp = lane / 16, sl = lane % 16;
  const int tr_row = 4 * hl + sl / 4;
  const int tr_col = 16 * (grp % 2) + 4 * (sl % 4);

  if (it.n > 0) {
    int tile, lo, hi;
    it.get(0, tile, lo, hi);
    gload(tile);
    lstore();
    __syncthreads();
  }

  for (int iter = 0; iter < it.n; ++iter) {
    int tile, lo, hi;
    it.get(iter, tile, lo, hi);
    if (iter + 1 < it.n) {
      int t2, l2, h2;
      it.get(iter + 1, t2, l2, h2);
      gload(t2);
    }

    // ---- S^T = K8 Q8^T: two 32-key blocks ----
    v16i s[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      s[blk] = v16i{};
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        const v4i kv = *(const v4i*)(k_lds + (32 * blk + (lane % 32)) * T::kStride + 32 * c + 16 * hl);
        s[blk] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kv, qreg[c], s[blk], 0, 0, 0);
      }
    }

    // ---- dequantize (+bias), mask, row max ----
    const int klo = lo - tile * BN, khi = hi - tile * BN;  // valid keys within the tile
    const bool full = (klo == 0 && khi == BN);
    float t[2][16];
    float mx = -INFINITY;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int kk0 = 32 * blk + 8 * g + 4 * hl;
        const float4 kv = *(const float4*)(ks_lds + kk0);
        float4 bv = make_float4(0.f, 0.f, 0.f, 0.f);
        if (HAS_BIAS) bv = *(const float4*)(lb_lds + kk0);
        const float kvs[4] = {kv.x, kv.y, kv.z, kv.w};
        const float bvs[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float u = (float)s[blk][4 * g + r] * kvs[r];
          float x = HAS_BIAS ? fmaf(u, crow, bvs[r]) : u * crow;
          if (!full) {
            const int kk = kk0 + r;
            x = (kk >= klo && kk < khi) ? x : -INFINITY;
          }
          t[blk][4 * g + r] = x;
          mx = fmaxf(mx, x);
        }
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));

    // ---- lazy rescale (wave-uniform branch) ----
    const bool need = mx > m_run + kRescaleSlack;
    if (__any(need)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int c = 0; c < KC; ++c) o[c] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == -INFINITY) ? 0.0f : m_run;

    // ---- p = exp2(t - m), row sum (kept per lane), PV ----
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(t[blk][r] - m_use);
        t[blk][r] = p;
        l_run += p;
      }
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        // B operand: P^T, keys 32*blk + 16*m + {0..3, 8..11} + 4*hl of this lane's row
        typedef typename std::conditional<VT == BF16, v8bf, v8h>::type pvec;
        pvec pb;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if constexpr (VT == BF16) pb[e] = (__bf16)t[blk][8 * m + e];
          else pb[e] = (_Float16)t[blk][8 * m + e];
        }
        const int krow = 32 * blk + 16 * m + tr_row;
#pragma unroll
        for (int c = 0; c < KC; ++c) {
          const unsigned char* p0 = v_lds + krow * T::vStride + (32 * c + tr_col) * 2;
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

    __syncthreads();
    if (iter + 1 < it.n) {
      lstore();
      __syncthreads();
    }
  }

  // ---- epilogue: O = O_acc / l * v_scale, LSE ----
  const float l_tot = l_run + __shfl_xor(l_run, 32);
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
