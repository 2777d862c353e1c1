// K mean and per-token symmetric int8 quantization of Q and K for gfx950.
//
// Method: FastVideo API docs, "minimax_h3_sparse_int8" (module description:
// per-token Q/K scales, K centring as a softmax-invariant shift; listing of
// sparse_sm89_attention: mean of K over the sequence divided by the number of
// valid tokens, then Q quantized uncentred and K centred); model-kernels
// issue #3 (symmetric [-127,127] codes, absmax and quantize loops over the
// same (row, channel) decomposition).
//
// Both kernels are HBM-bound streaming passes: 16-byte loads, one row of D
// channels spread over D/8 lanes, the row absmax reduced across those lanes.
#include "qfa_internal.h"

#include <float.h>

namespace qfa {
namespace {

// Error-free sum of two doubles (Knuth's two-sum): hi + lo == a + b exactly.
__device__ __forceinline__ void two_sum(double a, double b, double& s, double& e) {
  s = a + b;
  double bb = s - a;
  e = (a - (s - bb)) + (b - bb);
}

// Double-double accumulator. With bf16/fp16 inputs every partial sum stays a
// multiple of the smallest input ulp with a modest magnitude, so hi + lo holds
// the exact sum whenever the data's bit span stays below ~100 bits (always for
// fp16; bf16 data within a 2^+-40 magnitude band). Hence the result does not
// depend on the reduction order.
struct DD {
  double hi, lo;
  __device__ __forceinline__ void add(double x) {
    double s, e;
    two_sum(hi, x, s, e);
    hi = s;
    lo += e;
  }
  __device__ __forceinline__ void add(const DD& o) {
    double s, e;
    two_sum(hi, o.hi, s, e);
    hi = s;
    lo = lo + o.lo + e;
  }
};

__device__ __forceinline__ bool is_pad(const int32_t* vbs, int64_t j) {
  return vbs != nullptr && (int32_t)(j & 63) >= vbs[j >> 6];
}

// Partial column sums of K over one chunk of kMeanChunkRows rows of one (b,h).
// 1-D grid over (b,h) x chunks; block: 256 threads = D/8 channel groups x
// (2048/D) row slots, each slot loading 4 rows at a time (16 bytes each).
template <int DT, int D>
__global__ __launch_bounds__(256) void kmean_partial_kernel(MeanArgs a) {
  constexpr int G = D / 8;          // lanes per row
  constexpr int RP = 256 / G;       // row slots per block
  constexpr int U = 4;              // rows per slot in flight
  __shared__ double2 red[RP][D];

  const int bid = blockIdx.x;
  const int chunk = bid % a.nchunks;
  const int64_t bh = bid / a.nchunks;
  const int64_t b = bh / a.H, h = bh % a.H;
  const int cg = threadIdx.x % G, rs = threadIdx.x / G;
  const int64_t r0 = (int64_t)chunk * kMeanChunkRows;
  const int64_t r1 = min(r0 + kMeanChunkRows, a.S);
  const uint16_t* base = (const uint16_t*)a.k + b * a.sb + h * a.sh + cg * 8;

  DD acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = DD{0.0, 0.0};
  for (int64_t j = r0 + rs; j < r1; j += RP * U) {
    uint4 w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t jj = j + u * RP;
      const bool live = jj < r1 && !is_pad(a.vbs, jj);
      w[u] = live ? *(const uint4*)(base + jj * a.ss) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float f[8];
      unpack8<DT>(w[u], f);   // a skipped row adds exact zeros
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i].add((double)f[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) red[rs][cg * 8 + i] = make_double2(acc[i].hi, acc[i].lo);
  __syncthreads();
  for (int c = threadIdx.x; c < D; c += 256) {
    DD s{0.0, 0.0};
    for (int r = 0; r < RP; ++r) s.add(DD{red[r][c].x, red[r][c].y});
    a.partial[(bh * a.nchunks + chunk) * D + c] = make_double2(s.hi, s.lo);
  }
}

// mean[bh, c] = fp32( fp64(hi + lo) / n ) over the chunk partials. 1-D grid
// over (b,h) x 32-channel groups; block: 32 channels x 8 slices of chunks,
// the slices' exact partial sums combined in LDS.
__global__ __launch_bounds__(256) void kmean_finalize_kernel(MeanArgs a) {
  __shared__ long long nsum[256];
  __shared__ double2 red[8][32];
  const int groups = (int)(a.D / 32);
  const int64_t bh = blockIdx.x / groups;
  const int c = (blockIdx.x % groups) * 32 + (int)threadIdx.x % 32;
  const int slice = threadIdx.x / 32;
  long long n = 0;
  if (a.vbs) {
    const int64_t T = (a.S + 63) / 64;
    for (int64_t t = threadIdx.x; t < T; t += 256) n += a.vbs[t];
  }
  nsum[threadIdx.x] = n;
  DD s{0.0, 0.0};
  for (int k = slice; k < a.nchunks; k += 8) {
    const double2 p = a.partial[(bh * a.nchunks + k) * a.D + c];
    s.add(DD{p.x, p.y});
  }
  red[slice][threadIdx.x % 32] = make_double2(s.hi, s.lo);
  __syncthreads();
  for (int st = 128; st > 0; st >>= 1) {
    if ((int)threadIdx.x < st) nsum[threadIdx.x] += nsum[threadIdx.x + st];
    __syncthreads();
  }
  if (slice == 0) {
    DD t{0.0, 0.0};
    for (int k = 0; k < 8; ++k) t.add(DD{red[k][threadIdx.x].x, red[k][threadIdx.x].y});
    long long cnt = a.vbs ? nsum[0] : a.S;
    if (cnt < 1) cnt = 1;
    const double total = t.hi + t.lo;  // the exact sum rounded once to fp64
    a.mean[bh * a.D + c] = (float)(total / (double)cnt);
  }
}

// One row of D channels per D/8 lanes; each lane owns 8 consecutive channels.
// 1-D grid over (b,h) x row blocks of RPB*U rows; each lane loads its chunk of
// U rows first, then quantizes them one by one.
template <int DT, int D>
__global__ __launch_bounds__(256) void quantize_rows_kernel(QuantRowsArgs a, int rblocks) {
  constexpr int G = D / 8;
  constexpr int RPB = 256 / G;
  constexpr int U = 4;
  const int cg = threadIdx.x % G;
  const int64_t bh = blockIdx.x / rblocks;
  const int64_t j0 = (int64_t)(blockIdx.x % rblocks) * (RPB * U) + threadIdx.x / G;
  const int64_t b = bh / a.H, h = bh % a.H;
  // the mean row of this row's K/V head (grouped-query: runs of H / mean_heads heads share one)
  const int64_t mrow = b * a.mean_heads + (int)h / (int)(a.H / a.mean_heads);
  const uint16_t* src = (const uint16_t*)a.x + b * a.sb + h * a.sh + cg * 8;

  uint4 w[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t j = j0 + u * RPB;
    const bool live = j < a.S && !is_pad(a.vbs, j);
    w[u] = live ? *(const uint4*)(src + j * a.ss) : make_uint4(0u, 0u, 0u, 0u);
  }
  float qm[8], mm[8];
  if (a.qmu_mean) {
    const float4 m0 = *(const float4*)(a.qmu_mean + mrow * D + cg * 8);
    const float4 m1 = *(const float4*)(a.qmu_mean + mrow * D + cg * 8 + 4);
    qm[0] = m0.x; qm[1] = m0.y; qm[2] = m0.z; qm[3] = m0.w; qm[4] = m1.x; qm[5] = m1.y; qm[6] = m1.z; qm[7] = m1.w;
  }
  if (a.mean) {
    const float4 m0 = *(const float4*)(a.mean + mrow * D + cg * 8);
    const float4 m1 = *(const float4*)(a.mean + mrow * D + cg * 8 + 4);
    mm[0] = m0.x; mm[1] = m0.y; mm[2] = m0.z; mm[3] = m0.w; mm[4] = m1.x; mm[5] = m1.y; mm[6] = m1.z; mm[7] = m1.w;
  }

#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t j = j0 + u * RPB;
    if (j >= a.S) break;   // uniform across the row's G lanes (G divides 64)
    const int64_t r = bh * a.S + j;
    const bool pad = is_pad(a.vbs, j);
    float x[8];
    unpack8<DT>(w[u], x);   // zeros for a pad row

    float qmu = 0.0f;
    if (a.qmu_mean) {
#pragma unroll
      for (int i = 0; i < 8; ++i) qmu += x[i] * qm[i];
    }
    if (a.mean) {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = __fsub_rn(x[i], mm[i]);  // one fp32 subtraction
    }

    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
#pragma unroll
    for (int off = G / 2; off > 0; off >>= 1) {
      amax = fmaxf(amax, __shfl_xor(amax, off, G));
      if (a.qmu) qmu += __shfl_xor(qmu, off, G);
    }

    uint32_t lo = 0, hi = 0;
    float scale = 0.0f;
    if (!pad && amax >= 127.0f * FLT_MIN) {
      scale = amax / 127.0f;                  // correctly rounded fp32 division
      const float inv = 127.0f / amax;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float y = __builtin_rintf(__fmul_rn(x[i], inv));  // round half to even
        y = fminf(fmaxf(y, -127.0f), 127.0f);
        const uint32_t code = (uint32_t)((int)y) & 0xffu;
        if (i < 4) lo |= code << (8 * i);
        else hi |= code << (8 * (i - 4));
      }
    }
    *(uint2*)(a.codes + r * D + cg * 8) = make_uint2(lo, hi);
    if (cg == 0) {
      a.scale[r] = scale;
      if (a.qmu) a.qmu[r] = pad ? 0.0f : qmu;
    }
  }
}

}  // namespace

hipError_t launch_kmean(const MeanArgs& a, hipStream_t s) {
  const unsigned grid = (unsigned)(a.nchunks * a.B * a.H);
  if (grid == 0) return hipSuccess;   // no (b,h) pair or no rows: nothing to average
  if (a.D == 128) {
    if (a.dtype == BF16) kmean_partial_kernel<BF16, 128><<<grid, 256, 0, s>>>(a);
    else kmean_partial_kernel<FP16, 128><<<grid, 256, 0, s>>>(a);
  } else {
    if (a.dtype == BF16) kmean_partial_kernel<BF16, 64><<<grid, 256, 0, s>>>(a);
    else kmean_partial_kernel<FP16, 64><<<grid, 256, 0, s>>>(a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  kmean_finalize_kernel<<<(unsigned)(a.B * a.H * (a.D / 32)), 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_quantize_rows(const QuantRowsArgs& a, hipStream_t s) {
  const int rpb = 4 * (256 / (int)(a.D / 8));   // rows per block: 4 per row slot
  const int rblocks = (int)((a.S + rpb - 1) / rpb);
  const unsigned grid = (unsigned)(rblocks * a.B * a.H);
  if (grid == 0) return hipSuccess;
  if (a.D == 128) {
    if (a.dtype == BF16) quantize_rows_kernel<BF16, 128><<<grid, 256, 0, s>>>(a, rblocks);
    else quantize_rows_kernel<FP16, 128><<<grid, 256, 0, s>>>(a, rblocks);
  } else {
    if (a.dtype == BF16) quantize_rows_kernel<BF16, 64><<<grid, 256, 0, s>>>(a, rblocks);
    else quantize_rows_kernel<FP16, 64><<<grid, 256, 0, s>>>(a, rblocks);
  }
  return hipGetLastError();
}

}  // namespace qfa
