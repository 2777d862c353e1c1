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
// Block: 256 threads; D/8 channel groups x (2048/D) row slots.
template <int DT, int D>
__global__ __launch_bounds__(256) void kmean_partial_kernel(MeanArgs a) {
  constexpr int G = D / 8;          // lanes per row
  constexpr int RP = 256 / G;       // rows in flight per block
  __shared__ double2 red[RP][D];

  const int chunk = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int64_t b = bh / a.H, h = bh % a.H;
  const int cg = threadIdx.x % G, rs = threadIdx.x / G;
  const int64_t r0 = (int64_t)chunk * kMeanChunkRows;
  const int64_t r1 = min(r0 + kMeanChunkRows, a.S);
  const uint16_t* base = (const uint16_t*)a.k + b * a.sb + h * a.sh + cg * 8;

  DD acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = DD{0.0, 0.0};
  for (int64_t j = r0 + rs; j < r1; j += RP) {
    if (is_pad(a.vbs, j)) continue;
    const uint4 w = *(const uint4*)(base + j * a.ss);
    float f[8];
    unpack8<DT>(w, f);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i].add((double)f[i]);
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

// mean[bh, c] = fp32( fp64(hi + lo) / n ) over the chunk partials.
__global__ __launch_bounds__(256) void kmean_finalize_kernel(MeanArgs a) {
  __shared__ long long nsum[256];
  const int64_t bh = blockIdx.x;
  long long n = 0;
  if (a.vbs) {
    const int64_t T = (a.S + 63) / 64;
    for (int64_t t = threadIdx.x; t < T; t += 256) n += a.vbs[t];
  }
  nsum[threadIdx.x] = n;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) nsum[threadIdx.x] += nsum[threadIdx.x + s];
    __syncthreads();
  }
  long long cnt = a.vbs ? nsum[0] : a.S;
  if (cnt < 1) cnt = 1;
  for (int64_t c = threadIdx.x; c < a.D; c += 256) {
    DD s{0.0, 0.0};
    for (int k = 0; k < a.nchunks; ++k) {
      const double2 p = a.partial[(bh * a.nchunks + k) * a.D + c];
      s.add(DD{p.x, p.y});
    }
    const double total = s.hi + s.lo;  // the exact sum rounded once to fp64
    a.mean[bh * a.D + c] = (float)(total / (double)cnt);
  }
}

// One row of D channels per D/8 lanes; each lane owns 8 consecutive channels.
template <int DT, int D>
__global__ __launch_bounds__(256) void quantize_rows_kernel(QuantRowsArgs a) {
  constexpr int G = D / 8;
  constexpr int RPB = 256 / G;
  const int cg = threadIdx.x % G;
  const int64_t r = (int64_t)blockIdx.x * RPB + threadIdx.x / G;
  const int64_t rows = a.B * a.H * a.S;
  if (r >= rows) return;  // whole row groups leave together (G divides 64)
  const int64_t bh = r / a.S, j = r % a.S;
  const int64_t b = bh / a.H, h = bh % a.H;
  // the mean row of this row's K/V head (grouped-query: runs of H / mean_heads heads share one)
  const int64_t mrow = b * a.mean_heads + (int)h / (int)(a.H / a.mean_heads);

  const bool pad = is_pad(a.vbs, j);
  float x[8];
  if (!pad) {
    const uint4 w = *(const uint4*)((const uint16_t*)a.x + b * a.sb + h * a.sh + j * a.ss + cg * 8);
    unpack8<DT>(w, x);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = 0.0f;
  }

  float qmu = 0.0f;
  if (a.qmu_mean) {
    const float4 m0 = *(const float4*)(a.qmu_mean + mrow * D + cg * 8);
    const float4 m1 = *(const float4*)(a.qmu_mean + mrow * D + cg * 8 + 4);
    const float mm[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) qmu += x[i] * mm[i];
  }
  if (a.mean) {
    const float4 m0 = *(const float4*)(a.mean + mrow * D + cg * 8);
    const float4 m1 = *(const float4*)(a.mean + mrow * D + cg * 8 + 4);
    const float mm[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
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

}  // namespace

hipError_t launch_kmean(const MeanArgs& a, hipStream_t s) {
  const dim3 grid(a.nchunks, (unsigned)(a.B * a.H));
  if (a.D == 128) {
    if (a.dtype == BF16) kmean_partial_kernel<BF16, 128><<<grid, 256, 0, s>>>(a);
    else kmean_partial_kernel<FP16, 128><<<grid, 256, 0, s>>>(a);
  } else {
    if (a.dtype == BF16) kmean_partial_kernel<BF16, 64><<<grid, 256, 0, s>>>(a);
    else kmean_partial_kernel<FP16, 64><<<grid, 256, 0, s>>>(a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  kmean_finalize_kernel<<<(unsigned)(a.B * a.H), 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_quantize_rows(const QuantRowsArgs& a, hipStream_t s) {
  const int64_t rows = a.B * a.H * a.S;
  const int rpb = 256 / (int)(a.D / 8);
  const unsigned grid = (unsigned)((rows + rpb - 1) / rpb);
  if (a.D == 128) {
    if (a.dtype == BF16) quantize_rows_kernel<BF16, 128><<<grid, 256, 0, s>>>(a);
    else quantize_rows_kernel<FP16, 128><<<grid, 256, 0, s>>>(a);
  } else {
    if (a.dtype == BF16) quantize_rows_kernel<BF16, 64><<<grid, 256, 0, s>>>(a);
    else quantize_rows_kernel<FP16, 64><<<grid, 256, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace qfa
