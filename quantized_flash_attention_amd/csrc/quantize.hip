// K mean and per-token symmetric int8 quantization of Q and K for gfx950.
//
// Method: FastVideo API docs, "minimax_h3_sparse_int8" (module description:
// per-token Q/K scales, K centring as a softmax-invariant shift; listing of
// sparse_sm89_attention: mean of K over the sequence divided by the number of
// valid tokens, then Q quantized uncentred and K centred); model-kernels
// issue #3 (symmetric [-127,127] codes, absmax and quantize loops over the
// same (row, channel) decomposition).
//
// Three launches, the two big ones HBM-bound streaming passes with 16-byte
// loads and one row of D channels spread over D/8 lanes:
//   kmean_partial_kernel   exact column sums of K over row chunks of each
//                          (b, K/V head)
//   kmean_finalize_kernel  each head's chunk sums combined (exactly, so in any
//                          order) into the mean: a few KB per head
//   quantize_kernel        every K row (centred), then every Q row (and q.mu):
//                          one grid. K rows run in reverse order of the mean
//                          pass, so the rows that pass read last, still held
//                          in the 256 MB MALL, are read again first.
#include "qfa_internal.h"

#include <float.h>

#include <mutex>

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
// depend on the reduction order. A NaN or +-inf input makes lo (and so the
// mean) NaN.
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

// K mean, first pass. 1-D grid over (b, K/V head) x chunks of chunk_rows
// rows; block: 256 threads = D/8 channel groups x (2048/D) row slots, each
// slot loading 4 rows at a time. The block's exact column sums go to its
// partial slot.
//
// Each lane sums its values of a channel in plain fp64, which is exact when
// every partial sum is representable. The lane tracks its largest and smallest
// nonzero magnitude; every value is a multiple of 2^(emin - (P - 1)) for the
// smallest one's exponent emin and the input's P significand bits (8 for
// bf16, 11 for fp16, whose subnormals are multiples of 2^-24 and so qualify
// too), and every partial sum stays below 2^(emax + 1) times the count, so the
// sum is exact when (emax - emin) + P + log2(values summed) <= 53. A lane whose
// values span more (tiny values beside large ones, bf16 subnormals, a NaN or
// inf) sums its rows again in double-double. The slots' sums are combined in
// double-double.
template <int DT, int D>
__global__ __launch_bounds__(256) void kmean_partial_kernel(QuantArgs a, int nchunks, int64_t chunk_rows) {
  constexpr int G = D / 8;          // lanes per row
  constexpr int RP = 256 / G;       // row slots per block
  constexpr int U = 4;              // rows per slot in flight
  __shared__ double2 red[RP][D];

  const int chunk = (int)(blockIdx.x % nchunks);
  const int64_t bh = blockIdx.x / nchunks;
  const int64_t b = bh / a.Hkv, h = bh % a.Hkv;
  const int cg = threadIdx.x % G, rs = threadIdx.x / G;
  const int64_t r0 = chunk * chunk_rows;
  const int64_t r1 = min(r0 + chunk_rows, a.Sk);
  const uint16_t* base = (const uint16_t*)a.k + b * a.k_sb + h * a.k_sh + cg * 8;

  double fsum[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) fsum[i] = 0.0;
  // largest magnitude, and smallest nonzero magnitude minus one (fp32 bits,
  // unsigned, so a zero wraps to the top and never counts)
  uint32_t amax = 0u, amin_m1 = 0xffffffffu;
  int64_t nvals = 0;   // values this lane adds per channel
  for (int64_t j = r0 + rs; j < r1; j += RP * U) {
    uint4 w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t jj = j + u * RP;
      const bool live = jj < r1 && !is_pad(a.vbs, jj);
      w[u] = live ? *(const uint4*)(base + jj * a.k_ss) : make_uint4(0u, 0u, 0u, 0u);
    }
    nvals += U;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float f[8];
      unpack8<DT>(w[u], f);   // a skipped row adds exact zeros
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        fsum[i] += (double)f[i];
        const uint32_t m = __float_as_uint(f[i]) & 0x7fffffffu;
        amax = max(amax, m);
        amin_m1 = min(amin_m1, m - 1u);
      }
    }
  }
  bool exact = true;
  if (amax != 0u) {
    constexpr int P = DT == BF16 ? 8 : 11;   // significand bits of the input type
    // exponents of the extreme magnitudes (an fp32 subnormal, i.e. a bf16
    // one, counts as 2^-149, which always fails the test below)
    const int emax = (int)(amax >> 23) - 127;
    const uint32_t amin = amin_m1 + 1u;
    const int emin = (amin >> 23) == 0u ? -149 : (int)(amin >> 23) - 127;
    const int lgn = 64 - __clzll((unsigned long long)max(nvals, (int64_t)1));   // > log2(nvals)
    exact = emax - emin + P + lgn <= 53;
  }
  DD acc[8];
  if (exact) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = DD{fsum[i], 0.0};
  } else {
    // the same rows again, summed in double-double
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = DD{0.0, 0.0};
    for (int64_t j = r0 + rs; j < r1; j += RP) {
      const bool live = !is_pad(a.vbs, j);
      const uint4 w = live ? *(const uint4*)(base + j * a.k_ss) : make_uint4(0u, 0u, 0u, 0u);
      float f[8];
      unpack8<DT>(w, f);
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
    ((double2*)a.workspace)[(bh * nchunks + chunk) * D + c] = make_double2(s.hi, s.lo);
  }
}

// K mean, second pass: mean[bh, c] = fp32( fp64(exact sum) / n ), n = Sk or
// max(1, sum(vbs)). 1-D grid over (b, K/V head) x 32-channel groups; block:
// 32 channels x 8 slices of the head's chunks, combined in LDS.
__global__ __launch_bounds__(256) void kmean_finalize_kernel(QuantArgs a, int nchunks) {
  __shared__ long long nsum[256];
  __shared__ double2 red[8][32];
  const int groups = (int)(a.D / 32);
  const int64_t bh = blockIdx.x / groups;
  const int c = (blockIdx.x % groups) * 32 + (int)threadIdx.x % 32;
  const int slice = threadIdx.x / 32;
  const double2* partial = (const double2*)a.workspace;
  long long n = 0;
  if (a.vbs) {
    const int64_t T = (a.Sk + 63) / 64;
    for (int64_t t = threadIdx.x; t < T; t += 256) n += a.vbs[t];
  }
  nsum[threadIdx.x] = n;
  DD s{0.0, 0.0};
  for (int k = slice; k < nchunks; k += 8) {
    const double2 p = partial[(bh * nchunks + k) * a.D + c];
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
    long long cnt = a.vbs ? nsum[0] : a.Sk;
    if (cnt < 1) cnt = 1;
    const double total = t.hi + t.lo;  // the exact sum rounded once to fp64
    a.kmean[bh * a.D + c] = (float)(total / (double)cnt);
  }
}

// Every K row, then every Q row. One row of D channels per D/8 lanes, each
// lane owning 8 consecutive channels; a block covers RPB*U rows of one head,
// each lane loading its U rows first and then quantizing them one by one.
// Per row x (K rows centred first, x - mu in one fp32 subtraction):
//   a = max |x|; a < 127*FLT_MIN -> codes 0, scale 0;
//   else scale = a/127, inv = 127/a (both correctly rounded),
//        code = clamp(rint(x*inv), -127, 127);
//   a NaN or +-inf in the row -> codes 0, scale NaN (and q.mu NaN).
// Q rows with centring also give qmu = sum_c x_c * mu_c (fp32).
template <int DT, int D>
__global__ __launch_bounds__(256) void quantize_kernel(QuantArgs a, int64_t k_blocks, int k_rblocks, int q_rblocks) {
  constexpr int G = D / 8;
  constexpr int RPB = 256 / G;
  constexpr int U = 4;
  const int cg = threadIdx.x % G;
  // block-uniform choice of the operand
  const bool is_k = (int64_t)blockIdx.x < k_blocks;
  const int64_t idx = is_k ? k_blocks - 1 - (int64_t)blockIdx.x : (int64_t)blockIdx.x - k_blocks;
  const int rblocks = is_k ? k_rblocks : q_rblocks;
  const int64_t bh = idx / rblocks;
  const int64_t heads = is_k ? a.Hkv : a.H;
  const int64_t S = is_k ? a.Sk : a.Sq;
  const int64_t ss = is_k ? a.k_ss : a.q_ss;
  const int64_t b = bh / heads, h = bh % heads;
  // the K/V head of this row (grouped-query: runs of H / Hkv query heads share one)
  const int64_t mrow = b * a.Hkv + (is_k ? h : h / (a.H / a.Hkv));
  const float* mean = is_k ? a.kmean : nullptr;               // centre K rows
  const float* qmu_mean = is_k ? nullptr : a.kmean;           // q.mu of Q rows
  float* qmu_out = is_k || !a.kmean ? nullptr : a.qmu;
  int8_t* codes = is_k ? a.k8 : a.q8;
  float* scales = is_k ? a.ks : a.qs;
  const uint16_t* src = (const uint16_t*)(is_k ? a.k : a.q) + b * (is_k ? a.k_sb : a.q_sb) +
                        h * (is_k ? a.k_sh : a.q_sh) + cg * 8;
  const int64_t j0 = (int64_t)(idx % rblocks) * (RPB * U) + threadIdx.x / G;

  uint4 w[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t j = j0 + u * RPB;
    const bool live = j < S && !is_pad(a.vbs, j);
    w[u] = live ? *(const uint4*)(src + j * ss) : make_uint4(0u, 0u, 0u, 0u);
  }
  float qm[8], mm[8];
  if (qmu_mean) {
    const float4 m0 = *(const float4*)(qmu_mean + mrow * D + cg * 8);
    const float4 m1 = *(const float4*)(qmu_mean + mrow * D + cg * 8 + 4);
    qm[0] = m0.x; qm[1] = m0.y; qm[2] = m0.z; qm[3] = m0.w; qm[4] = m1.x; qm[5] = m1.y; qm[6] = m1.z; qm[7] = m1.w;
  }
  if (mean) {
    const float4 m0 = *(const float4*)(mean + mrow * D + cg * 8);
    const float4 m1 = *(const float4*)(mean + mrow * D + cg * 8 + 4);
    mm[0] = m0.x; mm[1] = m0.y; mm[2] = m0.z; mm[3] = m0.w; mm[4] = m1.x; mm[5] = m1.y; mm[6] = m1.z; mm[7] = m1.w;
  }

#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t j = j0 + u * RPB;
    if (j >= S) break;   // uniform across the row's G lanes (G divides 64)
    const int64_t r = bh * S + j;
    const bool pad = is_pad(a.vbs, j);
    float x[8];
    unpack8<DT>(w[u], x);   // zeros for a pad row

    float qmu = 0.0f;
    if (qmu_mean) {
#pragma unroll
      for (int i = 0; i < 8; ++i) qmu += x[i] * qm[i];
    }
    if (mean) {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = __fsub_rn(x[i], mm[i]);  // one fp32 subtraction
    }

    float amax = 0.0f;
    bool finite = true;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      amax = fmaxf(amax, fabsf(x[i]));
      finite = finite && fabsf(x[i]) <= FLT_MAX;   // false for NaN and +-inf
    }
#pragma unroll
    for (int off = G / 2; off > 0; off >>= 1) {
      amax = fmaxf(amax, __shfl_xor(amax, off, G));
      if (qmu_out) qmu += __shfl_xor(qmu, off, G);
    }
    // a row with a non-finite element (on any of its G lanes, which are
    // consecutive lanes of the wave) gets codes 0, scale NaN and a NaN
    // centring term; the rows of lanes that left the loop are absent from
    // the ballot and do not matter here
    const uint64_t bad_lanes = __ballot(!finite);
    const int row_lane0 = (int)(threadIdx.x % 64) & ~(G - 1);
    const bool bad_row = ((bad_lanes >> row_lane0) & ((1ull << G) - 1ull)) != 0ull;   // G <= 16

    uint32_t lo = 0, hi = 0;
    float scale = bad_row ? __builtin_nanf("") : 0.0f;
    if (!pad && !bad_row && amax >= 127.0f * FLT_MIN) {
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
    *(uint2*)(codes + r * D + cg * 8) = make_uint2(lo, hi);
    if (cg == 0) {
      scales[r] = scale;
      if (qmu_out) qmu_out[r] = pad ? 0.0f : (bad_row ? __builtin_nanf("") : qmu);
    }
  }
}

template <int DT, int D>
hipError_t launch_dt_d(const QuantArgs& a, hipStream_t s) {
  const char* dn = DT == BF16 ? "bf16" : "fp16";
  const int64_t BHk = a.B * a.Hkv;
  if (a.kmean && a.Sk > 0 && BHk > 0) {
    const int nchunks = kmean_chunks(BHk, a.Sk);
    const int64_t chunk_rows = (a.Sk + nchunks - 1) / nchunks;
    const unsigned grid = (unsigned)(BHk * nchunks);
    debug_log("kmean_partial_kernel<%s, D=%d> grid %u x 256 (B*Hkv %lld, %d chunks of %lld rows); "
              "kmean_finalize_kernel grid %lld x 256", dn, D, grid, (long long)BHk, nchunks, (long long)chunk_rows,
              (long long)(BHk * (D / 32)));
    kmean_partial_kernel<DT, D><<<grid, 256, 0, s>>>(a, nchunks, chunk_rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    kmean_finalize_kernel<<<(unsigned)(BHk * (D / 32)), 256, 0, s>>>(a, nchunks);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  } else if (a.kmean && BHk > 0) {
    // no keys: the mean of nothing is 0 (the count is clamped to 1)
    const hipError_t e = launch_zero_words(a.kmean, BHk * D, s);
    if (e != hipSuccess) return e;
  }
  constexpr int rpb = 4 * (256 / (D / 8));   // rows per block: 4 per row slot
  const int k_rblocks = (int)((a.Sk + rpb - 1) / rpb);
  const int q_rblocks = (int)((a.Sq + rpb - 1) / rpb);
  const int64_t k_blocks = BHk * k_rblocks;
  const int64_t grid = k_blocks + a.B * a.H * q_rblocks;
  if (grid == 0) return hipSuccess;
  debug_log("quantize_kernel<%s, D=%d> grid %lld x 256 (K rows %lld in %lld blocks, centred %d; Q rows %lld, qmu %d)",
            dn, D, (long long)grid, (long long)(BHk * a.Sk), (long long)k_blocks, a.kmean != nullptr,
            (long long)(a.B * a.H * a.Sq), a.kmean != nullptr && a.qmu != nullptr);
  quantize_kernel<DT, D><<<(unsigned)grid, 256, 0, s>>>(a, k_blocks, k_rblocks, q_rblocks);
  return hipGetLastError();
}

}  // namespace

// Scratch of qfa_quantize_qk_noalloc: the K-mean partials of a call, at most
// kMeanSlots slots of up to 128 channels (8 MiB). Every slot a call reads was
// written earlier in the same call, so nothing in it needs clearing; calls
// that overlap on one GPU share it and race.
constexpr size_t kNoAllocScratchBytes = (size_t)kMeanSlots * 128 * 16;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void** ptr, size_t* bytes) {
  // the device address of each GPU's copy of `scratch`, taken once per device
  // with that device current (host code never uses the array's name itself)
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* per_device[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (per_device[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    per_device[dev] = p;
  }
  *ptr = per_device[dev];
  *bytes = kNoAllocScratchBytes;
  return hipSuccess;
}

hipError_t launch_quantize(const QuantArgs& a, hipStream_t s) {
  if (a.D == 128) return a.dtype == BF16 ? launch_dt_d<BF16, 128>(a, s) : launch_dt_d<FP16, 128>(a, s);
  return a.dtype == BF16 ? launch_dt_d<BF16, 64>(a, s) : launch_dt_d<FP16, 64>(a, s);
}

}  // namespace qfa
