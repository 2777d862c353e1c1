// Exact merge of two partial softmaxes by their LSE (comfy-kitchen issue
// #177, Question 2: a window split into an unmasked core call and a masked
// skirt call; FlyDSL PR #886: combining splits from the combined max and
// denominator). HBM-bound: one row of D channels per D/8 lanes, 8 channels
// per lane, fp32 arithmetic.
#include "qfa_internal.h"

namespace qfa {
namespace {

__device__ __forceinline__ void load8(const void* p, int dtype, int64_t off, float* f) {
  if (dtype == FP32) {
    const float4 a = *(const float4*)((const float*)p + off);
    const float4 b = *(const float4*)((const float*)p + off + 4);
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  } else {
    const uint4 w = *(const uint4*)((const uint16_t*)p + off);
    if (dtype == BF16) unpack8<BF16>(w, f);
    else unpack8<FP16>(w, f);
  }
}

__device__ __forceinline__ void store8(void* p, int dtype, int64_t off, const float* f) {
  if (dtype == FP32) {
    *(float4*)((float*)p + off) = make_float4(f[0], f[1], f[2], f[3]);
    *(float4*)((float*)p + off + 4) = make_float4(f[4], f[5], f[6], f[7]);
  } else {
    uint32_t w[4];
    for (int i = 0; i < 4; ++i) {
      if (dtype == BF16) w[i] = float_to_bf16_bits(f[2 * i]) | (float_to_bf16_bits(f[2 * i + 1]) << 16);
      else w[i] = float_to_half_bits(f[2 * i]) | (float_to_half_bits(f[2 * i + 1]) << 16);
    }
    *(uint4*)((uint16_t*)p + off) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

template <int D>
__global__ __launch_bounds__(256) void lse_merge_kernel(MergeArgs a) {
  constexpr int G = D / 8;
  constexpr int RPB = 256 / G;
  const int cg = threadIdx.x % G;
  const int64_t r = (int64_t)blockIdx.x * RPB + threadIdx.x / G;
  if (r >= a.B * a.H * a.S) return;
  const int64_t bh = r / a.S, s = r % a.S, b = bh / a.H, h = bh % a.H;
  const float la = a.la[r], lb = a.lb[r];
  const float m = fmaxf(la, lb);
  float out[8];
  float L;
  if (m == -INFINITY) {
    for (int i = 0; i < 8; ++i) out[i] = 0.0f;
    L = -INFINITY;
  } else {
    const float wa = expf(la - m), wb = expf(lb - m);
    const float inv = 1.0f / (wa + wb);
    float fa[8], fb[8];
    load8(a.oa, a.a_dtype, b * a.a_sb + h * a.a_sh + s * a.a_ss + cg * 8, fa);
    load8(a.ob, a.b_dtype, b * a.b_sb + h * a.b_sh + s * a.b_ss + cg * 8, fb);
    for (int i = 0; i < 8; ++i) out[i] = (wa * fa[i] + wb * fb[i]) * inv;
    L = m + logf(wa + wb);
  }
  store8(a.o, a.o_dtype, b * a.o_sb + h * a.o_sh + s * a.o_ss + cg * 8, out);
  if (a.l && cg == 0) a.l[r] = L;
}

// n partials of one row: m = max_k L_k; w_k = exp(L_k - m); O = sum_k w_k O_k
// / sum_k w_k; L = m + log(sum_k w_k) (FlyDSL PR #886: the split-K combine
// from the combined max and denominator). Empty partials (L_k = -inf) weigh
// 0 and are not read; a row empty in every split gives O = 0, L = -inf.
template <int D>
__global__ __launch_bounds__(256) void split_combine_kernel(CombineArgs a) {
  constexpr int G = D / 8;
  constexpr int RPB = 256 / G;
  const int cg = threadIdx.x % G;
  const int64_t rows = a.B * a.H * a.S;
  const int64_t r = (int64_t)blockIdx.x * RPB + threadIdx.x / G;
  if (r >= rows) return;
  const int64_t bh = r / a.S, s = r % a.S, b = bh / a.H, h = bh % a.H;
  float m = -INFINITY;
  for (int k = 0; k < a.nsplit; ++k) m = fmaxf(m, a.pl[k * rows + r]);
  float out[8];
  for (int i = 0; i < 8; ++i) out[i] = 0.0f;
  float L = -INFINITY;
  if (m != -INFINITY) {
    float wsum = 0.0f;
    for (int k = 0; k < a.nsplit; ++k) {
      const float lk = a.pl[k * rows + r];
      if (lk == -INFINITY) continue;
      const float w = expf(lk - m);
      wsum += w;
      float f[8];
      load8(a.po, FP32, (k * rows + r) * D + cg * 8, f);
      for (int i = 0; i < 8; ++i) out[i] += w * f[i];
    }
    const float inv = 1.0f / wsum;
    for (int i = 0; i < 8; ++i) out[i] *= inv;
    L = m + logf(wsum);
  }
  store8(a.o, a.o_dtype, b * a.o_sb + h * a.o_sh + s * a.o_ss + cg * 8, out);
  if (a.l && cg == 0) a.l[r] = L;
}

}  // namespace

hipError_t launch_split_combine(const CombineArgs& a, hipStream_t s) {
  const int64_t rows = a.B * a.H * a.S;
  if (rows == 0) return hipSuccess;
  const int rpb = 256 / (int)(a.D / 8);
  const unsigned grid = (unsigned)((rows + rpb - 1) / rpb);
  debug_log("split_combine_kernel<D=%lld> grid %u x 256 (rows %lld, splits %d)", (long long)a.D, grid, (long long)rows,
            a.nsplit);
  if (a.D == 128) split_combine_kernel<128><<<grid, 256, 0, s>>>(a);
  else split_combine_kernel<64><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_lse_merge(const MergeArgs& a, hipStream_t s) {
  const int64_t rows = a.B * a.H * a.S;
  if (rows == 0) return hipSuccess;
  const int rpb = 256 / (int)(a.D / 8);
  const unsigned grid = (unsigned)((rows + rpb - 1) / rpb);
  debug_log("lse_merge_kernel<D=%lld> grid %u x 256 (rows %lld)", (long long)a.D, grid, (long long)rows);
  if (a.D == 128) lse_merge_kernel<128><<<grid, 256, 0, s>>>(a);
  else lse_merge_kernel<64><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace qfa
