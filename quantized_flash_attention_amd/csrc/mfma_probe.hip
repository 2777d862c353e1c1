// On-box ceiling of the attention kernel's matrix-core work (measurement
// only; not part of the attention path). Every wave issues, per iteration,
// the MFMA mix of one 32-row x 64-key attention tile: 8 x
// v_mfma_i32_32x32x32_i8 (Q K^T) and 16 x v_mfma_f32_32x32x16_bf16 (P V),
// into independent accumulators like the kernel's, on operands drawn at random
// per lane and rotated over four register sets so that consecutive MFMAs see
// different data (the power the matrix cores draw depends on it). The launch
// shape is the attention kernel's: 256-thread blocks, two per CU.
// Wave 0 of each block records the shader-clock counter (s_memtime) and the
// constant 100 MHz counter (s_memrealtime) around its loop, so the host gets
// the clock the loop ran at.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qfa_probe.h"

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  // a 32-bit integer hash (xor-shift-multiply) for the operand draws
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// a bf16 of roughly unit scale from 16 random bits: sign, exponent 2^-2..2^1, 7 mantissa bits
__device__ __forceinline__ uint16_t rand_bf16(uint32_t r) {
  const uint32_t sign = (r & 1u) << 15, e = 125u + ((r >> 1) & 3u), m = (r >> 3) & 0x7fu;
  return (uint16_t)(sign | (e << 7) | m);
}

// The VALU work of one attention tile per wave (32 scores per lane): dequantize
// (fma), row max (max3 tree), exp argument (fma), exp2, pack pairs to bf16,
// row sum of the packed pairs (dot2): 64 fma + 16 max + 32 exp + 16 cvt + 16
// dot2. Independent of the MFMA operands and results; the inputs change with
// every iteration through the carried sums, so nothing is hoisted.
__device__ __forceinline__ void valu_tile(const float (&x)[32], float (&acc)[4], float& carry) {
  typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
  const float ka = 1.0f + carry * 1e-30f, kb = carry * 1e-30f - 0.5f;
  float t[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) t[i] = fmaf(x[i], ka, kb);
  float m = t[0];
#pragma unroll
  for (int i = 1; i < 31; i += 2) m = fmaxf(m, fmaxf(t[i], t[i + 1]));
  m = fmaxf(m, t[31]);
  const float kc = 1.4426950408889634f;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const float p0 = __builtin_amdgcn_exp2f(fmaf(t[2 * e], kc, -m));
    const float p1 = __builtin_amdgcn_exp2f(fmaf(t[2 * e + 1], kc, -m));
    const v2bf pair = {(__bf16)p0, (__bf16)p1};
    acc[e & 3] = __builtin_amdgcn_fdot2_f32_bf16(pair, v2bf{(__bf16)1.0f, (__bf16)1.0f}, acc[e & 3], false);
  }
  carry = acc[0] + m;
}

// MFMAs whose accumulators live in AccVGPRs (inline assembly with the "a"
// constraint), for mixes 9 and 10
__device__ __forceinline__ void mfma_bf16_acc(v16f& c, const v8bf& a, const v8bf& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_i8_acc(v16i& c, const v4i& a, const v4i& b) {
  asm volatile("v_mfma_i32_32x32x32_i8 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}

template <int MIX>
__global__ __launch_bounds__(256, 2) void mfma_probe_kernel(int iters, unsigned long long* clocks, float* sink) {
  const uint32_t seed = (uint32_t)(blockIdx.x * 256 + threadIdx.x) * 0x9e3779b9u;
  v4i a8[4], b8[4];
  v8bf af[4], bf[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // int8 codes of the full symmetric range [-127, 127]
      uint32_t w = 0, r = mix32(seed + 97u * (16u * s + i));
#pragma unroll
      for (int byte = 0; byte < 4; ++byte) {
        const uint32_t code = (uint32_t)((int)((r >> (8 * byte)) % 255u) - 127) & 0xffu;
        w |= code << (8 * byte);
      }
      if (i < 4) a8[s][i] = (int)w;
      else b8[s][i - 4] = (int)w;
    }
    uint16_t ha[8], hb[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ha[i] = rand_bf16(mix32(seed + 131u * (8u * s + i) + 7u));
      hb[i] = rand_bf16(mix32(seed + 131u * (8u * s + i) + 11u));
    }
    if (MIX >= 5) {
      // constant operands: every int8 code 1, every bf16 value 1.0 (no data toggling)
#pragma unroll
      for (int i = 0; i < 8; ++i) ha[i] = hb[i] = 0x3f80u;
#pragma unroll
      for (int i = 0; i < 4; ++i) a8[s][i] = b8[s][i] = 0x01010101;
    }
    af[s] = __builtin_bit_cast(v8bf, ha);
    bf[s] = __builtin_bit_cast(v8bf, hb);
  }
  v16i acc_i[2] = {v16i{}, v16i{}};
  v16f acc_f[4] = {v16f{}, v16f{}, v16f{}, v16f{}};
  float xv[32], vacc[4] = {0.0f, 0.0f, 0.0f, 0.0f}, carry = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) xv[i] = (float)(mix32(seed + 1000u + i) & 0xffffu) * (8.0f / 65536.0f) - 4.0f;

  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  // four iterations per pass, so every operand rotation is a constant register choice
  for (int it = 0; it < iters; it += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (MIX >= 3) valu_tile(xv, vacc, carry);
      if (MIX == 9 || MIX == 10) {
        // accumulators in AccVGPRs: bf16 (PV-like) ones in mix 9, all in mix 10
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          if (MIX == 10) mfma_i8_acc(acc_i[k & 1], a8[k & 3], b8[(k + u) & 3]);
          else acc_i[k & 1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a8[k & 3], b8[(k + u) & 3], acc_i[k & 1], 0, 0, 0);
        }
#pragma unroll
        for (int k = 0; k < 16; ++k) mfma_bf16_acc(acc_f[k & 3], af[(k >> 2) & 3], bf[(k + u) & 3]);
        continue;
      }
      if (MIX != 2 && MIX != 4 && MIX != 5) {
#pragma unroll
        for (int k = 0; k < 8; ++k)
          acc_i[k & 1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a8[k & 3], b8[(k + u) & 3], acc_i[k & 1], 0, 0, 0);
      }
      if (MIX != 1 && MIX != 4) {
#pragma unroll
        for (int k = 0; k < 16; ++k)
          acc_f[k & 3] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[(k >> 2) & 3], bf[(k + u) & 3], acc_f[k & 3], 0, 0, 0);
      }
    }
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();

  float s = vacc[0] + vacc[1] + vacc[2] + vacc[3] + carry;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s += (float)(acc_i[0][r] ^ acc_i[1][r]);
    s += acc_f[0][r] + acc_f[1][r] + acc_f[2][r] + acc_f[3][r];
  }
  sink[blockIdx.x * 256 + threadIdx.x] = s;   // keeps every MFMA live
  if (threadIdx.x == 0) {
    clocks[2 * blockIdx.x] = t1 - t0;
    clocks[2 * blockIdx.x + 1] = r1 - r0;
  }
}

// Two groups of 4 waves per block (one block per CU, so each SIMD holds one
// wave of each group), alternating a matrix phase (the tile's 24 MFMAs) and a
// vector phase (the tile's softmax VALU work) between block barriers. OFFSET:
// the second group runs one phase behind, so at any time one wave of each SIMD
// is in its matrix phase and the other in its vector phase; without it both
// waves of a SIMD run the same phase.
template <bool OFFSET>
__global__ __launch_bounds__(512, 1) void pingpong_probe_kernel(int iters, unsigned long long* clocks, float* sink) {
  const uint32_t seed = (uint32_t)(blockIdx.x * 512 + threadIdx.x) * 0x9e3779b9u;
  const int group = threadIdx.x / 256;
  v4i a8[4], b8[4];
  v8bf af[4], bf[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t w = 0, r = mix32(seed + 97u * (16u * s + i));
#pragma unroll
      for (int byte = 0; byte < 4; ++byte) {
        const uint32_t code = (uint32_t)((int)((r >> (8 * byte)) % 255u) - 127) & 0xffu;
        w |= code << (8 * byte);
      }
      if (i < 4) a8[s][i] = (int)w;
      else b8[s][i - 4] = (int)w;
    }
    uint16_t ha[8], hb[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ha[i] = rand_bf16(mix32(seed + 131u * (8u * s + i) + 7u));
      hb[i] = rand_bf16(mix32(seed + 131u * (8u * s + i) + 11u));
    }
    af[s] = __builtin_bit_cast(v8bf, ha);
    bf[s] = __builtin_bit_cast(v8bf, hb);
  }
  v16i acc_i[2] = {v16i{}, v16i{}};
  v16f acc_f[4] = {v16f{}, v16f{}, v16f{}, v16f{}};
  float xv[32], vacc[4] = {0.0f, 0.0f, 0.0f, 0.0f}, carry = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) xv[i] = (float)(mix32(seed + 1000u + i) & 0xffffu) * (8.0f / 65536.0f) - 4.0f;
  auto barrier = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  if (OFFSET && group == 1) barrier();
  for (int it = 0; it < iters; it += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      valu_tile(xv, vacc, carry);
      barrier();
#pragma unroll
      for (int k = 0; k < 8; ++k)
        acc_i[k & 1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a8[k & 3], b8[(k + u) & 3], acc_i[k & 1], 0, 0, 0);
#pragma unroll
      for (int k = 0; k < 16; ++k)
        acc_f[k & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[(k >> 2) & 3], bf[(k + u) & 3], acc_f[k & 3], 0, 0, 0);
      barrier();
    }
  }
  if (OFFSET && group == 0) barrier();
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();

  float s = vacc[0] + vacc[1] + vacc[2] + vacc[3] + carry;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s += (float)(acc_i[0][r] ^ acc_i[1][r]);
    s += acc_f[0][r] + acc_f[1][r] + acc_f[2][r] + acc_f[3][r];
  }
  sink[blockIdx.x * 512 + threadIdx.x] = s;
  if (threadIdx.x == 0) {
    clocks[2 * blockIdx.x] = t1 - t0;
    clocks[2 * blockIdx.x + 1] = r1 - r0;
  }
}

}  // namespace

extern "C" int qfa_probe_mfma(int blocks, int iters, int mix, unsigned long long* clocks, float* sink, void* stream) {
  if (blocks <= 0 || iters <= 0 || iters % 4 || !clocks || !sink || mix < 0 || mix > 10) return 1;
  hipStream_t s = (hipStream_t)stream;
  if (mix == 0) mfma_probe_kernel<0><<<blocks, 256, 0, s>>>(iters, clocks, sink);
  else if (mix == 1) mfma_probe_kernel<1><<<blocks, 256, 0, s>>>(iters, clocks, sink);
  else if (mix == 2) mfma_probe_kernel<2><<<blocks, 256, 0, s>>>(iters, clocks, sink);
  else if (mix == 3) mfma_probe_kernel<3><<<blocks, 256, 0, s>>>(iters, clocks, sink);
  else if (mix == 4) mfma_probe_kernel<4><<<blocks, 256, 0, s>>>(iters, clocks, sink);
  else if (mix == 5) mfma_probe_kernel<5><<<blocks, 256, 0, s>>>(iters, clocks, sink);
  else if (mix == 6) mfma_probe_kernel<6><<<blocks, 256, 0, s>>>(iters, clocks, sink);
  // blocks of 8 waves, one per CU: half as many blocks for the same waves per SIMD
  else if (mix == 7) pingpong_probe_kernel<true><<<(blocks + 1) / 2, 512, 0, s>>>(iters, clocks, sink);
  else if (mix == 8) pingpong_probe_kernel<false><<<(blocks + 1) / 2, 512, 0, s>>>(iters, clocks, sink);
  else if (mix == 9) mfma_probe_kernel<9><<<blocks, 256, 0, s>>>(iters, clocks, sink);
  else mfma_probe_kernel<10><<<blocks, 256, 0, s>>>(iters, clocks, sink);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}
