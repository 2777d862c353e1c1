// Internal interface between the C-ABI layer (api.cpp) and the gfx950 kernels.
// Argument checking happens in api.cpp; the launchers below trust their input.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qfa {

enum DType : int { BF16 = 1, FP16 = 2, FP32 = 3, BOOL = 4 };

// K mean: partial sums per (bh, chunk) in double-double, then one finalize.
constexpr int kMeanChunkRows = 256;

struct MeanArgs {
  const void* k;
  int dtype;
  int64_t B, H, S, D;
  int64_t sb, sh, ss;
  const int32_t* vbs;   // nullable
  double2* partial;     // [B*H, nchunks, D] (hi, lo)
  float* mean;          // [B*H, D]
  int nchunks;
};
hipError_t launch_kmean(const MeanArgs& a, hipStream_t s);

struct QuantRowsArgs {
  const void* x;
  int dtype;
  int64_t B, H, S, D;
  int64_t sb, sh, ss;
  const float* mean;    // nullable: centre rows by mean[b, h / (H / mean_heads), :]
  const float* qmu_mean;// nullable: compute qmu = x . qmu_mean[b, h / (H / mean_heads), :] into qmu
  int64_t mean_heads;   // heads of mean / qmu_mean (K's heads; divides H)
  const int32_t* vbs;   // nullable
  int8_t* codes;        // [B*H*S, D]
  float* scale;         // [B*H*S]
  float* qmu;           // nullable [B*H*S]
};
hipError_t launch_quantize_rows(const QuantRowsArgs& a, hipStream_t s);

// Clears `words` 32-bit words with a fill kernel (never a memset node, so a
// captured graph replays it faithfully).
hipError_t launch_zero_words(void* p, int64_t words, hipStream_t s);

hipError_t launch_blockmask_to_index(const uint8_t* mask, int64_t rows, int64_t Tk, int32_t* index,
                                     int32_t* count, hipStream_t s);

struct AttnArgs {
  int B, H, Hkv, Sq, Sk, D;   // query head h reads K/V head h / (H / Hkv)
  const int8_t* q8;
  const float* qs;
  const float* qmu;     // nullable
  const int8_t* k8;
  const float* ks;
  // unquantized Q K^T (qf != nullptr): Q [B,H,Sq,D] and K [B,Hkv,Sk,D] of
  // v_dtype with element strides; q8, qs, qmu, k8, ks are then unused
  const void* qf;
  const void* kf;
  int64_t q_sb, q_sh, q_ss, k_sb, k_sh, k_ss;
  const void* v;
  int v_dtype;
  int64_t v_sb, v_sh, v_ss;
  float sm_scale;
  const void* bias;     // nullable; bias_dtype BOOL: a keep mask (nonzero bytes attend)
  int bias_dtype;
  int64_t bias_sb, bias_sh;
  int64_t bias_sq;      // 0: one value per key shared by every query; else the query stride
  const int32_t* index; // nullable (dense)
  const int32_t* count;
  const int32_t* vbs;   // nullable
  const float* v_scale; // nullable [Hkv, D]
  int nseg;
  int seg_lo[4], seg_hi[4];
  int causal;           // self-attention with key j > row i excluded (Sq == Sk, one segment [0, Sk))
  int ncu;              // compute units of the device (block order of causal calls)
  // split-K: each (query block, head) walk is cut into nsplit contiguous
  // ranges, one block each; with nsplit > 1 a block writes its normalised
  // fp32 partial O to part_o [nsplit][B*H*Sq][D] and its LSE to part_lse
  // [nsplit][B*H*Sq] instead of out/lse (dense calls only)
  int nsplit;
  float* part_o;
  float* part_lse;
  // derived by the launcher from the segments: first key tile of segment g,
  // number of tiles before segment g (INT32_MAX for absent segments), and
  // the total number of key tiles of the call
  int seg_t0[4], seg_cum[4];
  int seg_ntiles;
  void* out;
  int out_dtype;
  int64_t o_sb, o_sh, o_ss;
  float* lse;           // nullable
};
hipError_t launch_attn_fwd(const AttnArgs& a, hipStream_t s);
// compute units of the current device (cached per device)
hipError_t device_cu_count(int* ncu);
// int32 scores of the attention kernel's QK stage into a.out (int32 [B,H,Sq,Sk]);
// uses q8, k8, sizes and one segment [0, Sk).
hipError_t launch_qk_scores(const AttnArgs& a, hipStream_t s);

struct MergeArgs {
  int64_t B, H, S, D;
  const void* oa; int a_dtype; int64_t a_sb, a_sh, a_ss; const float* la;
  const void* ob; int b_dtype; int64_t b_sb, b_sh, b_ss; const float* lb;
  void* o; int o_dtype; int64_t o_sb, o_sh, o_ss; float* l;
};
hipError_t launch_lse_merge(const MergeArgs& a, hipStream_t s);

// n-way combine of split partials by their LSE into O (+ LSE)
struct CombineArgs {
  int64_t B, H, S, D;
  int nsplit;
  const float* po;      // [nsplit][B*H*S][D] fp32, normalised partial outputs
  const float* pl;      // [nsplit][B*H*S] fp32 partial LSEs (-inf: nothing attended)
  void* o; int o_dtype; int64_t o_sb, o_sh, o_ss; float* l;   // l nullable
};
hipError_t launch_split_combine(const CombineArgs& a, hipStream_t s);

// ---- device helpers ----------------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_float(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
  _Float16 x = __builtin_bit_cast(_Float16, (uint16_t)h);
  return (float)x;
}

// Unpack 8 16-bit values held in a 16-byte word.
template <int DT>
__device__ __forceinline__ void unpack8(const uint4 w, float* f) {
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (DT == BF16) {
      f[2 * i] = bf16_bits_to_float(u[i] & 0xffffu);
      f[2 * i + 1] = bf16_bits_to_float(u[i] >> 16);
    } else {
      f[2 * i] = half_bits_to_float(u[i] & 0xffffu);
      f[2 * i + 1] = half_bits_to_float(u[i] >> 16);
    }
  }
}

// Round-to-nearest-even fp32 -> bf16 bits (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint32_t float_to_bf16_bits(float f) {
  __bf16 b = (__bf16)f;
  return (uint32_t)__builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ uint32_t float_to_half_bits(float f) {
  _Float16 h = (_Float16)f;
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

}  // namespace qfa
