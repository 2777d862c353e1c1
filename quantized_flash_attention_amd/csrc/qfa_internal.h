// Internal interface between the C-ABI layer (api.cpp) and the gfx950 kernels.
// Argument checking happens in api.cpp; the launchers below trust their input.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qfa {

enum DType : int { BF16 = 1, FP16 = 2, FP32 = 3, BOOL = 4 };

// Quantize step: K mean, then int8 codes of every Q and K row.
//  - The K mean is summed in double-double partials over row chunks of at
//    least kMeanMinChunkRows rows per (b, K/V head), at most kMeanMaxChunks
//    chunks per head and kMeanSlots in all (fewer chunks per head when B*Hkv
//    is large). Smaller chunks measured slower on short heads (more partials
//    to combine, blocks too short to hide their start-up); the chunk cap
//    lets long heads spread over the whole chip. A second small launch
//    combines each head's partials into the mean. (Combining them in the
//    last block of each head instead needs a device-scope fence in every
//    block, an L2-wide write-back and invalidate that serialise per XCD: it
//    measured 8x slower than the whole partial pass.)
//  - One launch then quantizes all K rows (centred) and all Q rows.
constexpr int kMeanMaxChunks = 256;
constexpr int64_t kMeanSlots = 4096;
constexpr int64_t kMeanMinChunkRows = 256;

// chunks per (b, K/V head) of a call with BH = B*Hkv heads of Sk keys
__host__ __device__ inline int kmean_chunks(int64_t BH, int64_t Sk) {
  if (BH <= 0 || Sk <= 0) return 0;
  int64_t p = (Sk + kMeanMinChunkRows - 1) / kMeanMinChunkRows;
  if (p > kMeanMaxChunks) p = kMeanMaxChunks;
  const int64_t cap = kMeanSlots / BH;
  if (p > cap) p = cap;
  return (int)(p < 1 ? 1 : p);
}

// workspace of a centring call: the partials [BH][chunks][D] (double2)
__host__ __device__ inline int64_t quantize_workspace_size(int64_t BH, int64_t Sk, int64_t D) {
  return BH > 0 && Sk > 0 ? BH * kmean_chunks(BH, Sk) * D * 16 : 0;
}

struct QuantArgs {
  int dtype;                      // BF16 or FP16 (Q and K)
  int64_t B, H, Hkv, Sq, Sk, D;
  const void* q;
  int64_t q_sb, q_sh, q_ss;
  const void* k;
  int64_t k_sb, k_sh, k_ss;
  const int32_t* vbs;             // nullable: per-tile valid counts (Sq == Sk)
  int8_t* q8;                     // [B*H*Sq, D]
  float* qs;                      // [B*H*Sq]
  float* qmu;                     // nullable [B*H*Sq] (centring only)
  int8_t* k8;                     // [B*Hkv*Sk, D]
  float* ks;                      // [B*Hkv*Sk]
  float* kmean;                   // nullable [B*Hkv, D]: centre K
  void* workspace;                // quantize_workspace_size bytes (centring with Sk > 0)
};
hipError_t launch_quantize(const QuantArgs& a, hipStream_t s);
// device address and size of this GPU's scratch for qfa_quantize_qk_noalloc
hipError_t noalloc_scratch(void** ptr, size_t* bytes);

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

// Launch log: with the environment variable QFA_DEBUG set to a nonzero
// value, every launch prints one line to stderr naming the kernel instance,
// its grid and its arguments' shape. Checked once per process.
bool debug_enabled();
void debug_log(const char* fmt, ...) __attribute__((format(printf, 1, 2)));

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
