// Tile mask -> ascending key-tile lists (FastVideo API docs,
// "minimax_h3_sparse_int8", sparse_sm89_attention: map_to_index turns the
// [B,H,T,T] tile mask into per-query-tile index lists and counts).
//
// One wave per mask row. Rows of 16-byte aligned bytes (Tk a multiple of 16,
// aligned base): each lane takes 16 mask bytes per step (1024 per wave),
// counts its set tiles, and a wave prefix sum of the counts gives it its
// first slot; lane order is tile order, so the list comes out ascending.
// Other rows: each step reads one byte per lane, a ballot marks the set tiles
// and mbcnt gives every set lane its slot.
#include "qfa_internal.h"

namespace qfa {
namespace {

__global__ __launch_bounds__(256) void blockmask_to_index_kernel(const uint8_t* mask, int64_t rows, int64_t Tk,
                                                                 int32_t* index, int32_t* count) {
  const int64_t row = (int64_t)blockIdx.x * 4 + threadIdx.x / 64;
  const int lane = threadIdx.x % 64;
  if (row >= rows) return;  // whole waves leave together
  const uint8_t* m = mask + row * Tk;
  int32_t* out = index + row * Tk;
  int32_t c = 0;
  for (int64_t t0 = 0; t0 < Tk; t0 += 64) {
    const int64_t t = t0 + lane;
    const bool f = t < Tk && m[t] != 0;
    const uint64_t bal = __ballot(f);
    const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
    if (f) out[c + below] = (int32_t)t;
    c += (int32_t)__popcll(bal);
  }
  if (lane == 0) count[row] = c;
}

__global__ __launch_bounds__(256) void blockmask_to_index16_kernel(const uint8_t* mask, int64_t rows, int64_t Tk,
                                                                   int32_t* index, int32_t* count) {
  const int64_t row = (int64_t)blockIdx.x * 4 + threadIdx.x / 64;
  const int lane = threadIdx.x % 64;
  if (row >= rows) return;  // whole waves leave together
  const uint8_t* m = mask + row * Tk;
  int32_t* out = index + row * Tk;
  int32_t c = 0;
  for (int64_t t0 = 0; t0 < Tk; t0 += 1024) {
    const int64_t tl = t0 + 16 * lane;
    uint32_t bits = 0;   // bit b: tile tl + b is attended
    if (tl < Tk) {       // Tk is a multiple of 16: the lane's 16 bytes lie inside the row
      const uint4 w = *(const uint4*)(m + tl);
      const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int b = 0; b < 4; ++b) bits |= (((wd[i] >> (8 * b)) & 0xffu) != 0u ? 1u : 0u) << (4 * i + b);
    }
    const int n = __popc(bits);
    int incl = n;   // inclusive prefix sum of the lane counts
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(incl, d, 64);
      if (lane >= d) incl += y;
    }
    int pos = c + incl - n;
    while (bits) {
      const int b = __builtin_ctz(bits);
      bits &= bits - 1u;
      out[pos++] = (int32_t)(tl + b);
    }
    c += __shfl(incl, 63, 64);
  }
  if (lane == 0) count[row] = c;
}

__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0u;
}

}  // namespace

hipError_t launch_zero_words(void* p, int64_t words, hipStream_t s) {
  if (words <= 0) return hipSuccess;
  const int64_t blocks = (words + 255) / 256;
  debug_log("zero_words_kernel grid %lld x 256 (words %lld)", (long long)(blocks < 4096 ? blocks : 4096), (long long)words);
  zero_words_kernel<<<(unsigned)(blocks < 4096 ? blocks : 4096), 256, 0, s>>>((uint32_t*)p, words);
  return hipGetLastError();
}

hipError_t launch_blockmask_to_index(const uint8_t* mask, int64_t rows, int64_t Tk, int32_t* index, int32_t* count,
                                     hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const unsigned grid = (unsigned)((rows + 3) / 4);
  debug_log("%s grid %u x 256 (rows %lld, Tk %lld)",
            Tk % 16 == 0 && (uintptr_t)mask % 16 == 0 ? "blockmask_to_index16_kernel" : "blockmask_to_index_kernel", grid,
            (long long)rows, (long long)Tk);
  if (Tk % 16 == 0 && (uintptr_t)mask % 16 == 0)
    blockmask_to_index16_kernel<<<grid, 256, 0, s>>>(mask, rows, Tk, index, count);
  else
    blockmask_to_index_kernel<<<grid, 256, 0, s>>>(mask, rows, Tk, index, count);
  return hipGetLastError();
}

}  // namespace qfa
