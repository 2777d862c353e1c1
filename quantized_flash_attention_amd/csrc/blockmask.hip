// Tile mask -> ascending key-tile lists (FastVideo API docs,
// "minimax_h3_sparse_int8", sparse_sm89_attention: map_to_index turns the
// [B,H,T,T] tile mask into per-query-tile index lists and counts).
//
// One wave per mask row: each step reads 64 mask bytes, a ballot marks the
// attended tiles and mbcnt gives every set lane its slot, so the list comes
// out in ascending order with one coalesced store per step.
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

__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0u;
}

}  // namespace

hipError_t launch_zero_words(void* p, int64_t words, hipStream_t s) {
  if (words <= 0) return hipSuccess;
  const int64_t blocks = (words + 255) / 256;
  zero_words_kernel<<<(unsigned)(blocks < 4096 ? blocks : 4096), 256, 0, s>>>((uint32_t*)p, words);
  return hipGetLastError();
}

hipError_t launch_blockmask_to_index(const uint8_t* mask, int64_t rows, int64_t Tk, int32_t* index, int32_t* count,
                                     hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const unsigned grid = (unsigned)((rows + 3) / 4);
  blockmask_to_index_kernel<<<grid, 256, 0, s>>>(mask, rows, Tk, index, count);
  return hipGetLastError();
}

}  // namespace qfa
