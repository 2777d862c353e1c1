// Host dispatch of the attention forward: derived segment tables, the CU
// count, and the choice of the (head dimension, V type) instance set; the
// kernel is in attn_fwd_kernel.h, its instances in attn_fwd_inst_*.hip
// (four translation units compiled in parallel).
#include "attn_fwd_kernel.h"

#include <atomic>

namespace qfa {

hipError_t launch_attn_d128_bf16(const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_d128_fp16(const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_d64_bf16(const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_d64_fp16(const AttnArgs& a, hipStream_t s);
hipError_t launch_qk_dump_d128(const AttnArgs& a, hipStream_t s);
hipError_t launch_qk_dump_d64(const AttnArgs& a, hipStream_t s);

namespace {

// Derived segment tables of a dense call (up to 4 key segments).
void derive_segments(AttnArgs& a) {
  int cum = 0;
  for (int g = 0; g < 4; ++g) {
    const bool live = g < a.nseg && a.seg_hi[g] > a.seg_lo[g];
    a.seg_t0[g] = live ? a.seg_lo[g] / BN : 0;
    a.seg_cum[g] = g < a.nseg ? cum : INT32_MAX;
    if (live) cum += (a.seg_hi[g] + BN - 1) / BN - a.seg_lo[g] / BN;
  }
  a.seg_ntiles = cum;
}

}  // namespace

hipError_t device_cu_count(int* ncu) {
  // queried once per device
  static std::atomic<int> ncu_of[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  int n = dev >= 0 && dev < 64 ? ncu_of[dev].load(std::memory_order_relaxed) : 0;
  if (n == 0) {
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < 64) ncu_of[dev].store(n, std::memory_order_relaxed);
  }
  *ncu = n;
  return hipSuccess;
}

hipError_t launch_qk_scores(const AttnArgs& args, hipStream_t s) {
  AttnArgs a = args;
  derive_segments(a);
  return a.D == 128 ? launch_qk_dump_d128(a, s) : launch_qk_dump_d64(a, s);
}

hipError_t launch_attn_fwd(const AttnArgs& args, hipStream_t s) {
  AttnArgs a = args;
  derive_segments(a);
  if (a.nsplit < 1 || a.index) a.nsplit = 1;
  if (a.causal) {
    const hipError_t e = device_cu_count(&a.ncu);
    if (e != hipSuccess) return e;
  }
  if (a.D == 128) return a.v_dtype == BF16 ? launch_attn_d128_bf16(a, s) : launch_attn_d128_fp16(a, s);
  return a.v_dtype == BF16 ? launch_attn_d64_bf16(a, s) : launch_attn_d64_fp16(a, s);
}

}  // namespace qfa
