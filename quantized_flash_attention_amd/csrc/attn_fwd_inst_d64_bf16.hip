// Instances of the attention kernel (attn_fwd_kernel.h) for head dimension
// 64 and bf16 V: one of four translation units compiled in parallel.
#include "attn_fwd_kernel.h"

namespace qfa {

hipError_t launch_attn_d64_bf16(const AttnArgs& a, hipStream_t s) { return launch_d_vt<64, BF16>(a, s); }
hipError_t launch_qk_dump_d64(const AttnArgs& a, hipStream_t s) { return launch_qk_dump_d<64>(a, s); }

}  // namespace qfa
