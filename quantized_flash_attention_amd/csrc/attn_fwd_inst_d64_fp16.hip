// Instances of the attention kernel (attn_fwd_kernel.h) for head dimension
// 64 and fp16 V: one of four translation units compiled in parallel.
#include "attn_fwd_kernel.h"

namespace qfa {

hipError_t launch_attn_d64_fp16(const AttnArgs& a, hipStream_t s) { return launch_d_vt<64, FP16>(a, s); }

}  // namespace qfa
