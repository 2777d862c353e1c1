// Instances of the attention kernel (attn_fwd_kernel.h) for head dimension
// 128 and bf16 V: one of four translation units compiled in parallel.
#include "attn_fwd_kernel.h"

namespace qfa {

hipError_t launch_attn_d128_bf16(const AttnArgs& a, hipStream_t s) { return launch_d_vt<128, BF16>(a, s); }
hipError_t launch_qk_dump_d128(const AttnArgs& a, hipStream_t s) { return launch_qk_dump_d<128>(a, s); }

}  // namespace qfa
