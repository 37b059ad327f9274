// Host launcher of the paged decode kernels for the BI-V100 page's cache
// layouts (x-packed K [num_blocks, H_kv, D/8, 16, 8], transposed V
// [num_blocks, H_kv, D, 16]); the kernels are in decode_kernels.h.
#include "decode_kernels.h"

namespace pa {

hipError_t launch_decode_xpacked(const DecodeArgs &a) { return launch_detail::launch_decode_t<false, true>(a); }

}  // namespace pa
