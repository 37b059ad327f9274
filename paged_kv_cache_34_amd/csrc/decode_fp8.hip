// Host launcher of the paged decode kernels for an FP8 (OCP E4M3) KV cache
// with per-position dequant scales (the kernels are in decode_kernels.h).
#include "decode_kernels.h"

namespace pa {

hipError_t launch_decode_fp8(const DecodeArgs &a) { return launch_detail::launch_decode_t<true, false>(a); }

}  // namespace pa
