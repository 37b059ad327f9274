// Host launcher of the paged decode kernels for a token-granular cache (page
// size 1: K/V [num_slots, H_kv, D], addressed through kv_indptr and page
// indices); the kernels are in decode_kernels.h.
#include "decode_kernels.h"

namespace pa {

hipError_t launch_decode_tokens(const DecodeArgs &a) {
    return launch_detail::launch_decode_t<false, false, true>(a);
}

}  // namespace pa
