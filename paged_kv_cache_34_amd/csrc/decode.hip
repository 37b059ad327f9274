// Host launchers of the bf16 paged decode kernels and of the cross-partition
// merge kernels (the kernels themselves are in decode_kernels.h).
#include "decode_kernels.h"

namespace pa {

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
namespace {
constexpr int kReduceWaves = 4;
}  // namespace

hipError_t launch_decode(const DecodeArgs &a) { return launch_detail::launch_decode_t<false, false>(a); }

hipError_t launch_reduce(const ReduceArgs &a) {
    const int rows = 256 / a.head_dim;  // rows of the one-wave merge
    if (a.max_num_partitions <= rows * kWaveReduceUnroll * kWaveReduceMaxRounds) {
        const long pairs = (long)a.num_seqs * a.num_q_heads;
        dim3 grid((unsigned)((pairs + 3) / 4));
        auto kern = a.head_dim == 64 ? paged_reduce_wave_kernel<64>
                  : a.head_dim == 128 ? paged_reduce_wave_kernel<128> : paged_reduce_wave_kernel<256>;
        hipLaunchKernelGGL(kern, grid, dim3(256), 0, a.stream, a.max_logits, a.exp_sums, a.tmp_out,
                           a.seq_lens, a.kv_indptr, a.num_seqs, a.num_q_heads, a.partition_size,
                           a.max_num_partitions, a.out);
        return hipGetLastError();
    }
    dim3 grid(a.head_dim / kReduceChunk, a.num_q_heads, a.num_seqs);
    dim3 block(kReduceWaves * 64);
    hipLaunchKernelGGL((paged_reduce_kernel<kReduceWaves>), grid, block, 0, a.stream, a.max_logits,
                       a.exp_sums, a.tmp_out, a.seq_lens, a.kv_indptr, a.num_q_heads, a.head_dim,
                       a.partition_size, a.max_num_partitions, a.out);
    return hipGetLastError();
}

}  // namespace pa
