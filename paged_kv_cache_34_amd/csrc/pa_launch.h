// Host-side launch descriptors shared by the C ABI (api.hip) and the kernel
// translation units.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace pa {

// Per-device caches of launch facts (devices beyond kMaxDevices are queried
// on every call).
constexpr int kMaxDevices = 64;

// Compute units of the current device (256 if the query fails).
inline int device_cu_count() {
    static std::atomic<int> cached[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    const bool slot = dev >= 0 && dev < kMaxDevices;
    if (slot) {
        const int c = cached[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    if (slot) cached[dev].store(n, std::memory_order_relaxed);
    return n;
}

// Workgroups of KERN (at `threads` threads each, no dynamic LDS) resident per
// compute unit of the current device, at least 1; cached per kernel and device.
template <auto KERN>
inline int resident_per_cu(int threads) {
    static std::atomic<int> cached[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = -1;
    const bool slot = dev >= 0 && dev < kMaxDevices;
    if (slot) {
        const int c = cached[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, KERN, threads, 0) != hipSuccess || n <= 0) n = 1;
    if (slot) cached[dev].store(n, std::memory_order_relaxed);
    return n;
}

struct DecodeArgs {
    const uint16_t *q;
    const uint16_t *k_cache;
    const uint16_t *v_cache;
    const int32_t *block_tables;
    const int32_t *seq_lens;
    int num_seqs, num_q_heads, num_kv_heads, head_dim;
    int max_blocks_per_seq;
    float scale_log2;          // scale * log2(e)
    int partition_size;        // 0 = single pass
    int num_partitions;        // grid.x
    int max_num_partitions;    // row stride of the partial buffers
    uint16_t *out;
    float *max_logits, *exp_sums, *tmp_out;
    int32_t *counters;         // fused merge counters, or null
    // FP8 cache: k_cache / v_cache hold E4M3 codes and these the per-position
    // dequant scales [num_blocks, H_kv, block_size]; null for a bf16 cache
    const float *k_scales = nullptr, *v_scales = nullptr;
    // token-granular cache: block_tables holds the page indices, kv_indptr
    // [num_seqs + 1] the per-sequence offsets into them; null otherwise
    const int32_t *kv_indptr = nullptr;
    hipStream_t stream;
};

struct ReduceArgs {
    const float *max_logits, *exp_sums, *tmp_out;
    const int32_t *seq_lens;
    const int32_t *kv_indptr = nullptr;  // lengths from adjacent entries instead of seq_lens
    int num_seqs, num_q_heads, head_dim, partition_size, max_num_partitions;
    uint16_t *out;
    hipStream_t stream;
};

// Split-KV prefill limits: the chunk list is built in LDS.
constexpr int kPfMaxSeqs = 1024;    // sequences
constexpr int kPfMaxPairs = 1024;   // (sequence, query tile) pairs
constexpr int kPfMaxChunk = 8192;   // key chunk, tokens
constexpr int kPfRowSlots = 256;    // (row, head) query slots of a prefill workgroup
constexpr int kPfMaxHeads = 128;    // query heads (the merge keeps a row's chunk weights in LDS)

struct PrefillArgs {
    const uint16_t *q;
    const uint16_t *k_cache;
    const uint16_t *v_cache;
    const int32_t *block_tables;
    const int32_t *seq_lens;
    const int32_t *cu_seqlens;
    int num_seqs, total_q, max_q_len, num_q_heads, num_kv_heads, head_dim;
    int max_blocks_per_seq;
    float scale_log2;
    uint16_t *out;
    // split-KV (chunk > 0): partial records [total_q, H_q, max_splits] (+ D for
    // the outputs) and two int counters, zero on entry and left zero
    int chunk, max_splits;
    float *ws_m, *ws_l, *ws_o;
    int32_t *counters;
    hipStream_t stream;
};

// KV append (bf16 copy or FP8 quantization) of new rows into their cache slots.
struct AppendArgs {
    const void *k_new, *v_new;          // bf16 [num_tokens, H_kv, D]
    const int32_t *block_tables, *seq_lens, *cu_seqlens;
    int num_seqs, max_new_tokens, num_kv_heads, head_dim, max_blocks_per_seq;
    void *k_cache, *v_cache;            // bf16 values or E4M3 codes [num_blocks, H_kv, 16, D]
    float *k_scales, *v_scales;         // FP8: dequant scales [num_blocks, H_kv, 16]
    hipStream_t stream;
};

hipError_t launch_decode(const DecodeArgs &a);
hipError_t launch_decode_fp8(const DecodeArgs &a);
hipError_t launch_decode_xpacked(const DecodeArgs &a);
hipError_t launch_decode_tokens(const DecodeArgs &a);
hipError_t launch_reduce(const ReduceArgs &a);
hipError_t launch_prefill(const PrefillArgs &a);
hipError_t launch_kv_append(const AppendArgs &a);
hipError_t launch_kv_append_fp8(const AppendArgs &a);
hipError_t launch_kv_append_xpacked(const AppendArgs &a);
hipError_t launch_gather_probe(const void *k_cache, const void *v_cache, const int32_t *block_tables,
                               const int32_t *block_prefix, int num_seqs, int num_kv_heads, int head_dim,
                               int max_blocks_per_seq, int whole_blocks, uint32_t *partial, int num_workgroups,
                               hipStream_t stream);
hipError_t launch_read_probe(const void *buf, long long bytes, uint32_t *partial, int num_workgroups,
                             hipStream_t stream);

}  // namespace pa
