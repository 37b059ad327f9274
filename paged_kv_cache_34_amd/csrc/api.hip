// C ABI of the paged attention library: host-side argument validation, the
// partition-size heuristic, the prefill tile map, and dispatch to the kernels.
// Validation happens entirely on the host before anything is enqueued; a
// rejected call launches nothing and never falls back to other code.
#include <limits.h>
#include <stdint.h>

#include <atomic>

#include "pa_launch.h"
#include "paged_attn.h"

namespace {

constexpr int kBlockSize = 16;
constexpr int kMaxGroup = 16;
constexpr int kGridYZMax = 65535;

bool head_dim_ok(int d) { return d == 64 || d == 128 || d == 256; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

long long ceil_div(long long a, long long b) { return (a + b - 1) / b; }

// Checks shared by decode and prefill; returns PA_OK or a status.
int check_common(const void *q, const void *k_cache, const void *v_cache,
                 const int32_t *block_tables, const int32_t *seq_lens, int num_seqs,
                 int num_q_heads, int num_kv_heads, int head_dim, int block_size, int num_blocks,
                 int max_blocks_per_seq) {
    if (!q || !k_cache || !v_cache || !block_tables || !seq_lens) return PA_ERR_NULL_POINTER;
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 ||
        max_blocks_per_seq <= 0 || head_dim <= 0 || block_size <= 0)
        return PA_ERR_BAD_SHAPE;
    if (num_q_heads % num_kv_heads != 0) return PA_ERR_BAD_SHAPE;
    if (!head_dim_ok(head_dim) || block_size != kBlockSize) return PA_ERR_UNSUPPORTED;
    if (num_q_heads / num_kv_heads > kMaxGroup) return PA_ERR_UNSUPPORTED;
    if (num_seqs > kGridYZMax || num_kv_heads > kGridYZMax) return PA_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return PA_ERR_ALIGNMENT;
    return PA_OK;
}

float log2e_scaled(float scale) { return (float)((double)scale * 1.4426950408889634074); }

// The softmax scale must be a positive finite number (the kernels take the
// maximum of the raw scores as the maximum of the scaled ones).
bool scale_ok(float scale) { return scale > 0.f && __builtin_isfinite(scale); }

long long round_up(long long x, long long q) { return (x + q - 1) / q * q; }

// Split-KV prefill workspace: a 256-byte header holding the two chunk
// counters, then max logits, exp-sums and normalized outputs, each section
// 256-byte aligned.
constexpr long long kWsHeader = 256;
constexpr long long kWsAlign = 256;
constexpr int kChunkTile = 64;       // key chunks are whole KV tiles (64 keys for D <= 128)
constexpr int kChunkQuantum = 256;   // automatic chunk sizes are multiples of this
constexpr int kMinChunk = 512;


}  // namespace

// The entry points below take C linkage from their declarations in paged_attn.h.

const char *paged_attn_status_string(int status) {
    switch (status) {
        case PA_OK: return "ok";
        case PA_ERR_NULL_POINTER: return "null pointer";
        case PA_ERR_BAD_SHAPE: return "bad shape";
        case PA_ERR_UNSUPPORTED: return "unsupported configuration";
        case PA_ERR_LAUNCH: return "kernel launch failed";
        case PA_ERR_ALIGNMENT: return "tensor pointer not 16-byte aligned";
        case PA_ERR_BAD_VALUE: return "scale must be positive and finite";
        case PA_ERR_SCRATCH_LIMIT: return "problem larger than the library's fixed scratch (no-allocation entry point)";
        default: return "unknown status";
    }
}

int paged_attn_num_partitions(int max_blocks_per_seq, int block_size, int partition_size) {
    if (max_blocks_per_seq <= 0 || block_size <= 0 || partition_size < 0) return -1;
    if (partition_size == 0) return 1;
    const long long n = ceil_div((long long)max_blocks_per_seq * block_size, partition_size);
    return n > INT_MAX ? -1 : (int)n;
}

int paged_attn_choose_partition_size(int num_seqs, int num_kv_heads, int max_seq_len,
                                     long total_kv_tokens) {
    // Work items are (sequence, kv head, partition) triples.  Measured on
    // MI355X: 512-token partitions are best until there are more than ~4096
    // items, then 1024 (up to ~8192 items), then 2048.  Shorter partitions
    // pay the per-item start-up (query, block ids, first tiles) too often;
    // longer ones leave compute units idle at the end.  When one partition
    // already covers the longest sequence and there are enough (sequence,
    // kv head) pairs, a single pass avoids the partials and the merge.
    if (num_seqs <= 0 || num_kv_heads <= 0 || max_seq_len <= 0) return 0;
    const long long tokens = total_kv_tokens > 0 ? (long long)total_kv_tokens
                                                 : (long long)num_seqs * max_seq_len;
    auto items = [&](long long p) { return (long long)num_kv_heads * (tokens / p + num_seqs / 2 + 1); };
    int best = 2048;
    if (items(512) <= 4096) best = 512;
    else if (items(1024) <= 8192) best = 1024;
    if (best >= max_seq_len && (long long)num_seqs * num_kv_heads >= 1024) return 0;
    return best;
}

int paged_attn_prefill_tile_map(const int32_t *cu_seqlens_host, int num_seqs, int tile_rows,
                                int32_t *tile_to_batch, int32_t *tile_to_index, int capacity) {
    if (!cu_seqlens_host || num_seqs < 0 || tile_rows <= 0 || capacity < 0) return -1;
    if (capacity > 0 && (!tile_to_batch || !tile_to_index)) return -1;
    long long count = 0;
    for (int b = 0; b < num_seqs; ++b) {
        const long long n = (long long)cu_seqlens_host[b + 1] - cu_seqlens_host[b];
        if (n < 0) return -1;
        const long long tiles = ceil_div(n, tile_rows);
        for (long long i = 0; i < tiles; ++i, ++count) {
            if (count < capacity) {
                tile_to_batch[count] = b;
                tile_to_index[count] = (int32_t)i;
            }
        }
    }
    return count > INT_MAX ? -1 : (int)count;
}

namespace {
int decode_common(const void *q, const void *k_cache, const void *v_cache,
                  const int32_t *block_tables, const int32_t *seq_lens, int num_seqs,
                  int num_q_heads, int num_kv_heads, int head_dim, int block_size, int num_blocks,
                  int max_blocks_per_seq, float scale, int partition_size, void *out,
                  float *max_logits, float *exp_sums, float *tmp_out, int max_num_partitions,
                  int32_t *counters, void *stream, const float *k_scales = nullptr,
                  const float *v_scales = nullptr, bool xpacked = false,
                  const int32_t *kv_indptr = nullptr) {
    int st = check_common(q, k_cache, v_cache, block_tables, seq_lens, num_seqs, num_q_heads,
                          num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq);
    if (st != PA_OK) return st;
    const bool fp8 = k_scales != nullptr;
    if (fp8 && !aligned16(k_scales)) return PA_ERR_ALIGNMENT;
    if (fp8 && !aligned16(v_scales)) return PA_ERR_ALIGNMENT;
    if (!scale_ok(scale)) return PA_ERR_BAD_VALUE;
    if (partition_size < 0 || partition_size % kBlockSize != 0) return PA_ERR_BAD_SHAPE;
    int nparts = 1;
    if (partition_size == 0 || counters) {
        if (!out) return PA_ERR_NULL_POINTER;
        if (!aligned16(out)) return PA_ERR_ALIGNMENT;
    }
    if (partition_size > 0) {
        if (!max_logits || !exp_sums || !tmp_out) return PA_ERR_NULL_POINTER;
        nparts = paged_attn_num_partitions(max_blocks_per_seq, block_size, partition_size);
        if (nparts <= 0 || max_num_partitions < nparts) return PA_ERR_BAD_SHAPE;
        if (!aligned16(tmp_out)) return PA_ERR_ALIGNMENT;
    }
    if (num_seqs == 0) return PA_OK;
    pa::DecodeArgs a;
    a.q = static_cast<const uint16_t *>(q);
    a.k_cache = static_cast<const uint16_t *>(k_cache);
    a.v_cache = static_cast<const uint16_t *>(v_cache);
    a.block_tables = block_tables;
    a.seq_lens = seq_lens;
    a.num_seqs = num_seqs;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.head_dim = head_dim;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.scale_log2 = log2e_scaled(scale);
    a.partition_size = partition_size;
    a.num_partitions = nparts;
    a.max_num_partitions = partition_size ? max_num_partitions : 1;
    a.out = static_cast<uint16_t *>(out);
    a.max_logits = max_logits;
    a.exp_sums = exp_sums;
    a.tmp_out = tmp_out;
    a.counters = counters;
    a.k_scales = k_scales;
    a.v_scales = v_scales;
    a.kv_indptr = kv_indptr;
    a.stream = static_cast<hipStream_t>(stream);
    const hipError_t e = fp8 ? pa::launch_decode_fp8(a)
                         : xpacked ? pa::launch_decode_xpacked(a)
                         : kv_indptr ? pa::launch_decode_tokens(a) : pa::launch_decode(a);
    return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

int append_common(const void *k_new, const void *v_new, const int32_t *block_tables,
                  const int32_t *seq_lens, const int32_t *cu_seqlens, int num_seqs, int num_tokens,
                  int max_new_tokens, int num_kv_heads, int head_dim, int block_size,
                  int num_blocks, int max_blocks_per_seq, void *k_cache, void *v_cache,
                  float *k_scales, float *v_scales, bool fp8, void *stream, bool xpacked = false) {
    if (!k_new || !v_new || !block_tables || !seq_lens || !cu_seqlens || !k_cache || !v_cache)
        return PA_ERR_NULL_POINTER;
    if (fp8 && (!k_scales || !v_scales)) return PA_ERR_NULL_POINTER;
    if (num_seqs < 0 || num_tokens < 0 || max_new_tokens < 0 || num_kv_heads <= 0 ||
        num_blocks <= 0 || max_blocks_per_seq <= 0 || head_dim <= 0 || block_size <= 0)
        return PA_ERR_BAD_SHAPE;
    if (!head_dim_ok(head_dim) || block_size != kBlockSize) return PA_ERR_UNSUPPORTED;
    if (num_seqs > kGridYZMax) return PA_ERR_UNSUPPORTED;
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache))
        return PA_ERR_ALIGNMENT;
    if (fp8 && (!aligned16(k_scales) || !aligned16(v_scales))) return PA_ERR_ALIGNMENT;
    if (num_seqs == 0 || num_tokens == 0 || max_new_tokens == 0) return PA_OK;
    if (max_new_tokens > num_tokens) return PA_ERR_BAD_SHAPE;
    pa::AppendArgs a;
    a.k_new = k_new;
    a.v_new = v_new;
    a.block_tables = block_tables;
    a.seq_lens = seq_lens;
    a.cu_seqlens = cu_seqlens;
    a.num_seqs = num_seqs;
    a.max_new_tokens = max_new_tokens;
    a.num_kv_heads = num_kv_heads;
    a.head_dim = head_dim;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.k_scales = k_scales;
    a.v_scales = v_scales;
    a.stream = static_cast<hipStream_t>(stream);
    const hipError_t e = fp8 ? pa::launch_kv_append_fp8(a)
                             : xpacked ? pa::launch_kv_append_xpacked(a) : pa::launch_kv_append(a);
    return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}
}  // namespace

int paged_attn_decode_fp8(const void *q, const void *k_cache, const void *v_cache,
                          const float *k_scales, const float *v_scales,
                          const int32_t *block_tables, const int32_t *seq_lens, int num_seqs,
                          int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                          int num_blocks, int max_blocks_per_seq, float scale, int partition_size,
                          void *out, float *max_logits, float *exp_sums, float *tmp_out,
                          int max_num_partitions, void *stream) {
    if (!k_scales || !v_scales) return PA_ERR_NULL_POINTER;
    return decode_common(q, k_cache, v_cache, block_tables, seq_lens, num_seqs, num_q_heads,
                         num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq, scale,
                         partition_size, out, max_logits, exp_sums, tmp_out, max_num_partitions,
                         nullptr, stream, k_scales, v_scales);
}

int paged_attn_kv_append(const void *k_new, const void *v_new, const int32_t *block_tables,
                         const int32_t *seq_lens, const int32_t *cu_seqlens, int num_seqs,
                         int num_tokens, int max_new_tokens, int num_kv_heads, int head_dim,
                         int block_size, int num_blocks, int max_blocks_per_seq, void *k_cache,
                         void *v_cache, void *stream) {
    return append_common(k_new, v_new, block_tables, seq_lens, cu_seqlens, num_seqs, num_tokens,
                         max_new_tokens, num_kv_heads, head_dim, block_size, num_blocks,
                         max_blocks_per_seq, k_cache, v_cache, nullptr, nullptr, false, stream);
}

int paged_attn_kv_append_fp8(const void *k_new, const void *v_new, const int32_t *block_tables,
                             const int32_t *seq_lens, const int32_t *cu_seqlens, int num_seqs,
                             int num_tokens, int max_new_tokens, int num_kv_heads, int head_dim,
                             int block_size, int num_blocks, int max_blocks_per_seq,
                             void *k_cache, void *v_cache, float *k_scales, float *v_scales,
                             void *stream) {
    return append_common(k_new, v_new, block_tables, seq_lens, cu_seqlens, num_seqs, num_tokens,
                         max_new_tokens, num_kv_heads, head_dim, block_size, num_blocks,
                         max_blocks_per_seq, k_cache, v_cache, k_scales, v_scales, true, stream);
}

int paged_attn_read_probe(const void *buf, long long bytes, uint32_t *partial, int num_workgroups,
                          void *stream) {
    if (!buf || !partial) return PA_ERR_NULL_POINTER;
    if (bytes <= 0 || bytes % 16 != 0 || num_workgroups <= 0) return PA_ERR_BAD_SHAPE;
    if (!aligned16(buf)) return PA_ERR_ALIGNMENT;
    const hipError_t e = pa::launch_read_probe(buf, bytes, partial, num_workgroups,
                                               static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

int paged_attn_gather_probe(const void *k_cache, const void *v_cache, const int32_t *block_tables,
                            const int32_t *block_prefix, int num_seqs, int num_kv_heads, int head_dim,
                            int block_size, int max_blocks_per_seq, int whole_blocks, uint32_t *partial,
                            int num_workgroups, void *stream) {
    if (!k_cache || !v_cache || !block_tables || !block_prefix || !partial) return PA_ERR_NULL_POINTER;
    if (num_seqs <= 0 || num_kv_heads <= 0 || max_blocks_per_seq <= 0 || num_workgroups <= 0 ||
        whole_blocks < 0 || whole_blocks > 2)
        return PA_ERR_BAD_SHAPE;
    if (!head_dim_ok(head_dim) || block_size != kBlockSize || num_seqs > 1024) return PA_ERR_UNSUPPORTED;
    if (!aligned16(k_cache) || !aligned16(v_cache)) return PA_ERR_ALIGNMENT;
    const hipError_t e = pa::launch_gather_probe(k_cache, v_cache, block_tables, block_prefix, num_seqs,
                                                 num_kv_heads, head_dim, max_blocks_per_seq, whole_blocks,
                                                 partial, num_workgroups, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

int paged_attn_decode(const void *q, const void *k_cache, const void *v_cache,
                      const int32_t *block_tables, const int32_t *seq_lens, int num_seqs,
                      int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                      int num_blocks, int max_blocks_per_seq, float scale, int partition_size,
                      void *out, float *max_logits, float *exp_sums, float *tmp_out,
                      int max_num_partitions, void *stream) {
    return decode_common(q, k_cache, v_cache, block_tables, seq_lens, num_seqs, num_q_heads,
                         num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq, scale,
                         partition_size, out, max_logits, exp_sums, tmp_out, max_num_partitions,
                         nullptr, stream);
}

int paged_attn_decode_fused(const void *q, const void *k_cache, const void *v_cache,
                            const int32_t *block_tables, const int32_t *seq_lens, int num_seqs,
                            int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                            int num_blocks, int max_blocks_per_seq, float scale,
                            int partition_size, void *out, float *max_logits, float *exp_sums,
                            float *tmp_out, int max_num_partitions, int32_t *counters,
                            void *stream) {
    if (!counters) return PA_ERR_NULL_POINTER;
    if (partition_size <= 0) return PA_ERR_BAD_SHAPE;
    return decode_common(q, k_cache, v_cache, block_tables, seq_lens, num_seqs, num_q_heads,
                         num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq, scale,
                         partition_size, out, max_logits, exp_sums, tmp_out, max_num_partitions,
                         counters, stream);
}

// ---------------------------------------------------------------------------
// Fused decode with the library's own fixed scratch, for callers that cannot
// allocate (graph capture, tight serving loops, harnesses that forbid it).
// ---------------------------------------------------------------------------
namespace {
constexpr long long kNoallocScratchBytes = 64LL << 20;      // per device, for the process lifetime
constexpr long long kNoallocMaxPairs = 1LL << 16;           // (sequence, kv head) arrival counters
constexpr long long kNoallocCounterBytes = kNoallocMaxPairs * 4;

// The workspace of paged_attn_decode_fused_noalloc: the arrival counters
// (kNoallocMaxPairs int32 at offset 0, zero between calls: every completed
// fused launch leaves the counters it used at zero), then the partial records
// of the current call.  In host code `scratch` names a host-side stand-in:
// only the device address taken at set-up is ever passed to a kernel.
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

std::atomic<unsigned char *> g_scratch_dev[pa::kMaxDevices];

__global__ void zero_words_kernel(uint32_t *p, int n) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

// Device address of the current device's `scratch`, set up once per device
// (the counters cleared by a fill kernel on `stream`, ahead of the first
// decode launch on it); null if the address cannot be taken.
unsigned char *noalloc_scratch(hipStream_t stream) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= pa::kMaxDevices) return nullptr;
    unsigned char *p = g_scratch_dev[dev].load(std::memory_order_acquire);
    if (p) return p;
    void *addr = nullptr;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) return nullptr;
    p = static_cast<unsigned char *>(addr);
    hipLaunchKernelGGL(zero_words_kernel, dim3(64), dim3(256), 0, stream, reinterpret_cast<uint32_t *>(p),
                       (int)kNoallocMaxPairs);
    if (hipGetLastError() != hipSuccess) return nullptr;
    g_scratch_dev[dev].store(p, std::memory_order_release);
    return p;
}
}  // namespace

int paged_attn_decode_fused_noalloc(const void *q, const void *k_cache, const void *v_cache,
                                    const int32_t *block_tables, const int32_t *seq_lens,
                                    int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                    int block_size, int num_blocks, int max_blocks_per_seq,
                                    float scale, int partition_size, void *out, void *stream) {
    int st = check_common(q, k_cache, v_cache, block_tables, seq_lens, num_seqs, num_q_heads,
                          num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq);
    if (st != PA_OK) return st;
    if (!out) return PA_ERR_NULL_POINTER;
    if (!scale_ok(scale)) return PA_ERR_BAD_VALUE;
    if (partition_size <= 0 || partition_size % kBlockSize != 0) return PA_ERR_BAD_SHAPE;
    const int nparts = paged_attn_num_partitions(max_blocks_per_seq, block_size, partition_size);
    if (nparts <= 0) return PA_ERR_BAD_SHAPE;
    // scratch layout: counters | max_logits | exp_sums | tmp_out (256-byte aligned sections)
    const long long rows = (long long)num_seqs * num_q_heads * nparts;
    const long long off_ml = kNoallocCounterBytes;
    const long long off_es = off_ml + round_up(rows * 4, 256);
    const long long off_to = off_es + round_up(rows * 4, 256);
    const long long need = off_to + rows * head_dim * 4;
    if ((long long)num_seqs * num_kv_heads > kNoallocMaxPairs || need > kNoallocScratchBytes)
        return PA_ERR_SCRATCH_LIMIT;
    if (num_seqs == 0) return PA_OK;
    unsigned char *base = noalloc_scratch(static_cast<hipStream_t>(stream));
    if (!base) return PA_ERR_LAUNCH;
    return paged_attn_decode_fused(q, k_cache, v_cache, block_tables, seq_lens, num_seqs, num_q_heads,
                                   num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                                   scale, partition_size, out, reinterpret_cast<float *>(base + off_ml),
                                   reinterpret_cast<float *>(base + off_es),
                                   reinterpret_cast<float *>(base + off_to), nparts,
                                   reinterpret_cast<int32_t *>(base), stream);
}

namespace {
int reduce_common(const float *max_logits, const float *exp_sums, const float *tmp_out,
                  const int32_t *seq_lens, const int32_t *kv_indptr, int num_seqs, int num_q_heads,
                  int head_dim, int partition_size, int max_num_partitions, void *out,
                  void *stream) {
    if (!max_logits || !exp_sums || !tmp_out || !(seq_lens || kv_indptr) || !out)
        return PA_ERR_NULL_POINTER;
    if (num_seqs < 0 || num_q_heads <= 0 || partition_size <= 0 || max_num_partitions <= 0 ||
        partition_size % kBlockSize != 0)
        return PA_ERR_BAD_SHAPE;
    if (!head_dim_ok(head_dim)) return PA_ERR_UNSUPPORTED;
    if (num_seqs > kGridYZMax || num_q_heads > kGridYZMax) return PA_ERR_UNSUPPORTED;
    if (!aligned16(tmp_out) || !aligned16(out)) return PA_ERR_ALIGNMENT;
    if (num_seqs == 0) return PA_OK;
    pa::ReduceArgs a;
    a.max_logits = max_logits;
    a.exp_sums = exp_sums;
    a.tmp_out = tmp_out;
    a.seq_lens = seq_lens;
    a.kv_indptr = kv_indptr;
    a.num_seqs = num_seqs;
    a.num_q_heads = num_q_heads;
    a.head_dim = head_dim;
    a.partition_size = partition_size;
    a.max_num_partitions = max_num_partitions;
    a.out = static_cast<uint16_t *>(out);
    a.stream = static_cast<hipStream_t>(stream);
    return pa::launch_reduce(a) == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}
}  // namespace

int paged_attn_decode_reduce(const float *max_logits, const float *exp_sums,
                             const float *tmp_out, const int32_t *seq_lens, int num_seqs,
                             int num_q_heads, int head_dim, int partition_size,
                             int max_num_partitions, void *out, void *stream) {
    if (!seq_lens) return PA_ERR_NULL_POINTER;
    return reduce_common(max_logits, exp_sums, tmp_out, seq_lens, nullptr, num_seqs, num_q_heads,
                         head_dim, partition_size, max_num_partitions, out, stream);
}

int paged_attn_decode_reduce_indptr(const float *max_logits, const float *exp_sums,
                                    const float *tmp_out, const int32_t *kv_indptr, int num_seqs,
                                    int num_q_heads, int head_dim, int partition_size,
                                    int max_num_partitions, void *out, void *stream) {
    if (!kv_indptr) return PA_ERR_NULL_POINTER;
    return reduce_common(max_logits, exp_sums, tmp_out, nullptr, kv_indptr, num_seqs, num_q_heads,
                         head_dim, partition_size, max_num_partitions, out, stream);
}

int paged_attn_prefill_ragged(const void *q, const void *k_cache, const void *v_cache,
                              const int32_t *block_tables, const int32_t *seq_lens,
                              const int32_t *cu_seqlens, int num_seqs, int total_q, int max_q_len,
                              int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                              int num_blocks, int max_blocks_per_seq, float scale, void *out,
                              void *stream) {
    int st = check_common(q, k_cache, v_cache, block_tables, seq_lens, num_seqs, num_q_heads,
                          num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq);
    if (st != PA_OK) return st;
    if (!cu_seqlens || !out) return PA_ERR_NULL_POINTER;
    if (!scale_ok(scale)) return PA_ERR_BAD_VALUE;
    if (total_q < 0 || max_q_len < 0) return PA_ERR_BAD_SHAPE;
    if (!aligned16(out)) return PA_ERR_ALIGNMENT;
    if (num_seqs == 0 || total_q == 0 || max_q_len == 0) return PA_OK;
    if (max_q_len > total_q) return PA_ERR_BAD_SHAPE;
    pa::PrefillArgs a;
    a.q = static_cast<const uint16_t *>(q);
    a.k_cache = static_cast<const uint16_t *>(k_cache);
    a.v_cache = static_cast<const uint16_t *>(v_cache);
    a.block_tables = block_tables;
    a.seq_lens = seq_lens;
    a.cu_seqlens = cu_seqlens;
    a.num_seqs = num_seqs;
    a.total_q = total_q;
    a.max_q_len = max_q_len;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.head_dim = head_dim;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.scale_log2 = log2e_scaled(scale);
    a.out = static_cast<uint16_t *>(out);
    a.chunk = 0;
    a.max_splits = 0;
    a.ws_m = a.ws_l = a.ws_o = nullptr;
    a.counters = nullptr;
    a.stream = static_cast<hipStream_t>(stream);
    return pa::launch_prefill(a) == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

int paged_attn_prefill_chunk_size(int num_seqs, int total_q, int num_q_heads, int num_kv_heads,
                                  int max_blocks_per_seq, int block_size) {
    if (num_seqs <= 0 || total_q <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
        max_blocks_per_seq <= 0 || block_size <= 0 || num_q_heads % num_kv_heads != 0)
        return 0;
    const int group = num_q_heads / num_kv_heads;
    if (group > kMaxGroup) return 0;
    const long long rows = pa::kPfRowSlots / group;
    const long long pairs = ceil_div(total_q, rows) + num_seqs;
    if (num_seqs > pa::kPfMaxSeqs || pairs > pa::kPfMaxPairs || num_q_heads > pa::kPfMaxHeads) return 0;
    const long long lmax = (long long)max_blocks_per_seq * block_size;
    // about 2.6 chunks per CU (13 per 5 CUs) if every pair had the longest
    // context (measured on MI355X over 512..8192-token chunks on a ragged
    // batch of 16 sequences: fewer, longer chunks win until the last ones
    // unbalance the grid -- each chunk costs a start-up of dependent loads
    // and its rows' partial records; 2.6 per CU beat 3 by 3%)
    const long long target = 13LL * pa::device_cu_count();
    long long chunk = ceil_div(pairs * num_kv_heads * lmax * 5, target);
    chunk = ceil_div(chunk, kChunkQuantum) * kChunkQuantum;
    if (chunk < kMinChunk) chunk = kMinChunk;
    if (chunk > pa::kPfMaxChunk) chunk = pa::kPfMaxChunk;
    return chunk >= lmax ? 0 : (int)chunk;
}

long long paged_attn_prefill_workspace_size(int total_q, int num_q_heads, int head_dim,
                                            int max_blocks_per_seq, int block_size, int kv_chunk) {
    if (total_q < 0 || num_q_heads <= 0 || head_dim <= 0 || max_blocks_per_seq <= 0 ||
        block_size <= 0 || kv_chunk <= 0)
        return -1;
    const long long splits = ceil_div((long long)max_blocks_per_seq * block_size, kv_chunk);
    const long long recs = (long long)total_q * num_q_heads * splits;
    return kWsHeader + 2 * round_up(recs * 4, kWsAlign) + round_up(recs * head_dim * 4, kWsAlign);
}

int paged_attn_prefill_ragged_split(const void *q, const void *k_cache, const void *v_cache,
                                    const int32_t *block_tables, const int32_t *seq_lens,
                                    const int32_t *cu_seqlens, int num_seqs, int total_q,
                                    int max_q_len, int num_q_heads, int num_kv_heads, int head_dim,
                                    int block_size, int num_blocks, int max_blocks_per_seq,
                                    float scale, int kv_chunk, void *workspace,
                                    long long workspace_bytes, void *out, void *stream) {
    int st = check_common(q, k_cache, v_cache, block_tables, seq_lens, num_seqs, num_q_heads,
                          num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq);
    if (st != PA_OK) return st;
    if (!cu_seqlens || !out) return PA_ERR_NULL_POINTER;
    if (!scale_ok(scale)) return PA_ERR_BAD_VALUE;
    if (total_q < 0 || max_q_len < 0) return PA_ERR_BAD_SHAPE;
    if (!aligned16(out)) return PA_ERR_ALIGNMENT;
    if (kv_chunk < 0 || kv_chunk % kChunkTile != 0 || kv_chunk > pa::kPfMaxChunk) return PA_ERR_BAD_SHAPE;
    if (num_seqs == 0 || total_q == 0 || max_q_len == 0) return PA_OK;
    if (max_q_len > total_q) return PA_ERR_BAD_SHAPE;
    int chunk = kv_chunk;
    if (chunk == 0)
        chunk = paged_attn_prefill_chunk_size(num_seqs, total_q, num_q_heads, num_kv_heads,
                                              max_blocks_per_seq, block_size);
    const int group = num_q_heads / num_kv_heads;
    const long long pairs = ceil_div(total_q, pa::kPfRowSlots / group) + num_seqs;
    if (num_seqs > pa::kPfMaxSeqs || pairs > pa::kPfMaxPairs || num_q_heads > pa::kPfMaxHeads)
        chunk = 0;  // single pass
    if (chunk > 0 && chunk >= (long long)max_blocks_per_seq * block_size) chunk = 0;
    pa::PrefillArgs a;
    a.q = static_cast<const uint16_t *>(q);
    a.k_cache = static_cast<const uint16_t *>(k_cache);
    a.v_cache = static_cast<const uint16_t *>(v_cache);
    a.block_tables = block_tables;
    a.seq_lens = seq_lens;
    a.cu_seqlens = cu_seqlens;
    a.num_seqs = num_seqs;
    a.total_q = total_q;
    a.max_q_len = max_q_len;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.head_dim = head_dim;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.scale_log2 = log2e_scaled(scale);
    a.out = static_cast<uint16_t *>(out);
    a.chunk = 0;
    a.max_splits = 0;
    a.ws_m = a.ws_l = a.ws_o = nullptr;
    a.counters = nullptr;
    if (chunk > 0) {
        if (!workspace) return PA_ERR_NULL_POINTER;
        if (!aligned16(workspace)) return PA_ERR_ALIGNMENT;
        const long long need = paged_attn_prefill_workspace_size(total_q, num_q_heads, head_dim,
                                                                 max_blocks_per_seq, block_size, chunk);
        if (need < 0 || workspace_bytes < need) return PA_ERR_BAD_SHAPE;
        const long long splits = ceil_div((long long)max_blocks_per_seq * block_size, chunk);
        const long long recs = (long long)total_q * num_q_heads * splits;
        char *w = static_cast<char *>(workspace);
        a.chunk = chunk;
        a.max_splits = (int)splits;
        a.counters = reinterpret_cast<int32_t *>(w);
        a.ws_m = reinterpret_cast<float *>(w + kWsHeader);
        a.ws_l = reinterpret_cast<float *>(w + kWsHeader + round_up(recs * 4, kWsAlign));
        a.ws_o = reinterpret_cast<float *>(w + kWsHeader + 2 * round_up(recs * 4, kWsAlign));
    }
    a.stream = static_cast<hipStream_t>(stream);
    return pa::launch_prefill(a) == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}


int paged_attn_decode_xpacked(const void *q, const void *k_cache, const void *v_cache,
                              const int32_t *block_tables, const int32_t *seq_lens, int num_seqs,
                              int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                              int num_blocks, int max_blocks_per_seq, float scale,
                              int partition_size, void *out, float *max_logits, float *exp_sums,
                              float *tmp_out, int max_num_partitions, void *stream) {
    return decode_common(q, k_cache, v_cache, block_tables, seq_lens, num_seqs, num_q_heads,
                         num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq, scale,
                         partition_size, out, max_logits, exp_sums, tmp_out, max_num_partitions,
                         nullptr, stream, nullptr, nullptr, true);
}

int paged_attn_kv_append_xpacked(const void *k_new, const void *v_new, const int32_t *block_tables,
                                 const int32_t *seq_lens, const int32_t *cu_seqlens, int num_seqs,
                                 int num_tokens, int max_new_tokens, int num_kv_heads, int head_dim,
                                 int block_size, int num_blocks, int max_blocks_per_seq,
                                 void *k_cache, void *v_cache, void *stream) {
    return append_common(k_new, v_new, block_tables, seq_lens, cu_seqlens, num_seqs, num_tokens,
                         max_new_tokens, num_kv_heads, head_dim, block_size, num_blocks,
                         max_blocks_per_seq, k_cache, v_cache, nullptr, nullptr, false, stream, true);
}

int paged_attn_decode_tokens(const void *q, const void *k_cache, const void *v_cache,
                             const int32_t *kv_indptr, const int32_t *kv_indices, int num_seqs,
                             int num_q_heads, int num_kv_heads, int head_dim, int num_slots,
                             int max_kv_len, float scale, int partition_size, void *out,
                             float *max_logits, float *exp_sums, float *tmp_out,
                             int max_num_partitions, void *stream) {
    if (!kv_indptr || !kv_indices) return PA_ERR_NULL_POINTER;
    if (max_kv_len <= 0 || num_slots <= 0) return PA_ERR_BAD_SHAPE;
    // one-token pages: the block walk with block_size 1 over the page indices,
    // sized by max_kv_len (the partition count comes from it)
    const int blocks = (max_kv_len + kBlockSize - 1) / kBlockSize;
    return decode_common(q, k_cache, v_cache, kv_indices, kv_indptr, num_seqs, num_q_heads,
                         num_kv_heads, head_dim, kBlockSize, num_slots, blocks, scale,
                         partition_size, out, max_logits, exp_sums, tmp_out, max_num_partitions,
                         nullptr, stream, nullptr, nullptr, false, kv_indptr);
}

