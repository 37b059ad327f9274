// HBM read-stream probe: the measured read ceiling that the decode's achieved
// bandwidth is set against (the AstrAI "CUDA Kernels" page, section "Known
// Optimization Targets", judges its decode by achieved against theoretical
// bandwidth; this kernel supplies the achievable figure on the machine at
// hand).  Not part of the attention path.
//
// Every 16-byte word of the buffer is read exactly once: lane i of the grid
// reads words i, i + stride, ... (stride = all lanes of the grid), kUnroll
// nontemporal loads in flight per lane.  The words are XOR-folded so the loads
// cannot be dropped, and workgroup w writes the XOR of everything it read to
// partial[w]; the XOR of all partial words is the XOR of the buffer's 32-bit
// words, which makes the probe checkable bit for bit.
#include "pa_common.h"
#include "pa_launch.h"

namespace pa {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;
constexpr int kBlock16 = 16;                     // tokens per physical KV block
constexpr int kProbeBufferFlags = 0x00020000;    // raw buffer descriptor word 3 (32-bit data)

__global__ __launch_bounds__(kProbeThreads) void hbm_read_probe_kernel(const u32x4 *__restrict__ p,
                                                                       long long n16,
                                                                       uint32_t *__restrict__ partial) {
    const long long stride = (long long)gridDim.x * kProbeThreads;
    long long i = (long long)blockIdx.x * kProbeThreads + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
        u32x4 v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) acc ^= (v[u][0] ^ v[u][1]) ^ (v[u][2] ^ v[u][3]);
    }
    for (; i < n16; i += stride) {
        const u32x4 v = __builtin_nontemporal_load(p + i);
        acc ^= (v[0] ^ v[1]) ^ (v[2] ^ v[3]);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o);
    __shared__ uint32_t wave_acc[kProbeThreads / 64];
    if ((threadIdx.x & 63) == 0) wave_acc[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t x = 0;
#pragma unroll
        for (int w = 0; w < kProbeThreads / 64; ++w) x ^= wave_acc[w];
        partial[blockIdx.x] = x;
    }
}

// ---------------------------------------------------------------------------
// Paged-gather read probe: the K/V bytes one decode of a batch reads (every
// tile of every kv head of every used block, tail slots included), found
// through the block table and read with the decode's 16-byte nontemporal
// loads, XOR-folded, and nothing else -- the gather ceiling the decode's
// achieved bandwidth is set against (the BI-V100 page, section 3 "Paged K/V
// Gather", counts the gather's memory accesses; this measures what they cost).
// A piece is two 16 * D * 2-byte tiles, read by one wave with a ring of two
// pieces in flight (each lane 2 * D / 32 loads per piece):
//   whole_blocks = 0: the K tile and the V tile of one (sequence, kv head,
//                     logical block), pieces ordered (sequence, kv head,
//                     block), the decode's own walk: the GPU reads scattered
//                     (block, kv head) tiles;
//   whole_blocks = 1: tiles 2i, 2i + 1 of [K block | V block] of one
//                     (sequence, logical block), pieces ordered (sequence,
//                     block, i): consecutive waves read each block's
//                     contiguous H_kv * 16 * D K and V rows.
//   whole_blocks = 2: the pieces of mode 0, read with load-to-LDS
//                     instructions (`buffer_load_dwordx4 ... lds`) into a
//                     per-wave ring of two pieces in LDS, each waited for
//                     with a counted vmcnt and then folded from LDS: the
//                     gather a direct-to-LDS tile ring would see.
// All modes read the same bytes.  Wave v of the grid takes pieces
// [v * n, (v + 1) * n), n = ceil(pieces / waves); absent pieces have empty
// buffer descriptors, whose loads return zeros without touching memory.
constexpr int kGatherMaxSeqs = 1024;

// The LDS destination of a load-to-LDS instruction, as a wave-uniform
// address.  The probe orders these writes itself (a counted vmcnt wait before
// a stage is read, the wave's own loads only), so the compiler is not left to
// pair them with the reads of the other stage.
__device__ __forceinline__ __attribute__((address_space(3))) void *lds_dest(u32x4 *p) {
    const uint32_t a = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) u32x4 *)p;
    return (__attribute__((address_space(3))) void *)(uintptr_t)__builtin_amdgcn_readfirstlane((int)a);
}

template <int D, bool TO_LDS>
__global__ __launch_bounds__(kProbeThreads) void paged_gather_probe_kernel(
    const char *__restrict__ k_cache, const char *__restrict__ v_cache, const int32_t *__restrict__ block_tables,
    const int32_t *__restrict__ block_prefix, int num_seqs, int num_kv_heads, int max_blocks_per_seq,
    int whole_blocks, uint32_t *__restrict__ partial) {
    constexpr int TILE = kBlock16 * D * 2;   // bytes of one (block, kv head) tile
    constexpr int W = TILE / (64 * 16);      // 16-byte loads per lane per tile
    __shared__ int pref[kGatherMaxSeqs + 1];
    __shared__ uint32_t wave_acc[kProbeThreads / 64];
    __shared__ __attribute__((aligned(16))) u32x4 lring[TO_LDS ? (kProbeThreads / 64) * 2 * 2 * W * 64 : 1];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    for (int i = tid; i <= num_seqs; i += kProbeThreads) pref[i] = block_prefix[i];
    __syncthreads();
    const int hkv = num_kv_heads;
    const long long total = (long long)__builtin_amdgcn_readfirstlane(pref[num_seqs]) * hkv;
    const long long waves = (long long)gridDim.x * (kProbeThreads / 64);
    const long long per = (total + waves - 1) / waves;
    const long long first = ((long long)blockIdx.x * (kProbeThreads / 64) + wave) * per;
    const long long last = first + per < total ? first + per : total;
    const long long blk_stride = (long long)hkv * TILE;
    auto search = [&](long long x) {  // the sequence whose blocks hold global block x
        int lo = 0, hi = num_seqs;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (pref[mid] <= x) lo = mid; else hi = mid;
        }
        return lo;
    };
    uint32_t acc = 0;
    for (long long p0 = first; p0 < last; p0 += 64) {
        const int n = (int)(last - p0 < 64 ? last - p0 : 64);
        // lane i resolves piece p0 + i into two tile addresses
        const char *a0 = k_cache, *a1 = k_cache;
        if (lane < n) {
            const long long p = p0 + lane;
            if (!whole_blocks) {
                const int s = search(p / hkv);
                const int nb = pref[s + 1] - pref[s];
                const long long r = p - (long long)pref[s] * hkv;
                const int kvh = (int)(r / nb), blk = (int)(r % nb);
                const long long phys = block_tables[(long long)s * max_blocks_per_seq + blk];
                a0 = k_cache + phys * blk_stride + (long long)kvh * TILE;
                a1 = v_cache + phys * blk_stride + (long long)kvh * TILE;
            } else {
                const long long b = p / hkv;
                const int part = (int)(p % hkv);
                const int s = search(b);
                const long long phys = block_tables[(long long)s * max_blocks_per_seq + (b - pref[s])];
                const int t0 = 2 * part, t1 = 2 * part + 1;
                a0 = (t0 < hkv ? k_cache + phys * blk_stride + (long long)t0 * TILE
                               : v_cache + phys * blk_stride + (long long)(t0 - hkv) * TILE);
                a1 = (t1 < hkv ? k_cache + phys * blk_stride + (long long)t1 * TILE
                               : v_cache + phys * blk_stride + (long long)(t1 - hkv) * TILE);
            }
        }
        const uint64_t u0 = reinterpret_cast<uint64_t>(a0), u1 = reinterpret_cast<uint64_t>(a1);
        if constexpr (TO_LDS) {
            // two stages of one piece (K tile then V tile, 64 lanes x 16
            // bytes per load) in this wave's LDS region
            auto stage = [&](int st) { return &lring[((wave * 2 + st) * 2 * W) * 64]; };
            auto issue_lds = [&](int i, int st) {
                const int j = i < n ? i : 0;
                const int bytes = i < n ? TILE : 0;
                const uint64_t b0 = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(u0 >> 32), j) << 32) |
                                    (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u0, j);
                const uint64_t b1 = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(u1 >> 32), j) << 32) |
                                    (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u1, j);
                const auto r0 = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(b0), 0, bytes, kProbeBufferFlags);
                const auto r1 = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(b1), 0, bytes, kProbeBufferFlags);
                u32x4 *dst = stage(st);
#pragma unroll
                for (int w = 0; w < W; ++w) {
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(r0, lds_dest(dst + w * 64), 16, 16 * lane + 1024 * w, 0, 0, 2);
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(r1, lds_dest(dst + (W + w) * 64), 16, 16 * lane + 1024 * w, 0,
                                                             0, 2);
                }
            };
            // (vmcnt in the s_waitcnt encoding: low 4 bits, high 2 bits at
            // 14..15; expcnt 7 and lgkmcnt 15 mean no wait on those counters)
            constexpr int NL = 2 * W;  // load instructions of one piece
            auto fold_lds = [&](int st) {
                __builtin_amdgcn_s_waitcnt((NL & 15) | ((NL >> 4) << 14) | (7 << 4) | (15 << 8));
                const u32x4 *src = stage(st);
#pragma unroll
                for (int w = 0; w < 2 * W; ++w) {
                    const u32x4 r = src[w * 64 + lane];
                    acc ^= (r[0] ^ r[1]) ^ (r[2] ^ r[3]);
                }
                // the stage's reads complete before the next loads into it are issued
                __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
            };
            issue_lds(0, 0);
            for (int i = 0; i < n; i += 2) {
                issue_lds(i + 1, 1);
                fold_lds(0);  // piece i (the one issued before piece i + 1)
                issue_lds(i + 2, 0);
                fold_lds(1);
            }
            __builtin_amdgcn_s_waitcnt(0);  // the last issue (zeros) lands before the next chunk
            continue;
        }
        u32x4 ring[2][2 * W];
        auto issue = [&](int i, u32x4 (&r)[2 * W]) {
            const int j = i < n ? i : 0;
            const int bytes = i < n ? TILE : 0;
            const uint64_t b0 = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(u0 >> 32), j) << 32) |
                                (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u0, j);
            const uint64_t b1 = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(u1 >> 32), j) << 32) |
                                (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u1, j);
            const auto r0 = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(b0), 0, bytes, kProbeBufferFlags);
            const auto r1 = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(b1), 0, bytes, kProbeBufferFlags);
#pragma unroll
            for (int w = 0; w < W; ++w) {
                r[w] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r0, 16 * lane + 1024 * w, 0, 2));
                r[W + w] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r1, 16 * lane + 1024 * w, 0, 2));
            }
        };
        auto fold = [&](const u32x4 (&r)[2 * W]) {
#pragma unroll
            for (int w = 0; w < 2 * W; ++w) acc ^= (r[w][0] ^ r[w][1]) ^ (r[w][2] ^ r[w][3]);
        };
        issue(0, ring[0]);
        for (int i = 0; i < n; i += 2) {
            issue(i + 1, ring[1]);
            fold(ring[0]);
            issue(i + 2, ring[0]);
            fold(ring[1]);
        }
        __builtin_amdgcn_s_waitcnt(0);  // the last issue (nothing, or zeros) completes before the next chunk
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o);
    if (lane == 0) wave_acc[wave] = acc;
    __syncthreads();
    if (tid == 0) {
        uint32_t x = 0;
#pragma unroll
        for (int w = 0; w < kProbeThreads / 64; ++w) x ^= wave_acc[w];
        partial[blockIdx.x] = x;
    }
}

}  // namespace

hipError_t launch_gather_probe(const void *k_cache, const void *v_cache, const int32_t *block_tables,
                               const int32_t *block_prefix, int num_seqs, int num_kv_heads, int head_dim,
                               int max_blocks_per_seq, int whole_blocks, uint32_t *partial, int num_workgroups,
                               hipStream_t stream) {
    auto kern = whole_blocks == 2
                    ? (head_dim == 64    ? paged_gather_probe_kernel<64, true>
                       : head_dim == 128 ? paged_gather_probe_kernel<128, true>
                                         : paged_gather_probe_kernel<256, true>)
                    : (head_dim == 64    ? paged_gather_probe_kernel<64, false>
                       : head_dim == 128 ? paged_gather_probe_kernel<128, false>
                                         : paged_gather_probe_kernel<256, false>);
    hipLaunchKernelGGL(kern, dim3((unsigned)num_workgroups), dim3(kProbeThreads), 0, stream,
                       static_cast<const char *>(k_cache), static_cast<const char *>(v_cache), block_tables,
                       block_prefix, num_seqs, num_kv_heads, max_blocks_per_seq, whole_blocks, partial);
    return hipGetLastError();
}

hipError_t launch_read_probe(const void *buf, long long bytes, uint32_t *partial, int num_workgroups,
                             hipStream_t stream) {
    hipLaunchKernelGGL(hbm_read_probe_kernel, dim3((unsigned)num_workgroups), dim3(kProbeThreads), 0,
                       stream, static_cast<const u32x4 *>(buf), bytes / 16, partial);
    return hipGetLastError();
}

}  // namespace pa
