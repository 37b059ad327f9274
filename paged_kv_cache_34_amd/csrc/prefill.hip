// Ragged paged prefill with a causal mask for gfx950 (CDNA4), on bf16 MFMA.
//
// What is computed: sequence s owns the packed query rows
// [cu_seqlens[s], cu_seqlens[s+1]) (the qo_indptr of the AstrAI "CUDA Kernels"
// page, "Q Scheduling and KV Addressing"); its n new tokens are the last n of
// its seq_lens[s] cached tokens, so row j sits at absolute position c + j
// (c = seq_lens[s] - n) and attends to keys t <= c + j -- the causal rule of
// the RL.cu "Add Cuda Kernel" page's prefill kernel, aligned to the end of the
// context.  K/V rows are gathered through the block table as in decode.
//
// Work decomposition:
//   * a workgroup of NW waves owns NW*32 (row, head) query slots of one kv
//     head: R = NW*32 / G consecutive rows times the G query heads sharing the
//     kv head (the AstrAI page's GQA head packing), so every K/V tile is read
//     once for all of them; wave w owns slots 32w .. 32w+31;
//   * KV is walked in 32-token tiles up to the last row's causal limit.  Each
//     thread keeps a ring of DEPTH+1 register tiles (global loads issued DEPTH
//     tiles ahead); K and V are staged row-major in a double-buffered LDS
//     tile, one barrier per tile;
//   * S^T = K Q^T is v_mfma_f32_32x32x16_bf16 with K (from LDS) as the A
//     operand and the wave's query slots (registers) as B; the accumulator
//     gives each lane 16 tokens of one slot, which is exactly the bf16 B
//     operand layout of O^T += V^T P^T on the same instruction.  The V^T A
//     operand is read from the row-major V tile with ds_read_b64_tr_b16 (two
//     reads of 4 tokens per 32x16 operand);
//   * online softmax per slot with a lazy running max (rescale only when a
//     tile's max exceeds it by more than 2^8), fp32 accumulation.
//
// Two launch forms:
//   * single pass: one workgroup per (query tile, kv head, sequence) walks all
//     of its keys and writes bf16 rows;
//   * split-KV: a (query tile, kv head) is cut into key chunks of C tokens
//     (the BI-V100 page's partitioning, section 2 "Level 3", applied to the
//     query tiles of a prefill).  A persistent grid takes the chunks from a
//     device counter, full chunks first and then the remainder chunks longest
//     first, so the long contexts no longer set the critical path.  Rows whose
//     keys all fall in the first chunk are written directly; the other rows
//     leave one partial record (running max, exp-sum, normalized output) per
//     chunk, and a merge kernel combines them with the page's combine rule.
#include <type_traits>

#include "pa_common.h"
#include "pa_launch.h"

namespace pa {

namespace {
constexpr int kPfWaves = 8;
constexpr int kPfSlots = kPfWaves * 32;  // (row, head) query slots per workgroup
static_assert(kPfSlots == kPfRowSlots, "slots per workgroup");
// KV tokens per tile: 64 (two S accumulators per wave) where the LDS allows
template <int D> constexpr int pf_tile() { return D >= 256 ? 32 : 64; }
constexpr int kTileMin = 32;
constexpr int kPfDepth = 2;              // register tiles in flight ahead of the one consumed
constexpr float kPfTau = 8.0f;
constexpr int kPfIdsLds = 1024;          // block ids staged in LDS (covers 16,384 tokens)
// Fourth word of a raw buffer descriptor on the GFX9 family (32-bit data, no swizzle).
constexpr int kPfBufferFlags = 0x00020000;
constexpr int kPfMaxBuckets = kPfMaxChunk / kTileMin + 1;  // remainder-length buckets (32 keys)

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2_pf __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_pf __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float max_xor32_pf(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32_pf(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
}  // namespace

// Kernel argument block (validated on the host).
struct PfParams {
    const uint16_t *q, *k_cache, *v_cache;
    const int32_t *block_tables, *seq_lens, *cu_seqlens;
    int num_seqs, total_q, num_q_heads, num_kv_heads, max_blocks_per_seq;
    float scale_log2;
    uint16_t *out;
    // split-KV only
    int chunk, max_splits;  // key chunk C (multiple of the tile); partial slots per (row, head)
    float *ws_m, *ws_l, *ws_o;
    int *counters;          // [0] next chunk to take, [1] workgroups done
};

// LDS of the tile pipeline.
template <int D>
struct __attribute__((aligned(16))) PfLds {
    uint16_t k[2][pf_tile<D>() * (D + 8)];   // K rows, +8 bf16 pad: conflict-free b128 reads
    uint16_t v[2][pf_tile<D>() * (D + 32)];  // V rows, +32 bf16 pad: the 4 rows x 64 bytes a
                                        // transposed read takes per 32 lanes hit all 64 banks
    int ids[kPfIdsLds];
};

// Keys [key_begin, key_end) of query tile `qtile` of sequence `seq`, kv head
// `kvh` (key_begin a multiple of the tile).  split < 0: the range is the
// tile's whole causal range and every row is written as bf16.  split >= 0:
// chunk `split` of size prm.chunk; rows whose keys all lie in the first chunk
// are written as bf16 (by chunk 0), the others leave a partial record for
// every chunk holding at least one of their keys.  `after_loop` runs in every
// thread once the last tile is done, before the results are written.
template <int D, int G, typename AfterLoop>
__device__ __forceinline__ void prefill_range(const PfParams &prm, PfLds<D> &lds, int seq, int kvh,
                                              int qtile, int key_begin, int key_end, int split,
                                              AfterLoop &&after_loop) {
    constexpr int R = kPfSlots / G;        // query rows per workgroup
    constexpr int KROW = D + 8;
    constexpr int VROW = D + 32;
    constexpr int NK = D / 16;             // k-steps of S^T
    constexpr int ND = D / 32;             // 32-dim tiles of O^T
    constexpr int CPT = D / 8;             // 16-byte chunks per token row
    constexpr int TPP = kPfWaves * 64 / CPT;  // tokens loaded per pass
    constexpr int KT = pf_tile<D>();       // keys per tile
    constexpr int NSA = KT / 32;           // S^T accumulators (32 keys each) per tile
    constexpr int PASSES = (KT + TPP - 1) / TPP;
    constexpr int DEPTH = D >= 256 ? 1 : kPfDepth;
    static_assert(DEPTH >= 1 && DEPTH <= 3, "ring depth");
    const uint16_t *__restrict__ k_cache = prm.k_cache;
    const uint16_t *__restrict__ v_cache = prm.v_cache;
    const float scale_log2 = prm.scale_log2;
    const int num_q_heads = prm.num_q_heads;

    const int q0 = prm.cu_seqlens[seq];
    const int n = prm.cu_seqlens[seq + 1] - q0;
    const int r0 = qtile * R;
    const int L = prm.seq_lens[seq];
    const int c = L - n;
    const int rows = min(R, n - r0);
    const int tb = key_begin / KT;
    const int te = (key_end + KT - 1) / KT;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31, grp = lane >> 5;
    // slots are row-major (slot = row * G + head), so the waves of a short
    // last query tile that hold only padding rows are the high ones, one per
    // SIMD (waves w and w + 4 share a SIMD), and skip their math
    const int slot = wave * 32 + col;
    const int hq = slot % G, rq = slot / G;          // head within group, row within tile
    const bool q_ok = rq < rows;
    const bool wave_live = __builtin_amdgcn_readfirstlane((wave * 32) / G) < rows;
    const int limit = c + r0 + rq;                   // last visible key of this slot

    // query slot as the B operand of S^T: 8 consecutive d per lane per k-step
    u32x4 qf[NK];
    {
        const uint16_t *qrow =
            prm.q + ((long)(q0 + r0 + (q_ok ? rq : 0)) * num_q_heads + kvh * G + (q_ok ? hq : 0)) * D +
            grp * 8;
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
            const u32x4 v = load_u32x4(qrow + kk * 16);
            qf[kk] = q_ok ? v : u32x4{0u, 0u, 0u, 0u};
        }
    }

    f32x16 o[ND];
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    const int32_t *bt_row = prm.block_tables + (long)seq * prm.max_blocks_per_seq;
    const long tile_elems = 16L * D;
    const long blk_stride = (long)prm.num_kv_heads * tile_elems;
    const int ld_tok = tid / CPT, ld_chunk = tid % CPT;
    // the block ids of the range, staged once (no table read in the loop)
    const int b0 = key_begin / 16;
    const int nblk = (key_end + 15) / 16 - b0;
    for (int b = tid; b < min(nblk, kPfIdsLds); b += kPfWaves * 64) lds.ids[b] = bt_row[b0 + b];
    __syncthreads();

    // Tile tt's rows for this thread: one 16-byte chunk of token ps*TPP + ld_tok.
    // The 512/D tokens a wave loads in one pass lie in one 16-token block, so
    // the block id and the buffer descriptor are wave-uniform.  The descriptor
    // covers only the block's rows below key_end, so the rest of the last tile
    // and whole tiles past it read as zeros without touching memory, and the
    // loads stay unconditional.  Block ids come from LDS (staged above) or,
    // past the staged range, from the table with a scalar load.
    const int wtok = __builtin_amdgcn_readfirstlane(wave * (64 / CPT));  // wave's first token in a pass
    const int ld_voff = ((ld_tok & 15) * D + ld_chunk * 8) * 2;          // bytes within a block tile
    const auto *bt_const = (const __attribute__((address_space(4))) int32_t *)bt_row;
    auto load_regs = [&](int tt, u32x4 (&kr)[PASSES], u32x4 (&vr)[PASSES]) {
#pragma unroll
        for (int ps = 0; ps < PASSES; ++ps) {
            const int tl0 = ps * TPP + wtok;   // the wave's first token within the tile
            const int b = (tt * KT + tl0) >> 4;
            const int rows = tl0 < KT ? min(max(key_end - b * 16, 0), 16) : 0;
            int phys = 0;
            if (rows > 0) phys = b - b0 < kPfIdsLds ? lds.ids[b - b0] : bt_const[b];
            phys = __builtin_amdgcn_readfirstlane(phys);
            const long base = (long)phys * blk_stride + kvh * tile_elems;
            const int bytes = rows * D * 2;
            const auto krs = __builtin_amdgcn_make_buffer_rsrc((void *)(k_cache + base), 0, bytes, kPfBufferFlags);
            const auto vrs = __builtin_amdgcn_make_buffer_rsrc((void *)(v_cache + base), 0, bytes, kPfBufferFlags);
            kr[ps] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, ld_voff, 0, 0));
            vr[ps] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs, ld_voff, 0, 0));
        }
    };
    auto store_lds = [&](int buf, const u32x4 (&kr)[PASSES], const u32x4 (&vr)[PASSES]) {
#pragma unroll
        for (int ps = 0; ps < PASSES; ++ps) {
            const int tl = ps * TPP + ld_tok;
            if (tl < KT) {
                *reinterpret_cast<u32x4 *>(&lds.k[buf][tl * KROW + ld_chunk * 8]) = kr[ps];
                *reinterpret_cast<u32x4 *>(&lds.v[buf][tl * VROW + ld_chunk * 8]) = vr[ps];
            }
        }
    };

    // transposed-read lane address pieces (16-lane group gamma, lane rho in it)
    const int rho = lane & 15, gamma = lane >> 4;
    const int vt_row = 4 * (gamma >> 1) + (rho >> 2);                 // + 16 ks + 8 h
    const int vt_col = 16 * (gamma & 1) + 4 * (rho & 3);              // + 32 dt

    auto compute = [&](int tt, int buf) {
        // S^T of the tile's NSA blocks of 32 keys: independent accumulator
        // chains, interleaved
        f32x16 s[NSA];
#pragma unroll
        for (int a = 0; a < NSA; ++a)
#pragma unroll
            for (int i = 0; i < 16; ++i) s[a][i] = 0.f;
        const uint16_t *kl = &lds.k[buf][col * KROW + grp * 8];
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
#pragma unroll
            for (int a = 0; a < NSA; ++a) {
                const u32x4 ka = *reinterpret_cast<const u32x4 *>(kl + a * 32 * KROW + kk * 16);
                s[a] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ka),
                                                               __builtin_bit_cast(bf16x8, qf[kk]), s[a], 0, 0, 0);
            }
        }
        // keep SAHEAD K operand reads in flight ahead of the MFMAs (the
        // compiler's own order issues them one MFMA ahead); D = 256 has no
        // registers to spare for them
        if constexpr (D <= 128) {
            constexpr int NSM = NK * NSA, SAHEAD = NSM < 4 ? NSM : 4;
            __builtin_amdgcn_sched_group_barrier(0x100, SAHEAD, 0);  // DS reads
#pragma unroll
            for (int z = 0; z < NSM - SAHEAD; ++z) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, SAHEAD, 0);
        }
        // lane holds tokens 32a + (i/4)*8 + 4*grp + i%4 of this tile for query
        // slot `col`; only tiles reaching past the first row's causal limit
        // (or the end of the visible keys) need the mask.  With scale > 0 the
        // max of the raw scores gives the max of the scaled ones, and the
        // scaling folds into the exponent's FMA below.
        const int tbase = tt * KT + 4 * grp;
        float mr = -INFINITY;
        if (tt * KT + KT - 1 > c + r0) {
#pragma unroll
            for (int a = 0; a < NSA; ++a)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int t = tbase + 32 * a + (i >> 2) * 8 + (i & 3);
                    s[a][i] = (t <= limit) ? s[a][i] : -INFINITY;
                    mr = fmaxf(mr, s[a][i]);
                }
        } else {
#pragma unroll
            for (int a = 0; a < NSA; ++a)
#pragma unroll
                for (int i = 0; i < 16; ++i) mr = fmaxf(mr, s[a][i]);
        }
        const float bm = max_xor32_pf(mr) * scale_log2;  // tile max, log2 units
        if (__any(bm > m_run + kPfTau)) {
            const float mn = fmaxf(m_run, bm);
            const float al = (mn == -INFINITY) ? 1.f : fast_exp2(m_run - mn);
            m_run = mn;
            l_run *= al;
#pragma unroll
            for (int dt = 0; dt < ND; ++dt) o[dt] *= al;
        }
        // a slot that has seen no visible key yet keeps m_run = -inf; its
        // probabilities are zero (exp2(-inf) after shifting by a finite 0)
        const float msh = (m_run == -INFINITY) ? 0.f : m_run;
        u32x4 pk[2 * NSA];
        float ls = 0.f;
#pragma unroll
        for (int a = 0; a < NSA; ++a)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const float x0 = fast_exp2(fmaf(s[a][8 * h + 2 * k], scale_log2, -msh));
                    const float x1 = fast_exp2(fmaf(s[a][8 * h + 2 * k + 1], scale_log2, -msh));
                    ls += x0 + x1;
                    pk[2 * a + h][k] =
                        __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_pf{x0, x1}, bf16x2_pf));
                }
            }
        l_run += ls;
        const uint16_t *vl = &lds.v[buf][0];
#pragma unroll
        for (int ks = 0; ks < 2 * NSA; ++ks) {
#pragma unroll
            for (int dt = 0; dt < ND; ++dt) {
                // A operand: V[16 ks + 8 h + 4 (lane/32) + 0..3][dim lane%32 + 32 dt], h = 0, 1
                const uint16_t *a0 = vl + (16 * ks + vt_row) * VROW + 32 * dt + vt_col;
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (s16x4 __attribute__((address_space(3))) *)(a0));
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (s16x4 __attribute__((address_space(3))) *)(a0 + 8 * VROW));
                const u32x4 va = {__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                                  __builtin_bit_cast(u32x2, hi)[0], __builtin_bit_cast(u32x2, hi)[1]};
                o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, va),
                                                                __builtin_bit_cast(bf16x8, pk[ks]), o[dt],
                                                                0, 0, 0);
            }
        }
    };

    // software pipeline: ring of DEPTH+1 register tiles, double-buffered LDS
    u32x4 kreg[DEPTH + 1][PASSES], vreg[DEPTH + 1][PASSES];
#pragma unroll
    for (int d = 0; d <= DEPTH; ++d) load_regs(tb + d, kreg[d], vreg[d]);
    store_lds(tb & 1, kreg[0], vreg[0]);
    __syncthreads();
    // One step: compute tile tt from LDS; tile tt+1 (ring slot u+1) goes to
    // the other LDS buffer; slot u is refilled with tile tt + DEPTH + 1.
    auto step = [&](int tt, auto uc) {
        constexpr int u = decltype(uc)::value;
        if (wave_live) compute(tt, tt & 1);
        store_lds((tt + 1) & 1, kreg[(u + 1) % (DEPTH + 1)], vreg[(u + 1) % (DEPTH + 1)]);
        load_regs(tt + DEPTH + 1, kreg[u], vreg[u]);
        __syncthreads();
    };
    // Full groups of DEPTH + 1 steps have no guards, so the loop's back edge
    // always comes after the last slot's refill (the compiler's wait counts
    // for the ring stay exact); the remaining steps follow the loop.
    int t0 = tb;
    for (; t0 + DEPTH < te; t0 += DEPTH + 1) {
        step(t0, std::integral_constant<int, 0>{});
        if constexpr (DEPTH >= 1) step(t0 + 1, std::integral_constant<int, 1>{});
        if constexpr (DEPTH >= 2) step(t0 + 2, std::integral_constant<int, 2>{});
        if constexpr (DEPTH >= 3) step(t0 + 3, std::integral_constant<int, 3>{});
    }
    if (t0 < te) step(t0, std::integral_constant<int, 0>{});
    if constexpr (DEPTH >= 2) if (t0 + 1 < te) step(t0 + 1, std::integral_constant<int, 1>{});
    if constexpr (DEPTH >= 3) if (t0 + 2 < te) step(t0 + 2, std::integral_constant<int, 2>{});

    after_loop();
    const float l_tot = sum_xor32_pf(l_run);
    if (!q_ok) return;
    if (split >= 0 && limit < key_begin) return;  // no key of this row in the chunk
    const int row = q0 + r0 + rq, head = kvh * G + hq;
    if (split < 0 || limit < prm.chunk) {
        const float inv = 1.f / l_tot;
        uint16_t *orow = prm.out + ((long)row * num_q_heads + head) * D;
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int d0 = dt * 32 + i4 * 8 + 4 * grp;
                u32x2 w;
                w[0] = pack_bf16x2(o[dt][4 * i4] * inv, o[dt][4 * i4 + 1] * inv);
                w[1] = pack_bf16x2(o[dt][4 * i4 + 2] * inv, o[dt][4 * i4 + 3] * inv);
                *reinterpret_cast<u32x2 *>(orow + d0) = w;
            }
    } else {
        const long rec = ((long)row * num_q_heads + head) * prm.max_splits + split;
        if (grp == 0) {
            prm.ws_m[rec] = m_run;
            prm.ws_l[rec] = l_tot;
        }
        const float inv = 1.f / l_tot;
        float *orec = prm.ws_o + rec * D;
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int d0 = dt * 32 + i4 * 8 + 4 * grp;
                *reinterpret_cast<f32x4 *>(orec + d0) =
                    f32x4{o[dt][4 * i4] * inv, o[dt][4 * i4 + 1] * inv, o[dt][4 * i4 + 2] * inv,
                          o[dt][4 * i4 + 3] * inv};
            }
    }
}

// Single pass: one workgroup per (query tile, kv head, sequence).
template <int D, int G>
__global__ __launch_bounds__(kPfWaves * 64) void paged_prefill_kernel(PfParams prm) {
    constexpr int R = kPfSlots / G;
    __shared__ PfLds<D> lds;
    const int qtile = blockIdx.x, kvh = blockIdx.y, seq = blockIdx.z;
    const int q0 = prm.cu_seqlens[seq];
    const int n = prm.cu_seqlens[seq + 1] - q0;
    const int r0 = qtile * R;
    if (r0 >= n) return;
    const int c = prm.seq_lens[seq] - n;
    const int kv_end = c + r0 + min(R, n - r0);  // keys [0, kv_end) are visible to some row
    prefill_range<D, G>(prm, lds, seq, kvh, qtile, 0, kv_end, -1, [] {});
}

// Split-KV, persistent.  Every workgroup builds the same chunk list in LDS:
//   pairs (sequence, query tile) in sequence order, with kv_end = the pair's
//   last row's causal limit + 1;
//   chunks: for every pair floor(kv_end / C) full chunks, then one remainder
//   chunk if kv_end % C > 0; each chunk once per kv head.
// Chunk order: all full chunks (pair, kv head, chunk), then the remainder
// chunks by decreasing length (pair order among equals; a bitonic sort of the
// pairs keeps it deterministic, so every workgroup sees the same list).
// Workgroup w takes chunk w first, then chunk indices gridDim.x +
// counters[0]++; the last workgroup to finish resets both counters to zero
// for the next launch.
template <int D, int G>
__global__ __launch_bounds__(kPfWaves * 64) void paged_prefill_split_kernel(PfParams prm) {
    constexpr int R = kPfSlots / G;
    constexpr int T = kPfWaves * 64;
    constexpr int SPT = (kPfMaxSeqs + T - 1) / T;   // sequences per thread
    constexpr int PPT = (kPfMaxPairs + T - 1) / T;  // pairs per thread
    static_assert(kPfMaxPairs == 2 * T, "one compare-exchange per thread and sort stage");
    __shared__ PfLds<D> lds;
    __shared__ int pr_seq[kPfMaxPairs], pr_qt[kPfMaxPairs], pr_kv[kPfMaxPairs];
    __shared__ int fpref[kPfMaxPairs], rorder[kPfMaxPairs];
    __shared__ int wtot[kPfWaves], bcast[1];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int S = prm.num_seqs, C = prm.chunk, hkv = prm.num_kv_heads;

    // workgroup-wide exclusive scan of one value per thread
    auto block_scan = [&](int v, int &total) {
        int incl = v;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int y = __shfl_up(incl, d);
            if (lane >= d) incl += y;
        }
        if (lane == 63) wtot[wave] = incl;
        __syncthreads();
        int run = incl - v, tot = 0;
#pragma unroll
        for (int w = 0; w < kPfWaves; ++w) {
            if (w < wave) run += wtot[w];
            tot += wtot[w];
        }
        __syncthreads();
        total = tot;
        return run;
    };

    // 1. pairs (sequence, query tile); the lengths are all loaded in one round
    int nq[SPT], nn[SPT], sq[SPT];
    int local = 0;
#pragma unroll
    for (int k = 0; k < SPT; ++k) {
        const int i = tid * SPT + k;
        nn[k] = 0;
        sq[k] = 0;
        if (i < S) {
            nn[k] = prm.cu_seqlens[i + 1] - prm.cu_seqlens[i];
            sq[k] = prm.seq_lens[i];
        }
        nq[k] = (nn[k] + R - 1) / R;
        local += nq[k];
    }
    int NP = 0;
    int run = block_scan(local, NP);
    NP = min(NP, kPfMaxPairs);
#pragma unroll
    for (int k = 0; k < SPT; ++k) {
        const int i = tid * SPT + k;
        if (i < S) {
            const int n = nn[k];
            const int c = sq[k] - n;
            for (int qt = 0; qt < nq[k] && run + qt < kPfMaxPairs; ++qt) {
                pr_seq[run + qt] = i;
                pr_qt[run + qt] = qt;
                pr_kv[run + qt] = c + qt * R + min(R, n - qt * R);
            }
        }
        run += nq[k];
    }
    __syncthreads();

    // 2. full chunks: prefix over pairs; remainders: sort keys
    int fl[PPT];
    int flocal = 0;
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
        const int p = tid * PPT + k;
        fl[k] = p < NP ? (pr_kv[p] / C) * hkv : 0;
        flocal += fl[k];
        int key = 0x7fffffff;
        if (p < NP) {
            const int rem = pr_kv[p] % C;
            if (rem > 0) key = ((kPfMaxBuckets - (rem + kTileMin - 1) / kTileMin) << 11) | p;
        }
        rorder[p] = key;
    }
    int F = 0;
    int frun = block_scan(flocal, F);
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
        const int p = tid * PPT + k;
        fpref[p] = frun;
        frun += fl[k];
    }
    // bitonic sort of the keys, ascending (longest remainder first, then
    // pair), over the first power of two >= NP entries (the rest are unused
    // pairs, keyed last already).  Up to 64 entries one wave sorts them in
    // registers; up to 128 one wave sorts them in LDS (its LDS accesses
    // execute in program order, so no barrier is needed between stages); more
    // entries take the workgroup, a barrier per stage.
    int n2 = 2;
    while (n2 < NP) n2 <<= 1;
    auto cmp_exchange = [&](int t, int k, int j) {
        const int i = 2 * t - (t & (j - 1));
        const int l = i + j;
        const int a = rorder[i], b = rorder[l];
        if ((a > b) == ((i & k) == 0)) {
            rorder[i] = b;
            rorder[l] = a;
        }
    };
    if (n2 <= 64) {
        // one key per lane of wave 0; each stage exchanges with lane ^ j
        // (the same network, in registers)
        if (wave == 0) {
            int key = rorder[lane];
            for (int k = 2; k <= n2; k <<= 1)
                for (int j = k >> 1; j > 0; j >>= 1) {
                    const int other = __shfl_xor(key, j);
                    const bool up = (lane & k) == 0, lower = (lane & j) == 0;
                    key = (lower == up) ? min(key, other) : max(key, other);
                }
            if (lane < n2) rorder[lane] = key;
        }
        __syncthreads();
    } else if (n2 <= 128) {
        if (wave == 0) {
            for (int k = 2; k <= n2; k <<= 1)
                for (int j = k >> 1; j > 0; j >>= 1) {
                    if (lane < n2 / 2) cmp_exchange(lane, k, j);
                    __builtin_amdgcn_wave_barrier();
                }
        }
        __syncthreads();
    } else {
        for (int k = 2; k <= n2; k <<= 1)
            for (int j = k >> 1; j > 0; j >>= 1) {
                if (tid < n2 / 2) cmp_exchange(tid, k, j);
                __syncthreads();
            }
    }
    int nrem_local = 0;
#pragma unroll
    for (int k = 0; k < PPT; ++k) nrem_local += rorder[tid * PPT + k] != 0x7fffffff;
    int NR = 0;
    block_scan(nrem_local, NR);
    const int total = F + NR * hkv;

    // 3. take chunks: the first is blockIdx.x, the later ones come from the
    // device counter (offset by the grid).  The claim of the next chunk is
    // issued once the current one's tiles are done, before its results are
    // written, and travels through LDS, so neither its round trip nor the
    // results' stores hold up the next chunk's start.
    int it = blockIdx.x;
    while (it < total) {
        int p, kvh, split;
        if (it < F) {
            int lo = 0, hi = NP;  // the last pair with fpref[p] <= it
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (fpref[mid] <= it) lo = mid; else hi = mid;
            }
            p = __builtin_amdgcn_readfirstlane(lo);
            const int nf = __builtin_amdgcn_readfirstlane(pr_kv[p] / C);
            const int r = it - fpref[p];
            kvh = r / nf;
            split = r % nf;
        } else {
            const int r = it - F;
            p = rorder[r / hkv] & 2047;
            kvh = r % hkv;
            split = pr_kv[p] / C;
        }
        p = __builtin_amdgcn_readfirstlane(p);
        kvh = __builtin_amdgcn_readfirstlane(kvh);
        split = __builtin_amdgcn_readfirstlane(split);
        const int kv_end = __builtin_amdgcn_readfirstlane(pr_kv[p]);
        const int kb = split * C;
        int claim = 0;
        prefill_range<D, G>(prm, lds, __builtin_amdgcn_readfirstlane(pr_seq[p]), kvh,
                            __builtin_amdgcn_readfirstlane(pr_qt[p]), kb, min(kb + C, kv_end), split, [&] {
                                if (tid == 0) claim = (int)gridDim.x + atomicAdd(prm.counters, 1);
                            });
        if (tid == 0) bcast[0] = claim;
        lds_barrier();
        it = __builtin_amdgcn_readfirstlane(bcast[0]);
    }
    if (tid == 0) {
        const int done = __hip_atomic_fetch_add(prm.counters + 1, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        if (done == (int)gridDim.x - 1) {
            __hip_atomic_store(prm.counters, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(prm.counters + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// Merge of the split-KV partial records (the BI-V100 page's combine rule):
// one workgroup per (new row, sequence); rows whose keys all lie in the first
// chunk were written by the prefill kernel and are skipped.  The chunk maxima
// and exp-sums of every head are staged in LDS with one round of independent
// loads; each head's maximum M and sum S = sum_j 2^(m_j - M) l_j come from
// LDS; the weights w_j = 2^(m_j - M) l_j / S replace the staged maxima; then
// each thread forms 4 consecutive output dims of one head from 16-byte loads
// of the chunk outputs, chunks in a fixed order.  Rows with more chunks than
// one LDS pass holds take several passes (the running sum is parked in chunk
// 0's record between them).
constexpr int kMergeThreads = 256;
constexpr int kMergeMaxHeads = kPfMaxHeads;  // query heads per row held in LDS
constexpr int kMergeSplits = 32;             // chunks per row held in LDS per pass
constexpr int kMergeSpecChunks = 4;          // fast path: at most this many chunks per row ...
constexpr int kMergeSpecCols = 4;            // ... and 4-dim columns per thread

template <int D>
__global__ __launch_bounds__(kMergeThreads) void paged_prefill_merge_kernel(PfParams prm) {
    __shared__ float sm[kMergeMaxHeads * kMergeSplits];  // chunk maxima, then weights
    __shared__ float sl[kMergeMaxHeads * kMergeSplits];  // chunk exp-sums
    __shared__ float hmax[kMergeMaxHeads], hsum[kMergeMaxHeads];
    constexpr int T = kMergeThreads, SP = kMergeSplits;
    const int s = blockIdx.y, jrow = blockIdx.x;  // sequence, new row within it
    const int q0 = prm.cu_seqlens[s];
    const int n = prm.cu_seqlens[s + 1] - q0;
    if (jrow >= n) return;
    const int visible = prm.seq_lens[s] - n + jrow + 1;
    const int ns = (visible + prm.chunk - 1) / prm.chunk;
    if (ns <= 1) return;
    const int row = q0 + jrow, hq = prm.num_q_heads;
    const long rec_row = (long)row * hq * prm.max_splits;
    auto stage = [&](int j0, int nj) {
        for (int e = threadIdx.x; e < hq * nj; e += T) {
            const int h = e / nj, j = e - h * nj;
            const long r = rec_row + (long)h * prm.max_splits + j0 + j;
            sm[h * SP + j] = prm.ws_m[r];
            sl[h * SP + j] = prm.ws_l[r];
        }
    };
    // Few chunks and at most kMergeSpecCols columns per thread: the chunk
    // outputs are loaded together with the maxima and exp-sums (one round of
    // loads instead of two); the arithmetic is that of the general path below.
    if (ns <= kMergeSpecChunks && hq * (D / 4) <= kMergeSpecCols * T) {
        f32x4 ov[kMergeSpecCols][kMergeSpecChunks];
#pragma unroll
        for (int k = 0; k < kMergeSpecCols; ++k) {
            const int e = threadIdx.x + k * T;
            if (e < hq * (D / 4)) {
                const int h = e / (D / 4), d0 = (e % (D / 4)) * 4;
                const float *o = prm.ws_o + (rec_row + (long)h * prm.max_splits) * D + d0;
#pragma unroll
                for (int j = 0; j < kMergeSpecChunks; ++j)
                    if (j < ns) ov[k][j] = *reinterpret_cast<const f32x4 *>(o + (long)j * D);
            }
        }
        stage(0, ns);
        __syncthreads();
        for (int h = threadIdx.x; h < hq; h += T) {
            float M = -INFINITY, S = 0.f;
            for (int j = 0; j < ns; ++j) {
                const float mj = sm[h * SP + j];
                if (mj > M) {
                    S *= fast_exp2(M - mj);
                    M = mj;
                }
                S += fast_exp2(mj - M) * sl[h * SP + j];
            }
            hmax[h] = M;
            hsum[h] = S;
        }
        __syncthreads();
        for (int e = threadIdx.x; e < hq * ns; e += T) {
            const int h = e / ns, j = e - h * ns;
            sm[h * SP + j] = fast_exp2(sm[h * SP + j] - hmax[h]) * sl[h * SP + j] / hsum[h];
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kMergeSpecCols; ++k) {
            const int e = threadIdx.x + k * T;
            if (e < hq * (D / 4)) {
                const int h = e / (D / 4), d0 = (e % (D / 4)) * 4;
                const float *w = sm + h * SP;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < kMergeSpecChunks; ++j)
                    if (j < ns) acc += w[j] * ov[k][j];
                uint16_t *orow = prm.out + ((long)row * hq + h) * D + d0;
                u32x2 wv;
                wv[0] = pack_bf16x2(acc[0], acc[1]);
                wv[1] = pack_bf16x2(acc[2], acc[3]);
                *reinterpret_cast<u32x2 *>(orow) = wv;
            }
        }
        return;
    }
    // per-head maximum and exp-sum over all chunks (online across passes)
    for (int j0 = 0; j0 < ns; j0 += SP) {
        const int nj = min(SP, ns - j0);
        if (j0 > 0) __syncthreads();
        stage(j0, nj);
        __syncthreads();
        for (int h = threadIdx.x; h < hq; h += T) {
            float M = j0 ? hmax[h] : -INFINITY, S = j0 ? hsum[h] : 0.f;
            for (int j = 0; j < nj; ++j) {
                const float mj = sm[h * SP + j];
                if (mj > M) {
                    S *= fast_exp2(M - mj);
                    M = mj;
                }
                S += fast_exp2(mj - M) * sl[h * SP + j];
            }
            hmax[h] = M;
            hsum[h] = S;
        }
    }
    // weights and the weighted sum, pass by pass
    for (int j0 = 0; j0 < ns; j0 += SP) {
        const int nj = min(SP, ns - j0);
        __syncthreads();
        if (ns > SP) {  // (a single pass still holds its records in LDS)
            stage(j0, nj);
            __syncthreads();
        }
        for (int e = threadIdx.x; e < hq * nj; e += T) {
            const int h = e / nj, j = e - h * nj;
            sm[h * SP + j] = fast_exp2(sm[h * SP + j] - hmax[h]) * sl[h * SP + j] / hsum[h];
        }
        __syncthreads();
        for (int e = threadIdx.x; e < hq * (D / 4); e += T) {
            const int h = e / (D / 4), d0 = (e % (D / 4)) * 4;
            const float *w = sm + h * SP;
            const float *o = prm.ws_o + (rec_row + (long)h * prm.max_splits + j0) * D + d0;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            if (j0 > 0) {  // continue the earlier passes' sum, parked in chunk 0's record
                const float *prev = prm.ws_o + (rec_row + (long)h * prm.max_splits) * D + d0;
                acc = *reinterpret_cast<const f32x4 *>(prev);
            }
            int j = 0;
            for (; j + 4 <= nj; j += 4) {
                const f32x4 a0 = *reinterpret_cast<const f32x4 *>(o + (long)(j + 0) * D);
                const f32x4 a1 = *reinterpret_cast<const f32x4 *>(o + (long)(j + 1) * D);
                const f32x4 a2 = *reinterpret_cast<const f32x4 *>(o + (long)(j + 2) * D);
                const f32x4 a3 = *reinterpret_cast<const f32x4 *>(o + (long)(j + 3) * D);
                acc += w[j] * a0;
                acc += w[j + 1] * a1;
                acc += w[j + 2] * a2;
                acc += w[j + 3] * a3;
            }
            for (; j < nj; ++j) acc += w[j] * *reinterpret_cast<const f32x4 *>(o + (long)j * D);
            if (j0 + nj < ns) {
                float *first = prm.ws_o + (rec_row + (long)h * prm.max_splits) * D + d0;
                *reinterpret_cast<f32x4 *>(first) = acc;
            } else {
                uint16_t *orow = prm.out + ((long)row * hq + h) * D + d0;
                u32x2 wv;
                wv[0] = pack_bf16x2(acc[0], acc[1]);
                wv[1] = pack_bf16x2(acc[2], acc[3]);
                *reinterpret_cast<u32x2 *>(orow) = wv;
            }
        }
    }
}

namespace {

template <int D, int G>
hipError_t launch_prefill_dg(const PrefillArgs &a) {
    constexpr int R = kPfSlots / G;
    PfParams prm{a.q, a.k_cache, a.v_cache, a.block_tables, a.seq_lens, a.cu_seqlens,
                 a.num_seqs, a.total_q, a.num_q_heads, a.num_kv_heads, a.max_blocks_per_seq,
                 a.scale_log2, a.out, a.chunk, a.max_splits, a.ws_m, a.ws_l, a.ws_o, a.counters};
    dim3 block(kPfWaves * 64);
    if (a.chunk > 0) {
        const int per_cu = resident_per_cu<paged_prefill_split_kernel<D, G>>(block.x);
        hipLaunchKernelGGL((paged_prefill_split_kernel<D, G>), dim3(device_cu_count() * per_cu), block, 0,
                           a.stream, prm);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((paged_prefill_merge_kernel<D>), dim3(a.max_q_len, a.num_seqs), dim3(kMergeThreads), 0,
                           a.stream, prm);
        return hipGetLastError();
    }
    dim3 grid((a.max_q_len + R - 1) / R, a.num_kv_heads, a.num_seqs);
    hipLaunchKernelGGL((paged_prefill_kernel<D, G>), grid, block, 0, a.stream, prm);
    return hipGetLastError();
}

template <int D>
hipError_t launch_prefill_d(const PrefillArgs &a, int G) {
    switch (G) {
        case 1: return launch_prefill_dg<D, 1>(a);
        case 2: return launch_prefill_dg<D, 2>(a);
        case 3: return launch_prefill_dg<D, 3>(a);
        case 4: return launch_prefill_dg<D, 4>(a);
        case 5: return launch_prefill_dg<D, 5>(a);
        case 6: return launch_prefill_dg<D, 6>(a);
        case 7: return launch_prefill_dg<D, 7>(a);
        case 8: return launch_prefill_dg<D, 8>(a);
        case 9: return launch_prefill_dg<D, 9>(a);
        case 10: return launch_prefill_dg<D, 10>(a);
        case 11: return launch_prefill_dg<D, 11>(a);
        case 12: return launch_prefill_dg<D, 12>(a);
        case 13: return launch_prefill_dg<D, 13>(a);
        case 14: return launch_prefill_dg<D, 14>(a);
        case 15: return launch_prefill_dg<D, 15>(a);
        case 16: return launch_prefill_dg<D, 16>(a);
        default: return hipErrorInvalidValue;
    }
}
}  // namespace

hipError_t launch_prefill(const PrefillArgs &a) {
    const int G = a.num_q_heads / a.num_kv_heads;
    switch (a.head_dim) {
        case 64: return launch_prefill_d<64>(a, G);
        case 128: return launch_prefill_d<128>(a, G);
        case 256: return launch_prefill_d<256>(a, G);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pa
