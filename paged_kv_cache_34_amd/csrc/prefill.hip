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
#include <type_traits>

#include "pa_common.h"
#include "pa_launch.h"

namespace pa {

namespace {
constexpr int kPfWaves = 8;
constexpr int kPfSlots = kPfWaves * 32;  // (row, head) query slots per workgroup
constexpr int kKvTile = 32;              // KV tokens per tile
constexpr int kPfDepth = 3;              // register tiles in flight ahead of the one consumed
constexpr float kPfTau = 8.0f;
constexpr int kPfIdsLds = 1024;          // block ids staged in LDS (covers 16,384 tokens)
// Fourth word of a raw buffer descriptor on the GFX9 family (32-bit data, no swizzle).
constexpr int kPfBufferFlags = 0x00020000;

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

template <int D, int G>
__global__ __launch_bounds__(kPfWaves * 64) void paged_prefill_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k_cache,
    const uint16_t *__restrict__ v_cache, const int32_t *__restrict__ block_tables,
    const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ cu_seqlens,
    int num_q_heads, int num_kv_heads, int max_blocks_per_seq, float scale_log2,
    uint16_t *__restrict__ out) {
    constexpr int R = kPfSlots / G;        // query rows per workgroup
    constexpr int KROW = D + 8;            // bf16 per staged K row (conflict-free b128 reads)
    constexpr int VROW = D + 32;           // bf16 per staged V row: the 4 rows x 64 bytes a
                                           // transposed read takes per 32 lanes hit all 64 banks
    constexpr int NK = D / 16;             // k-steps of S^T
    constexpr int ND = D / 32;             // 32-dim tiles of O^T
    constexpr int CPT = D / 8;             // 16-byte chunks per token row
    constexpr int TPP = kPfWaves * 64 / CPT;  // tokens loaded per pass
    constexpr int PASSES = (kKvTile + TPP - 1) / TPP;
    constexpr int DEPTH = D >= 256 ? 1 : kPfDepth;
    static_assert(DEPTH >= 1 && DEPTH <= 3, "ring depth");
    __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][kKvTile * KROW];
    __shared__ __attribute__((aligned(16))) uint16_t v_lds[2][kKvTile * VROW];
    __shared__ int ids_lds[kPfIdsLds];

    const int qtile = blockIdx.x, kvh = blockIdx.y, seq = blockIdx.z;
    const int q0 = cu_seqlens[seq];
    const int n = cu_seqlens[seq + 1] - q0;
    const int r0 = qtile * R;
    if (r0 >= n) return;
    const int L = seq_lens[seq];
    const int c = L - n;
    const int rows = min(R, n - r0);
    const int kv_end = c + r0 + rows;  // keys [0, kv_end) are visible to some row
    const int ntiles = (kv_end + kKvTile - 1) / kKvTile;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31, grp = lane >> 5;
    const int slot = wave * 32 + col;
    const int hq = slot / R, rq = slot % R;          // head within group, row within tile
    const bool q_ok = hq < G && rq < rows;
    const int limit = c + r0 + rq;                   // last visible key of this slot

    // query slot as the B operand of S^T: 8 consecutive d per lane per k-step
    u32x4 qf[NK];
    {
        const uint16_t *qrow =
            q + ((long)(q0 + r0 + (q_ok ? rq : 0)) * num_q_heads + kvh * G + (q_ok ? hq : 0)) * D +
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

    const int32_t *bt_row = block_tables + (long)seq * max_blocks_per_seq;
    const long tile_elems = 16L * D;
    const long blk_stride = (long)num_kv_heads * tile_elems;
    const int ld_tok = tid / CPT, ld_chunk = tid % CPT;
    // the block ids this workgroup walks, staged once (no table read in the loop)
    const int nblk = (kv_end + 15) / 16;
    for (int b = tid; b < min(nblk, kPfIdsLds); b += kPfWaves * 64) ids_lds[b] = bt_row[b];
    __syncthreads();

    // Tile tt's rows for this thread: one 16-byte chunk of token ps*TPP + ld_tok.
    // The 512/D tokens a wave loads in one pass lie in one 16-token block, so
    // the block id and the buffer descriptor are wave-uniform.  The descriptor
    // covers only the block's rows below kv_end, so the rest of the last tile
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
            const int b = (tt * kKvTile + tl0) >> 4;
            const int rows = tl0 < kKvTile ? min(max(kv_end - b * 16, 0), 16) : 0;
            int phys = 0;
            if (rows > 0) phys = b < kPfIdsLds ? ids_lds[b] : bt_const[b];
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
            if (tl < kKvTile) {
                *reinterpret_cast<u32x4 *>(&k_lds[buf][tl * KROW + ld_chunk * 8]) = kr[ps];
                *reinterpret_cast<u32x4 *>(&v_lds[buf][tl * VROW + ld_chunk * 8]) = vr[ps];
            }
        }
    };

    // transposed-read lane address pieces (16-lane group gamma, lane rho in it)
    const int rho = lane & 15, gamma = lane >> 4;
    const int vt_row = 4 * (gamma >> 1) + (rho >> 2);                 // + 16 ks + 8 h
    const int vt_col = 16 * (gamma & 1) + 4 * (rho & 3);              // + 32 dt

    auto compute = [&](int tt, int buf) {
        f32x16 s;
#pragma unroll
        for (int i = 0; i < 16; ++i) s[i] = 0.f;
        const uint16_t *kl = &k_lds[buf][col * KROW + grp * 8];
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
            const u32x4 ka = *reinterpret_cast<const u32x4 *>(kl + kk * 16);
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ka),
                                                        __builtin_bit_cast(bf16x8, qf[kk]), s, 0, 0, 0);
        }
        // lane holds tokens (i/4)*8 + 4*grp + i%4 of this tile for query slot `col`;
        // only tiles reaching past the first row's causal limit (or the end
        // of the visible keys) need the mask.  With scale > 0 the max of the
        // raw scores gives the max of the scaled ones, and the scaling folds
        // into the exponent's FMA below.
        const int tbase = tt * kKvTile + 4 * grp;
        float mr = -INFINITY;
        if (tt * kKvTile + kKvTile - 1 > c + r0) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int t = tbase + (i >> 2) * 8 + (i & 3);
                s[i] = (t <= limit) ? s[i] : -INFINITY;
                mr = fmaxf(mr, s[i]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) mr = fmaxf(mr, s[i]);
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
        u32x4 pk[2];
        float ls = 0.f;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float a = fast_exp2(fmaf(s[8 * h + 2 * k], scale_log2, -msh));
                const float b = fast_exp2(fmaf(s[8 * h + 2 * k + 1], scale_log2, -msh));
                ls += a + b;
                pk[h][k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_pf{a, b}, bf16x2_pf));
            }
        }
        l_run += ls;
        const uint16_t *vl = &v_lds[buf][0];
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
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
    for (int d = 0; d <= DEPTH; ++d) load_regs(d, kreg[d], vreg[d]);
    store_lds(0, kreg[0], vreg[0]);
    __syncthreads();
    // One step: compute tile tt from LDS; tile tt+1 (ring slot u+1) goes to
    // the other LDS buffer; slot u is refilled with tile tt + DEPTH + 1.
    auto step = [&](int tt, auto uc) {
        constexpr int u = decltype(uc)::value;
        compute(tt, tt & 1);
        store_lds((tt + 1) & 1, kreg[(u + 1) % (DEPTH + 1)], vreg[(u + 1) % (DEPTH + 1)]);
        load_regs(tt + DEPTH + 1, kreg[u], vreg[u]);
        __syncthreads();
    };
    // Full groups of DEPTH + 1 steps have no guards, so the loop's back edge
    // always comes after the last slot's refill (the compiler's wait counts
    // for the ring stay exact); the remaining steps follow the loop.
    int t0 = 0;
    for (; t0 + DEPTH < ntiles; t0 += DEPTH + 1) {
        step(t0, std::integral_constant<int, 0>{});
        if constexpr (DEPTH >= 1) step(t0 + 1, std::integral_constant<int, 1>{});
        if constexpr (DEPTH >= 2) step(t0 + 2, std::integral_constant<int, 2>{});
        if constexpr (DEPTH >= 3) step(t0 + 3, std::integral_constant<int, 3>{});
    }
    if (t0 < ntiles) step(t0, std::integral_constant<int, 0>{});
    if constexpr (DEPTH >= 2) if (t0 + 1 < ntiles) step(t0 + 1, std::integral_constant<int, 1>{});
    if constexpr (DEPTH >= 3) if (t0 + 2 < ntiles) step(t0 + 2, std::integral_constant<int, 2>{});

    const float l_tot = sum_xor32_pf(l_run);
    if (q_ok) {
        const float inv = 1.f / l_tot;
        uint16_t *orow = out + ((long)(q0 + r0 + rq) * num_q_heads + kvh * G + hq) * D;
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
    }
}

namespace {
template <int D, int G>
hipError_t launch_prefill_dg(const PrefillArgs &a) {
    constexpr int R = kPfSlots / G;
    dim3 grid((a.max_q_len + R - 1) / R, a.num_kv_heads, a.num_seqs);
    dim3 block(kPfWaves * 64);
    hipLaunchKernelGGL((paged_prefill_kernel<D, G>), grid, block, 0, a.stream, a.q, a.k_cache,
                       a.v_cache, a.block_tables, a.seq_lens, a.cu_seqlens, a.num_q_heads,
                       a.num_kv_heads, a.max_blocks_per_seq, a.scale_log2, a.out);
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
