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
//   * a workgroup owns 128 (row, head) query slots of one kv head: R = 128 / G
//     consecutive rows times the G query heads that share the kv head (the
//     AstrAI page's GQA head packing), so every K/V tile is read once for all
//     G heads; wave w owns slots 32w .. 32w+31;
//   * KV is walked in 32-token tiles (two 16-token blocks) up to the last
//     row's causal limit; K is staged row-major and V transposed in LDS,
//     double buffered;
//   * S^T = K Q^T is v_mfma_f32_32x32x16_bf16 with K as the A operand and the
//     wave's query rows (kept in registers) as the B operand; the accumulator
//     gives each lane 16 tokens of one query slot, which is exactly the bf16
//     B operand layout of O^T += V^T P^T, so the probabilities never move
//     between lanes.  The V^T tile is stored with token bits 2 and 3 swapped so
//     that the A operand of that product is one 16-byte LDS read;
//   * online softmax per query slot with a lazy running max (rescale only when
//     a tile's max exceeds it by more than 2^8), fp32 accumulation.
#include "pa_common.h"
#include "pa_launch.h"

namespace pa {

namespace {
constexpr int kPfWaves = 4;
constexpr int kPfSlots = kPfWaves * 32;  // (row, head) query slots per workgroup
constexpr int kKvTile = 32;              // KV tokens per tile
constexpr float kPfTau = 8.0f;

// storage column of token t (0..31) in the V^T tile: swaps bits 2 and 3.
__device__ __forceinline__ int vt_pos(int t) { return (t & ~12) | ((t & 4) << 1) | ((t & 8) >> 1); }
}  // namespace

template <int D, int G>
__global__ __launch_bounds__(kPfWaves * 64) void paged_prefill_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k_cache,
    const uint16_t *__restrict__ v_cache, const int32_t *__restrict__ block_tables,
    const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ cu_seqlens,
    int num_q_heads, int num_kv_heads, int max_blocks_per_seq, float scale_log2,
    uint16_t *__restrict__ out) {
    constexpr int R = kPfSlots / G;        // query rows per workgroup
    constexpr int KROW = D + 8;            // bf16 per K row in LDS (padded)
    constexpr int VROW = kKvTile + 8;      // bf16 per V^T row in LDS (padded)
    constexpr int NK = D / 16;             // k-steps of S^T
    constexpr int ND = D / 32;             // 32-row tiles of O^T
    constexpr int CPT = D / 8;             // 16-byte chunks per token row
    constexpr int TPP = kPfWaves * 64 / CPT;  // tokens loaded per pass
    constexpr int PASSES = kKvTile / TPP;
    static_assert(kKvTile % TPP == 0, "tile load passes");
    __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][kKvTile * KROW];
    __shared__ __attribute__((aligned(16))) uint16_t v_lds[2][D * VROW];

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

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
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

    u32x4 kreg[PASSES], vreg[PASSES];
    auto load_regs = [&](int tt) {
#pragma unroll
        for (int ps = 0; ps < PASSES; ++ps) {
            const int t = tt * kKvTile + ps * TPP + ld_tok;
            if (t < L) {
                const long phys = bt_row[t >> 4];
                const long off = phys * blk_stride + kvh * tile_elems + (t & 15) * D + ld_chunk * 8;
                kreg[ps] = load_u32x4(k_cache + off);
                vreg[ps] = load_u32x4(v_cache + off);
            } else {
                kreg[ps] = u32x4{0u, 0u, 0u, 0u};
                vreg[ps] = u32x4{0u, 0u, 0u, 0u};
            }
        }
    };
    auto store_lds = [&](int buf) {
#pragma unroll
        for (int ps = 0; ps < PASSES; ++ps) {
            const int t = ps * TPP + ld_tok;
            *reinterpret_cast<u32x4 *>(&k_lds[buf][t * KROW + ld_chunk * 8]) = kreg[ps];
            const int pos = vt_pos(t);
            uint16_t *vt = &v_lds[buf][(ld_chunk * 8) * VROW + pos];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                vt[(2 * k) * VROW] = (uint16_t)(vreg[ps][k] & 0xffffu);
                vt[(2 * k + 1) * VROW] = (uint16_t)(vreg[ps][k] >> 16);
            }
        }
    };

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
        // lane holds tokens (i/4)*8 + 4*grp + i%4 of this tile for query slot `col`
        const int tbase = tt * kKvTile + 4 * grp;
        float bm = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int t = tbase + (i >> 2) * 8 + (i & 3);
            s[i] = (t <= limit) ? s[i] * scale_log2 : -INFINITY;
            bm = fmaxf(bm, s[i]);
        }
        bm = fmaxf(bm, xor_lane(bm, 32));
        const bool need = bm > m_run + kPfTau;
        if (__any(need)) {
            const float mn = fmaxf(m_run, bm);
            const float al = (mn == -INFINITY) ? 1.f : fast_exp2(m_run - mn);
            m_run = mn;
            l_run *= al;
#pragma unroll
            for (int dt = 0; dt < ND; ++dt)
#pragma unroll
                for (int i = 0; i < 16; ++i) o[dt][i] *= al;
        }
        u32x4 pk[2];
        float ls = 0.f;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float a = (m_run == -INFINITY) ? 0.f : fast_exp2(s[8 * h + 2 * k] - m_run);
                const float b = (m_run == -INFINITY) ? 0.f : fast_exp2(s[8 * h + 2 * k + 1] - m_run);
                ls += a + b;
                pk[h][k] = pack_bf16x2(a, b);
            }
        }
        l_run += ls;
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) {
            const uint16_t *vl = &v_lds[buf][(dt * 32 + col) * VROW + 8 * grp];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const u32x4 va = *reinterpret_cast<const u32x4 *>(vl + ks * 16);
                o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, va),
                                                                __builtin_bit_cast(bf16x8, pk[ks]), o[dt],
                                                                0, 0, 0);
            }
        }
    };

    load_regs(0);
    store_lds(0);
    __syncthreads();
    for (int tt = 0; tt < ntiles; ++tt) {
        const int buf = tt & 1;
        if (tt + 1 < ntiles) load_regs(tt + 1);
        compute(tt, buf);
        if (tt + 1 < ntiles) store_lds(buf ^ 1);
        __syncthreads();
    }

    const float l_tot = l_run + xor_lane(l_run, 32);
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
