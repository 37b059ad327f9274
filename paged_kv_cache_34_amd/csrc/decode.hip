// Paged GQA decode for gfx950 (CDNA4): split-KV partition kernel and the
// cross-partition merge kernel.
//
// What is computed (BI-V100 paged-attention design page, section 1 "Problem
// Definition"; block-table walk of the RL.cu "Add Cuda Kernel" page's paged
// decode kernel): for each sequence and query head, softmax(scale * q . K^T) V
// over the sequence's tokens, whose K/V rows live in 16-token physical blocks
// named by the block table.
//
// Work decomposition (the BI-V100 page's section 4 GQA grouping and section 6
// two-phase launch, re-designed for wave64 and MFMA):
//   * one workgroup per (partition, kv head, sequence); its 4 waves take the
//     partition's 16-token blocks round-robin, so one K/V load serves all G
//     query heads of the kv head;
//   * QK^T of a block is v_mfma_f32_16x16x32_bf16 with the G query rows as the
//     A operand and the block's K tile as the B operand, loaded straight from
//     HBM into the operand layout (lane: token = lane % 16, 16-byte chunk
//     4j + lane / 16), so no LDS staging is needed for K;
//   * the online softmax runs on the MFMA result (lane holds heads
//     4*(lane/16)+i of token lane%16): per-head block max with DPP row
//     reductions, a lazy running max (rescale only when a block's max exceeds
//     it by more than 2^8), exact max kept separately for the partial record;
//   * probabilities go through a per-wave LDS slot to the PV lanes; PV runs on
//     the VALU in a coalesced V layout (lane: 16-byte chunk lane % (D/8) of
//     token lane / (D/8) + j * 512/D), so each lane keeps only 8*G fp32
//     accumulators;
//   * at the end the waves are merged in LDS with the combine rule of the
//     BI-V100 page (section 2, "combine"), in a fixed order (deterministic).
// Every step depends only on logical token positions, so permuting physical
// blocks (with the table updated) gives bit-identical output.
#include "pa_common.h"
#include "pa_launch.h"

namespace pa {

constexpr int kBlock = 16;        // tokens per physical KV block
constexpr float kLazyTau = 8.0f;  // log2 headroom of the lazy running max

template <int D, int G, int NW>
struct DecodeShape {
    static constexpr int GP = (G + 3) / 4 * 4;   // head slots per token in LDS
    static constexpr int NJ = D / 32;            // MFMA k-steps = 16-byte loads per lane per tile
    static constexpr int LPT = D / 8;            // lanes per token row in the V layout
    static constexpr int TPI = 64 / LPT;         // tokens per V load instruction
    static constexpr int P_FLOATS = NW * (kBlock * GP + GP);
    static constexpr int RED_FLOATS = NW * G * D;
    static constexpr int MAIN_FLOATS = RED_FLOATS > P_FLOATS ? RED_FLOATS : P_FLOATS;
    static constexpr int STAT_FLOATS = 3 * NW * GP;
};

template <int D, int G, int NW>
__global__ __launch_bounds__(NW * 64) void paged_decode_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k_cache,
    const uint16_t *__restrict__ v_cache, const int32_t *__restrict__ block_tables,
    const int32_t *__restrict__ seq_lens, int num_q_heads, int num_kv_heads,
    int max_blocks_per_seq, float scale_log2, int partition_size, int max_num_partitions,
    uint16_t *__restrict__ out, float *__restrict__ max_logits, float *__restrict__ exp_sums,
    float *__restrict__ tmp_out) {
    using S = DecodeShape<D, G, NW>;
    constexpr int GP = S::GP, NJ = S::NJ, LPT = S::LPT, TPI = S::TPI;
    __shared__ __attribute__((aligned(16))) float lds[S::MAIN_FLOATS + S::STAT_FLOATS];

    const int part = blockIdx.x, kvh = blockIdx.y, seq = blockIdx.z;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int h0 = kvh * G;
    const int L = seq_lens[seq];
    const int t_begin = partition_size ? part * partition_size : 0;
    if (t_begin >= L) {
        if (partition_size == 0) {  // empty sequence, single pass: zeros
            uint16_t *o = out + ((long)seq * num_q_heads + h0) * D;
            for (int e = tid; e < G * D; e += NW * 64) o[e] = 0;
        }
        return;
    }
    const int t_end = partition_size ? min(L, t_begin + partition_size) : L;
    const int b_begin = t_begin / kBlock;
    const int nb = (t_end + kBlock - 1) / kBlock - b_begin;
    const int my_nb = nb > wave ? (nb - wave + NW - 1) / NW : 0;

    // S layout / MFMA operand lanes: r = token (B) or head row (A), cg = k group.
    const int r = lane & 15, cg = lane >> 4;
    // V layout lanes.
    const int vcol = lane % LPT, vrow = lane / LPT;

    u32x4 qa[NJ];
    {
        const uint16_t *qrow = q + ((long)seq * num_q_heads + h0 + (r < G ? r : 0)) * D;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            u32x4 v = load_u32x4(qrow + (4 * j + cg) * 8);
            qa[j] = (r < G) ? v : u32x4{0u, 0u, 0u, 0u};
        }
    }

    const long tile = (long)kBlock * D;
    const long blk_stride = (long)num_kv_heads * tile;
    const uint16_t *kbase = k_cache + kvh * tile + r * D + cg * 8;
    const uint16_t *vbase = v_cache + kvh * tile + vrow * D + vcol * 8;
    const int32_t *bt_row = block_tables + (long)seq * max_blocks_per_seq + b_begin + wave;

    int ids = (lane < my_nb) ? bt_row[NW * lane] : 0;

    float m_run[4], m_ex[4], l_run[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        m_run[i] = -INFINITY;
        m_ex[i] = -INFINITY;
        l_run[i] = 0.f;
    }
    float acc[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;

    float *p_lds = lds + wave * (kBlock * GP + GP);
    float *a_lds = p_lds + kBlock * GP;

    auto load_tile = [&](int i, u32x4 (&kr)[NJ], u32x4 (&vr)[NJ]) {
        if ((i & 63) == 0 && i > 0) ids = (lane + i < my_nb) ? bt_row[NW * (lane + i)] : 0;
        const long phys = __builtin_amdgcn_readlane(ids, i & 63);
        const uint16_t *kp = kbase + phys * blk_stride;
        const uint16_t *vp = vbase + phys * blk_stride;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            kr[j] = load_u32x4(kp + j * 32);
            vr[j] = load_u32x4(vp + j * TPI * D);
        }
    };

    auto compute_tile = [&](int i, const u32x4 (&kr)[NJ], const u32x4 (&vr)[NJ]) {
        const int tb = (b_begin + wave + NW * i) * kBlock;  // logical index of slot 0
        f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qa[j]),
                                                         __builtin_bit_cast(bf16x8, kr[j]), sc, 0, 0, 0);
        const bool tok_ok = tb + r < t_end;
        float z[4], bm[4];
        bool need = false;
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) {
            z[i2] = tok_ok ? sc[i2] * scale_log2 : -INFINITY;
            bm[i2] = row16_max(z[i2]);
            need |= bm[i2] > m_run[i2] + kLazyTau;
        }
        const bool rescale = __any(need);
        if (rescale) {
            float al[4];
#pragma unroll
            for (int i2 = 0; i2 < 4; ++i2) {
                const float mn = fmaxf(m_run[i2], bm[i2]);
                al[i2] = fast_exp2(m_run[i2] - mn);
                m_run[i2] = mn;
                l_run[i2] *= al[i2];
            }
            if (r == 0 && 4 * cg < GP)
                *reinterpret_cast<f32x4 *>(a_lds + 4 * cg) = f32x4{al[0], al[1], al[2], al[3]};
        }
        float p[4];
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) {
            m_ex[i2] = fmaxf(m_ex[i2], bm[i2]);
            p[i2] = fast_exp2(z[i2] - m_run[i2]);
            l_run[i2] += p[i2];
        }
        if (4 * cg < GP) *reinterpret_cast<f32x4 *>(p_lds + r * GP + 4 * cg) = f32x4{p[0], p[1], p[2], p[3]};
        wave_lds_sync();
        if (rescale) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float al = a_lds[h];
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] *= al;
            }
        }
        const bool tail = tb + kBlock > t_end;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int t = vrow + j * TPI;
            float pv[GP];
#pragma unroll
            for (int h4 = 0; h4 < GP; h4 += 4) {
                const f32x4 w = *reinterpret_cast<const f32x4 *>(p_lds + t * GP + h4);
                pv[h4] = w[0];
                pv[h4 + 1] = w[1];
                pv[h4 + 2] = w[2];
                pv[h4 + 3] = w[3];
            }
            float v[8];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                v[2 * k] = bf16_lo(vr[j][k]);
                v[2 * k + 1] = bf16_hi(vr[j][k]);
            }
            if (tail && tb + t >= t_end) {
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = 0.f;
            }
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(pv[h], v[e], acc[h][e]);
        }
        wave_lds_sync();
    };

    {
        u32x4 ka[NJ], va[NJ], kb[NJ], vb[NJ];
        if (my_nb > 0) load_tile(0, ka, va);
        for (int i = 0; i < my_nb; i += 2) {
            if (i + 1 < my_nb) load_tile(i + 1, kb, vb);
            compute_tile(i, ka, va);
            if (i + 2 < my_nb) load_tile(i + 2, ka, va);
            if (i + 1 < my_nb) compute_tile(i + 1, kb, vb);
        }
    }

    // ---- per-wave totals -------------------------------------------------
#pragma unroll
    for (int i2 = 0; i2 < 4; ++i2) l_run[i2] = row16_sum(l_run[i2]);
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float a = acc[h][e];
#pragma unroll
            for (int mask = LPT; mask < 64; mask <<= 1) a += xor_lane(a, mask);
            acc[h][e] = a;
        }

    __syncthreads();  // every wave is done with its p slot before the buffer is reused
    float *red = lds;                      // [NW][G][D]
    float *st_m = lds + S::MAIN_FLOATS;    // [NW][GP] running max (log2 units)
    float *st_x = st_m + NW * GP;          // [NW][GP] exact max (log2 units)
    float *st_l = st_x + NW * GP;          // [NW][GP] exp-sum relative to running max
    if (lane < LPT) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float *dst = red + (wave * G + h) * D + vcol * 8;
            *reinterpret_cast<f32x4 *>(dst) = f32x4{acc[h][0], acc[h][1], acc[h][2], acc[h][3]};
            *reinterpret_cast<f32x4 *>(dst + 4) = f32x4{acc[h][4], acc[h][5], acc[h][6], acc[h][7]};
        }
    }
    if (r == 0 && 4 * cg < GP) {
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) {
            st_m[wave * GP + 4 * cg + i2] = m_run[i2];
            st_x[wave * GP + 4 * cg + i2] = m_ex[i2];
            st_l[wave * GP + 4 * cg + i2] = l_run[i2];
        }
    }
    __syncthreads();

    // ---- merge the waves (fixed order) and write ---------------------------
    const long row0 = (long)seq * num_q_heads + h0;
    for (int e = tid; e < G * D; e += NW * 64) {
        const int h = e / D, d = e % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, st_m[w * GP + h]);
        float lsum = 0.f, o = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float f = fast_exp2(st_m[w * GP + h] - M);
            lsum = fmaf(f, st_l[w * GP + h], lsum);
            o = fmaf(f, red[(w * G + h) * D + d], o);
        }
        o = o / lsum;
        if (partition_size == 0)
            out[(row0 + h) * D + d] = (uint16_t)f32_to_bf16_bits(o);
        else
            tmp_out[((row0 + h) * max_num_partitions + part) * D + d] = o;
    }
    if (partition_size != 0 && tid < G) {
        const int h = tid;
        float M = -INFINITY, X = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            M = fmaxf(M, st_m[w * GP + h]);
            X = fmaxf(X, st_x[w * GP + h]);
        }
        float lsum = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) lsum = fmaf(fast_exp2(st_m[w * GP + h] - M), st_l[w * GP + h], lsum);
        max_logits[(row0 + h) * max_num_partitions + part] = X * kLn2;
        exp_sums[(row0 + h) * max_num_partitions + part] = lsum * fast_exp2(M - X);
    }
}

// Cross-partition merge: one workgroup per (query head, sequence).  Slots of
// D/4 lanes each take partitions round-robin with 16-byte loads; slot sums are
// folded in LDS in a fixed order.
template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void paged_reduce_kernel(
    const float *__restrict__ max_logits, const float *__restrict__ exp_sums,
    const float *__restrict__ tmp_out, const int32_t *__restrict__ seq_lens, int num_q_heads,
    int partition_size, int max_num_partitions, uint16_t *__restrict__ out) {
    constexpr int LPP = D / 4;
    constexpr int PPW = 64 / LPP;
    constexpr int SLOTS = NW * PPW;
    __shared__ __attribute__((aligned(16))) float red[SLOTS * D];
    __shared__ float wred[SLOTS];
    __shared__ float smax[NW];

    const int h = blockIdx.x, seq = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int L = seq_lens[seq];
    const int n = L > 0 ? (L + partition_size - 1) / partition_size : 0;
    const long row = (long)seq * num_q_heads + h;
    uint16_t *o = out + row * D;
    if (n == 0) {
        for (int d = tid; d < D; d += NW * 64) o[d] = 0;
        return;
    }
    const float *mlr = max_logits + row * max_num_partitions;
    const float *esr = exp_sums + row * max_num_partitions;

    float M = -INFINITY;
    for (int p = tid; p < n; p += NW * 64) M = fmaxf(M, mlr[p]);
    M = row16_max(M);
    M = fmaxf(M, xor_lane(M, 16));
    M = fmaxf(M, xor_lane(M, 32));
    if (lane == 0) smax[wave] = M;
    __syncthreads();
    M = smax[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, smax[w]);

    const int slot = tid / LPP, dl = tid % LPP;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float wsum = 0.f;
    const float *base = tmp_out + row * (long)max_num_partitions * D + dl * 4;
    for (int p = slot; p < n; p += SLOTS) {
        const float w = fast_exp2((mlr[p] - M) * kLog2e) * esr[p];
        const f32x4 v = *reinterpret_cast<const f32x4 *>(base + (long)p * D);
        acc[0] = fmaf(w, v[0], acc[0]);
        acc[1] = fmaf(w, v[1], acc[1]);
        acc[2] = fmaf(w, v[2], acc[2]);
        acc[3] = fmaf(w, v[3], acc[3]);
        wsum += w;
    }
    *reinterpret_cast<f32x4 *>(red + slot * D + dl * 4) = acc;
    if (dl == 0) wred[slot] = wsum;
    __syncthreads();
    for (int d = tid; d < D; d += NW * 64) {
        float a = 0.f, ws = 0.f;
#pragma unroll
        for (int sl = 0; sl < SLOTS; ++sl) {
            a += red[sl * D + d];
            ws += wred[sl];
        }
        o[d] = (uint16_t)f32_to_bf16_bits(a / ws);
    }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
namespace {
constexpr int kDecodeWaves = 4;
constexpr int kReduceWaves = 4;

template <int D, int G>
hipError_t launch_decode_dg(const DecodeArgs &a) {
    dim3 grid(a.num_partitions, a.num_kv_heads, a.num_seqs);
    dim3 block(kDecodeWaves * 64);
    hipLaunchKernelGGL((paged_decode_kernel<D, G, kDecodeWaves>), grid, block, 0, a.stream,
                       a.q, a.k_cache, a.v_cache, a.block_tables, a.seq_lens, a.num_q_heads,
                       a.num_kv_heads, a.max_blocks_per_seq, a.scale_log2, a.partition_size,
                       a.max_num_partitions, a.out, a.max_logits, a.exp_sums, a.tmp_out);
    return hipGetLastError();
}

template <int D>
hipError_t launch_decode_d(const DecodeArgs &a, int G) {
    switch (G) {
        case 1: return launch_decode_dg<D, 1>(a);
        case 2: return launch_decode_dg<D, 2>(a);
        case 3: return launch_decode_dg<D, 3>(a);
        case 4: return launch_decode_dg<D, 4>(a);
        case 5: return launch_decode_dg<D, 5>(a);
        case 6: return launch_decode_dg<D, 6>(a);
        case 7: return launch_decode_dg<D, 7>(a);
        case 8: return launch_decode_dg<D, 8>(a);
        case 9: return launch_decode_dg<D, 9>(a);
        case 10: return launch_decode_dg<D, 10>(a);
        case 11: return launch_decode_dg<D, 11>(a);
        case 12: return launch_decode_dg<D, 12>(a);
        case 13: return launch_decode_dg<D, 13>(a);
        case 14: return launch_decode_dg<D, 14>(a);
        case 15: return launch_decode_dg<D, 15>(a);
        case 16: return launch_decode_dg<D, 16>(a);
        default: return hipErrorInvalidValue;
    }
}

template <int D>
hipError_t launch_reduce_d(const ReduceArgs &a) {
    dim3 grid(a.num_q_heads, a.num_seqs);
    dim3 block(kReduceWaves * 64);
    hipLaunchKernelGGL((paged_reduce_kernel<D, kReduceWaves>), grid, block, 0, a.stream,
                       a.max_logits, a.exp_sums, a.tmp_out, a.seq_lens, a.num_q_heads,
                       a.partition_size, a.max_num_partitions, a.out);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_decode(const DecodeArgs &a) {
    const int G = a.num_q_heads / a.num_kv_heads;
    switch (a.head_dim) {
        case 64: return launch_decode_d<64>(a, G);
        case 128: return launch_decode_d<128>(a, G);
        case 256: return launch_decode_d<256>(a, G);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_reduce(const ReduceArgs &a) {
    switch (a.head_dim) {
        case 64: return launch_reduce_d<64>(a);
        case 128: return launch_reduce_d<128>(a);
        case 256: return launch_reduce_d<256>(a);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pa
