// Paged GQA decode kernels for gfx950 (CDNA4): the split-KV partition kernel
// (bf16 or FP8 KV cache) and the cross-partition merge kernels.
//
// What is computed (BI-V100 paged-attention design page, section 1 "Problem
// Definition"; block-table walk of the RL.cu "Add Cuda Kernel" page's paged
// decode kernel): for each sequence and query head, softmax(scale * q . K^T) V
// over the sequence's tokens, whose K/V rows live in 16-token physical blocks
// named by the block table.  With an FP8 cache (the B200 page, "Stage D: FP8
// Paged KV Gather"), K and V are OCP E4M3 codes with one dequant scale per
// (position, kv head), applied after the gather.
//
// Work decomposition (the BI-V100 page's section 4 GQA grouping and section 6
// two-phase launch, re-designed for wave64 and MFMA):
//   * a work item is (sequence, kv head, partition of P tokens), processed by
//     one workgroup of NW waves that take the partition's 16-token blocks
//     round-robin, so one K/V load serves all G query heads of the kv head;
//   * QK^T of a block is v_mfma_f32_16x16x32_bf16 with the block's K tile as
//     the A operand and the G query rows as the B operand; a row-major K tile
//     (bf16, or FP8 codes) is loaded in contiguous 1 KB runs of whole rows and
//     passes through the wave's LDS stage on its way into the operand layout
//     (an x-packed tile loads straight into it); the result S^T leaves lane l with the
//     scores of head l % 16 for 4 tokens;
//   * the online softmax runs on that layout: per-head block max over the 4
//     lane groups with permlane swaps, a lazy running max (rescale only when a
//     block's max exceeds it by more than 2^8), the exact max kept separately
//     for the partial record;
//   * PV is O^T += V^T P^T on v_mfma_f32_16x16x16_bf16: V^T comes from the
//     row-major V tile staged in LDS through transposed reads, P^T is the
//     lane's own probabilities;
//   * at the end the waves are merged in LDS with the combine rule of the
//     BI-V100 page (section 2, "combine"), in a fixed order (deterministic).
// Every step depends only on logical token positions, so permuting physical
// blocks (with the table updated) gives bit-identical output.
#pragma once

#include "pa_common.h"
#include "pa_launch.h"

namespace pa {

constexpr int kBlock = 16;        // tokens per physical KV block
constexpr float kLazyTau = 8.0f;  // log2 headroom of the lazy running max
// Fourth word of a raw buffer descriptor on the GFX9 family (32-bit data, no swizzle).
constexpr int kBufferFlags = 0x00020000;
// Cache policy of the K/V stream loads: nontemporal (the CDNA3/4 "nt" bit).
// Every cached byte is read once per decode step, so nothing is gained by
// keeping it in L2 or the Infinity Cache; measured on MI355X on the
// Llama-3-8B-shaped batch (three rotated pool copies), the step drops from
// 64.8 to 57.0 us with the bit set.
constexpr int kStreamPolicy = 2;

template <int D, int G, int NW>
struct DecodeShape {
    static_assert(D == 64 || D == 128 || D == 256, "head_dim");
    static_assert(G >= 1 && G <= 16, "GQA group");
    static constexpr int NJ = D / 32;            // K chunk loads per lane = S^T k-steps
    static constexpr int NDT = D / 16;           // 16-dim tiles of O^T
    static constexpr int LPT = D / 8;            // lanes per token row in the V layout
    static constexpr int TPI = 64 / LPT;         // tokens per V load instruction
    static constexpr int VROW = D + 16;          // bf16 per staged V row (32-byte pad)
    static constexpr int STAGE_FLOATS = NW * kBlock * VROW / 2;
    static constexpr int RED_FLOATS = NW * G * D;
    static constexpr int MAIN_FLOATS = RED_FLOATS > STAGE_FLOATS ? RED_FLOATS : STAGE_FLOATS;
    static constexpr int STAT_FLOATS = 3 * NW * 16;
};

// Kernel argument block (validated on the host).
struct DecodeParams {
    const uint16_t *q, *k_cache, *v_cache;
    const int32_t *block_tables, *seq_lens;
    int num_seqs, num_q_heads, num_kv_heads, max_blocks_per_seq;
    float scale_log2;
    int partition_size, max_num_partitions;
    uint16_t *out;
    float *max_logits, *exp_sums, *tmp_out;
    int *counters;  // fused merge: one arrival counter per (sequence, kv head); null = no merge
    // fused merge, stream-K schedule: the smallest unit (in 16-token tiles)
    // that keeps every (sequence, kv head) within max_num_partitions records
    int sk_min_tiles;
    // FP8 cache: dequant multipliers [num_blocks, H_kv, 16] (k_cache / v_cache
    // then hold E4M3 codes [num_blocks, H_kv, 16, D]); null for a bf16 cache
    const float *k_scales, *v_scales;
    // token-granular cache (page size 1): K/V [num_slots, H_kv, D], sequence
    // s's token t in slot block_tables[kv_indptr[s] + t] (block_tables then
    // holds the page indices); null for a block cache
    const int32_t *kv_indptr;
};

// Tokens of sequence `seq`: seq_lens, or adjacent kv_indptr entries.
__device__ __forceinline__ int seq_len_of(const DecodeParams &prm, int seq) {
    return prm.kv_indptr ? prm.kv_indptr[seq + 1] - prm.kv_indptr[seq] : prm.seq_lens[seq];
}

// Slot ids a wave stages in LDS per chunk of 64 tiles (token-granular cache).
constexpr int kTokIdsPerWave = 64 * 16;

// 16-byte words per lane of one ring slot: the K (or V) tile, plus, for an
// FP8 cache, the dequant scales of the lane's 4 score tokens.
template <int D, bool FP8>
struct KvWords {
    static constexpr int N = FP8 ? D / 64 + 1 : D / 32;
};

// Two E4M3 codes (bytes 0, 1 of w, or 2, 3 when HI) -> two bf16, exactly
// (every E4M3 value is a bf16 value).
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
// Eight E4M3 codes (two dwords) -> eight bf16 (an MFMA operand).
__device__ __forceinline__ u32x4 e4m3x8_to_bf16x8(uint32_t w0, uint32_t w1) {
    return u32x4{e4m3x2_to_bf16x2<false>(w0), e4m3x2_to_bf16x2<true>(w0), e4m3x2_to_bf16x2<false>(w1),
                 e4m3x2_to_bf16x2<true>(w1)};
}

__device__ __forceinline__ float max_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// One work item: partition `part` of kv head `kvh` of sequence `seq` (the whole
// sequence when partition_size == 0), processed by the NW waves of the
// calling workgroup; `lds` is the workgroup's scratch (DecodeShape floats).
//
// Per 16-token tile a wave computes, with the MFMA lane layouts
// (col = lane % 16, grp = lane / 16):
//   S^T = K Q^T   (v_mfma_f32_16x16x32_bf16; A = the K tile, lane: token
//                  col, 16-byte chunk 4j + grp, read from the wave's LDS stage
//                  (row-major) or loaded so (x-packed); B = the
//                  query rows) -> lane holds scores of head col for tokens
//                  4 grp + i;
//   online softmax per head (block max over the 4 lane groups with permlane
//   swaps, lazy running max);
//   O^T += V^T P^T (v_mfma_f32_16x16x16_bf16; A = V^T read from the staged
//                  row-major V tile with ds_read_b64_tr_b16, B = the lane's own
//                  probabilities, split into bf16 high and low parts so the
//                  product keeps ~16 mantissa bits) -> lane holds dims
//                  16 dt + 4 grp + i of head col.
// The probabilities never leave the lane that computed them, and V is never
// converted on the VALU.
// Partial-record element stores: plain, or agent-scope (coherent across the
// XCDs' L2 caches) when the fused merge of another workgroup will read them.
__device__ __forceinline__ void store_partial(float *p, float v, bool coherent) {
    if (coherent)
        __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
        *p = v;
}
__device__ __forceinline__ float load_partial(float *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A work item as one wave of the workgroup sees it: partition `part` of kv
// head `kvh` of sequence `seq` (the whole sequence when partition_size == 0;
// `L` = seq_lens[seq]).  The wave takes the item's 16-token blocks wave,
// wave + NW, ...; `ids` holds the block ids of its first 64 (one per lane).
struct DecodeItem {
    int seq, kvh, part, L;
    int t_end, b_begin, my_nb, ids;
    int nrec;  // records of the item's (sequence, kv head): its partitions, or its stream-K segments
};

// Token-granular cache, persistent launch: the 16 slot ids of the lane's tile
// of an item (tokens past the end: slot 0), held in registers until staged.
struct TokIds {
    u32x4 v[4];
};

template <int NW, bool TOK = false>
__device__ __forceinline__ DecodeItem make_item(const DecodeParams &prm, int seq, int kvh, int part,
                                                int L, int wave, int lane) {
    DecodeItem it;
    L = __builtin_amdgcn_readfirstlane(L);  // uniform (the compiler cannot see it when L comes from LDS)
    const int P = prm.partition_size;
    const int t_begin = P ? part * P : 0;
    it.seq = seq;
    it.kvh = kvh;
    it.part = part;
    it.L = L;
    it.t_end = P ? min(L, t_begin + P) : L;
    it.nrec = P ? (L + P - 1) / P : 1;
    it.b_begin = t_begin / kBlock;
    const int nb = (it.t_end + kBlock - 1) / kBlock - it.b_begin;
    it.my_nb = nb > wave ? (nb - wave + NW - 1) / NW : 0;
    const int32_t *bt_row = prm.block_tables + (long)seq * prm.max_blocks_per_seq + it.b_begin + wave;
    it.ids = (!TOK && lane < min(64, it.my_nb)) ? bt_row[NW * lane] : 0;  // (token ids: staged in LDS)
    return it;
}

// A stream-K segment: tiles [tile0, tile1) of kv head `kvh` of sequence
// `seq`, record `ord` of the pair's `nrec` (bf16 block cache only).
template <int NW>
__device__ __forceinline__ DecodeItem make_segment(const DecodeParams &prm, int seq, int kvh, int ord, int nrec,
                                                   int L, int tile0, int tile1, int wave, int lane) {
    DecodeItem it;
    L = __builtin_amdgcn_readfirstlane(L);
    it.seq = seq;
    it.kvh = kvh;
    it.part = ord;
    it.nrec = nrec;
    it.L = L;
    it.t_end = min(L, tile1 * kBlock);
    it.b_begin = tile0;
    const int nb = tile1 - tile0;
    it.my_nb = nb > wave ? (nb - wave + NW - 1) / NW : 0;
    const int32_t *bt_row = prm.block_tables + (long)seq * prm.max_blocks_per_seq + it.b_begin + wave;
    it.ids = lane < min(64, it.my_nb) ? bt_row[NW * lane] : 0;
    return it;
}

// Token-granular cache: the slot ids of the lane's tile of item `it`
// (sequence it.seq's indices start at kv_indptr[it.seq]).
template <int NW>
__device__ __forceinline__ TokIds load_item_ids(const DecodeParams &prm, const DecodeItem &it, int wave,
                                                int lane) {
    int v[kBlock];
    const bool mine = lane < min(64, it.my_nb);
    const int tok0 = (it.b_begin + wave + NW * lane) * kBlock;
    const int32_t *idx = prm.block_tables + (mine ? prm.kv_indptr[it.seq] : 0);
#pragma unroll
    for (int k = 0; k < kBlock; ++k) v[k] = (mine && tok0 + k < it.t_end) ? idx[tok0 + k] : 0;
    TokIds t;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        t.v[k] = u32x4{(uint32_t)v[4 * k], (uint32_t)v[4 * k + 1], (uint32_t)v[4 * k + 2], (uint32_t)v[4 * k + 3]};
    return t;
}

// ... and into the wave's LDS id region (tile `lane` at 16 * lane).
__device__ __forceinline__ void stage_item_ids(const DecodeItem &it, const TokIds &t, int *ids, int lane) {
    if (lane < min(64, it.my_nb)) {
#pragma unroll
        for (int k = 0; k < 4; ++k) *reinterpret_cast<u32x4 *>(ids + lane * kBlock + 4 * k) = t.v[k];
    }
    wave_lds_sync();
}

// Processes item `it` with the NW waves of the calling workgroup; `lds` is
// the workgroup's scratch (DecodeShape floats).  `qb` (the item's query rows)
// and the ring `kbuf`/`vbuf` (its first DEPTH tiles, tile j in slot j) are
// either loaded here (`primed` false) or were issued by the previous item.
// When `has_next`, the item issues the same for `nx` before its epilogue, so
// the next item's first loads are in flight while this one merges its waves.
// ONE_CHUNK: the caller guarantees at most 64 tiles per wave (NW * 1024
// tokens per item), so the block ids are never reloaded inside the item.
//
// Per 16-token tile a wave computes, with the MFMA lane layouts
// (col = lane % 16, grp = lane / 16):
//   S^T = K Q^T   (v_mfma_f32_16x16x32_bf16; A = the K tile, lane: token
//                  col, 16-byte chunk 4j + grp, read from the wave's LDS stage
//                  (row-major) or loaded so (x-packed); B = the
//                  query rows) -> lane holds scores of head col for tokens
//                  4 grp + i;
//   online softmax per head (block max over the 4 lane groups with permlane
//   swaps, lazy running max);
//   O^T += V^T P^T (v_mfma_f32_16x16x16_bf16; A = V^T read from the staged
//                  row-major V tile with ds_read_b64_tr_b16, B = the lane's own
//                  probabilities, split into bf16 high and low parts so the
//                  product keeps ~16 mantissa bits) -> lane holds dims
//                  16 dt + 4 grp + i of head col.
// Lanes with col >= G carry a copy of head 0; their results are never stored.
template <int D, int G, int NW, int DEPTH, bool ONE_CHUNK, bool FP8, bool XP, bool TOK = false>
__device__ __forceinline__ void decode_item(const DecodeParams &prm, const DecodeItem &it,
                                            const DecodeItem &nx, bool has_next, bool primed,
                                            u32x4 (&qb)[D / 32],
                                            u32x4 (&kbuf)[DEPTH + 1][KvWords<D, FP8>::N],
                                            u32x4 (&vbuf)[DEPTH + 1][KvWords<D, FP8>::N], float *lds,
                                            int *tok_lds = nullptr, int *tok_nx_lds = nullptr,
                                            const TokIds *nx_tk = nullptr) {
    using S = DecodeShape<D, G, NW>;
    static_assert(!(FP8 && XP), "the x-packed layout holds bf16");
    static_assert(!(TOK && (FP8 || XP)), "the token-granular cache holds bf16 rows");
    constexpr int NJ = S::NJ, NDT = S::NDT, VROW = S::VROW;
    constexpr int NW16 = KvWords<D, FP8>::N;      // words per ring slot
    // V tile loads: a token row is LPT lanes of 16 bytes (8 bf16 or 16 E4M3
    // codes); one load instruction covers TPI rows; NV loads per lane
    constexpr int LPT = FP8 ? D / 16 : D / 8, TPI = 64 / LPT, NV = kBlock / TPI;
    constexpr int NK = FP8 ? D / 64 : D / 32;     // K tile loads per lane
    constexpr int EB = FP8 ? 1 : 2;               // bytes per cached element
    const int num_q_heads = prm.num_q_heads;
    const int partition_size = prm.partition_size, max_num_partitions = prm.max_num_partitions;
    const float scale_log2 = prm.scale_log2;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    // (the item fields are wave-uniform; say so, since values carried around
    // the persistent loop may sit in vector registers)
    const int seq = __builtin_amdgcn_readfirstlane(it.seq), kvh = __builtin_amdgcn_readfirstlane(it.kvh);
    const int part = __builtin_amdgcn_readfirstlane(it.part);
    const int t_end = __builtin_amdgcn_readfirstlane(it.t_end);
    const int b_begin = __builtin_amdgcn_readfirstlane(it.b_begin);
    const int my_nb = __builtin_amdgcn_readfirstlane(it.my_nb);
    const int nx_kvh = __builtin_amdgcn_readfirstlane(nx.kvh);
    const int nx_nb = __builtin_amdgcn_readfirstlane(nx.my_nb);
    const int h0 = kvh * G;
    const int col = lane & 15, grp = lane >> 4;
    const int vcol = lane % LPT, vrow = lane / LPT;  // V load lane: 16-byte chunk vcol of row vrow

    // query rows as the B operand of S^T: lane holds q[head col][chunk 4j + grp]
    // (FP8: K step j = 2m + h holds dims 64m + 16 grp + 8h + 0..7, the order in
    // which one 16-byte load of 16 codes arrives; the dot product is the same)
    auto load_q = [&](int s, int g) {
        const uint16_t *qrow = prm.q + ((long)s * num_q_heads + g * G + (col < G ? col : 0)) * D;
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            qb[j] = load_u32x4(qrow + (FP8 ? 64 * (j >> 1) + 16 * grp + 8 * (j & 1) : (4 * j + grp) * 8));
    };

    const long tile = (long)kBlock * D * EB;       // bytes of one (block, kv head) tile
    const long blk_stride = (long)prm.num_kv_heads * tile;
    const char *kc = reinterpret_cast<const char *>(prm.k_cache);
    const char *vc = reinterpret_cast<const char *>(prm.v_cache);
    const char *kv_k = kc + kvh * tile, *kv_v = vc + kvh * tile;
    const char *nx_k = kc + nx_kvh * tile, *nx_v = vc + nx_kvh * tile;
    // bytes within a tile: K lane = (token col, chunk grp (+ 4j)); V lane = (row vrow, chunk vcol)
    // (x-packed K [D/8][16][8]: chunk 4j + grp of token col at ((4j + grp) * 16 + col) * 16 bytes;
    //  transposed V [D][16]: the PV A operand of dims 16 dt + col, tokens 4 grp + 0..3 is the
    //  8 bytes at (16 dt + col) * 32 + 8 grp)
    // A bf16 row-major K tile is loaded like V (each load instruction one
    // contiguous 1 KB run of whole token rows) and staged in LDS, from where
    // each lane reads its MFMA operand; loading the operand layout directly
    // would make every instruction touch 16 rows in 64-byte pieces, which
    // measured ~3% slower on MI355X.
    // (An FP8 tile likewise, its codes staged as bytes and converted after the
    // operand read.)
    constexpr bool KST = !XP && !TOK;
    const int v_voff = XP ? col * 32 + 8 * grp : (vrow * D * EB) + vcol * 16;
    const int k_voff = XP ? (grp * 16 + col) * 16 : v_voff;
    constexpr int K_STEP = 1024;  // bytes between a lane's K loads (one whole-row run each)
    // FP8 scales: [num_blocks, H_kv, 16] floats, the lane's 4 score tokens 4 grp + 0..3
    const float *ks_cur = FP8 ? prm.k_scales + kvh * kBlock : nullptr;
    const float *vs_cur = FP8 ? prm.v_scales + kvh * kBlock : nullptr;
    const float *ks_nx = FP8 ? prm.k_scales + nx_kvh * kBlock : nullptr;
    const float *vs_nx = FP8 ? prm.v_scales + nx_kvh * kBlock : nullptr;
    const long sc_stride = (long)prm.num_kv_heads * kBlock;
    const int32_t *bt_row = prm.block_tables + (long)seq * prm.max_blocks_per_seq + b_begin + wave;

    // per-wave V staging tile [16][VROW] bf16
    uint16_t *vstage = reinterpret_cast<uint16_t *>(lds) + wave * kBlock * VROW;
    uint16_t *vst_wr = vstage + vrow * VROW + vcol * (FP8 ? 16 : 8);
    const uint16_t *vst_rd = vstage + (4 * grp + (col >> 2)) * VROW + 4 * (col & 3);

    f32x4 oT[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) oT[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, m_ex = -INFINITY, l_run = 0.f;

    // Issues tile j of the current chunk (n tiles, block ids `ids` one per
    // lane) into a ring slot with buffer loads whose descriptor covers exactly
    // that tile.  In the item's last chunk the tiles past its end are the next
    // item's first tiles, counted from the first multiple of DEPTH + 1 at or
    // after n so that they land in ring slots 0, 1, ...; any other slot gets an
    // empty descriptor, whose loads return zeros without touching memory.  All
    // choices are wave-uniform and the loads unconditional, so the compiler's
    // wait counts stay exact.
    // Token-granular cache: per-lane row gathers.  The slot ids of the wave's
    // chunk sit in LDS (stage_tok_ids); tiles past the chunk read slot 0 (they
    // are prefetched but never computed), so every load stays in bounds.
    // (persistent launch: the caller staged this item's ids, and this item
    // stages the next one's into `nx_ids` before issuing its first tiles)
    int *my_ids = TOK ? tok_lds + wave * kTokIdsPerWave : nullptr;
    int *nx_ids = (TOK && ONE_CHUNK) ? tok_nx_lds + wave * kTokIdsPerWave : nullptr;
    auto load_rows = [&](const int *ids, int hk, bool cur, int j, u32x4 (&kr)[NW16], u32x4 (&vr)[NW16]) {
        const long row_stride = (long)prm.num_kv_heads * D;  // elements per slot
        const long sk = cur ? ids[j * kBlock + col] : 0;
        const uint16_t *kp = prm.k_cache + sk * row_stride + hk * D + (grp * 8);
#pragma unroll
        for (int j2 = 0; j2 < NK; ++j2)
            kr[j2] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(kp + j2 * 32));
#pragma unroll
        for (int j2 = 0; j2 < NV; ++j2) {
            const long sv = cur ? ids[j * kBlock + vrow + j2 * TPI] : 0;
            vr[j2] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4 *>(prm.v_cache + sv * row_stride + hk * D + vcol * 8));
        }
    };
    auto load_tile_tok = [&](int j, int n, u32x4 (&kr)[NW16], u32x4 (&vr)[NW16]) {
        load_rows(my_ids, kvh, j < n, j, kr, vr);
    };
    auto load_tile = [&](int ids, int j, int n, bool last, u32x4 (&kr)[NW16], u32x4 (&vr)[NW16]) {
        if constexpr (TOK) {
            load_tile_tok(j, n, kr, vr);
            return;
        }
        const int base = (n + DEPTH) / (DEPTH + 1) * (DEPTH + 1);
        const int jn = j - base;
        const bool cur = j < n;
        const bool nxt = !cur && last && has_next && jn >= 0 && jn < min(64, nx_nb);
        const long phys = cur ? __builtin_amdgcn_readlane(ids, j)
                              : __builtin_amdgcn_readlane(nx.ids, nxt ? jn : 0);
        const int bytes = (cur || nxt) ? (int)tile : 0;
        const auto krs = __builtin_amdgcn_make_buffer_rsrc((void *)((cur ? kv_k : nx_k) + phys * blk_stride),
                                                           0, bytes, kBufferFlags);
        const auto vrs = __builtin_amdgcn_make_buffer_rsrc((void *)((cur ? kv_v : nx_v) + phys * blk_stride),
                                                           0, bytes, kBufferFlags);
#pragma unroll
        for (int j2 = 0; j2 < NK; ++j2)
            kr[j2] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, k_voff + j2 * K_STEP, 0, kStreamPolicy));
        if constexpr (XP) {
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const auto w = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(vrs, v_voff + dt * 512, 0, kStreamPolicy));
                vr[dt >> 1][2 * (dt & 1)] = w[0];
                vr[dt >> 1][2 * (dt & 1) + 1] = w[1];
            }
        } else {
#pragma unroll
            for (int j2 = 0; j2 < NV; ++j2)
                vr[j2] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs, v_voff + j2 * TPI * D * EB, 0, kStreamPolicy));
        }
        if constexpr (FP8) {
            const int sbytes = (cur || nxt) ? kBlock * 4 : 0;
            const auto ksr = __builtin_amdgcn_make_buffer_rsrc((void *)((cur ? ks_cur : ks_nx) + phys * sc_stride),
                                                               0, sbytes, kBufferFlags);
            const auto vsr = __builtin_amdgcn_make_buffer_rsrc((void *)((cur ? vs_cur : vs_nx) + phys * sc_stride),
                                                               0, sbytes, kBufferFlags);
            kr[NK] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ksr, 16 * grp, 0, kStreamPolicy));
            vr[NV] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vsr, 16 * grp, 0, kStreamPolicy));
        }
    };

    auto compute_tile = [&](int i, const u32x4 (&kr)[NW16], const u32x4 (&vr)[NW16]) {
        const int tb = (b_begin + wave + NW * i) * kBlock;  // logical index of slot 0
        const bool tail = tb + kBlock > t_end;
        // K through the wave's stage first (row-major bf16): rows as loaded,
        // then the QK^T A operand (token col, 16-byte chunk 4j + grp); the
        // reads complete before V takes the stage over
        // (FP8: rows of D code bytes on the same 2 * VROW-byte pitch; lane reads
        // the 16 codes of dims 64 m + 16 grp + 0..15 of token col)
        u32x4 ks[KST ? NK : 1];
        if constexpr (KST) {
            unsigned char *kst = reinterpret_cast<unsigned char *>(vstage);
#pragma unroll
            for (int j = 0; j < NK; ++j)
                *reinterpret_cast<u32x4 *>(kst + (vrow + j * TPI) * (2 * VROW) + vcol * 16) = kr[j];
            wave_lds_sync();
#pragma unroll
            for (int j = 0; j < NK; ++j)
                ks[j] = *reinterpret_cast<const u32x4 *>(kst + col * (2 * VROW) + (FP8 ? 64 * j + 16 * grp : (4 * j + grp) * 16));
            wave_lds_sync();
        }
        // stage V as bf16 (FP8 codes converted exactly; token rows past the end
        // are zeroed so stale slots never reach PV); the x-packed layout's V
        // is already the PV operand
#pragma unroll
        for (int j = 0; j < (XP ? 0 : NV); ++j) {
            const bool dead = tail && tb + vrow + j * TPI >= t_end;
            if constexpr (FP8) {
                // every lane converts (a per-lane choice would put each
                // conversion under its own exec mask); only the sequence's
                // last tile, a wave-uniform case, masks its dead rows after
                const u32x4 w = vr[j];
                u32x4 lo = e4m3x8_to_bf16x8(w[0], w[1]);
                u32x4 hi = e4m3x8_to_bf16x8(w[2], w[3]);
                if (tail) {
                    const uint32_t keep = dead ? 0u : 0xffffffffu;
                    lo &= keep;
                    hi &= keep;
                }
                *reinterpret_cast<u32x4 *>(vst_wr + j * TPI * VROW) = lo;
                *reinterpret_cast<u32x4 *>(vst_wr + j * TPI * VROW + 8) = hi;
            } else {
                *reinterpret_cast<u32x4 *>(vst_wr + j * TPI * VROW) = dead ? u32x4{0u, 0u, 0u, 0u} : vr[j];
            }
        }
        f32x4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            u32x4 ka;
            if constexpr (FP8)
                ka = e4m3x8_to_bf16x8(ks[j >> 1][2 * (j & 1)], ks[j >> 1][2 * (j & 1) + 1]);
            else if constexpr (KST)
                ka = ks[j];
            else
                ka = kr[j];
            st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ka),
                                                         __builtin_bit_cast(bf16x8, qb[j]), st, 0, 0, 0);
        }
        float z[4];
        float bm = -INFINITY;
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) {
            // (FP8: the K dequant scale of the token multiplies its score)
            const float sk = FP8 ? __uint_as_float(kr[NK][i2]) * scale_log2 : scale_log2;
            z[i2] = (tb + 4 * grp + i2 < t_end) ? st[i2] * sk : -INFINITY;
            bm = fmaxf(bm, z[i2]);
        }
        bm = max_xor32(max_xor16(bm));
        if (__any(bm > m_run + kLazyTau)) {
            const float mn = fmaxf(m_run, bm);
            const float al = fast_exp2(m_run - mn);
            m_run = mn;
            l_run *= al;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) oT[dt] *= al;
        }
        m_ex = fmaxf(m_ex, bm);
        float p[4];
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) p[i2] = fast_exp2(z[i2] - m_run);
        l_run += (p[0] + p[1]) + (p[2] + p[3]);
        if constexpr (FP8) {
            // the V dequant scale of each token weights its probability in PV
            // (masked tokens: 0, whatever their unused scale slot holds)
#pragma unroll
            for (int i2 = 0; i2 < 4; ++i2)
                p[i2] = (tb + 4 * grp + i2 < t_end) ? p[i2] * __uint_as_float(vr[NV][i2]) : 0.f;
        }
        const uint32_t h01 = cvt_pk_bf16(p[0], p[1]), h23 = cvt_pk_bf16(p[2], p[3]);
        const uint32_t l01 = cvt_pk_bf16(p[0] - bf16_lo(h01), p[1] - bf16_hi(h01));
        const uint32_t l23 = cvt_pk_bf16(p[2] - bf16_lo(h23), p[3] - bf16_hi(h23));
        const s16x4 phi = __builtin_bit_cast(s16x4, u32x2{h01, h23});
        const s16x4 plo = __builtin_bit_cast(s16x4, u32x2{l01, l23});
        if constexpr (XP) {
            // the lane's 4 tokens of each V operand: zero those past the end
            uint32_t keep0 = 0xffffffffu, keep1 = 0xffffffffu;
            if (tail) {
                const int t0 = tb + 4 * grp;
                keep0 = (t0 < t_end ? 0x0000ffffu : 0u) | (t0 + 1 < t_end ? 0xffff0000u : 0u);
                keep1 = (t0 + 2 < t_end ? 0x0000ffffu : 0u) | (t0 + 3 < t_end ? 0xffff0000u : 0u);
            }
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const u32x2 w = {vr[dt >> 1][2 * (dt & 1)] & keep0, vr[dt >> 1][2 * (dt & 1) + 1] & keep1};
                const s16x4 a = __builtin_bit_cast(s16x4, w);
                oT[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, phi, oT[dt], 0, 0, 0);
                oT[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, plo, oT[dt], 0, 0, 0);
            }
        } else {
            wave_lds_sync();
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (s16x4 __attribute__((address_space(3))) *)(vst_rd + dt * 16));
                oT[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, phi, oT[dt], 0, 0, 0);
                oT[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, plo, oT[dt], 0, 0, 0);
            }
            wave_lds_sync();
        }
    };

    // token-granular cache: the slot ids of the wave's tiles c0 .. c0 + n - 1
    // (16 per tile; tokens past the end get slot 0) into the wave's LDS region
    auto stage_tok_ids = [&](int c0, int n) {
        if constexpr (TOK) {
            if (lane < n) {
                const int tok0 = (b_begin + wave + NW * (c0 + lane)) * kBlock;
                const int32_t *idx = prm.block_tables + prm.kv_indptr[seq];
#pragma unroll
                for (int k = 0; k < kBlock; ++k) my_ids[lane * kBlock + k] = (tok0 + k < t_end) ? idx[tok0 + k] : 0;
            }
            wave_lds_sync();
        }
    };
    if (TOK && !ONE_CHUNK) stage_tok_ids(0, min(64, my_nb));
    if (!primed) {
        load_q(seq, kvh);
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) load_tile(it.ids, d, min(64, my_nb), my_nb <= 64, kbuf[d], vbuf[d]);
    }

    // Tiles are processed in chunks of 64 whose block ids sit one per lane;
    // within a chunk a ring of DEPTH + 1 register tiles keeps tile i + DEPTH
    // in flight while tile i is consumed.
    auto run_chunk = [&](int ids, int c0, int n, bool last) {
        for (int i = 0; i < n; i += DEPTH + 1) {
#pragma unroll
            for (int u = 0; u <= DEPTH; ++u) {
                load_tile(ids, i + u + DEPTH, n, last, kbuf[(u + DEPTH) % (DEPTH + 1)],
                          vbuf[(u + DEPTH) % (DEPTH + 1)]);
                if (i + u < n) compute_tile(c0 + i + u, kbuf[u], vbuf[u]);
            }
        }
    };
    if (ONE_CHUNK) {
        run_chunk(it.ids, 0, my_nb, true);
    } else {
        for (int c0 = 0; c0 < my_nb; c0 += 64) {
            const int n = min(64, my_nb - c0);
            const bool last = c0 + 64 >= my_nb;
            const int ids = (TOK || c0 == 0) ? it.ids : ((lane < n) ? bt_row[NW * (c0 + lane)] : 0);
            if (c0 > 0) {
                if (TOK) stage_tok_ids(c0, n);
#pragma unroll
                for (int d = 0; d < DEPTH; ++d) load_tile(ids, d, n, last, kbuf[d], vbuf[d]);
            }
            run_chunk(ids, c0, n, last);
        }
    }
    if (has_next) {
        if constexpr (TOK) {
            // the next item's slot ids (loaded when this item began) into
            // its LDS region, then its first tiles
            stage_item_ids(nx, *nx_tk, nx_ids, lane);
            const int nn = min(64, nx_nb);
#pragma unroll
            for (int d = 0; d < DEPTH; ++d) load_rows(nx_ids, nx_kvh, d < nn, d, kbuf[d], vbuf[d]);
        } else if (my_nb == 0) {
            // a wave that streamed nothing has not issued the next item's tiles yet
#pragma unroll
            for (int d = 0; d < DEPTH; ++d) load_tile(0, d, 0, true, kbuf[d], vbuf[d]);
        }
        load_q(__builtin_amdgcn_readfirstlane(nx.seq), nx_kvh);
    }

    // ---- per-wave totals -------------------------------------------------
    // (the waves exchange partials through LDS only: LDS-only barriers keep
    // the next item's prefetched loads in flight; a full __syncthreads would
    // wait for them on every item)
    const bool fused = prm.counters != nullptr;
    auto wg_sync = [&]() { lds_barrier(); };
    l_run = sum_xor32(sum_xor16(l_run));
    wg_sync();  // every wave is done with its staging tile before the buffer is reused
    float *red = lds;                      // [NW][G][D]
    float *st_m = lds + S::MAIN_FLOATS;    // [NW][16] running max (log2 units)
    float *st_x = st_m + NW * 16;          // [NW][16] exact max (log2 units)
    float *st_l = st_x + NW * 16;          // [NW][16] exp-sum relative to running max
    if (col < G) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
            *reinterpret_cast<f32x4 *>(red + (wave * G + col) * D + 16 * dt + 4 * grp) = oT[dt];
        if (grp == 0) {
            st_m[wave * 16 + col] = m_run;
            st_x[wave * 16 + col] = m_ex;
            st_l[wave * 16 + col] = l_run;
        }
    }
    wg_sync();

    // ---- merge the waves (fixed order) and write ---------------------------
    // The item writes bf16 output directly when it is the whole sequence
    // (single pass, or the fused mode with one partition); otherwise its
    // partial record.
    const long row0 = (long)seq * num_q_heads + h0;
    const int nparts = __builtin_amdgcn_readfirstlane(it.nrec);
    const bool direct = partition_size == 0 || (fused && nparts == 1);
    for (int e = tid; e < G * D; e += NW * 64) {
        const int h = e / D, d = e % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, st_m[w * 16 + h]);
        float lsum = 0.f, o = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float f = fast_exp2(st_m[w * 16 + h] - M);
            lsum = fmaf(f, st_l[w * 16 + h], lsum);
            o = fmaf(f, red[(w * G + h) * D + d], o);
        }
        o = o / lsum;
        if (direct)
            prm.out[(row0 + h) * D + d] = (uint16_t)f32_to_bf16_bits(o);
        else
            store_partial(prm.tmp_out + ((row0 + h) * max_num_partitions + part) * D + d, o, fused);
    }
    if (!direct && tid < G) {
        const int h = tid;
        float M = -INFINITY, X = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            M = fmaxf(M, st_m[w * 16 + h]);
            X = fmaxf(X, st_x[w * 16 + h]);
        }
        float lsum = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) lsum = fmaf(fast_exp2(st_m[w * 16 + h] - M), st_l[w * 16 + h], lsum);
        store_partial(prm.max_logits + (row0 + h) * max_num_partitions + part, X * kLn2, fused);
        store_partial(prm.exp_sums + (row0 + h) * max_num_partitions + part, lsum * fast_exp2(M - X), fused);
    }
    if (!direct && fused) {
        // Fused cross-partition merge (the BI-V100 page, section 2 "Level 3":
        // the merge may instead run in whichever partition block finishes
        // last): publish the partial device-wide, count arrivals of the
        // (sequence, kv head) records, and let the workgroup that completes
        // the set merge them in record order.
        // Ordering, as the gfx950 ISA provides it: the records are written
        // with agent-scope atomic stores (device-coherent: they bypass the
        // per-XCD L2 caches), each wave waits until its stores are
        // acknowledged (s_waitcnt 0, also a compiler barrier), the workgroup
        // barrier then orders every wave's acknowledged stores before thread
        // 0's arrival on the counter, and the last arrival reads the records
        // with agent-scope atomic loads, which are served device-coherently.
        // The same edge written as a C++-model release on the arrival and an
        // acquire fence in the merging workgroup makes the compiler write
        // back and invalidate the whole L2 of the XCD at each one: measured
        // on MI355X on the Llama-3-8B-shaped batch, 62.7 us per step become
        // 95-99 us with the release (66 us with the acquire fence alone).
        __builtin_amdgcn_s_waitcnt(0);
        asm volatile("" ::: "memory");
        __syncthreads();
        int *flag = reinterpret_cast<int *>(st_m);
        if (tid == 0) {
            const int old = __hip_atomic_fetch_add(prm.counters + (long)seq * prm.num_kv_heads + kvh, 1,
                                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            flag[0] = (old == nparts - 1);
        }
        lds_barrier();  // the verdict travels through LDS
        if (flag[0]) {
            // The merge runs over (column, slot) pairs: a column is 4
            // consecutive dims of one head; a column's SL slots take the
            // partitions round-robin, 4 at a time with every load issued
            // before any is used, each slot keeping a running max; then the
            // slots are folded in LDS in slot order (deterministic).
            constexpr int T = NW * 64;
            constexpr int COLS = G * D / 4;
            constexpr int SL = T / COLS >= 1 ? T / COLS : 1;
            constexpr int MU = 4;
            float *fold = lds;  // [SL][COLS][6]: max, weight sum, 4 accumulators
            static_assert(SL * COLS * 6 <= S::MAIN_FLOATS, "merge fold fits the scratch");
            for (int pr = tid; pr < COLS * SL; pr += T) {
                const int c = pr % COLS, sl = pr / COLS;
                const int h = c / (D / 4), d0 = 4 * (c % (D / 4));
                float *mlr = prm.max_logits + (row0 + h) * max_num_partitions;
                float *esr = prm.exp_sums + (row0 + h) * max_num_partitions;
                float *tor = prm.tmp_out + (row0 + h) * max_num_partitions * (long)D + d0;
                float m = -INFINITY, wsum = 0.f;
                float acc[4] = {0.f, 0.f, 0.f, 0.f};
                for (int p0 = sl; p0 < nparts; p0 += SL * MU) {
                    float mp[MU], lp[MU], op[MU][4];
#pragma unroll
                    for (int u = 0; u < MU; ++u) {
                        const int p = p0 + u * SL;
                        const bool ok = p < nparts;
                        mp[u] = ok ? load_partial(mlr + p) : -INFINITY;
                        lp[u] = ok ? load_partial(esr + p) : 0.f;
#pragma unroll
                        for (int k = 0; k < 4; ++k) op[u][k] = ok ? load_partial(tor + (long)p * D + k) : 0.f;
                    }
#pragma unroll
                    for (int u = 0; u < MU; ++u) {
                        if (p0 + u * SL >= nparts) continue;
                        if (mp[u] > m) {
                            const float f = fast_exp2((m - mp[u]) * kLog2e);
                            wsum *= f;
#pragma unroll
                            for (int k = 0; k < 4; ++k) acc[k] *= f;
                            m = mp[u];
                        }
                        const float w = fast_exp2((mp[u] - m) * kLog2e) * lp[u];
                        wsum += w;
#pragma unroll
                        for (int k = 0; k < 4; ++k) acc[k] = fmaf(w, op[u][k], acc[k]);
                    }
                }
                float *f6 = fold + (sl * COLS + c) * 6;
                f6[0] = m;
                f6[1] = wsum;
#pragma unroll
                for (int k = 0; k < 4; ++k) f6[2 + k] = acc[k];
            }
            lds_barrier();
            for (int c = tid; c < COLS; c += T) {
                const int h = c / (D / 4), d0 = 4 * (c % (D / 4));
                float M = -INFINITY;
#pragma unroll
                for (int sl = 0; sl < SL; ++sl) M = fmaxf(M, fold[(sl * COLS + c) * 6]);
                float ws = 0.f, a[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int sl = 0; sl < SL; ++sl) {
                    const float *f6 = fold + (sl * COLS + c) * 6;
                    const float f = f6[1] > 0.f ? fast_exp2((f6[0] - M) * kLog2e) : 0.f;
                    ws = fmaf(f, f6[1], ws);
#pragma unroll
                    for (int k = 0; k < 4; ++k) a[k] = fmaf(f, f6[2 + k], a[k]);
                }
                const float inv = 1.f / ws;
                u32x2 wv;
                wv[0] = pack_bf16x2(a[0] * inv, a[1] * inv);
                wv[1] = pack_bf16x2(a[2] * inv, a[3] * inv);
                *reinterpret_cast<u32x2 *>(prm.out + (row0 + h) * D + d0) = wv;
            }
            if (tid == 0)
                __hip_atomic_store(prm.counters + (long)seq * prm.num_kv_heads + kvh, 0, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    wg_sync();  // the next item of a persistent workgroup reuses `lds`
}

// One workgroup per (partition, kv head, sequence); workgroups whose partition
// starts past the sequence end exit at once.
template <int D, int G, int NW, int DEPTH, bool FP8, bool XP, bool TOK = false>
__global__ __launch_bounds__(NW * 64) void paged_decode_grid_kernel(DecodeParams prm) {
    using S = DecodeShape<D, G, NW>;
    __shared__ __attribute__((aligned(16))) float lds[S::MAIN_FLOATS + S::STAT_FLOATS];
    __shared__ __attribute__((aligned(16))) int tok_ids[TOK ? NW * kTokIdsPerWave : 1];
    const int seq = blockIdx.z, kvh = blockIdx.y, part = blockIdx.x;
    const int L = seq_len_of(prm, seq);
    const int P = prm.partition_size;
    if ((P ? part * P : 0) >= L) {
        // An empty sequence has no partition to write its output: in the
        // single pass, and in the fused merge (which writes `out` itself),
        // the first partition slot of each kv head writes its zero rows.
        if (P == 0 || (prm.counters && L <= 0 && part == 0)) {
            uint16_t *o = prm.out + ((long)seq * prm.num_q_heads + kvh * G) * D;
            for (int e = threadIdx.x; e < G * D; e += NW * 64) o[e] = 0;
        }
        return;
    }
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const DecodeItem it = make_item<NW, TOK>(prm, seq, kvh, part, L, wave, threadIdx.x & 63);
    u32x4 qb[D / 32], kbuf[DEPTH + 1][KvWords<D, FP8>::N], vbuf[DEPTH + 1][KvWords<D, FP8>::N];
    decode_item<D, G, NW, DEPTH, false, FP8, XP, TOK>(prm, it, it, false, false, qb, kbuf, vbuf, lds, tok_ids);
}

// Compact persistent split-KV.  Every workgroup first builds, in LDS, two
// prefixes over sequences: of their full partitions (H_kv * floor(L / P)
// items) and of their short last partitions (H_kv items when P does not
// divide L).  Items are numbered full partitions first (sequence, kv head,
// partition), then the short ones (sequence, kv head), so the last round of
// the schedule holds the smallest items.  Workgroup w takes items w,
// w + active, w + 2 active, ...  With `total` items over a grid of gridDim.x
// workgroups the busiest ones take k = ceil(total / gridDim.x) items; when
// ceil(total / k) workgroups (all holding k or k - 1 items) still fill at
// least seven eighths of the grid, only those take part, so that no
// workgroup runs a last item alone while the rest of the GPU idles;
// otherwise all gridDim.x do.  Only partitions that exist are visited.  Each
// item issues the next one's query rows and first K/V tiles before its
// epilogue.
constexpr int kCompactMaxSeqs = 1024;

// Zero output rows for the zero-length sequences (lengths staged in LDS):
// sequence s by workgroup s mod grid.
template <int D>
__device__ __forceinline__ void write_empty_rows(const DecodeParams &prm, const int *lens) {
    const int T = blockDim.x, row = prm.num_q_heads * D;
    for (int s = blockIdx.x; s < prm.num_seqs; s += gridDim.x) {
        if (lens[s] > 0) continue;
        uint16_t *o = prm.out + (long)s * row;
        for (int e = threadIdx.x; e < row; e += T) o[e] = 0;
    }
}

template <int D, int G, int NW, int DEPTH, bool FP8, bool XP, bool TOK = false>
__global__ __launch_bounds__(NW * 64) void paged_decode_compact_kernel(DecodeParams prm) {
    using S = DecodeShape<D, G, NW>;
    constexpr int T = NW * 64;
    constexpr int PER = (kCompactMaxSeqs + T - 1) / T;
    __shared__ __attribute__((aligned(16))) float lds[S::MAIN_FLOATS + S::STAT_FLOATS];
    // token-granular cache: two id regions per wave (this item, the next)
    __shared__ __attribute__((aligned(16))) int tok_ids[TOK ? 2 * NW * kTokIdsPerWave : 1];
    __shared__ int fpref[kCompactMaxSeqs + 1];  // full-partition items before sequence s
    __shared__ int tpref[kCompactMaxSeqs + 1];  // short-partition items before sequence s
    __shared__ int lens[kCompactMaxSeqs];
    __shared__ int wtot[2][NW];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nseq = prm.num_seqs, P = prm.partition_size, hkv = prm.num_kv_heads;

    int cf[PER], ct[PER];
    int lf = 0, lt = 0;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int i = tid * PER + k;
        int f = 0, t = 0;
        if (i < nseq) {
            const int L = TOK ? prm.kv_indptr[i + 1] - prm.kv_indptr[i] : prm.seq_lens[i];
            if (L > 0) {
                f = hkv * (L / P);
                t = (L % P) ? hkv : 0;
            }
            lens[i] = L;
        }
        cf[k] = f;
        ct[k] = t;
        lf += f;
        lt += t;
    }
    int inf = lf, intl = lt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int yf = __shfl_up(inf, d), yt = __shfl_up(intl, d);
        if (lane >= d) {
            inf += yf;
            intl += yt;
        }
    }
    if (lane == 63) {
        wtot[0][wave] = inf;
        wtot[1][wave] = intl;
    }
    __syncthreads();
    int runf = inf - lf, runt = intl - lt;
    for (int w = 0; w < wave; ++w) {
        runf += wtot[0][w];
        runt += wtot[1][w];
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int i = tid * PER + k;
        runf += cf[k];
        runt += ct[k];
        if (i < nseq) {
            fpref[i + 1] = runf;
            tpref[i + 1] = runt;
        }
    }
    if (tid == 0) {
        fpref[0] = 0;
        tpref[0] = 0;
    }
    __syncthreads();

    const int nfull = __builtin_amdgcn_readfirstlane(fpref[nseq]);
    const int total = nfull + __builtin_amdgcn_readfirstlane(tpref[nseq]);  // uniform loop bound
    const int per_wg = (total + (int)gridDim.x - 1) / (int)gridDim.x;
    // (measured on MI355X: worth it when it idles at most an eighth of the
    // grid; below that, the lost memory parallelism costs more than the
    // last round's imbalance)
    const int balanced = per_wg > 0 ? (total + per_wg - 1) / per_wg : 0;
    const int active = 8 * balanced >= 7 * (int)gridDim.x ? balanced : min(total, (int)gridDim.x);
    // item -> (sequence, kv head, partition): the largest s with pref[s] <=
    // item (a sequence that has items of that kind), then the rest within it
    auto search = [&](const int *pref, int item) {
        int lo = 0, hi = nseq;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (pref[mid] <= item) lo = mid; else hi = mid;
        }
        return __builtin_amdgcn_readfirstlane(lo);
    };
    auto locate = [&](int item) {
        int seq, kvh, part;
        if (item < nfull) {
            seq = search(fpref, item);
            const int nf = (fpref[seq + 1] - fpref[seq]) / hkv;
            const int rr = item - fpref[seq];
            kvh = rr / nf;
            part = rr % nf;
        } else {
            const int r = item - nfull;
            seq = search(tpref, r);
            kvh = r - tpref[seq];
            part = lens[seq] / P;
        }
        return make_item<NW, TOK>(prm, seq, __builtin_amdgcn_readfirstlane(kvh),
                                  __builtin_amdgcn_readfirstlane(part), lens[seq], wave, lane);
    };
    // the fused merge writes `out` itself: zero-length sequences, which have
    // no items, get zero rows here (a workgroup per sequence, round-robin)
    if (prm.counters) write_empty_rows<D>(prm, lens);
    int item = blockIdx.x;
    if (item >= active) return;
    DecodeItem it = locate(item);
    // Settle the first item's block-id load here: the wait the compiler would
    // otherwise place at the top of the item loop (where it would also drain
    // the prefetched loads of every later item) becomes a no-op.
    __builtin_amdgcn_s_waitcnt(0);
    int buf = 0;  // token-granular cache: the id region of the current item
    if constexpr (TOK) stage_item_ids(it, load_item_ids<NW>(prm, it, wave, lane), tok_ids + wave * kTokIdsPerWave, lane);
    u32x4 qb[D / 32], kbuf[DEPTH + 1][KvWords<D, FP8>::N], vbuf[DEPTH + 1][KvWords<D, FP8>::N];
    bool primed = false;
    for (;;) {
        // the next item's block (or slot) ids are fetched while this one streams
        const int next = item + active;
        const bool has_next = next < total;
        const DecodeItem nx = has_next ? locate(next) : it;
        TokIds nx_tk;
        if constexpr (TOK) {
            if (has_next) nx_tk = load_item_ids<NW>(prm, nx, wave, lane);
        }
        decode_item<D, G, NW, DEPTH, true, FP8, XP, TOK>(prm, it, nx, has_next, primed, qb, kbuf, vbuf, lds,
                                                         tok_ids + buf * NW * kTokIdsPerWave,
                                                         tok_ids + (buf ^ 1) * NW * kTokIdsPerWave, &nx_tk);
        if (!has_next) break;
        item = next;
        it = nx;
        primed = true;
        buf ^= 1;
    }
}

// Fused merge, stream-K schedule (bf16 block cache): the tiles of all
// (sequence, kv head) pairs laid end to end, pair-major in (sequence, kv head)
// order, are cut into equal units of at most NW * 64 tiles (one block-id
// chunk per wave) and workgroup w takes k consecutive units, so every
// workgroup streams the same number of tiles however the lengths are spread.
// A unit's part of one pair is a segment, processed as one item; its record
// goes to slot (unit - first unit of the pair) of the pair's records, and the
// workgroup completing a pair's records merges them in slot order (the fused
// epilogue of decode_item).  `sk_min_tiles` (host) bounds the records per
// pair by max_num_partitions: a pair of nt <= max_blocks_per_seq tiles meets
// at most ceil(nt / unit) + 1 units.
template <int D, int G, int NW, int DEPTH>
__global__ __launch_bounds__(NW * 64) void paged_decode_streamk_kernel(DecodeParams prm) {
    using S = DecodeShape<D, G, NW>;
    constexpr int T = NW * 64;
    constexpr int PER = (kCompactMaxSeqs + T - 1) / T;
    constexpr long kUnitMax = NW * 64;
    __shared__ __attribute__((aligned(16))) float lds[S::MAIN_FLOATS + S::STAT_FLOATS];
    __shared__ int tp[kCompactMaxSeqs + 1];  // tiles of one kv head of the sequences before s
    __shared__ int lens[kCompactMaxSeqs];
    __shared__ int wtot[NW];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nseq = prm.num_seqs, hkv = prm.num_kv_heads;

    int ct[PER];
    int lt = 0;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int i = tid * PER + k;
        int nt = 0;
        if (i < nseq) {
            const int L = prm.seq_lens[i];
            nt = L > 0 ? (L + kBlock - 1) / kBlock : 0;
            lens[i] = L;
        }
        ct[k] = nt;
        lt += nt;
    }
    int incl = lt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(incl, d);
        if (lane >= d) incl += y;
    }
    if (lane == 63) wtot[wave] = incl;
    __syncthreads();
    int run = incl - lt;
    for (int w = 0; w < wave; ++w) run += wtot[w];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int i = tid * PER + k;
        run += ct[k];
        if (i < nseq) tp[i + 1] = run;
    }
    if (tid == 0) tp[0] = 0;
    __syncthreads();
    write_empty_rows<D>(prm, lens);

    const long total = (long)__builtin_amdgcn_readfirstlane(tp[nseq]) * hkv;
    const long grid = gridDim.x;
    const long per = (total + grid - 1) / grid;
    const long k = (per + kUnitMax - 1) / kUnitMax;  // units per workgroup
    long unit = k > 0 ? (total + grid * k - 1) / (grid * k) : 1;
    if (unit < prm.sk_min_tiles) unit = prm.sk_min_tiles;
    const long x0 = (long)blockIdx.x * k * unit;
    const long xe = min(total, x0 + k * unit);
    if (x0 >= xe) return;

    // the segment starting at tile x of the global order, and where it ends
    auto segment = [&](long x, long &end) {
        int lo = 0, hi = nseq;  // the largest s with tp[s] * hkv <= x (a sequence with tiles, as x < total)
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if ((long)tp[mid] * hkv <= x) lo = mid; else hi = mid;
        }
        const int seq = __builtin_amdgcn_readfirstlane(lo);
        const int nt = tp[seq + 1] - tp[seq];
        const long base = (long)tp[seq] * hkv;
        const int kvh = __builtin_amdgcn_readfirstlane((int)((x - base) / nt));
        const long ps = base + (long)kvh * nt, pe = ps + nt;
        const long u = x / unit;
        end = min(pe, (u + 1) * unit);
        const int ord = __builtin_amdgcn_readfirstlane((int)(u - ps / unit));
        const int nrec = __builtin_amdgcn_readfirstlane((int)((pe - 1) / unit - ps / unit + 1));
        return make_segment<NW>(prm, seq, kvh, ord, nrec, lens[seq], (int)(x - ps), (int)(end - ps), wave, lane);
    };
    long x_end;
    DecodeItem it = segment(x0, x_end);
    __builtin_amdgcn_s_waitcnt(0);
    u32x4 qb[D / 32], kbuf[DEPTH + 1][KvWords<D, false>::N], vbuf[DEPTH + 1][KvWords<D, false>::N];
    bool primed = false;
    for (;;) {
        const bool has_next = x_end < xe;
        long nx_end = x_end;
        DecodeItem nx = it;
        if (has_next) nx = segment(x_end, nx_end);
        decode_item<D, G, NW, DEPTH, true, false, false>(prm, it, nx, has_next, primed, qb, kbuf, vbuf, lds);
        if (!has_next) break;
        it = nx;
        x_end = nx_end;
        primed = true;
    }
}

// Cross-partition merge (the BI-V100 page's combine rule): one workgroup per
// (64-dim chunk, query head, sequence).  Its 16 slots of 16 lanes (4 dims per
// lane) take partitions round-robin, 4 at a time, each slot keeping a running
// max so that a single pass suffices; the slots are then folded in LDS in a
// fixed order (deterministic).
constexpr int kReduceChunk = 64;   // dims per workgroup
constexpr int kReduceUnroll = 4;   // partitions in flight per slot

template <int NW>
__global__ __launch_bounds__(NW * 64) void paged_reduce_kernel(
    const float *__restrict__ max_logits, const float *__restrict__ exp_sums,
    const float *__restrict__ tmp_out, const int32_t *__restrict__ seq_lens,
    const int32_t *__restrict__ kv_indptr, int num_q_heads, int head_dim, int partition_size,
    int max_num_partitions, uint16_t *__restrict__ out) {
    constexpr int LPP = kReduceChunk / 4;  // lanes per partition row
    constexpr int SLOTS = NW * 64 / LPP;
    __shared__ __attribute__((aligned(16))) float red[SLOTS * kReduceChunk];
    __shared__ float sm[SLOTS], sw[SLOTS];

    const int chunk = blockIdx.x, h = blockIdx.y, seq = blockIdx.z;
    const int tid = threadIdx.x;
    const long row = (long)seq * num_q_heads + h;
    const float *mlr = max_logits + row * max_num_partitions;
    const float *esr = exp_sums + row * max_num_partitions;
    const int slot = tid / LPP, dl = tid % LPP;
    const float *base = tmp_out + row * (long)max_num_partitions * head_dim + chunk * kReduceChunk + dl * 4;
    // When the partial buffers hold at most one record per slot, the first
    // round is loaded before the sequence length is known (records past the
    // sequence's partitions are discarded by selection, never used in
    // arithmetic), which takes one dependent memory round trip off the
    // kernel.  With more partition slots than that, most of them are unused
    // for short sequences, so the length comes first and only existing
    // partitions are read.
    const bool speculate = max_num_partitions <= SLOTS;
    int n = 0;
    if (!speculate) {
        const int L = kv_indptr ? kv_indptr[seq + 1] - kv_indptr[seq] : seq_lens[seq];
        n = L > 0 ? (L + partition_size - 1) / partition_size : 0;
    }
    const int first_bound = speculate ? max_num_partitions : n;
    float mv[kReduceUnroll], ev[kReduceUnroll];
    f32x4 v[kReduceUnroll];
#pragma unroll
    for (int u = 0; u < kReduceUnroll; ++u) {
        const int p = slot + u * SLOTS;
        const bool in = p < first_bound;
        mv[u] = in ? mlr[p] : -INFINITY;
        ev[u] = in ? esr[p] : 0.f;
        v[u] = in ? *reinterpret_cast<const f32x4 *>(base + (long)p * head_dim) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (speculate) {
        const int L = kv_indptr ? kv_indptr[seq + 1] - kv_indptr[seq] : seq_lens[seq];
        n = L > 0 ? (L + partition_size - 1) / partition_size : 0;
    }
    uint16_t *o = out + row * head_dim + chunk * kReduceChunk;
    if (n == 0) {
        for (int d = tid; d < kReduceChunk; d += NW * 64) o[d] = 0;
        return;
    }

    float m = -INFINITY, wsum = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int p0 = slot;; p0 += SLOTS * kReduceUnroll) {
#pragma unroll
        for (int u = 0; u < kReduceUnroll; ++u) {
            if (p0 + u * SLOTS >= n) continue;
            if (mv[u] > m) {  // rescale what was accumulated to the new max
                const float f = fast_exp2((m - mv[u]) * kLog2e);
                acc *= f;
                wsum *= f;
                m = mv[u];
            }
            const float w = fast_exp2((mv[u] - m) * kLog2e) * ev[u];
            acc[0] = fmaf(w, v[u][0], acc[0]);
            acc[1] = fmaf(w, v[u][1], acc[1]);
            acc[2] = fmaf(w, v[u][2], acc[2]);
            acc[3] = fmaf(w, v[u][3], acc[3]);
            wsum += w;
        }
        const int q0 = p0 + SLOTS * kReduceUnroll;
        if (q0 >= n) break;
#pragma unroll
        for (int u = 0; u < kReduceUnroll; ++u) {
            const int p = q0 + u * SLOTS;
            const bool ok = p < n;
            mv[u] = ok ? mlr[p] : -INFINITY;
            ev[u] = ok ? esr[p] : 0.f;
            v[u] = ok ? *reinterpret_cast<const f32x4 *>(base + (long)p * head_dim) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    *reinterpret_cast<f32x4 *>(red + slot * kReduceChunk + dl * 4) = acc;
    if (dl == 0) {
        sm[slot] = m;
        sw[slot] = wsum;
    }
    __syncthreads();
    for (int d = tid; d < kReduceChunk; d += NW * 64) {
        float M = -INFINITY;
#pragma unroll
        for (int sl = 0; sl < SLOTS; ++sl) M = fmaxf(M, sm[sl]);
        float a = 0.f, ws = 0.f;
#pragma unroll
        for (int sl = 0; sl < SLOTS; ++sl) {
            const float f = sw[sl] > 0.f ? fast_exp2((sm[sl] - M) * kLog2e) : 0.f;
            a = fmaf(f, red[sl * kReduceChunk + d], a);
            ws = fmaf(f, sw[sl], ws);
        }
        o[d] = (uint16_t)f32_to_bf16_bits(a / ws);
    }
}

// Cross-partition merge for partial buffers with few partition slots (a
// batch of many sequences with a handful of partitions each): one wave per
// (sequence, query head).  The wave's lanes form R = 256 / D rows of D / 4
// lanes (4 dims per lane); the rows take partitions round-robin, 4 at a time
// with every load issued before any is used, each row keeping a running max.
// The rows are then folded with lane swaps (rows 16 and 32 lanes apart) using
// only symmetric operations, so every lane of a fold holds the same result.
// When every slot fits in the first round, the records are loaded before the
// sequence length is known (records past the sequence's partitions are
// discarded by selection, never used in arithmetic).
constexpr int kWaveReduceUnroll = 4;
constexpr int kWaveReduceMaxRounds = 8;  // slots per row beyond this use paged_reduce_kernel

template <int D>
__global__ __launch_bounds__(256) void paged_reduce_wave_kernel(
    const float *__restrict__ max_logits, const float *__restrict__ exp_sums,
    const float *__restrict__ tmp_out, const int32_t *__restrict__ seq_lens,
    const int32_t *__restrict__ kv_indptr, int num_seqs, int num_q_heads, int partition_size,
    int max_num_partitions, uint16_t *__restrict__ out) {
    constexpr int LPR = D / 4;   // lanes per row
    constexpr int R = 64 / LPR;  // rows per wave
    constexpr int U = kWaveReduceUnroll;
    const int lane = threadIdx.x & 63;
    const long pair = (long)blockIdx.x * 4 + (threadIdx.x >> 6);  // sequence * H_q + head
    if (pair >= (long)num_seqs * num_q_heads) return;
    const int seq = (int)(pair / num_q_heads);
    const int r = lane / LPR, d0 = 4 * (lane % LPR);
    const float *mlr = max_logits + pair * max_num_partitions;
    const float *esr = exp_sums + pair * max_num_partitions;
    const float *base = tmp_out + pair * (long)max_num_partitions * D + d0;
    const bool speculate = max_num_partitions <= R * U;
    int n = 0;
    if (!speculate) {
        const int L = kv_indptr ? kv_indptr[seq + 1] - kv_indptr[seq] : seq_lens[seq];
        n = L > 0 ? (L + partition_size - 1) / partition_size : 0;
    }
    const int first_bound = speculate ? max_num_partitions : n;
    float mv[U], ev[U];
    f32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int p = r + u * R;
        const bool in = p < first_bound;
        mv[u] = in ? mlr[p] : -INFINITY;
        ev[u] = in ? esr[p] : 0.f;
        v[u] = in ? *reinterpret_cast<const f32x4 *>(base + (long)p * D) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (speculate) {
        const int L = kv_indptr ? kv_indptr[seq + 1] - kv_indptr[seq] : seq_lens[seq];
        n = L > 0 ? (L + partition_size - 1) / partition_size : 0;
    }
    uint16_t *o = out + pair * D + d0;
    if (n == 0) {
        if (r == 0) *reinterpret_cast<u32x2 *>(o) = u32x2{0u, 0u};
        return;
    }
    float m = -INFINITY, wsum = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int p0 = r;; p0 += R * U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (p0 + u * R >= n) continue;
            if (mv[u] > m) {  // rescale what was accumulated to the new max
                const float f = fast_exp2((m - mv[u]) * kLog2e);
                acc *= f;
                wsum *= f;
                m = mv[u];
            }
            const float w = fast_exp2((mv[u] - m) * kLog2e) * ev[u];
            acc[0] = fmaf(w, v[u][0], acc[0]);
            acc[1] = fmaf(w, v[u][1], acc[1]);
            acc[2] = fmaf(w, v[u][2], acc[2]);
            acc[3] = fmaf(w, v[u][3], acc[3]);
            wsum += w;
        }
        const int q0 = p0 + R * U;
        if (__all(q0 >= n)) break;  // wave-uniform exit; rows past n load nothing below
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int p = q0 + u * R;
            const bool ok = p < n;
            mv[u] = ok ? mlr[p] : -INFINITY;
            ev[u] = ok ? esr[p] : 0.f;
            v[u] = ok ? *reinterpret_cast<const f32x4 *>(base + (long)p * D) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    // fold the rows: rescale each to the common max, then sum
    auto fold = [&](auto max_x, auto sum_x) {
        const float M = max_x(m);
        const float f = wsum > 0.f ? fast_exp2((m - M) * kLog2e) : 0.f;
        wsum = sum_x(f * wsum);
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[k] = sum_x(f * acc[k]);
        m = M;
    };
    if constexpr (R >= 4) fold([](float x) { return max_xor16(x); }, [](float x) { return sum_xor16(x); });
    if constexpr (R >= 2) fold([](float x) { return max_xor32(x); }, [](float x) { return sum_xor32(x); });
    if (r == 0) {
        const float inv = 1.f / wsum;
        *reinterpret_cast<u32x2 *>(o) = u32x2{pack_bf16x2(acc[0] * inv, acc[1] * inv),
                                             pack_bf16x2(acc[2] * inv, acc[3] * inv)};
    }
}

// ---------------------------------------------------------------------------
// host-side launch of the partition kernels (instantiated per cache type by
// decode.hip and decode_fp8.hip)
// ---------------------------------------------------------------------------
namespace launch_detail {
// Waves per decode workgroup and register prefetch depth (tiles in flight per
// wave while one is consumed; deeper costs D/4 VGPRs per tile).
#ifndef PA_DECODE_WAVES
#define PA_DECODE_WAVES 4
#endif
constexpr int kDecodeWaves = PA_DECODE_WAVES;
#ifndef PA_DECODE_DEPTH
#define PA_DECODE_DEPTH 1
#endif
#ifndef PA_DECODE_DEPTH_FP8
#define PA_DECODE_DEPTH_FP8 1
#endif
constexpr int decode_depth(int, bool fp8) { return fp8 ? PA_DECODE_DEPTH_FP8 : PA_DECODE_DEPTH; }
#ifndef PA_DECODE_PERSIST_PER_CU
#define PA_DECODE_PERSIST_PER_CU 0   // 0 = as many workgroups per CU as fit
#endif
// FP8 caches: at most two persistent workgroups per CU where the grid has
// many items, three where it has at most kFp8FewItemsPerCu per CU.  An FP8
// tile is half the bytes of a bf16 one, so a few long items leave too little
// in flight with two; with many items a third only adds cache pressure
// (measured on MI355X: three take a 72k-token Llama-3-8B-shaped batch of
// 2,048 items from 36.2-36.6 to 33.4-33.9 us, and a 432k-token ragged G=8
// batch from 193.5 to 199.8 us; a 400k-token D=256 batch is unchanged).
#ifndef PA_FP8_FEW_ITEMS_PERSIST_PER_CU
#define PA_FP8_FEW_ITEMS_PERSIST_PER_CU 3  // (2 reproduces the cap before the rule)
#endif
constexpr int kFp8PersistPerCu = 2;
constexpr int kFp8FewItemsPersistPerCu = PA_FP8_FEW_ITEMS_PERSIST_PER_CU;
constexpr int kFp8FewItemsPerCu = 8;


template <int D, int G, bool FP8, bool XP, bool TOK>
hipError_t launch_decode_dg(const DecodeArgs &a) {
    constexpr int DEPTH = decode_depth(D, FP8);
    DecodeParams prm{a.q, a.k_cache, a.v_cache, a.block_tables, a.seq_lens, a.num_seqs,
                     a.num_q_heads, a.num_kv_heads, a.max_blocks_per_seq, a.scale_log2,
                     a.partition_size, a.max_num_partitions, a.out, a.max_logits, a.exp_sums,
                     a.tmp_out, a.counters, 0, a.k_scales, a.v_scales, a.kv_indptr};
    dim3 block(kDecodeWaves * 64);
    // Fused merge over a bf16 block cache: the stream-K schedule, when its
    // smallest unit that keeps each pair within max_num_partitions records
    // (ceil(max_blocks_per_seq / (max_num_partitions - 1)) tiles) fits one
    // block-id chunk per wave.
    if constexpr (!FP8 && !XP && !TOK) {
        const long unit_max = kDecodeWaves * 64;
        if (a.counters && a.partition_size > 0 && a.num_seqs <= kCompactMaxSeqs && a.max_num_partitions >= 2) {
            const long sk_min = ((long)a.max_blocks_per_seq + a.max_num_partitions - 2) / (a.max_num_partitions - 1);
            if (sk_min <= unit_max) {
                prm.sk_min_tiles = (int)sk_min;
                const int per_cu = resident_per_cu<paged_decode_streamk_kernel<D, G, kDecodeWaves, DEPTH>>(block.x);
                dim3 grid((unsigned)(device_cu_count() * per_cu));
                hipLaunchKernelGGL((paged_decode_streamk_kernel<D, G, kDecodeWaves, DEPTH>), grid, block, 0,
                                   a.stream, prm);
                return hipGetLastError();
            }
        }
    }
    if (a.partition_size > 0 && a.partition_size <= kDecodeWaves * 64 * kBlock &&
        a.num_seqs <= kCompactMaxSeqs) {
        int per_cu = PA_DECODE_PERSIST_PER_CU > 0
                         ? PA_DECODE_PERSIST_PER_CU
                         : resident_per_cu<paged_decode_compact_kernel<D, G, kDecodeWaves, DEPTH, FP8, XP, TOK>>(block.x);
        const long upper = (long)a.num_seqs * a.num_kv_heads * a.num_partitions;
        if (FP8) {
            const int most = upper <= (long)kFp8FewItemsPerCu * device_cu_count() ? kFp8FewItemsPersistPerCu
                                                                                   : kFp8PersistPerCu;
            if (per_cu > most) per_cu = most;
        }
        const long cap = (long)device_cu_count() * per_cu;
        dim3 grid((unsigned)(upper < cap ? upper : cap));
        hipLaunchKernelGGL((paged_decode_compact_kernel<D, G, kDecodeWaves, DEPTH, FP8, XP, TOK>), grid, block, 0,
                           a.stream, prm);
    } else {
        dim3 grid(a.num_partitions, a.num_kv_heads, a.num_seqs);
        hipLaunchKernelGGL((paged_decode_grid_kernel<D, G, kDecodeWaves, DEPTH, FP8, XP, TOK>), grid, block, 0,
                           a.stream, prm);
    }
    return hipGetLastError();
}

template <int D, bool FP8, bool XP, bool TOK>
hipError_t launch_decode_d(const DecodeArgs &a, int G) {
    switch (G) {
        case 1: return launch_decode_dg<D, 1, FP8, XP, TOK>(a);
        case 2: return launch_decode_dg<D, 2, FP8, XP, TOK>(a);
        case 3: return launch_decode_dg<D, 3, FP8, XP, TOK>(a);
        case 4: return launch_decode_dg<D, 4, FP8, XP, TOK>(a);
        case 5: return launch_decode_dg<D, 5, FP8, XP, TOK>(a);
        case 6: return launch_decode_dg<D, 6, FP8, XP, TOK>(a);
        case 7: return launch_decode_dg<D, 7, FP8, XP, TOK>(a);
        case 8: return launch_decode_dg<D, 8, FP8, XP, TOK>(a);
        case 9: return launch_decode_dg<D, 9, FP8, XP, TOK>(a);
        case 10: return launch_decode_dg<D, 10, FP8, XP, TOK>(a);
        case 11: return launch_decode_dg<D, 11, FP8, XP, TOK>(a);
        case 12: return launch_decode_dg<D, 12, FP8, XP, TOK>(a);
        case 13: return launch_decode_dg<D, 13, FP8, XP, TOK>(a);
        case 14: return launch_decode_dg<D, 14, FP8, XP, TOK>(a);
        case 15: return launch_decode_dg<D, 15, FP8, XP, TOK>(a);
        case 16: return launch_decode_dg<D, 16, FP8, XP, TOK>(a);
        default: return hipErrorInvalidValue;
    }
}

// Decode launch for a bf16 (FP8 false) or FP8 cache, in the row-major tile
// layout, (XP) the x-packed K / transposed V layout, or (TOK) a
// token-granular cache addressed through kv_indptr and page indices.
template <bool FP8, bool XP, bool TOK = false>
hipError_t launch_decode_t(const DecodeArgs &a) {
    const int G = a.num_q_heads / a.num_kv_heads;
    switch (a.head_dim) {
        case 64: return launch_decode_d<64, FP8, XP, TOK>(a, G);
        case 128: return launch_decode_d<128, FP8, XP, TOK>(a, G);
        case 256: return launch_decode_d<256, FP8, XP, TOK>(a, G);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace launch_detail

}  // namespace pa
