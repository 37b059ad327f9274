// KV cache writes for gfx950: the K/V rows of new tokens go to their cache
// slots -- the write that comes before decode and prefill (on the AstrAI
// page the backend layer is responsible for cache writes as well as reads).
// Either copied as bf16, or
// quantized to FP8 (OCP E4M3) with one dequant scale per (position, kv head)
// (the B200 page, "FP8 KV Quantize/Dequant" and the per-position dequant scale
// of "Stage D: FP8 Paged KV Gather").
//
// Placement: sequence s owns new rows [cu[s], cu[s+1]); they are the last
// n = cu[s+1] - cu[s] of its seq_lens[s] tokens, so row j goes to position
// c + j (c = seq_lens[s] - n), block table entry (c + j) / 16, slot
// (c + j) % 16 -- where the prefill kernel expects the rows it attends to.
//
// The bf16 kernel also writes the BI-V100 page's layouts (x-packed K,
// transposed V).  Both kernels are HBM-bound copies: grid (token groups, sequences), each
// workgroup moving kAppendTokens new tokens with 16-byte loads and stores.
#include "pa_common.h"
#include "pa_launch.h"

namespace pa {
namespace {

constexpr int kAppendTokens = 8;     // new tokens per workgroup
constexpr int kAppendThreads = 256;
constexpr int kSlots = 16;           // tokens per cache block
constexpr float kE4m3Max = 448.0f;   // largest finite E4M3 magnitude

// bf16: every (token, K/V, kv head, 16-byte chunk) is one copy.  In the
// BI-V100 page's layouts (XP) the K chunk lands at its x-packed place
// [D/8][16][8] (still 16 contiguous bytes) and the V chunk's 8 values are
// scattered down the token column of the transposed tile [D][16].
template <int D, bool XP>
__global__ __launch_bounds__(kAppendThreads) void paged_kv_append_kernel(AppendArgs a) {
    const int s = blockIdx.y;
    const int row0 = a.cu_seqlens[s];
    const int n = a.cu_seqlens[s + 1] - row0;
    const int j0 = blockIdx.x * kAppendTokens;
    if (j0 >= n) return;
    const int c = a.seq_lens[s] - n;
    const int nt = min(kAppendTokens, n - j0);
    constexpr int CPR = D / 8;                  // 16-byte chunks per row
    const int hkv = a.num_kv_heads;
    const int per_tensor = hkv * CPR;
    const int per_tok = 2 * per_tensor;
    const int32_t *bt = a.block_tables + (long)s * a.max_blocks_per_seq;
    const uint16_t *kn = static_cast<const uint16_t *>(a.k_new);
    const uint16_t *vn = static_cast<const uint16_t *>(a.v_new);
    uint16_t *kc = static_cast<uint16_t *>(a.k_cache);
    uint16_t *vc = static_cast<uint16_t *>(a.v_cache);
    for (int e = threadIdx.x; e < nt * per_tok; e += kAppendThreads) {
        const int tj = e / per_tok, r = e - tj * per_tok;
        const bool is_v = r >= per_tensor;
        const int r2 = is_v ? r - per_tensor : r;
        const int h = r2 / CPR, ch = r2 - h * CPR;
        const int j = j0 + tj, pos = c + j;
        const long phys = bt[pos / kSlots];
        const long src = ((long)(row0 + j) * hkv + h) * D + ch * 8;
        const u32x4 w = *reinterpret_cast<const u32x4 *>((is_v ? vn : kn) + src);
        if constexpr (XP) {
            const long tile = (phys * hkv + h) * kSlots * D;
            const int slot = pos % kSlots;
            if (!is_v) {
                *reinterpret_cast<u32x4 *>(kc + tile + (ch * kSlots + slot) * 8) = w;
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    vc[tile + (ch * 8 + e) * kSlots + slot] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
            }
        } else {
            const long dst = ((phys * hkv + h) * kSlots + pos % kSlots) * D + ch * 8;
            *reinterpret_cast<u32x4 *>((is_v ? vc : kc) + dst) = w;
        }
    }
}

// Non-negative fp32 y (at most 448 up to one rounding of the scale) -> the
// E4M3 magnitude code nearest to it, ties to the even code, saturating at 448.
// Normal range (y >= 2^-6): round the fp32 mantissa to 3 bits (ties to even)
// and re-bias the exponent from 127 to 7; a mantissa carry moves into the
// exponent by itself.  Subnormal range: the code is y * 2^9 rounded to an
// integer, ties to even (8 lands on 2^-6, code 0x08).
__device__ __forceinline__ uint32_t e4m3_code(float y) {
    if (y >= kE4m3Max) return 0x7Eu;
    if (y < 0.015625f) return (uint32_t)__builtin_rintf(y * 512.0f);
    const uint32_t u = __float_as_uint(y);
    const uint32_t r = u + 0x7FFFFu + ((u >> 20) & 1u);
    const uint32_t code = (r >> 20) - (120u << 3);
    return code < 0x7Eu ? code : 0x7Eu;
}

__device__ __forceinline__ float row_max_lanes8(float x) {
    x = fmaxf(x, dpp_f<kDppQuadXor1>(x));
    x = fmaxf(x, dpp_f<kDppQuadXor2>(x));
    return fmaxf(x, dpp_f<kDppRowHalfMirror>(x));
}

// Max over the LPR consecutive lanes (8, 16 or 32) that hold one row.
template <int LPR>
__device__ __forceinline__ float row_max(float x) {
    if constexpr (LPR == 8) return row_max_lanes8(x);
    x = row16_max(x);
    if constexpr (LPR == 32) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
    return x;
}

// FP8: a row is (token, K or V, kv head), D values held by D / 8 consecutive
// lanes (8 each); amax over the row, scale = amax / 448, code = nearest E4M3
// to x / scale (both divisions correctly rounded in fp32), sign kept; a row of
// zeros gets scale 0 and zero codes.  The trip count over rows is the same
// for every lane, so the row reductions always run on full waves.
template <int D>
__global__ __launch_bounds__(kAppendThreads) void paged_kv_append_fp8_kernel(AppendArgs a) {
    constexpr int LPR = D / 8;                  // lanes per row
    constexpr int RPP = kAppendThreads / LPR;   // rows per pass
    const int s = blockIdx.y;
    const int row0 = a.cu_seqlens[s];
    const int n = a.cu_seqlens[s + 1] - row0;
    const int j0 = blockIdx.x * kAppendTokens;
    if (j0 >= n) return;
    const int c = a.seq_lens[s] - n;
    const int nt = min(kAppendTokens, n - j0);
    const int hkv = a.num_kv_heads;
    const int rows = nt * 2 * hkv;
    const int li = threadIdx.x % LPR;
    const int32_t *bt = a.block_tables + (long)s * a.max_blocks_per_seq;
    for (int r0 = 0; r0 < rows; r0 += RPP) {
        const int r = r0 + threadIdx.x / LPR;
        const bool ok = r < rows;
        const int rr = ok ? r : 0;
        const int tj = rr / (2 * hkv), rem = rr - tj * 2 * hkv;
        const bool is_v = rem >= hkv;
        const int h = is_v ? rem - hkv : rem;
        const int j = j0 + tj, pos = c + j;
        const long src = ((long)(row0 + j) * hkv + h) * D + li * 8;
        u32x4 w = {0u, 0u, 0u, 0u};
        if (ok) w = *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(is_v ? a.v_new : a.k_new) + src);
        float x[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            x[2 * k] = bf16_lo(w[k]);
            x[2 * k + 1] = bf16_hi(w[k]);
        }
        float amax = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(x[k]));
        amax = row_max<LPR>(amax);
        const float sc = __fdiv_rn(amax, kE4m3Max);
        uint32_t packed[2] = {0u, 0u};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const uint32_t mag = sc > 0.f ? e4m3_code(__fdiv_rn(fabsf(x[k]), sc)) : 0u;
            const uint32_t code = ((__float_as_uint(x[k]) >> 31) << 7) | mag;
            packed[k >> 2] |= code << (8 * (k & 3));
        }
        if (ok) {
            const long phys = bt[pos / kSlots];
            const long slot_row = (phys * hkv + h) * kSlots + pos % kSlots;
            uint8_t *cache = static_cast<uint8_t *>(is_v ? a.v_cache : a.k_cache);
            *reinterpret_cast<u32x2 *>(cache + slot_row * D + li * 8) = u32x2{packed[0], packed[1]};
            if (li == 0) (is_v ? a.v_scales : a.k_scales)[slot_row] = sc;
        }
    }
}

template <bool FP8, bool XP>
hipError_t launch_append(const AppendArgs &a) {
    static_assert(!(FP8 && XP), "the x-packed layout holds bf16");
    dim3 grid((a.max_new_tokens + kAppendTokens - 1) / kAppendTokens, a.num_seqs);
    dim3 block(kAppendThreads);
    switch (a.head_dim) {
        case 64:
            hipLaunchKernelGGL((FP8 ? paged_kv_append_fp8_kernel<64> : paged_kv_append_kernel<64, XP>), grid, block,
                               0, a.stream, a);
            break;
        case 128:
            hipLaunchKernelGGL((FP8 ? paged_kv_append_fp8_kernel<128> : paged_kv_append_kernel<128, XP>), grid,
                               block, 0, a.stream, a);
            break;
        case 256:
            hipLaunchKernelGGL((FP8 ? paged_kv_append_fp8_kernel<256> : paged_kv_append_kernel<256, XP>), grid,
                               block, 0, a.stream, a);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_kv_append(const AppendArgs &a) { return launch_append<false, false>(a); }
hipError_t launch_kv_append_fp8(const AppendArgs &a) { return launch_append<true, false>(a); }
hipError_t launch_kv_append_xpacked(const AppendArgs &a) { return launch_append<false, true>(a); }

}  // namespace pa
