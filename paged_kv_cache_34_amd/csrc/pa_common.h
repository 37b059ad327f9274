// Device-side helpers shared by the gfx950 kernels of the paged attention
// library: vector types for MFMA operands, bf16 <-> fp32 bit conversions and
// wave64 DPP row reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;

// bf16 element in the low / high half of a packed dword, widened exactly.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// 2^x on the hardware exponential unit (v_exp_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// DPP controls of the GFX9 family (row = 16 lanes).
enum : int {
    kDppQuadXor1 = 0xB1,    // quad_perm [1,0,3,2]
    kDppQuadXor2 = 0x4E,    // quad_perm [2,3,0,1]
    kDppRowHalfMirror = 0x141,
    kDppRowMirror = 0x140,
    kDppRowRor8 = 0x128,
};

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Max / sum over the 16 lanes of a DPP row; every lane of the row gets the result.
__device__ __forceinline__ float row16_max(float x) {
    x = fmaxf(x, dpp_f<kDppQuadXor1>(x));
    x = fmaxf(x, dpp_f<kDppQuadXor2>(x));
    x = fmaxf(x, dpp_f<kDppRowHalfMirror>(x));
    x = fmaxf(x, dpp_f<kDppRowMirror>(x));
    return x;
}

__device__ __forceinline__ float row16_sum(float x) {
    x += dpp_f<kDppQuadXor1>(x);
    x += dpp_f<kDppQuadXor2>(x);
    x += dpp_f<kDppRowHalfMirror>(x);
    x += dpp_f<kDppRowMirror>(x);
    return x;
}

// Value of lane (lane ^ mask) for masks >= 16 (crosses DPP rows): ds_bpermute.
__device__ __forceinline__ float xor_lane(float x, int mask) {
    int lane = __lane_id();
    return __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, __float_as_int(x)));
}

// Sum of x over lane pairs (l, l ^ 32): both halves of the wave get the total.
__device__ __forceinline__ float sum_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum of x over lane pairs (l, l ^ 16).
__device__ __forceinline__ float sum_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Orders this wave's LDS writes before its later LDS reads of other lanes' data.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Workgroup barrier for LDS traffic only: unlike __syncthreads it does not
// wait for the wave's outstanding global loads or stores, so prefetched tiles and
// written results stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ u32x4 load_u32x4(const uint16_t *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}

}  // namespace pa
