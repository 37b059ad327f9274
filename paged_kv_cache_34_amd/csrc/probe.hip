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

}  // namespace

hipError_t launch_read_probe(const void *buf, long long bytes, uint32_t *partial, int num_workgroups,
                             hipStream_t stream) {
    hipLaunchKernelGGL(hbm_read_probe_kernel, dim3((unsigned)num_workgroups), dim3(kProbeThreads), 0,
                       stream, static_cast<const u32x4 *>(buf), bytes / 16, partial);
    return hipGetLastError();
}

}  // namespace pa
