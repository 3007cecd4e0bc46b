// qmm_probe.hip -- the reference streaming read the decode kernels' HBM time is set against: a
// plain read of a buffer in one launch, 16-byte loads, eight in flight per thread, no compute
// beyond an XOR that keeps the loads live.
#include "qmm_device.h"
#include "qmm_host.h"

namespace qmm {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;

// Thread t of a grid of T threads reads 16-byte chunks t, t + T, t + 2T, ... (eight per round,
// issued together) and writes the XOR of their words to out[t].
__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const uint8_t* __restrict__ p, uint64_t n16,
                                                                    uint32_t* __restrict__ out) {
    const uint64_t t = (uint64_t)blockIdx.x * kProbeThreads + threadIdx.x;
    const uint64_t nt = (uint64_t)gridDim.x * kProbeThreads;
    const u32x4* src = (const u32x4*)p;
    uint32_t acc = 0;
    for (uint64_t i = t; i < n16; i += nt * kProbeUnroll) {
        u32x4 v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) {
            const uint64_t j = i + (uint64_t)u * nt;
            v[u] = j < n16 ? src[j] : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    out[t] = acc;
}

}  // namespace qmm

using namespace qmm;

extern "C" int qmm_debug_stream_read(const void* p, uint64_t nbytes, uint32_t* out, int grid, void* stream) {
    if (!p || !out || nbytes == 0 || nbytes % 16 || grid < 1) return QMM_EINVAL;
    if (!aligned(p, 16) || !aligned(out, 4)) return QMM_EALIGN;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3(kProbeThreads), 0, as_stream(stream),
                       (const uint8_t*)p, nbytes / 16, out);
    return launch_status();
}
