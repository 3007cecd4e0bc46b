// qmm_probe.hip -- reference kernels the hot path's measurements are set against: a plain
// streaming read of a buffer in one launch (16-byte loads, eight in flight per thread, no
// compute beyond an XOR that keeps the loads live), and a register-only loop of the fp16 MFMA
// instruction the prefill GEMM uses (eight independent accumulators per wave, no memory).
#include "qmm_device.h"
#include "qmm_host.h"

namespace qmm {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

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

constexpr int kMfmaChains = 8;

// Each wave: kMfmaChains accumulators, `iters` rounds of one v_mfma_f32_32x32x16_f16 per
// accumulator (32 x 32 x 16 multiply-adds each); lane l writes its sum to out[t].
__global__ __launch_bounds__(kProbeThreads) void mfma_loop_kernel(float* __restrict__ out, int iters) {
    const uint32_t l = threadIdx.x;
    half8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (_Float16)(float)((l + e) & 7);
        b[e] = (_Float16)(float)((l * 3 + e) & 7);
    }
    f32x16 acc[kMfmaChains];
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c) acc[c] = f32x16{};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int c = 0; c < kMfmaChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[c], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[c][r];
    out[(uint64_t)blockIdx.x * kProbeThreads + l] = s;
}

}  // namespace qmm

using namespace qmm;

extern "C" int qmm_debug_mfma_loop(float* out, int grid, int iters, void* stream) {
    if (!out || grid < 1 || iters < 1) return QMM_EINVAL;
    if (!aligned(out, 4)) return QMM_EALIGN;
    hipLaunchKernelGGL(mfma_loop_kernel, dim3((unsigned)grid), dim3(kProbeThreads), 0, as_stream(stream), out, iters);
    return launch_status();
}

extern "C" int qmm_debug_stream_read(const void* p, uint64_t nbytes, uint32_t* out, int grid, void* stream) {
    if (!p || !out || nbytes == 0 || nbytes % 16 || grid < 1) return QMM_EINVAL;
    if (!aligned(p, 16) || !aligned(out, 4)) return QMM_EALIGN;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3(kProbeThreads), 0, as_stream(stream),
                       (const uint8_t*)p, nbytes / 16, out);
    return launch_status();
}
