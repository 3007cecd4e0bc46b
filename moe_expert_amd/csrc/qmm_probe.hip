// qmm_probe.hip -- reference kernels the hot path's measurements are set against: a plain
// streaming read of a buffer in one launch (16-byte raw-buffer loads, U in flight per thread,
// contiguous runs per workgroup, no compute beyond an XOR that keeps the loads live), and a
// register-only loop of the fp16 MFMA instruction the prefill GEMM uses (eight independent
// accumulators per wave, no memory).
#include "qmm_device.h"
#include "qmm_host.h"

namespace qmm {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kProbeThreads = 256;

// Workgroup w of `grid` reads the w-th of `grid` contiguous runs of the buffer (whole 16-byte
// chunks); thread t of TH reads chunks t, t + TH, ... of its run, U loads issued together per
// round, through a raw buffer resource over the buffer (the loads the decode GEMV uses: a chunk
// past the end reads zeros, no branch per load); it writes the XOR of the words to out[t].
template <int TH, int U>
__global__ __launch_bounds__(TH) void stream_read_kernel(const uint8_t* __restrict__ p, uint32_t nbytes,
                                                         uint32_t run16, uint32_t* __restrict__ out) {
    const rsrc_t r = make_rsrc(p, nbytes);
    const uint32_t base = blockIdx.x * run16;
    uint32_t acc = 0;
    for (uint32_t i = threadIdx.x; i < run16; i += TH * U) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t j = i + (uint32_t)(u * TH);  // past the run: read at the end (zeros)
            v[u] = ld128(r, j < run16 ? (base + j) * 16u : nbytes);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    out[(uint64_t)blockIdx.x * TH + threadIdx.x] = acc;
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

extern "C" int qmm_debug_stream_read(const void* p, uint64_t nbytes, uint32_t* out, int grid, int threads, int unroll,
                                     void* stream) {
    if (!p || !out || nbytes == 0 || nbytes % 16 || grid < 1) return QMM_EINVAL;
    if ((threads != 256 && threads != 512 && threads != 1024) || (unroll != 4 && unroll != 8 && unroll != 16))
        return QMM_EUNSUPPORTED;
    if (!aligned(p, 16) || !aligned(out, 4)) return QMM_EALIGN;
    if (nbytes + 16ull * (uint64_t)grid > 0xFFFFFFF0ull) return QMM_EUNSUPPORTED;
    const uint64_t n16 = nbytes / 16;
    const uint32_t run16 = (uint32_t)((n16 + grid - 1) / grid);
    const hipStream_t st = as_stream(stream);
    auto go = [&](auto kern, int th) {
        hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(th), 0, st, (const uint8_t*)p, (uint32_t)nbytes, run16, out);
    };
#define QMM_SR(TH)                                                                  \
    if (threads == TH) {                                                            \
        if (unroll == 4) go(stream_read_kernel<TH, 4>, TH);                         \
        else if (unroll == 8) go(stream_read_kernel<TH, 8>, TH);                    \
        else go(stream_read_kernel<TH, 16>, TH);                                    \
    }
    QMM_SR(256) QMM_SR(512) QMM_SR(1024)
#undef QMM_SR
    return launch_status();
}
