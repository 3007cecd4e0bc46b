// qmm_quant.hip -- q8_1 activation quantization and FP16 weight dequantization for gfx950.
//
// q8_1 [DQ, Change: the q8_1 quantizer's 32-value blocks; GP, What changed]: per block
// d = amax/127 (binary32), q = x/d (binary32 IEEE division) rounded half away from zero,
// stored d = fp16(d), s = fp16(d * sum q); an all-zero block is all zeros.
// FP16 dequant [DQ, Change: one thread per 8 outputs and one 16-byte store; every value the
// exact product rounded once to nearest even].  Q8_0 / IQ4_NL: the factor, formed exactly as
// a binary16 integer, times the binary16 scale in one packed binary16 multiply (a single
// rounding of the exact product); the prefill GEMM converts its weights with the same code.
// CB3 (factor up to 8 x 31 x 15): the binary32 product is exact, one v_cvt_f16_f32 rounds it.
#include "qmm_device.h"
#include "qmm_host.h"

namespace qmm {

// One lane per value, one aligned half wave per q8_1 block.  x: [ncols][ldx] floats.
__global__ __launch_bounds__(256) void quantize_q8_1_kernel(const float* __restrict__ x, int64_t ldx, int nb,
                                                            int ncols, uint8_t* __restrict__ xq) {
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t blk = g >> 5;
    const int j = (int)(g & 31);
    const bool ok = blk < (int64_t)nb * ncols;
    float v = 0.0f;
    if (ok) {
        const int c = (int)(blk / nb), b = (int)(blk - (int64_t)c * nb);
        v = x[c * ldx + 32 * b + j];
    }
    uint32_t hdr;
    const int q = quantize_lanes32(v, hdr);
    const uint32_t word = pack4_lanes(q);
    if (ok) {
        uint32_t* dst = (uint32_t*)(xq + blk * 36);
        if (j == 0) dst[0] = hdr;
        if ((j & 3) == 0) dst[1 + (j >> 2)] = word;
    }
}

// Integer factors of values [j0, j0+8) of a row (j0 a multiple of 8), and the fp16 scale of
// their block.  Byte-granular reads: the dequant kernel is written for its stores.
template <int WT>
__device__ __forceinline__ void factors8(const uint8_t* __restrict__ row, const uint8_t* __restrict__ grid,
                                         int j0, int* f, uint32_t* dbits) {
    if constexpr (WT == kQ8_0) {
        const uint8_t* b = row + (j0 / 32) * 34;
        *dbits = b[0] | (b[1] << 8);
#pragma unroll
        for (int t = 0; t < 8; ++t) f[t] = (int8_t)b[2 + (j0 % 32) + t];
    } else if constexpr (WT == kIQ4_NL) {
        const uint8_t* b = row + (j0 / 32) * 18;
        *dbits = b[0] | (b[1] << 8);
        const int jj = j0 % 32;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int e = jj + t;
            const int nib = e < 16 ? (b[2 + e] & 15) : (b[2 + e - 16] >> 4);
            f[t] = kIQ4NLLevels[nib];
        }
    } else {
        const uint8_t* b = row + (j0 / 256) * kCB3Bytes;
        *dbits = b[0] | (b[1] << 8);
        const int v0 = j0 % 256;
        const int s = v0 / 32;
        const int mul = 1 + 2 * ((b[kCB3Scales + s / 2] >> (4 * (s % 2))) & 15);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int v = v0 + t;
            const int i = v / 4;
            const int idx = b[kCB3Qs + i] | (((b[kCB3Qh + i / 8] >> (i % 8)) & 1) << 8);
            const int mag = grid[idx * 4 + v % 4];
            const int neg = (b[kCB3Signs + v / 8] >> (v % 8)) & 1;
            f[t] = mul * (neg ? -mag : mag);
        }
    }
}

// Each thread writes 8 consecutive outputs of a row; a workgroup covers `rpw` rows.
template <int WT, bool VEC>
__global__ __launch_bounds__(256) void dequant_f16_kernel(const uint8_t* __restrict__ w, const uint8_t* __restrict__ grid,
                                                          int64_t nrows, int k, int64_t rb, int rpw,
                                                          uint16_t* __restrict__ out, int64_t ld) {
    const unsigned per_row = (unsigned)k / 8u;
    const int64_t r0 = (int64_t)blockIdx.x * rpw;
    for (unsigned u = threadIdx.x; u < per_row * (unsigned)rpw; u += blockDim.x) {
        const unsigned rr = u / per_row;
        const int64_t r = r0 + rr;
        if (r >= nrows) break;
        const int j0 = (int)(u - rr * per_row) * 8;
        int f[8];
        uint32_t dbits;
        factors8<WT>(w + r * rb, grid, j0, f, &dbits);
        uint32_t h[8];
        if constexpr (WT == kCB3) {
            // integer factor times multiplier exceeds a byte: binary32 product (exact), one RNE
            const float d = h2f(dbits);
#pragma unroll
            for (int i = 0; i < 8; ++i) h[i] = f2h(opaque(d * (float)f[i]));
        } else {
            // the packed binary16 conversion the prefill GEMM uses for its weights
            const half2_t dd = splat_h2(dbits);
#pragma unroll
            for (int i = 0; i < 8; i += 4) {
                const uint32_t u = (uint32_t)(f[i] + 128) | ((uint32_t)(f[i + 1] + 128) << 8) |
                                   ((uint32_t)(f[i + 2] + 128) << 16) | ((uint32_t)(f[i + 3] + 128) << 24);
                uint32_t lo, hi;
                u8x4_to_f16(u, dd, lo, hi);
                h[i] = lo & 0xFFFFu;
                h[i + 1] = lo >> 16;
                h[i + 2] = hi & 0xFFFFu;
                h[i + 3] = hi >> 16;
            }
        }
        uint16_t* dst = out + r * ld + j0;
        if constexpr (VEC) {
            u32x4 v;
            v.x = h[0] | (h[1] << 16);
            v.y = h[2] | (h[3] << 16);
            v.z = h[4] | (h[5] << 16);
            v.w = h[6] | (h[7] << 16);
            *(u32x4*)dst = v;
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) dst[i] = (uint16_t)h[i];
        }
    }
}

template <int WT>
static void launch_dequant(const void* w, const uint8_t* grid, int64_t nrows, int64_t k, uint16_t* out, int64_t ld,
                           bool vec, hipStream_t st) {
    const int64_t per_row = k / 8;
    const int rpw = per_row >= 256 ? 1 : (int)(256 / per_row);
    const dim3 g((unsigned)((nrows + rpw - 1) / rpw));
    const int64_t rb = qmm_row_bytes(WT, k);
    if (vec)
        hipLaunchKernelGGL((dequant_f16_kernel<WT, true>), g, dim3(256), 0, st, (const uint8_t*)w, grid, nrows, (int)k, rb,
                           rpw, out, ld);
    else
        hipLaunchKernelGGL((dequant_f16_kernel<WT, false>), g, dim3(256), 0, st, (const uint8_t*)w, grid, nrows, (int)k, rb,
                           rpw, out, ld);
}

}  // namespace qmm

using namespace qmm;

extern "C" int qmm_quantize_q8_1(const float* x, int64_t k, int ncols, int64_t ldx, void* xq, void* stream) {
    if (!x || !xq || k < 32 || k % 32 || ncols < 1 || ldx < k) return QMM_EINVAL;
    if (!aligned(x, 4) || !aligned(xq, 4)) return QMM_EALIGN;
    if (k > (int64_t)1 << 30 || (int64_t)ncols * (k / 32) > ((int64_t)1 << 31)) return QMM_EUNSUPPORTED;
    const int nb = (int)(k / 32);
    const int64_t n = (int64_t)nb * ncols * 32;
    hipLaunchKernelGGL(quantize_q8_1_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, as_stream(stream), x, ldx,
                       nb, ncols, (uint8_t*)xq);
    return launch_status();
}

extern "C" int qmm_dequant_f16(int wtype, const void* w, const uint8_t* grid, int64_t nrows, int64_t k, uint16_t* out,
                               int64_t ld, void* stream) {
    if (!valid_wtype(wtype) || !w || !out || nrows < 1 || ld < k) return QMM_EINVAL;
    if (qmm_row_bytes(wtype, k) == 0) return QMM_EINVAL;
    if (wtype == QMM_CB3 && !grid) return QMM_EINVAL;
    if (!aligned(w, 2) || !aligned(out, 2)) return QMM_EALIGN;
    if (k > (int64_t)1 << 24 || nrows > 0x7FFFFFFF) return QMM_EUNSUPPORTED;
    const bool vec = aligned(out, 16) && ld % 8 == 0;
    const hipStream_t st = as_stream(stream);
    switch (wtype) {
        case QMM_Q8_0: launch_dequant<kQ8_0>(w, grid, nrows, k, out, ld, vec, st); break;
        case QMM_IQ4_NL: launch_dequant<kIQ4_NL>(w, grid, nrows, k, out, ld, vec, st); break;
        default: launch_dequant<kCB3>(w, grid, nrows, k, out, ld, vec, st); break;
    }
    return launch_status();
}
