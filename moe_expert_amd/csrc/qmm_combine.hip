// qmm_combine.hip -- MoE combine for gfx950: each token's expert rows after the down product,
// weighted by the router and summed in k order.
//
// Method [DQ, Change: the combine is one block per token with a fixed thread-to-element mapping
// and k order; profile block: moe_combine4 runs at bandwidth]: out[t][j] = sum over k of
// w[t][k] * y[row_idx[t][k]][j], from +0, adding in k order, each product and each sum rounded
// once in binary32 (no fused multiply-add); an index outside the rows adds nothing.
//
// Mapping: workgroup (t, c) takes token t and chunk c of its row; thread i of the chunk owns the
// 16-byte pieces i, i + 256, ... (S of them) and keeps that mapping for every k, so each piece's
// sum runs in k order in one lane.  The token's indices and weights are the same for the whole
// workgroup (scalar loads).  Each k reads its row through a raw buffer resource over that row
// alone (range 0 for an index outside the rows, and its weight taken as 0), so every load is
// unconditional: a piece past the row, or any piece of a skipped row, reads zeros.  Adding
// 0 * 0 = +0 is the same as adding nothing, because the sum starts at +0 and a binary32 sum is
// -0 only when both of its operands are.  For each group of 8 k values, the 8 S row loads are
// issued before the first sum.  Every y byte is read once and every out byte written once:
// HBM-bound.
#include "qmm_device.h"

namespace qmm {

constexpr int kCbThreads = 256;
constexpr int kCbGroup = 8;  // k values whose loads are issued together
constexpr int kCbMaxTopk = 64;

typedef float f4 __attribute__((ext_vector_type(4)));

template <int S>
__global__ __launch_bounds__(kCbThreads) void combine_kernel(const float* __restrict__ y, int nrows, int h4,
                                                             const int32_t* __restrict__ row_idx,
                                                             const float* __restrict__ wts, int topk,
                                                             float* __restrict__ out, int64_t ldo) {
#pragma clang fp contract(off)
    const int t = blockIdx.x;
    const uint32_t voff = (blockIdx.y * (kCbThreads * S) + threadIdx.x) * 16u;
    const int32_t* ri = row_idx + (int64_t)t * topk;
    const float* wt = wts + (int64_t)t * topk;
    const uint32_t row_bytes = (uint32_t)h4 * 16u;
    f4 acc[S];
#pragma unroll
    for (int s = 0; s < S; ++s) acc[s] = f4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int k0 = 0; k0 < topk; k0 += kCbGroup) {
        f4 v[kCbGroup][S];
        float ww[kCbGroup];
#pragma unroll
        for (int g = 0; g < kCbGroup; ++g) {
            const int k = k0 + g < topk ? k0 + g : topk - 1;
            const int r = __builtin_amdgcn_readfirstlane(ri[k]);
            const float wk = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, wt[k])));
            const bool ok = k0 + g < topk && r >= 0 && r < nrows;
            ww[g] = ok ? wk : 0.0f;
            const rsrc_t rs = make_rsrc(y + (ok ? (int64_t)r * h4 * 4 : 0), ok ? row_bytes : 0u);
#pragma unroll
            for (int s = 0; s < S; ++s) v[g][s] = __builtin_bit_cast(f4, ld128(rs, voff + s * kCbThreads * 16u));
        }
#pragma unroll
        for (int g = 0; g < kCbGroup; ++g) {
#pragma unroll
            for (int s = 0; s < S; ++s) {
                const f4 p = ww[g] * v[g][s];
                acc[s] = acc[s] + p;
            }
        }
    }
    f4* o = (f4*)(out + (int64_t)t * ldo);
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const uint32_t i = voff / 16u + s * kCbThreads;
        if (i < (uint32_t)h4) o[i] = acc[s];
    }
}

}  // namespace qmm

#include "qmm_host.h"

using namespace qmm;

extern "C" int qmm_moe_combine(const float* y, int64_t nrows, int64_t hidden, const int32_t* row_idx,
                               const float* weights, int64_t ntok, int topk, float* out, int64_t ldo, void* stream) {
    if (!y || !row_idx || !weights || !out || nrows < 1 || hidden < 1 || ntok < 0 || topk < 1 || ldo < hidden)
        return QMM_EINVAL;
    if (topk > kCbMaxTopk) return QMM_EUNSUPPORTED;
    if (hidden % 4 || ldo % 4) return QMM_EUNSUPPORTED;
    if (!aligned(y, 16) || !aligned(out, 16) || !aligned(row_idx, 4) || !aligned(weights, 4)) return QMM_EALIGN;
    if (ntok > 0x7FFFFFFF || nrows > 0x7FFFFFFF || hidden > ((int64_t)1 << 28)) return QMM_EUNSUPPORTED;
    if (ntok == 0) return QMM_OK;
    const int h4 = (int)(hidden / 4);
    const int s = h4 <= kCbThreads ? 1 : h4 <= 2 * kCbThreads ? 2 : h4 <= 3 * kCbThreads ? 3 : 4;
    const int chunks = (h4 + kCbThreads * s - 1) / (kCbThreads * s);
    if (chunks > 65535) return QMM_EUNSUPPORTED;
    const dim3 grid((unsigned)ntok, (unsigned)chunks);
    const hipStream_t st = as_stream(stream);
    switch (s) {
        case 1: hipLaunchKernelGGL(combine_kernel<1>, grid, dim3(kCbThreads), 0, st, y, (int)nrows, h4, row_idx, weights, topk, out, ldo); break;
        case 2: hipLaunchKernelGGL(combine_kernel<2>, grid, dim3(kCbThreads), 0, st, y, (int)nrows, h4, row_idx, weights, topk, out, ldo); break;
        case 3: hipLaunchKernelGGL(combine_kernel<3>, grid, dim3(kCbThreads), 0, st, y, (int)nrows, h4, row_idx, weights, topk, out, ldo); break;
        default: hipLaunchKernelGGL(combine_kernel<4>, grid, dim3(kCbThreads), 0, st, y, (int)nrows, h4, row_idx, weights, topk, out, ldo); break;
    }
    return launch_status();
}
