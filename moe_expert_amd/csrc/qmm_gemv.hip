// qmm_gemv.hip -- multi-column decode GEMV over Q8_0 / IQ4_NL / CB3 weight blocks and q8_1
// activations, for gfx950.
//
// Method [IQ, What it does]: every weight block of the call is loaded and decoded once and
// applied to each column of the pass (1, 2, 4 or 8 columns; passes of 8 beyond 8), with the
// same integer chain and the same float expression for every column, so each column equals a
// one-column call bit for bit.  Activations are staged once per workgroup in LDS as an int8
// plane plus block scales [GP, What changed]; the per-block integer dot is v_dot4_i32_i8;
// a row's partial sums are combined across its lanes by a butterfly with no barrier.
//
// Mapping (wave64): 8 lanes per row, 8 rows per wave, 4 waves (32 rows) per workgroup.  Lane
// l of a row takes weight units l, l+8, l+16, ... (a unit = a 4-byte aligned pair of Q8_0 /
// IQ4_NL blocks, or sub-block l of every CB3 super-block), so the 8 lanes of a row read
// consecutive bytes and every weight byte of the matrix is read once per call.
#include "qmm_device.h"
#include "qmm_host.h"

namespace qmm {

constexpr int kLanesPerRow = 8;
constexpr int kRowsPerWG = 32;
constexpr int kThreads = 256;
constexpr int kUnitChunk = 5;  // units whose loads are issued together per lane

template <int WT>
__host__ __device__ constexpr int row_bytes_dev(int K) {
    return WT == kQ8_0 ? (K / 32) * 34 : WT == kIQ4_NL ? (K / 32) * 18 : (K / 256) * kCB3Bytes;
}

// Per-lane iteration count and the unit covered at step i by lane l8.
template <int WT>
__device__ __forceinline__ int units_per_lane(int K) {
    return WT == kCB3 ? K / 256 : (K / 64 + kLanesPerRow - 1) / kLanesPerRow;
}

// Partial sums of one lane over its units of row `row`, for columns [0, ncp) staged in `act`.
// With SUMS, writes the per-block integer sums to `sums` instead (test hook).
template <int WT, int NC, bool SUMS>
__device__ __forceinline__ void lane_partials(rsrc_t wr, uint32_t row_off, int K, int l8, ActLds act,
                                              int ncp, const uint32_t* grid, float (&acc)[NC],
                                              int32_t* sums, int64_t sums_col_stride, bool row_ok) {
    using UT = Unit<WT>;
    const int niter = units_per_lane<WT>(K);
    const int npairs = K / 64;
    for (int i0 = 0; i0 < niter; i0 += kUnitChunk) {
        uint32_t raw[kUnitChunk][UT::RAW];
#pragma unroll
        for (int u = 0; u < kUnitChunk; ++u) {
            const int i = i0 + u;
            if constexpr (WT == kCB3) {
                if (i < niter) UT::load(wr, row_off + (uint32_t)i * kCB3Bytes, l8, raw[u]);
            } else {
                const int p = l8 + kLanesPerRow * i;
                if (i < niter && p < npairs) {
                    UT::load(wr, row_off + (uint32_t)p * UT::UNIT_BYTES, raw[u]);
                } else {
#pragma unroll
                    for (int j = 0; j < UT::RAW; ++j) raw[u][j] = 0;
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kUnitChunk; ++u) {
            const int i = i0 + u;
            if (i >= niter) break;
            uint32_t W[UT::BLK][8];
            uint32_t dw[UT::BLK];
            int mult[UT::BLK];
            int blk0;
            if constexpr (WT == kCB3) {
                UT::decode(raw[u], row_off + (uint32_t)i * kCB3Bytes, l8, grid, W, dw, mult);
                blk0 = 8 * i + l8;
            } else {
                UT::decode(raw[u], W, dw, mult);
                blk0 = 2 * (l8 + kLanesPerRow * i);
            }
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                if (c < ncp) {
#pragma unroll
                    for (int bk = 0; bk < UT::BLK; ++bk) {
                        const int b = blk0 + bk;
                        if (b >= act.nb) continue;  // pair beyond the row (odd block count is declined)
                        const uint32_t* a = act.q + c * act.kw + b * 8;
                        const u32x4 a0 = *(const u32x4*)a;
                        const u32x4 a1 = *(const u32x4*)(a + 4);
                        int s = dot4(W[bk][0], a0.x, 0);
                        s = dot4(W[bk][1], a0.y, s);
                        s = dot4(W[bk][2], a0.z, s);
                        s = dot4(W[bk][3], a0.w, s);
                        s = dot4(W[bk][4], a1.x, s);
                        s = dot4(W[bk][5], a1.y, s);
                        s = dot4(W[bk][6], a1.z, s);
                        s = dot4(W[bk][7], a1.w, s);
                        const int isum = s * mult[bk];
                        if constexpr (SUMS) {
                            if (row_ok) sums[c * sums_col_stride + b] = isum;
                        } else {
                            const float dd = h2f(dw[bk]) * act.d[c * act.nb + b];
                            acc[c] = __builtin_fmaf(dd, (float)isum, acc[c]);
                        }
                    }
                }
            }
        }
    }
}

// Sum a value over the 8 lanes of a row (lanes 8r..8r+7 of the wave); every lane gets the sum.
__device__ __forceinline__ float row8_sum(float v) {
    v += __shfl_xor(v, 1, 64);
    v += __shfl_xor(v, 2, 64);
    v += __shfl_xor(v, 4, 64);
    return v;
}

__device__ __forceinline__ void stage_grid(const uint8_t* grid, uint32_t* lds_grid) {
    const rsrc_t gr = make_rsrc(grid, 2048);
    for (int i = threadIdx.x; i < 512; i += blockDim.x) lds_grid[i] = ld32(gr, 4u * i);
}

// One pass of up to NC columns.  Grid: ceil(nrows / 32) workgroups of 256 threads.
template <int WT, int NC, bool SUMS>
__global__ __launch_bounds__(kThreads) void gemv_kernel(const uint8_t* __restrict__ w, uint32_t wbytes,
                                                        int nrows, int K, const uint8_t* __restrict__ grid,
                                                        const uint8_t* __restrict__ xq, uint32_t xqbytes,
                                                        int col0, int ncp, float* __restrict__ y, int64_t ldy,
                                                        int32_t* __restrict__ sums) {
    extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
    ActLds act;
    act.kw = K / 4;
    act.nb = K / 32;
    act.q = lds;
    act.d = (float*)(lds + ncp * act.kw);
    uint32_t* lds_grid = (uint32_t*)(act.d + ncp * act.nb);

    const rsrc_t xr = make_rsrc(xq, xqbytes);
    for (int i = threadIdx.x; i < ncp * act.nb; i += blockDim.x) {
        const int c = i / act.nb, b = i - c * act.nb;
        stage_block(xr, (uint32_t)(col0 + c) * act.nb + b, act, c, b);
    }
    if constexpr (WT == kCB3) stage_grid(grid, lds_grid);
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int l8 = lane & 7;
    const int row = blockIdx.x * kRowsPerWG + (threadIdx.x >> 6) * 8 + (lane >> 3);
    const bool row_ok = row < nrows;
    const int rowc = row_ok ? row : nrows - 1;
    const uint32_t rb = row_bytes_dev<WT>(K);
    const rsrc_t wr = make_rsrc(w, wbytes);

    float acc[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[c] = 0.0f;
    lane_partials<WT, NC, SUMS>(wr, (uint32_t)rowc * rb, K, l8, act, ncp, lds_grid, acc,
                                sums + ((int64_t)col0 * nrows + rowc) * act.nb, (int64_t)nrows * act.nb,
                                row_ok);
    if constexpr (!SUMS) {
        float out = 0.0f;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const float s = row8_sum(acc[c]);
            if (l8 == c) out = s;
        }
        if (row_ok && l8 < ncp) y[(int64_t)(col0 + l8) * ldy + row] = out;
    }
}

template <int WT, bool SUMS>
static int launch_gemv(const void* w, uint64_t wbytes, const uint8_t* grid, int64_t nrows, int64_t k,
                       const void* xq, uint64_t xqbytes, int ncols, float* y, int64_t ldy, int32_t* sums,
                       hipStream_t st) {
    const int64_t nb = k / 32;
    const size_t per_col = (size_t)k + (size_t)nb * 4;
    const size_t fixed = WT == kCB3 ? 2048 : 0;
    const size_t lds_cap = 65536;
    int max_pass = (int)((lds_cap - fixed) / per_col);
    if (max_pass > 8) max_pass = 8;
    if (max_pass < 1) return QMM_EUNSUPPORTED;
    const dim3 grid_dim((unsigned)((nrows + kRowsPerWG - 1) / kRowsPerWG));
    for (int c0 = 0; c0 < ncols; c0 += max_pass) {
        const int ncp = ncols - c0 < max_pass ? ncols - c0 : max_pass;
        const size_t lds = per_col * ncp + fixed;
        auto args = [&](auto kern) {
            hipLaunchKernelGGL(kern, grid_dim, dim3(kThreads), lds, st, (const uint8_t*)w, (uint32_t)wbytes,
                               (int)nrows, (int)k, grid, (const uint8_t*)xq, (uint32_t)xqbytes, c0, ncp, y, ldy,
                               sums);
        };
        if (ncp == 1) args(gemv_kernel<WT, 1, SUMS>);
        else if (ncp == 2) args(gemv_kernel<WT, 2, SUMS>);
        else if (ncp <= 4) args(gemv_kernel<WT, 4, SUMS>);
        else args(gemv_kernel<WT, 8, SUMS>);
        const int rc = launch_status();
        if (rc) return rc;
    }
    return QMM_OK;
}

static int check_gemv_args(int wtype, const void* w, const uint8_t* grid, int64_t nrows, int64_t k,
                           const void* xq, int ncols, const void* out, uint64_t* wbytes, uint64_t* xqbytes) {
    if (!valid_wtype(wtype) || !w || !xq || !out || nrows < 1 || ncols < 1 || k < 1) return QMM_EINVAL;
    if (wtype == QMM_CB3 && !grid) return QMM_EINVAL;
    if (k % 32) return QMM_EINVAL;
    if (wtype == QMM_CB3 ? (k % 256) : (k % 64)) return QMM_EUNSUPPORTED;
    if (k > kMaxK) return QMM_EUNSUPPORTED;
    if (!aligned(w, 4) || !aligned(xq, 4) || !aligned(out, 4)) return QMM_EALIGN;
    *wbytes = (uint64_t)nrows * (uint64_t)qmm_row_bytes(wtype, k);
    *xqbytes = (uint64_t)ncols * (uint64_t)(k / 32) * 36u;
    if (*wbytes > kMaxBufferBytes || *xqbytes > kMaxBufferBytes) return QMM_EUNSUPPORTED;
    if ((uint64_t)nrows > 0x7FFFFFFFull) return QMM_EUNSUPPORTED;
    return QMM_OK;
}

}  // namespace qmm

using namespace qmm;

extern "C" int qgemv_dense(int wtype, const void* w, const uint8_t* grid, int64_t nrows, int64_t k,
                           const void* xq, int ncols, float* y, int64_t ldy, void* stream) {
    uint64_t wbytes, xqbytes;
    int rc = check_gemv_args(wtype, w, grid, nrows, k, xq, ncols, y, &wbytes, &xqbytes);
    if (rc) return rc;
    if (ldy < nrows) return QMM_EINVAL;
    const hipStream_t st = as_stream(stream);
    switch (wtype) {
        case QMM_Q8_0: return launch_gemv<kQ8_0, false>(w, wbytes, grid, nrows, k, xq, xqbytes, ncols, y, ldy, nullptr, st);
        case QMM_IQ4_NL: return launch_gemv<kIQ4_NL, false>(w, wbytes, grid, nrows, k, xq, xqbytes, ncols, y, ldy, nullptr, st);
        default: return launch_gemv<kCB3, false>(w, wbytes, grid, nrows, k, xq, xqbytes, ncols, y, ldy, nullptr, st);
    }
}

extern "C" int qmm_debug_block_sums(int wtype, const void* w, const uint8_t* grid, int64_t nrows, int64_t k,
                                    const void* xq, int ncols, int32_t* sums, void* stream) {
    uint64_t wbytes, xqbytes;
    int rc = check_gemv_args(wtype, w, grid, nrows, k, xq, ncols, sums, &wbytes, &xqbytes);
    if (rc) return rc;
    const hipStream_t st = as_stream(stream);
    switch (wtype) {
        case QMM_Q8_0: return launch_gemv<kQ8_0, true>(w, wbytes, grid, nrows, k, xq, xqbytes, ncols, nullptr, 0, sums, st);
        case QMM_IQ4_NL: return launch_gemv<kIQ4_NL, true>(w, wbytes, grid, nrows, k, xq, xqbytes, ncols, nullptr, 0, sums, st);
        default: return launch_gemv<kCB3, true>(w, wbytes, grid, nrows, k, xq, xqbytes, ncols, nullptr, 0, sums, st);
    }
}
