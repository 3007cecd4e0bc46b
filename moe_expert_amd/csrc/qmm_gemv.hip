// qmm_gemv.hip -- multi-column decode GEMV over Q8_0 / IQ4_NL / CB3 weight blocks and q8_1
// activations, for gfx950.
//
// Method [IQ, What it does]: every weight block of the call is loaded and decoded once and
// applied to each column of the pass (1, 2, 4 or 8 columns; passes of 8 beyond 8), with the
// same integer chain and the same float expression for every column, so each column equals a
// one-column call bit for bit.  Activations are staged once per workgroup in LDS as an int8
// plane plus block scales [GP, What changed]; the per-block integer dot is v_dot4_i32_i8;
// a row's partial sums are combined across its 16 lanes with DPP, no barrier.
//
// Mapping (wave64): 16 lanes per row (one DPP row), 4 rows per wave, 8 waves (32 rows) per
// workgroup, two waves per SIMD; passes of 1-2 columns use 16-row workgroups (twice as many),
// rows of more than 96 blocks one row per wave (64 lanes, a DPP row sum and two cross-row
// shuffles).  Lane l of a row takes the 32-value blocks l, l+L, l+2L, ... of its row (L lanes),
// so the lanes of a row read consecutive blocks and every weight byte of the matrix is read
// once per call.  A lane issues the loads of its first chunk of blocks before
// the activation staging and the barrier, so weight latency and staging overlap; longer rows
// are processed in double-buffered chunks.
#include "qmm_gemv.h"

namespace qmm {

template <int WT, bool SUMS, int NC, int U, bool MULTI, int NS, int LPR, int TH>
__global__ __launch_bounds__(TH) void gemv_kernel(const uint8_t* __restrict__ w, uint32_t wbytes, int nrows, int K,
                                                  const uint8_t* __restrict__ grid, const uint8_t* __restrict__ xq,
                                                  uint32_t xqbytes, int col0, int ncp, float* __restrict__ y,
                                                  int64_t ldy, int32_t* __restrict__ sums) {
    extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
    gemv_tile<WT, SUMS, NC, U, MULTI, NS, LPR, TH, NC / 2 + 1>(make_rsrc_dw(w, wbytes), nrows, K, grid,
                                                               make_rsrc(xq, xqbytes), col0, ncp, y, ldy, sums,
                                                               blockIdx.x * (TH / LPR), lds);
}

// Workgroup shapes: LPR lanes per row, TH threads (TH / LPR rows per workgroup).
//   kWide   16 x 512: 32 rows, the default
//   kNarrow 16 x 256: 16 rows, twice the workgroups, for 1-2 column passes
//   kLong   64 x 512:  8 rows, one row per wave, for rows of more than 96 blocks
enum GemvShape { kWide, kNarrow, kLong };

// Pick the kernel instance for a pass of ncp columns, `lb` blocks per lane and `ns` staging
// slots per thread.  Blocks per lane are covered by chunks of 2, 3, 5 or 6 (a chunk longer than
// the lane's count re-reads its last block), double-buffered chunks of 6 beyond 6.
template <int WT, bool SUMS, int NC, int NS, int LPR, int TH, typename F>
static void dispatch_u(int lb, F&& go) {
    if constexpr (SUMS) {
        go(gemv_kernel<WT, SUMS, NC, 6, true, NS, LPR, TH>);
    } else if constexpr (LPR == 64) {
        if (lb <= 2) go(gemv_kernel<WT, SUMS, NC, 2, false, NS, LPR, TH>);
        else if (lb <= 3) go(gemv_kernel<WT, SUMS, NC, 3, false, NS, LPR, TH>);
        else if (lb <= 6) go(gemv_kernel<WT, SUMS, NC, 6, false, NS, LPR, TH>);
        else go(gemv_kernel<WT, SUMS, NC, 6, true, NS, LPR, TH>);
    } else {
        if (lb <= 2) go(gemv_kernel<WT, SUMS, NC, 2, false, NS, LPR, TH>);
        else if (lb <= 5) go(gemv_kernel<WT, SUMS, NC, 5, false, NS, LPR, TH>);
        else if (lb == 6) go(gemv_kernel<WT, SUMS, NC, 6, false, NS, LPR, TH>);
        else go(gemv_kernel<WT, SUMS, NC, 6, true, NS, LPR, TH>);
    }
}
template <int WT, bool SUMS, int NC, int LPR, int TH, typename F>
static void dispatch_ns(int ns, int lb, F&& go) {
    if (ns == 1) dispatch_u<WT, SUMS, NC, 1, LPR, TH>(lb, go);
    else if (ns == 2) dispatch_u<WT, SUMS, NC, 2, LPR, TH>(lb, go);
    else dispatch_u<WT, SUMS, NC, 4, LPR, TH>(lb, go);
}
template <int WT, bool SUMS, int LPR, int TH, typename F>
static void dispatch_nc(int ncp, int ns, int lb, F&& go) {
    if (ncp == 1) dispatch_ns<WT, SUMS, 1, LPR, TH>(ns, lb, go);
    else if (ncp == 2) dispatch_ns<WT, SUMS, 2, LPR, TH>(ns, lb, go);
    else if constexpr (TH == 256) return;  // the narrow shape serves passes of 1-2 columns only
    else if (ncp <= 4) dispatch_ns<WT, SUMS, 4, LPR, TH>(ns, lb, go);
    else dispatch_ns<WT, SUMS, 8, LPR, TH>(ns, lb, go);
}

// The shape of a pass: one wave per row for long rows (enough workgroups and at most a few
// blocks per lane), 16-row workgroups for passes of 1-2 columns (twice the workgroups, half the
// staging per workgroup), 32-row workgroups otherwise.  The block-sum hook keeps the default.
static GemvShape gemv_shape(bool sums, int64_t k, int ncp) {
    if (sums) return kWide;
    if (k / 32 > 96) return kLong;
    return ncp <= 2 && (int64_t)ncp * pow2_ceil(k / 32) <= (int64_t)kStageSlots * 256 ? kNarrow : kWide;
}
static int shape_threads(GemvShape s) { return s == kNarrow ? 256 : 512; }
static int shape_lpr(GemvShape s) { return s == kLong ? 64 : 16; }

template <int WT, bool SUMS>
static int launch_gemv(const void* w, uint64_t wbytes, const uint8_t* grid, int64_t nrows, int64_t k, const void* xq,
                       uint64_t xqbytes, int ncols, float* y, int64_t ldy, int32_t* sums, hipStream_t st) {
    // widest pass the LDS allows, and at most kStageSlots q8_1 blocks staged per thread
    // (numbered with the block count rounded up to a power of two) in a 512-thread shape
    int max_pass = gemv_max_pass(WT, k);
    const int64_t slot_cap = (int64_t)kStageSlots * 512 / pow2_ceil(k / 32);
    if (max_pass > slot_cap) max_pass = (int)slot_cap;
    if (max_pass < 1) return QMM_EUNSUPPORTED;
    for (int c0 = 0; c0 < ncols; c0 += max_pass) {
        const int ncp = ncols - c0 < max_pass ? ncols - c0 : max_pass;
        const GemvShape shape = gemv_shape(SUMS, k, ncp);
        const int th = shape_threads(shape), lpr = shape_lpr(shape);
        const dim3 grid_dim((unsigned)((nrows + th / lpr - 1) / (th / lpr)));
        const size_t lds = gemv_lds_bytes(WT, k, ncp);
        auto go = [&](auto kern) {
            hipLaunchKernelGGL(kern, grid_dim, dim3(th), lds, st, (const uint8_t*)w, (uint32_t)wbytes, (int)nrows,
                               (int)k, grid, (const uint8_t*)xq, (uint32_t)xqbytes, c0, ncp, y, ldy, sums);
        };
        const int ns = stage_slots(k, ncp, th), lb = lane_blocks(k, lpr);
        if (shape == kLong) dispatch_nc<WT, SUMS, 64, 512>(ncp, ns, lb, go);
        else if (shape == kNarrow) dispatch_nc<WT, SUMS, 16, 256>(ncp, ns, lb, go);
        else dispatch_nc<WT, SUMS, 16, 512>(ncp, ns, lb, go);
        const int rc = launch_status();
        if (rc) return rc;
    }
    return QMM_OK;
}

static int check_gemv_args(int wtype, const void* w, const uint8_t* grid, int64_t nrows, int64_t k, const void* xq,
                           int ncols, const void* out, uint64_t* wbytes, uint64_t* xqbytes) {
    if (!valid_wtype(wtype) || !w || !xq || !out || nrows < 1 || ncols < 1 || k < 1) return QMM_EINVAL;
    if (wtype == QMM_CB3 && !grid) return QMM_EINVAL;
    if (k % 32) return QMM_EINVAL;
    if (wtype == QMM_CB3 && k % 256) return QMM_EINVAL;
    if (k > kMaxK) return QMM_EUNSUPPORTED;
    if (!aligned(w, 4) || !aligned(xq, 4) || !aligned(out, 4)) return QMM_EALIGN;
    *wbytes = (uint64_t)nrows * (uint64_t)qmm_row_bytes(wtype, k);
    *xqbytes = (uint64_t)ncols * (uint64_t)(k / 32) * 36u;
    if (*wbytes > kMaxBufferBytes || *xqbytes > kMaxBufferBytes) return QMM_EUNSUPPORTED;
    return QMM_OK;
}

}  // namespace qmm

using namespace qmm;

extern "C" int qgemv_dense(int wtype, const void* w, const uint8_t* grid, int64_t nrows, int64_t k, const void* xq,
                           int ncols, float* y, int64_t ldy, void* stream) {
    uint64_t wbytes, xqbytes;
    const int rc = check_gemv_args(wtype, w, grid, nrows, k, xq, ncols, y, &wbytes, &xqbytes);
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
    const int rc = check_gemv_args(wtype, w, grid, nrows, k, xq, ncols, sums, &wbytes, &xqbytes);
    if (rc) return rc;
    const hipStream_t st = as_stream(stream);
    switch (wtype) {
        case QMM_Q8_0: return launch_gemv<kQ8_0, true>(w, wbytes, grid, nrows, k, xq, xqbytes, ncols, nullptr, 0, sums, st);
        case QMM_IQ4_NL: return launch_gemv<kIQ4_NL, true>(w, wbytes, grid, nrows, k, xq, xqbytes, ncols, nullptr, 0, sums, st);
        default: return launch_gemv<kCB3, true>(w, wbytes, grid, nrows, k, xq, xqbytes, ncols, nullptr, 0, sums, st);
    }
}
