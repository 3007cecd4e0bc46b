// qmm_gemv.hip -- multi-column decode GEMV over Q8_0 / IQ4_NL / CB3 weight blocks and q8_1
// activations, for gfx950.
//
// Method [IQ, What it does]: every weight block of the call is loaded and decoded once and
// applied to each column of the pass (1, 2, 4 or 8 columns; passes of 8 beyond 8), with the
// same integer chain and the same float expression for every column, so each column equals a
// one-column call bit for bit.  Activations are staged once per workgroup in LDS as int8
// values plus block scales [GP, What changed], in the order the lanes read them; the
// per-block integer dot is v_dot4_i32_i8; a row's partial sums are combined across its lanes
// with DPP, no barrier.
//
// Mapping (wave64): 16 lanes per row (one DPP row), 4 rows per wave, 4 waves (16 rows) per
// workgroup, two workgroups per CU (32-row workgroups of 8 waves where a smaller one cannot
// stage the pass); rows of more than 96 blocks one row per wave (64 lanes, a DPP row sum and
// two cross-row shuffles).  Lane l of a row takes the 32-value blocks l, l+L, l+2L, ... of its row (L lanes),
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
    gemv_tile<WT, SUMS, NC, U, MULTI, NS, LPR, TH>(make_rsrc_dw(w, wbytes), nrows, K, grid, make_rsrc(xq, xqbytes),
                                                   xqbytes, col0, ncp, y, ldy, sums, blockIdx.x * (TH / LPR), lds);
}

// NC fp32 columns, quantized to q8_1 by every workgroup for itself (16 lanes per row, one slot).
template <int WT, int U, int NC, int TH>
__global__ __launch_bounds__(TH) void gemv_f32_kernel(const uint8_t* __restrict__ w, uint32_t wbytes, int nrows, int K,
                                                      const uint8_t* __restrict__ grid, const float* __restrict__ x,
                                                      uint32_t xbytes, float* __restrict__ y, int64_t ldy) {
    extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
    gemv_tile<WT, false, NC, U, false, 1, 16, TH, false, 100, true>(make_rsrc_dw(w, wbytes), nrows, K, grid,
                                                                    make_rsrc(x, xbytes), xbytes, 0, NC, y, ldy,
                                                                    nullptr, blockIdx.x * (TH / 16), lds);
}

// Workgroup shapes: LPR lanes per row, TH threads (TH / LPR rows per workgroup).
//   kWide   16 x 512: 32 rows, where 256 threads cannot stage the pass (and the block-sum hook)
//   kNarrow 16 x 256: 16 rows, the default
//   kLong   64 x 512:  8 rows, one row per wave, for rows of more than 96 blocks
enum GemvShape { kWide, kNarrow, kLong };

// Pick the kernel instance for a pass of NC columns, the chunk `ch` and `ns` staging slots per
// thread (the same chunk choice as gemv_chunk).
template <int WT, bool SUMS, int NC, int NS, int LPR, int TH, typename F>
static void dispatch_u(Chunk ch, F&& go) {
    if constexpr (SUMS) {
        go(gemv_kernel<WT, SUMS, NC, 6, true, NS, LPR, TH>);
    } else {
        if (ch.multi) go(gemv_kernel<WT, SUMS, NC, 6, true, NS, LPR, TH>);
        else if (ch.u == 2) go(gemv_kernel<WT, SUMS, NC, 2, false, NS, LPR, TH>);
        else if (LPR == 64 && ch.u == 3) go(gemv_kernel<WT, SUMS, NC, 3, false, NS, LPR, TH>);
        else if (LPR != 64 && ch.u == 5) go(gemv_kernel<WT, SUMS, NC, 5, false, NS, LPR, TH>);
        else go(gemv_kernel<WT, SUMS, NC, 6, false, NS, LPR, TH>);
    }
}
template <int WT, bool SUMS, int NC, int LPR, int TH, typename F>
static void dispatch_ns(int ns, Chunk ch, F&& go) {
    if (ns == 1) dispatch_u<WT, SUMS, NC, 1, LPR, TH>(ch, go);
    else if (ns == 2) dispatch_u<WT, SUMS, NC, 2, LPR, TH>(ch, go);
    else if (ns == 3) dispatch_u<WT, SUMS, NC, 3, LPR, TH>(ch, go);
    else dispatch_u<WT, SUMS, NC, 4, LPR, TH>(ch, go);
}
template <int WT, bool SUMS, int LPR, int TH, typename F>
static void dispatch_nc(int nc, int ns, Chunk ch, F&& go) {
    if (nc == 1) dispatch_ns<WT, SUMS, 1, LPR, TH>(ns, ch, go);
    else if (nc == 2) dispatch_ns<WT, SUMS, 2, LPR, TH>(ns, ch, go);
    else if (nc == 4) dispatch_ns<WT, SUMS, 4, LPR, TH>(ns, ch, go);
    else dispatch_ns<WT, SUMS, 8, LPR, TH>(ns, ch, go);
}

// Lanes per row: one wave per row for rows of more than 96 blocks (not for the block-sum hook).
static int pass_lpr(bool sums, int64_t k) { return !sums && k / 32 > 96 ? 64 : 16; }
static Chunk pass_chunk(bool sums, int64_t k) {
    const int lpr = pass_lpr(sums, k);
    return gemv_chunk(lane_blocks(k, lpr), lpr, sums);
}

// Whether a workgroup of `th` threads can stage a pass of nc columns within the LDS budget.
static bool shape_fits(int wt, int64_t k, int nc, int th, int lpr, Chunk ch) {
    return stage_slots(k, nc, th, lpr, ch.u) != 0 && gemv_lds_bytes(wt, k, nc, lpr, ch.u, th) <= kLdsCap;
}

// The shape of a pass: one wave per row for long rows (enough workgroups and at most a few
// blocks per lane), otherwise 16-row workgroups where a 256-thread workgroup can stage the pass
// (twice the workgroups of the 32-row shape: two per CU progress independently and each
// barrier spans 4 waves), 32-row workgroups beyond.  The block-sum hook keeps the default.
static GemvShape gemv_shape(int wt, bool sums, int64_t k, int ncp) {
    if (sums) return kWide;
    if (pass_lpr(sums, k) == 64) return kLong;
    return shape_fits(wt, k, (int)pow2_ceil(ncp), 256, 16, pass_chunk(sums, k)) ? kNarrow : kWide;
}
static int shape_threads(GemvShape s) { return s == kNarrow ? 256 : 512; }

// Widest pass (1, 2, 4 or 8 columns) that one of the shapes can stage.
static int gemv_max_pass(int wt, bool sums, int64_t k) {
    const int lpr = pass_lpr(sums, k);
    const Chunk ch = pass_chunk(sums, k);
    for (int nc = 8; nc >= 1; nc /= 2)
        if (shape_fits(wt, k, nc, 512, lpr, ch) || (!sums && lpr == 16 && shape_fits(wt, k, nc, 256, lpr, ch))) return nc;
    return 0;
}

template <int WT, bool SUMS>
static int launch_gemv(const void* w, uint64_t wbytes, const uint8_t* grid, int64_t nrows, int64_t k, const void* xq,
                       uint64_t xqbytes, int ncols, float* y, int64_t ldy, int32_t* sums, hipStream_t st) {
    const int max_pass = gemv_max_pass(WT, SUMS, k);
    if (max_pass < 1) return QMM_EUNSUPPORTED;
    const int lpr = pass_lpr(SUMS, k);
    const Chunk ch = pass_chunk(SUMS, k);
    for (int c0 = 0; c0 < ncols; c0 += max_pass) {
        const int ncp = ncols - c0 < max_pass ? ncols - c0 : max_pass;
        const int nc = (int)pow2_ceil(ncp);
        const GemvShape shape = gemv_shape(WT, SUMS, k, ncp);
        const int th = shape_threads(shape);
        const dim3 grid_dim((unsigned)((nrows + th / lpr - 1) / (th / lpr)));
        const size_t lds = gemv_lds_bytes(WT, k, nc, lpr, ch.u, th);
        auto go = [&](auto kern) {
            hipLaunchKernelGGL(kern, grid_dim, dim3(th), lds, st, (const uint8_t*)w, (uint32_t)wbytes, (int)nrows,
                               (int)k, grid, (const uint8_t*)xq, (uint32_t)xqbytes, c0, ncp, y, ldy, sums);
        };
        const int ns = stage_slots(k, nc, th, lpr, ch.u);
        if (shape == kLong) dispatch_nc<WT, SUMS, 64, 512>(nc, ns, ch, go);
        else if (shape == kNarrow) dispatch_nc<WT, SUMS, 16, 256>(nc, ns, ch, go);
        else dispatch_nc<WT, SUMS, 16, 512>(nc, ns, ch, go);
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
    if (*wbytes > kMaxBufferBytes || *xqbytes > kMaxActBytes) return QMM_EUNSUPPORTED;
    return QMM_OK;
}

// The fused GEMV on 1, 2 or 4 fp32 columns: rows of at most 96 blocks (16 lanes per row,
// chunks of 2, 5 or 6 blocks), in 32-row workgroups of 512 threads with one staging slot: each
// workgroup quantizes the columns in NC * 96 / 64 passes of 64 blocks, for twice the rows of a
// 256-thread workgroup.
template <int WT>
static int launch_gemv_f32(const void* w, uint64_t wbytes, const uint8_t* grid, int64_t nrows, int64_t k,
                           const float* x, int ncols, float* y, int64_t ldy, hipStream_t st) {
    constexpr int TH = 512;
    const Chunk ch = pass_chunk(false, k);
    if (pass_lpr(false, k) != 16 || ch.multi || k / 32 > 96) return QMM_EUNSUPPORTED;
    if (ncols != 1 && ncols != 2 && ncols != 4) return QMM_EUNSUPPORTED;
    if (stage_slots(k, ncols, TH, 16, ch.u) != 1 || gemv_lds_bytes(WT, k, ncols, 16, ch.u, TH) > kLdsCap)
        return QMM_EUNSUPPORTED;
    const dim3 grid_dim((unsigned)((nrows + TH / 16 - 1) / (TH / 16)));
    const size_t lds = gemv_lds_bytes(WT, k, ncols, 16, ch.u, TH);
    const uint32_t xbytes = (uint32_t)(ncols * k * 4);
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid_dim, dim3(TH), lds, st, (const uint8_t*)w, (uint32_t)wbytes, (int)nrows, (int)k,
                           grid, x, xbytes, y, ldy);
    };
    auto by_u = [&](auto nc_c) {
        constexpr int NC = decltype(nc_c)::value;
        if (ch.u == 2) go(gemv_f32_kernel<WT, 2, NC, TH>);
        else if (ch.u == 5) go(gemv_f32_kernel<WT, 5, NC, TH>);
        else go(gemv_f32_kernel<WT, 6, NC, TH>);
    };
    if (ncols == 1) by_u(std::integral_constant<int, 1>{});
    else if (ncols == 2) by_u(std::integral_constant<int, 2>{});
    else by_u(std::integral_constant<int, 4>{});
    return launch_status();
}

// Repack into planes: one thread per block of a row copies the block's factor bytes to its
// place in the tile's factor area and its scale to the tile's scale area (a one-time layout
// change: byte copies, no arithmetic).
template <int BB>
__global__ __launch_bounds__(256) void pack_planes_kernel(const uint8_t* __restrict__ w, uint8_t* __restrict__ out,
                                                          int64_t nrows, int nb) {
    constexpr int FB = BB - 2;
    const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (g >= nrows * nb) return;
    const int64_t r = g / nb;
    const int b = (int)(g - r * nb);
    const int t0 = b & ~15, n = nb - t0 < 16 ? nb - t0 : 16, i = b - t0;
    const uint8_t* blk = w + (r * nb + b) * BB;
    uint8_t* tile = out + (r * nb + t0) * BB;
#pragma unroll
    for (int j = 0; j < FB; ++j) tile[i * FB + j] = blk[2 + j];
    tile[n * FB + 2 * i] = blk[0];
    tile[n * FB + 2 * i + 1] = blk[1];
}

static int check_planes_args(int wtype, const void* src, const void* dst, int64_t nrows, int64_t k) {
    if ((wtype != QMM_Q8_0 && wtype != QMM_IQ4_NL) || !src || !dst || nrows < 1 || k < 32 || k % 32)
        return QMM_EINVAL;
    if ((uint64_t)nrows * (uint64_t)qmm_row_bytes(wtype, k) > ((uint64_t)1 << 40)) return QMM_EUNSUPPORTED;
    return QMM_OK;
}

static int launch_pack(int wtype, const void* w, void* out, int64_t nrows, int64_t k, hipStream_t st) {
    const int nb = (int)(k / 32);
    const dim3 g((unsigned)((nrows * nb + 255) / 256));
    if (wtype == QMM_Q8_0)
        hipLaunchKernelGGL(pack_planes_kernel<34>, g, dim3(256), 0, st, (const uint8_t*)w, (uint8_t*)out, nrows, nb);
    else
        hipLaunchKernelGGL(pack_planes_kernel<18>, g, dim3(256), 0, st, (const uint8_t*)w, (uint8_t*)out, nrows, nb);
    return launch_status();
}

}  // namespace qmm

using namespace qmm;

extern "C" int qmm_pack_planes(int wtype, const void* w, int64_t nrows, int64_t k, void* planes, void* stream) {
    const int rc = check_planes_args(wtype, w, planes, nrows, k);
    if (rc) return rc;
    if (k > ((int64_t)1 << 24) || nrows * (k / 32) > ((int64_t)1 << 40)) return QMM_EUNSUPPORTED;
    return launch_pack(wtype, w, planes, nrows, k, as_stream(stream));
}

extern "C" int qmm_planes_alloc(int wtype, const void* w, int64_t nrows, int64_t k, void** planes, void* stream) {
    if (!planes) return QMM_EINVAL;
    *planes = nullptr;
    const int rc = check_planes_args(wtype, w, w, nrows, k);
    if (rc) return rc;
    void* p = nullptr;
    if (hipMalloc(&p, (size_t)nrows * (size_t)qmm_row_bytes(wtype, k)) != hipSuccess) return QMM_EHIP;
    const int prc = qmm_pack_planes(wtype, w, nrows, k, p, stream);
    if (prc) {
        (void)hipFree(p);
        return prc;
    }
    *planes = p;
    return QMM_OK;
}

extern "C" int qmm_planes_release(void* planes) {
    if (!planes) return QMM_OK;
    return hipFree(planes) == hipSuccess ? QMM_OK : QMM_EHIP;
}

extern "C" int qgemv_planes(int wtype, const void* planes, int64_t nrows, int64_t k, const void* xq, int ncols, float* y,
                            int64_t ldy, void* stream) {
    if (wtype != QMM_Q8_0 && wtype != QMM_IQ4_NL) return QMM_EINVAL;
    uint64_t wbytes, xqbytes;
    const int rc = check_gemv_args(wtype, planes, nullptr, nrows, k, xq, ncols, y, &wbytes, &xqbytes);
    if (rc) return rc;
    if (ldy < nrows) return QMM_EINVAL;
    if (k % 512) return QMM_EUNSUPPORTED;       // rows of whole 16-block tiles
    if (!aligned(planes, 16)) return QMM_EALIGN;
    const hipStream_t st = as_stream(stream);
    if (wtype == QMM_Q8_0)
        return launch_gemv<kQ8_0P, false>(planes, wbytes, nullptr, nrows, k, xq, xqbytes, ncols, y, ldy, nullptr, st);
    return launch_gemv<kIQ4_NLP, false>(planes, wbytes, nullptr, nrows, k, xq, xqbytes, ncols, y, ldy, nullptr, st);
}

extern "C" int qgemv_dense_f32(int wtype, const void* w, const uint8_t* grid, int64_t nrows, int64_t k, const float* x,
                               int ncols, float* y, int64_t ldy, void* stream) {
    uint64_t wbytes, xqbytes;
    // (the shape and weight checks of the q8_1 GEMV; the columns are at most 4 x 3072 fp32 values)
    const int rc = check_gemv_args(wtype, w, grid, nrows, k, x, ncols, y, &wbytes, &xqbytes);
    if (rc) return rc;
    if (ldy < nrows) return QMM_EINVAL;
    const hipStream_t st = as_stream(stream);
    switch (wtype) {
        case QMM_Q8_0: return launch_gemv_f32<kQ8_0>(w, wbytes, grid, nrows, k, x, ncols, y, ldy, st);
        case QMM_IQ4_NL: return launch_gemv_f32<kIQ4_NL>(w, wbytes, grid, nrows, k, x, ncols, y, ldy, st);
        default: return launch_gemv_f32<kCB3>(w, wbytes, grid, nrows, k, x, ncols, y, ldy, st);
    }
}

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
