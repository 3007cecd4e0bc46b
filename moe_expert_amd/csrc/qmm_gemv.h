// qmm_gemv.h -- the decode-GEMV row engine shared by the dense GEMV and the grouped-expert
// kernels: per-lane block loads, decode once, apply to every column of the pass.
#pragma once

#include "qmm_device.h"
#include "qmm_host.h"

namespace qmm {

constexpr int kGemvLanesPerRow = 16;  // one DPP row (the default row width)
constexpr int kGemvThreads = 512;     // 8 waves, two per SIMD (the default workgroup)
constexpr int kGemvRowsPerWG = 32;    // 8 waves x 4 rows
constexpr int kGemvChunk = 6;         // blocks per lane whose loads are issued together
constexpr size_t kLdsCap = 65536;     // LDS a workgroup may use

template <int WT>
__host__ __device__ constexpr int row_bytes_dev(int K) {
    return WT == kQ8_0 ? (K / 32) * 34 : WT == kIQ4_NL ? (K / 32) * 18 : (K / 256) * kCB3Bytes;
}

// LDS of a pass of ncp columns: int8 plane + float scales, plus the CB3 codebook.
__host__ __device__ inline size_t gemv_lds_bytes(int wt, int64_t k, int ncp) {
    return (size_t)ncp * ((size_t)k + (size_t)(k / 32) * 4) + (wt == kCB3 ? 2048 : 0);
}
inline int gemv_max_pass(int wt, int64_t k) {
    const size_t per = (size_t)k + (size_t)(k / 32) * 4;
    const size_t fixed = wt == kCB3 ? 2048 : 0;
    if (kLdsCap < fixed + per) return 0;
    const int m = (int)((kLdsCap - fixed) / per);
    return m > 8 ? 8 : m;
}

__device__ __forceinline__ ActLds act_lds_layout(uint32_t* lds, int K, int ncp) {
    ActLds a;
    a.kw = K / 4;
    a.nb = K / 32;
    a.q = lds;
    a.d = (float*)(lds + ncp * a.kw);
    return a;
}
__device__ __forceinline__ uint32_t* act_lds_end(ActLds a, int ncp) { return (uint32_t*)(a.d + ncp * a.nb); }

__device__ __forceinline__ void stage_grid(const uint8_t* grid, uint32_t* lds_grid) {
    const rsrc_t gr = make_rsrc(grid, 2048);
    for (int i = threadIdx.x; i < 512; i += blockDim.x) lds_grid[i] = ld32(gr, 4u * i);
}

// The 512-word codebook staged by a workgroup of TH threads (512 / TH words per thread), split
// into an early load and a late LDS write like the activations.
template <int TH = kGemvThreads>
struct GridStage {
    static_assert(512 % TH == 0 || TH % 512 == 0, "the codebook must split evenly over the workgroup");
    static constexpr int N = TH >= 512 ? 1 : 512 / TH;
    uint32_t v[N];
    // threads past the first 512 of a larger workgroup re-read word tid % 512 and store nothing
    __device__ __forceinline__ void load(const uint8_t* grid) {
#pragma unroll
        for (int i = 0; i < N; ++i) v[i] = ld32(make_rsrc(grid, 2048), 4u * ((threadIdx.x + i * TH) & 511u));
    }
    __device__ __forceinline__ void store(uint32_t* lds_grid) const {
#pragma unroll
        for (int i = 0; i < N; ++i)
            if (TH <= 512 || threadIdx.x < 512) lds_grid[threadIdx.x + i * TH] = v[i];
    }
};

// Activation staging in two halves so that its global loads can be issued before the weight
// loads and its LDS writes after them: a thread stages up to kStageSlots q8_1 blocks, the pass's
// (column, block) pairs being numbered column * 2^ceil(log2(blocks)) + block.
constexpr int kStageSlots = 4;

template <int NS>
struct ActStage {
    uint32_t h[NS];
    u32x4 q0[NS], q1[NS];
    int lsh;   // log2 of the block count rounded up to a power of two
    int last;  // last valid (column, block) slot index

    // Slot index i -> column i >> lsh, block i & (2^lsh - 1); indices past the pass or past a
    // column's blocks are clamped to the pass's last block.  Loads are unconditional so the
    // code stays straight-line.
    __device__ __forceinline__ int slot(int j, const ActLds& act, int ncp) const {
        const int i = (int)threadIdx.x + j * (int)blockDim.x;
        const int c = i >> lsh, b = i & ((1 << lsh) - 1);
        return (c < ncp && b < act.nb) ? i : last;
    }
    __device__ __forceinline__ void setup(const ActLds& act, int ncp) {
        lsh = 32 - __builtin_clz((unsigned)act.nb - 1u);
        if (act.nb == 1) lsh = 0;
        last = ((ncp - 1) << lsh) | (act.nb - 1);
    }
    __device__ __forceinline__ void load_slot(rsrc_t xr, const ActLds& act, int j, int src_col, int i) {
        const uint32_t off = __umul24((uint32_t)(src_col * act.nb + (i & ((1 << lsh) - 1))), 36u);
        h[j] = ld32(xr, off);
        q0[j] = ld128(xr, off + 4);
        q1[j] = ld128(xr, off + 20);
    }
    // Columns col0 .. col0 + ncp - 1 of the activations.
    __device__ __forceinline__ void load(rsrc_t xr, const ActLds& act, int col0, int ncp) {
        setup(act, ncp);
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            const int i = slot(j, act, ncp);
            load_slot(xr, act, j, col0 + (i >> lsh), i);
        }
    }
    // Pass column c taken from activation column entry_col[c0 + c]; a column outside
    // [0, ncols) reads the zeros past the end of the activations.
    __device__ __forceinline__ void load_entries(rsrc_t xr, const ActLds& act, int ncp, const int32_t* entry_col, int c0,
                                                 int ncols) {
        setup(act, ncp);
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            const int i = slot(j, act, ncp);
            int col = entry_col[c0 + (i >> lsh)];
            col = (col >= 0 && col < ncols) ? col : ncols;
            load_slot(xr, act, j, col, i);
        }
    }
    // Unconditional too: a slot past the pass rewrites the pass's last block with the same
    // bytes (identical values, so the overlapping writes are benign).  Keeping the stores
    // unconditional keeps the loads where they are written (otherwise the compiler sinks them
    // into the store's branch, behind the weight loads).
    __device__ __forceinline__ void store(const ActLds& act, int ncp) {
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            const int i = slot(j, act, ncp);
            const int c = i >> lsh, b = i & ((1 << lsh) - 1);
            uint32_t* dst = act.q + __umul24((uint32_t)c, (uint32_t)act.kw) + b * 8;
            *(u32x4*)dst = q0[j];
            *(u32x4*)(dst + 4) = q1[j];
            act.d[__umul24((uint32_t)c, (uint32_t)act.nb) + b] = h2f(h[j]);
        }
    }
};

// One lane's share of one row of LPR lanes: blocks s = l + LPR i, i = 0, 1, ...  U blocks are
// loaded per chunk; MULTI = the row has more than U blocks per lane (double-buffered chunks),
// otherwise U is at least the lane's block count.  Loads are unconditional (a block past the
// row is read at the row's last block and not used), so the code between the loads and their
// uses stays straight-line and each use waits only for its own load.  NCMIN: columns every pass
// of this instance has (NC / 2 + 1 for the dense GEMV, whose NC is the smallest of 1, 2, 4, 8
// that holds the pass; 1 where passes may be narrower).
template <int WT, int NC, bool SUMS, int U, bool MULTI, int LPR = kGemvLanesPerRow, int NCMIN = 1>
struct RowEngine {
    static constexpr int RAW = Unit<WT>::RAW;
    rsrc_t wr;
    uint32_t row_off;
    int nunits, niter, l16;
    uint32_t A[U][RAW], B[MULTI ? U : 1][RAW];
    IQ4Consts kc;

    __device__ __forceinline__ RowEngine(rsrc_t wr_, uint32_t row_off_, int K, int l_)
        : wr(wr_), row_off(row_off_), nunits(K / 32), niter((K / 32 + LPR - 1) / LPR), l16(l_) {}

    __device__ __forceinline__ uint32_t unit_off(int s) const {
        // 32-bit multiply-add (a 64-bit one would tie a dead high half to a pending load)
        if constexpr (WT == kCB3) return row_off + __umul24((uint32_t)(s >> 3), (uint32_t)kCB3Bytes);
        else return row_off + __umul24((uint32_t)s, (uint32_t)Unit<WT>::BYTES);
    }

    template <int N>
    __device__ __forceinline__ void load(uint32_t (&buf)[N][RAW], int i0) {
#pragma unroll
        for (int u = 0; u < N; ++u) {
            int s = l16 + LPR * (i0 + u);
            s = s < nunits ? s : nunits - 1;
            if constexpr (WT == kCB3) Unit<WT>::load(wr, unit_off(s), s & 7, buf[u]);
            else Unit<WT>::load(wr, unit_off(s), buf[u]);
        }
    }

    __device__ __forceinline__ void load_first() { load(A, 0); }

    template <int N>
    __device__ __forceinline__ void compute(const uint32_t (&buf)[N][RAW], int i0, const ActLds& act, int ncp,
                                            const uint32_t* grid, float (&acc)[NC], int32_t* srow, int64_t scol,
                                            bool row_ok) {
#pragma unroll
        for (int u = 0; u < N; ++u) {
            const int s = l16 + LPR * (i0 + u);
            if (s < nunits) {
                uint32_t W[8];
                uint32_t dw;
                int mult;
                if constexpr (WT == kCB3) Unit<WT>::decode(buf[u], unit_off(s), s & 7, grid, W, dw, mult);
                else Unit<WT>::decode(buf[u], unit_off(s), W, dw, mult, kc);
                const float dwf = h2f(dw);
                // Columns below NCMIN always exist in the pass and run straight-line (their LDS
                // reads can be issued ahead); the others only when the pass has them.
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    if (c >= NCMIN && c >= ncp) continue;
                    const uint32_t cc = (uint32_t)c;
                    const uint32_t* a = act.q + __umul24(cc, (uint32_t)act.kw) + s * 8;
                    const u32x4 a0 = *(const u32x4*)a;
                    const u32x4 a1 = *(const u32x4*)(a + 4);
                    int v = dot4(W[0], a0.x, 0);
                    v = dot4(W[1], a0.y, v);
                    v = dot4(W[2], a0.z, v);
                    v = dot4(W[3], a0.w, v);
                    v = dot4(W[4], a1.x, v);
                    v = dot4(W[5], a1.y, v);
                    v = dot4(W[6], a1.z, v);
                    v = dot4(W[7], a1.w, v);
                    // |v| < 2^23 and mult <= 31: the 24-bit multiply is exact
                    const int isum = WT == kCB3 ? __mul24(v, mult) : v;
                    if constexpr (SUMS) {
                        if (row_ok) srow[c * scol + s] = isum;
                    } else {
                        const float dd = dwf * act.d[__umul24(cc, (uint32_t)act.nb) + s];
                        acc[c] = __builtin_fmaf(dd, (float)isum, acc[c]);
                    }
                }
            }
        }
    }

    // All of the lane's blocks; the first chunk must already be loaded (load_first).
    __device__ __forceinline__ void run(const ActLds& act, int ncp, const uint32_t* grid, float (&acc)[NC],
                                        int32_t* srow, int64_t scol, bool row_ok) {
        if constexpr (!MULTI) {
            compute(A, 0, act, ncp, grid, acc, srow, scol, row_ok);
        } else {
            for (int i0 = 0; i0 < niter; i0 += 2 * U) {
                const bool more = i0 + U < niter;
                if (more) load(B, i0 + U);
                compute(A, i0, act, ncp, grid, acc, srow, scol, row_ok);
                if (more) {
                    if (i0 + 2 * U < niter) load(A, i0 + 2 * U);
                    compute(B, i0 + U, act, ncp, grid, acc, srow, scol, row_ok);
                }
            }
        }
    }
};

// Sum over the LPR lanes of a row (16: one DPP row; 64: the wave); every lane of the row gets
// the same value, added in the same order for every column.
template <int LPR>
__device__ __forceinline__ float row_sum(float v) {
    v = row16_sum(v);
    if constexpr (LPR == 64) {
        v += __shfl_xor(v, 16, 64);
        v += __shfl_xor(v, 32, 64);
    }
    return v;
}

// One workgroup's TH / 64 * (64 / LPR) rows starting at row0 of a decode GEMV pass: columns
// [col0, col0 + ncp) of the q8_1 activations behind `xr` (column c is q8_1 blocks c*K/32 ...),
// results to y[(col0 + c) * ldy + row] (or the per-block integer sums, SUMS).  LPR lanes per
// row (16 or 64).  Order of work: activation loads, then this lane's weight loads, then the
// activation LDS writes (they wait only for the activation loads), barrier, decode + apply as
// the weights arrive, cross-lane row sums.
template <int WT, bool SUMS, int NC, int U, bool MULTI, int NS, int LPR = kGemvLanesPerRow, int TH = kGemvThreads,
          int NCMIN = 1>
__device__ __forceinline__ void gemv_tile(rsrc_t wr, int nrows, int K, const uint8_t* grid, rsrc_t xr, int col0, int ncp,
                                          float* y, int64_t ldy, int32_t* sums, int row0, uint32_t* lds) {
    static_assert(LPR == 16 || LPR == 64, "a row is one DPP row or one wave");
    ActLds act = act_lds_layout(lds, K, ncp);
    uint32_t* lds_grid = act_lds_end(act, ncp);

    const int lane = threadIdx.x & 63;
    const int l16 = lane & (LPR - 1);
    const int row = row0 + (threadIdx.x >> 6) * (64 / LPR) + lane / LPR;
    const bool row_ok = row < nrows;
    const int rowc = row_ok ? row : nrows - 1;
    const uint32_t row_off = (uint32_t)rowc * (uint32_t)row_bytes_dev<WT>(K);

    ActStage<NS> stage;
    stage.load(xr, act, col0, ncp);
    GridStage<TH> gstage;
    if constexpr (WT == kCB3) gstage.load(grid);
    __builtin_amdgcn_sched_barrier(0);
    RowEngine<WT, NC, SUMS, U, MULTI, LPR, NCMIN> eng(wr, row_off, K, l16);
    eng.load_first();
    __builtin_amdgcn_sched_barrier(0);
    stage.store(act, ncp);
    if constexpr (WT == kCB3) gstage.store(lds_grid);
    __syncthreads();

    float acc[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[c] = 0.0f;
    int32_t* srow = nullptr;
    int64_t scol = 0;
    if constexpr (SUMS) {
        srow = sums + ((int64_t)col0 * nrows + rowc) * act.nb;
        scol = (int64_t)nrows * act.nb;
    }
    eng.run(act, ncp, lds_grid, acc, srow, scol, row_ok);
    if constexpr (!SUMS) {
        float out = 0.0f;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const float s = row_sum<LPR>(acc[c]);
            if (l16 == c) out = s;
        }
        if (row_ok && l16 < ncp) y[(int64_t)(col0 + l16) * ldy + row] = out;
    }
}

// Blocks per lane of a row of k values (lpr lanes per row).
inline int lane_blocks(int64_t k, int lpr = kGemvLanesPerRow) { return (int)((k / 32 + lpr - 1) / lpr); }

// Staging slots per thread for a pass of ncp columns of k values.
inline int stage_slots(int64_t k, int ncp, int threads) {
    const int64_t n = (int64_t)ncp * pow2_ceil(k / 32);
    return n <= threads ? 1 : n <= 2 * threads ? 2 : 4;
}

}  // namespace qmm
