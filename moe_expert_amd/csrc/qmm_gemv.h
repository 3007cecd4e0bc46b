// qmm_gemv.h -- the decode-GEMV row engine shared by the dense GEMV and the grouped-expert
// kernels: per-lane block loads, decode once, apply to every column of the pass.
#pragma once

#include "qmm_device.h"
#include "qmm_host.h"

namespace qmm {

constexpr int kGemvLanesPerRow = 16;  // one DPP row (the default row width)
constexpr int kGemvThreads = 512;     // 8 waves, two per SIMD (the default workgroup)
constexpr int kGemvRowsPerWG = 32;    // 8 waves x 4 rows
constexpr size_t kLdsCap = 65536;     // LDS a workgroup may use
constexpr int kStageSlots = 4;        // most q8_1 blocks one thread stages

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int WT>
__host__ __device__ constexpr int row_bytes_dev(int K) {
    return (WT == kQ8_0 || WT == kQ8_0P)     ? (K / 32) * 34
           : (WT == kIQ4_NL || WT == kIQ4_NLP) ? (K / 32) * 18
           : WT == kF16                        ? K * 2
                                               : (K / 256) * kCB3Bytes;
}

// ------------------------------------------------------------------ activations in LDS
//
// The q8_1 columns of a pass are staged once per workgroup as int8 values plus float block
// scales [GP, What changed], in the order the readers take them.  Lane l of a row of L lanes
// takes the blocks s = l + L i of its row, i = 0, 1, ... ("slots"); a kernel instance of pass
// width NC lays slot i of column c out as
//   int8   half h (16 bytes) of block l + L i  at  ((i NC + c) 2 + h) 16 L + 16 l
//   scale  of block l + L i                     at  S + ((i NC/G + c/G) L + l) 4 G + 4 (c mod G)
// with G = min(NC, 4) and S the size of the int8 area.  A lane then reads every column of a
// slot at compile-time offsets from one address, and the L lanes of a row read 16 L
// consecutive bytes per instruction (no bank conflicts; the rows of a wave read the same
// bytes).  The slot count is the lane's block count rounded up to the chunk U the kernel loads
// at a time, and blocks past k/32 hold zeros, so every slot a lane computes is defined.

// Slots (blocks per lane) of a row of k values over lpr lanes.
__host__ __device__ inline int lane_blocks(int64_t k, int lpr) { return (int)((k / 32 + lpr - 1) / lpr); }
// Slots held in LDS: the lane's blocks rounded up to whole chunks of u.
__host__ __device__ inline int lds_slots(int64_t k, int lpr, int u) {
    const int n = lane_blocks(k, lpr);
    return (n + u - 1) / u * u;
}
// Staging slots per thread for a pass of nc columns (the kernel's pass width) in a workgroup of
// `threads`: the lanes' slots, for every column, spread over the threads; 0 when more than
// kStageSlots would be needed (or the workgroup is narrower than a slot of the pass).
__host__ __device__ inline int stage_slots(int64_t k, int nc, int threads, int lpr, int u) {
    if (threads % (nc * lpr) != 0) return 0;
    const int64_t n = ((int64_t)lds_slots(k, lpr, u) * lpr * nc + threads - 1) / threads;
    return n <= kStageSlots ? (int)n : 0;
}
// The area holds every q8_1 block the threads stage: slots x threads blocks of 36 bytes.
__host__ __device__ inline size_t act_lds_bytes(int64_t k, int nc, int lpr, int u, int threads) {
    return (size_t)stage_slots(k, nc, threads, lpr, u) * (size_t)threads * 36u;
}
// LDS of a pass: activations, plus the CB3 codebook.
__host__ __device__ inline size_t gemv_lds_bytes(int wt, int64_t k, int nc, int lpr, int u, int threads) {
    return act_lds_bytes(k, nc, lpr, u, threads) + (wt == kCB3 ? 2048 : 0);
}

struct ActLds {
    uint8_t* base;   // start of the area
    int nb;          // q8_1 blocks per column (k/32)
    uint32_t dbyte;  // byte offset of the scales
};
template <int NC, int NS, int TH>
__device__ __forceinline__ ActLds act_lds_layout(uint32_t* lds, int K) {
    ActLds a;
    a.base = (uint8_t*)lds;
    a.nb = K / 32;
    a.dbyte = (uint32_t)(NS * TH * 32);
    return a;
}
template <int NS, int TH>
__device__ __forceinline__ uint32_t* act_lds_end(const ActLds& a) {
    return (uint32_t*)(a.base + NS * TH * 36);
}

// A lane's view of the area: its int8 and scale addresses of slot 0, column 0.
struct ActView {
    const uint8_t* q;
    const uint8_t* d;
};
template <int NC>
__device__ __forceinline__ ActView act_view(const ActLds& a, int l) {
    constexpr int G = NC >= 4 ? 4 : NC;
    return ActView{a.base + 16 * l, a.base + a.dbyte + 4 * G * l};
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
// loads and its LDS writes after them.  The area's q8_1 blocks ("pairs": a column and a block)
// are numbered in LDS order, p = (slot NC + column) L + lane, and thread t stages pairs
// t, t + TH, ... (NS of them).  TH is a multiple of NC L, so a thread keeps its column and lane
// in every slot it stages and its pairs lie a constant number of slots apart: their sources and
// destinations differ by constants.  A pair of a column past the pass or of a block past the row
// reads from `zero_off`, at or past the end of the buffer, where the hardware returns zeros.
template <int NS, int NC, int LPR, int TH>
struct ActStage {
    static constexpr int G = NC >= 4 ? 4 : NC;
    static constexpr int kLogL = LPR == 64 ? 6 : 4;
    static constexpr int kLogN = NC == 8 ? 3 : NC == 4 ? 2 : NC == 2 ? 1 : 0;
    static_assert((1 << kLogL) == LPR && (1 << kLogN) == NC, "power-of-two row and pass widths");
    static_assert(TH % (NC * LPR) == 0, "the workgroup covers whole slots");
    static constexpr int kStep = TH / (NC * LPR) * LPR;  // blocks between a thread's pairs
    uint32_t h[NS];
    u32x4 q0[NS], q1[NS];

    __device__ __forceinline__ static int col() { return ((int)threadIdx.x >> kLogL) & (NC - 1); }
    __device__ __forceinline__ static int block0() {
        return (((int)threadIdx.x >> (kLogL + kLogN)) << kLogL) | ((int)threadIdx.x & (LPR - 1));
    }
    // q8_1 block `base` of the buffer and the blocks kStep, 2 kStep, ... after it (pair j is
    // block b0 + j kStep of its column, read when ok and b0 + j kStep < nb).  A full 32-bit
    // multiply: buffers of up to kMaxActBytes hold more than 2^24 blocks.
    __device__ __forceinline__ void load_blocks(rsrc_t xr, const ActLds& act, uint32_t base, int b0, bool ok,
                                                uint32_t zero_off) {
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            const uint32_t off = (ok && b0 + j * kStep < act.nb) ? base * 36u + 36u * kStep * j : zero_off;
            h[j] = ld32(xr, off);
            q0[j] = ld128(xr, off + 4);
            q1[j] = ld128(xr, off + 20);
        }
    }
    // Columns col0 .. col0 + ncp - 1 of the activations (zero_off: the buffer's size).
    __device__ __forceinline__ void load(rsrc_t xr, const ActLds& act, int col0, int ncp, uint32_t zero_off) {
        const int c = col(), b0 = block0();
        load_blocks(xr, act, (uint32_t)((col0 + c) * act.nb + b0), b0, c < ncp, zero_off);
    }
    // Pass column c taken from activation column entry_col[c0 + c]; a column outside
    // [0, ncols) reads zeros as well (zero_off: the buffer's size).  The pass's entry indices
    // are read as uniform (scalar) loads and picked per lane.
    __device__ __forceinline__ void load_entries(rsrc_t xr, const ActLds& act, int ncp, const int32_t* entry_col, int c0,
                                                 int ncols, uint32_t zero_off) {
        const int c = col(), b0 = block0();
        int src = 0;
#pragma unroll
        for (int k = 0; k < NC; ++k) {
            const int e = entry_col[c0 + (k < ncp ? k : 0)];
            src = c == k ? e : src;
        }
        const bool ok = c < ncp && src >= 0 && src < ncols;
        load_blocks(xr, act, (uint32_t)((ok ? src : 0) * act.nb + b0), b0, ok, zero_off);
    }
    // A use of every loaded value (on a path that needs none of them, so that the loads are not
    // moved onto the other paths).
    __device__ __forceinline__ void keep() const {
#pragma unroll
        for (int j = 0; j < NS; ++j) asm volatile("" ::"v"(h[j]), "v"(q0[j]), "v"(q1[j]));
    }
    // LDS addresses of the first pair of thread t: its int8 values, (si NC + c) 32 L + 16 l, and
    // its scale (the next pairs lie 32 TH and 4 TH bytes on).
    __device__ __forceinline__ static uint8_t* q_at(const ActLds& act, uint32_t t) {
        return act.base + 16u * (t + (t & ~(uint32_t)(LPR - 1)));
    }
    __device__ __forceinline__ static float* d_at(const ActLds& act, uint32_t t) {
        const uint32_t c = (t >> kLogL) & (NC - 1), l = t & (LPR - 1), si = t >> (kLogL + kLogN);
        return (float*)(act.base + act.dbyte + ((si * (NC / G) + c / G) * LPR + l) * (4u * G) + 4u * (c % G));
    }
    // Unconditional too: keeping the stores unconditional keeps the loads where they are
    // written (otherwise the compiler sinks them into the store's branch, behind the weight
    // loads).
    __device__ __forceinline__ void store(const ActLds& act) {
        uint8_t* dq = q_at(act, threadIdx.x);
        float* dd = d_at(act, threadIdx.x);
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            *(u32x4*)(dq + 32 * TH * j) = q0[j];
            *(u32x4*)(dq + 32 * TH * j + 16 * LPR) = q1[j];
            dd[TH * j] = h2f(h[j]);
        }
    }
    // Re-staging within the area: pass column col() takes the pairs that column `src` of the
    // area holds (zeros where !ok).  Every thread reads (read_column), a barrier, every thread
    // writes (store_column): a column may feed several pass columns, or none.
    __device__ __forceinline__ void read_column(const ActLds& act, int src, bool ok, float (&d)[NS]) {
        const uint32_t t = threadIdx.x;
        const uint32_t ts = (t & ~((uint32_t)(NC - 1) << kLogL)) | ((uint32_t)(ok ? src : 0) << kLogL);
        const uint8_t* sq = q_at(act, ts);
        const float* sd = d_at(act, ts);
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            const u32x4 z = {0u, 0u, 0u, 0u};
            q0[j] = ok ? *(const u32x4*)(sq + 32 * TH * j) : z;
            q1[j] = ok ? *(const u32x4*)(sq + 32 * TH * j + 16 * LPR) : z;
            d[j] = ok ? sd[TH * j] : 0.0f;
        }
    }
    __device__ __forceinline__ void store_column(const ActLds& act, const float (&d)[NS]) {
        uint8_t* dq = q_at(act, threadIdx.x);
        float* dd = d_at(act, threadIdx.x);
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            *(u32x4*)(dq + 32 * TH * j) = q0[j];
            *(u32x4*)(dq + 32 * TH * j + 16 * LPR) = q1[j];
            dd[TH * j] = d[j];
        }
    }
};

// ------------------------------------------------------------------ the row engine
//
// One lane's share of one row of LPR lanes: slots i = 0, 1, ... (blocks s = l + LPR i).  U
// blocks are loaded per chunk; MULTI = the row has more than U blocks per lane (double-buffered
// chunks), otherwise U is at least the lane's block count.  Loads are unconditional (a block
// past the row is read at the row's last block; its activations are zeros and its scale is
// taken as 0, so it adds nothing), so the code between the loads and their uses stays
// straight-line and each use waits only for its own load.
//
// A pass computes NCP columns, NCP the pass's column count rounded up to a power of two (VAR:
// one straight-line copy of the code per NCP <= NC, picked once per pass; otherwise NCP = NC).
// Columns past the pass run on whatever LDS holds there and are never stored.  The columns of a
// slot are applied in groups of CG; the LDS reads of the next group are issued before the
// current group's integer dots (a slot's decode sits between the reads of its first group and
// their use), so LDS latency hides behind VALU work.
//
// CG is the widest power of two whose double-buffered activation registers (9 per column), with
// the raw weight chunks, the decoded block and the accumulators, stay within a budget of VGPRs
// (about 100 by default, so that two 512-thread workgroups fit a CU).  A budget of 0 reads one
// column at a time just before its use (for kernels held to 128 registers per lane).
template <int WT, int NC, int U, bool MULTI, int BUDGET>
constexpr int pick_cg() {
    constexpr int fixed = Unit<WT>::RAW * U * (MULTI ? 2 : 1) + 8 + NC;
    int cg = NC;
    while (cg > 1 && 18 * cg + fixed > BUDGET) cg /= 2;
    return cg;
}

// SGRID (CB3): `grid` is the signed codebook (cb3_signed_word) rather than the plain one.
template <int WT, int NC, bool SUMS, int U, bool MULTI, int LPR = kGemvLanesPerRow, bool VAR = false,
          int BUDGET = 100, bool SGRID = false>
struct RowEngine {
    static constexpr int RAW = Unit<WT>::RAW;
    static constexpr int kWT = WT;
    static constexpr bool kMulti = MULTI, kSignedGrid = SGRID;
    static constexpr int CGMAX = pick_cg<WT, NC, U, MULTI, BUDGET>();
    static constexpr int G = NC >= 4 ? 4 : NC;  // scales per slot group in LDS
    static constexpr uint32_t kSlotQ = 32u * LPR * NC, kColQ = 32u * LPR, kSlotD = 4u * LPR * NC;
    // bytes between consecutive blocks of a lane (LPR blocks, or LPR / 8 super-blocks)
    static constexpr uint32_t lane_stride() {
        if constexpr (WT == kCB3) return (uint32_t)(LPR / 8) * kCB3Bytes;
        else return (uint32_t)LPR * Unit<WT>::BYTES;
    }
    static constexpr uint32_t kStride = lane_stride();
    rsrc_t wr;
    uint32_t row_off;
    int nunits, niter, l16;
    typename Unit<WT>::Frame fr;
    uint32_t A[U][RAW], B[MULTI ? U : 1][RAW];
    typename Unit<WT>::Consts kc;

    template <int CG>
    struct Cols {
        u32x4 x0[CG], x1[CG];
        float d[CG];
    };

    RowEngine() = default;
    __device__ __forceinline__ RowEngine(rsrc_t wr_, uint32_t row_off_, int K, int l_) { init(wr_, row_off_, K, l_); }
    __device__ __forceinline__ void init(rsrc_t wr_, uint32_t row_off_, int K, int l_) {
        wr = wr_;
        row_off = row_off_;
        nunits = K / 32;
        niter = (K / 32 + LPR - 1) / LPR;
        l16 = l_;
        // (CB3: the sub-block of the lane's first block; planes: the lane's position in its tiles)
        fr = Unit<WT>::frame(unit_off(l16), WT == kCB3 ? (l16 & 7) : l16);
    }

    // byte offset of block s of the row (CB3: of its super-block)
    __device__ __forceinline__ uint32_t unit_off(int s) const {
        // 32-bit multiply-add (a 64-bit one would tie a dead high half to a pending load)
        if constexpr (WT == kCB3) return row_off + __umul24((uint32_t)(s >> 3), (uint32_t)kCB3Bytes);
        else return row_off + __umul24((uint32_t)s, (uint32_t)Unit<WT>::BYTES);
    }

    // Blocks i0 .. i0 + N - 1 of the lane.  Q8_0 and CB3: the lane frame plus a constant; a
    // block past the row end reads the bytes that follow (the next row, or zeros past the
    // buffer) and decodes to garbage that its zero scale discards.  IQ4_NL: each block's own
    // address (clamped to the row's last block), computed just before its loads: on cold
    // weights the loads issued this way, a few instructions apart, finished ~0.2 us sooner
    // per call than the same loads issued back to back (the reverse held for Q8_0).
    template <int N, int U0 = 0, int U1 = N>
    __device__ __forceinline__ void load(uint32_t (&buf)[N][RAW], int i0) {
#pragma unroll
        for (int u = U0; u < U1; ++u) {
            if constexpr (WT == kIQ4_NL) {
                const int s = l16 + LPR * (i0 + u);
                Unit<WT>::load(wr, Unit<WT>::frame(unit_off(s < nunits ? s : nunits - 1), 0), 0, buf[u]);
            } else {
                Unit<WT>::load(wr, fr, (uint32_t)(i0 + u) * kStride, buf[u]);
            }
        }
    }

    // FIRST < U (single chunk only): blocks 0 .. FIRST - 1 now, the others once block 0 has been
    // applied (run<FIRST>); the first blocks then land sooner and the last loads are issued
    // while block 0 computes.
    template <int FIRST = U>
    __device__ __forceinline__ void load_first() {
        if constexpr (MULTI || FIRST >= U) load(A, 0);
        else load<U, 0, FIRST>(A, 0);
    }

    // LDS reads of columns g CG .. g CG + CG - 1 of slot i (addresses relative to the chunk's
    // slot 0)
    template <int CG>
    __device__ __forceinline__ static void read_cols(Cols<CG>& a, const uint8_t* q, const uint8_t* d, int i, int g) {
        constexpr int SG = CG < G ? CG : G;  // scales per read
#pragma unroll
        for (int k = 0; k < CG; ++k) {
            const uint8_t* p = q + i * kSlotQ + (g * CG + k) * kColQ;
            a.x0[k] = *(const u32x4*)p;
            a.x1[k] = *(const u32x4*)(p + 16 * LPR);
        }
#pragma unroll
        for (int k = 0; k < CG; k += SG) {
            const int c = g * CG + k;
            const uint8_t* p = d + i * kSlotD + (c / G) * (4u * G * LPR) + 4 * (c % G);
            if constexpr (SG == 4) {
                const f32x4 v = *(const f32x4*)p;
                a.d[k] = v.x;
                a.d[k + 1] = v.y;
                a.d[k + 2] = v.z;
                a.d[k + 3] = v.w;
            } else if constexpr (SG == 2) {
                const f32x2 v = *(const f32x2*)p;
                a.d[k] = v.x;
                a.d[k + 1] = v.y;
            } else {
                a.d[k] = *(const float*)p;
            }
        }
    }

    template <int NCP, int FIRST = U, int N>
    __device__ __forceinline__ void compute(const uint32_t (&buf)[N][RAW], int i0, const ActView& av, int ncp,
                                            const uint32_t* grid, float (&acc)[NC], int32_t* srow, int64_t scol,
                                            bool row_ok) {
        constexpr int CG = CGMAX < NCP ? CGMAX : NCP;
        constexpr int NG = NCP / CG;
        const uint8_t* q = av.q + (uint32_t)i0 * kSlotQ;
        const uint8_t* d = av.d + (uint32_t)i0 * kSlotD;
        constexpr bool kAhead = BUDGET > 0;  // otherwise each group is read just before its use
        Cols<CG> cols[kAhead ? 2 : 1];
        if constexpr (kAhead) read_cols<CG>(cols[0], q, d, 0, 0);
        uint32_t W[8];
        uint32_t dw = 0;
        int mult = 1;
#pragma unroll
        for (int n = 0; n < N * NG; ++n) {
            const int u = n / NG, g = n % NG;
            if constexpr (kAhead) {
                if (n + 1 < N * NG) read_cols<CG>(cols[(n + 1) & 1], q, d, (n + 1) / NG, (n + 1) % NG);
            } else {
                read_cols<CG>(cols[0], q, d, u, g);
            }
            const int s = l16 + LPR * (i0 + u);
            if (g == 0) {
                const uint32_t* rw = buf[u];
                if constexpr (WT == kCB3 && SGRID) Unit<WT>::decode_signed(rw, fr, grid, W, dw, mult);
                else if constexpr (WT == kCB3) Unit<WT>::decode(rw, fr, grid, W, dw, mult);
                else Unit<WT>::decode(rw, fr, W, dw, mult, kc);
            }
            const Cols<CG>& a = cols[kAhead ? (n & 1) : 0];
            const bool ok = s < nunits;
            const float dwf = ok ? h2f(dw) : 0.0f;
#pragma unroll
            for (int k = 0; k < CG; ++k) {
                const int c = g * CG + k;
                int v = dot4_first(W[0], a.x0[k].x);
                v = dot4(W[1], a.x0[k].y, v);
                v = dot4(W[2], a.x0[k].z, v);
                v = dot4(W[3], a.x0[k].w, v);
                v = dot4(W[4], a.x1[k].x, v);
                v = dot4(W[5], a.x1[k].y, v);
                v = dot4(W[6], a.x1[k].z, v);
                v = dot4(W[7], a.x1[k].w, v);
                // |v| < 2^23 and mult <= 31: the 24-bit multiply is exact
                const int isum = WT == kCB3 ? __mul24(v, mult) : v;
                if constexpr (SUMS) {
                    if (row_ok && ok && c < ncp) srow[c * scol + s] = isum;
                } else {
                    // dwf * d is exact (two binary16 significands) and so is float(isum): the
                    // fma rounds each block's term once (a row with one non-zero term gives
                    // that term correctly rounded)
                    acc[c] = __builtin_fmaf(dwf * a.d[k], (float)isum, acc[c]);
                }
            }
            if constexpr (!MULTI && FIRST < U) {
                if (n == NG - 1) load<U, FIRST, U>(A, 0);
            }
            // keeps the reads of later groups from being hoisted here (two buffers at most)
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    template <int NCP, int FIRST>
    __device__ __forceinline__ void run_pass(const ActView& av, int ncp, const uint32_t* grid, float (&acc)[NC],
                                             int32_t* srow, int64_t scol, bool row_ok) {
        if constexpr (!MULTI) {
            compute<NCP, FIRST>(A, 0, av, ncp, grid, acc, srow, scol, row_ok);
        } else {
            for (int i0 = 0; i0 < niter; i0 += 2 * U) {
                const bool more = i0 + U < niter;
                if (more) load(B, i0 + U);
                compute<NCP>(A, i0, av, ncp, grid, acc, srow, scol, row_ok);
                if (more) {
                    if (i0 + 2 * U < niter) load(A, i0 + 2 * U);
                    compute<NCP>(B, i0 + U, av, ncp, grid, acc, srow, scol, row_ok);
                }
            }
        }
    }

    // All of the lane's blocks; the first chunk must already be loaded (load_first<FIRST>).
    template <int FIRST = U>
    __device__ __forceinline__ void run(const ActView& av, int ncp, const uint32_t* grid, float (&acc)[NC],
                                        int32_t* srow, int64_t scol, bool row_ok) {
        if constexpr (!VAR || NC == 1) {
            run_pass<NC, FIRST>(av, ncp, grid, acc, srow, scol, row_ok);
        } else {
            if (ncp > NC / 2) run_pass<NC, FIRST>(av, ncp, grid, acc, srow, scol, row_ok);
            else if constexpr (NC >= 4) {
                if (ncp > NC / 4) run_pass<NC / 2, FIRST>(av, ncp, grid, acc, srow, scol, row_ok);
                else if constexpr (NC >= 8) {
                    if (ncp > 1) run_pass<2, FIRST>(av, ncp, grid, acc, srow, scol, row_ok);
                    else run_pass<1, FIRST>(av, ncp, grid, acc, srow, scol, row_ok);
                } else {
                    run_pass<1, FIRST>(av, ncp, grid, acc, srow, scol, row_ok);
                }
            } else {
                run_pass<1, FIRST>(av, ncp, grid, acc, srow, scol, row_ok);
            }
        }
    }
};

// Sums over the LPR lanes of a row (16: one DPP row; 64: the wave, whose four DPP rows are then
// added across) of the NC per-lane partials: lane l ends with column row_col<NC>(l mod 16).
template <int NC, int LPR>
__device__ __forceinline__ float row_sums(const float (&acc)[NC], int l) {
    float v = row16_sums<NC>(acc, l & 15);
    if constexpr (LPR == 64) {
        v += __shfl_xor(v, 16, 64);
        v += __shfl_xor(v, 32, 64);
    }
    return v;
}

// NC fp32 activation columns (column c at c K floats) quantized to q8_1 inside the workgroup,
// into the layout the NC-column ActStage writes with 16 lanes per row and one staging slot
// (block b of column c is the slot-0 block of staging thread ((b / 16) NC + c) 16 + b % 16:
// its int8 values at q_at, q_at + 16 LPR, its scale at d_at).  Eight lanes per 32-value
// block, four consecutive values per lane (one 16-byte load), TH / 8 block tasks a pass, task
// i taking column i % NC, block i / NC; blocks past the row (up to 96) read and stage zeros.
// The arithmetic is the q8_1 quantizer's [DQ, Change]: amax over the block (exact in any
// order), d = amax / 127 and q = x / d rounded half away from zero, IEEE binary32, clamped to
// +-127, so the staged bytes equal the ones the standalone quantizer writes; only d (as fp16)
// is staged.
// Only the first SB blocks of each column are staged: the row engine reads no others (SB = 16
// lanes x its chunk); the tasks of the blocks beyond skip their loads, their arithmetic and their
// LDS writes (whole waves of them in the last pass).
template <int NC, int TH, int SB = 96>
struct F32Stage {
    static constexpr int kLogN = NC == 8 ? 3 : NC == 4 ? 2 : NC == 2 ? 1 : 0;
    static constexpr int kBlocks = TH / 8;                            // block tasks per pass
    static constexpr int kPass = (NC * SB + kBlocks - 1) / kBlocks;  // rows of at most SB blocks
    static_assert(SB <= 96, "rows of at most 96 blocks");
    u32x4 v[kPass];
    __device__ __forceinline__ void load(rsrc_t xr, int nb, int K, uint32_t zero_off) {
        const uint32_t j = threadIdx.x & 7u, h = threadIdx.x >> 3;
#pragma unroll
        for (int p = 0; p < kPass; ++p) {
            const uint32_t bt = (uint32_t)p * kBlocks + h;
            const uint32_t c = bt & (NC - 1), b = bt >> kLogN;
            if (b < (uint32_t)SB) v[p] = ld128(xr, b < (uint32_t)nb ? (c * (uint32_t)K + b * 32u) * 4u + 16u * j : zero_off);
        }
    }
    template <int NS, int LPR>
    __device__ __forceinline__ void store(const ActLds& act) {
        static_assert(NS == 1 && LPR == 16 && NC <= 4 && TH / NC >= 96, "16 lanes per row, every block in slot 0");
        const uint32_t j = threadIdx.x & 7u, h = threadIdx.x >> 3;
#pragma unroll
        for (int p = 0; p < kPass; ++p) {
            const uint32_t bt = (uint32_t)p * kBlocks + h;
            const uint32_t c = bt & (NC - 1), b = bt >> kLogN;
            if (b >= (uint32_t)SB) continue;
            const uint32_t ts = ((b >> 4) << (4 + kLogN)) | (c << 4) | (b & 15u);
            // (each element copied out first: __builtin_bit_cast of a vector element in place
            // reads element 0 with this compiler)
            float x[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t e = v[p][i];
                x[i] = __builtin_bit_cast(float, e);
            }
            float amax = __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(x[0]), __builtin_fabsf(x[1])),
                                         __builtin_fmaxf(__builtin_fabsf(x[2]), __builtin_fabsf(x[3])));
            // over the 8 lanes of the block: quad partners, the other pair of the quad, then the
            // mirrored lane of the other quad in the half row
            amax = __builtin_fmaxf(amax, dpp<0xB1>(amax));
            amax = __builtin_fmaxf(amax, dpp<0x4E>(amax));
            amax = __builtin_fmaxf(amax, dpp<0x141>(amax));
            const float d = amax / 127.0f;
            const bool zero = amax == 0.0f || d == 0.0f;
            uint32_t w4 = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                int q = zero ? 0 : round_away(x[i] / d);
                q = q > 127 ? 127 : (q < -127 ? -127 : q);
                w4 |= (uint32_t)(q & 0xFF) << (8 * i);
            }
            uint8_t* dq = ActStage<NS, NC, LPR, TH>::q_at(act, ts);
            *(uint32_t*)(dq + (j < 4 ? 4u * j : 16u * LPR + 4u * (j - 4))) = w4;
            if (j == 0) *ActStage<NS, NC, LPR, TH>::d_at(act, ts) = zero ? 0.0f : h2f(f2h(d));
        }
    }
};

// One workgroup's TH / 64 * (64 / LPR) rows starting at row0 of a decode GEMV pass: columns
// [col0, col0 + ncp) of the q8_1 activations behind `xr` (xbytes long; column c is q8_1 blocks
// c*K/32 ...),
// results to y[(col0 + c) * ldy + row] (or the per-block integer sums, SUMS).  LPR lanes per
// row (16 or 64).  Order of work: activation loads, then this lane's weight loads, then the
// activation LDS writes (they wait only for the activation loads), barrier, decode + apply as
// the weights arrive, cross-lane row sums.  F32: `xr` holds the pass's NC fp32 columns
// instead, which the workgroup quantizes to q8_1 itself (F32Stage).
template <int WT, bool SUMS, int NC, int U, bool MULTI, int NS, int LPR = kGemvLanesPerRow, int TH = kGemvThreads,
          bool VAR = false, int BUDGET = 100, bool F32 = false>
__device__ __forceinline__ void gemv_tile(rsrc_t wr, int nrows, int K, const uint8_t* grid, rsrc_t xr, uint32_t xbytes,
                                          int col0, int ncp, float* y, int64_t ldy, int32_t* sums, int row0,
                                          uint32_t* lds) {
    static_assert(LPR == 16 || LPR == 64, "a row is one DPP row or one wave");
    const ActLds act = act_lds_layout<NC, NS, TH>(lds, K);
    uint32_t* lds_grid = act_lds_end<NS, TH>(act);

    const int lane = threadIdx.x & 63;
    const int l16 = lane & (LPR - 1);
    const int row = row0 + (threadIdx.x >> 6) * (64 / LPR) + lane / LPR;
    const bool row_ok = row < nrows;
    const int rowc = row_ok ? row : nrows - 1;
    // (kept apart from the lane offset the row engine adds: fused, the two become a 64-bit
    // multiply-add whose unused high addend may sit in a register a pending load writes)
    const uint32_t row_off = IQ4Consts::opaque_u((uint32_t)rowc * (uint32_t)row_bytes_dev<WT>(K));

    ActStage<NS, NC, LPR, TH> stage;
    F32Stage<NC, TH, (LPR * U < 96 ? LPR * U : 96)> fstage;
    if constexpr (F32) fstage.load(xr, act.nb, K, xbytes);
    else stage.load(xr, act, col0, ncp, xbytes);
    GridStage<TH> gstage;
    if constexpr (WT == kCB3) gstage.load(grid);
    __builtin_amdgcn_sched_barrier(0);
    RowEngine<WT, NC, SUMS, U, MULTI, LPR, VAR, BUDGET> eng(wr, row_off, K, l16);
    // IQ4_NL on fp32 columns: the lane's weight loads are split (measured, one column on cold
    // weights, same box: IQ4_NL 8192 x 2560 5.04 -> 4.58 us; not taken where it measured slower:
    // the q8_1-input calls, 4.47 -> 4.70 us, and Q8_0 12288 x 2560, 8.49 -> 8.98 us)
    constexpr int kFirst = F32 && !MULTI && WT == kIQ4_NL ? (U + 1) / 2 : U;
    eng.template load_first<kFirst>();
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (F32) fstage.template store<NS, LPR>(act);
    else stage.store(act);
    if constexpr (WT == kCB3) gstage.store(lds_grid);
    __syncthreads();
    // the weight decode stays after the barrier (hoisted above it, each wave would wait for its
    // first weight block before the workgroup could pass)
    __builtin_amdgcn_sched_barrier(0);

    float acc[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[c] = 0.0f;
    int32_t* srow = nullptr;
    int64_t scol = 0;
    if constexpr (SUMS) {
        srow = sums + ((int64_t)col0 * nrows + rowc) * act.nb;
        scol = (int64_t)nrows * act.nb;
    }
    eng.template run<kFirst>(act_view<NC>(act, l16), ncp, lds_grid, acc, srow, scol, row_ok);
    if constexpr (!SUMS) {
        const float s = row_sums<NC, LPR>(acc, l16);
        const int c = row_col<NC>(l16 & 15);
        // one lane per column: the lowest of the lanes holding it, in the row's first 16 lanes
        const bool writer = (l16 & (16 / NC - 1)) == 0 && l16 < 16;
        if (row_ok && writer && c < ncp) y[(int64_t)(col0 + c) * ldy + row] = s;
    }
}

// The chunk a kernel instance loads per lane for rows of `lb` blocks per lane: chunks of 2, 3,
// 5 or 6 (a chunk longer than the lane's count re-reads its last block), double-buffered
// chunks of `um` beyond 6 (or always, for the block-sum hook).
struct Chunk {
    int u;
    bool multi;
};
inline Chunk gemv_chunk(int lb, int lpr, bool sums, int um = 6) {
    if (sums) return {6, true};
    if (lb <= 2) return {2, false};
    if (lpr == 64 && lb <= 3) return {3, false};
    if (lb <= 5 && lpr != 64) return {5, false};
    if (lb <= 6) return {6, false};
    return {um, true};
}

}  // namespace qmm
