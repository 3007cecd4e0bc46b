// qmm_grouped.hip -- grouped MoE-expert decode for gfx950: gate/up GEMV + SwiGLU + q8_1 of H,
// then the down GEMV, over groups (experts) x entries (routed token slots).
//
// Method [IQ, What it does: native_gu / native_down decode each weight part once for every
// entry of a group; DQ, Change: swiglu, then q8_1 of H for the down product, H never stored in
// fp32]:
//   gate/up kernel : workgroup (t, g) takes intermediate rows [32t, 32t + 32) of expert
//                    group_expert[g], both its gate and its up row for each index (one DPP row
//                    of 16 lanes per index runs both), and every entry of the group in passes
//                    of 8.  Each weight block is loaded once and applied to all entries of the
//                    pass.  The 32 x 8 gate and up sums go through LDS to a half wave per
//                    entry, which forms h = silu(g) * u and quantizes the 32 values to one q8_1
//                    block of H.
//   down kernel    : the decode GEMV tile over W_down[e] with the group's H blocks (the entries
//                    of a group are consecutive, so their H blocks are too).
// silu(z) = z / (1 + e^-z) in binary32 (expf within 1 ulp, IEEE division).
#include "qmm_gemv.h"

#include <mutex>

namespace qmm {

constexpr int kGroupPass = 8;  // entries per pass

// silu(z) * u in binary32 with the library expf (documented maximum error 1 ulp), an IEEE
// division and a product: within a few ulp of the same expression evaluated exactly.
__device__ __forceinline__ float silu_mul(float z, float u) {
    const float e = expf(-z);
    const float den = opaque(1.0f + e);
    const float sl = opaque(z / den);
    return sl * u;
}

// Uniform group bounds: expert e and entry range [k0, k1), clamped to the valid ranges.
struct GroupInfo {
    int e, k0, k1;
    __device__ __forceinline__ bool load(const int32_t* group_expert, const int32_t* group_off, int g, int nexperts,
                                         int nentries) {
        e = __builtin_amdgcn_readfirstlane(group_expert[g]);
        k0 = __builtin_amdgcn_readfirstlane(group_off[g]);
        k1 = __builtin_amdgcn_readfirstlane(group_off[g + 1]);
        k0 = k0 < 0 ? 0 : k0;
        k1 = k1 > nentries ? nentries : k1;
        return e >= 0 && e < nexperts && k1 > k0;
    }
};

// gate/up workgroup.  PAIR (CB3 rows whose pass fits two workgroups per CU): 512 threads, 8
// waves, two workgroups per CU (4 waves per SIMD, 128 registers per lane, so the row engines
// read each column's activations just before use), which keeps the grid of inter / 32 x groups
// workgroups (512 for 16 groups of a 1024-row expert) resident at once.  Wave w takes
// intermediate indices 4w .. 4w + 3 of the 32 of one q8_1 block of H, a DPP row of 16 lanes
// each, and each lane holds two row engines, the gate and the up row of its index, whose loads
// are all issued before either computes.  Otherwise (Q8_0 and IQ4_NL, whose raw blocks do not
// fit twice in those registers, and CB3 rows too long for the 512-thread staging): 1024
// threads, one workgroup per CU, waves 0..7 on the gate rows and 8..15 on the up rows, one row
// engine per lane.
template <bool PAIR>
constexpr int gu_threads() { return PAIR ? 512 : 1024; }
constexpr size_t kGuPairLds = 48 << 10;  // dynamic LDS that leaves room for two per CU

// v_perm selector taking byte k from the second operand (k) or, where bit k of n is set, from
// the first (k + 4).
constexpr uint32_t sign_select(int n) {
    return 0x03020100u | ((n & 1) ? 0x4u : 0u) | ((n & 2) ? 0x400u : 0u) | ((n & 4) ? 0x40000u : 0u) |
           ((n & 8) ? 0x4000000u : 0u);
}

constexpr bool high_variants_set_bit26() {
    for (int n = 0; n < 8; ++n)
        if (sign_select(8 + n) != (sign_select(n) | (1u << 26)) || (sign_select(n) & (1u << 26))) return false;
    return true;
}
static_assert(high_variants_set_bit26(), "variants 8..15 take byte 3 from the negated entry");

// The signed CB3 codebook of a gate/up workgroup (static LDS, beside the dynamic area).
__device__ __forceinline__ uint32_t* cb3_signed_lds() {
    __shared__ __attribute__((aligned(16))) uint32_t t[kCB3SignedWords];
    return t;
}

// State of one gate/up workgroup and one pass over entries [c0, c0 + 8) of its group.
template <int WT, int U, bool MULTI, int NS, bool PAIR_>
struct GuWorkgroup {
    static constexpr bool PAIR = PAIR_;
    static constexpr int TH = gu_threads<PAIR>();
    using Stage = ActStage<NS, kGroupPass, kGemvLanesPerRow, TH>;
    const ActLds act;
    float* gl;  // [8][32] gate sums
    float* ul;  // [8][32] up sums
    const uint32_t* sgrid;
    int l16, rg, i, inter, hidden, xq_cols, nbh, k1;
    uint32_t rb, xqbytes;
    rsrc_t xr, wgr, wur;  // activations, the expert's gate rows, its up rows
    bool up;              // one row per lane: this wave runs up rows
    const uint8_t* grid;
    const int32_t* entry_col;
    uint8_t* hq;
    float *dbg_g, *dbg_u;

    // FIRST: the workgroup's first pass (builds the signed codebook from gword); VAR: the row
    // engine's straight-line copies per pass width (the later passes, rare, take the full-width
    // copy, whose columns are bitwise the same); DENSE (first pass only): `pre` holds the loads
    // of activation columns 0 .. 7 (all of them), issued before the group was known; they are
    // staged as they are and re-staged in LDS to the pass's entry columns unless those are
    // 0, 1, 2, ... already.  Otherwise the pass loads its entry columns once their indices are
    // known.
    template <bool FIRST, bool VAR, bool DENSE>
    __device__ __forceinline__ void pass(int c0, Stage& pre, uint32_t gword) {
        static_assert(FIRST || !DENSE, "the activations loaded up front serve the first pass");
        const int ncp = k1 - c0 < kGroupPass ? k1 - c0 : kGroupPass;
        // The row engine is rebuilt each pass from values the compiler cannot see through, so
        // per-pass address arithmetic is not hoisted out of the pass loop (which would hold it
        // in registers, or spill it, across the whole loop).
        using Eng = RowEngine<WT, kGroupPass, false, U, MULTI, kGemvLanesPerRow, VAR, 0, true>;
        // (the gate and up rows sit at the same offset of their matrices: one set of lane
        // offsets serves both engines; with one row per lane, eg runs this wave's row)
        const uint32_t roff = IQ4Consts::opaque_u((uint32_t)i * rb);
        const int lo = (int)IQ4Consts::opaque_u((uint32_t)l16);
        Eng eg(PAIR || !up ? wgr : wur, roff, hidden, lo);
        Eng eu(wur, roff, hidden, lo);
        Stage own;
        int ecol[kGroupPass];  // DENSE: the pass's entry columns, read now, needed after the staging
        if constexpr (DENSE) {
#pragma unroll
            for (int k = 0; k < kGroupPass; ++k) ecol[k] = entry_col[c0 + (k < ncp ? k : 0)];
        } else {
            own.load_entries(xr, act, ncp, entry_col, c0, xq_cols, xqbytes);
        }
        Stage& stage = DENSE ? pre : own;
        __builtin_amdgcn_sched_barrier(0);
        // every pass loads the rows (a later pass re-reads the group's rows from L2); the up
        // row's loads go out once the staged activations have left their registers.  Each row
        // loads its first (U + 1) / 2 blocks now and the rest once its block 0 has been applied:
        // fewer registers held by loads in flight (no spills where whole rows spilled) and the
        // first blocks land sooner (CB3 2560-wide rows, 16 groups: 22.1 / 27.9 / 35.2 ->
        // 21.5 / 26.5 / 34.0 us at m = 1 / 4 / 8, same box)
        constexpr int kFirst = (U + 1) / 2;
        eg.template load_first<kFirst>();
        __builtin_amdgcn_sched_barrier(0);
        stage.store(act);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (PAIR) eu.template load_first<kFirst>();
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (WT == kCB3 && FIRST) {
            // variant n: byte k negated where bit k of n is set; with every byte of the entry
            // non-zero, ~g + 0x01010101 negates all four bytes without carries, and one v_perm
            // picks each byte from g or from it.  The 16 variants of entry e are words 16 e ..
            // 16 e + 15: thread t writes VPT of them (selector sign_select(n mod 8), with bit 26
            // for n >= 8).
            constexpr int VPT = kCB3SignedWords / TH;
            static_assert(VPT == 8 || VPT == 16, "a thread writes half or all of one entry's variants");
            const uint32_t neg = ~gword + 0x01010101u;
            const int n0 = VPT == 8 ? 8 * (int)(threadIdx.x & 1u) : 0;
            uint32_t v[VPT];
#pragma unroll
            for (int n = 0; n < VPT; ++n) v[n] = perm(neg, gword, sign_select(n & 7) | (n0 + n >= 8 ? 1u << 26 : 0u));
            u32x4* dst = (u32x4*)(cb3_signed_lds() + VPT * threadIdx.x);
#pragma unroll
            for (int j = 0; j < VPT / 4; ++j) dst[j] = u32x4{v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]};
        }
        lds_barrier();
        if constexpr (DENSE) {
            // pass column k reads activation column ecol[k] (zeros outside [0, xq_cols))
            const int cl = Stage::col();
            int src = 0, moved = 0;
#pragma unroll
            for (int k = 0; k < kGroupPass; ++k) {
                // (kept here: computed early, each use would wait for its load before the next
                // load was issued)
                asm volatile("" : "+s"(ecol[k]));
                src = cl == k ? ecol[k] : src;
                moved |= k < ncp ? ecol[k] ^ k : 0;
            }
            if (moved) {
                float d[NS];
                stage.read_column(act, src, cl < ncp && src >= 0 && src < xq_cols, d);
                lds_barrier();
                stage.store_column(act, d);
                lds_barrier();
            }
        }
        __builtin_amdgcn_sched_barrier(0);  // decode after the barrier

        // the gate row, then (pair) the up row, with one set of accumulators; the up row's
        // loads stay in flight while the gate row computes
        float acc[kGroupPass];
#pragma unroll
        for (int c = 0; c < kGroupPass; ++c) acc[c] = 0.0f;
        eg.template run<kFirst>(act_view<kGroupPass>(act, l16), ncp, sgrid, acc, nullptr, 0, true);
        const float sg = row16_sums<kGroupPass>(acc, l16);
        float su = 0.0f;
        if constexpr (PAIR) {
#pragma unroll
            for (int c = 0; c < kGroupPass; ++c) acc[c] = 0.0f;
            eu.template run<kFirst>(act_view<kGroupPass>(act, l16), ncp, sgrid, acc, nullptr, 0, true);
            su = row16_sums<kGroupPass>(acc, l16);
        }
        // (the lane's index and row, recomputed from the thread index: kept across the row
        // engines' runs they would take registers the runs need)
        const uint32_t tid = IQ4Consts::opaque_u(threadIdx.x);
        const int lb = (int)(tid & 15u);
        const int rgb = (int)(((tid >> 6) & 7u) * 4u + ((tid & 63u) >> 4));
        const int ib = (int)blockIdx.x * 32 + rgb;
        const int c = row_col<kGroupPass>(lb);
        if ((lb & 1) == 0 && c < ncp) {
            if (PAIR || !up) {
                gl[c * 32 + rgb] = sg;
                if (dbg_g) dbg_g[(int64_t)(c0 + c) * inter + ib] = sg;
            }
            if (PAIR || up) {
                ul[c * 32 + rgb] = PAIR ? su : sg;
                if (dbg_u) dbg_u[(int64_t)(c0 + c) * inter + ib] = PAIR ? su : sg;
            }
        }
        lds_barrier();
        // SwiGLU -> q8_1: one half wave per entry (waves 0..3), value j = intermediate 32t + j
        if (threadIdx.x < kGroupPass * 32) {
            const int c = threadIdx.x >> 5, j = threadIdx.x & 31;
            const bool ok = c < ncp;
            const float h = ok ? silu_mul(gl[c * 32 + j], ul[c * 32 + j]) : 0.0f;
            uint32_t hdr;
            const int q = quantize_lanes32(h, hdr);
            const uint32_t word = pack4_lanes(q);
            if (ok) {
                uint32_t* dst = (uint32_t*)(hq + ((int64_t)(c0 + c) * nbh + blockIdx.x) * 36);
                if (j == 0) dst[0] = hdr;
                if ((j & 3) == 0) dst[1 + (j >> 2)] = word;
            }
        }
    }
};

template <int WT, int U, bool MULTI, int NS, bool DENSE, bool PAIR>
__global__ __launch_bounds__(gu_threads<PAIR>(), PAIR ? 4 : 1) void gu_kernel(
    const uint8_t* __restrict__ wg, const uint8_t* __restrict__ wu, int64_t gu_stride, uint32_t expert_bytes,
    int nexperts, const uint8_t* __restrict__ grid, int hidden, int inter, const uint8_t* __restrict__ xq,
    uint32_t xqbytes, int xq_cols, const int32_t* __restrict__ group_expert, const int32_t* __restrict__ group_off,
    const int32_t* __restrict__ entry_col, int nentries, uint8_t* __restrict__ hq, float* __restrict__ dbg_g,
    float* __restrict__ dbg_u) {
    extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
    using WG = GuWorkgroup<WT, U, MULTI, NS, PAIR>;
    const ActLds act = act_lds_layout<kGroupPass, NS, WG::TH>(lds, hidden);
    // Loads that need nothing from the group first (their latency then overlaps the group
    // lookup's): with at most 8 activation columns (DENSE), all of them; the codebook entry.
    typename WG::Stage pre;
    if constexpr (DENSE) pre.load(make_rsrc(xq, xqbytes), act, 0, xq_cols, xqbytes);
    uint32_t gword = 0;
    if constexpr (WT == kCB3) gword = ld32(make_rsrc(grid, 2048), 4u * (threadIdx.x / (WG::TH / 512)));
    __builtin_amdgcn_sched_barrier(0);
    GroupInfo gi;
    if (!gi.load(group_expert, group_off, blockIdx.y, nexperts, nentries)) {
        // (a use on this path too, so the loads above are not moved behind the group lookup)
        if constexpr (DENSE) pre.keep();
        asm volatile("" ::"v"(gword));
        return;
    }

    float* gl = (float*)act_lds_end<NS, WG::TH>(act);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int rg = (wave & 7) * 4 + (lane >> 4);  // 0..31
    WG w{act, gl, gl + kGroupPass * 32,
         // CB3: the signed codebook (16 sign variants of each entry), built in the first pass:
         // each thread loads its entry with the activations and, once the weight loads are
         // issued, writes its share of the entry's variants
         WT == kCB3 ? cb3_signed_lds() : nullptr,
         lane & 15, rg, (int)blockIdx.x * 32 + rg, inter, hidden, xq_cols, inter / 32,
         gi.k1, (uint32_t)row_bytes_dev<WT>(hidden), xqbytes, make_rsrc(xq, xqbytes),
         make_rsrc_dw(wg + gi.e * gu_stride, expert_bytes), make_rsrc_dw(wu + gi.e * gu_stride, expert_bytes),
         !WG::PAIR && wave >= 8, grid, entry_col, hq, dbg_g, dbg_u};
    // The first pass outside the loop: its loads start with nothing outstanding.  Later passes
    // first wait for the previous pass's memory operations (which the compiler would otherwise
    // count as outstanding across the loop) and LDS reads.
    w.template pass<true, true, DENSE>(gi.k0, pre, gword);
    for (int c0 = gi.k0 + kGroupPass; c0 < gi.k1; c0 += kGroupPass) {
        vm_drain();
        lds_barrier();
        w.template pass<false, false, false>(c0, pre, 0);
    }
}

// Down kernel: a workgroup takes 32 consecutive rows of one group.  Rows of at most 2 blocks
// per lane (Q8_0, IQ4_NL; the decode workload's 1024-value rows): 256 threads in two sets of 16
// rows (4 rows per wave and set); the workgroup stages the group's H columns once and issues
// both sets' weight loads before either computes, and at most 96 registers per lane keep five
// workgroups per CU resident (5 waves per SIMD), so that the 16 groups x 2560 rows of the
// workload (1280 workgroups) run in one round.  Other rows: 512 threads, one set of 32 rows
// (the staging of longer rows needs the wider workgroup).
template <int WT, int U, bool MULTI>
constexpr bool down_short() { return U <= 2 && !MULTI && WT != kCB3; }
template <int WT, int U, bool MULTI>
constexpr int down_threads() { return down_short<WT, U, MULTI>() ? 256 : 512; }
template <int WT, int U, bool MULTI>
constexpr int down_waves_per_simd() { return down_short<WT, U, MULTI>() ? 5 : 2; }
constexpr int kDownRows = 32;  // rows per workgroup
static int down_threads_host(int wt, Chunk ch) { return ch.u <= 2 && !ch.multi && wt != QMM_CB3 ? 256 : 512; }

// One pass (columns [col0, col0 + ncp) of H) over the R row sets from row0: the decode GEMV
// tile's steps (H loads, weight loads, H into LDS, barrier, decode and apply, row sums) with R
// row engines per lane.  Each row's sum is the single-set tile's, bitwise.
template <int WT, int U, int NS, int TH>
__device__ __forceinline__ void down_sets(rsrc_t wr, int nrows, int K, const uint8_t* grid, rsrc_t hr,
                                          uint32_t hbytes, int col0, int ncp, float* y, int64_t ldy, int row0,
                                          uint32_t* lds) {
    constexpr int R = kDownRows / (TH / 16);  // row sets
    const ActLds act = act_lds_layout<kGroupPass, NS, TH>(lds, K);
    uint32_t* lds_grid = act_lds_end<NS, TH>(act);
    const int lane = threadIdx.x & 63;
    const int l16 = lane & 15;
    const int rbase = row0 + (int)(threadIdx.x >> 6) * 4 + (lane >> 4);
    ActStage<NS, kGroupPass, kGemvLanesPerRow, TH> stage;
    stage.load(hr, act, col0, ncp, hbytes);
    GridStage<TH> gstage;
    if constexpr (WT == kCB3) gstage.load(grid);
    __builtin_amdgcn_sched_barrier(0);
    using Eng = RowEngine<WT, kGroupPass, false, U, false, kGemvLanesPerRow, true, R == 1 ? 40 : 0>;
    Eng eng[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int row = rbase + (TH / 16) * r;
        const int rowc = row < nrows ? row : nrows - 1;
        eng[r].init(wr, IQ4Consts::opaque_u((uint32_t)rowc * (uint32_t)row_bytes_dev<WT>(K)), K, l16);
        eng[r].load_first();
    }
    __builtin_amdgcn_sched_barrier(0);
    stage.store(act);
    if constexpr (WT == kCB3) gstage.store(lds_grid);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int row = rbase + (TH / 16) * r;
        float acc[kGroupPass];
#pragma unroll
        for (int c = 0; c < kGroupPass; ++c) acc[c] = 0.0f;
        eng[r].run(act_view<kGroupPass>(act, l16), ncp, lds_grid, acc, nullptr, 0, row < nrows);
        const float sum = row_sums<kGroupPass, kGemvLanesPerRow>(acc, l16);
        const int c = row_col<kGroupPass>(l16);
        if (row < nrows && (l16 & 1) == 0 && c < ncp) y[(int64_t)(col0 + c) * ldy + row] = sum;
    }
}

template <int WT, int U, bool MULTI, int NS>
__global__ __launch_bounds__((down_threads<WT, U, MULTI>()), (down_waves_per_simd<WT, U, MULTI>())) void down_kernel(const uint8_t* __restrict__ wd, int64_t d_stride,
                                                            uint32_t expert_bytes, int nexperts,
                                                            const uint8_t* __restrict__ grid, int hidden, int inter,
                                                            const uint8_t* __restrict__ hq, uint32_t hqbytes,
                                                            const int32_t* __restrict__ group_expert,
                                                            const int32_t* __restrict__ group_off, int nentries,
                                                            float* __restrict__ y) {
    extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
    GroupInfo gi;
    if (!gi.load(group_expert, group_off, blockIdx.y, nexperts, nentries)) return;
    const rsrc_t wr = make_rsrc_dw(wd + gi.e * d_stride, expert_bytes);
    const rsrc_t hr = make_rsrc(hq, hqbytes);
    constexpr int TH = down_threads<WT, U, MULTI>();
    for (int c0 = gi.k0; c0 < gi.k1; c0 += kGroupPass) {
        const int ncp = gi.k1 - c0 < kGroupPass ? gi.k1 - c0 : kGroupPass;
        if (c0 != gi.k0) __syncthreads();
        if constexpr (MULTI) {
            // (long rows: the decode GEMV tile with its double-buffered engine)
            gemv_tile<WT, false, kGroupPass, U, MULTI, NS, kGemvLanesPerRow, TH, true, 40>(
                wr, hidden, inter, grid, hr, hqbytes, c0, ncp, y, hidden, nullptr, blockIdx.x * kDownRows, lds);
        } else {
            down_sets<WT, U, NS, TH>(wr, hidden, inter, grid, hr, hqbytes, c0, ncp, y, hidden, blockIdx.x * kDownRows,
                                     lds);
        }
    }
}

// UM: chunk of the double-buffered (MULTI) instance, for rows of more than 6 blocks per lane
// (2 in the gate/up kernels, whose lanes have 128 registers).
// go(WT, U, MULTI, NS) receives the instance as std::integral_constant tags.
template <int V>
using IntC = std::integral_constant<int, V>;
template <int WT, int UM = 6, typename F>
static void dispatch_u_ns(Chunk ch, int ns, F&& go) {
    auto by_u = [&](auto ns_c) {
        if (ch.multi) go(IntC<WT>{}, IntC<UM>{}, std::true_type{}, ns_c);
        else if (ch.u == 2) go(IntC<WT>{}, IntC<2>{}, std::false_type{}, ns_c);
        else if (ch.u == 5) go(IntC<WT>{}, IntC<5>{}, std::false_type{}, ns_c);
        else go(IntC<WT>{}, IntC<6>{}, std::false_type{}, ns_c);
    };
    if (ns == 1) by_u(IntC<1>{});
    else if (ns == 2) by_u(IntC<2>{});
    else if (ns == 3) by_u(IntC<3>{});
    else by_u(IntC<4>{});
}

struct GroupedArgs {
    int wtype_gu, wtype_down, nexperts, ngroups, nentries, xq_cols;
    const uint8_t *w_gate, *w_up, *w_down, *grid, *xq;
    int64_t gu_stride, d_stride, hidden, inter;
    const int32_t *group_expert, *group_off, *entry_col;
    float* y;
    uint8_t* ws;
    unsigned flags;
    hipStream_t st;
};

static size_t grouped_h_bytes(int64_t inter, int nentries) { return (size_t)nentries * (size_t)(inter / 32) * 36; }

// Chunks, LDS and staging slots of the two kernels (gate/up: 512 or 1024 threads, double-buffered
// chunks of 2 for long rows; down: 256 threads).
static Chunk gu_chunk(int64_t hidden) { return gemv_chunk(lane_blocks(hidden, kGemvLanesPerRow), kGemvLanesPerRow, false, 2); }
static Chunk down_chunk(int64_t inter) { return gemv_chunk(lane_blocks(inter, kGemvLanesPerRow), kGemvLanesPerRow, false); }
// (dynamic LDS: activations and the gate/up sums; the signed CB3 codebook is static)
static size_t gu_lds_bytes(bool pair, int64_t hidden) {
    return act_lds_bytes(hidden, kGroupPass, kGemvLanesPerRow, gu_chunk(hidden).u, pair ? 512 : 1024) +
           2 * kGroupPass * 32 * sizeof(float);
}
static size_t down_lds_bytes(int wt, int64_t inter) {
    return gemv_lds_bytes(wt, inter, kGroupPass, kGemvLanesPerRow, down_chunk(inter).u,
                          down_threads_host(wt, down_chunk(inter)));
}
static int gu_slots(bool pair, int64_t hidden) {
    return stage_slots(hidden, kGroupPass, pair ? 512 : 1024, kGemvLanesPerRow, gu_chunk(hidden).u);
}
// CB3 rows whose pass the 512-thread workgroup stages, two workgroups per CU, and whose two
// engines fit the registers (chunks of at most 5 blocks, or double-buffered chunks of 2)
static bool gu_pair_host(int wt, int64_t hidden) {
    const Chunk ch = gu_chunk(hidden);
    return wt == QMM_CB3 && (ch.multi || ch.u <= 5) && gu_slots(true, hidden) != 0 &&
           gu_lds_bytes(true, hidden) <= kGuPairLds;
}
static int down_slots(int wt, int64_t inter) {
    return stage_slots(inter, kGroupPass, down_threads_host(wt, down_chunk(inter)), kGemvLanesPerRow,
                       down_chunk(inter).u);
}
static size_t align16(size_t v) { return (v + 15) & ~(size_t)15; }

static int launch_grouped(const GroupedArgs& a) {
    const uint32_t gu_bytes = (uint32_t)(a.inter * qmm_row_bytes(a.wtype_gu, a.hidden));
    const uint32_t d_bytes = (uint32_t)(a.hidden * qmm_row_bytes(a.wtype_down, a.inter));
    const size_t hbytes = grouped_h_bytes(a.inter, a.nentries);
    float* dbg_g = nullptr;
    float* dbg_u = nullptr;
    if (a.flags & QMM_FLAG_DEBUG_INTERMEDIATES) {
        dbg_g = (float*)(a.ws + align16(hbytes));
        dbg_u = dbg_g + (size_t)a.nentries * a.inter;
    }
    const uint32_t xqbytes = (uint32_t)((uint64_t)a.xq_cols * (a.hidden / 32) * 36);
    {
        const bool pair = gu_pair_host(a.wtype_gu, a.hidden);
        const size_t lds = gu_lds_bytes(pair, a.hidden);
        const dim3 grid_dim((unsigned)(a.inter / 32), (unsigned)a.ngroups);
        // at most 8 activation columns: load them all before the group lookup
        const bool dense = a.xq_cols <= kGroupPass;
        auto launch = [&](auto kern, int threads) {
            hipLaunchKernelGGL(kern, grid_dim, dim3(threads), lds, a.st, a.w_gate, a.w_up, a.gu_stride, gu_bytes,
                               a.nexperts, a.grid, (int)a.hidden, (int)a.inter, a.xq, xqbytes, a.xq_cols,
                               a.group_expert, a.group_off, a.entry_col, a.nentries, a.ws, dbg_g, dbg_u);
        };
        auto go = [&](auto wt_c, auto u_c, auto multi_c, auto ns_c) {
            constexpr int WT = decltype(wt_c)::value, U = decltype(u_c)::value, NS = decltype(ns_c)::value;
            constexpr bool MULTI = decltype(multi_c)::value;
            if constexpr (WT == kCB3 && (MULTI || U <= 5)) {
                if (pair) {
                    launch(dense ? gu_kernel<WT, U, MULTI, NS, true, true> : gu_kernel<WT, U, MULTI, NS, false, true>,
                           gu_threads<true>());
                    return;
                }
            }
            launch(dense ? gu_kernel<WT, U, MULTI, NS, true, false> : gu_kernel<WT, U, MULTI, NS, false, false>,
                   gu_threads<false>());
        };
        const Chunk ch = gu_chunk(a.hidden);
        const int ns = gu_slots(pair, a.hidden);
        if (a.wtype_gu == QMM_Q8_0) dispatch_u_ns<kQ8_0, 2>(ch, ns, go);
        else if (a.wtype_gu == QMM_IQ4_NL) dispatch_u_ns<kIQ4_NL, 2>(ch, ns, go);
        else dispatch_u_ns<kCB3, 2>(ch, ns, go);
        const int rc = launch_status();
        if (rc) return rc;
    }
    {
        const size_t lds = down_lds_bytes(a.wtype_down, a.inter);
        const dim3 grid_dim((unsigned)((a.hidden + kDownRows - 1) / kDownRows), (unsigned)a.ngroups);
        auto go = [&](auto wt_c, auto u_c, auto multi_c, auto ns_c) {
            constexpr int WT = decltype(wt_c)::value, U = decltype(u_c)::value, NS = decltype(ns_c)::value;
            constexpr bool MULTI = decltype(multi_c)::value;
            hipLaunchKernelGGL((down_kernel<WT, U, MULTI, NS>), grid_dim, dim3(down_threads<WT, U, MULTI>()), lds, a.st,
                               a.w_down,
                               a.d_stride, d_bytes, a.nexperts, a.grid, (int)a.hidden, (int)a.inter, a.ws,
                               (uint32_t)hbytes, a.group_expert, a.group_off, a.nentries, a.y);
        };
        const Chunk ch = down_chunk(a.inter);
        const int ns = down_slots(a.wtype_down, a.inter);
        if (a.wtype_down == QMM_Q8_0) dispatch_u_ns<kQ8_0>(ch, ns, go);
        else if (a.wtype_down == QMM_IQ4_NL) dispatch_u_ns<kIQ4_NL>(ch, ns, go);
        else dispatch_u_ns<kCB3>(ch, ns, go);
        return launch_status();
    }
}

// ------------------------------------------------------------------ allocation-free variant
//
// For callers that cannot allocate (code under graph capture, serving loops): H lives in a
// file-scope device array.  In host code `scratch` names a host-side stand-in, not the device
// array, so host code never passes it to a kernel: the device address is taken once per device
// with hipGetSymbolAddress (with that device current) and used from then on.  Every call on a
// device shares its array; calls that overlap on one device race.
constexpr size_t kNoAllocScratchBytes = (size_t)4 << 20;  // H of 3640 entries at inter 1024
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

// The device address of `scratch` on the current device (nullptr if it cannot be had).
static void* scratch_ptr() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

}  // namespace qmm

using namespace qmm;

extern "C" size_t qgemv_grouped_experts_workspace(int64_t inter, int nentries, unsigned flags) {
    if (inter <= 0 || nentries < 0) return 0;
    size_t b = align16(grouped_h_bytes(inter, nentries));
    if (flags & QMM_FLAG_DEBUG_INTERMEDIATES) b += 2 * (size_t)nentries * (size_t)inter * sizeof(float);
    return b;
}

// Argument checks shared by both entry points (everything but the workspace), then the call.
static int grouped_call(int wtype_gu, const void* w_gate, const void* w_up, int64_t gu_expert_stride, int wtype_down,
                        const void* w_down, int64_t down_expert_stride, int nexperts, const uint8_t* grid, int64_t hidden,
                        int64_t inter, const void* xq, int xq_cols, const int32_t* group_expert,
                        const int32_t* group_entry_off, int ngroups, const int32_t* entry_col, int nentries, float* y,
                        void* ws, size_t ws_bytes, unsigned flags, void* stream) {
    if (!valid_wtype(wtype_gu) || !valid_wtype(wtype_down)) return QMM_EINVAL;
    if (!w_gate || !w_up || !w_down || !xq || !group_expert || !group_entry_off || !entry_col || !y || !ws)
        return QMM_EINVAL;
    if ((wtype_gu == QMM_CB3 || wtype_down == QMM_CB3) && !grid) return QMM_EINVAL;
    if (nexperts < 1 || ngroups < 0 || nentries < 0 || xq_cols < 1 || hidden < 32 || inter < 32) return QMM_EINVAL;
    if (qmm_row_bytes(wtype_gu, hidden) == 0 || qmm_row_bytes(wtype_down, inter) == 0) return QMM_EINVAL;
    if (hidden > kMaxK || inter > kMaxK || ngroups > 65535) return QMM_EUNSUPPORTED;
    const int64_t gu_bytes = inter * qmm_row_bytes(wtype_gu, hidden);
    const int64_t d_bytes = hidden * qmm_row_bytes(wtype_down, inter);
    if (gu_expert_stride < gu_bytes || down_expert_stride < d_bytes) return QMM_EINVAL;
    if (gu_expert_stride % 4 || down_expert_stride % 4) return QMM_EALIGN;
    if (!aligned(w_gate, 4) || !aligned(w_up, 4) || !aligned(w_down, 4) || !aligned(xq, 4) || !aligned(y, 4) ||
        !aligned(ws, 16))
        return QMM_EALIGN;
    // a pass of 8 entries must fit the workgroup's LDS and staging slots
    const bool pair = gu_pair_host(wtype_gu, hidden);
    if (gu_lds_bytes(pair, hidden) > kLdsCap || down_lds_bytes(wtype_down, inter) > kLdsCap ||
        gu_slots(pair, hidden) == 0 || down_slots(wtype_down, inter) == 0)
        return QMM_EUNSUPPORTED;
    if ((uint64_t)xq_cols * (hidden / 32) * 36 > kMaxActBytes || grouped_h_bytes(inter, nentries) > kMaxActBytes)
        return QMM_EUNSUPPORTED;
    if (ws_bytes < qgemv_grouped_experts_workspace(inter, nentries, flags)) return QMM_ESPACE;
    if (ngroups == 0 || nentries == 0) return QMM_OK;
    GroupedArgs a;
    a.wtype_gu = wtype_gu;
    a.wtype_down = wtype_down;
    a.nexperts = nexperts;
    a.ngroups = ngroups;
    a.nentries = nentries;
    a.xq_cols = xq_cols;
    a.w_gate = (const uint8_t*)w_gate;
    a.w_up = (const uint8_t*)w_up;
    a.w_down = (const uint8_t*)w_down;
    a.grid = grid;
    a.xq = (const uint8_t*)xq;
    a.gu_stride = gu_expert_stride;
    a.d_stride = down_expert_stride;
    a.hidden = hidden;
    a.inter = inter;
    a.group_expert = group_expert;
    a.group_off = group_entry_off;
    a.entry_col = entry_col;
    a.y = y;
    a.ws = (uint8_t*)ws;
    a.flags = flags;
    a.st = as_stream(stream);
    return launch_grouped(a);
}

extern "C" int qgemv_grouped_experts(int wtype_gu, const void* w_gate, const void* w_up, int64_t gu_expert_stride,
                                     int wtype_down, const void* w_down, int64_t down_expert_stride, int nexperts,
                                     const uint8_t* grid, int64_t hidden, int64_t inter, const void* xq, int xq_cols,
                                     const int32_t* group_expert, const int32_t* group_entry_off, int ngroups,
                                     const int32_t* entry_col, int nentries, float* y, void* ws, size_t ws_bytes,
                                     unsigned flags, void* stream) {
    return grouped_call(wtype_gu, w_gate, w_up, gu_expert_stride, wtype_down, w_down, down_expert_stride, nexperts,
                        grid, hidden, inter, xq, xq_cols, group_expert, group_entry_off, ngroups, entry_col, nentries,
                        y, ws, ws_bytes, flags, stream);
}

extern "C" size_t qgemv_grouped_experts_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

extern "C" int qgemv_grouped_experts_noalloc(int wtype_gu, const void* w_gate, const void* w_up,
                                             int64_t gu_expert_stride, int wtype_down, const void* w_down,
                                             int64_t down_expert_stride, int nexperts, const uint8_t* grid,
                                             int64_t hidden, int64_t inter, const void* xq, int xq_cols,
                                             const int32_t* group_expert, const int32_t* group_entry_off,
                                             int ngroups, const int32_t* entry_col, int nentries, float* y,
                                             void* stream) {
    if (inter < 32 || nentries < 0) return QMM_EINVAL;
    if (qgemv_grouped_experts_workspace(inter, nentries, 0) > kNoAllocScratchBytes) return QMM_ESPACE;
    void* ws = scratch_ptr();
    if (!ws) return QMM_EHIP;
    return grouped_call(wtype_gu, w_gate, w_up, gu_expert_stride, wtype_down, w_down, down_expert_stride, nexperts,
                        grid, hidden, inter, xq, xq_cols, group_expert, group_entry_off, ngroups, entry_col, nentries,
                        y, ws, kNoAllocScratchBytes, 0u, stream);
}
