// qmm_prefill.hip -- prefill grouped expert GEMM for gfx950: weights dequantized to FP16 in LDS,
// fp16 MFMA with fp32 sums, SwiGLU epilogue, down GEMM.
//
// Method [PF, Summary: each K chunk of an expert's weight rows is dequantized into shared memory
// and fed to FP16 matrix math over the rows sorted per expert; the FP16 weights are the
// standalone dequantizer's, in the same k order; an expert's last partial tile is masked]:
//   schedule kernel : expert_off -> a list of (expert, first row, rows) tiles of <= 128 sorted rows
//   gate/up kernel  : tile x 64 intermediate columns: G, U = X16[tok] . W16^T for the gate and up
//                     rows of those columns (128 B rows), K in steps of 32; epilogue
//                     H16 = fp16(silu(G) * U)
//   down kernel     : tile x 128 output columns: Y = H16 . Wd16^T
// Every K step: the 128 x 32 activation chunk is copied and the 128 weight blocks dequantized
// into LDS in the MFMA fragment order (lane l of a fragment holds row l % 32, k 8*(l/32)..+7),
// then each of the 4 waves runs v_mfma_f32_32x32x16_f16 on its 32 rows x 128 columns.  The
// next step's global loads are issued before the MFMAs so their latency hides behind them.
// Dequantized values: the integer factor times the fp16 scale (times the CB3 multiplier) is
// exact in binary32, one v_cvt_f16_f32 rounds it to nearest even: the same bits as
// qmm_dequant_f16.
#include "qmm_gemv.h"

namespace qmm {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kPfBM = 128;      // rows per tile
constexpr int kPfThreads = 256; // 4 waves, 32 rows each
constexpr int kPfBK = 32;       // k per step (one 32-value block per weight row)
constexpr int kPfBNRows = 128;  // weight rows per tile (gate 64 + up 64, or 128 down rows)

struct Tile {
    int e, row0, nrows;
};

// ---------------------------------------------------------------- schedule

__global__ __launch_bounds__(1024) void schedule_kernel(const int32_t* __restrict__ expert_off, int nexperts, int nentries,
                                                        int32_t* __restrict__ tiles, int max_tiles) {
    __shared__ int scan[1024];
    __shared__ int base;
    if (threadIdx.x == 0) base = 0;
    __syncthreads();
    for (int e0 = 0; e0 < nexperts; e0 += 1024) {
        const int e = e0 + (int)threadIdx.x;
        int o0 = 0, o1 = 0;
        if (e < nexperts) {
            o0 = expert_off[e];
            o1 = expert_off[e + 1];
            o0 = o0 < 0 ? 0 : (o0 > nentries ? nentries : o0);
            o1 = o1 < o0 ? o0 : (o1 > nentries ? nentries : o1);
        }
        const int n = (o1 - o0 + kPfBM - 1) / kPfBM;
        scan[threadIdx.x] = n;
        __syncthreads();
        for (int s = 1; s < 1024; s <<= 1) {  // inclusive scan
            const int v = threadIdx.x >= (unsigned)s ? scan[threadIdx.x - s] : 0;
            __syncthreads();
            scan[threadIdx.x] += v;
            __syncthreads();
        }
        const int first = base + scan[threadIdx.x] - n;
        for (int i = 0; i < n; ++i) {
            const int t = first + i;
            if (t < max_tiles) {
                tiles[1 + 3 * t] = e;
                tiles[2 + 3 * t] = o0 + i * kPfBM;
                tiles[3 + 3 * t] = (o1 - o0 - i * kPfBM) < kPfBM ? (o1 - o0 - i * kPfBM) : kPfBM;
            }
        }
        __syncthreads();
        if (threadIdx.x == 1023) base += scan[1023];
        __syncthreads();
    }
    if (threadIdx.x == 0) tiles[0] = base < max_tiles ? base : max_tiles;
}

// ---------------------------------------------------------------- dequant of 16 values

// Raw bytes a thread needs for values [16h, 16h+16) of block kb of a weight row.
template <int WT>
struct DqRaw;

template <>
struct DqRaw<kQ8_0> {
    uint32_t w[5];
    uint32_t d;
    __device__ __forceinline__ void load(rsrc_t r, uint32_t row_off, int kb, int h, int) {
        const uint32_t blk = row_off + (uint32_t)kb * 34u;
        const uint32_t o = blk + 2u + 16u * h;
        const u32x4 x = ld128(r, o & ~3u);
        w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
        w[4] = ld32(r, (o & ~3u) + 16u);
        d = ld16(r, blk);
    }
    // int8 factors (4 dwords) and the binary32 multiplier of the integer factor
    __device__ __forceinline__ void decode(uint32_t row_off, int kb, int h, const uint32_t*, uint32_t* q, float& dm) const {
        const uint32_t sh = (row_off + (uint32_t)kb * 34u + 2u + 16u * h) & 3u;
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = align8(w[i + 1], w[i], sh);
        dm = h2f(d);
    }
};

template <>
struct DqRaw<kIQ4_NL> {
    uint32_t w[5];
    __device__ __forceinline__ void load(rsrc_t r, uint32_t row_off, int kb, int, int) {
        Unit<kIQ4_NL>::load(r, row_off + (uint32_t)kb * 18u, w);
    }
    __device__ __forceinline__ void decode(uint32_t row_off, int kb, int h, const uint32_t*, uint32_t* q, float& dm) const {
        const uint32_t off = row_off + (uint32_t)kb * 18u;
        const uint32_t sel = realign_sel(off);
        const IQ4Consts k;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t x = perm(w[i + 1], w[i], sel) >> (4 * h);  // low or high nibbles
            q[i] = iq4nl_lookup(x & k.m7, ((x >> 1) & k.m4) | k.c0123);
        }
        dm = h2f(realign_scale(w[0], off));
    }
};

template <>
struct DqRaw<kCB3> {
    uint32_t w[Unit<kCB3>::RAW];
    __device__ __forceinline__ void load(rsrc_t r, uint32_t row_off, int kb, int, int) {
        Unit<kCB3>::load(r, row_off + (uint32_t)(kb >> 3) * kCB3Bytes, kb & 7, w);
    }
    __device__ __forceinline__ void decode(uint32_t row_off, int kb, int h, const uint32_t* grid, uint32_t* q,
                                           float& dm) const {
        uint32_t W[8], dw;
        int mult;
        Unit<kCB3>::decode(w, row_off + (uint32_t)(kb >> 3) * kCB3Bytes, kb & 7, grid, W, dw, mult);
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = W[4 * h + i];
        dm = h2f(dw) * (float)mult;  // exact: 11 + 5 significant bits
    }
};

// 4 dwords of int8 factors times dm -> 16 binary16 values (8 dwords).  (float)(q + 128) is exact,
// fma(dm, u, -128 dm) = dm * q exactly (at most 24 significant bits), one RNE to binary16.
__device__ __forceinline__ void to_f16x16(const uint32_t* q, float dm, uint32_t* out) {
    const float nb = -128.0f * dm;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t u = q[i] ^ 0x80808080u;
        uint32_t h[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const float v = __builtin_fmaf(dm, (float)((u >> (8 * b)) & 0xFFu), nb);
            h[b] = f2h(opaque(v));
        }
        out[2 * i] = h[0] | (h[1] << 16);
        out[2 * i + 1] = h[2] | (h[3] << 16);
    }
}

// LDS fragment offset (in 16-byte units) of (row-or-column block `blk`, k half `kh`, lane).
__device__ __forceinline__ int frag16(int blk, int kh, int lane) { return (blk * 2 + kh) * 64 + lane; }

// ---------------------------------------------------------------- the GEMM core

// A chunk loader: the 128 x 32 fp16 chunk of step ks; thread t owns rows t/4 and t/4 + 64,
// 8-value chunk t % 4 of each.
struct AChunk {
    u32x4 v[2];
    __device__ __forceinline__ void load(rsrc_t ar, const uint32_t* row_byte_off, int ks) {
        const uint32_t koff = (uint32_t)ks * (kPfBK * 2) + (threadIdx.x & 3u) * 16u;
        v[0] = ld128(ar, row_byte_off[0] + koff);
        v[1] = ld128(ar, row_byte_off[1] + koff);
    }
    __device__ __forceinline__ void store(u32x4* lds_a) const {
        const int c = threadIdx.x & 3;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int r = (int)(threadIdx.x >> 2) + 64 * s;
            lds_a[frag16(r >> 5, c >> 1, (r & 31) + 32 * (c & 1))] = v[s];
        }
    }
};

// B chunk: 128 weight rows x 32 values; thread t owns weight row t/2, values 16(t%2)..+15.
template <int WT>
struct BChunk {
    DqRaw<WT> raw;
    __device__ __forceinline__ void load(rsrc_t wr, uint32_t row_off, int ks) {
        raw.load(wr, row_off, ks, (int)(threadIdx.x & 1u), 0);
    }
    __device__ __forceinline__ void store(uint32_t row_off, int ks, const uint32_t* grid, u32x4* lds_b) const {
        const int h = threadIdx.x & 1;
        const int jr = threadIdx.x >> 1;
        uint32_t q[4], f[8];
        float dm;
        raw.decode(row_off, ks, h, grid, q, dm);
        to_f16x16(q, dm, f);
        const int cb = jr >> 5, j = jr & 31;
        lds_b[frag16(cb, h, j)] = u32x4{f[0], f[1], f[2], f[3]};
        lds_b[frag16(cb, h, j + 32)] = u32x4{f[4], f[5], f[6], f[7]};
    }
};

// Runs the K loop of one tile: acc[cb] (cb = 0..3, 32 columns each) of this wave's 32 rows.
template <int WT>
__device__ __forceinline__ void gemm_tile(rsrc_t ar, const uint32_t* a_row_off, rsrc_t wr, uint32_t b_row_off, int nk,
                                          const uint32_t* grid, u32x4* lds_a, u32x4* lds_b, f32x16 (&acc)[4]) {
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[cb] = f32x16{};
    AChunk a;
    BChunk<WT> b;
    a.load(ar, a_row_off, 0);
    b.load(wr, b_row_off, 0);
    for (int ks = 0; ks < nk; ++ks) {
        a.store(lds_a);
        b.store(b_row_off, ks, grid, lds_b);
        __syncthreads();
        if (ks + 1 < nk) {
            a.load(ar, a_row_off, ks + 1);
            b.load(wr, b_row_off, ks + 1);
        }
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
            const half8 av = __builtin_bit_cast(half8, lds_a[frag16(w, kh, lane)]);
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                const half8 bv = __builtin_bit_cast(half8, lds_b[frag16(cb, kh, lane)]);
                acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bv, acc[cb], 0, 0, 0);
            }
        }
        __syncthreads();
    }
}

__device__ __forceinline__ bool load_tile(const int32_t* tiles, Tile& t) {
    const int n = __builtin_amdgcn_readfirstlane(tiles[0]);
    if ((int)blockIdx.x >= n) return false;
    t.e = __builtin_amdgcn_readfirstlane(tiles[1 + 3 * blockIdx.x]);
    t.row0 = __builtin_amdgcn_readfirstlane(tiles[2 + 3 * blockIdx.x]);
    t.nrows = __builtin_amdgcn_readfirstlane(tiles[3 + 3 * blockIdx.x]);
    return true;
}

// Row (within the tile) and column (within the 32-column block) of accumulator register r.
__device__ __forceinline__ int acc_row(int lane, int r) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

template <int WT>
__global__ __launch_bounds__(kPfThreads) void pf_gateup_kernel(
    const uint8_t* __restrict__ wg, const uint8_t* __restrict__ wu, int64_t gu_stride, uint32_t expert_bytes,
    int nexperts, const uint8_t* __restrict__ grid, int hidden, int inter, const uint16_t* __restrict__ x16,
    uint32_t xbytes, int ntok, const int32_t* __restrict__ sorted_tok, const int32_t* __restrict__ tiles,
    uint16_t* __restrict__ h16, float* __restrict__ dbg_g, float* __restrict__ dbg_u) {
    __shared__ u32x4 lds_a[kPfBM * kPfBK * 2 / 16];
    __shared__ u32x4 lds_b[kPfBNRows * kPfBK * 2 / 16];
    __shared__ uint32_t lds_grid[WT == kCB3 ? 512 : 1];
    Tile t;
    if (!load_tile(tiles, t) || t.e < 0 || t.e >= nexperts) return;
    if constexpr (WT == kCB3) {
        stage_grid(grid, lds_grid);
        __syncthreads();
    }
    // this thread's two activation rows (token gather; rows past the tile read zeros)
    uint32_t a_off[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const int r = (int)(threadIdx.x >> 2) + 64 * s;
        int tok = r < t.nrows ? sorted_tok[t.row0 + r] : -1;
        a_off[s] = (tok >= 0 && tok < ntok) ? (uint32_t)tok * (uint32_t)hidden * 2u : xbytes;
    }
    // this thread's weight row: gate rows 0..63, up rows 64..127 of the tile
    const int jr = threadIdx.x >> 1;
    const int col = blockIdx.y * 64 + (jr & 63);
    const uint8_t* wbase = (jr < 64 ? wg : wu) + t.e * gu_stride;
    const rsrc_t wr = make_rsrc_dw(wbase, expert_bytes);
    const uint32_t b_row_off = (uint32_t)col * (uint32_t)row_bytes_dev<WT>(hidden);
    f32x16 acc[4];
    gemm_tile<WT>(make_rsrc(x16, xbytes), a_off, wr, b_row_off, hidden / kPfBK, lds_grid, lds_a, lds_b, acc);

    // epilogue: acc[0..1] gate, acc[2..3] up for columns 64 y + 32 cb + lane % 32
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
        const int c = blockIdx.y * 64 + 32 * cb + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = 32 * w + acc_row(lane, r);
            if (row < t.nrows) {
                const int64_t p = t.row0 + row;
                const float gv = acc[cb][r], uv = acc[cb + 2][r];
                const float hv = [&] {
                    const float e = (float)exp(-(double)gv);
                    const float den = opaque(1.0f + e);
                    const float sl = opaque(gv / den);
                    return opaque(sl * uv);
                }();
                h16[p * inter + c] = (uint16_t)f2h(hv);
                if (dbg_g) {
                    dbg_g[p * inter + c] = gv;
                    dbg_u[p * inter + c] = uv;
                }
            }
        }
    }
}

template <int WT>
__global__ __launch_bounds__(kPfThreads) void pf_down_kernel(const uint8_t* __restrict__ wd, int64_t d_stride,
                                                             uint32_t expert_bytes, int nexperts,
                                                             const uint8_t* __restrict__ grid, int hidden, int inter,
                                                             const uint16_t* __restrict__ h16, uint32_t hbytes,
                                                             const int32_t* __restrict__ tiles, float* __restrict__ y) {
    __shared__ u32x4 lds_a[kPfBM * kPfBK * 2 / 16];
    __shared__ u32x4 lds_b[kPfBNRows * kPfBK * 2 / 16];
    __shared__ uint32_t lds_grid[WT == kCB3 ? 512 : 1];
    Tile t;
    if (!load_tile(tiles, t) || t.e < 0 || t.e >= nexperts) return;
    if constexpr (WT == kCB3) {
        stage_grid(grid, lds_grid);
        __syncthreads();
    }
    uint32_t a_off[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const int r = (int)(threadIdx.x >> 2) + 64 * s;
        a_off[s] = r < t.nrows ? (uint32_t)(t.row0 + r) * (uint32_t)inter * 2u : hbytes;
    }
    const int jr = threadIdx.x >> 1;
    const int col = blockIdx.y * 128 + jr;
    const rsrc_t wr = make_rsrc_dw(wd + t.e * d_stride, expert_bytes);
    const uint32_t b_row_off = (uint32_t)(col < hidden ? col : hidden - 1) * (uint32_t)row_bytes_dev<WT>(inter);
    f32x16 acc[4];
    gemm_tile<WT>(make_rsrc(h16, hbytes), a_off, wr, b_row_off, inter / kPfBK, lds_grid, lds_a, lds_b, acc);

    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
        const int c = blockIdx.y * 128 + 32 * cb + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = 32 * w + acc_row(lane, r);
            if (row < t.nrows && c < hidden) y[(int64_t)(t.row0 + row) * hidden + c] = acc[cb][r];
        }
    }
}

static size_t align16(size_t v) { return (v + 15) & ~(size_t)15; }
static int64_t max_tiles_of(int nexperts, int64_t nentries) { return (nentries + kPfBM - 1) / kPfBM + nexperts; }

struct PfLayout {
    size_t h_off, tiles_off, g_off, u_off, total;
};
static PfLayout pf_layout(int nexperts, int64_t inter, int64_t nentries, unsigned flags) {
    PfLayout l;
    l.h_off = 0;
    l.tiles_off = align16((size_t)nentries * (size_t)inter * 2);
    l.g_off = align16(l.tiles_off + 4 * (size_t)(1 + 3 * max_tiles_of(nexperts, nentries)));
    l.u_off = l.g_off;
    l.total = l.g_off;
    if (flags & QMM_FLAG_DEBUG_INTERMEDIATES) {
        l.u_off = l.g_off + (size_t)nentries * (size_t)inter * 4;
        l.total = l.u_off + (size_t)nentries * (size_t)inter * 4;
    }
    return l;
}

}  // namespace qmm

using namespace qmm;

extern "C" size_t qgemm_prefill_experts_workspace(int nexperts, int64_t inter, int64_t nentries, unsigned flags) {
    if (nexperts < 1 || inter < 1 || nentries < 0) return 0;
    return pf_layout(nexperts, inter, nentries, flags).total;
}

extern "C" int qgemm_prefill_experts(int wtype_gu, const void* w_gate, const void* w_up, int64_t gu_expert_stride,
                                     int wtype_down, const void* w_down, int64_t down_expert_stride, int nexperts,
                                     int64_t hidden, int64_t inter, const uint16_t* x_f16, int64_t ntok,
                                     const int32_t* sorted_tok, const int32_t* expert_off, int64_t nentries, float* y,
                                     void* ws, size_t ws_bytes, unsigned flags, void* stream) {
    if (!valid_wtype(wtype_gu) || !valid_wtype(wtype_down)) return QMM_EINVAL;
    if (!w_gate || !w_up || !w_down || !x_f16 || !sorted_tok || !expert_off || !y || !ws) return QMM_EINVAL;
    if (nexperts < 1 || hidden < 32 || inter < 32 || ntok < 1 || nentries < 0) return QMM_EINVAL;
    if (qmm_row_bytes(wtype_gu, hidden) == 0 || qmm_row_bytes(wtype_down, inter) == 0) return QMM_EINVAL;
    if (wtype_gu == QMM_CB3 || wtype_down == QMM_CB3) return QMM_EUNSUPPORTED;  // no codebook argument here
    if (hidden % 128 || inter % 64) return QMM_EUNSUPPORTED;
    const int64_t gu_bytes = inter * qmm_row_bytes(wtype_gu, hidden);
    const int64_t d_bytes = hidden * qmm_row_bytes(wtype_down, inter);
    if (gu_expert_stride < gu_bytes || down_expert_stride < d_bytes) return QMM_EINVAL;
    if (gu_expert_stride % 4 || down_expert_stride % 4) return QMM_EALIGN;
    if (!aligned(w_gate, 4) || !aligned(w_up, 4) || !aligned(w_down, 4) || !aligned(x_f16, 16) || !aligned(y, 4) ||
        !aligned(ws, 16))
        return QMM_EALIGN;
    if ((uint64_t)ntok * hidden * 2 > kMaxBufferBytes || (uint64_t)nentries * inter * 2 > kMaxBufferBytes ||
        gu_bytes > (int64_t)kMaxBufferBytes || d_bytes > (int64_t)kMaxBufferBytes || nentries > 0x7FFFFFFF)
        return QMM_EUNSUPPORTED;
    const PfLayout lay = pf_layout(nexperts, inter, nentries, flags);
    if (ws_bytes < lay.total) return QMM_ESPACE;
    if (nentries == 0) return QMM_OK;
    const hipStream_t st = as_stream(stream);
    uint8_t* wsb = (uint8_t*)ws;
    uint16_t* h16 = (uint16_t*)(wsb + lay.h_off);
    int32_t* tiles = (int32_t*)(wsb + lay.tiles_off);
    float* dbg_g = (flags & QMM_FLAG_DEBUG_INTERMEDIATES) ? (float*)(wsb + lay.g_off) : nullptr;
    float* dbg_u = (flags & QMM_FLAG_DEBUG_INTERMEDIATES) ? (float*)(wsb + lay.u_off) : nullptr;
    const int64_t max_tiles = max_tiles_of(nexperts, nentries);
    if (max_tiles > 0x7FFFFFFF) return QMM_EUNSUPPORTED;

    hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(1024), 0, st, expert_off, nexperts, (int)nentries, tiles,
                       (int)max_tiles);
    int rc = launch_status();
    if (rc) return rc;
    const uint32_t xbytes = (uint32_t)(ntok * hidden * 2);
    const uint32_t hbytes = (uint32_t)(nentries * inter * 2);
    {
        const dim3 g((unsigned)max_tiles, (unsigned)(inter / 64));
        auto go = [&](auto kern) {
            hipLaunchKernelGGL(kern, g, dim3(kPfThreads), 0, st, (const uint8_t*)w_gate, (const uint8_t*)w_up,
                               gu_expert_stride, (uint32_t)gu_bytes, nexperts, (const uint8_t*)nullptr, (int)hidden,
                               (int)inter, x_f16, xbytes, (int)ntok, sorted_tok, tiles, h16, dbg_g, dbg_u);
        };
        if (wtype_gu == QMM_Q8_0) go(pf_gateup_kernel<kQ8_0>);
        else go(pf_gateup_kernel<kIQ4_NL>);
        rc = launch_status();
        if (rc) return rc;
    }
    {
        const dim3 g((unsigned)max_tiles, (unsigned)(hidden / 128));
        auto go = [&](auto kern) {
            hipLaunchKernelGGL(kern, g, dim3(kPfThreads), 0, st, (const uint8_t*)w_down, down_expert_stride,
                               (uint32_t)d_bytes, nexperts, (const uint8_t*)nullptr, (int)hidden, (int)inter, h16,
                               hbytes, tiles, y);
        };
        if (wtype_down == QMM_Q8_0) go(pf_down_kernel<kQ8_0>);
        else go(pf_down_kernel<kIQ4_NL>);
        return launch_status();
    }
}
