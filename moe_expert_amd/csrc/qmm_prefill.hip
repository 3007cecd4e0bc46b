// qmm_prefill.hip -- prefill grouped expert GEMM for gfx950: quantized expert weights converted
// to FP16 in registers, fp16 MFMA with fp32 sums, SwiGLU epilogue, down GEMM.
//
// Method [PF, Summary: the weights of an expert are dequantized to FP16 chunk by chunk and fed
// to FP16 matrix math over the token rows sorted per expert; the FP16 weights are the standalone
// dequantizer's; an expert's partial last tile is masked]:
//   schedule kernel : expert_off -> (expert, first row, rows) tiles; an expert's rows are split
//                     into ceil(n/T) tiles of equal size rounded up to 32 rows (T = 256 here,
//                     128 in the MMQ-style path)
//   gate/up kernel  : tile x 128 intermediate columns: G, U = X16[tok] . W16^T for the gate and
//                     up rows of those columns; epilogue H16 = fp16(silu(G) * U)
//   down kernel     : tile x 256 output columns: Y = H16 . Wd16^T
//
// Workgroup: 8 waves, two per SIMD, so one wave's conversion work, loads and waits run while
// the other's MFMAs occupy the matrix unit.  Wave w owns 32 weight rows (one 32-column MFMA
// block) and every row of the tile (up to 8 blocks of 32 rows, 128 accumulator registers); it
// converts only its own weights, straight into the B operand of v_mfma_f32_32x32x16_f16, one
// k16 fragment ahead of its use.  Only the activations are shared, through LDS.  K advances 64
// values (two quantized blocks) per step:
//   - activations: 256 rows x 64 fp16 (32 KiB) per step in four LDS stages (128 KiB), loaded
//     straight into LDS (buffer_load ... lds) three steps ahead, in a row-major layout whose
//     16-byte chunks are XOR-swizzled by the row (no bank conflicts for the fragment reads);
//     fragment reads run one k16 slice ahead, across step boundaries; one barrier per step;
//   - weights: each lane pair reads its row's two blocks of a step once (one block per lane)
//     and trades halves through v_permlane32_swap; the raw bytes for step s + 3 are loaded
//     in the last slice of step s, into the registers of step s + 1 (prepared just before).
// Lane l of a 32x32x16 fragment holds row (or column) l % 32 and k = 8 (l / 32) + 0..7; the
// accumulator register r of lane l holds row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32.
// Weight values: the integer factor as an exact binary16 integer times the binary16 scale in
// one packed multiply, i.e. the exact product rounded once to nearest even (qmm_dequant_f16
// uses the same conversion).
#include "qmm_gemv.h"

#include <algorithm>

namespace qmm {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kPfRows = 256;                      // rows per tile (8 MFMA blocks of 32)
constexpr int kPfThreads = 512;                   // 8 waves
constexpr int kPfStepK = 64;                      // k per step: two 32-value blocks
constexpr int kPfStage = kPfRows * kPfStepK * 2;  // LDS bytes of one activation stage
constexpr int kPfGuCols = 128;                    // intermediate columns per gate/up workgroup
constexpr int kPfDownCols = 256;                  // output columns per down workgroup

struct Tile {
    int e, row0, nrows;
};

// ---------------------------------------------------------------- schedule

__global__ __launch_bounds__(1024) void schedule_kernel(const int32_t* __restrict__ expert_off, int nexperts, int nentries,
                                                        int32_t* __restrict__ tiles, int max_tiles, int tile_rows) {
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
        const int rows = o1 - o0;
        int per = 0, n = 0;
        if (rows > 0) {
            const int t = (rows + tile_rows - 1) / tile_rows;
            per = ((rows + t - 1) / t + 31) & ~31;  // <= tile_rows, >= rows / t
            n = (rows + per - 1) / per;             // <= t
        }
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
                tiles[2 + 3 * t] = o0 + i * per;
                tiles[3 + 3 * t] = rows - i * per < per ? rows - i * per : per;
            }
        }
        __syncthreads();
        if (threadIdx.x == 1023) base += scan[1023];
        __syncthreads();
    }
    if (threadIdx.x == 0) tiles[0] = base < max_tiles ? base : max_tiles;
}

// Workgroup -> (tile, column tile).  Workgroups are handed to the 8 XCDs round robin; XCD c
// takes a contiguous run of tiles (mostly of one expert) and all column tiles of each, so an
// activation tile and an expert's weight slices are reused from that XCD's L2.
__device__ __forceinline__ bool pf_tile(const int32_t* tiles, int ny, Tile& t, int& y) {
    const int n = __builtin_amdgcn_readfirstlane(tiles[0]);
    const int per_xcd = (n + 7) >> 3;
    const int c = (int)(blockIdx.x & 7u), q = (int)(blockIdx.x >> 3);
    const int xi = q / ny;
    y = q - xi * ny;
    const int x = c * per_xcd + xi;
    if (xi >= per_xcd || x >= n) return false;
    t.e = __builtin_amdgcn_readfirstlane(tiles[1 + 3 * x]);
    t.row0 = __builtin_amdgcn_readfirstlane(tiles[2 + 3 * x]);
    t.nrows = __builtin_amdgcn_readfirstlane(tiles[3 + 3 * x]);
    return true;
}

// ---------------------------------------------------------------- weights -> B fragments
//
// A lane's weight row contributes, per step, the values 8 h .. 8 h + 7 (fragment j = 2 bi) and
// 16 + 8 h .. + 7 (fragment j = 2 bi + 1) of its two quantized blocks bi = 0, 1, h = lane / 32.
// Loading: lane l < 32 reads block 0 of its row whole, lane l + 32 block 1 (adjacent bytes), so
// a load instruction touches each row's step bytes once; prepare() realigns the block and
// trades halves with the partner lane through v_permlane32_swap (the low half-wave keeps bytes
// 0..7 of each 16-byte run, the high half-wave bytes 8..15), giving every lane its bytes of
// both blocks.  convert(j, i) then produces the 4 values 4 i .. 4 i + 3 of fragment j as two
// binary16 pairs (dwords 2 i, 2 i + 1 of the fragment).

// permlane32_swap(x, y): lanes 0..31 get {x, x of lane + 32}, lanes 32..63 {y of lane - 32, y}.
__device__ __forceinline__ void swap32(uint32_t x, uint32_t y, uint32_t& r0, uint32_t& r1) {
    const auto r = __builtin_amdgcn_permlane32_swap(x, y, false, false);
    r0 = r[0];
    r1 = r[1];
}

template <int WT>
struct BPrep;
template <int WT>
struct BRow;

// Q8_0: 34-byte blocks (fp16 d, 32 int8); the 9 dwords around a block.
template <>
struct BPrep<kQ8_0> {
    uint32_t x[2][2][2];  // [run][block][dword]: bytes 16 run + 8 h .. + 7 of block bi
    uint32_t d[2];
    __device__ __forceinline__ void convert(int j, int i, const IQ4Consts&, u32x4& f) const {
        const int bi = j >> 1;
        uint32_t lo, hi;
        u8x4_to_f16(x[j & 1][bi][i] ^ 0x80808080u, splat_h2(d[bi]), lo, hi);
        if (i) { f.z = lo; f.w = hi; } else { f.x = lo; f.y = hi; }
    }
};
template <>
struct BRow<kQ8_0> {
    static constexpr uint32_t kBytes = 34;
    static constexpr int kLoads = 3;
    u32x4 a, b;
    uint32_t c;
    __device__ __forceinline__ static uint32_t off(uint32_t row, int blk0, uint32_t hh) {
        return row + ((uint32_t)blk0 + hh) * kBytes;
    }
    __device__ __forceinline__ void load(rsrc_t r, uint32_t row, int blk0, uint32_t hh) {
        const uint32_t w0 = off(row, blk0, hh) & ~3u;
        a = ld128(r, w0);
        b = ld128(r, w0 + 16u);
        c = ld32(r, w0 + 32u);
    }
    __device__ __forceinline__ void prepare(uint32_t row, int blk0, uint32_t hh, BPrep<kQ8_0>& P) const {
        const uint32_t o = off(row, blk0, hh);
        const uint32_t sel = realign_sel(o);
        const uint32_t raw[9] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w, c};
        uint32_t q[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = perm(raw[i + 1], raw[i], sel);
#pragma unroll
        for (int run = 0; run < 2; ++run)
#pragma unroll
            for (int i = 0; i < 2; ++i) swap32(q[4 * run + i], q[4 * run + 2 + i], P.x[run][0][i], P.x[run][1][i]);
        const uint32_t ds = realign_scale(a.x, o);
        swap32(ds, ds, P.d[0], P.d[1]);
    }
};

// IQ4_NL: 18-byte blocks (fp16 d, 16 bytes of indices; value i < 16 in the low nibble of byte
// i, value 16 + i in its high nibble); the 5 dwords around a block.  Index bytes 8 h .. 8 h + 7
// feed fragment 2 bi (low nibbles) and 2 bi + 1 (high nibbles).
template <>
struct BPrep<kIQ4_NL> {
    uint32_t x[2][2];  // [block][dword]: index bytes 8 h .. + 7 of block bi
    uint32_t d[2];
    __device__ __forceinline__ void convert(int j, int i, const IQ4Consts& k, u32x4& f) const {
        const int bi = j >> 1;
        uint32_t q = x[bi][i];
        if (j & 1) q >>= 4;  // high nibbles
        uint32_t lo, hi;
        u8x4_to_f16(iq4nl_lookup_u(q & k.m7, ((q >> 1) & k.m4) | k.c0123), splat_h2(d[bi]), lo, hi);
        if (i) { f.z = lo; f.w = hi; } else { f.x = lo; f.y = hi; }
    }
};
template <>
struct BRow<kIQ4_NL> {
    static constexpr uint32_t kBytes = 18;
    static constexpr int kLoads = 2;
    u32x4 a;
    uint32_t b;
    __device__ __forceinline__ static uint32_t off(uint32_t row, int blk0, uint32_t hh) {
        return row + ((uint32_t)blk0 + hh) * kBytes;
    }
    __device__ __forceinline__ void load(rsrc_t r, uint32_t row, int blk0, uint32_t hh) {
        const uint32_t w0 = off(row, blk0, hh) & ~3u;
        a = ld128(r, w0);
        b = ld32(r, w0 + 16u);
    }
    __device__ __forceinline__ void prepare(uint32_t row, int blk0, uint32_t hh, BPrep<kIQ4_NL>& P) const {
        const uint32_t o = off(row, blk0, hh);
        const uint32_t sel = realign_sel(o);
        const uint32_t q0 = perm(a.y, a.x, sel), q1 = perm(a.z, a.y, sel), q2 = perm(a.w, a.z, sel),
                       q3 = perm(b, a.w, sel);
        swap32(q0, q2, P.x[0][0], P.x[1][0]);
        swap32(q1, q3, P.x[0][1], P.x[1][1]);
        const uint32_t ds = realign_scale(a.x, o);
        swap32(ds, ds, P.d[0], P.d[1]);
    }
};

// F16: binary16 weights as they are (the FP16 dequantization's output).  Per step a lane reads,
// for each of the step's four k16 fragments j = 2 bi + jj, its row's 8 values k = 32 bi + 16 jj +
// 8 h .. + 7: one 16-byte load each (4 per lane and step), nothing to convert.
template <>
struct BPrep<kF16> {
    u32x4 f[4];
    __device__ __forceinline__ void convert(int j, int i, const IQ4Consts&, u32x4& F) const {
        if (i) { F.z = f[j].z; F.w = f[j].w; } else { F.x = f[j].x; F.y = f[j].y; }
    }
};
template <>
struct BRow<kF16> {
    static constexpr uint32_t kBytes = 64;  // bytes per 32 values
    static constexpr int kLoads = 4;
    u32x4 f[4];
    __device__ __forceinline__ void load(rsrc_t r, uint32_t row, int blk0, uint32_t hh) {
        const uint32_t base = row + (uint32_t)blk0 * kBytes + 16u * hh;
#pragma unroll
        for (int j = 0; j < 4; ++j) f[j] = ld128(r, base + 32u * j);
    }
    __device__ __forceinline__ void prepare(uint32_t, int, uint32_t, BPrep<kF16>& P) const {
#pragma unroll
        for (int j = 0; j < 4; ++j) P.f[j] = f[j];
    }
};

// ---------------------------------------------------------------- activations -> LDS
//
// Stage layout: row r (0..255) at 128 r bytes, its 16-byte chunk c (k 8c .. 8c + 7) at slot
// c ^ swz(r), swz(r) = ((r >> 1) & 7) ^ 4 (r & 1).  A fragment read (lanes 0..31: rows r0 + l,
// one chunk) then puts any 8 consecutive lanes on 8 distinct 16-byte slots of a 128-byte bank
// window and any 16 consecutive lanes on 16 distinct slots of a 256-byte window.
// The stages are filled by buffer_load ... lds (16 bytes per lane, lane l's bytes at
// M0 + 16 l): wave w fills rows 32 w .. 32 w + 31 with 4 loads of 8 rows; lane l of load i
// moves the chunk that belongs at slot l % 8 of row 32 w + 8 i + l / 8.
__device__ __forceinline__ uint32_t pf_swz(uint32_t r) { return ((r >> 1) & 7u) ^ ((r & 1u) << 2); }

// Row (within the tile) whose chunk lane t moves with load i.
__device__ __forceinline__ int pf_arow(int i) { return 32 * (int)(threadIdx.x >> 6) + 8 * i + (int)((threadIdx.x & 63) >> 3); }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// ---------------------------------------------------------------- the K loop
//
// Step ks reads LDS stage ks % 4: its four k16 slices, then slice 0 of step ks + 1 from the next
// stage.  In its first slice it starts the loads of step ks + 3's activations into the stage
// step ks - 1 read; before the barrier that ends it, it waits for step ks + 2's activations
// (started a step earlier), which slice 3 of step ks + 1 reads first.  During slice j it
// converts the weight fragment of the next slice; in its last slice it prepares step ks + 1's
// raw weights and loads step ks + 3's into the same registers (two register sets, each load
// two steps ahead of its use).  One barrier per step orders every wave's stage fills before
// the reads of the next step and every read of a stage before its refill.  Instruction order is
// fixed by hand: each M block of a slice is one scheduling region with its MFMA, the next
// fragment read for that block and a share of the other work.
template <int WT, int MB>
struct PfLoop {
    rsrc_t ar, wr;
    uint32_t voff[4];  // per load i: activation row offset + swizzled chunk offset
    uint32_t b_row;
    uint32_t raddr[4];
    uint32_t hh, wrow;  // hh: lane / 32; wrow: byte offset of this wave's 32 rows in a stage
    int last;
    uint8_t* lds;
    IQ4Consts kc;

    static constexpr int kBLoads = BRow<WT>::kLoads;
    // vmcnt that leaves outstanding only what was issued after step ks + 2's activation loads:
    // the raw weights of steps ks + 2 and ks + 3 and step ks + 3's activation loads
    static constexpr int kWait = 2 * kBLoads + 4;

    __device__ __forceinline__ half8 read_a(uint32_t st, int j, int m) const {
        return __builtin_bit_cast(half8, *(const u32x4*)(lds + st + raddr[j] + 4096 * m));
    }
    __device__ __forceinline__ void fill(int i, uint32_t st, uint32_t kbyte) const {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, (lds_ptr_t)(lds + st + wrow + 1024 * i), 16, voff[i], kbyte, 0, 0);
    }

    // One step.  Bl: raw weights of step ks + 1 (prepared in the last slice, then reloaded with
    // step ks + 3's); P: prepared weights of this step (replaced by step ks + 1's in the last
    // slice).  Stage of step ks: ks % 4.
    __device__ __forceinline__ void step(int ks, BRow<WT>& Bl, BPrep<WT>& P, u32x4& Fa, u32x4& Fb, half8 (&a0)[MB],
                                         half8 (&a1)[MB], f32x16 (&acc)[MB]) const {
        const int nblk = 2 * min(ks + 1, last);
        const int lblk = 2 * min(ks + 3, last);
        const uint32_t kbyte = (uint32_t)min(ks + 3, last) * 128u;
        const uint32_t s_cur = (uint32_t)(ks & 3) * kPfStage;
        const uint32_t s_next = (uint32_t)((ks + 1) & 3) * kPfStage;
        const uint32_t s_fill = (uint32_t)((ks + 3) & 3) * kPfStage;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            half8 (&cur)[MB] = (j & 1) ? a1 : a0;
            half8 (&nxt)[MB] = (j & 1) ? a0 : a1;
            const u32x4& F = (j & 1) ? Fb : Fa;  // fragment j of this step
            u32x4& Fn = (j & 1) ? Fa : Fb;       // fragment j + 1 (slice 0 of the next step for j = 3)
            const half8 b = __builtin_bit_cast(half8, F);
#pragma unroll
            for (int m = 0; m < MB; ++m) {
                acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_f16(cur[m], b, acc[m], 0, 0, 0);
                nxt[m] = j < 3 ? read_a(s_cur, j + 1, m) : read_a(s_next, 0, m);
                if (j == 0) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if ((i * MB) / 4 == m) fill(i, s_fill, kbyte);
                }
                if (j == 3 && m == 0) Bl.prepare(b_row, nblk, hh, P);
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    if (min((i * MB) / 2 + 1, MB - 1) == m) P.convert(j < 3 ? j + 1 : 0, i, kc, Fn);
                if (j == 3 && m == MB - 1) Bl.load(wr, b_row, lblk, hh);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // The barrier: this wave's fragment reads done (lgkmcnt 0) and its fill of step ks + 2's
        // stage landed (vmcnt kWait; gfx9 s_waitcnt: vmcnt bits [3:0] and [15:14], expcnt [6:4],
        // 7 = no wait, lgkmcnt [11:8]).  No fence: a workgroup release fence would also wait for
        // the fill started in this step.  The empty asm statements keep the compiler from moving
        // memory accesses across.
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt((kWait & 15) | ((kWait >> 4) << 14) | (7 << 4));
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    }
};

// acc[m]: rows 32 m .. 32 m + 31 of the tile, this wave's 32 weight rows.  a_off[i]: byte offset
// of row pf_arow(i) in the activation buffer (past its end for rows beyond the tile, which then
// read zeros); b_row: byte offset of this lane's weight row in the matrix of resource wr.
// Steps run in pairs so the raw-weight register roles are constants; an odd last step runs
// after the loop.
template <int WT, int MB>
__device__ __forceinline__ void pf_gemm(rsrc_t ar, const uint32_t (&a_off)[4], rsrc_t wr, uint32_t b_row, int nk,
                                        uint8_t* lds, f32x16 (&acc)[MB]) {
    const uint32_t lane = threadIdx.x & 63u;
    PfLoop<WT, MB> L;
    L.ar = ar;
    L.wr = wr;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t r = (uint32_t)pf_arow(i);
        L.voff[i] = a_off[i] + (((lane & 7u) ^ pf_swz(r)) * 16u);
    }
    L.b_row = b_row;
    L.hh = lane >> 5;
    L.wrow = (uint32_t)__builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) * 32u * 128u;
#pragma unroll
    for (int j = 0; j < 4; ++j) L.raddr[j] = (lane & 31u) * 128u + ((((uint32_t)(2 * j) + (lane >> 5)) ^ pf_swz(lane & 31u)) * 16u);
    L.last = nk - 1;
    L.lds = lds;
#pragma unroll
    for (int m = 0; m < MB; ++m) acc[m] = f32x16{};

    BRow<WT> R0, R1;
    BPrep<WT> P;
    u32x4 Fa, Fb;
    half8 a0[MB], a1[MB];
    // prologue, issued in this order: step 0's raw weights, stages 0, 1, 2, step 1's raw
    // weights, then (once step 0's have landed and are prepared) step 2's.  Step 0 starts once
    // stages 0 and 1 have landed (it reads slice 0 of stage 1 last), with stage 2 and the later
    // weights still in flight: vmcnt(4 + 2 kBLoads) leaves outstanding only what was issued
    // after stage 1.  Step 0's barrier waits for stage 2 (kWait, as in every step: issued after
    // stage 2 are the raw weights of steps 1 and 2 and step 0's own loads).
    R0.load(wr, b_row, 0, L.hh);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 3; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i) L.fill(i, s * kPfStage, (uint32_t)min(s, L.last) * 128u);
    __builtin_amdgcn_sched_barrier(0);
    R1.load(wr, b_row, 2 * min(1, L.last), L.hh);
    __builtin_amdgcn_sched_barrier(0);
    R0.prepare(b_row, 0, L.hh, P);
    R0.load(wr, b_row, 2 * min(2, L.last), L.hh);
    __builtin_amdgcn_sched_barrier(0);
    P.convert(0, 0, L.kc, Fa);
    P.convert(0, 1, L.kc, Fa);
    // (a plain barrier: a workgroup fence would wait for every stage fill)
    constexpr int kPro = 4 + 2 * BRow<WT>::kLoads;
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((kPro & 15) | ((kPro >> 4) << 14) | (7 << 4) | (15 << 8));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
#pragma unroll
    for (int m = 0; m < MB; ++m) a0[m] = L.read_a(0, 0, m);
    int ks = 0;
    for (; ks + 1 < nk; ks += 2) {
        L.step(ks, R1, P, Fa, Fb, a0, a1, acc);
        L.step(ks + 1, R0, P, Fa, Fb, a0, a1, acc);
    }
    if (ks < nk) L.step(ks, R1, P, Fa, Fb, a0, a1, acc);
    // the last steps started (clamped) stage fills: let every wave's land before LDS is reused
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
    __syncthreads();
}

// Row (within the 32-row block) of accumulator register r.
__device__ __forceinline__ int acc_row(int lane, int r) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// silu(g) * u in binary32: the library expf (documented maximum error 1 ulp), 1 + e rounded,
// v_rcp_f32 (1 ulp; 1 + e >= 1, so its input is never subnormal) and two rounded products:
// at most about 4 ulp from the same expression evaluated exactly.  The reciprocal takes 2
// instructions where the IEEE division takes 11, a third of the epilogue's per-value work.
__device__ __forceinline__ float silu_mul_f(float g, float u) {
    const float e = expf(-g);
    const float r = opaque(__builtin_amdgcn_rcpf(opaque(1.0f + e)));
    const float sl = opaque(g * r);
    return opaque(sl * u);
}

// Byte offsets of this thread's four activation rows pf_arow(i) (gate/up: gathered tokens).
__device__ __forceinline__ void token_rows(const int32_t* sorted_tok, const Tile& t, int ntok, int hidden,
                                           uint32_t past_end, uint32_t (&a_off)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = pf_arow(i);
        const int tok = r < t.nrows ? sorted_tok[t.row0 + r] : -1;
        a_off[i] = (tok >= 0 && tok < ntok) ? (uint32_t)tok * (uint32_t)hidden * 2u : past_end;
    }
}

// ---------------------------------------------------------------- gate/up

struct GuArgs {
    const uint8_t* wg;
    const uint8_t* wu;
    int64_t stride;
    uint32_t expert_bytes;
    int nexperts, hidden, inter, ntok;
    const uint16_t* x16;
    uint32_t xbytes;
    const int32_t* sorted_tok;
    const int32_t* tiles;
    uint16_t* h16;
    float* dbg_g;
    float* dbg_u;
};

// The accumulators of rows 64 q .. 64 q + 63 (blocks 2q, 2q+1) go to an LDS tile of 64 rows x
// 256 fp32 columns (row stride 264 floats: the two row groups of one register write land on
// disjoint banks); the caller's loop then reads it back row-wise.
constexpr int kPfEpiLd = 264;

template <int MB>
__device__ __forceinline__ void epi_put(const f32x16 (&acc)[MB], int q, float* tile) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
        const int m = 2 * q + mm;
        if (m < MB) {
#pragma unroll
            for (int r = 0; r < 16; ++r) tile[(32 * mm + acc_row(lane, r)) * kPfEpiLd + 32 * w + (lane & 31)] = acc[m][r];
        }
    }
}

// Waves 0..3 multiply by the gate rows of intermediate columns y*128 + 32 w + 0..31, waves 4..7
// by the up rows of the same columns.  Epilogue per 64-row quarter: G (tile columns 0..127) and
// U (128..255) through LDS, then each thread forms 8 consecutive H16 values of a row
// (H16 = fp16(silu(G) U)) and writes them with one 16-byte store.
template <int WT, int MB>
__device__ __forceinline__ void gateup_tile(const GuArgs& p, const Tile& t, int y, uint8_t* lds) {
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));  // uniform: the weight resource is picked per wave
    uint32_t a_off[4];
    token_rows(p.sorted_tok, t, p.ntok, p.hidden, p.xbytes, a_off);
    const int col = y * kPfGuCols + 32 * (w & 3) + (lane & 31);
    const uint32_t roff = (uint32_t)(col < p.inter ? col : p.inter - 1) * (uint32_t)row_bytes_dev<WT>(p.hidden);
    const rsrc_t wr = make_rsrc_dw((w >= 4 ? p.wu : p.wg) + (int64_t)t.e * p.stride, p.expert_bytes);
    f32x16 acc[MB];
    pf_gemm<WT, MB>(make_rsrc(p.x16, p.xbytes), a_off, wr, roff, p.hidden / kPfStepK, lds, acc);

    float* tile = (float*)lds;
    const int c8 = (int)(threadIdx.x & 15) * 8;  // 8 columns of the 128
    const int c0 = y * kPfGuCols + c8;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        if (2 * q >= MB) break;
        epi_put<MB>(acc, q, tile);
        __syncthreads();
#pragma unroll 1
        for (int rr = (int)(threadIdx.x >> 4); rr < 64; rr += kPfThreads / 16) {
            const int row = 64 * q + rr;
            if (row >= t.nrows || c0 >= p.inter) continue;
            const float* tr = tile + rr * kPfEpiLd;
            const f32x4 g0 = *(const f32x4*)(tr + c8), g1 = *(const f32x4*)(tr + c8 + 4);
            const f32x4 u0 = *(const f32x4*)(tr + 128 + c8), u1 = *(const f32x4*)(tr + 128 + c8 + 4);
            uint32_t h[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                h[i] = f2h(silu_mul_f(g0[i], u0[i]));
                h[i + 4] = f2h(silu_mul_f(g1[i], u1[i]));
            }
            const int64_t o = (int64_t)(t.row0 + row) * p.inter + c0;
            *(u32x4*)(p.h16 + o) = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
            if (p.dbg_g) {
                *(f32x4*)(p.dbg_g + o) = g0;
                *(f32x4*)(p.dbg_g + o + 4) = g1;
                *(f32x4*)(p.dbg_u + o) = u0;
                *(f32x4*)(p.dbg_u + o + 4) = u1;
            }
        }
        __syncthreads();
    }
}

template <int WT>
__global__ __launch_bounds__(kPfThreads) void pf_gateup_kernel(GuArgs p) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[4 * kPfStage];
    Tile t;
    int y;
    if (!pf_tile(p.tiles, (p.inter + kPfGuCols - 1) / kPfGuCols, t, y) || t.e < 0 || t.e >= p.nexperts) return;
    switch ((t.nrows + 31) >> 5) {
        case 1: gateup_tile<WT, 1>(p, t, y, lds); break;
        case 2: gateup_tile<WT, 2>(p, t, y, lds); break;
        case 3: gateup_tile<WT, 3>(p, t, y, lds); break;
        case 4: gateup_tile<WT, 4>(p, t, y, lds); break;
        case 5: gateup_tile<WT, 5>(p, t, y, lds); break;
        case 6: gateup_tile<WT, 6>(p, t, y, lds); break;
        case 7: gateup_tile<WT, 7>(p, t, y, lds); break;
        case 8: gateup_tile<WT, 8>(p, t, y, lds); break;
        default: break;
    }
}

// ---------------------------------------------------------------- down

struct DownArgs {
    const uint8_t* wd;
    int64_t stride;
    uint32_t expert_bytes;
    int nexperts, hidden, inter;
    const uint16_t* h16;
    uint32_t hbytes;
    const int32_t* tiles;
    float* y;
};

template <int WT, int MB>
__device__ __forceinline__ void down_tile(const DownArgs& p, const Tile& t, int y, uint8_t* lds) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    uint32_t a_off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = pf_arow(i);
        a_off[i] = r < t.nrows ? (uint32_t)(t.row0 + r) * (uint32_t)p.inter * 2u : p.hbytes;
    }
    // output column y*256 + 32 w + lane % 32
    const int col = y * kPfDownCols + 32 * w + (lane & 31);
    const uint32_t roff = (uint32_t)(col < p.hidden ? col : p.hidden - 1) * (uint32_t)row_bytes_dev<WT>(p.inter);
    f32x16 acc[MB];
    pf_gemm<WT, MB>(make_rsrc(p.h16, p.hbytes), a_off, make_rsrc_dw(p.wd + (int64_t)t.e * p.stride, p.expert_bytes),
                    roff, p.inter / kPfStepK, lds, acc);

    // Straight from the accumulators: register r of block m holds row 32 m + acc_row(lane, r),
    // column col, so one store instruction writes 32 consecutive floats (128 bytes) of each of
    // two rows.  No LDS round trip and no barrier.
    if (col < p.hidden) {
        float* yc = p.y + (int64_t)t.row0 * p.hidden + col;
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = 32 * m + acc_row(lane, r);
                if (row < t.nrows) yc[(int64_t)row * p.hidden] = acc[m][r];
            }
    }
}

template <int WT>
__global__ __launch_bounds__(kPfThreads) void pf_down_kernel(DownArgs p) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[4 * kPfStage];
    Tile t;
    int y;
    if (!pf_tile(p.tiles, (p.hidden + kPfDownCols - 1) / kPfDownCols, t, y) || t.e < 0 || t.e >= p.nexperts) return;
    switch ((t.nrows + 31) >> 5) {
        case 1: down_tile<WT, 1>(p, t, y, lds); break;
        case 2: down_tile<WT, 2>(p, t, y, lds); break;
        case 3: down_tile<WT, 3>(p, t, y, lds); break;
        case 4: down_tile<WT, 4>(p, t, y, lds); break;
        case 5: down_tile<WT, 5>(p, t, y, lds); break;
        case 6: down_tile<WT, 6>(p, t, y, lds); break;
        case 7: down_tile<WT, 7>(p, t, y, lds); break;
        case 8: down_tile<WT, 8>(p, t, y, lds); break;
        default: break;
    }
}

// ---------------------------------------------------------------- dense prompt projections
//
// Y = X16 . W16^T over the prompt's tokens [DQ, Change: the dense weights as FP16 for a matrix
// product over the prompt; PF, Summary: FP16 products with FP32 sums]: the K loop above with the
// token rows in order (no routing) and one weight matrix.  Workgroup (token tile of 256 rows,
// column tile of 256 weight rows); the tiles go to the 8 XCDs in contiguous runs (XCD c takes
// token tiles in order with all their column tiles), so a token tile and the weight slices are
// reused from that XCD's L2.  Y is stored straight from the accumulators as in the down GEMM.

struct DenseArgs {
    const uint8_t* w;
    uint32_t wbytes;
    int nrows, k, ntok, ntt, nct;
    const uint16_t* x;
    uint32_t xbytes;
    float* y;
    int64_t ldy;
};

template <int WT, int MB>
__device__ __forceinline__ void dense_tile(const DenseArgs& p, int tt, int ct, uint8_t* lds) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int row0 = tt * kPfRows;
    const int rows = p.ntok - row0 < kPfRows ? p.ntok - row0 : kPfRows;
    uint32_t a_off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = pf_arow(i);
        a_off[i] = r < rows ? (uint32_t)(row0 + r) * (uint32_t)p.k * 2u : p.xbytes;
    }
    const int col = ct * kPfDownCols + 32 * w + (lane & 31);
    const uint32_t roff = (uint32_t)(col < p.nrows ? col : p.nrows - 1) * (uint32_t)row_bytes_dev<WT>(p.k);
    f32x16 acc[MB];
    pf_gemm<WT, MB>(make_rsrc(p.x, p.xbytes), a_off, make_rsrc_dw(p.w, p.wbytes), roff, p.k / kPfStepK, lds, acc);
    if (col < p.nrows) {
        float* yc = p.y + (int64_t)row0 * p.ldy + col;
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = 32 * m + acc_row(lane, r);
                if (row < rows) yc[(int64_t)row * p.ldy] = acc[m][r];
            }
    }
}

template <int WT>
__global__ __launch_bounds__(kPfThreads) void dense_kernel(DenseArgs p) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[4 * kPfStage];
    const int total = p.ntt * p.nct;
    const int per_xcd = (total + 7) >> 3;
    const int lin = (int)(blockIdx.x & 7u) * per_xcd + (int)(blockIdx.x >> 3);
    if ((int)(blockIdx.x >> 3) >= per_xcd || lin >= total) return;
    const int tt = lin / p.nct, ct = lin - tt * p.nct;
    const int rows = p.ntok - tt * kPfRows < kPfRows ? p.ntok - tt * kPfRows : kPfRows;
    switch ((rows + 31) >> 5) {
        case 1: dense_tile<WT, 1>(p, tt, ct, lds); break;
        case 2: dense_tile<WT, 2>(p, tt, ct, lds); break;
        case 3: dense_tile<WT, 3>(p, tt, ct, lds); break;
        case 4: dense_tile<WT, 4>(p, tt, ct, lds); break;
        case 5: dense_tile<WT, 5>(p, tt, ct, lds); break;
        case 6: dense_tile<WT, 6>(p, tt, ct, lds); break;
        case 7: dense_tile<WT, 7>(p, tt, ct, lds); break;
        case 8: dense_tile<WT, 8>(p, tt, ct, lds); break;
        default: break;
    }
}

// ---------------------------------------------------------------- MMQ-style prefill: int8 MFMA
//
// [DQ, Change: the prefill's second path takes q8_1 activations against the quantized weights
// (MMQ), with SwiGLU and the q8_1 quantization of H fused between gate/up and down, H never in
// fp32; IQ, What it does: the per-block integer dot and float expression of the decode path]:
// the grouped decode's arithmetic over the sorted rows of the prefill.  Per 32-value block b of
// an output (row p, column c):  isum = sum_j w_int[c][32b + j] q_a[p][32b + j]  (exact int32),
// t = (d_w[c][b] d_a[p][b]) isum,  acc += t  in binary32, blocks in order.
//   - isum: v_mfma_i32_32x32x32_i8 per 32x32 tile and block (lane l: row or column l % 32,
//     k = 16 (l / 32) .. + 15 of the block);
//   - d_w d_a: the tile's 32 x 32 products as a rank-one v_mfma_f32_32x32x2f32 (A = d_a in the
//     k = 0 lanes, 0 in the k = 1 lanes; B = d_w): exact, a product of two binary16 values, and
//     on the matrix unit, not the VALU;
//   - acc = fma(d_w d_a, float(isum), acc): the two VALU operations per output and block that
//     remain (the per-block scales are what make this path VALU-bound on gfx950).
// Activations (the tokens' q8_1 and H) are held as planes: int8 values [rows][k] and their
// binary16 scales [rows][k/32], so a step's 128 rows x 64 values are staged in LDS by 16-byte
// direct-to-LDS loads like the FP16 path's.  Tiles are at most 128 rows (4 blocks of 32): the
// per-block rescale keeps two 16-register MFMA results live beside the accumulators, and 8
// blocks of accumulators would not fit 256 registers.  Each wave owns 32 weight rows as in the
// FP16 path;
// a lane pair (l, l + 32) reads its row's two blocks of a step once (one each) and trades halves
// through v_permlane32_swap.  Three LDS stages, activations and raw weights two steps ahead.

constexpr int kMqRows = 128;                         // rows per tile (4 MFMA blocks of 32)
constexpr int kMqStageQ = kMqRows * 64;              // int8 values of a step: 8 KiB
constexpr int kMqStageD = 8 * 256;                   // scales: 256 bytes per wave of 16 rows
constexpr int kMqStage = kMqStageQ + kMqStageD;      // 10 KiB
constexpr int kMqStages = 3;

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

// Stage layout: row r's 16-byte chunk c (k 16 c .. 16 c + 15 of the step) at 64 r + 16 (c ^
// mq_swz(r)): a fragment read (32 lanes, rows r0 .. r0 + 31, one chunk) puts any 16 consecutive
// lanes on 16 distinct 16-byte slots of a 256-byte window.  Scales: the two binary16 scales of
// row r (blocks 2 s, 2 s + 1) at kMqStageQ + 256 (r / 16) + 4 (r % 16) (wave w stages rows
// 16 w .. 16 w + 15; its 64-lane dword load writes 256 bytes, the rows' 64 and 192 of zeros).
__device__ __forceinline__ uint32_t mq_swz(uint32_t r) { return (r >> 2) & 3u; }

// A row's raw weights of a step -> the int8 B fragments of its two blocks and their scales.
template <int WT>
struct MqB;
template <>
struct MqB<kQ8_0> {
    i32x4 f[2];
    uint32_t d[2];
    __device__ __forceinline__ void prepare(const BRow<kQ8_0>& R, uint32_t row, int blk0, uint32_t hh,
                                            const IQ4Consts&) {
        const uint32_t o = BRow<kQ8_0>::off(row, blk0, hh);
        const uint32_t sel = realign_sel(o);
        const uint32_t raw[9] = {R.a.x, R.a.y, R.a.z, R.a.w, R.b.x, R.b.y, R.b.z, R.b.w, R.c};
        uint32_t q[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = perm(raw[i + 1], raw[i], sel);
        // lane l < 32 holds block 0 and needs bytes 0..15 of both blocks; lane l + 32 holds
        // block 1 and needs bytes 16..31 of both
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t r0, r1;
            swap32(q[i], q[4 + i], r0, r1);
            f[0][i] = (int)r0;
            f[1][i] = (int)r1;
        }
        const uint32_t ds = realign_scale(R.a.x, o);
        swap32(ds, ds, d[0], d[1]);
    }
};
template <>
struct MqB<kIQ4_NL> {
    i32x4 f[2];
    uint32_t d[2];
    __device__ __forceinline__ void prepare(const BRow<kIQ4_NL>& R, uint32_t row, int blk0, uint32_t hh,
                                            const IQ4Consts& k) {
        const uint32_t o = BRow<kIQ4_NL>::off(row, blk0, hh);
        const uint32_t sel = realign_sel(o);
        const uint32_t q[4] = {perm(R.a.y, R.a.x, sel), perm(R.a.z, R.a.y, sel), perm(R.a.w, R.a.z, sel),
                               perm(R.b, R.a.w, sel)};
        // both lanes of a pair need all 16 index bytes of both blocks: lane l < 32 their low
        // nibbles (values 0..15), lane l + 32 their high nibbles (values 16..31)
        const uint32_t shift = 4u * hh;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t b0, b1;
            swap32(q[i], q[i], b0, b1);
            const uint32_t w0 = b0 >> shift, w1 = b1 >> shift;
            f[0][i] = (int)iq4nl_lookup_s(w0 & k.m7, ((w0 >> 1) & k.m4) | k.c0123);
            f[1][i] = (int)iq4nl_lookup_s(w1 & k.m7, ((w1 >> 1) & k.m4) | k.c0123);
        }
        const uint32_t ds = realign_scale(R.a.x, o);
        swap32(ds, ds, d[0], d[1]);
    }
};

// acc[m]: rows 32 m .. 32 m + 31 of the tile, this wave's 32 weight rows.  q_off[i] / d_off: byte
// offsets in the planes of the activation row this thread stages (past the end for rows beyond
// the tile, which read zeros); b_row: this lane's weight row in the matrix of resource wr.
template <int WT, int MB>
__device__ __forceinline__ void mq_gemm(rsrc_t aq, rsrc_t ad, uint32_t q_off, uint32_t d_off, rsrc_t wr,
                                        uint32_t b_row, int nk, uint8_t* lds, f32x16 (&acc)[MB]) {
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wv = (uint32_t)__builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const uint32_t hh = lane >> 5;
    const int last = nk - 1;
    const IQ4Consts kc;
    // fill: wave w stages rows 16 w .. 16 w + 15 (lane: row 16 w + lane / 4, slot lane % 4)
    const uint32_t voff = q_off + (((lane & 3u) ^ mq_swz(16u * wv + (lane >> 2))) * 16u);
    auto fill = [&](int st, int ks) {
        uint8_t* base = lds + st * kMqStage;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(aq, (lds_ptr_t)(base + 1024u * wv), 16, voff, (uint32_t)ks * 64u, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ad, (lds_ptr_t)(base + kMqStageQ + 256u * wv), 4, d_off,
                                                 (uint32_t)ks * 4u, 0, 0);
    };
    // fragment read addresses (row 32 m + lane % 32, chunk 2 b + lane / 32) and scale reads
    uint32_t ra[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) ra[b] = (lane & 31u) * 64u + (((2u * b + hh) ^ mq_swz(lane & 31u)) * 16u);
    const uint32_t rd = kMqStageQ + 256u * ((lane & 31u) >> 4) + 4u * (lane & 15u);
#pragma unroll
    for (int m = 0; m < MB; ++m) acc[m] = f32x16{};

    BRow<WT> R0, R1;
    fill(0, 0);
    R0.load(wr, b_row, 0, hh);
    fill(1, min(1, last));
    R1.load(wr, b_row, 2 * min(1, last), hh);
    constexpr int kWait = 2 + BRow<WT>::kLoads;  // the fills and raw weights of the next step
    // One step; R holds its raw weights and is reloaded with those of step ks + 2.  Steps run in
    // pairs so the two raw-weight register sets keep fixed roles (a runtime index would put them
    // in scratch memory).
    auto step = [&](int ks, BRow<WT>& R) {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt((kWait & 15) | ((kWait >> 4) << 14) | (7 << 4));
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        fill((ks + 2) % kMqStages, min(ks + 2, last));
        MqB<WT> B;
        B.prepare(R, b_row, 2 * ks, hh, kc);
        R.load(wr, b_row, 2 * min(ks + 2, last), hh);
        const float dw[2] = {h2f(B.d[0]), h2f(B.d[1])};
        const uint8_t* st = lds + (ks % kMqStages) * kMqStage;
        // the step's A fragments and row scales first (pair i = (row block i / 2, block i % 2)),
        // then a pipeline over the pairs: the two MFMAs of pair i + 1 are issued before the
        // VALU rescale of pair i, so the matrix unit and the VALU overlap within the wave
        constexpr int P = 2 * MB;
        i32x4 a[P];
        float da[P];
#pragma unroll
        for (int i = 0; i < P; ++i) {
            const int m = i >> 1, b = i & 1;
            a[i] = *(const i32x4*)(st + ra[b] + 2048u * m);
            uint32_t dbits = *(const uint32_t*)(st + rd + 512u * m);
            asm volatile("" : "+v"(dbits));  // read by every lane (kept out of a branch)
            const float v = h2f(b ? dbits >> 16 : dbits);
            da[i] = hh ? 0.0f : v;           // the k = 1 half of the rank-one product is zero
        }
        i32x16 is[2];
        f32x16 sc[2];
        auto issue = [&](int i) {
            is[i & 1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], B.f[i & 1], i32x16{}, 0, 0, 0);
            sc[i & 1] = __builtin_amdgcn_mfma_f32_32x32x2f32(da[i], dw[i & 1], f32x16{}, 0, 0, 0);
        };
        issue(0);
#pragma unroll
        for (int i = 0; i < P; ++i) {
            if (i + 1 < P) issue(i + 1);
            __builtin_amdgcn_sched_barrier(0);
            const int m = i >> 1;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float v = __builtin_fmaf(sc[i & 1][r], (float)is[i & 1][r], acc[m][r]);
                // pinned here: left to itself the compiler sinks these updates into the next
                // step, holding every pair's result registers live at once
                asm volatile("" : "+v"(v));
                acc[m][r] = v;
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    int ks = 0;
    for (; ks + 1 < nk; ks += 2) {
        step(ks, R0);
        step(ks + 1, R1);
    }
    if (ks < nk) step(ks, R0);
    // the last steps started (clamped) fills: let every wave's land before LDS is reused
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
    __syncthreads();
}

// q8_1 planes of rows of binary16 values: one aligned half wave per 32-value block, the q8_1
// quantizer's arithmetic (quantize_lanes32) on the exact binary32 value of each input.
__global__ __launch_bounds__(256) void quantize_planes_kernel(const uint16_t* __restrict__ x, int64_t nblocks,
                                                              int8_t* __restrict__ q, uint16_t* __restrict__ d) {
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t blk = g >> 5;
    const int j = (int)(g & 31);
    const bool ok = blk < nblocks;
    const float v = ok ? h2f(x[blk * 32 + j]) : 0.0f;
    uint32_t hdr;
    const int qv = quantize_lanes32(v, hdr);
    const uint32_t word = pack4_lanes(qv);
    if (ok) {
        if ((j & 3) == 0) *(uint32_t*)(q + blk * 32 + j) = word;
        if (j == 0) d[blk] = (uint16_t)(hdr & 0xFFFFu);
    }
}

struct MqGuArgs {
    const uint8_t* wg;
    const uint8_t* wu;
    int64_t stride;
    uint32_t expert_bytes;
    int nexperts, hidden, inter, ntok;
    const int8_t* xq;
    const uint16_t* xd;
    uint32_t xq_bytes, xd_bytes;
    const int32_t* sorted_tok;
    const int32_t* tiles;
    int8_t* hq;
    uint16_t* hd;
    float* dbg_g;
    float* dbg_u;
};

// Gate/up tile: waves 0..3 the gate rows of intermediate columns y 128 + 32 w + 0..31, waves
// 4..7 the up rows of the same columns.  Epilogue per 64-row quarter: G and U through LDS, then
// one half wave per (row, 32-column group) forms h = silu(G) U and its q8_1 block (the
// quantizer's arithmetic), written to the H planes; h is never stored.
template <int WT, int MB>
__device__ __forceinline__ void mq_gateup_tile(const MqGuArgs& p, const Tile& t, int y, uint8_t* lds) {
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int nb = p.hidden / 32;
    uint32_t q_off, d_off;
    {
        const int r = 16 * w + (lane >> 2);
        const int tok = r < t.nrows ? p.sorted_tok[t.row0 + r] : -1;
        q_off = (tok >= 0 && tok < p.ntok) ? (uint32_t)tok * (uint32_t)p.hidden : p.xq_bytes;
    }
    {
        const int r = 16 * w + (lane & 15);
        const int tok = (lane < 16 && r < t.nrows) ? p.sorted_tok[t.row0 + r] : -1;
        d_off = (tok >= 0 && tok < p.ntok) ? (uint32_t)tok * (uint32_t)nb * 2u : p.xd_bytes;
    }
    const int col = y * kPfGuCols + 32 * (w & 3) + (lane & 31);
    const uint32_t roff = (uint32_t)(col < p.inter ? col : p.inter - 1) * (uint32_t)row_bytes_dev<WT>(p.hidden);
    const rsrc_t wr = make_rsrc_dw((w >= 4 ? p.wu : p.wg) + (int64_t)t.e * p.stride, p.expert_bytes);
    f32x16 acc[MB];
    mq_gemm<WT, MB>(make_rsrc(p.xq, p.xq_bytes), make_rsrc(p.xd, p.xd_bytes), q_off, d_off, wr, roff,
                    p.hidden / kPfStepK, lds, acc);

    float* tile = (float*)lds;
    const int nbh = p.inter / 32;
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
        if (2 * qq >= MB) break;
        epi_put<MB>(acc, qq, tile);
        __syncthreads();
        // 64 rows x 4 groups of 32 columns: 16 half waves per round
#pragma unroll 1
        for (int it = (int)(threadIdx.x >> 5); it < 64 * 4; it += kPfThreads / 32) {
            const int rr = it >> 2, grp = it & 3, j = threadIdx.x & 31;
            const int row = 64 * qq + rr;
            const int c = y * kPfGuCols + 32 * grp + j;
            const bool ok = row < t.nrows && c < p.inter;
            const float g = tile[rr * kPfEpiLd + 32 * grp + j];
            const float u = tile[rr * kPfEpiLd + 128 + 32 * grp + j];
            const float h = ok ? silu_mul_f(g, u) : 0.0f;
            uint32_t hdr;
            const int qv = quantize_lanes32(h, hdr);
            const uint32_t word = pack4_lanes(qv);
            if (ok) {
                const int64_t e = t.row0 + row;
                if ((j & 3) == 0) *(uint32_t*)(p.hq + e * p.inter + c) = word;
                if (j == 0) p.hd[e * nbh + c / 32] = (uint16_t)(hdr & 0xFFFFu);
                if (p.dbg_g) {
                    p.dbg_g[e * p.inter + c] = g;
                    p.dbg_u[e * p.inter + c] = u;
                }
            }
        }
        __syncthreads();
    }
}

template <int WT>
__global__ __launch_bounds__(kPfThreads) void mq_gateup_kernel(MqGuArgs p) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[kMqStages * kMqStage > 64 * kPfEpiLd * 4 ? kMqStages * kMqStage
                                                                                                 : 64 * kPfEpiLd * 4];
    static_assert(kMqRows == 128, "the epilogue's quarters of 64 rows cover two of them");
    Tile t;
    int y;
    if (!pf_tile(p.tiles, (p.inter + kPfGuCols - 1) / kPfGuCols, t, y) || t.e < 0 || t.e >= p.nexperts) return;
    switch ((t.nrows + 31) >> 5) {
        case 1: mq_gateup_tile<WT, 1>(p, t, y, lds); break;
        case 2: mq_gateup_tile<WT, 2>(p, t, y, lds); break;
        case 3: mq_gateup_tile<WT, 3>(p, t, y, lds); break;
        case 4: mq_gateup_tile<WT, 4>(p, t, y, lds); break;
        default: break;
    }
}

struct MqDownArgs {
    const uint8_t* wd;
    int64_t stride;
    uint32_t expert_bytes;
    int nexperts, hidden, inter;
    const int8_t* hq;
    const uint16_t* hd;
    uint32_t hq_bytes, hd_bytes;
    const int32_t* tiles;
    float* y;
};

template <int WT, int MB>
__device__ __forceinline__ void mq_down_tile(const MqDownArgs& p, const Tile& t, int y, uint8_t* lds) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int nbh = p.inter / 32;
    uint32_t q_off, d_off;
    {
        const int r = 16 * w + (lane >> 2);
        q_off = r < t.nrows ? (uint32_t)(t.row0 + r) * (uint32_t)p.inter : p.hq_bytes;
    }
    {
        const int r = 16 * w + (lane & 15);
        d_off = (lane < 16 && r < t.nrows) ? (uint32_t)(t.row0 + r) * (uint32_t)nbh * 2u : p.hd_bytes;
    }
    const int col = y * kPfDownCols + 32 * w + (lane & 31);
    const uint32_t roff = (uint32_t)(col < p.hidden ? col : p.hidden - 1) * (uint32_t)row_bytes_dev<WT>(p.inter);
    f32x16 acc[MB];
    mq_gemm<WT, MB>(make_rsrc(p.hq, p.hq_bytes), make_rsrc(p.hd, p.hd_bytes), q_off, d_off,
                    make_rsrc_dw(p.wd + (int64_t)t.e * p.stride, p.expert_bytes), roff, p.inter / kPfStepK, lds, acc);
    if (col < p.hidden) {
        float* yc = p.y + (int64_t)t.row0 * p.hidden + col;
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = 32 * m + acc_row(lane, r);
                if (row < t.nrows) yc[(int64_t)row * p.hidden] = acc[m][r];
            }
    }
}

template <int WT>
__global__ __launch_bounds__(kPfThreads) void mq_down_kernel(MqDownArgs p) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[kMqStages * kMqStage];
    Tile t;
    int y;
    if (!pf_tile(p.tiles, (p.hidden + kPfDownCols - 1) / kPfDownCols, t, y) || t.e < 0 || t.e >= p.nexperts) return;
    switch ((t.nrows + 31) >> 5) {
        case 1: mq_down_tile<WT, 1>(p, t, y, lds); break;
        case 2: mq_down_tile<WT, 2>(p, t, y, lds); break;
        case 3: mq_down_tile<WT, 3>(p, t, y, lds); break;
        case 4: mq_down_tile<WT, 4>(p, t, y, lds); break;
        default: break;
    }
}

static size_t align16(size_t v) { return (v + 15) & ~(size_t)15; }
static int64_t max_tiles_of(int nexperts, int64_t nentries, int rows = kPfRows) {
    return (nentries + rows - 1) / rows + nexperts;
}

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
    if (hidden % kPfStepK || inter % kPfStepK) return QMM_EUNSUPPORTED;
    const int64_t gu_bytes = inter * qmm_row_bytes(wtype_gu, hidden);
    const int64_t d_bytes = hidden * qmm_row_bytes(wtype_down, inter);
    if (gu_expert_stride < gu_bytes || down_expert_stride < d_bytes) return QMM_EINVAL;
    if (gu_expert_stride % 4 || down_expert_stride % 4) return QMM_EALIGN;
    if (!aligned(w_gate, 4) || !aligned(w_up, 4) || !aligned(w_down, 4) || !aligned(x_f16, 16) || !aligned(y, 16) ||
        !aligned(ws, 16))
        return QMM_EALIGN;
    // A row outside the tile (or an invalid token) is read at the buffer's end plus up to 2 k + 112
    // bytes (chunk and step offsets), which must not wrap the 32-bit offset back into the buffer.
    if ((uint64_t)ntok * hidden * 2 + 2 * (uint64_t)hidden + 128 > kMaxBufferBytes ||
        (uint64_t)nentries * inter * 2 + 2 * (uint64_t)inter + 128 > kMaxBufferBytes ||
        gu_bytes > (int64_t)kMaxBufferBytes || d_bytes > (int64_t)kMaxBufferBytes || nentries > 0x7FFFFFFF ||
        hidden > kMaxK || inter > kMaxK)
        return QMM_EUNSUPPORTED;
    const PfLayout lay = pf_layout(nexperts, inter, nentries, flags);
    if (ws_bytes < lay.total) return QMM_ESPACE;
    if (nentries == 0) return QMM_OK;
    const hipStream_t st = as_stream(stream);
    uint8_t* wsb = (uint8_t*)ws;
    uint16_t* h16 = (uint16_t*)(wsb + lay.h_off);
    int32_t* tiles = (int32_t*)(wsb + lay.tiles_off);
    const int64_t max_tiles = max_tiles_of(nexperts, nentries);
    const int64_t per_xcd = (max_tiles + 7) / 8;
    const int64_t ny_max = std::max((inter + kPfGuCols - 1) / kPfGuCols, (hidden + kPfDownCols - 1) / kPfDownCols);
    if (8 * per_xcd * ny_max > 0x7FFFFFFF) return QMM_EUNSUPPORTED;

    hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(1024), 0, st, expert_off, nexperts, (int)nentries, tiles,
                       (int)max_tiles, kPfRows);
    int rc = launch_status();
    if (rc) return rc;
    {
        GuArgs a;
        a.wg = (const uint8_t*)w_gate;
        a.wu = (const uint8_t*)w_up;
        a.stride = gu_expert_stride;
        a.expert_bytes = (uint32_t)gu_bytes;
        a.nexperts = nexperts;
        a.hidden = (int)hidden;
        a.inter = (int)inter;
        a.ntok = (int)ntok;
        a.x16 = x_f16;
        a.xbytes = (uint32_t)(ntok * hidden * 2);
        a.sorted_tok = sorted_tok;
        a.tiles = tiles;
        a.h16 = h16;
        a.dbg_g = (flags & QMM_FLAG_DEBUG_INTERMEDIATES) ? (float*)(wsb + lay.g_off) : nullptr;
        a.dbg_u = (flags & QMM_FLAG_DEBUG_INTERMEDIATES) ? (float*)(wsb + lay.u_off) : nullptr;
        const int64_t ny = (inter + kPfGuCols - 1) / kPfGuCols;
        const dim3 g((unsigned)(8 * per_xcd * ny));
        if (wtype_gu == QMM_Q8_0) hipLaunchKernelGGL(pf_gateup_kernel<kQ8_0>, g, dim3(kPfThreads), 0, st, a);
        else hipLaunchKernelGGL(pf_gateup_kernel<kIQ4_NL>, g, dim3(kPfThreads), 0, st, a);
        rc = launch_status();
        if (rc) return rc;
    }
    {
        DownArgs a;
        a.wd = (const uint8_t*)w_down;
        a.stride = down_expert_stride;
        a.expert_bytes = (uint32_t)d_bytes;
        a.nexperts = nexperts;
        a.hidden = (int)hidden;
        a.inter = (int)inter;
        a.h16 = h16;
        a.hbytes = (uint32_t)(nentries * inter * 2);
        a.tiles = tiles;
        a.y = y;
        const int64_t ny = (hidden + kPfDownCols - 1) / kPfDownCols;
        const dim3 g((unsigned)(8 * per_xcd * ny));
        if (wtype_down == QMM_Q8_0) hipLaunchKernelGGL(pf_down_kernel<kQ8_0>, g, dim3(kPfThreads), 0, st, a);
        else hipLaunchKernelGGL(pf_down_kernel<kIQ4_NL>, g, dim3(kPfThreads), 0, st, a);
        return launch_status();
    }
}

extern "C" int qgemm_dense(int wtype, const void* w, int64_t nrows, int64_t k, const uint16_t* x_f16, int64_t ntok,
                           float* y, int64_t ldy, void* stream) {
    if (wtype != QMM_Q8_0 && wtype != QMM_IQ4_NL && wtype != QMM_F16) return QMM_EINVAL;
    if (!w || !x_f16 || !y || nrows < 1 || k < 1 || ntok < 0 || ldy < nrows) return QMM_EINVAL;
    if (qmm_row_bytes(wtype, k) == 0) return QMM_EINVAL;
    if (k % kPfStepK) return QMM_EUNSUPPORTED;
    if (!aligned(w, wtype == QMM_F16 ? 16 : 4) || !aligned(x_f16, 16) || !aligned(y, 4)) return QMM_EALIGN;
    if (wtype == QMM_F16 && k % 8) return QMM_EALIGN;
    const uint64_t wbytes = (uint64_t)nrows * (uint64_t)qmm_row_bytes(wtype, k);
    if (k > kMaxK || nrows > 0x7FFFFFFF || wbytes > kMaxBufferBytes ||
        (uint64_t)ntok * k * 2 + 2 * (uint64_t)k + 128 > kMaxBufferBytes)
        return QMM_EUNSUPPORTED;
    if (ntok == 0) return QMM_OK;
    DenseArgs a;
    a.w = (const uint8_t*)w;
    a.wbytes = (uint32_t)wbytes;
    a.nrows = (int)nrows;
    a.k = (int)k;
    a.ntok = (int)ntok;
    a.ntt = (int)((ntok + kPfRows - 1) / kPfRows);
    a.nct = (int)((nrows + kPfDownCols - 1) / kPfDownCols);
    a.x = x_f16;
    a.xbytes = (uint32_t)(ntok * k * 2);
    a.y = y;
    a.ldy = ldy;
    const int64_t total = (int64_t)a.ntt * a.nct;
    if (total > 0x0FFFFFFF) return QMM_EUNSUPPORTED;
    const dim3 g((unsigned)(8 * ((total + 7) / 8)));
    const hipStream_t st = as_stream(stream);
    if (wtype == QMM_Q8_0) hipLaunchKernelGGL(dense_kernel<kQ8_0>, g, dim3(kPfThreads), 0, st, a);
    else if (wtype == QMM_IQ4_NL) hipLaunchKernelGGL(dense_kernel<kIQ4_NL>, g, dim3(kPfThreads), 0, st, a);
    else hipLaunchKernelGGL(dense_kernel<kF16>, g, dim3(kPfThreads), 0, st, a);
    return launch_status();
}

// ---------------------------------------------------------------- MMQ-style prefill: entry point

struct MqLayout {
    size_t xq, xd, hq, hd, tiles, g, u, total;
};
static MqLayout mq_layout(int nexperts, int64_t hidden, int64_t inter, int64_t ntok, int64_t nentries, unsigned flags) {
    MqLayout l;
    l.xq = 0;
    l.xd = align16((size_t)ntok * (size_t)hidden);
    l.hq = align16(l.xd + (size_t)ntok * (size_t)(hidden / 32) * 2);
    l.hd = align16(l.hq + (size_t)nentries * (size_t)inter);
    l.tiles = align16(l.hd + (size_t)nentries * (size_t)(inter / 32) * 2);
    l.g = align16(l.tiles + 4 * (size_t)(1 + 3 * max_tiles_of(nexperts, nentries, kMqRows)));
    l.u = l.g;
    l.total = l.g;
    if (flags & QMM_FLAG_DEBUG_INTERMEDIATES) {
        l.u = l.g + (size_t)nentries * (size_t)inter * 4;
        l.total = l.u + (size_t)nentries * (size_t)inter * 4;
    }
    return l;
}

extern "C" size_t qgemm_prefill_experts_q8_workspace(int nexperts, int64_t hidden, int64_t inter, int64_t ntok,
                                                     int64_t nentries, unsigned flags) {
    if (nexperts < 1 || hidden < 32 || inter < 32 || ntok < 0 || nentries < 0) return 0;
    return mq_layout(nexperts, hidden, inter, ntok, nentries, flags).total;
}

extern "C" int qgemm_prefill_experts_q8(int wtype_gu, const void* w_gate, const void* w_up, int64_t gu_expert_stride,
                                        int wtype_down, const void* w_down, int64_t down_expert_stride, int nexperts,
                                        int64_t hidden, int64_t inter, const uint16_t* x_f16, int64_t ntok,
                                        const int32_t* sorted_tok, const int32_t* expert_off, int64_t nentries,
                                        float* y, void* ws, size_t ws_bytes, unsigned flags, void* stream) {
    if (!valid_wtype(wtype_gu) || !valid_wtype(wtype_down)) return QMM_EINVAL;
    if (!w_gate || !w_up || !w_down || !x_f16 || !sorted_tok || !expert_off || !y || !ws) return QMM_EINVAL;
    if (nexperts < 1 || hidden < 32 || inter < 32 || ntok < 1 || nentries < 0) return QMM_EINVAL;
    if (qmm_row_bytes(wtype_gu, hidden) == 0 || qmm_row_bytes(wtype_down, inter) == 0) return QMM_EINVAL;
    if (wtype_gu == QMM_CB3 || wtype_down == QMM_CB3) return QMM_EUNSUPPORTED;
    if (hidden % kPfStepK || inter % kPfStepK) return QMM_EUNSUPPORTED;
    const int64_t gu_bytes = inter * qmm_row_bytes(wtype_gu, hidden);
    const int64_t d_bytes = hidden * qmm_row_bytes(wtype_down, inter);
    if (gu_expert_stride < gu_bytes || down_expert_stride < d_bytes) return QMM_EINVAL;
    if (gu_expert_stride % 4 || down_expert_stride % 4) return QMM_EALIGN;
    if (!aligned(w_gate, 4) || !aligned(w_up, 4) || !aligned(w_down, 4) || !aligned(x_f16, 4) || !aligned(y, 4) ||
        !aligned(ws, 16))
        return QMM_EALIGN;
    // planes read at their end plus up to a row of values (or of scales) must not wrap 4 GiB
    if ((uint64_t)ntok * hidden + (uint64_t)hidden + 64 > kMaxBufferBytes ||
        (uint64_t)nentries * inter + (uint64_t)inter + 64 > kMaxBufferBytes || gu_bytes > (int64_t)kMaxBufferBytes ||
        d_bytes > (int64_t)kMaxBufferBytes || nentries > 0x7FFFFFFF || hidden > kMaxK || inter > kMaxK)
        return QMM_EUNSUPPORTED;
    const MqLayout lay = mq_layout(nexperts, hidden, inter, ntok, nentries, flags);
    if (ws_bytes < lay.total) return QMM_ESPACE;
    if (nentries == 0) return QMM_OK;
    const hipStream_t st = as_stream(stream);
    uint8_t* wsb = (uint8_t*)ws;
    int8_t* xq = (int8_t*)(wsb + lay.xq);
    uint16_t* xd = (uint16_t*)(wsb + lay.xd);
    int8_t* hq = (int8_t*)(wsb + lay.hq);
    uint16_t* hd = (uint16_t*)(wsb + lay.hd);
    int32_t* tiles = (int32_t*)(wsb + lay.tiles);
    const int64_t max_tiles = max_tiles_of(nexperts, nentries, kMqRows);
    const int64_t per_xcd = (max_tiles + 7) / 8;
    const int64_t ny_max = std::max((inter + kPfGuCols - 1) / kPfGuCols, (hidden + kPfDownCols - 1) / kPfDownCols);
    if (8 * per_xcd * ny_max > 0x7FFFFFFF) return QMM_EUNSUPPORTED;

    const int64_t xblocks = ntok * (hidden / 32);
    hipLaunchKernelGGL(quantize_planes_kernel, dim3((unsigned)((xblocks * 32 + 255) / 256)), dim3(256), 0, st, x_f16,
                       xblocks, xq, xd);
    int rc = launch_status();
    if (rc) return rc;
    hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(1024), 0, st, expert_off, nexperts, (int)nentries, tiles,
                       (int)max_tiles, kMqRows);
    rc = launch_status();
    if (rc) return rc;
    {
        MqGuArgs a;
        a.wg = (const uint8_t*)w_gate;
        a.wu = (const uint8_t*)w_up;
        a.stride = gu_expert_stride;
        a.expert_bytes = (uint32_t)gu_bytes;
        a.nexperts = nexperts;
        a.hidden = (int)hidden;
        a.inter = (int)inter;
        a.ntok = (int)ntok;
        a.xq = xq;
        a.xd = xd;
        a.xq_bytes = (uint32_t)(ntok * hidden);
        a.xd_bytes = (uint32_t)(ntok * (hidden / 32) * 2);
        a.sorted_tok = sorted_tok;
        a.tiles = tiles;
        a.hq = hq;
        a.hd = hd;
        a.dbg_g = (flags & QMM_FLAG_DEBUG_INTERMEDIATES) ? (float*)(wsb + lay.g) : nullptr;
        a.dbg_u = (flags & QMM_FLAG_DEBUG_INTERMEDIATES) ? (float*)(wsb + lay.u) : nullptr;
        const dim3 g((unsigned)(8 * per_xcd * ((inter + kPfGuCols - 1) / kPfGuCols)));
        if (wtype_gu == QMM_Q8_0) hipLaunchKernelGGL(mq_gateup_kernel<kQ8_0>, g, dim3(kPfThreads), 0, st, a);
        else hipLaunchKernelGGL(mq_gateup_kernel<kIQ4_NL>, g, dim3(kPfThreads), 0, st, a);
        rc = launch_status();
        if (rc) return rc;
    }
    {
        MqDownArgs a;
        a.wd = (const uint8_t*)w_down;
        a.stride = down_expert_stride;
        a.expert_bytes = (uint32_t)d_bytes;
        a.nexperts = nexperts;
        a.hidden = (int)hidden;
        a.inter = (int)inter;
        a.hq = hq;
        a.hd = hd;
        a.hq_bytes = (uint32_t)(nentries * inter);
        a.hd_bytes = (uint32_t)(nentries * (inter / 32) * 2);
        a.tiles = tiles;
        a.y = y;
        const dim3 g((unsigned)(8 * per_xcd * ((hidden + kPfDownCols - 1) / kPfDownCols)));
        if (wtype_down == QMM_Q8_0) hipLaunchKernelGGL(mq_down_kernel<kQ8_0>, g, dim3(kPfThreads), 0, st, a);
        else hipLaunchKernelGGL(mq_down_kernel<kIQ4_NL>, g, dim3(kPfThreads), 0, st, a);
        return launch_status();
    }
}
