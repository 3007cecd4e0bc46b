// qmm_device.h -- device-side building blocks of libqmm for gfx950 (CDNA4, wave64).
//
// Sources (cited by page title and section):
//   [PF] #2356 "pf_wmma: a second Volta prompt-expert kernel for IQ2_S gate/up and IQ4_NL down"
//   [DQ] #1525 "prefill: dense IQ4_XS / Q8_0 to FP16 with 16-byte stores, swiglu + q8_1 ..."
//   [IQ] #242  "IQ kernels: decode each weight part once for every column and entry, bitwise identical"
//   [GP] #1424 "Pascal GP100: a Q8_0 decode GEMV ... and IQ3_XXS / IQ3_S tables in shared memory"
//
// Memory access: every weight / activation read goes through a raw buffer resource whose
// record count is the size of the buffer, so a read past the end returns zeros instead of
// faulting (used for the last block's aligned over-read and for clamped rows).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmm {

enum : int { kQ8_0 = 1, kIQ4_NL = 2, kCB3 = 3 };

// ------------------------------------------------------------------ buffer loads

using rsrc_t = __amdgpu_buffer_rsrc_t;

// gfx9 raw buffer: stride 0, DATA_FORMAT 32 (third word 0x00020000), range = nbytes.
__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t nbytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)nbytes, 0x00020000);
}

__device__ __forceinline__ uint32_t ld32(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}
__device__ __forceinline__ uint32_t ld16(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}
__device__ __forceinline__ uint32_t ld8(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b8(r, (int)off, 0, 0);
}
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 ld64(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
}
__device__ __forceinline__ u32x3 ld96(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b96(r, (int)off, 0, 0);
}
__device__ __forceinline__ u32x4 ld128(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}

// ------------------------------------------------------------------ fp16

__device__ __forceinline__ float h2f(uint32_t bits) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits & 0xFFFFu));
}
// binary32 -> binary16, round to nearest even (v_cvt_f16_f32 under the default mode; fp16
// denormals are kept).
__device__ __forceinline__ uint32_t f2h(float f) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

// Materialise a binary32 value so the compiler cannot fuse the operation that produced it
// with a following conversion (a product followed by fp16 conversion would otherwise become
// v_fma_mix with a +0 addend, which turns a -0 product into +0 and skips the binary32
// rounding of the product).
__device__ __forceinline__ float opaque(float v) {
    asm volatile("" : "+v"(v));
    return v;
}

// bytes {a:b} >> 8*s, low dword (s in 0..3)
__device__ __forceinline__ uint32_t align8(uint32_t hi, uint32_t lo, uint32_t s) {
    return __builtin_amdgcn_alignbyte(hi, lo, s);
}
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
    return __builtin_amdgcn_perm(hi, lo, sel);
}
__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

// ------------------------------------------------------------------ IQ4_NL

// The sixteen IQ4_NL levels packed four to a dword (byte i of word j = level 4j+i).
constexpr int8_t kIQ4NLLevels[16] = {-127, -104, -83, -65, -49, -35, -22, -10,
                                     1,    13,   25,  38,  53,  69,  89,  113};
constexpr uint32_t kv_word(int j) {
    return (uint32_t)(uint8_t)kIQ4NLLevels[4 * j] | ((uint32_t)(uint8_t)kIQ4NLLevels[4 * j + 1] << 8) |
           ((uint32_t)(uint8_t)kIQ4NLLevels[4 * j + 2] << 16) |
           ((uint32_t)(uint8_t)kIQ4NLLevels[4 * j + 3] << 24);
}

// Four 4-bit indices (one per byte, low 3 bits in `i7`, bit 3 moved to bit 2 in `i8`) ->
// four int8 levels.  Two v_perm pick from the low and high halves of the table, a third
// picks per byte between them.
__device__ __forceinline__ uint32_t iq4nl_lookup(uint32_t i7, uint32_t i8) {
    const uint32_t lo = perm(kv_word(1), kv_word(0), i7);
    const uint32_t hi = perm(kv_word(3), kv_word(2), i7);
    return perm(hi, lo, i8 | 0x03020100u);
}

// One dword of IQ4_NL index bytes (elements j..j+3 in the low nibbles, j+16..j+19 in the
// high nibbles) -> the int8 levels of both element groups.
__device__ __forceinline__ void iq4nl_decode_word(uint32_t q, uint32_t& lo, uint32_t& hi) {
    lo = iq4nl_lookup(q & 0x07070707u, (q >> 1) & 0x04040404u);
    hi = iq4nl_lookup((q >> 4) & 0x07070707u, (q >> 5) & 0x04040404u);
}

// ------------------------------------------------------------------ weight units
//
// A "unit" is what one lane loads and decodes in one step; it covers BLK 32-value blocks,
// each delivered as 8 dwords of int8 factors (values 4i..4i+3 in dword i) plus its fp16
// scale and an integer multiplier (1 except CB3).
//   Q8_0   : a pair of blocks (68 bytes, 17 dwords, 4-byte aligned when the row is)
//   IQ4_NL : a pair of blocks (36 bytes, 9 dwords)
//   CB3    : one 32-value sub-block of a 256-value super-block

template <int WT>
struct Unit;

template <>
struct Unit<kQ8_0> {
    static constexpr int BLK = 2;
    static constexpr int RAW = 17;
    static constexpr int UNIT_BYTES = 68;
    __device__ static __forceinline__ void load(rsrc_t r, uint32_t off, uint32_t* raw) {
        const u32x4 a = ld128(r, off), b = ld128(r, off + 16), c = ld128(r, off + 32), d = ld128(r, off + 48);
        raw[0] = a.x; raw[1] = a.y; raw[2] = a.z; raw[3] = a.w;
        raw[4] = b.x; raw[5] = b.y; raw[6] = b.z; raw[7] = b.w;
        raw[8] = c.x; raw[9] = c.y; raw[10] = c.z; raw[11] = c.w;
        raw[12] = d.x; raw[13] = d.y; raw[14] = d.z; raw[15] = d.w;
        raw[16] = ld32(r, off + 64);
    }
    __device__ static __forceinline__ void decode(const uint32_t* raw, uint32_t (*W)[8], uint32_t* dw,
                                                  int* mult) {
        dw[0] = raw[0] & 0xFFFFu;
#pragma unroll
        for (int i = 0; i < 8; ++i) W[0][i] = align8(raw[i + 1], raw[i], 2);
        dw[1] = raw[8] >> 16;
#pragma unroll
        for (int i = 0; i < 8; ++i) W[1][i] = raw[9 + i];
        mult[0] = mult[1] = 1;
    }
};

template <>
struct Unit<kIQ4_NL> {
    static constexpr int BLK = 2;
    static constexpr int RAW = 9;
    static constexpr int UNIT_BYTES = 36;
    __device__ static __forceinline__ void load(rsrc_t r, uint32_t off, uint32_t* raw) {
        const u32x4 a = ld128(r, off), b = ld128(r, off + 16);
        raw[0] = a.x; raw[1] = a.y; raw[2] = a.z; raw[3] = a.w;
        raw[4] = b.x; raw[5] = b.y; raw[6] = b.z; raw[7] = b.w;
        raw[8] = ld32(r, off + 32);
    }
    __device__ static __forceinline__ void decode(const uint32_t* raw, uint32_t (*W)[8], uint32_t* dw,
                                                  int* mult) {
        dw[0] = raw[0] & 0xFFFFu;
#pragma unroll
        for (int i = 0; i < 4; ++i) iq4nl_decode_word(align8(raw[i + 1], raw[i], 2), W[0][i], W[0][i + 4]);
        dw[1] = raw[4] >> 16;
#pragma unroll
        for (int i = 0; i < 4; ++i) iq4nl_decode_word(raw[5 + i], W[1][i], W[1][i + 4]);
        mult[0] = mult[1] = 1;
    }
};

// CB3 super-block field offsets
constexpr int kCB3Bytes = 110, kCB3Qs = 2, kCB3Qh = 66, kCB3Signs = 74, kCB3Scales = 106;

// Expand 4 sign bits into a per-byte mask word x with x byte j = bit j (0 or 1).
__device__ __forceinline__ uint32_t sign_bits_to_bytes(uint32_t nib) {
    return __umul24(nib, 0x00204081u) & 0x01010101u;
}

// Apply per-byte signs to four codebook magnitudes: (g ^ mask) + (mask & 0x01010101) negates
// each selected byte [GP, What changed: sign masks].  No magnitude is 0, so a negated byte
// never carries into its neighbour.
__device__ __forceinline__ uint32_t cb3_signed(uint32_t g, uint32_t nib) {
    const uint32_t x = sign_bits_to_bytes(nib);
    const uint32_t mask = (x << 8) - x;
    return (g ^ mask) + x;
}

template <>
struct Unit<kCB3> {
    static constexpr int BLK = 1;
    static constexpr int RAW = 8;
    // raw: [0..2] qs window, [3..4] signs window, [5] qh byte, [6] scales byte, [7] d
    // `off` = byte offset of the super-block, `ss` = sub-block 0..7.
    __device__ static __forceinline__ void load(rsrc_t r, uint32_t off, int ss, uint32_t* raw) {
        const uint32_t oq = off + kCB3Qs + 8 * ss;
        const u32x3 q = ld96(r, oq & ~3u);
        raw[0] = q.x; raw[1] = q.y; raw[2] = q.z;
        const uint32_t os = off + kCB3Signs + 4 * ss;
        const u32x2 s = ld64(r, os & ~3u);
        raw[3] = s.x; raw[4] = s.y;
        raw[5] = ld8(r, off + kCB3Qh + ss);
        raw[6] = ld8(r, off + kCB3Scales + (ss >> 1));
        raw[7] = ld16(r, off);
    }
    // grid: 512 codebook words in LDS.  `off` and `ss` as in load (the low bits of the field
    // offsets give the alignment shifts).
    __device__ static __forceinline__ void decode(const uint32_t* raw, uint32_t off, int ss,
                                                  const uint32_t* grid, uint32_t (*W)[8], uint32_t* dw,
                                                  int* mult) {
        const uint32_t shq = (off + kCB3Qs) & 3u;        // 8*ss keeps the low bits
        const uint32_t shs = (off + kCB3Signs) & 3u;
        const uint32_t q0 = align8(raw[1], raw[0], shq);
        const uint32_t q1 = align8(raw[2], raw[1], shq);
        const uint32_t sg = align8(raw[4], raw[3], shs);
        const uint32_t qh = raw[5];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t qb = ((e < 4 ? q0 : q1) >> (8 * (e & 3))) & 0xFFu;
            const uint32_t idx = qb | (((qh >> e) & 1u) << 8);
            W[0][e] = cb3_signed(grid[idx], (sg >> (4 * e)) & 15u);
        }
        dw[0] = raw[7];
        mult[0] = 1 + 2 * (int)((raw[6] >> (4 * (ss & 1))) & 15u);
    }
};

// ------------------------------------------------------------------ activations in LDS
//
// The q8_1 columns of a pass are staged once per workgroup as an int8 plane (32 bytes per
// block, 16-byte aligned) plus a float plane of the block scales [GP, What changed].

struct ActLds {
    uint32_t* q;  // [ncols][k/4] dwords
    float* d;     // [ncols][k/32]
    int kw;       // k/4
    int nb;       // k/32
};

// Copy q8_1 block b of column `src_col` of xq into LDS column c.
__device__ __forceinline__ void stage_block(rsrc_t xr, uint32_t src_block, ActLds a, int c, int b) {
    const uint32_t off = src_block * 36u;
    const uint32_t h = ld32(xr, off);
    const u32x4 q0 = ld128(xr, off + 4);
    const u32x4 q1 = ld128(xr, off + 20);
    uint32_t* dst = a.q + c * a.kw + b * 8;
    *(u32x4*)dst = q0;
    *(u32x4*)(dst + 4) = q1;
    a.d[c * a.nb + b] = h2f(h);
}

}  // namespace qmm
