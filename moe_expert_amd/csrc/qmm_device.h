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

// Q8_0P, IQ4_NLP: the same blocks repacked into planes (tiles of 16 blocks: their factor bytes,
// then their scales; see Unit<kQ8_0P>).
// F16: binary16 weights [rows][k] (the FP16 dequantization's output), read by the prefill-style
// MFMA GEMM as they are.
enum : int { kQ8_0 = 1, kIQ4_NL = 2, kCB3 = 3, kQ8_0P = 4, kIQ4_NLP = 5, kF16 = 6 };

// ------------------------------------------------------------------ buffer loads

using rsrc_t = __amdgpu_buffer_rsrc_t;

// gfx9 raw buffer: stride 0, DATA_FORMAT 32 (third word 0x00020000), range = nbytes.
__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t nbytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)nbytes, 0x00020000);
}

// Range rounded up to whole dwords, for buffers whose data ends inside a dword (weight blocks
// of 34 or 18 bytes): the hardware drops a dword that is partly past the range, and the dword
// holding the last byte of a 4-byte aligned buffer lies in the same page as that byte.
__device__ __forceinline__ rsrc_t make_rsrc_dw(const void* p, uint32_t nbytes) {
    const uint64_t r = ((uint64_t)nbytes + 3u) & ~(uint64_t)3u;
    return make_rsrc(p, r > 0xFFFFFFFCull ? 0xFFFFFFFCu : (uint32_t)r);
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
// The first product of a chain, dot4(a, b) with a zero accumulator, in the VOP3P form whose third
// operand is the inline constant 0 (written through the builtin, the zero would be moved into
// the destination register first for the accumulate-in-place form).
__device__ __forceinline__ int dot4_first(uint32_t a, uint32_t b) {
    int r;
    asm("v_dot4_i32_i8 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
    return r;
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

// Constants of the IQ4_NL decode, held in VGPRs: gfx9 VOP3 instructions take no literal
// and at most one SGPR, so register-resident constants let v_and_or_b32 fold two operations.
struct IQ4Consts {
    uint32_t m7, m4, c0123;
    __device__ __forceinline__ IQ4Consts() : m7(opaque_u(0x07070707u)), m4(opaque_u(0x04040404u)), c0123(opaque_u(0x03020100u)) {}
    __device__ static __forceinline__ uint32_t opaque_u(uint32_t v) {
        asm volatile("" : "+v"(v));
        return v;
    }
};
// ... plus the four signed level words, so they are not re-materialized for every block.
struct IQ4Levels : IQ4Consts {
    uint32_t t0, t1, t2, t3;
    __device__ __forceinline__ IQ4Levels()
        : t0(opaque_u(kv_word(0))), t1(opaque_u(kv_word(1))), t2(opaque_u(kv_word(2))), t3(opaque_u(kv_word(3))) {}
};
struct NoConsts {};

// One dword of IQ4_NL index bytes (elements j..j+3 in the low nibbles, j+16..j+19 in the
// high nibbles) -> the int8 levels of both element groups (13 VALU).  Per group of four
// indices: two v_perm look the low 3 bits up in each half of the level table, a third picks
// per byte (byte k of the selector = k, or k + 4 when the index's bit 3 is set).
__device__ __forceinline__ void iq4nl_decode_word(uint32_t q, uint32_t& lo, uint32_t& hi, const IQ4Levels& k) {
    const uint32_t l7 = q & k.m7, h7 = (q >> 4) & k.m7;
    lo = perm(perm(k.t3, k.t2, l7), perm(k.t1, k.t0, l7), ((q >> 1) & k.m4) | k.c0123);
    hi = perm(perm(k.t3, k.t2, h7), perm(k.t1, k.t0, h7), ((q >> 5) & k.m4) | k.c0123);
}

// ------------------------------------------------------------------ FP16 dequantization
//
// Integer factors q in [-128, 127] held as biased bytes u = q + 128 (q ^ 0x80).  Placing u under
// the exponent byte 0x64 forms the binary16 value 1024 + u exactly; subtracting 1152 (exact, all
// integers below 2048) gives q; one binary16 multiply by the block scale d rounds the exact
// product d*q once to nearest even (fp16 denormals kept).  Two values per packed instruction.

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// Biased level table of IQ4_NL (byte i of word j = level 4j+i + 128).
constexpr uint32_t kvu_word(int j) { return kv_word(j) ^ 0x80808080u; }

// Four biased bytes -> four binary16 values d*q (two dwords, value order kept).
__device__ __forceinline__ void u8x4_to_f16(uint32_t u, half2_t dd, uint32_t& lo, uint32_t& hi) {
    const half2_t bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
    const uint32_t a = perm(0x64646464u, u, 0x04010400u);  // [u0, 0x64, u1, 0x64]
    const uint32_t b = perm(0x64646464u, u, 0x04030402u);  // [u2, 0x64, u3, 0x64]
    const half2_t qa = __builtin_bit_cast(half2_t, a) + bias;
    const half2_t qb = __builtin_bit_cast(half2_t, b) + bias;
    lo = __builtin_bit_cast(uint32_t, qa * dd);
    hi = __builtin_bit_cast(uint32_t, qb * dd);
}

__device__ __forceinline__ half2_t splat_h2(uint32_t dbits) {
    const _Float16 d = __builtin_bit_cast(_Float16, (uint16_t)(dbits & 0xFFFFu));
    return half2_t{d, d};
}

// IQ4_NL: four 4-bit indices (the low 3 bits in i7, the bit-3 selector in i8, as
// iq4nl_decode_word forms them) -> the four signed int8 levels.
__device__ __forceinline__ uint32_t iq4nl_lookup_s(uint32_t i7, uint32_t i8) {
    const uint32_t lo = perm(kv_word(1), kv_word(0), i7);
    const uint32_t hi = perm(kv_word(3), kv_word(2), i7);
    return perm(hi, lo, i8);
}

// IQ4_NL: four 4-bit indices (as for iq4nl_lookup) -> four biased levels.
__device__ __forceinline__ uint32_t iq4nl_lookup_u(uint32_t i7, uint32_t i8) {
    const uint32_t lo = perm(kvu_word(1), kvu_word(0), i7);
    const uint32_t hi = perm(kvu_word(3), kvu_word(2), i7);
    return perm(hi, lo, i8);
}

// ------------------------------------------------------------------ weight units
//
// A "unit" is one 32-value block of a row: what one lane loads and decodes in one step.  It is
// delivered as 8 dwords of int8 factors (values 4i..4i+3 in dword i), the fp16 scale of its
// block and an integer multiplier (1 except CB3).
//   Q8_0   : 34-byte block, read as the 9 aligned dwords around it
//   IQ4_NL : 18-byte block, read as the 5 aligned dwords around it
//   CB3    : one 32-value sub-block of a 256-value super-block
// Blocks of 34 and 18 bytes start on a 4-byte or a 2-byte boundary; the loads start at the
// enclosing 4-byte boundary and one v_perm per dword realigns them (selector 0x05040302 when
// the block is 4-byte aligned, 0x07060504 when it is 2 bytes past one).
//
// The blocks one lane takes from a row lie a whole number of dwords apart (16 or 64 blocks of
// 34 or 18 bytes; 2 or 8 super-blocks of 110 bytes), so they share their offset mod 4: a
// per-lane Frame holds the 4-byte-aligned field addresses and the realignment of the lane's
// first block, and block j of the lane is read at those addresses plus j times the lane
// stride (a constant the loads carry as their immediate offset).

template <int WT>
struct Unit;

__device__ __forceinline__ uint32_t realign_sel(uint32_t off) { return (off & 2u) ? 0x07060504u : 0x05040302u; }
__device__ __forceinline__ uint32_t realign_scale(uint32_t w0, uint32_t off) { return (off & 2u) ? (w0 >> 16) : (w0 & 0xFFFFu); }

// Q8_0 / IQ4_NL lane frame: the 4-byte boundary at or before the lane's first block, and 2 if
// that block starts 2 bytes past it (else 0).
struct AlignFrame {
    uint32_t a, hi;
    __device__ static __forceinline__ AlignFrame of(uint32_t off) { return {off & ~3u, off & 2u}; }
};

template <>
struct Unit<kQ8_0> {
    using Consts = NoConsts;
    static constexpr int RAW = 9;
    static constexpr int BYTES = 34;
    using Frame = AlignFrame;
    __device__ static __forceinline__ Frame frame(uint32_t off, int) { return AlignFrame::of(off); }
    __device__ static __forceinline__ void load(rsrc_t r, const Frame& f, uint32_t jb, uint32_t* raw) {
        const uint32_t a = f.a + jb;
        const u32x4 x = ld128(r, a), y = ld128(r, a + 16);
        raw[0] = x.x; raw[1] = x.y; raw[2] = x.z; raw[3] = x.w;
        raw[4] = y.x; raw[5] = y.y; raw[6] = y.z; raw[7] = y.w;
        raw[8] = ld32(r, a + 32);
    }
    __device__ static __forceinline__ void decode(const uint32_t* raw, const Frame& f, uint32_t* W, uint32_t& dw,
                                                  int& mult, const NoConsts&) {
        const uint32_t sel = realign_sel(f.hi);
        dw = realign_scale(raw[0], f.hi);
#pragma unroll
        for (int i = 0; i < 8; ++i) W[i] = perm(raw[i + 1], raw[i], sel);
        mult = 1;
    }
};

template <>
struct Unit<kIQ4_NL> {
    using Consts = IQ4Levels;
    static constexpr int RAW = 5;
    static constexpr int BYTES = 18;
    using Frame = AlignFrame;
    __device__ static __forceinline__ Frame frame(uint32_t off, int) { return AlignFrame::of(off); }
    __device__ static __forceinline__ void load(rsrc_t r, const Frame& f, uint32_t jb, uint32_t* raw) {
        const uint32_t a = f.a + jb;
        const u32x4 x = ld128(r, a);
        raw[0] = x.x; raw[1] = x.y; raw[2] = x.z; raw[3] = x.w;
        raw[4] = ld32(r, a + 16);
    }
    __device__ static __forceinline__ void decode(const uint32_t* raw, const Frame& f, uint32_t* W, uint32_t& dw,
                                                  int& mult, const IQ4Levels& k) {
        const uint32_t sel = realign_sel(f.hi);
        dw = realign_scale(raw[0], f.hi);
#pragma unroll
        for (int i = 0; i < 4; ++i) iq4nl_decode_word(perm(raw[i + 1], raw[i], sel), W[i], W[i + 4], k);
        mult = 1;
    }
};

// Planes [GP, What changed: GGUF blocks repacked into an int8 plane plus scales]: a row of
// Q8_0 / IQ4_NL blocks is cut into tiles of 16 blocks, each the 16 blocks' factor bytes back to
// back (32 or 16 per block) followed by their 16 fp16 scales, so a tile takes the bytes of its 16
// blocks and a row keeps its size.  The kernels take rows of whole tiles (k a multiple of 512).
// The lanes of a row take blocks l, l + L, ... with L a multiple of 16, so lane l always sits at
// position p = l mod 16 of its tiles: its factor bytes start 16-byte aligned at the tile start
// plus FB p, its scale at the tile start plus 16 FB + 2 p.  The frame holds both addresses of
// the lane's first block (computed from the block-layout offset the row engine passes, tile
// start + BYTES p); block j of the lane lies j times the lane stride (whole tiles) further.
struct PlaneFrame {
    uint32_t q, d;
};

template <>
struct Unit<kQ8_0P> {
    using Consts = NoConsts;
    static constexpr int RAW = 9;
    static constexpr int BYTES = 34;
    using Frame = PlaneFrame;
    __device__ static __forceinline__ Frame frame(uint32_t off, int l) {
        const uint32_t p = (uint32_t)l & 15u;
        return {off - 2u * p, off + 512u - 32u * p};
    }
    __device__ static __forceinline__ void load(rsrc_t r, const Frame& f, uint32_t jb, uint32_t* raw) {
        const u32x4 x = ld128(r, f.q + jb), y = ld128(r, f.q + jb + 16);
        raw[0] = x.x; raw[1] = x.y; raw[2] = x.z; raw[3] = x.w;
        raw[4] = y.x; raw[5] = y.y; raw[6] = y.z; raw[7] = y.w;
        raw[8] = ld16(r, f.d + jb);
    }
    __device__ static __forceinline__ void decode(const uint32_t* raw, const Frame&, uint32_t* W, uint32_t& dw, int& mult,
                                                  const NoConsts&) {
#pragma unroll
        for (int i = 0; i < 8; ++i) W[i] = raw[i];
        dw = raw[8];
        mult = 1;
    }
};

template <>
struct Unit<kIQ4_NLP> {
    using Consts = IQ4Levels;
    static constexpr int RAW = 5;
    static constexpr int BYTES = 18;
    using Frame = PlaneFrame;
    __device__ static __forceinline__ Frame frame(uint32_t off, int l) {
        const uint32_t p = (uint32_t)l & 15u;
        return {off - 2u * p, off + 256u - 16u * p};
    }
    __device__ static __forceinline__ void load(rsrc_t r, const Frame& f, uint32_t jb, uint32_t* raw) {
        const u32x4 x = ld128(r, f.q + jb);
        raw[0] = x.x; raw[1] = x.y; raw[2] = x.z; raw[3] = x.w;
        raw[4] = ld16(r, f.d + jb);
    }
    __device__ static __forceinline__ void decode(const uint32_t* raw, const Frame&, uint32_t* W, uint32_t& dw, int& mult,
                                                  const IQ4Levels& k) {
#pragma unroll
        for (int i = 0; i < 4; ++i) iq4nl_decode_word(raw[i], W[i], W[i + 4], k);
        dw = raw[4];
        mult = 1;
    }
};

// Byte k of q, shifted left by 6 (one SDWA instruction).
__device__ __forceinline__ uint32_t byte_shl6(uint32_t q, int k) {
    uint32_t r;
    switch (k) {
        case 0: asm("v_lshlrev_b32_sdwa %0, 6, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_0" : "=v"(r) : "v"(q)); break;
        case 1: asm("v_lshlrev_b32_sdwa %0, 6, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_1" : "=v"(r) : "v"(q)); break;
        case 2: asm("v_lshlrev_b32_sdwa %0, 6, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_2" : "=v"(r) : "v"(q)); break;
        default: asm("v_lshlrev_b32_sdwa %0, 6, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_3" : "=v"(r) : "v"(q)); break;
    }
    return r;
}

// CB3 super-block field offsets
constexpr int kCB3Bytes = 110, kCB3Qs = 2, kCB3Qh = 66, kCB3Signs = 74, kCB3Scales = 106;

// Expand 4 sign bits into a per-byte mask word x with x byte j = bit j (0 or 1).
__device__ __forceinline__ uint32_t sign_bits_to_bytes(uint32_t nib) {
    return __umul24(nib, 0x00204081u) & 0x01010101u;
}

// Apply per-byte signs to four codebook magnitudes [GP, What changed: sign masks]: each byte
// whose sign bit is set is replaced by its two's-complement negation (all ones XOR the byte,
// plus one), the other bytes pass unchanged.  No magnitude is 0, so the added one never carries
// into the neighbouring byte.
__device__ __forceinline__ uint32_t cb3_signed(uint32_t g, uint32_t nib) {
    const uint32_t x = sign_bits_to_bytes(nib);
    // (x << 8) - x = x * 255; kept as a shift and a subtract (the compiler would otherwise emit
    // a quarter-rate v_mul_lo_u32)
    const uint32_t mask = IQ4Consts::opaque_u(x << 8) - x;
    return (g ^ mask) + x;
}

template <>
struct Unit<kCB3> {
    using Consts = NoConsts;
    static constexpr int RAW = 8;
    static_assert((kCB3Signs - kCB3Qs) % 4 == 0, "qs and sign windows share their realignment");
    // Lane frame for sub-block ss of the super-block at byte `off` (even): the 4-byte-aligned
    // addresses of the qs window, the sign window and the dwords holding the qh byte, the scales
    // byte and d, and the shifts that realign them.
    struct Frame {
        uint32_t q, s, qh, sc, d;
        uint32_t shq, shqh, shsc, shd;
    };
    __device__ static __forceinline__ Frame frame(uint32_t off, int ss) {
        Frame f;
        f.q = (off + kCB3Qs + 8 * ss) & ~3u;
        f.s = (off + kCB3Signs + 4 * ss) & ~3u;
        f.qh = (off + kCB3Qh + ss) & ~3u;
        f.sc = (off + kCB3Scales + (ss >> 1)) & ~3u;
        f.d = off & ~3u;
        f.shq = (off + kCB3Qs) & 3u;  // 8 ss and 4 ss keep the low bits
        f.shqh = 8u * ((off + kCB3Qh + ss) & 3u);
        f.shsc = 8u * ((off + kCB3Scales + (ss >> 1)) & 3u) + 4u * (ss & 1);
        f.shd = 8u * (off & 2u);
        return f;
    }
    // raw: [0..2] qs window, [3..4] signs window, [5] the dword holding the qh byte, [6] the dword
    // holding the scales byte, [7] the dword holding d.  Whole dwords, no 8/16-bit loads: their
    // zero-extension would be computed (and waited for) where the loaded values are first
    // shared.
    __device__ static __forceinline__ void load(rsrc_t r, const Frame& f, uint32_t jb, uint32_t* raw) {
        const u32x3 q = ld96(r, f.q + jb);
        raw[0] = q.x; raw[1] = q.y; raw[2] = q.z;
        const u32x2 s = ld64(r, f.s + jb);
        raw[3] = s.x; raw[4] = s.y;
        raw[5] = ld32(r, f.qh + jb);
        raw[6] = ld32(r, f.sc + jb);
        raw[7] = ld32(r, f.d + jb);
    }
    // realigned qs and sign words, qh byte, multiplier and d bits of a loaded sub-block
    __device__ static __forceinline__ void fields(const uint32_t* raw, const Frame& f, uint32_t& q0, uint32_t& q1,
                                                  uint32_t& sg, uint32_t& qh, uint32_t& dw, int& mult) {
        q0 = align8(raw[1], raw[0], f.shq);
        q1 = align8(raw[2], raw[1], f.shq);
        sg = align8(raw[4], raw[3], f.shq);
        qh = raw[5] >> f.shqh;
        mult = 1 + 2 * (int)((raw[6] >> f.shsc) & 15u);
        dw = (raw[7] >> f.shd) & 0xFFFFu;
    }
    // grid: the 512 codebook words in LDS
    __device__ static __forceinline__ void decode(const uint32_t* raw, const Frame& f, const uint32_t* grid, uint32_t* W,
                                                  uint32_t& dw, int& mult) {
        uint32_t q0, q1, sg, qh;
        fields(raw, f, q0, q1, sg, qh, dw, mult);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t qb = ((e < 4 ? q0 : q1) >> (8 * (e & 3))) & 0xFFu;
            const uint32_t idx = qb | (((qh >> e) & 1u) << 8);
            W[e] = cb3_signed(grid[idx], (sg >> (4 * e)) & 15u);
        }
    }
    // The same with the signs already applied: sgrid is the signed codebook in LDS.
    __device__ static __forceinline__ void decode_signed(const uint32_t* raw, const Frame& f, const uint32_t* sgrid,
                                                         uint32_t* W, uint32_t& dw, int& mult) {
        uint32_t q0, q1, sg, qh;
        fields(raw, f, q0, q1, sg, qh, dw, mult);
        // byte address of word (qs byte | qh bit << 8) * 16 + sign nibble: qs byte << 6 (one
        // SDWA shift), | nibble << 2, | qh bit << 14 (the table's own address is the constant
        // offset of the LDS read)
        const uint32_t base = (uint32_t)(size_t)(__attribute__((address_space(3))) const uint32_t*)sgrid;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t t = byte_shl6(e < 4 ? q0 : q1, e & 3);
            const uint32_t a = (__builtin_amdgcn_ubfe(qh, e, 1) << 14) | ((__builtin_amdgcn_ubfe(sg, 4 * e, 4) << 2) | t);
            W[e] = *(__attribute__((address_space(3))) const uint32_t*)(size_t)(base + a);
        }
    }
};

// The signed codebook: word 16 idx + n = codebook entry idx with the signs of nibble n applied.
constexpr int kCB3SignedWords = 512 * 16;  // 32 KiB

// ------------------------------------------------------------------ DPP lane moves

// The value of the lane that DPP control CTRL selects within this lane's row of 16 (quad_perm
// 0x00-0xFF, row_mirror 0x140, row_half_mirror 0x141).
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, dpp_i<CTRL>(__builtin_bit_cast(int, v)));
}

// ------------------------------------------------------------------ q8_1 quantization

// x / d rounded half away from zero (exact: v - trunc(v) is exact in binary32).
__device__ __forceinline__ int round_away(float v) {
    const float t = __builtin_truncf(v);
    const float r = __builtin_fabsf(v - t) >= 0.5f ? t + __builtin_copysignf(1.0f, v) : t;
    return (int)r;
}

// q8_1 of one 32-value block held by 32 consecutive lanes (an aligned half wave), lane j
// holding value j [DQ, Change: the q8_1 quantizer's 32-value blocks]: amax over the half wave,
// d = amax / 127 (IEEE binary32 division), q_j = x_j / d rounded half away from zero,
// s = fp16(d * sum q) with the product in binary32; an all-zero block is all zeros.  Returns
// q_j; `hdr` (d | s << 16) is the same in all 32 lanes.  Every lane of the wave must call it.
__device__ __forceinline__ int quantize_lanes32(float v, uint32_t& hdr) {
    // the maximum and the integer sum over the half wave: within a row of 16 lanes by DPP (quad
    // partners, then the other quad of the half row, then the other half row), then across the
    // two rows with one lane exchange; both are exact in any order
    float amax = __builtin_fabsf(v);
    amax = __builtin_fmaxf(amax, dpp<0xB1>(amax));
    amax = __builtin_fmaxf(amax, dpp<0x4E>(amax));
    amax = __builtin_fmaxf(amax, dpp<0x141>(amax));
    amax = __builtin_fmaxf(amax, dpp<0x140>(amax));
    amax = __builtin_fmaxf(amax, __shfl_xor(amax, 16, 64));
    const float d = amax / 127.0f;
    const bool zero = amax == 0.0f || d == 0.0f;
    int q = 0;
    if (!zero) {
        q = round_away(v / d);
        q = q > 127 ? 127 : (q < -127 ? -127 : q);
    }
    int sum = q;
    sum += dpp_i<0xB1>(sum);
    sum += dpp_i<0x4E>(sum);
    sum += dpp_i<0x141>(sum);
    sum += dpp_i<0x140>(sum);
    sum += __shfl_xor(sum, 16, 64);
    hdr = zero ? 0u : (f2h(d) | (f2h(opaque(d * (float)sum)) << 16));
    return q;
}

// Pack the int8 q of lanes j..j+3 (j a multiple of 4) into one dword, valid in lane j (DPP
// quad broadcasts of lanes 1, 2, 3 of the quad).
__device__ __forceinline__ uint32_t pack4_lanes(int q) {
    const int b = q & 0xFF;
    const uint32_t b1 = (uint32_t)dpp_i<0x55>(b), b2 = (uint32_t)dpp_i<0xAA>(b), b3 = (uint32_t)dpp_i<0xFF>(b);
    return (uint32_t)b | (b1 << 8) | (b2 << 16) | (b3 << 24);
}

// Wait for every vector memory operation of this wave (vmcnt 0; expcnt and lgkmcnt not
// waited).  Used on the back edge of a pass loop: with nothing outstanding when a pass starts,
// the compiler's wait counting does not carry the previous pass's loads into the next pass
// (where it would wait for them between the next pass's loads).
__device__ __forceinline__ void vm_drain() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Workgroup barrier for LDS written with ds_write: waits for this wave's LDS operations only
// (a __syncthreads release fence would also wait for outstanding direct-to-LDS loads).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt: no wait
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// ------------------------------------------------------------------ cross-lane sums


// Lane l (of a 16-lane DPP row) pairs with lane l ^ m in the four steps m = 15, 7, 2, 1
// (row_mirror, row_half_mirror, quad_perm [2,3,0,1], quad_perm [1,0,3,2]).  One step adds the
// value a lane keeps to the value its partner sends.  With NC per-lane partials (NC = 1, 2, 4,
// 8), the first log2 NC steps also halve the values a lane holds: the lanes whose bit 3 (then
// 2, then 1) is set keep the upper half of the columns, the partner the lower half.  Each
// column's sum is then the same addition tree whatever NC (partners add the same two values,
// in either order), and lane l ends with the sum over the row of column row_col<NC>(l).
template <int NC>
__device__ __forceinline__ int row_col(int l) {
    return NC == 8 ? (l >> 1) & 7 : NC == 4 ? (l >> 2) & 3 : NC == 2 ? (l >> 3) & 1 : 0;
}
template <int CTRL, int N>
__device__ __forceinline__ void row_step(float (&a)[8], bool upper) {
    if constexpr (N == 1) {
        a[0] += dpp<CTRL>(a[0]);
    } else {
        float keep[N / 2], send[N / 2];
#pragma unroll
        for (int k = 0; k < N / 2; ++k) {
            keep[k] = upper ? a[k + N / 2] : a[k];
            send[k] = upper ? a[k] : a[k + N / 2];
        }
#pragma unroll
        for (int k = 0; k < N / 2; ++k) a[k] = keep[k] + dpp<CTRL>(send[k]);
    }
}
template <int NC>
__device__ __forceinline__ float row16_sums(const float (&acc)[NC], int l) {
    static_assert(NC == 1 || NC == 2 || NC == 4 || NC == 8, "1, 2, 4 or 8 columns");
    float a[8];
#pragma unroll
    for (int c = 0; c < NC; ++c) a[c] = acc[c];
    row_step<0x140, NC>(a, (l & 8) != 0);
    row_step<0x141, (NC >= 2 ? NC / 2 : 1)>(a, (l & 4) != 0);
    row_step<0x4E, (NC >= 4 ? NC / 4 : 1)>(a, (l & 2) != 0);
    row_step<0xB1, 1>(a, false);
    return a[0];
}

}  // namespace qmm
