/*
 * qmm.h -- C ABI of libqmm: block-quantized weight x q8_1 activation products on MI355X (gfx950).
 *
 * Sources (cited by page title and section):
 *   [PF] #2356 "pf_wmma: a second Volta prompt-expert kernel for IQ2_S gate/up and IQ4_NL down"
 *   [DQ] #1525 "prefill: dense IQ4_XS / Q8_0 to FP16 with 16-byte stores, swiglu + q8_1 and the
 *        MoE combine + hyper-connection write fused"
 *   [IQ] #242  "IQ kernels: decode each weight part once for every column and entry, bitwise identical"
 *   [GP] #1424 "Pascal GP100: a Q8_0 decode GEMV ... and IQ3_XXS / IQ3_S tables in shared memory"
 *
 * General rules for every entry point:
 *   - All pointers are DEVICE pointers unless a comment says "host".  The caller owns every
 *     buffer; the library allocates nothing and keeps no state between calls (reentrant),
 *     except where an entry point says otherwise (qmm_planes_alloc owns a packed copy until
 *     qmm_planes_release).
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Calls are
 *     asynchronous on that stream; outputs are ready when the stream reaches the call.
 *   - Argument errors are reported synchronously by the return value, before anything is
 *     launched; a launch error is reported as QMM_EHIP.  Faults inside a kernel surface at the
 *     caller's next synchronisation.
 *   - Weight formats (little-endian, every block starts with its fp16 scale d):
 *       QMM_Q8_0   34 B per 32 values : d, int8 q[32]                    value = d*q
 *       QMM_IQ4_NL 18 B per 32 values : d, 16 bytes of 4-bit indices into the sixteen IQ4_NL
 *                                       levels; value j<16 = low nibble of byte j, j>=16 = high
 *                                       nibble of byte j-16                value = d*level
 *       QMM_CB3   110 B per 256 values: d, qs[64], qh[8], signs[32], scales[4] (IQ3_S-like
 *                                       codebook: 9-bit index = qs[i] | bit i%8 of qh[i/8] << 8
 *                                       selects 4 magnitudes from `grid`; sign bit v%8 of
 *                                       signs[v/8]; sub-block s of 32 values has multiplier
 *                                       1 + 2*((scales[s/2] >> 4*(s%2)) & 15))
 *     A weight matrix is row-major: nrows rows of qmm_row_bytes(wtype, k) bytes each.
 *     `grid` (CB3 only) is 512 entries x 4 uint8 magnitudes (2048 bytes), each in [1, 63].
 *   - q8_1 activations: 36 B per 32 values = fp16 d, fp16 s, int8 q[32]; a column of k values
 *     is k/32 consecutive blocks, columns are consecutive ([ncols][k/32][36]).
 */
#ifndef QMM_H
#define QMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* weight formats */
#define QMM_Q8_0 1
#define QMM_IQ4_NL 2
#define QMM_CB3 3
#define QMM_F16 4 /* binary16 weights [rows][k] (qgemm_dense only): 2 bytes per value */

/* status codes */
#define QMM_OK 0
#define QMM_EINVAL (-1)       /* bad argument: null pointer, size out of range, ... */
#define QMM_EUNSUPPORTED (-2) /* a shape or format the kernels decline (caller keeps another path) */
#define QMM_EALIGN (-3)       /* a pointer or stride is not aligned as documented */
#define QMM_EHIP (-4)         /* the HIP runtime reported an error at launch */
#define QMM_ESPACE (-5)       /* workspace smaller than the *_workspace() query returned */

/* flags */
#define QMM_FLAG_DEBUG_INTERMEDIATES 1u /* also write fp32 intermediates into the workspace */

/* Version of this ABI (major*100 + minor). */
int qmm_version(void);

/* Host-only.  Human-readable text of a status code (never NULL). */
const char* qmm_status_str(int status);

/* Host-only.  Bytes of one weight row of k values, or 0 when k is not a positive multiple of
 * the format's block (32 values; 256 for CB3; 1 for QMM_F16) or wtype is unknown. */
int64_t qmm_row_bytes(int wtype, int64_t k);

/* q8_1 quantization of activations [DQ, Change: the q8_1 quantizer's 32-value blocks; GP, What
 * changed: q8_1 activations].  Per 32-value block: amax = max |x|; d = amax/127 (binary32);
 * q_j = x_j/d (binary32 division) rounded half away from zero; an all-zero block gives
 * d = q = s = 0; stored d = fp16(d), s = fp16(d * sum q).
 *   x   : float [ncols][ldx], column c's k values at x + c*ldx; ldx >= k; 4-byte aligned.
 *   xq  : output, ncols*(k/32)*36 bytes, 4-byte aligned.
 *   k   : multiple of 32, > 0.  ncols >= 1.
 * Errors: QMM_EINVAL (null, k, ncols, ldx), QMM_EALIGN. */
int qmm_quantize_q8_1(const float* x, int64_t k, int ncols, int64_t ldx, void* xq, void* stream);

/* FP16 dequantization [DQ, Change: dequant to FP16 with 16-byte stores; PF, Summary: the FP16
 * weights the tensor cores get].  out[r*ld + j] = binary16 nearest-even rounding of the exact
 * value of weight (r, j); columns k..ld-1 are not written.
 *   w    : nrows * qmm_row_bytes(wtype, k) bytes, 2-byte aligned.
 *   grid : CB3 codebook (2048 bytes), ignored (may be NULL) for other formats.
 *   out  : uint16 (binary16 bits) [nrows][ld], ld >= k, 2-byte aligned.  When out is 16-byte
 *          aligned and ld % 8 == 0 every thread writes 8 values with one 16-byte store.
 * Errors: QMM_EINVAL, QMM_EALIGN. */
int qmm_dequant_f16(int wtype, const void* w, const uint8_t* grid, int64_t nrows, int64_t k,
                    uint16_t* out, int64_t ld, void* stream);

/* Dense multi-column decode GEMV [IQ, What it does: the weight side is loaded and decoded once
 * and applied to every column, 1/2/4/8 columns per pass, 8 at a time beyond 8; GP, What
 * changed: 16-byte weight loads, activations staged once per workgroup].
 *   y[c*ldy + r] = sum over 32-value blocks b of  (d_w(r,b) * d_a(c,b)) * isum(r,b,c)
 * in binary32, isum the exact integer dot of the block's integer weight factors with the q8_1
 * int8 values (for CB3 the sub-block multiplier is folded into isum).  Every column of an
 * n-column call is bitwise equal to a one-column call on that column.
 *   w    : nrows x qmm_row_bytes(wtype, k) bytes, 4-byte aligned.
 *   grid : CB3 codebook or NULL.
 *   xq   : q8_1 [ncols][k/32][36], 4-byte aligned.   y: float, ldy >= nrows, 4-byte aligned.
 *   k    : multiple of 32 (of 256 for CB3), at most 32768.  ncols >= 1 (any count; passes
 *          of 8).
 * Errors: QMM_EINVAL (k not a multiple of 32 / 256, no rows or columns), QMM_EALIGN,
 *         QMM_EUNSUPPORTED (k above 32768, a buffer of 4 GiB or more). */
int qgemv_dense(int wtype, const void* w, const uint8_t* grid, int64_t nrows, int64_t k,
                const void* xq, int ncols, float* y, int64_t ldy, void* stream);

/* Decode GEMV on 1, 2 or 4 fp32 activation columns, quantized to q8_1 inside the kernel [IQ,
 * What it does: decode GEMV on q8_1 activations; DQ, Change: the q8_1 quantizer]: y equals
 * qgemv_dense(wtype, w, grid, nrows, k, qmm_quantize_q8_1(x), ncols, y, ldy) bit for bit, in
 * one launch instead of two (every workgroup quantizes the columns for itself; the q8_1 bytes
 * are not written out).
 *   w, grid : as qgemv_dense.   x: float [ncols][k], 4-byte aligned.
 *   y    : float, y[c*ldy + r], ldy >= nrows, 4-byte aligned.
 *   k    : multiple of 32 (of 256 for CB3), at most 3072 (rows of at most 96 blocks).
 * Errors: QMM_EINVAL, QMM_EALIGN, QMM_EUNSUPPORTED (ncols other than 1, 2, 4; k above 3072; a
 *         weight buffer of 4 GiB or more). */
int qgemv_dense_f32(int wtype, const void* w, const uint8_t* grid, int64_t nrows, int64_t k,
                    const float* x, int ncols, float* y, int64_t ldy, void* stream);

/* Test hook: the per-block integer sums isum(r, b, c) of qgemv_dense, computed by the same
 * device decode and dot code.  sums: int32 [ncols][nrows][k/32].  Same argument rules as
 * qgemv_dense. */
int qmm_debug_block_sums(int wtype, const void* w, const uint8_t* grid, int64_t nrows, int64_t k,
                         const void* xq, int ncols, int32_t* sums, void* stream);

/* Measurement hook: a plain streaming read of nbytes from p in one launch of `grid` workgroups
 * of `threads` threads (256, 512 or 1024): workgroup w reads the w-th of grid contiguous runs,
 * `unroll` (4, 8 or 16) 16-byte raw-buffer loads in flight per thread, no other work.  The
 * reference for the HBM time of the decode kernels at the same byte count.  Thread t of
 * workgroup w writes the XOR of the words it read to out[w * threads + t].
 *   p    : device, 16-byte aligned; nbytes a multiple of 16, below 4 GiB.
 *   out  : device uint32 [grid * threads], 4-byte aligned.
 * Errors: QMM_EINVAL, QMM_EALIGN, QMM_EUNSUPPORTED (other threads / unroll), QMM_EHIP. */
int qmm_debug_stream_read(const void* p, uint64_t nbytes, uint32_t* out, int grid, int threads,
                          int unroll, void* stream);

/* Measurement hook: `grid` workgroups of 256 threads, each wave running 8 independent fp16 MFMA
 * accumulators (v_mfma_f32_32x32x16_f16, 32768 FLOP each) for `iters` rounds from registers
 * only: grid * 4 * 8 * iters * 32768 FLOP, the reference for the prefill GEMM's MFMA rate.
 *   out : device float [grid * 256] (the lanes' accumulator sums), 4-byte aligned.
 * Errors: QMM_EINVAL, QMM_EALIGN, QMM_EHIP. */
int qmm_debug_mfma_loop(float* out, int grid, int iters, void* stream);

/* Workspace bytes qgemv_grouped_experts needs (host). */
size_t qgemv_grouped_experts_workspace(int64_t inter, int nentries, unsigned flags);

/* Grouped MoE-expert decode [IQ, What it does: native_gu / native_down decode each weight part
 * once for every entry of a group; DQ, Change: swiglu then q8_1 of H for the down product].
 * Groups are experts; entries are the (token, slot) pairs routed to them.  For group g (expert
 * e = group_expert[g]) and every entry j in [group_entry_off[g], group_entry_off[g+1]):
 *   x  = q8_1 column entry_col[j] of xq (width hidden)
 *   gv = W_gate[e] x,  uv = W_up[e] x          (qgemv_dense arithmetic, inter rows)
 *   h  = silu(gv) * uv,  silu(z) = z / (1 + exp(-z)) in binary32 (device expf, <= 1 ulp;
 *        IEEE division)
 *   H  = q8_1(h) per 32 consecutive intermediate values          (workspace)
 *   y[j*hidden + r] = (W_down[e] H)[r]                            (binary32; unweighted)
 *   w_gate, w_up : expert e's matrix at byte offset e*gu_expert_stride, inter rows of width
 *                  hidden, format wtype_gu;  w_down: offset e*down_expert_stride, hidden rows of
 *                  width inter, format wtype_down; nexperts matrices each.  4-byte aligned;
 *                  strides multiples of 4 and at least one matrix.
 *   xq, xq_cols  : q8_1 activations [xq_cols][hidden/32][36]; an entry whose column is outside
 *                  [0, xq_cols) reads zeros.
 *   group_expert[ngroups], group_entry_off[ngroups+1], entry_col[nentries]: int32, device.
 *                  A group whose expert is outside [0, nexperts) is skipped; its entry range is
 *                  clamped to [0, nentries).  Entries of no group are not written.
 *   ws   : workspace of qgemv_grouped_experts_workspace() bytes, 16-byte aligned.  Layout:
 *          H q8_1 [nentries][inter/32][36] first; with QMM_FLAG_DEBUG_INTERMEDIATES then gv, uv
 *          as float [nentries][inter] (starting at the next 16-byte boundary).
 *   hidden, inter: multiples of 32 (256 where the format is CB3); a pass of 8 entries must fit
 *          the workgroup's 64 KiB of LDS (hidden, inter <= 6144 in practice).
 * Errors: QMM_EINVAL, QMM_EALIGN, QMM_EUNSUPPORTED, QMM_ESPACE. */
int qgemv_grouped_experts(int wtype_gu, const void* w_gate, const void* w_up,
                          int64_t gu_expert_stride, int wtype_down, const void* w_down,
                          int64_t down_expert_stride, int nexperts, const uint8_t* grid,
                          int64_t hidden, int64_t inter, const void* xq, int xq_cols,
                          const int32_t* group_expert, const int32_t* group_entry_off, int ngroups,
                          const int32_t* entry_col, int nentries, float* y, void* ws,
                          size_t ws_bytes, unsigned flags, void* stream);

/* Allocation-free grouped decode, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  Computes exactly
 * what qgemv_grouped_experts computes with flags = 0 (same kernels: y is bitwise the same), but
 * keeps H in a fixed device array of the library instead of a caller workspace, and calls no
 * allocating routine.  Limit: H of nentries * (inter/32) * 36 bytes must fit the array's
 * qgemv_grouped_experts_noalloc_max_bytes() bytes (4 MiB: 3640 entries at inter 1024), else
 * QMM_ESPACE.  Every call on a GPU uses that GPU's one array, so calls that overlap on one GPU
 * (two streams, two threads) race; the array keeps the last call's H.  Each GPU the library runs
 * on holds its own array until the process ends.  Arguments otherwise as qgemv_grouped_experts.
 * Errors: as qgemv_grouped_experts; QMM_ESPACE (H beyond the array), QMM_EHIP (the array's
 * device address could not be obtained). */
size_t qgemv_grouped_experts_noalloc_max_bytes(void);
int qgemv_grouped_experts_noalloc(int wtype_gu, const void* w_gate, const void* w_up,
                                  int64_t gu_expert_stride, int wtype_down, const void* w_down,
                                  int64_t down_expert_stride, int nexperts, const uint8_t* grid,
                                  int64_t hidden, int64_t inter, const void* xq, int xq_cols,
                                  const int32_t* group_expert, const int32_t* group_entry_off,
                                  int ngroups, const int32_t* entry_col, int nentries, float* y,
                                  void* stream);

/* Workspace bytes qgemm_prefill_experts needs (host). */
size_t qgemm_prefill_experts_workspace(int nexperts, int64_t inter, int64_t nentries,
                                       unsigned flags);

/* Prefill grouped expert GEMM [PF, Summary: weights of one expert dequantized to FP16 in the
 * workgroup's shared memory, FP16 matrix-core math with FP32 sums, over the rows sorted per
 * expert].  For expert e, entries p in [expert_off[e], expert_off[e+1]), token t = sorted_tok[p]:
 *   G = X16[t] . Wg16[e]^T,  U = X16[t] . Wu16[e]^T     (FP16 products, FP32 sums; Wg16/Wu16 are
 *                                                        the qmm_dequant_f16 values)
 *   H16 = fp16(silu(G) * U)                              (workspace; silu in binary32 with the
 *                                                        device expf, error <= 1 ulp)
 *   y[p*hidden + j] = (H16 . Wd16[e]^T)[j]               (FP32, one row per sorted entry;
 *                                                        y 16-byte aligned)
 *   x_f16      : binary16 [ntok][hidden], 16-byte aligned.
 *   sorted_tok : int32 [nentries]; a token outside [0, ntok) reads zeros.  expert_off: int32
 *                [nexperts+1], non-decreasing, expert_off[nexperts] == nentries (offsets are
 *                clamped to [0, nentries]; rows of no expert are not written).
 *   w_gate, w_up (format wtype_gu, inter rows of width hidden) and w_down (wtype_down, hidden
 *   rows of width inter) at e * stride; Q8_0 or IQ4_NL (CB3: QMM_EUNSUPPORTED); 4-byte
 *   aligned, strides multiples of 4.
 *   ws : qgemm_prefill_experts_workspace() bytes, 16-byte aligned.  Layout: H16 [nentries][inter]
 *        binary16 first, then the tile schedule; with QMM_FLAG_DEBUG_INTERMEDIATES then G, U
 *        float [nentries][inter].
 *   hidden, inter: multiples of 64, at most 32768; ntok * hidden * 2, nentries * inter * 2 and
 *   each expert matrix below 4 GiB.
 * Errors: QMM_EINVAL, QMM_EALIGN, QMM_EUNSUPPORTED, QMM_ESPACE. */
int qgemm_prefill_experts(int wtype_gu, const void* w_gate, const void* w_up,
                          int64_t gu_expert_stride, int wtype_down, const void* w_down,
                          int64_t down_expert_stride, int nexperts, int64_t hidden, int64_t inter,
                          const uint16_t* x_f16, int64_t ntok, const int32_t* sorted_tok,
                          const int32_t* expert_off, int64_t nentries, float* y, void* ws,
                          size_t ws_bytes, unsigned flags, void* stream);

/* Workspace bytes qgemm_prefill_experts_q8 needs (host). */
size_t qgemm_prefill_experts_q8_workspace(int nexperts, int64_t hidden, int64_t inter, int64_t ntok,
                                          int64_t nentries, unsigned flags);

/* MMQ-style prefill grouped expert GEMM [DQ, Change: the prefill path on q8_1 activations
 * against the quantized weights, with SwiGLU and the q8_1 quantization of H fused between
 * gate/up and down, H never stored in fp32; IQ, What it does: the decode path's per-block
 * integer dot and float expression].  Computes, over the rows sorted per expert, exactly what
 * qgemv_grouped_experts computes with groups = experts and entry_col = sorted_tok:
 *   xq  = q8_1(X16 as binary32) per 32-value block               (the quantizer's arithmetic)
 *   g,u = per 32-value block b: (d_w d_a) * isum in binary32, summed over b in order
 *   H   = q8_1(silu(g) * u) per 32 consecutive intermediate values (silu in binary32 with the
 *         device expf, error <= 1 ulp, and v_rcp_f32)
 *   y[p*hidden + j] = the same block sum of W_down[e] against H   (binary32; sorted order)
 * The block dots run on int8 MFMA, the per-block scale products on fp32 MFMA.
 *   Arguments as qgemm_prefill_experts (Q8_0 or IQ4_NL; hidden, inter multiples of 64).
 *   ws : qgemm_prefill_experts_q8_workspace() bytes, 16-byte aligned.  Layout (each part at the
 *        next 16-byte boundary): the tokens' q8_1 as planes (int8 [ntok][hidden], then the
 *        binary16 scales [ntok][hidden/32]), H as planes (int8 [nentries][inter], then scales
 *        [nentries][inter/32]), the tile schedule, and with QMM_FLAG_DEBUG_INTERMEDIATES g, u
 *        as float [nentries][inter].
 * Errors: QMM_EINVAL, QMM_EALIGN, QMM_EUNSUPPORTED, QMM_ESPACE. */
int qgemm_prefill_experts_q8(int wtype_gu, const void* w_gate, const void* w_up,
                             int64_t gu_expert_stride, int wtype_down, const void* w_down,
                             int64_t down_expert_stride, int nexperts, int64_t hidden,
                             int64_t inter, const uint16_t* x_f16, int64_t ntok,
                             const int32_t* sorted_tok, const int32_t* expert_off,
                             int64_t nentries, float* y, void* ws, size_t ws_bytes,
                             unsigned flags, void* stream);

/* Dense prompt projection [DQ, Change: dense Q8_0 / IQ4_XS weights dequantized to FP16 with
 * 16-byte stores for a matrix product over the prompt's tokens; PF, Summary: the FP16 weights the
 * matrix cores get, FP32 sums]:
 *   y[t*ldy + r] = sum over k of W16[r][k] * X16[t][k]      (FP16 products, FP32 sums)
 * with W16 the qmm_dequant_f16 values of w (wtype Q8_0 or IQ4_NL: converted in registers inside
 * the GEMM, bitwise those values) or w itself (wtype QMM_F16: binary16 [nrows][k], e.g. the
 * output of qmm_dequant_f16).  fp16 MFMA (32x32x16) with FP32 accumulation.
 *   w     : nrows x qmm_row_bytes(wtype, k) bytes (QMM_F16: 2k bytes per row, 16-byte aligned;
 *           the others 4-byte aligned).   x_f16: binary16 [ntok][k], 16-byte aligned.
 *   y     : float [ntok][ldy], ldy >= nrows, 4-byte aligned.
 *   k     : a multiple of 64, at most 32768.
 * Errors: QMM_EINVAL, QMM_EALIGN, QMM_EUNSUPPORTED (k not a multiple of 64, buffers of 4 GiB or
 *         more). */
int qgemm_dense(int wtype, const void* w, int64_t nrows, int64_t k, const uint16_t* x_f16,
                int64_t ntok, float* y, int64_t ldy, void* stream);

/* Weight planes [GP, What changed: a device-side repack of the GGUF blocks into planes (an int8
 * plane plus scales) for the decode GEMV, the packed copy owned through pack / release calls].
 * Layout (Q8_0 and IQ4_NL): each row is cut into tiles of 16 consecutive blocks (the last tile
 * of a row holds the blocks left); a tile is its n blocks' factor bytes back to back in block
 * order (Q8_0: 32 int8; IQ4_NL: 16 index bytes), then their n fp16 scales in block order.  A row
 * keeps its size and place, so the planes of a matrix take exactly its blocks' bytes and every
 * factor run of a lane starts 16-byte aligned.
 *
 * qmm_pack_planes: writes the planes of the nrows x k matrix w into `planes` (caller-owned,
 *   nrows * qmm_row_bytes(wtype, k) bytes, must not overlap w).  Byte copies only.
 * qmm_planes_alloc: allocates the planes buffer (hipMalloc; the one allocating entry point of the
 *   library), packs w into it on `stream` and returns it in *planes; the caller owns it until
 *   qmm_planes_release (hipFree; synchronizes the device).  *planes is NULL on error.
 * qgemv_planes: qgemv_dense on a planes buffer: the same kernels with the realignment of each
 *   block left out, so y is bitwise qgemv_dense's on the original blocks.  planes 16-byte
 *   aligned, k a multiple of 512 (rows of whole tiles); other arguments as qgemv_dense.
 * Errors: QMM_EINVAL (format other than Q8_0 / IQ4_NL, null, sizes), QMM_EALIGN,
 *         QMM_EUNSUPPORTED (qgemv_planes: k not a multiple of 512, or as qgemv_dense),
 *         QMM_EHIP (allocation or launch). */
int qmm_pack_planes(int wtype, const void* w, int64_t nrows, int64_t k, void* planes, void* stream);
int qmm_planes_alloc(int wtype, const void* w, int64_t nrows, int64_t k, void** planes, void* stream);
int qmm_planes_release(void* planes);
int qgemv_planes(int wtype, const void* planes, int64_t nrows, int64_t k, const void* xq, int ncols,
                 float* y, int64_t ldy, void* stream);

/* MoE combine [DQ, Change: the combine sums a token's expert rows with one fixed
 * thread-to-element mapping and k order; profile block: moe_combine4 reads them at bandwidth].
 *   out[t*ldo + j] = sum over k = 0 .. topk-1 of  weights[t*topk + k] * y[r*hidden + j],
 *                    r = row_idx[t*topk + k]
 * in binary32, from +0, adding in k order, each product and each sum rounded once (no fused
 * multiply-add); an index outside [0, nrows) adds nothing.  Decode: y is a grouped call's
 * [nentries][hidden] output and row_idx the entries of each token; prefill: y is the sorted-
 * entry output and row_idx each token's positions in the sorted order.
 *   y       : float [nrows][hidden], 16-byte aligned.   out: float [ntok][ldo], 16-byte aligned.
 *   row_idx : int32 [ntok][topk];  weights: float [ntok][topk] (both 4-byte aligned).
 *   hidden, ldo: multiples of 4, ldo >= hidden (columns hidden..ldo-1 are not written).
 *   topk    : 1 .. 64.
 * Errors: QMM_EINVAL, QMM_EALIGN, QMM_EUNSUPPORTED (hidden or ldo not a multiple of 4, topk
 *         above 64, sizes of 2^31 or more). */
int qmm_moe_combine(const float* y, int64_t nrows, int64_t hidden, const int32_t* row_idx,
                    const float* weights, int64_t ntok, int topk, float* out, int64_t ldo,
                    void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QMM_H */
