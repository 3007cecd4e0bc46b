/*
 * qmm_oracle.c -- plain CPU oracle for block-quantized weight x q8_1 activation products.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously correct definition the GPU
 * library is checked against.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load it.  It shares no code, header, table or helper with the HIP
 * library and includes nothing from it.
 *
 * Sources (cited by page title and section):
 *   [PF]  #2356 "pf_wmma: a second Volta prompt-expert kernel for IQ2_S gate/up and IQ4_NL down"
 *   [DQ]  #1525 "prefill: dense IQ4_XS / Q8_0 to FP16 with 16-byte stores, swiglu + q8_1 and the
 *         MoE combine + hyper-connection write fused"
 *   [IQ]  #242  "IQ kernels: decode each weight part once for every column and entry, bitwise identical"
 *   [GP]  #1424 "Pascal GP100: a Q8_0 decode GEMV ... and IQ3_XXS / IQ3_S tables in shared memory"
 *
 * Conventions (readings where the pages are silent; each is listed with its reason in the
 * design notes of the repository):
 *   - all multi-byte fields little-endian; every block starts with its fp16 scale d;
 *   - Q8_0   (34 B / 32 values): d, int8 q[32];                     w_j = d * q_j
 *   - IQ4_NL (18 B / 32 values): d, qs[16]; element j < 16 is the low nibble of qs[j],
 *     element j >= 16 the high nibble of qs[j-16];                  w_j = d * KV[nibble]
 *   - CB3    (110 B / 256 values, IQ3_S-like codebook): d, qs[64], qh[8], signs[32], scales[4];
 *     grid index i (0..63) = qs[i] | bit (i%8) of qh[i/8] << 8, covering values 4i..4i+3;
 *     value v is negative when bit (v%8) of signs[v/8] is set; sub-block s = v/32 has the
 *     4-bit scale nib_s = (scales[s/2] >> 4*(s%2)) & 15 and multiplier (1 + 2*nib_s);
 *     w_v = d * (1 + 2*nib_s) * grid[index][v%4] * sign
 *   - q8_1   (36 B / 32 values): d (fp16), s (fp16), int8 q[32]; x_hat_j = d * q_j
 *
 * Floating point: compiled with -ffp-contract=off and without fast-math, so every float
 * operation below is one IEEE-754 binary32 (or binary64) operation rounded to nearest even.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_Q8_0 1
#define OR_IQ4_NL 2
#define OR_CB3 3

/* The sixteen non-linear IQ4_NL levels (the format's fixed table). */
static const int OR_KV[16] = {-127, -104, -83, -65, -49, -35, -22, -10,
                              1,    13,   25,  38,  53,  69,  89,  113};

int or_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads the parallel loops below use from now on (n >= 1); timing only, no effect on any
 * result (every loop writes disjoint outputs). */
void or_set_num_threads(int n) {
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ---------------------------------------------------------------- IEEE half <-> float */

/* Exact value of an IEEE-754 binary16 bit pattern. */
float or_f16_to_f32(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);                 /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m + 1024), e - 25);     /* (1024 + m) * 2^(e-15-10) */
    return (float)(sign ? -v : v);
}

/* Round a double to the nearest integer, ties to even (done by hand so that no
 * floating-point rounding-mode state is involved). */
static double or_rne_int(double q) {
    double f = floor(q);
    double r = q - f;                                /* exact for |q| < 2^52 */
    if (r > 0.5) return f + 1.0;
    if (r < 0.5) return f;
    return (fmod(f, 2.0) == 0.0) ? f : f + 1.0;
}

/* binary16 nearest-even rounding of an exact double value (overflow -> +-inf,
 * gradual underflow kept).  Used for float inputs and for exact products. */
uint16_t or_f64_to_f16(double x) {
    if (isnan(x)) return 0x7E00;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (a >= 65520.0) return sign | 0x7C00;          /* halfway to 2^16 rounds to even = inf */
    if (a < ldexp(1.0, -14)) {                        /* subnormal range: units of 2^-24 */
        double m = or_rne_int(a * ldexp(1.0, 24));  /* m <= 1024; 1024 is the smallest normal */
        return sign | (uint16_t)m;
    }
    int ex;
    frexp(a, &ex);                                    /* a in [2^(ex-1), 2^ex) */
    int E = ex - 1;                                   /* -14 <= E <= 15 */
    double m = or_rne_int(ldexp(a, 10 - E));          /* in [1024, 2048] */
    if (m == 2048.0) { m = 1024.0; E += 1; }
    if (E > 15) return sign | 0x7C00;
    return sign | (uint16_t)(((E + 15) << 10) | ((int)m - 1024));
}

uint16_t or_f32_to_f16(float f) { return or_f64_to_f16((double)f); }

void or_f16_to_f32_array(const uint16_t* h, int64_t n, float* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = or_f16_to_f32(h[i]);
}
void or_f32_to_f16_array(const float* f, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = or_f32_to_f16(f[i]);
}

static uint16_t rd16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* ---------------------------------------------------------------- formats */

static int block_values(int wtype) {
    return wtype == OR_CB3 ? 256 : (wtype == OR_Q8_0 || wtype == OR_IQ4_NL) ? 32 : 0;
}
static int block_bytes(int wtype) {
    return wtype == OR_Q8_0 ? 34 : wtype == OR_IQ4_NL ? 18 : wtype == OR_CB3 ? 110 : 0;
}

int64_t or_row_bytes(int wtype, int64_t k) {
    int bv = block_values(wtype);
    if (bv == 0 || k <= 0 || k % bv) return 0;
    return (k / bv) * block_bytes(wtype);
}

/* Integer weight factor of value j of a row (the weight is d_block * factor), and the
 * fp16 scale d of the block holding it.  Written as the per-value definition of each
 * format (see the header comment); no grouping or table tricks. */
static int weight_int(int wtype, const uint8_t* row, const uint8_t* grid, int64_t j, uint16_t* d) {
    if (wtype == OR_Q8_0) {
        const uint8_t* b = row + (j / 32) * 34;
        *d = rd16(b);
        return (int)(int8_t)b[2 + j % 32];
    }
    if (wtype == OR_IQ4_NL) {
        const uint8_t* b = row + (j / 32) * 18;
        int jj = (int)(j % 32);
        *d = rd16(b);
        int nib = jj < 16 ? (b[2 + jj] & 15) : (b[2 + jj - 16] >> 4);
        return OR_KV[nib];
    }
    /* CB3 */
    const uint8_t* b = row + (j / 256) * 110;
    int v = (int)(j % 256);
    const uint8_t* qs = b + 2;
    const uint8_t* qh = b + 66;
    const uint8_t* signs = b + 74;
    const uint8_t* scales = b + 106;
    int i = v / 4;
    int idx = qs[i] | (((qh[i / 8] >> (i % 8)) & 1) << 8);
    int mag = grid[idx * 4 + v % 4];
    int neg = (signs[v / 8] >> (v % 8)) & 1;
    int s = v / 32;
    int nib = (scales[s / 2] >> (4 * (s % 2))) & 15;
    *d = rd16(b);
    return (1 + 2 * nib) * mag * (neg ? -1 : 1);
}

/* Exact dequantized values: out[r*k + j] = d * factor (exact in double). */
int or_dequant_f64(int wtype, const uint8_t* w, const uint8_t* grid, int64_t nrows, int64_t k,
                   double* out) {
    int64_t rb = or_row_bytes(wtype, k);
    if (!rb) return -1;
    for (int64_t r = 0; r < nrows; ++r)
        for (int64_t j = 0; j < k; ++j) {
            uint16_t d;
            int f = weight_int(wtype, w + r * rb, grid, j, &d);
            out[r * k + j] = (double)or_f16_to_f32(d) * (double)f;
        }
    return 0;
}

/* FP16 dequantization [DQ, Change; PF, Checks]: each value is the exact product rounded
 * once to nearest-even binary16 (never a rounded intermediate scale). */
int or_dequant_f16(int wtype, const uint8_t* w, const uint8_t* grid, int64_t nrows, int64_t k,
                   uint16_t* out, int64_t ld) {
    int64_t rb = or_row_bytes(wtype, k);
    if (!rb || ld < k) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < nrows; ++r)
        for (int64_t j = 0; j < k; ++j) {
            uint16_t d;
            int f = weight_int(wtype, w + r * rb, grid, j, &d);
            out[r * ld + j] = or_f64_to_f16((double)or_f16_to_f32(d) * (double)f);
        }
    return 0;
}

/* ---------------------------------------------------------------- q8_1 activations */

/* q8_1 quantization of 32 consecutive values [DQ, Change: swiglu then q8_1 of H; GP, What
 * changed: q8_1 activations].  The pages fix the block (32 int8 + fp16 d + fp16 sum) but not
 * the rounding; the reading used: d = amax / 127 in binary32, q_j = x_j / d rounded half
 * away from zero, an all-zero block gives d = q = s = 0, stored d = fp16(d),
 * s = fp16(d * sum q) with the product in binary32. */
void or_quantize_block_q8_1(const float* x, uint8_t* out) {
    float amax = 0.0f;
    for (int j = 0; j < 32; ++j) {
        float a = fabsf(x[j]);
        if (a > amax) amax = a;
    }
    float d = amax / 127.0f;
    memset(out, 0, 36);
    if (amax == 0.0f || d == 0.0f) return;
    int sum = 0;
    for (int j = 0; j < 32; ++j) {
        float v = x[j] / d;
        float r = roundf(v);                 /* C roundf: half away from zero, exact */
        int q = (int)r;
        if (q > 127) q = 127;
        if (q < -127) q = -127;
        out[4 + j] = (uint8_t)(int8_t)q;
        sum += q;
    }
    uint16_t dh = or_f32_to_f16(d);
    float s = d * (float)sum;
    uint16_t sh = or_f32_to_f16(s);
    out[0] = dh & 255; out[1] = dh >> 8;
    out[2] = sh & 255; out[3] = sh >> 8;
}

/* x: [ncols][ldx] floats, k values per column; xq: [ncols][k/32] blocks of 36 bytes. */
int or_quantize_q8_1(const float* x, int64_t k, int ncols, int64_t ldx, uint8_t* xq) {
    if (k <= 0 || k % 32 || ncols < 1 || ldx < k) return -1;
    int64_t nb = k / 32;
    for (int c = 0; c < ncols; ++c)
        for (int64_t b = 0; b < nb; ++b)
            or_quantize_block_q8_1(x + c * ldx + 32 * b, xq + (c * nb + b) * 36);
    return 0;
}

/* ---------------------------------------------------------------- block dot products */

/* Integer sum of one 32-value block [IQ, What it does: the load / apply split keeps the same
 * integer chain]: sumi = sum_j factor_j * q_j over the 32 values of activation block b.  For
 * CB3 the factor already includes the sub-block multiplier (1 + 2 nib). */
static int32_t block_isum(int wtype, const uint8_t* row, const uint8_t* grid, int64_t b,
                          const uint8_t* xblk, uint16_t* dw) {
    int32_t s = 0;
    for (int j = 0; j < 32; ++j) {
        uint16_t d;
        int f = weight_int(wtype, row, grid, 32 * b + j, &d);
        *dw = d;
        s += f * (int32_t)(int8_t)xblk[4 + j];
    }
    return s;
}

/* sums: [ncols][nrows][k/32] */
int or_block_sums(int wtype, const uint8_t* w, const uint8_t* grid, int64_t nrows, int64_t k,
                  const uint8_t* xq, int ncols, int32_t* sums) {
    int64_t rb = or_row_bytes(wtype, k);
    if (!rb || ncols < 1) return -1;
    int64_t nb = k / 32;
    for (int c = 0; c < ncols; ++c)
#pragma omp parallel for schedule(static)
        for (int64_t r = 0; r < nrows; ++r)
            for (int64_t b = 0; b < nb; ++b) {
                uint16_t dw;
                sums[(c * nrows + r) * nb + b] =
                    block_isum(wtype, w + r * rb, grid, b, xq + (c * nb + b) * 36, &dw);
            }
    return 0;
}

/* The per-block binary32 term: (d_w * d_a) * sumi, left to right [IQ, What it does: the same
 * float expression for every column].  d_w * d_a is exact in binary32 (two 11-bit
 * significands); the multiplication by sumi is the one rounding. */
static float block_term(uint16_t dw, uint16_t da, int32_t isum) {
    float dd = or_f16_to_f32(dw) * or_f16_to_f32(da);
    return dd * (float)isum;
}

/* Dense multi-column GEMV: y[c][r] = sum over blocks of the binary32 terms, accumulated in
 * double; abs_terms[c][r] = sum of |term| (the scale of the tolerance).  Either output may be
 * NULL. */
int or_gemv(int wtype, const uint8_t* w, const uint8_t* grid, int64_t nrows, int64_t k,
            const uint8_t* xq, int ncols, double* y, double* abs_terms) {
    int64_t rb = or_row_bytes(wtype, k);
    if (!rb || ncols < 1) return -1;
    int64_t nb = k / 32;
    for (int c = 0; c < ncols; ++c)
#pragma omp parallel for schedule(static)
        for (int64_t r = 0; r < nrows; ++r) {
            double acc = 0.0, aabs = 0.0;
            for (int64_t b = 0; b < nb; ++b) {
                const uint8_t* xb = xq + (c * nb + b) * 36;
                uint16_t dw;
                int32_t isum = block_isum(wtype, w + r * rb, grid, b, xb, &dw);
                float t = block_term(dw, rd16(xb), isum);
                acc += (double)t;
                aabs += fabs((double)t);
            }
            if (y) y[c * nrows + r] = acc;
            if (abs_terms) abs_terms[c * nrows + r] = aabs;
        }
    return 0;
}

/* ---------------------------------------------------------------- SwiGLU */

/* h = silu(g) * u with silu(z) = z / (1 + e^-z) [DQ, Change: swiglu, then q8_1 of H].  The
 * exponential is taken in double and rounded to binary32, the rest in binary32; z below
 * about -88.7 gives e = inf and silu = -0 (no NaN). */
float or_silu_mul(float g, float u) {
    float e = (float)exp(-(double)g);
    float den = 1.0f + e;
    float sl = g / den;
    return sl * u;
}

void or_silu_mul_array(const float* g, const float* u, int64_t n, float* h) {
    for (int64_t i = 0; i < n; ++i) h[i] = or_silu_mul(g[i], u[i]);
}

/* ---------------------------------------------------------------- grouped MoE decode */

/* Grouped experts [IQ, What it does: native_gu / native_down over groups and entries; DQ,
 * Change: swiglu then q8_1 of H for the down product].  For group gi (expert e) and each
 * entry k of it, with activation column x = xq column entry_col[k]:
 *   g = W_gate[e] x, u = W_up[e] x                  (dense GEMV terms, double sums)
 *   h = silu(float(g)) * float(u)                    (binary32)
 *   H = q8_1(h) per 32 consecutive intermediate values
 *   y = W_down[e] H                                  (double sum; unweighted, one row per entry)
 * Outputs ([nentries][inter] unless noted; any may be NULL):
 *   g, u, gabs, uabs (double); h (float); hq (q8_1 bytes, [nentries][inter/32][36]);
 *   y, yabs ([nentries][hidden], double). */
int or_grouped(int wtype_gu, const uint8_t* w_gate, const uint8_t* w_up, int64_t gu_stride,
               int wtype_down, const uint8_t* w_down, int64_t down_stride, const uint8_t* grid,
               int64_t hidden, int64_t inter, const uint8_t* xq, const int32_t* group_expert,
               const int32_t* group_off, int ngroups, const int32_t* entry_col, int nentries,
               double* g, double* u, double* gabs, double* uabs, float* h, uint8_t* hq,
               double* y, double* yabs) {
    int64_t rb_gu = or_row_bytes(wtype_gu, hidden), rb_d = or_row_bytes(wtype_down, inter);
    if (!rb_gu || !rb_d || inter % 32) return -1;
    int64_t nbx = hidden / 32, nbh = inter / 32;
    float* hbuf = (float*)malloc(sizeof(float) * inter);
    uint8_t* hqb = (uint8_t*)malloc(36 * nbh);
    double* gt = (double*)malloc(sizeof(double) * inter * 4);
    if (!hbuf || !hqb || !gt) { free(hbuf); free(hqb); free(gt); return -2; }
    for (int gi = 0; gi < ngroups; ++gi) {
        int e = group_expert[gi];
        const uint8_t* wg = w_gate + (int64_t)e * gu_stride;
        const uint8_t* wu = w_up + (int64_t)e * gu_stride;
        const uint8_t* wd = w_down + (int64_t)e * down_stride;
        for (int kk = group_off[gi]; kk < group_off[gi + 1]; ++kk) {
            if (kk < 0 || kk >= nentries) continue;
            const uint8_t* x = xq + (int64_t)entry_col[kk] * nbx * 36;
            or_gemv(wtype_gu, wg, grid, inter, hidden, x, 1, gt, gt + inter);
            or_gemv(wtype_gu, wu, grid, inter, hidden, x, 1, gt + 2 * inter, gt + 3 * inter);
            for (int64_t i = 0; i < inter; ++i) {
                hbuf[i] = or_silu_mul((float)gt[i], (float)gt[2 * inter + i]);
                if (g) g[kk * inter + i] = gt[i];
                if (gabs) gabs[kk * inter + i] = gt[inter + i];
                if (u) u[kk * inter + i] = gt[2 * inter + i];
                if (uabs) uabs[kk * inter + i] = gt[3 * inter + i];
                if (h) h[kk * inter + i] = hbuf[i];
            }
            or_quantize_q8_1(hbuf, inter, 1, inter, hqb);
            if (hq) memcpy(hq + (int64_t)kk * nbh * 36, hqb, 36 * nbh);
            or_gemv(wtype_down, wd, grid, hidden, inter, hqb, 1,
                    y ? y + (int64_t)kk * hidden : NULL, yabs ? yabs + (int64_t)kk * hidden : NULL);
        }
    }
    free(hbuf); free(hqb); free(gt);
    return 0;
}

/* ---------------------------------------------------------------- prefill grouped GEMM */

/* Prefill expert GEMM on sampled entries [PF, Summary: the weights are dequantized to FP16
 * and the tensor cores get those FP16 values; sorted rows per expert].  For each sampled
 * entry p (a position in the expert-sorted entry list), with expert e (expert_off[e] <= p <
 * expert_off[e+1]) and token t = sorted_tok[p]:
 *   G_i = sum_k Wg16[i][k] X16[t][k],  U_i likewise   (FP16 weights = RNE of exact; double)
 *   H16_i = fp16(silu(float(G_i)) * float(U_i))
 *   Y_j = sum_i Wd16[j][i] H16_i                      (double)
 * Outputs per sample s (any may be NULL): G, U, Gabs, Uabs ([ns][inter], double; abs = sum
 * of |w x|), H16 ([ns][inter] binary16 bits), Y, Yabs ([ns][hidden], double). */
int or_prefill_rows(int wtype_gu, const uint8_t* w_gate, const uint8_t* w_up, int64_t gu_stride,
                    int wtype_down, const uint8_t* w_down, int64_t down_stride, const uint8_t* grid,
                    int nexperts, int64_t hidden, int64_t inter, const uint16_t* x16, int64_t ntok,
                    const int32_t* sorted_tok, const int32_t* expert_off, const int64_t* samples,
                    int64_t ns, double* G, double* U, double* Gabs, double* Uabs, uint16_t* H16,
                    double* Y, double* Yabs) {
    if (!or_row_bytes(wtype_gu, hidden) || !or_row_bytes(wtype_down, inter)) return -1;
    double* wg = (double*)malloc(sizeof(double) * inter * hidden);
    double* wu = (double*)malloc(sizeof(double) * inter * hidden);
    double* wd = (double*)malloc(sizeof(double) * hidden * inter);
    uint16_t* t16 = (uint16_t*)malloc(sizeof(uint16_t) * inter * hidden);
    if (!wg || !wu || !wd || !t16) { free(wg); free(wu); free(wd); free(t16); return -2; }
    int rc = 0;
    for (int e = 0; e < nexperts && rc == 0; ++e) {
        int any = 0;
        for (int64_t s = 0; s < ns; ++s)
            if (samples[s] >= expert_off[e] && samples[s] < expert_off[e + 1]) any = 1;
        if (!any) continue;
        /* FP16 weights of expert e, held as doubles */
        or_dequant_f16(wtype_gu, w_gate + (int64_t)e * gu_stride, grid, inter, hidden, t16, hidden);
        for (int64_t i = 0; i < inter * hidden; ++i) wg[i] = or_f16_to_f32(t16[i]);
        or_dequant_f16(wtype_gu, w_up + (int64_t)e * gu_stride, grid, inter, hidden, t16, hidden);
        for (int64_t i = 0; i < inter * hidden; ++i) wu[i] = or_f16_to_f32(t16[i]);
        or_dequant_f16(wtype_down, w_down + (int64_t)e * down_stride, grid, hidden, inter, t16, inter);
        for (int64_t i = 0; i < hidden * inter; ++i) wd[i] = or_f16_to_f32(t16[i]);
#pragma omp parallel for schedule(dynamic)
        for (int64_t s = 0; s < ns; ++s) {
            int64_t p = samples[s];
            if (p < expert_off[e] || p >= expert_off[e + 1]) continue;
            int32_t t = sorted_tok[p];
            if (t < 0 || t >= ntok) continue;
            const uint16_t* xr = x16 + (int64_t)t * hidden;
            double* hrow = (double*)malloc(sizeof(double) * inter);
            for (int64_t i = 0; i < inter; ++i) {
                double ga = 0, ua = 0, gab = 0, uab = 0;
                for (int64_t kk = 0; kk < hidden; ++kk) {
                    double xv = or_f16_to_f32(xr[kk]);
                    ga += wg[i * hidden + kk] * xv;
                    ua += wu[i * hidden + kk] * xv;
                    gab += fabs(wg[i * hidden + kk] * xv);
                    uab += fabs(wu[i * hidden + kk] * xv);
                }
                uint16_t hb = or_f32_to_f16(or_silu_mul((float)ga, (float)ua));
                hrow[i] = or_f16_to_f32(hb);
                if (G) G[s * inter + i] = ga;
                if (U) U[s * inter + i] = ua;
                if (Gabs) Gabs[s * inter + i] = gab;
                if (Uabs) Uabs[s * inter + i] = uab;
                if (H16) H16[s * inter + i] = hb;
            }
            for (int64_t j = 0; j < hidden; ++j) {
                double ya = 0, yab = 0;
                for (int64_t i = 0; i < inter; ++i) {
                    ya += wd[j * inter + i] * hrow[i];
                    yab += fabs(wd[j * inter + i] * hrow[i]);
                }
                if (Y) Y[s * hidden + j] = ya;
                if (Yabs) Yabs[s * hidden + j] = yab;
            }
            free(hrow);
        }
    }
    free(wg); free(wu); free(wd); free(t16);
    return rc;
}

/* ---------------------------------------------------------------- MoE combine */

/* MoE combine [DQ, Change: the combine sums a token's expert rows in a fixed k order; profile
 * block: moe_combine4 reads the rows at bandwidth].  The pages fix the k order but not the
 * expression; the reading used: out[t][j] = sum over k = 0 .. topk-1 of w[t][k] * y[r][j] with
 * r = row_idx[t][k], starting from +0 and adding in k order, every product and every sum one
 * binary32 rounding (no fused multiply-add); a row index outside [0, nrows) adds nothing.
 *   y: [nrows][hidden]; row_idx, w: [ntok][topk]; out: [ntok][hidden]. */
int or_moe_combine(const float* y, int64_t nrows, int64_t hidden, const int32_t* row_idx,
                   const float* w, int64_t ntok, int topk, float* out) {
    if (hidden < 1 || topk < 1 || ntok < 0) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < ntok; ++t)
        for (int64_t j = 0; j < hidden; ++j) {
            float acc = 0.0f;
            for (int k = 0; k < topk; ++k) {
                int32_t r = row_idx[t * topk + k];
                if (r < 0 || r >= nrows) continue;
                float prod = w[t * topk + k] * y[r * hidden + j];
                acc = acc + prod;
            }
            out[t * hidden + j] = acc;
        }
    return 0;
}

/* ---------------------------------------------------------------- dense prompt projections */

/* Dense projection of prompt tokens on FP16-dequantized weights [DQ, Change: the dense weights
 * dequantized to FP16 for a matrix product over the prompt; PF, Summary: FP16 products, FP32
 * sums].  For each sampled token t: Y[s][r] = sum over k of W16[r][k] * X16[t][k], with W16 the
 * FP16 dequantization (or_dequant_f16), products exact in double, double sums; Yabs the sum of
 * |W16 X16| (the scale of the tolerance).  wtype 0 takes w as binary16 bits [nrows][k] already.
 *   x16: [ntok][k] binary16 bits; samples: token indices; Y, Yabs: [ns][nrows] (either may be
 *   NULL). */
int or_dense_rows(int wtype, const void* w, const uint8_t* grid, int64_t nrows, int64_t k,
                  const uint16_t* x16, int64_t ntok, const int64_t* samples, int64_t ns,
                  double* Y, double* Yabs) {
    if (nrows < 1 || k < 1) return -1;
    if (wtype != 0 && !or_row_bytes(wtype, k)) return -1;
    uint16_t* w16 = (uint16_t*)malloc(sizeof(uint16_t) * nrows * k);
    if (!w16) return -2;
    if (wtype == 0)
        memcpy(w16, w, sizeof(uint16_t) * nrows * k);
    else
        or_dequant_f16(wtype, (const uint8_t*)w, grid, nrows, k, w16, k);
#pragma omp parallel for schedule(dynamic)
    for (int64_t s = 0; s < ns; ++s) {
        int64_t t = samples[s];
        for (int64_t r = 0; r < nrows; ++r) {
            double acc = 0.0, aabs = 0.0;
            if (t >= 0 && t < ntok)
                for (int64_t kk = 0; kk < k; ++kk) {
                    double p = (double)or_f16_to_f32(w16[r * k + kk]) * (double)or_f16_to_f32(x16[t * k + kk]);
                    acc += p;
                    aabs += fabs(p);
                }
            if (Y) Y[s * nrows + r] = acc;
            if (Yabs) Yabs[s * nrows + r] = aabs;
        }
    }
    free(w16);
    return 0;
}

/* ---------------------------------------------------------------- weight planes */

/* Repack of Q8_0 / IQ4_NL rows into planes [GP, What changed: a device-side repack of the
 * GGUF blocks into planes, an int8 plane plus scales, owned by explicit pack / release calls].
 * The pages name the planes but not their layout; the reading used: a row is cut into tiles of
 * 16 consecutive blocks (the last tile of a row may hold fewer, n = the blocks left); a tile is
 * the factor bytes of its n blocks back to back in block order (Q8_0: the 32 int8 q; IQ4_NL: the
 * 16 index bytes), then the n fp16 scales in block order.  A row keeps its size and position,
 * so the planes of a matrix take exactly the bytes of its blocks. */
int or_pack_planes(int wtype, const uint8_t* w, int64_t nrows, int64_t k, uint8_t* out) {
    if (wtype != OR_Q8_0 && wtype != OR_IQ4_NL) return -1;
    int64_t rb = or_row_bytes(wtype, k);
    if (!rb) return -1;
    int64_t nb = k / 32;
    int bb = block_bytes(wtype);      /* 34 or 18 */
    int fb = bb - 2;                  /* factor bytes per block: 32 or 16 */
    for (int64_t r = 0; r < nrows; ++r) {
        const uint8_t* row = w + r * rb;
        uint8_t* dst = out + r * rb;
        for (int64_t b0 = 0; b0 < nb; b0 += 16) {
            int64_t n = nb - b0 < 16 ? nb - b0 : 16;
            uint8_t* tile = dst + b0 * bb;
            for (int64_t i = 0; i < n; ++i) {
                const uint8_t* blk = row + (b0 + i) * bb;
                memcpy(tile + i * fb, blk + 2, (size_t)fb);       /* factors */
                memcpy(tile + n * fb + 2 * i, blk, 2);            /* scale */
            }
        }
    }
    return 0;
}
