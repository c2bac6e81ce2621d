/*
 * mmq_oracle.c -- plain, slow CPU reference for block-quantized int8 MMQ.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header, table or helper
 * with the GPU library.
 *
 * What it computes (the operation the pages define):
 *   "When the Product Won't Collapse: A Negative Result on int8 Tensor-Core
 *    MMQ", section 2 (the displayed contraction): for every output (m, n),
 *      out[m,n] = sum over 32-element k-blocks b of
 *                 (activation scale[m,b] * weight scale[n,b]) *
 *                 (int8 dot of the 32 activation codes with the 32 weight codes)
 *   with the integer dot taken exactly inside one constant-scale block and
 *   the float scale applied once per block boundary (same section).
 *
 *   "When Does a Kernel Win Surface?", section 6.2 (the Q4_K x q8_1 affine
 *   identity): for Q4_K weights the block term is
 *      d1 * xs * dot(q4, xq)  -  m1 * xsum
 *   with d1 = d*sc and m1 = dmin*m of the weight sub-block, xs the activation
 *   block scale and xsum the activation block sum carried by q8_1.
 *
 *   "13 . r7-r8 raw-byte MMQ kernel", section 3.2 (quantize pass): the
 *   activation is quantized per 32-element chunk from its absolute maximum,
 *   by multiplying with an inverse scale and rounding to an integer code,
 *   with an integer sum of the codes kept beside it; section 3.1 notes that
 *   the absolute maximum is exact in any association order.
 *
 * Precision: fp32 everywhere the pages use fp32 (scales, products, the
 * per-block accumulation); fp16 only for the stored scale fields.  Build
 * with -O2 -ffp-contract=off and no fast-math so that every operation below
 * is exactly one IEEE fp32 operation; fmaf() is written where a fused
 * multiply-add is meant.
 *
 * Readings where the pages are silent (each is listed with its reason in
 * the design notes of the repository):
 *   R1  rounding of x*id: half away from zero (roundf), not ties-to-even.
 *   R2  the code is x * (1/d) with 1/d the correctly rounded fp32 reciprocal.
 *   R3  the fp32 d = amax/127 quantizes; fp16 is only the stored copy.
 *   R4  the q8_1 sum field is fp16(d * (float)sum of codes).
 *   R5  codes clamp to [-127, 127] (never binds for finite input).
 *   R6  amax == 0 gives d = id = 0, all codes 0, sum field +0; so does a
 *       block whose fp32 reciprocal 1/d overflows to infinity (amax below
 *       about 3.7e-37, where fp16(d) is 0 as well): id = 0, codes 0.
 *   R7  non-finite input is rejected (the function returns an error).
 *   R8  byte layouts (little-endian):
 *         q8_1 block (36 B): [0,2) fp16 d, [2,4) fp16 s, [4,36) int8 codes
 *         Q8_0 block (34 B): [0,2) fp16 d, [2,34) int8 codes
 *         Q4_K super-block (144 B, 256 values): [0,2) fp16 d, [2,4) fp16
 *           dmin, [4,16) packed 6-bit scales/mins, [16,144) 4-bit codes
 *   R9  Q4_K 6-bit packing and nibble order: the GGUF K-quant packing (see
 *       q4k_scale_min below); element e of a super-block lives in byte
 *       32*(e/64) + (e%32) of the code area, low nibble when (e%64) < 32.
 *   R21 Q5_K (a format the pages name in their list of K-quants without a
 *       layout; the GGUF K-quant layout is taken): super-block (176 B, 256
 *       values): [0,2) fp16 d, [2,4) fp16 dmin, [4,16) the Q4_K 6-bit
 *       scale/min packing, [16,48) high bits, [48,176) low nibbles in the
 *       Q4_K order; the 5-bit code of element e is its nibble plus 16 times
 *       bit e/32 of high-bit byte e%32.  Its block term is the Q4_K affine
 *       identity with 5-bit codes (0..31), computed as in R10-R11.
 *   R22 Q6_K (a format the pages name among the K-quants; "When Does a
 *       Kernel Win Surface?", section 4.1, reads its 16-element scale
 *       groups and centres its 6-bit codes at 32; the GGUF layout is taken):
 *       super-block (210 B, 256 values): [0,128) low four bits, [128,192)
 *       high two bits, [192,208) int8 scales, [208,210) fp16 d.  Element e
 *       (half h = e/128, quarter q = (e%128)/32, l = e%32) takes nibble q/2
 *       (low nibble when q < 2) of byte 64h + 32(q%2) + l and bits 2q, 2q+1
 *       of byte 128 + 32h + l; its 6-bit code c is low | high << 4, its
 *       signed weight code c - 32, its scale the int8 byte 192 + e/16.
 *   R23 Q6_K term per 16-element scale group g (two per 32-block, in
 *       ascending order): I_g = exact dot of the 16 activation codes with
 *       the codes c - 32, t = (d * sc_g) * (float)I_g (d * sc_g exact, one
 *       rounding), acc = fmaf(activation_scale of the block, t, acc).
 *   R10 per block: t = weight_scale * (float)I (one rounding), then
 *       acc = fmaf(activation_scale, t, acc).
 *   R11 the Q4_K min term is acc = fmaf(-(dmin*m), f32(s16), acc), using
 *       the stored fp16 sum field.
 *   R12 blocks are accumulated in ascending order from acc = 0.
 *   R13 the output is overwritten, not accumulated into.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define QK 32            /* values per block                */
#define QK_K 256         /* values per Q4_K super-block     */
#define Q8_1_BYTES 36
#define Q8_0_BYTES 34
#define Q4_K_BYTES 144
#define Q5_K_BYTES 176
#define Q6_K_BYTES 210
#define QG 16            /* values per Q6_K scale group     */

/* ------------------------------------------------------------------ */
/* IEEE binary16 <-> binary32, written from the format definition.      */
/* ------------------------------------------------------------------ */

/* Exact widening of an IEEE half to single precision (subnormals kept). */
float oracle_f16_to_f32(uint16_t h)
{
    uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
    uint32_t e = (h >> 10) & 0x1fu;
    uint32_t m = h & 0x3ffu;
    uint32_t bits;
    if (e == 0) {
        if (m == 0) {
            bits = sign;
        } else {
            /* value = m * 2^-24; normalise so the leading one is bit 10 */
            int sh = 0;
            while ((m & 0x400u) == 0) {
                m <<= 1;
                sh++;
            }
            m &= 0x3ffu;
            bits = sign | ((uint32_t)(113 - sh) << 23) | (m << 13);
        }
    } else if (e == 31) {
        bits = sign | 0x7f800000u | (m << 13);
    } else {
        bits = sign | ((e - 15 + 127) << 23) | (m << 13);
    }
    float f;
    memcpy(&f, &bits, 4);
    return f;
}

/* Round-to-nearest-even narrowing of a single to an IEEE half, with
 * gradual underflow and overflow to infinity. NaN stays a quiet NaN. */
uint16_t oracle_f32_to_f16(float f)
{
    uint32_t x;
    memcpy(&x, &f, 4);
    uint16_t sign = (uint16_t)((x >> 16) & 0x8000u);
    uint32_t exp = (x >> 23) & 0xffu;
    uint32_t man = x & 0x7fffffu;

    if (exp == 0xffu) {
        if (man != 0)
            return (uint16_t)(sign | 0x7e00u | (man >> 13));
        return (uint16_t)(sign | 0x7c00u);
    }
    if (exp == 0)           /* zero or fp32 subnormal: far below half's range */
        return sign;

    int E = (int)exp - 127;              /* unbiased exponent */
    if (E > 15)
        return (uint16_t)(sign | 0x7c00u);

    if (E >= -14) {                      /* half-normal candidate */
        uint32_t m = man >> 13;
        uint32_t rem = man & 0x1fffu;
        if (rem > 0x1000u || (rem == 0x1000u && (m & 1u)))
            m++;
        int he = E + 15;
        if (m == 0x400u) {               /* mantissa overflowed */
            m = 0;
            he++;
        }
        if (he >= 31)
            return (uint16_t)(sign | 0x7c00u);
        return (uint16_t)(sign | ((uint32_t)he << 10) | m);
    }

    /* half-subnormal: value = full * 2^(E-23), unit of result = 2^-24 */
    int s = -E - 1;                      /* right shift of the 24-bit significand */
    if (s > 25)
        return sign;
    uint64_t full = 0x800000u | man;
    uint64_t m = full >> s;
    uint64_t rem = full & ((1ull << s) - 1ull);
    uint64_t half = 1ull << (s - 1);
    if (rem > half || (rem == half && (m & 1ull)))
        m++;
    return (uint16_t)(sign | (uint16_t)m);   /* m == 0x400 is the smallest normal */
}

/* Bulk forms, used only by the tests that compare against a library. */
void oracle_f32_to_f16_array(const float *in, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = oracle_f32_to_f16(in[i]);
}

void oracle_f16_to_f32_array(const uint16_t *in, float *out, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = oracle_f16_to_f32(in[i]);
}

static uint16_t rd16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static void wr16(uint8_t *p, uint16_t v)
{
    p[0] = (uint8_t)(v & 0xffu);
    p[1] = (uint8_t)(v >> 8);
}

/* ------------------------------------------------------------------ */
/* Activation quantization fp32 -> q8_1 (one 32-value block at a time). */
/* ------------------------------------------------------------------ */

/* Quantize one block of 32 floats into the 36-byte q8_1 layout.
 * Returns 0 on success, -1 when a value is not finite (reading R7). */
int oracle_quantize_block_q8_1(const float *x, uint8_t *y)
{
    float amax = 0.0f;
    for (int i = 0; i < QK; i++) {
        if (!isfinite(x[i]))
            return -1;
        float a = fabsf(x[i]);
        if (a > amax)
            amax = a;
    }
    float d = amax / 127.0f;                        /* R3 */
    float id = (d != 0.0f) ? 1.0f / d : 0.0f;        /* R2, R6 */
    if (isinf(id))                                   /* R6: 1/d overflows fp32 */
        id = 0.0f;
    int32_t sum = 0;
    for (int i = 0; i < QK; i++) {
        float v = x[i] * id;
        float r = roundf(v);                         /* R1: half away from zero */
        int32_t q = (int32_t)r;
        if (q > 127) q = 127;                        /* R5 */
        if (q < -127) q = -127;
        y[4 + i] = (uint8_t)(int8_t)q;
        sum += q;
    }
    wr16(y + 0, oracle_f32_to_f16(d));
    wr16(y + 2, oracle_f32_to_f16(d * (float)sum)); /* R4 */
    return 0;
}

/* x: M x K fp32 row-major; y: M x (K/32) blocks of 36 bytes. K % 32 == 0.
 * Returns 0, or -1 on non-finite input, or -2 on a bad shape. */
int oracle_quantize_q8_1(const float *x, uint8_t *y, int64_t M, int64_t K)
{
    if (M < 0 || K < 0 || K % QK != 0)
        return -2;
    int64_t kb = K / QK;
    for (int64_t m = 0; m < M; m++)
        for (int64_t b = 0; b < kb; b++)
            if (oracle_quantize_block_q8_1(x + m * K + b * QK,
                                           y + (m * kb + b) * Q8_1_BYTES) != 0)
                return -1;
    return 0;
}

/* ------------------------------------------------------------------ */
/* Q4_K sub-block scales and mins (reading R9).                         */
/* ------------------------------------------------------------------ */

/* Sub-block j in 0..7 of a super-block: 6-bit scale and 6-bit min from the
 * 12 packed bytes.  Sub-blocks 0..3 keep their values in the low six bits
 * of bytes j (scale) and j+4 (min); sub-blocks 4..7 take their low four
 * bits from byte j+4 (scale: low nibble, min: high nibble) and their top
 * two bits from the spare top bits of bytes j-4 (scale) and j (min). */
void oracle_q4k_scale_min(const uint8_t *s12, int j, uint8_t *sc, uint8_t *mn)
{
    if (j < 4) {
        *sc = s12[j] & 63u;
        *mn = s12[j + 4] & 63u;
    } else {
        *sc = (uint8_t)((s12[j + 4] & 0x0fu) | ((s12[j - 4] >> 6) << 4));
        *mn = (uint8_t)((s12[j + 4] >> 4) | ((s12[j] >> 6) << 4));
    }
}

/* Inverse of oracle_q4k_scale_min over all eight sub-blocks. Values must be
 * in 0..63; returns -1 otherwise. */
int oracle_q4k_pack_scale_min(const uint8_t sc[8], const uint8_t mn[8], uint8_t *s12)
{
    for (int j = 0; j < 8; j++)
        if (sc[j] > 63u || mn[j] > 63u)
            return -1;
    memset(s12, 0, 12);
    for (int j = 0; j < 4; j++) {
        s12[j] = (uint8_t)(sc[j] | ((sc[j + 4] >> 4) << 6));
        s12[j + 4] = (uint8_t)(mn[j] | ((mn[j + 4] >> 4) << 6));
        s12[j + 8] = (uint8_t)((sc[j + 4] & 0x0fu) | ((mn[j + 4] & 0x0fu) << 4));
    }
    return 0;
}

/* 4-bit code of element e (0..255) of a super-block's 128-byte code area. */
static int q4k_code(const uint8_t *qs, int e)
{
    int g = e / 64, r = e % 64;
    uint8_t byte = qs[32 * g + (r % 32)];
    return (r < 32) ? (byte & 0x0f) : (byte >> 4);
}

/* Public forms for the layout tests. */
int oracle_q4k_code(const uint8_t *superblock, int e) { return q4k_code(superblock + 16, e); }

/* 5-bit code of element e (0..255) of a Q5_K super-block (reading R21). */
static int q5k_code(const uint8_t *blk, int e)
{
    int lo = q4k_code(blk + 48, e);
    int hi = (blk[16 + (e % 32)] >> (e / 32)) & 1;
    return lo | (hi << 4);
}

int oracle_q5k_code(const uint8_t *superblock, int e) { return q5k_code(superblock, e); }

/* 6-bit code (0..63) of element e (0..255) of a Q6_K super-block (R22). */
static int q6k_code(const uint8_t *blk, int e)
{
    int h = e / 128, q = (e % 128) / 32, l = e % 32;
    uint8_t lb = blk[64 * h + 32 * (q % 2) + l];
    int lo = (q < 2) ? (lb & 0x0f) : (lb >> 4);
    int hi = (blk[128 + 32 * h + l] >> (2 * q)) & 3;
    return lo | (hi << 4);
}

/* Scale (int8) of 16-element group g (0..15) of a Q6_K super-block. */
static int q6k_scale(const uint8_t *blk, int g) { return (int)(int8_t)blk[192 + g]; }

int oracle_q6k_code(const uint8_t *superblock, int e) { return q6k_code(superblock, e); }
int oracle_q6k_scale(const uint8_t *superblock, int g) { return q6k_scale(superblock, g); }

/* Dequantize one Q6_K super-block into 256 fp32 values (w = d*sc*(c-32)). */
void oracle_dequant_q6_K_block(const uint8_t *blk, float *w)
{
    float d = oracle_f16_to_f32(rd16(blk + 208));
    for (int e = 0; e < QK_K; e++)
        w[e] = (d * (float)q6k_scale(blk, e / QG)) * (float)(q6k_code(blk, e) - 32);
}

/* Dequantize one Q4_K super-block into 256 fp32 values (w = d*sc*q - dmin*m). */
void oracle_dequant_q4_K_block(const uint8_t *blk, float *w)
{
    float d = oracle_f16_to_f32(rd16(blk));
    float dmin = oracle_f16_to_f32(rd16(blk + 2));
    for (int j = 0; j < 8; j++) {
        uint8_t sc, mn;
        oracle_q4k_scale_min(blk + 4, j, &sc, &mn);
        float ds = d * (float)sc;
        float dm = dmin * (float)mn;
        for (int i = 0; i < QK; i++) {
            int e = QK * j + i;
            w[e] = ds * (float)q4k_code(blk + 16, e) - dm;
        }
    }
}

/* ------------------------------------------------------------------ */
/* Integer block dots (exact).                                          */
/* ------------------------------------------------------------------ */

static int32_t dot_q8_q8(const int8_t *a, const int8_t *b)
{
    int32_t s = 0;
    for (int i = 0; i < QK; i++)
        s += (int32_t)a[i] * (int32_t)b[i];
    return s;
}

/* dots[(m*N + n)*kb + b] = sum_i xq[m, 32b+i] * wq[n, 32b+i]  (Q8_0 weights) */
int oracle_block_dots_q8_0(const uint8_t *x, const uint8_t *w, int32_t *dots,
                           int64_t M, int64_t N, int64_t K)
{
    if (M < 0 || N < 0 || K < 0 || K % QK != 0)
        return -2;
    int64_t kb = K / QK;
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++)
            for (int64_t b = 0; b < kb; b++) {
                const int8_t *xq = (const int8_t *)(x + (m * kb + b) * Q8_1_BYTES + 4);
                const int8_t *wq = (const int8_t *)(w + (n * kb + b) * Q8_0_BYTES + 2);
                dots[(m * N + n) * kb + b] = dot_q8_q8(xq, wq);
            }
    return 0;
}

/* Same for Q4_K weights: the 4-bit codes (0..15) of sub-block b%8 of
 * super-block b/8 against the activation codes. K % 256 == 0. */
int oracle_block_dots_q4_K(const uint8_t *x, const uint8_t *w, int32_t *dots,
                           int64_t M, int64_t N, int64_t K)
{
    if (M < 0 || N < 0 || K < 0 || K % QK_K != 0)
        return -2;
    int64_t kb = K / QK, nsb = K / QK_K;
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++)
            for (int64_t b = 0; b < kb; b++) {
                const int8_t *xq = (const int8_t *)(x + (m * kb + b) * Q8_1_BYTES + 4);
                const uint8_t *blk = w + (n * nsb + b / 8) * Q4_K_BYTES;
                int32_t s = 0;
                for (int i = 0; i < QK; i++)
                    s += (int32_t)xq[i] * q4k_code(blk + 16, (int)(b % 8) * QK + i);
                dots[(m * N + n) * kb + b] = s;
            }
    return 0;
}

/* Same for Q5_K weights: the 5-bit codes (0..31) of sub-block b%8. */
int oracle_block_dots_q5_K(const uint8_t *x, const uint8_t *w, int32_t *dots,
                           int64_t M, int64_t N, int64_t K)
{
    if (M < 0 || N < 0 || K < 0 || K % QK_K != 0)
        return -2;
    int64_t kb = K / QK, nsb = K / QK_K;
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++)
            for (int64_t b = 0; b < kb; b++) {
                const int8_t *xq = (const int8_t *)(x + (m * kb + b) * Q8_1_BYTES + 4);
                const uint8_t *blk = w + (n * nsb + b / 8) * Q5_K_BYTES;
                int32_t s = 0;
                for (int i = 0; i < QK; i++)
                    s += (int32_t)xq[i] * q5k_code(blk, (int)(b % 8) * QK + i);
                dots[(m * N + n) * kb + b] = s;
            }
    return 0;
}

/* Q6_K: one dot per 16-element scale group (R23), the codes centred:
 * dots[(m*N + n)*(K/16) + g] = sum_i xq[m, 16g+i] * (c[n, 16g+i] - 32). */
int oracle_group_dots_q6_K(const uint8_t *x, const uint8_t *w, int32_t *dots,
                           int64_t M, int64_t N, int64_t K)
{
    if (M < 0 || N < 0 || K < 0 || K % QK_K != 0)
        return -2;
    int64_t kb = K / QK, nsb = K / QK_K, ng = K / QG;
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++)
            for (int64_t g = 0; g < ng; g++) {
                const int8_t *xq = (const int8_t *)(x + (m * kb + g / 2) * Q8_1_BYTES + 4) + QG * (g % 2);
                const uint8_t *blk = w + (n * nsb + g / 16) * Q6_K_BYTES;
                int32_t s = 0;
                for (int i = 0; i < QG; i++)
                    s += (int32_t)xq[i] * (q6k_code(blk, (int)(g % 16) * QG + i) - 32);
                dots[(m * N + n) * ng + g] = s;
            }
    return 0;
}

/* ------------------------------------------------------------------ */
/* The contractions, fp32 per-block accumulation (R10-R13).             */
/* ------------------------------------------------------------------ */

static int set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
    return omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

/* x: M x kb q8_1 blocks; w: N x kb Q8_0 blocks; out: M x N fp32 row-major.
 * Rows m0 <= m < m1 only (the whole matrix when m0 = 0, m1 = M), so that a
 * bounded row sample can be timed.  Returns the thread count used, or a
 * negative code on a bad shape. */
int oracle_gemm_q8_0_rows(const uint8_t *x, const uint8_t *w, float *out,
                          int64_t M, int64_t N, int64_t K, int64_t m0, int64_t m1,
                          int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || K % QK != 0 || m0 < 0 || m1 > M || m0 > m1)
        return -2;
    int used = set_threads(nthreads);
    int64_t kb = K / QK;
#pragma omp parallel for schedule(static)
    for (int64_t m = m0; m < m1; m++) {
        for (int64_t n = 0; n < N; n++) {
            float acc = 0.0f;
            for (int64_t b = 0; b < kb; b++) {
                const uint8_t *xb = x + (m * kb + b) * Q8_1_BYTES;
                const uint8_t *wb = w + (n * kb + b) * Q8_0_BYTES;
                int32_t I = dot_q8_q8((const int8_t *)(xb + 4), (const int8_t *)(wb + 2));
                float xd = oracle_f16_to_f32(rd16(xb));
                float wd = oracle_f16_to_f32(rd16(wb));
                float t = wd * (float)I;
                acc = fmaf(xd, t, acc);
            }
            out[m * N + n] = acc;
        }
    }
    return used;
}

int oracle_gemm_q8_0(const uint8_t *x, const uint8_t *w, float *out,
                     int64_t M, int64_t N, int64_t K, int nthreads)
{
    return oracle_gemm_q8_0_rows(x, w, out, M, N, K, 0, M, nthreads);
}

/* x: M x kb q8_1 blocks; w: N x (K/256) Q4_K super-blocks; out: M x N fp32. */
int oracle_gemm_q4_K_rows(const uint8_t *x, const uint8_t *w, float *out,
                          int64_t M, int64_t N, int64_t K, int64_t m0, int64_t m1,
                          int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || K % QK_K != 0 || m0 < 0 || m1 > M || m0 > m1)
        return -2;
    int used = set_threads(nthreads);
    int64_t kb = K / QK, nsb = K / QK_K;
#pragma omp parallel for schedule(static)
    for (int64_t m = m0; m < m1; m++) {
        for (int64_t n = 0; n < N; n++) {
            float acc = 0.0f;
            for (int64_t sb = 0; sb < nsb; sb++) {
                const uint8_t *blk = w + (n * nsb + sb) * Q4_K_BYTES;
                float d = oracle_f16_to_f32(rd16(blk));
                float dmin = oracle_f16_to_f32(rd16(blk + 2));
                for (int j = 0; j < 8; j++) {
                    int64_t b = sb * 8 + j;
                    const uint8_t *xb = x + (m * kb + b) * Q8_1_BYTES;
                    const int8_t *xq = (const int8_t *)(xb + 4);
                    uint8_t sc, mn;
                    oracle_q4k_scale_min(blk + 4, j, &sc, &mn);
                    int32_t I = 0;
                    for (int i = 0; i < QK; i++)
                        I += (int32_t)xq[i] * q4k_code(blk + 16, j * QK + i);
                    float ds = d * (float)sc;       /* exact: 11 x 6 bits */
                    float dm = dmin * (float)mn;    /* exact */
                    float xd = oracle_f16_to_f32(rd16(xb));
                    float xs = oracle_f16_to_f32(rd16(xb + 2));
                    float t = ds * (float)I;
                    acc = fmaf(xd, t, acc);
                    acc = fmaf(-dm, xs, acc);
                }
            }
            out[m * N + n] = acc;
        }
    }
    return used;
}

int oracle_gemm_q4_K(const uint8_t *x, const uint8_t *w, float *out,
                     int64_t M, int64_t N, int64_t K, int nthreads)
{
    return oracle_gemm_q4_K_rows(x, w, out, M, N, K, 0, M, nthreads);
}

/* x: M x kb q8_1 blocks; w: N x (K/256) Q5_K super-blocks; out: M x N fp32.
 * The Q4_K contraction above with 5-bit codes (reading R21). */
int oracle_gemm_q5_K_rows(const uint8_t *x, const uint8_t *w, float *out,
                          int64_t M, int64_t N, int64_t K, int64_t m0, int64_t m1,
                          int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || K % QK_K != 0 || m0 < 0 || m1 > M || m0 > m1)
        return -2;
    int used = set_threads(nthreads);
    int64_t kb = K / QK, nsb = K / QK_K;
#pragma omp parallel for schedule(static)
    for (int64_t m = m0; m < m1; m++) {
        for (int64_t n = 0; n < N; n++) {
            float acc = 0.0f;
            for (int64_t sb = 0; sb < nsb; sb++) {
                const uint8_t *blk = w + (n * nsb + sb) * Q5_K_BYTES;
                float d = oracle_f16_to_f32(rd16(blk));
                float dmin = oracle_f16_to_f32(rd16(blk + 2));
                for (int j = 0; j < 8; j++) {
                    int64_t b = sb * 8 + j;
                    const uint8_t *xb = x + (m * kb + b) * Q8_1_BYTES;
                    const int8_t *xq = (const int8_t *)(xb + 4);
                    uint8_t sc, mn;
                    oracle_q4k_scale_min(blk + 4, j, &sc, &mn);
                    int32_t I = 0;
                    for (int i = 0; i < QK; i++)
                        I += (int32_t)xq[i] * q5k_code(blk, j * QK + i);
                    float ds = d * (float)sc;       /* exact: 11 x 6 bits */
                    float dm = dmin * (float)mn;    /* exact */
                    float xd = oracle_f16_to_f32(rd16(xb));
                    float xs = oracle_f16_to_f32(rd16(xb + 2));
                    float t = ds * (float)I;
                    acc = fmaf(xd, t, acc);
                    acc = fmaf(-dm, xs, acc);
                }
            }
            out[m * N + n] = acc;
        }
    }
    return used;
}

int oracle_gemm_q5_K(const uint8_t *x, const uint8_t *w, float *out,
                     int64_t M, int64_t N, int64_t K, int nthreads)
{
    return oracle_gemm_q5_K_rows(x, w, out, M, N, K, 0, M, nthreads);
}

/* x: M x kb q8_1 blocks; w: N x (K/256) Q6_K super-blocks; out: M x N fp32.
 * Per 32-block, its two 16-element scale groups in order (R22-R23). */
int oracle_gemm_q6_K_rows(const uint8_t *x, const uint8_t *w, float *out,
                          int64_t M, int64_t N, int64_t K, int64_t m0, int64_t m1,
                          int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || K % QK_K != 0 || m0 < 0 || m1 > M || m0 > m1)
        return -2;
    int used = set_threads(nthreads);
    int64_t kb = K / QK, nsb = K / QK_K;
#pragma omp parallel for schedule(static)
    for (int64_t m = m0; m < m1; m++) {
        for (int64_t n = 0; n < N; n++) {
            float acc = 0.0f;
            for (int64_t sb = 0; sb < nsb; sb++) {
                const uint8_t *blk = w + (n * nsb + sb) * Q6_K_BYTES;
                float d = oracle_f16_to_f32(rd16(blk + 208));
                for (int j = 0; j < 8; j++) {
                    const uint8_t *xb = x + (m * kb + sb * 8 + j) * Q8_1_BYTES;
                    const int8_t *xq = (const int8_t *)(xb + 4);
                    float xd = oracle_f16_to_f32(rd16(xb));
                    for (int h = 0; h < 2; h++) {
                        int g = 2 * j + h;
                        int32_t I = 0;
                        for (int i = 0; i < QG; i++)
                            I += (int32_t)xq[QG * h + i] * (q6k_code(blk, g * QG + i) - 32);
                        float ws = d * (float)q6k_scale(blk, g);   /* exact: 11 x 8 bits */
                        float t = ws * (float)I;
                        acc = fmaf(xd, t, acc);
                    }
                }
            }
            out[m * N + n] = acc;
        }
    }
    return used;
}

int oracle_gemm_q6_K(const uint8_t *x, const uint8_t *w, float *out,
                     int64_t M, int64_t N, int64_t K, int nthreads)
{
    return oracle_gemm_q6_K_rows(x, w, out, M, N, K, 0, M, nthreads);
}

/* Indexed MoE ("When Does a Kernel Win Surface?", section 4.5, the fused
 * indexed-MoE prefill GEMM): routed row r = t*topk + j of out is token t's q8_1 row
 * times the weights of expert ids[r], i.e. the dense GEMM row above with
 * that expert's N x K matrix; experts are stored one after another.
 * fmt 0 = Q8_0, 1 = Q4_K, 2 = Q5_K, 3 = Q6_K.  Rows [r0, r1) of out (T*topk x N) are
 * written.
 * Returns the thread count used, -2 on a bad shape, -3 on an expert id out
 * of range. */
int oracle_moe_gemm(int fmt, const uint8_t *x, const uint8_t *w, const int32_t *ids, int topk,
                    float *out, int64_t T, int64_t N, int64_t K, int n_experts,
                    int64_t r0, int64_t r1, int nthreads)
{
    if (fmt < 0 || fmt > 3 || topk < 1 || n_experts < 1 || T < 0 || N < 0 || K < 0 ||
        K % (fmt == 0 ? QK : QK_K) != 0 || r0 < 0 || r1 > T * topk || r0 > r1)
        return -2;
    for (int64_t r = r0; r < r1; r++)
        if (ids[r] < 0 || ids[r] >= n_experts) return -3;
    const int64_t kb = K / QK;
    const int64_t wrow = fmt == 0 ? kb * Q8_0_BYTES
                       : (K / QK_K) * (fmt == 1 ? Q4_K_BYTES : fmt == 2 ? Q5_K_BYTES : Q6_K_BYTES);
    int used = set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t r = r0; r < r1; r++) {
        const uint8_t *xr = x + (r / topk) * kb * Q8_1_BYTES;
        const uint8_t *we = w + (int64_t)ids[r] * N * wrow;
        if (fmt == 0)
            oracle_gemm_q8_0_rows(xr, we, out + r * N, 1, N, K, 0, 1, 1);
        else if (fmt == 1)
            oracle_gemm_q4_K_rows(xr, we, out + r * N, 1, N, K, 0, 1, 1);
        else if (fmt == 2)
            oracle_gemm_q5_K_rows(xr, we, out + r * N, 1, N, K, 0, 1, 1);
        else
            oracle_gemm_q6_K_rows(xr, we, out + r * N, 1, N, K, 0, 1, 1);
    }
    return used;
}

