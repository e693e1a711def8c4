/*
 * orc.c -- the CPU oracle for FP8/FP4 tensor quantization.
 *
 * TEST INFRASTRUCTURE. This file defines, plainly and slowly, what each
 * quantization recipe computes, so that the GPU library can be checked
 * against it byte for byte. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load it. It shares no code, header or
 * table with the GPU library, and the GPU library never calls it.
 *
 * Sources (three web pages on FP8/FP4 training; cited by short label):
 *   [MP]  "混合精度训练：fp16 到 fp8" (garden.houmin.site, infra/mixed-precision-fp8)
 *   [CS]  "FP8 Current Scaling：量化、缩放与精度边界" (notes.kuangjux.top)
 *   [LP]  "从 BF16 到 FP8/FP4：大语言模型低精度训练与混合精度预训练" (r00kie-liu.github.io)
 *
 * Arithmetic: IEEE binary32 with round-to-nearest-even, as the pages fix a
 * single fp32 scale per unit ([CS] section "Current Scaling"). Build with
 * -ffp-contract=off and no fast-math, so that every product is rounded once
 * and divisions are correctly rounded. Value tables and the nearest-code
 * search use binary64, where every value involved is exact.
 *
 * Readings of the pages where they leave a step open are marked READING.
 *
 * Parity status per function is listed in the header of oracle/__init__.py.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_E4M3 0
#define ORC_E5M2 1
#define ORC_E2M1 2

#define ORC_IN_F32 0
#define ORC_IN_BF16 1

#define ORC_ROWWISE 1
#define ORC_COLWISE 2

/* ------------------------------------------------------------------ */
/* Element formats                                                     */
/* ------------------------------------------------------------------ */

/*
 * Bit layout of each element format: sign bit, then exponent bits, then
 * mantissa bits, with an exponent bias.
 *   E4M3: 1/4/3, bias 7.  No infinity; S.1111.111 is NaN.  ([MP] section
 *         "FP8 数据格式"; [CS] table of the two formats: max 448.)
 *   E5M2: 1/5/2, bias 15. IEEE-like: exponent all ones is Inf (mantissa 0)
 *         or NaN.  ([MP] "FP8 数据格式"; [CS] table: max 57344.)
 *   E2M1: 1/2/1, bias 1, four bits, every code finite.  ([MP] section
 *         "NVFP4", the float4_e2m1fn_x2 nibble layout and its list of 16
 *         values.)
 * Biases are those of the OCP 8-bit and MX formats the pages refer to.
 */
typedef struct {
    int bits, ebits, mbits, bias;
} orc_fmt_def;

static const orc_fmt_def FMT[3] = {
    {8, 4, 3, 7},  /* E4M3 */
    {8, 5, 2, 15}, /* E5M2 */
    {4, 2, 1, 1},  /* E2M1 */
};

/* Largest positive finite code of each format. */
unsigned orc_max_code(int fmt)
{
    switch (fmt) {
    case ORC_E4M3: return 0x7E; /* 0x7F is NaN */
    case ORC_E5M2: return 0x7B; /* 0x7C is +Inf */
    case ORC_E2M1: return 0x7;
    }
    return 0;
}

/* Value of an element code, from sign, exponent and mantissa fields. */
double orc_decode(int fmt, unsigned code)
{
    const orc_fmt_def *f = &FMT[fmt];
    unsigned sign = (code >> (f->bits - 1)) & 1u;
    unsigned e = (code >> f->mbits) & ((1u << f->ebits) - 1u);
    unsigned m = code & ((1u << f->mbits) - 1u);
    unsigned eall = (1u << f->ebits) - 1u;
    double v;
    if (fmt == ORC_E4M3 && e == eall && m == (1u << f->mbits) - 1u)
        return NAN;
    if (fmt == ORC_E5M2 && e == eall) {
        if (m != 0)
            return NAN;
        v = INFINITY;
    } else if (e == 0) {
        /* subnormal: 0.m x 2^(1-bias) */
        v = ldexp((double)m, 1 - f->bias - f->mbits);
    } else {
        /* normal: 1.m x 2^(e-bias) */
        v = ldexp((double)((1u << f->mbits) + m), (int)e - f->bias - f->mbits);
    }
    return sign ? -v : v;
}

/* Largest finite magnitude of a format (448, 57344, 6). */
float orc_fmax(int fmt) { return (float)orc_decode(fmt, orc_max_code(fmt)); }

/*
 * E8M0: an unsigned, exponent-only byte; code c stands for 2^(c-127), the
 * same field as an fp32 exponent; 0xFF is NaN.  ([MP] section "MXFP8", the
 * float8_e8m0fnu description.)
 */
double orc_decode_e8m0(unsigned code)
{
    if (code == 0xFF)
        return NAN;
    return ldexp(1.0, (int)code - 127);
}

/* Table of the positive finite values of each format, built on first use
 * from orc_decode; ascending in the code. */
static double g_tab[3][128];
static int g_tab_ready[3];

static const double *value_table(int fmt)
{
    if (!g_tab_ready[fmt]) {
        unsigned c;
        for (c = 0; c <= orc_max_code(fmt); c++)
            g_tab[fmt][c] = orc_decode(fmt, c);
        g_tab_ready[fmt] = 1;
    }
    return g_tab[fmt];
}

/*
 * Q_F(y): round the finite fp32 value y to format F, to nearest, ties to the
 * code whose last mantissa bit is 0 (round-to-nearest-even, [CS] section
 * "Current Scaling"; [MP] section "NVFP4" gives RTNE as the FP4 default).
 * READING (saturation): a magnitude at or above the largest finite value
 * gives that value, never NaN or Inf.  The sign of y is kept, also when the
 * result is zero.
 */
unsigned orc_encode(int fmt, float y)
{
    const double *v = value_table(fmt);
    unsigned top = orc_max_code(fmt);
    unsigned sign = signbit(y) ? (1u << (FMT[fmt].bits - 1)) : 0u;
    double a = fabs((double)y);
    unsigned k;
    if (a >= v[top]) {
        k = top;
    } else {
        /* find lo with v[lo] <= a < v[lo+1] */
        unsigned lo = 0, hi = top;
        while (hi - lo > 1) {
            unsigned mid = (lo + hi) / 2;
            if (v[mid] <= a)
                lo = mid;
            else
                hi = mid;
        }
        double half = 0.5 * (v[lo] + v[hi]); /* exact: both are short dyadics */
        if (a < half)
            k = lo;
        else if (a > half)
            k = hi;
        else
            k = (lo & 1u) ? hi : lo; /* tie: the even code */
    }
    return sign | k;
}

/* orc_encode over an array of n fp32 values. */
void orc_encode_array(int fmt, const float *y, int64_t n, uint8_t *q)
{
    int64_t i;
    for (i = 0; i < n; i++)
        q[i] = (uint8_t)orc_encode(fmt, y[i]);
}

/* ------------------------------------------------------------------ */
/* Inputs                                                              */
/* ------------------------------------------------------------------ */

/* Element i of the input as fp32; bf16 widens exactly (its bits are the top
 * half of the fp32 bits). */
static float load_x(const void *x, int dt, int64_t i)
{
    if (dt == ORC_IN_F32)
        return ((const float *)x)[i];
    uint32_t b = (uint32_t)((const uint16_t *)x)[i] << 16;
    float f;
    memcpy(&f, &b, 4);
    return f;
}

/* Inputs must be finite ([CS] section "Current Scaling" states the formula
 * for finite tensors).  Returns 0 if all are finite. */
static int check_finite(const void *x, int dt, int64_t n)
{
    int64_t i;
    for (i = 0; i < n; i++)
        if (!isfinite(load_x(x, dt, i)))
            return -1;
    return 0;
}

/* Transpose of a row-major [R,C] input into a row-major [C,R] copy of the
 * same element type. */
static void *transpose_input(const void *x, int dt, int64_t R, int64_t C)
{
    size_t es = dt == ORC_IN_F32 ? 4 : 2;
    char *t = (char *)malloc((size_t)(R * C) * es);
    int64_t r, c;
    if (!t)
        return NULL;
    for (r = 0; r < R; r++)
        for (c = 0; c < C; c++)
            memcpy(t + (size_t)(c * R + r) * es, (const char *)x + (size_t)(r * C + c) * es, es);
    return t;
}

/* Byte transpose [R,C] -> [C,R]. */
void orc_transpose_u8(const uint8_t *q, int64_t R, int64_t C, uint8_t *qt)
{
    int64_t r, c;
    for (r = 0; r < R; r++)
        for (c = 0; c < C; c++)
            qt[c * R + r] = q[r * C + c];
}

/* fp32 transpose [R,C] -> [C,R]. */
static void transpose_f32(const float *s, int64_t R, int64_t C, float *st)
{
    int64_t r, c;
    for (r = 0; r < R; r++)
        for (c = 0; c < C; c++)
            st[c * R + r] = s[r * C + c];
}

/* ------------------------------------------------------------------ */
/* Stochastic rounding of one output plane (defined with the generator  */
/* further down): on = 0 means round to nearest even.                  */
/* ------------------------------------------------------------------ */
typedef struct {
    int on;
    uint64_t seed, offset;
    unsigned plane;
} sr_ctx;

static const sr_ctx kNoSR = {0, 0, 0, 0};

unsigned orc_sr_bits(uint64_t seed, uint64_t offset, unsigned plane, int64_t e);
unsigned orc_encode_sr(int fmt, float y, unsigned u);

/* Element e of a plane: Q_fmt(y) to nearest, or stochastically with the
 * plane's random bits for e. */
static unsigned encode_plane(int fmt, float y, sr_ctx sr, int64_t e)
{
    return sr.on ? orc_encode_sr(fmt, y, orc_sr_bits(sr.seed, sr.offset, sr.plane, e)) : orc_encode(fmt, y);
}

/* ------------------------------------------------------------------ */
/* Per-tensor scaling                                                  */
/* ------------------------------------------------------------------ */

/* a = max_i |x_i| over a rectangle of a row-major [*, ld] input. */
static float amax_rect(const void *x, int dt, int64_t ld, int64_t r0, int64_t nr, int64_t c0, int64_t nc)
{
    float a = 0.0f;
    int64_t r, c;
    for (r = r0; r < r0 + nr; r++)
        for (c = c0; c < c0 + nc; c++) {
            float v = fabsf(load_x(x, dt, r * ld + c));
            if (v > a)
                a = v;
        }
    return a;
}

/* a = max_i |x_i| of the whole tensor ([CS] "Current Scaling"; [MP] FP8
 * recipe 3, step 1). */
float orc_amax(const void *x, int dt, int64_t n) { return amax_rect(x, dt, n, 0, 1, 0, n); }

/*
 * Scales from an amax a for a format whose largest value is fmax
 * ([CS] "Current Scaling": alpha = Fmax / a multiplies before the cast,
 * s = a / Fmax multiplies after it; [MP] "FP8 recipe": a unit's amax maps to
 * the format's largest value).
 * READING: both are fp32 and each is its own correctly rounded quotient (so
 * they need not be exact reciprocals in fp32); s is the one stored.
 * READING ([CS] says an all-zero tensor needs its own rule): a = 0 gives
 * alpha = s = 1.  An alpha that overflows fp32 is held at FLT_MAX.
 */
void orc_tensor_scales(float a, float fmax, float *alpha, float *s)
{
    if (a == 0.0f) {
        *alpha = 1.0f;
        *s = 1.0f;
        return;
    }
    float al = fmax / a;
    if (al > FLT_MAX)
        al = FLT_MAX;
    *alpha = al;
    *s = a / fmax;
}

/* q_i = Q(fp32(alpha * x_i)) over n elements ([CS] "Current Scaling"),
 * rounded to nearest or (sr.on) stochastically. */
static void cast_run(const void *x, int dt, int64_t n, float alpha, int fmt, sr_ctx sr, uint8_t *q)
{
    int64_t i;
    for (i = 0; i < n; i++) {
        float y = load_x(x, dt, i) * alpha;
        q[i] = (uint8_t)encode_plane(fmt, y, sr, i);
    }
}

/*
 * Per-tensor quantization with a given amax: the second half of current
 * scaling, and the sharded form where the amax was reduced across shards
 * first ([CS] section "成本与多 GPU 使用", all-gather example;
 * [MP] section "FP8 通信", TP all-gather steps).
 * Rowwise bytes are [R,C]; the colwise bytes are the transposed copy [C,R]
 * made with the same scale ([MP] section "Per-tensor Current Scaling",
 * cast + cast_transpose).
 */
static int with_amax_core(const void *x, int dt, int64_t R, int64_t C, int fmt, unsigned outputs, float amax,
                          int sr_on, uint64_t seed, uint64_t offset, uint8_t *q_row, uint8_t *q_col, float *s_out)
{
    float alpha, s;
    uint8_t *q;
    if (fmt != ORC_E4M3 && fmt != ORC_E5M2)
        return -2;
    if (R < 0 || C < 0)
        return -3;
    if (check_finite(x, dt, R * C))
        return -1;
    orc_tensor_scales(amax, orc_fmax(fmt), &alpha, &s);
    if (sr_on) {
        /* each plane rounded with its own random bits: the colwise copy is
         * the recipe applied to X^T, not the transposed rowwise bytes */
        sr_ctx sr_row = {1, seed, offset, 0}, sr_col = {1, seed, offset, 1};
        if ((outputs & ORC_ROWWISE) && q_row)
            cast_run(x, dt, R * C, alpha, fmt, sr_row, q_row);
        if ((outputs & ORC_COLWISE) && q_col) {
            void *xt = transpose_input(x, dt, R, C);
            if (!xt)
                return -4;
            cast_run(xt, dt, R * C, alpha, fmt, sr_col, q_col);
            free(xt);
        }
    } else {
        q = q_row ? q_row : (uint8_t *)malloc((size_t)(R * C));
        cast_run(x, dt, R * C, alpha, fmt, kNoSR, q);
        if ((outputs & ORC_COLWISE) && q_col)
            orc_transpose_u8(q, R, C, q_col);
        if (!q_row)
            free(q);
    }
    if (s_out)
        *s_out = s;
    return 0;
}

int orc_quantize_with_amax(const void *x, int dt, int64_t R, int64_t C, int fmt, unsigned outputs,
                           float amax, uint8_t *q_row, uint8_t *q_col, float *s_out)
{
    return with_amax_core(x, dt, R, C, fmt, outputs, amax, 0, 0, 0, q_row, q_col, s_out);
}

/*
 * Per-tensor scaling with stochastically rounded elements ([MP] section
 * "FP8 数据格式", rounding: round-to-nearest-even by default, stochastic
 * rounding as an option for training stability; [LP] section 2.4 item 5: on
 * gradients).  The scales are those of round-to-nearest; each element's
 * fp32(alpha x) is rounded by orc_encode_sr with the random bits of its
 * plane (orc_sr_bits, plane 0 rowwise, 1 colwise).
 */
int orc_quantize_with_amax_sr(const void *x, int dt, int64_t R, int64_t C, int fmt, unsigned outputs,
                              float amax, uint64_t seed, uint64_t offset, uint8_t *q_row, uint8_t *q_col,
                              float *s_out)
{
    return with_amax_core(x, dt, R, C, fmt, outputs, amax, 1, seed, offset, q_row, q_col, s_out);
}

/* Per-tensor current scaling: amax of this tensor, then scale and cast
 * ([MP] FP8 recipe 3; [CS] "Current Scaling"). */
int orc_quantize_current(const void *x, int dt, int64_t R, int64_t C, int fmt, unsigned outputs,
                         uint8_t *q_row, uint8_t *q_col, float *s_out, float *amax_out)
{
    if (R < 0 || C < 0)
        return -3;
    if (check_finite(x, dt, R * C))
        return -1;
    float a = orc_amax(x, dt, R * C);
    if (amax_out)
        *amax_out = a;
    return orc_quantize_with_amax(x, dt, R, C, fmt, outputs, a, q_row, q_col, s_out);
}

/*
 * Per-tensor delayed scaling, one step ([MP] FP8 recipe 2; window length
 * and the max rule from the Megatron flags in [LP] section 4.3).
 *   1. cast with the scale alpha left by the previous steps;
 *   2. record this tensor's amax a_t in the window: hist[step mod H] = a_t;
 *   3. the next scale comes from m = max over the window:
 *      alpha = Fmax/m, s = m/Fmax (as orc_tensor_scales).
 * READING: the state starts as hist = 0, alpha = s = 1; an all-zero window
 * (m = 0) leaves alpha and s unchanged.
 */
int orc_quantize_delayed(const void *x, int dt, int64_t R, int64_t C, int fmt, unsigned outputs,
                         float *hist, int32_t H, float *alpha, float *s, int64_t step,
                         uint8_t *q_row, uint8_t *q_col, float *amax_out)
{
    uint8_t *q;
    int32_t j;
    if (fmt != ORC_E4M3 && fmt != ORC_E5M2)
        return -2;
    if (H < 1 || step < 0 || R < 0 || C < 0)
        return -3;
    if (check_finite(x, dt, R * C))
        return -1;
    q = q_row ? q_row : (uint8_t *)malloc((size_t)(R * C));
    cast_run(x, dt, R * C, *alpha, fmt, kNoSR, q);
    if ((outputs & ORC_COLWISE) && q_col)
        orc_transpose_u8(q, R, C, q_col);
    if (!q_row)
        free(q);
    float a = orc_amax(x, dt, R * C);
    if (amax_out)
        *amax_out = a;
    hist[step % H] = a;
    float m = 0.0f;
    for (j = 0; j < H; j++)
        if (hist[j] > m)
            m = hist[j];
    if (m > 0.0f)
        orc_tensor_scales(m, orc_fmax(fmt), alpha, s);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Blockwise fp32 scaling                                              */
/* ------------------------------------------------------------------ */

/*
 * Each tile of br x bc elements is quantized as its own tensor with
 * per-tensor current scaling to E4M3; its scale s_B = a_B/448 is stored in
 * fp32 ([MP] FP8 recipe 4 and section "Blockwise scaling": 1x128 tiles for
 * inputs and gradients, 128x128 tiles for weights, fp32 scales, pure E4M3).
 * Data is [R,C]; scales are row-major [R/br, C/bc].
 */
unsigned orc_mx_code_fmt(float a, int fmt);

/*
 * READING (power-of-two tile scales, the pow2 option): [MP] "Blockwise
 * scaling" describes running the blockwise recipe on Blackwell as MXFP8
 * blocks that share one scaling factor per tile, i.e. an E8M0 power of two;
 * the tile's scale is then the MX rule applied to the tile amax,
 * s_B = 2^(floor(log2 a_B) - 8) (orc_mx_code_fmt), stored as its fp32 value,
 * and the elements are Q_E4M3(x * 2^-e) (exact scaling, saturating).
 */
static void block_rowwise(const void *x, int dt, int64_t R, int64_t C, int br, int bc, int pow2, sr_ctx sr,
                          uint8_t *q, float *sc)
{
    int64_t tr, tc, r, c;
    int64_t nbc = C / bc;
    for (tr = 0; tr < R / br; tr++)
        for (tc = 0; tc < nbc; tc++) {
            float a = amax_rect(x, dt, C, tr * br, br, tc * bc, bc);
            float alpha, s;
            int e = 0;
            if (pow2) {
                e = (int)orc_mx_code_fmt(a, ORC_E4M3) - 127;
                s = ldexpf(1.0f, e);
                alpha = 0.0f; /* unused */
            } else {
                orc_tensor_scales(a, 448.0f, &alpha, &s);
            }
            sc[tr * nbc + tc] = s;
            for (r = tr * br; r < (tr + 1) * br; r++)
                for (c = tc * bc; c < (tc + 1) * bc; c++) {
                    float v = load_x(x, dt, r * C + c);
                    q[r * C + c] = (uint8_t)encode_plane(ORC_E4M3, pow2 ? ldexpf(v, -e) : v * alpha, sr, r * C + c);
                }
        }
}

/*
 * Colwise copies ([MP] "Blockwise scaling", the three GEMMs):
 *   1-D tiles (1 x bc): the transposed tensor X^T [C,R] is quantized with
 *     1 x bc tiles, i.e. the tiles run down the columns of X.
 *   2-D tiles: the colwise copy is the transpose of the rowwise bytes and
 *     scales, since a square tile quantizes to the same values either way
 *     ([MP] "Blockwise scaling", the closing remark on 2-D tiles).
 */
static int block_core(const void *x, int dt, int64_t R, int64_t C, int br, int bc, int pow2, unsigned outputs,
                      int sr_on, uint64_t seed, uint64_t offset, uint8_t *q_row, float *s_row, uint8_t *q_col,
                      float *s_col)
{
    sr_ctx sr_row = {sr_on, seed, offset, 0}, sr_col = {sr_on, seed, offset, 1};
    if (R <= 0 || C <= 0)
        return -3;
    if (!((br == 1 && bc == 128) || (br == 128 && bc == 128)))
        return -2;
    if (sr_on && br != 1)
        return -2;
    if (R % br || C % bc)
        return -3;
    if (check_finite(x, dt, R * C))
        return -1;
    if (br == 1) {
        if (outputs & ORC_ROWWISE)
            block_rowwise(x, dt, R, C, 1, bc, pow2, sr_row, q_row, s_row);
        if (outputs & ORC_COLWISE) {
            if (R % bc)
                return -3;
            void *xt = transpose_input(x, dt, R, C);
            block_rowwise(xt, dt, C, R, 1, bc, pow2, sr_col, q_col, s_col);
            free(xt);
        }
    } else {
        uint8_t *q = q_row ? q_row : (uint8_t *)malloc((size_t)(R * C));
        float *s = s_row ? s_row : (float *)malloc(sizeof(float) * (size_t)((R / br) * (C / bc)));
        block_rowwise(x, dt, R, C, br, bc, pow2, kNoSR, q, s);
        if (outputs & ORC_COLWISE) {
            orc_transpose_u8(q, R, C, q_col);
            transpose_f32(s, R / br, C / bc, s_col);
        }
        if (!q_row)
            free(q);
        if (!s_row)
            free(s);
    }
    return 0;
}

int orc_quantize_block_mode(const void *x, int dt, int64_t R, int64_t C, int br, int bc, int pow2,
                            unsigned outputs, uint8_t *q_row, float *s_row, uint8_t *q_col, float *s_col)
{
    return block_core(x, dt, R, C, br, bc, pow2, outputs, 0, 0, 0, q_row, s_row, q_col, s_col);
}

int orc_quantize_block(const void *x, int dt, int64_t R, int64_t C, int br, int bc, unsigned outputs,
                       uint8_t *q_row, float *s_row, uint8_t *q_col, float *s_col)
{
    return orc_quantize_block_mode(x, dt, R, C, br, bc, 0, outputs, q_row, s_row, q_col, s_col);
}

/*
 * Blockwise 1x128 with stochastically rounded elements (gradients, [MP]
 * "FP8 数据格式" rounding options; the tiles of the blockwise recipe for
 * inputs and gradients).  Tile scales as in round-to-nearest (fp32 or
 * power-of-two); elements by orc_encode_sr, plane 0 rowwise, 1 colwise
 * (the recipe on X^T).  The 128x128 weight tiles stay round-to-nearest.
 */
int orc_quantize_block_sr(const void *x, int dt, int64_t R, int64_t C, int pow2, unsigned outputs, uint64_t seed,
                          uint64_t offset, uint8_t *q_row, float *s_row, uint8_t *q_col, float *s_col)
{
    return block_core(x, dt, R, C, 1, 128, pow2, outputs, 1, seed, offset, q_row, s_row, q_col, s_col);
}

/* ------------------------------------------------------------------ */
/* MXFP8                                                               */
/* ------------------------------------------------------------------ */

/*
 * E8M0 code of a 32-element block with amax a: the block scale is the power
 * of two 2^e with e = floor(log2 a) - emax, emax = floor(log2 Fmax) of the
 * element format: 8 for E4M3 (448), 15 for E5M2 (57344), 2 for E2M1 (6)
 * ([MP] section "MXFP8" and FP8 recipe 5: 32-element blocks sharing one E8M0
 * power-of-two scale, E4M3 or E5M2 elements; [LP] section 2.4: MXFP4 uses
 * 32-element blocks with a UE8M0 scale and E2M1 elements).
 * READING: the exponent rule is the one this engine is specified with for
 * E4M3 (8 = floor(log2 448)), carried to the other element formats by their
 * own floor(log2 Fmax); e is held to the E8M0 range [-127, 127]; a = 0
 * gives e = -127.  Scaled values above Fmax (block maxima with a large
 * mantissa) saturate.
 */
static int fmt_emax(int fmt)
{
    int ex;
    frexp((double)orc_fmax(fmt), &ex); /* Fmax = f * 2^ex, f in [0.5, 1) */
    return ex - 1;
}

unsigned orc_mx_code_fmt(float a, int fmt)
{
    int ex, e;
    if (a == 0.0f)
        return 0;
    frexp((double)a, &ex);          /* a = f * 2^ex with f in [0.5, 1) */
    e = (ex - 1) - fmt_emax(fmt);   /* floor(log2 a) - emax */
    if (e < -127)
        e = -127;
    if (e > 127)
        e = 127;
    return (unsigned)(e + 127);
}

unsigned orc_mx_code(float a)
{
    return orc_mx_code_fmt(a, ORC_E4M3);
}

static void pack_nibbles(const uint8_t *nib, int64_t R, int64_t C, uint8_t *p);

/* Rowwise 1x32 MX blocks of a row-major [R,C] input: q = Q_fmt(x * 2^-e);
 * E2M1 codes are packed two per byte. */
static void mx_rowwise(const void *x, int dt, int64_t R, int64_t C, int fmt, sr_ctx sr, uint8_t *q,
                       uint8_t *codes)
{
    int64_t r, b, c, nb = C / 32;
    uint8_t *nib = fmt == ORC_E2M1 ? (uint8_t *)malloc((size_t)(R * C)) : q;
    for (r = 0; r < R; r++)
        for (b = 0; b < nb; b++) {
            float a = amax_rect(x, dt, C, r, 1, b * 32, 32);
            unsigned code = orc_mx_code_fmt(a, fmt);
            int e = (int)code - 127;
            codes[r * nb + b] = (uint8_t)code;
            for (c = b * 32; c < b * 32 + 32; c++)
                nib[r * C + c] = (uint8_t)encode_plane(fmt, ldexpf(load_x(x, dt, r * C + c), -e), sr, r * C + c);
        }
    if (fmt == ORC_E2M1) {
        pack_nibbles(nib, R, C, q);
        free(nib);
    }
}

/*
 * MX: rowwise 1x32 blocks along the rows, and a colwise copy whose 32x1
 * blocks run down the columns, stored transposed: [C,R] codes (E2M1: [C,R/2]
 * packed) and [C,R/32] scale codes, i.e. the rowwise recipe applied to X^T
 * ([MP] section "MXFP8 recipe": rowwise and colwise copies of the same
 * tensor, 1x32 and 32x1).
 */
static int mx_core(const void *x, int dt, int64_t R, int64_t C, int fmt, unsigned outputs, int sr_on,
                   uint64_t seed, uint64_t offset, uint8_t *q_row, uint8_t *e_row, uint8_t *q_col, uint8_t *e_col)
{
    sr_ctx sr_row = {sr_on, seed, offset, 0}, sr_col = {sr_on, seed, offset, 1};
    if (R <= 0 || C <= 0)
        return -3;
    if (fmt != ORC_E4M3 && fmt != ORC_E5M2 && fmt != ORC_E2M1)
        return -2;
    if (sr_on && fmt == ORC_E2M1)
        return -2;
    if (C % 32)
        return -3;
    if ((outputs & ORC_COLWISE) && R % 32)
        return -3;
    if (check_finite(x, dt, R * C))
        return -1;
    if (outputs & ORC_ROWWISE)
        mx_rowwise(x, dt, R, C, fmt, sr_row, q_row, e_row);
    if (outputs & ORC_COLWISE) {
        void *xt = transpose_input(x, dt, R, C);
        mx_rowwise(xt, dt, C, R, fmt, sr_col, q_col, e_col);
        free(xt);
    }
    return 0;
}

int orc_quantize_mx_fmt(const void *x, int dt, int64_t R, int64_t C, int fmt, unsigned outputs,
                        uint8_t *q_row, uint8_t *e_row, uint8_t *q_col, uint8_t *e_col)
{
    return mx_core(x, dt, R, C, fmt, outputs, 0, 0, 0, q_row, e_row, q_col, e_col);
}

/*
 * MX with E4M3 or E5M2 elements rounded stochastically ([MP] "FP8 数据格式"
 * rounding options, "MXFP8 recipe" blocks).  E8M0 block scales as in
 * round-to-nearest; elements x * 2^-e (exact) by orc_encode_sr, plane 0
 * rowwise, 1 colwise.
 */
int orc_quantize_mx_sr(const void *x, int dt, int64_t R, int64_t C, int fmt, unsigned outputs, uint64_t seed,
                       uint64_t offset, uint8_t *q_row, uint8_t *e_row, uint8_t *q_col, uint8_t *e_col)
{
    return mx_core(x, dt, R, C, fmt, outputs, 1, seed, offset, q_row, e_row, q_col, e_col);
}

int orc_quantize_mx(const void *x, int dt, int64_t R, int64_t C, unsigned outputs,
                    uint8_t *q_row, uint8_t *e_row, uint8_t *q_col, uint8_t *e_col)
{
    return orc_quantize_mx_fmt(x, dt, R, C, ORC_E4M3, outputs, q_row, e_row, q_col, e_col);
}

/* ------------------------------------------------------------------ */
/* NVFP4                                                               */
/* ------------------------------------------------------------------ */

/*
 * NVFP4 ([MP] FP8 recipe 6: 1x16 blocks, E4M3 block scales, one extra fp32
 * tensor-level scale; [LP] section 2.4: E2M1 elements, 16-element blocks,
 * 16x16 blocks for weights, 1x16 for activations and gradients).
 * READING (the two levels): the block amaxes divided by 6 (E2M1's largest
 * value) form a small tensor {b_B}; that tensor is quantized to E4M3 with
 * per-tensor current scaling, whose fp32 scale S is the tensor-level scale.
 * Its amax is fp32(A/6), A the amax of the whole tensor.  Each block's
 * decode scale is d_B = dec(c_B) * S, and the elements are q = Q_E2M1(x/d_B)
 * computed as fp32(x * fp32(1/d_B)).
 */
typedef struct {
    float alpha_s, S;
} nvfp4_tensor;

static nvfp4_tensor nvfp4_tensor_scale(float A)
{
    nvfp4_tensor t;
    float b_amax = A / 6.0f;
    orc_tensor_scales(b_amax, 448.0f, &t.alpha_s, &t.S);
    return t;
}

/* ------------------------------------------------------------------ */
/* Stochastic rounding                                                 */
/* ------------------------------------------------------------------ */

/*
 * Philox4x32-10, the counter-based generator of Salmon, Moraes, Dror and
 * Shaw, "Parallel random numbers: as easy as 1, 2, 3" (SC 2011): ten rounds
 * over a 4 x 32-bit counter; each round multiplies counter words 0 and 2 by
 * the two published 32-bit multipliers (full 64-bit products), and the new
 * counter is (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0); the 2 x 32-bit key is
 * bumped by the two published Weyl constants after every round.
 */
void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3], k0 = key[0], k1 = key[1];
    int round;
    for (round = 0; round < 10; round++) {
        uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        c0 = hi1 ^ c1 ^ k0;
        c1 = lo1;
        c2 = hi0 ^ c3 ^ k1;
        c3 = lo0;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    out[0] = c0;
    out[1] = c1;
    out[2] = c2;
    out[3] = c3;
}

/*
 * READING (random numbers of stochastic rounding; the pages name the
 * technique, [MP] "NVFP4" and [LP] section 2.4 item 5, but fix no generator):
 * element e of an output plane (its index in that plane's row-major order)
 * takes 16 random bits.  Elements are grouped by 8: group h = e / 8 is one
 * Philox4x32-10 call with key (seed mod 2^32, seed >> 32) and counter
 * (h mod 2^32, h >> 32, s mod 2^32, s >> 32), where the stream number
 * s = 2 * offset + plane (mod 2^64), plane 0 for the rowwise copy and 1 for
 * the colwise one; element j = e % 8 of the group takes bits
 * 16*(j%2) .. 16*(j%2)+15 of output word j / 2.
 */
unsigned orc_sr_bits(uint64_t seed, uint64_t offset, unsigned plane, int64_t e)
{
    uint32_t ctr[4], key[2], out[4];
    uint64_t h = (uint64_t)(e / 8), s = 2 * offset + plane;
    int j = (int)(e % 8);
    ctr[0] = (uint32_t)h;
    ctr[1] = (uint32_t)(h >> 32);
    ctr[2] = (uint32_t)s;
    ctr[3] = (uint32_t)(s >> 32);
    key[0] = (uint32_t)seed;
    key[1] = (uint32_t)(seed >> 32);
    orc_philox4x32_10(ctr, key, out);
    return (out[j / 2] >> (16 * (j % 2))) & 0xFFFFu;
}

/*
 * READING (stochastic rounding to E2M1; the pages name the technique, not
 * its arithmetic).  Stochastic rounding rounds v, lo <= v < hi between two
 * neighbouring representable values, up with probability g = (v - lo) /
 * (hi - lo) (Croci, Fasi, Higham, Mary and Mikaitis, "Stochastic rounding:
 * implementation, error analysis and applications", R. Soc. Open Sci. 2022).
 * With a finite random number the probability must be discretized; this
 * oracle takes the form those authors and SR hardware use: r random bits are
 * added to the bits below the last kept bit and the sum is truncated, here
 * with r = 16.  So v rounds to hi iff u + g * 2^16 >= 2^16 (u the 16-bit
 * random number, g * 2^16 exact in fp32), i.e. with probability
 * floor(g * 2^16) / 2^16, within 2^-16 of g.  (The other discretization,
 * "up iff u < g * 2^16", goes up with probability ceil(g * 2^16) / 2^16 and
 * picks the low u; it is equally faithful to the definition and is not this
 * one.)  Magnitudes of 6 or more saturate to 6, as in round-to-nearest; the
 * sign of y is kept, also on zero.
 */
unsigned orc_encode_e2m1_sr(float y, unsigned u)
{
    unsigned sign = signbit(y) ? 0x8u : 0u, k = 0;
    float v = fabsf(y), lo, hi, g;
    if (v >= 6.0f)
        return sign | 0x7u;
    while (k < 7 && (float)orc_decode(ORC_E2M1, k + 1) <= v)
        k++;
    lo = (float)orc_decode(ORC_E2M1, k);
    hi = (float)orc_decode(ORC_E2M1, k + 1);
    g = (v - lo) / (hi - lo);
    /* u + g*2^16 >= 2^16, compared exactly: g*2^16 is exact, 2^16 - u an integer */
    if (g * 65536.0f >= (float)(65536u - u))
        k++;
    return sign | k;
}

void orc_encode_e2m1_sr_array(const float *y, const uint16_t *u, int64_t n, uint8_t *q)
{
    int64_t i;
    for (i = 0; i < n; i++)
        q[i] = (uint8_t)orc_encode_e2m1_sr(y[i], u[i]);
}

/*
 * Stochastic rounding to any element format (E4M3, E5M2 or E2M1), the
 * reading of orc_encode_e2m1_sr carried to the 8-bit grids: for |y| between
 * the neighbouring representable magnitudes lo <= |y| < hi of the format
 * (subnormals included), round up iff u + g * 2^16 >= 2^16 with
 * g = (|y| - lo) / (hi - lo); magnitudes at or above the largest finite
 * value give it; the sign is kept, also on zero.  Every quantity is exact
 * in binary64 (|y| - lo and the division by a power of two).
 */
unsigned orc_encode_sr(int fmt, float y, unsigned u)
{
    const double *v = value_table(fmt);
    unsigned top = orc_max_code(fmt);
    unsigned sign = signbit(y) ? (1u << (FMT[fmt].bits - 1)) : 0u;
    double a = fabs((double)y), g;
    unsigned lo = 0, hi = top;
    if (a >= v[top])
        return sign | top;
    while (hi - lo > 1) {
        unsigned mid = (lo + hi) / 2;
        if (v[mid] <= a)
            lo = mid;
        else
            hi = mid;
    }
    /* v[lo] <= a < v[hi], hi = lo + 1 */
    g = (a - v[lo]) / (v[hi] - v[lo]);
    return sign | (g * 65536.0 >= (double)(65536u - (u & 0xFFFFu)) ? hi : lo);
}

void orc_encode_sr_array(int fmt, const float *y, const uint16_t *u, int64_t n, uint8_t *q)
{
    int64_t i;
    for (i = 0; i < n; i++)
        q[i] = (uint8_t)orc_encode_sr(fmt, y[i], u[i]);
}


/* One block of NVFP4: returns the E4M3 scale code and writes the nibbles
 * (0..15) of its elements.  Only the elements are rounded stochastically
 * (when sr.on); the block scale is always rounded to nearest even. */
static unsigned nvfp4_block(const void *x, int dt, int64_t ld, int64_t r0, int br, int64_t c0, int bc,
                            nvfp4_tensor t, sr_ctx sr, uint8_t *nib /* [R,C] nibble per element */)
{
    float a = amax_rect(x, dt, ld, r0, br, c0, bc);
    float b = a / 6.0f;
    unsigned code = orc_encode(ORC_E4M3, b * t.alpha_s);
    float d = (float)orc_decode(ORC_E4M3, code) * t.S;
    float r = 0.0f;
    int64_t i, j;
    if (d != 0.0f) {
        r = 1.0f / d;
        if (r > FLT_MAX)
            r = FLT_MAX;
    }
    for (i = r0; i < r0 + br; i++)
        for (j = c0; j < c0 + bc; j++) {
            float y = load_x(x, dt, i * ld + j) * r;
            nib[i * ld + j] = (uint8_t)(sr.on ? orc_encode_e2m1_sr(y, orc_sr_bits(sr.seed, sr.offset, sr.plane,
                                                                                     i * ld + j))
                                              : orc_encode(ORC_E2M1, y));
        }
    return code;
}

/* READING: element 2k of a row goes to bits 3..0 of byte k, element 2k+1 to
 * bits 7..4 ([MP] "NVFP4": two FP4 values per byte, high and low nibble). */
static void pack_nibbles(const uint8_t *nib, int64_t R, int64_t C, uint8_t *p)
{
    int64_t r, k;
    for (r = 0; r < R; r++)
        for (k = 0; k < C / 2; k++)
            p[r * (C / 2) + k] = (uint8_t)(nib[r * C + 2 * k] | (nib[r * C + 2 * k + 1] << 4));
}

static void nvfp4_rowwise(const void *x, int dt, int64_t R, int64_t C, int br, int bc, nvfp4_tensor t,
                          sr_ctx sr, uint8_t *p, uint8_t *codes, uint8_t *nib_out)
{
    int64_t tr, tc, nbc = C / bc;
    uint8_t *nib = (uint8_t *)malloc((size_t)(R * C));
    for (tr = 0; tr < R / br; tr++)
        for (tc = 0; tc < nbc; tc++)
            codes[tr * nbc + tc] = (uint8_t)nvfp4_block(x, dt, C, tr * br, br, tc * bc, bc, t, sr, nib);
    pack_nibbles(nib, R, C, p);
    if (nib_out)
        memcpy(nib_out, nib, (size_t)(R * C));
    free(nib);
}

/*
 * Rowwise: packed data [R, C/2], E4M3 codes [R/br, C/bc], tensor scale S.
 * A is the tensor amax (given here, e.g. reduced across shards first).
 * Colwise (READING): 1x16 -> the same recipe on X^T, with the same tensor
 * scale (the amax of X^T is the amax of X); 16x16 -> the element codes of
 * the rowwise result transposed and re-packed along the rows of X^T, codes
 * transposed ([MP] closing remarks: FP4 GEMMs need two copies even for 2-D
 * weight tiles).
 */
static int nvfp4_core(const void *x, int dt, int64_t R, int64_t C, int br, int bc, unsigned outputs, float A,
                      int sr_on, uint64_t seed, uint64_t offset, uint8_t *p_row, uint8_t *c_row, uint8_t *p_col,
                      uint8_t *c_col, float *S_out, float *amax_out)
{
    sr_ctx sr_row = {sr_on, seed, offset, 0}, sr_col = {sr_on, seed, offset, 1};
    if (R <= 0 || C <= 0)
        return -3;
    if (!((br == 1 && bc == 16) || (br == 16 && bc == 16)))
        return -2;
    if (R % br || C % bc)
        return -3;
    if ((outputs & ORC_COLWISE) && (R % 16))
        return -3;
    if (check_finite(x, dt, R * C))
        return -1;
    nvfp4_tensor t = nvfp4_tensor_scale(A);
    if (S_out)
        *S_out = t.S;
    if (amax_out)
        *amax_out = A;
    if (sr_on && br != 1)
        return -2;
    if (br == 1) {
        if (outputs & ORC_ROWWISE)
            nvfp4_rowwise(x, dt, R, C, 1, bc, t, sr_row, p_row, c_row, NULL);
        if (outputs & ORC_COLWISE) {
            void *xt = transpose_input(x, dt, R, C);
            nvfp4_rowwise(xt, dt, C, R, 1, bc, t, sr_col, p_col, c_col, NULL);
            free(xt);
        }
    } else {
        uint8_t *nib = (uint8_t *)malloc((size_t)(R * C));
        uint8_t *p = p_row ? p_row : (uint8_t *)malloc((size_t)(R * C / 2));
        uint8_t *cd = c_row ? c_row : (uint8_t *)malloc((size_t)((R / br) * (C / bc)));
        nvfp4_rowwise(x, dt, R, C, br, bc, t, kNoSR, p, cd, nib);
        if (outputs & ORC_COLWISE) {
            uint8_t *nt = (uint8_t *)malloc((size_t)(R * C));
            orc_transpose_u8(nib, R, C, nt);
            pack_nibbles(nt, C, R, p_col);
            orc_transpose_u8(cd, R / br, C / bc, c_col);
            free(nt);
        }
        free(nib);
        if (!p_row)
            free(p);
        if (!c_row)
            free(cd);
    }
    return 0;
}

int orc_quantize_nvfp4_with_amax(const void *x, int dt, int64_t R, int64_t C, int br, int bc, unsigned outputs,
                                 float A, uint8_t *p_row, uint8_t *c_row, uint8_t *p_col, uint8_t *c_col,
                                 float *S_out, float *amax_out)
{
    return nvfp4_core(x, dt, R, C, br, bc, outputs, A, 0, 0, 0, p_row, c_row, p_col, c_col, S_out, amax_out);
}

/*
 * NVFP4 1x16 with stochastically rounded elements ([MP] "NVFP4": stochastic
 * rounding as an option for FP4; [LP] section 2.4 item 5: on gradients).
 * Everything but the element rounding is the round-to-nearest recipe above;
 * random bits from orc_sr_bits (plane 0 rowwise, 1 colwise).
 */
int orc_quantize_nvfp4_sr_with_amax(const void *x, int dt, int64_t R, int64_t C, unsigned outputs, float A,
                                    uint64_t seed, uint64_t offset, uint8_t *p_row, uint8_t *c_row,
                                    uint8_t *p_col, uint8_t *c_col, float *S_out, float *amax_out)
{
    return nvfp4_core(x, dt, R, C, 1, 16, outputs, A, 1, seed, offset, p_row, c_row, p_col, c_col, S_out,
                      amax_out);
}

/*
 * Random Hadamard transform of 16 consecutive values ([LP] section 2.4
 * item 3: applied to the inputs of the weight-gradient GEMM to spread
 * block-level outliers before FP4 quantization).
 * READING (the pages give no size, signs or arithmetic): y = (1/4) H16 (s.x),
 * H16 the 16 x 16 Sylvester Hadamard matrix (entry (i, j) = (-1)^popcount(i&j)),
 * s_i = -1 where bit i of `signs` is set, else +1; (1/4) H16 diag(s) is
 * orthogonal, so applying it to both GEMM operands along the contraction
 * leaves the product unchanged.  Arithmetic: the sign flips are exact; the
 * sums are the fast Walsh-Hadamard transform in fp32, stages h = 1, 2, 4, 8,
 * each replacing the pair (w_i, w_{i+h}), bit h of i clear, by
 * (w_i + w_{i+h}, w_i - w_{i+h}); the factor 1/4 is an exact multiply.
 */
void orc_rht16(const float *x, unsigned signs, float *y)
{
    float w[16];
    int i, h;
    for (i = 0; i < 16; i++)
        w[i] = ((signs >> i) & 1u) ? -x[i] : x[i];
    for (h = 1; h < 16; h *= 2)
        for (i = 0; i < 16; i++)
            if (!(i & h)) {
                float a = w[i], b = w[i + h];
                w[i] = a + b;
                w[i + h] = a - b;
            }
    for (i = 0; i < 16; i++)
        y[i] = w[i] * 0.25f;
}

void orc_rht16_array(const float *x, int64_t nchunks, unsigned signs, float *y)
{
    int64_t k;
    for (k = 0; k < nchunks; k++)
        orc_rht16(x + 16 * k, signs, y + 16 * k);
}

/*
 * NVFP4 1x16 colwise copy of a weight-gradient input with the RHT
 * ([LP] section 2.4 items 1, 3 and 5).  READING: the GEMM contracts X^T
 * [C,R] along R, so each row of X^T is transformed in 16-element chunks
 * (the 1x16 blocks) and the transformed tensor Y^T is quantized with the
 * NVFP4 recipe: its tensor amax A' = max|Y^T| (or the given amax of the
 * transformed tensor, e.g. reduced across shards) sets the tensor scale.
 * The rowwise copy (other GEMMs) is not transformed and is produced by the
 * plain recipe.  Elements may be rounded stochastically (plane 1 bits).
 */
int orc_quantize_nvfp4_rht(const void *x, int dt, int64_t R, int64_t C, unsigned signs, int use_amax, float A,
                           int sr_on, uint64_t seed, uint64_t offset, uint8_t *p_col, uint8_t *c_col,
                           float *S_out, float *amax_out)
{
    int64_t r, c;
    float *yt, a = 0.0f;
    if (R <= 0 || C <= 0)
        return -3;
    if (R % 16 || C % 16)
        return -3;
    if (check_finite(x, dt, R * C))
        return -1;
    yt = (float *)malloc(sizeof(float) * (size_t)(R * C));
    for (c = 0; c < C; c++)
        for (r = 0; r < R; r++)
            yt[c * R + r] = load_x(x, dt, r * C + c);
    orc_rht16_array(yt, R * C / 16, signs, yt);
    for (r = 0; r < R * C; r++)
        if (fabsf(yt[r]) > a)
            a = fabsf(yt[r]);
    if (use_amax)
        a = A;
    {
        nvfp4_tensor t = nvfp4_tensor_scale(a);
        sr_ctx sr = {sr_on, seed, offset, 1};
        if (S_out)
            *S_out = t.S;
        if (amax_out)
            *amax_out = a;
        nvfp4_rowwise(yt, ORC_IN_F32, C, R, 1, 16, t, sr, p_col, c_col, NULL);
    }
    free(yt);
    return 0;
}

/* NVFP4 with A = the amax of this tensor. */
int orc_quantize_nvfp4(const void *x, int dt, int64_t R, int64_t C, int br, int bc, unsigned outputs,
                       uint8_t *p_row, uint8_t *c_row, uint8_t *p_col, uint8_t *c_col, float *S_out,
                       float *amax_out)
{
    if (R <= 0 || C <= 0)
        return -3;
    if (check_finite(x, dt, R * C))
        return -1;
    return orc_quantize_nvfp4_with_amax(x, dt, R, C, br, bc, outputs, orc_amax(x, dt, R * C), p_row, c_row, p_col,
                                        c_col, S_out, amax_out);
}

/* ------------------------------------------------------------------ */
/* Dequantization                                                      */
/* ------------------------------------------------------------------ */

/* x_hat = fp32(dec(q) * s) over n codes ([CS] "Current Scaling": the value
 * is restored by multiplying the FP8 value by s). */
void orc_dequant_tensor(const uint8_t *q, int64_t n, int fmt, float s, float *y)
{
    int64_t i;
    for (i = 0; i < n; i++)
        y[i] = (float)orc_decode(fmt, q[i]) * s;
}

/* Blockwise: each element times its tile's s_B. */
void orc_dequant_block(const uint8_t *q, const float *sc, int64_t R, int64_t C, int br, int bc, float *y)
{
    int64_t r, c;
    for (r = 0; r < R; r++)
        for (c = 0; c < C; c++)
            y[r * C + c] = (float)orc_decode(ORC_E4M3, q[r * C + c]) * sc[(r / br) * (C / bc) + c / bc];
}

/* MX: each element times 2^(code-127) of its block ([MP] "MXFP8": value is
 * element times the block's shared scale). */
/* MX: element times 2^(code - 127); E2M1 elements packed two per byte
 * ([R, C/2]), element 2k in the low nibble. */
void orc_dequant_mx_fmt(const uint8_t *q, const uint8_t *codes, int64_t R, int64_t C, int fmt, float *y)
{
    int64_t r, c;
    for (r = 0; r < R; r++)
        for (c = 0; c < C; c++) {
            unsigned code;
            if (fmt == ORC_E2M1)
                code = (q[r * (C / 2) + c / 2] >> (4 * (c % 2))) & 0xFu;
            else
                code = q[r * C + c];
            y[r * C + c] = ldexpf((float)orc_decode(fmt, code), (int)codes[r * (C / 32) + c / 32] - 127);
        }
}

void orc_dequant_mx(const uint8_t *q, const uint8_t *codes, int64_t R, int64_t C, float *y)
{
    orc_dequant_mx_fmt(q, codes, R, C, ORC_E4M3, y);
}

/* NVFP4: each element times d_B = fp32(dec(c_B) * S). */
void orc_dequant_nvfp4(const uint8_t *p, const uint8_t *codes, float S, int64_t R, int64_t C, int br, int bc,
                       float *y)
{
    int64_t r, c;
    for (r = 0; r < R; r++)
        for (c = 0; c < C; c++) {
            uint8_t byte = p[r * (C / 2) + c / 2];
            unsigned nib = (c & 1) ? (byte >> 4) : (byte & 0xF);
            float d = (float)orc_decode(ORC_E4M3, codes[(r / br) * (C / bc) + c / bc]) * S;
            y[r * C + c] = (float)orc_decode(ORC_E2M1, nib) * d;
        }
}

/* ------------------------------------------------------------------ */
/* bf16 output and requantization                                      */
/* ------------------------------------------------------------------ */

/* fp32 -> bf16 bits, rounded to nearest even (the top 16 bits of the fp32
 * pattern after adding half an ulp of bf16 with ties to even). Finite inputs;
 * a NaN keeps a quiet NaN pattern. */
uint16_t orc_f32_to_bf16(float f)
{
    uint32_t b;
    memcpy(&b, &f, 4);
    if ((b & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((b >> 16) | 0x40u);
    uint32_t lsb = (b >> 16) & 1u;
    b += 0x7fffu + lsb;
    return (uint16_t)(b >> 16);
}

void orc_f32_to_bf16_array(const float *y, int64_t n, uint16_t *out)
{
    int64_t i;
    for (i = 0; i < n; i++)
        out[i] = orc_f32_to_bf16(y[i]);
}

/*
 * MXFP8 "de-quantize and re-quantize in the other direction" ([MP] section
 * "FP8 通信", the EP backward step): from the rowwise copy alone (codes and
 * E8M0 codes of 1x32 blocks), restore the fp32 values
 * x_hat = dec(q) * 2^(code-127), and quantize x_hat^T with the MX recipe, i.e.
 * 32x1 blocks down the columns, stored transposed. Power-of-two scales make
 * the restored values exact in fp32.
 */
int orc_requant_mx_colwise(const uint8_t *q_row, const uint8_t *e_row, int64_t R, int64_t C, uint8_t *q_col,
                           uint8_t *e_col)
{
    float *xhat, *xt;
    if (R <= 0 || C <= 0 || C % 32 || R % 32)
        return -3;
    xhat = (float *)malloc(sizeof(float) * (size_t)(R * C));
    orc_dequant_mx(q_row, e_row, R, C, xhat);
    xt = (float *)malloc(sizeof(float) * (size_t)(R * C));
    transpose_f32(xhat, R, C, xt);
    mx_rowwise(xt, ORC_IN_F32, C, R, ORC_E4M3, kNoSR, q_col, e_col);
    free(xt);
    free(xhat);
    return 0;
}

/*
 * The same step for the blockwise recipe with 1x128 tiles and power-of-two
 * scales, the DeepSeek-V3-like activation layout whose 1-D tiles run along
 * the token's hidden vector ([MP] section "FP8 通信": an FP8 expert-parallel
 * dispatch sends only the rowwise copy, and the scales must be powers of two
 * for the re-quantization to match a single quantization up to special
 * values such as subnormals; [MP] "Blockwise scaling": the colwise copy of a
 * 1-D tiling quantizes X^T with the same tiles). From q_row [R,C] and the
 * tile scales s_row [R, C/128]: x_hat = dec(q) * s (exact in fp32, the scale
 * being a power of two), then X_hat^T is quantized with 1x128 tiles and
 * power-of-two scales: q_col [C,R], s_col [C, R/128].
 */
int orc_requant_block_colwise(const uint8_t *q_row, const float *s_row, int64_t R, int64_t C, uint8_t *q_col,
                              float *s_col)
{
    float *xhat, *xt;
    if (R <= 0 || C <= 0 || C % 128 || R % 128)
        return -3;
    xhat = (float *)malloc(sizeof(float) * (size_t)(R * C));
    orc_dequant_block(q_row, s_row, R, C, 1, 128, xhat);
    xt = (float *)malloc(sizeof(float) * (size_t)(R * C));
    transpose_f32(xhat, R, C, xt);
    block_rowwise(xt, ORC_IN_F32, C, R, 1, 128, 1, kNoSR, q_col, s_col);
    free(xt);
    free(xhat);
    return 0;
}
