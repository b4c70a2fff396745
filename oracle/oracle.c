/*
 * oracle.c -- plain, slow, obviously-correct CPU definition of the scaled
 * linear layer with a fused epilogue.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this file: only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header, table or constant with
 * the HIP library; the two meet only at the byte arrays both consume.
 *
 * What is computed (for every output element m, n):
 *
 *   acc[m,n] = sum_k  dec(A[m,k]) * dec(B[n,k])                      (1)
 *   y        = acc * sa[m] * sb[n]            (per-token x per-channel) (2)
 *       or     sum_kb sa[m,kb] * sb[n/128,kb] * acc_kb   (block scales)
 *   y        = y + bias[n]                                            (3)
 *   y        = act(y)           none | ReLU | GELU (tanh form) | SiLU (4)
 *   r[m,n]   = y * alpha + residual[m,n]                              (5)
 *
 * Sources (the pages describe it; these notes restate it in our own words):
 *  - "Совместная работа Helion и TorchInductor: слияние операторов"
 *    (gurufy.ru), section on extensible epilogues in Helion: the kernel keeps
 *    an fp32 accumulator of A times B over the K loop, then adds a bias
 *    broadcast over rows, applies ReLU (activation code 1) or the tanh
 *    approximation of GELU with the constants sqrt(2/pi) ~ 0.79788456 and
 *    0.044715 (activation code 2), and narrows to a 16-bit float for the one
 *    store.  The section on the opacity barrier lists the decoder-block
 *    epilogue as scaling, residual add and activation; the section on
 *    prologue/epilogue strategies names bias, residual, GELU/SiLU and the
 *    fp32 -> 16-bit narrowing as epilogue work.
 *  - "helion-vllm-linear-backend" (aixai.ru), section "Одно ядро вместо трёх
 *    вариантов": FP8_Dynamic uses a per-token activation scale and a
 *    per-channel weight scale, W8A8_INT8 the same scaling in int8, and
 *    Block_FP8 1x128 activation and 128x128 weight scale blocks.
 *
 * Readings taken where the pages leave a step open:
 *  - Weight layout is B[N,K] (K contiguous), i.e. C = A * B^T.
 *  - FP8 is the OCP E4M3FN encoding (bias 7, max 448, codes 0x7F/0xFF NaN).
 *  - The epilogue order is act(acc*sa*sb + bias) * alpha + residual.
 *  - GELU is the tanh form; sqrt(2/pi) is taken exactly (in fp64) rather than
 *    as the 8-digit decimal the listing prints.
 *
 * Exactness: fp8 and bf16/fp16 codes decode exactly into fp64.  Products of
 * two e4m3 values are multiples of 2^-18 bounded by 448^2, so the fp64 sum in
 * (1) is exact for K <= 171196; int8 products are summed in int64 and must
 * fit int32.  bf16/fp16 sums are fp64 (error far below any tolerance used).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Quant-mode and activation codes (the same numbering as the library's public
 * header; written out here independently). */
enum { OQ_BF16 = 0, OQ_FP16 = 1, OQ_FP8_DYNAMIC = 2, OQ_W8A8_INT8 = 3, OQ_BLOCK_FP8 = 4,
       OQ_MXFP4 = 5 };
enum { OA_NONE = 0, OA_RELU = 1, OA_GELU_TANH = 2, OA_SILU = 3 };
enum { O_OK = 0, O_BAD_ARG = -1, O_INT32_OVERFLOW = -2 };

/* ---------------------------------------------------------------- decoders */

/* OCP E4M3FN: s eeee mmm.  e == 0: (-1)^s * 2^-6 * m/8 (subnormal);
 * otherwise (-1)^s * 2^(e-7) * (1 + m/8).  eeee mmm == 1111 111 is NaN; there
 * is no infinity. */
double oracle_e4m3_to_f64(uint8_t code) {
    int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m / 8.0, -6);
    else v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

/* 4-bit weights (the MI355X-native counterpart of the INT4 / NVFP4 weight
 * formats "helion-vllm-linear-backend" lists in its section "Зачем трогать
 * линейные слои"; the pages define no 4-bit format, so the format is taken
 * from the OCP Microscaling (MX) v1.0 specification, MXFP4):
 * E2M1 element: s ee m; e == 0: (-1)^s * m/2 (0 or 0.5); otherwise
 * (-1)^s * 2^(e-1) * (1 + m/2).  No infinity or NaN. */
double oracle_e2m1_to_f64(uint8_t code) {
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double v = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -v : v;
}

/* E8M0 shared scale of a block of 32 elements: 2^(e - 127); e == 255 is NaN. */
double oracle_e8m0_to_f64(uint8_t code) {
    return code == 255 ? NAN : ldexp(1.0, (int)code - 127);
}

/* bfloat16: the upper half of an IEEE binary32. */
double oracle_bf16_to_f64(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* IEEE binary16: s eeeee mmmmmmmmmm, bias 15. */
double oracle_fp16_to_f64(uint16_t bits) {
    int s = (bits >> 15) & 1, e = (bits >> 10) & 31, m = bits & 1023;
    double v;
    if (e == 31) v = m ? NAN : INFINITY;
    else if (e == 0) v = ldexp((double)m, -24);
    else v = ldexp(1.0 + (double)m / 1024.0, e - 15);
    return s ? -v : v;
}

/* fp64 -> bfloat16, round to nearest, ties to even (done on the exact value,
 * not through an fp32 intermediate).  NaN stays NaN, overflow goes to inf. */
uint16_t oracle_f64_to_bf16_rne(double x) {
    if (isnan(x)) return 0x7FC0;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);               /* a = f * 2^e, f in [0.5, 1) */
    int E = e - 1;              /* a = 1.xxx * 2^E */
    if (E < -126) E = -126;     /* subnormal range: fixed quantum 2^-133 */
    double q = ldexp(1.0, E - 7);          /* bf16 spacing at this exponent */
    double n = a / q;                      /* exact: scaling by a power of 2 */
    double fl = floor(n), rem = n - fl;
    double r = fl;
    if (rem > 0.5 || (rem == 0.5 && fmod(fl, 2.0) != 0.0)) r = fl + 1.0;
    double v = r * q;
    if (v >= ldexp(2.0, 127)) return sign | 0x7F80;  /* beyond max finite */
    float f = (float)v;                    /* exact: v is a bf16 value */
    uint32_t u;
    memcpy(&u, &f, 4);
    return sign | (uint16_t)((u >> 16) & 0x7FFF);
}

/* ------------------------------------------------------------- activations */

double oracle_act(int act, double y) {
    switch (act) {
    case OA_NONE: return y;
    case OA_RELU: return y > 0.0 ? y : 0.0;
    case OA_GELU_TANH: {
        const double c = sqrt(2.0 / 3.14159265358979323846);
        return 0.5 * y * (1.0 + tanh(c * (y + 0.044715 * y * y * y)));
    }
    case OA_SILU: return y / (1.0 + exp(-y));
    default: return NAN;
    }
}

/* --------------------------------------------------------------- the layer */

typedef struct {
    const void *A, *B;          /* A[M][K], B[N][K] raw codes */
    const float *sa, *sb;       /* scales (see the layouts below) */
    const uint16_t *bias;       /* [N] 16-bit float codes or NULL */
    const uint16_t *residual;   /* [M][N] 16-bit float codes or NULL */
    double alpha;
    int64_t M, N, K;
    int quant, act;
} olayer_t;

/* Lookup tables filled from the closed forms above (every code, once), so
 * the O(MNK) loops do not call ldexp per element. */
static double g_e4m3[256];
static double g_fp16[65536];
static int g_tables_ready = 0;

static void tables_init(void) {
    if (g_tables_ready) return;
    for (int c = 0; c < 256; ++c) g_e4m3[c] = oracle_e4m3_to_f64((uint8_t)c);
    for (int c = 0; c < 65536; ++c) g_fp16[c] = oracle_fp16_to_f64((uint16_t)c);
    g_tables_ready = 1;
}

static double dec16(int quant, uint16_t v) {
    return quant == OQ_FP16 ? g_fp16[v] : oracle_bf16_to_f64(v);
}

static double elem(const olayer_t *L, const void *X, int64_t idx) {
    switch (L->quant) {
    case OQ_BF16: return oracle_bf16_to_f64(((const uint16_t *)X)[idx]);
    case OQ_FP16: return g_fp16[((const uint16_t *)X)[idx]];
    case OQ_FP8_DYNAMIC:
    case OQ_BLOCK_FP8: return g_e4m3[((const uint8_t *)X)[idx]];
    default: return NAN;
    }
}

/* Step (1): the raw accumulator.  For int8 the exact int64 sum (the caller
 * checks that it fits int32); otherwise the fp64 sum. */
static int64_t dot_i8(const olayer_t *L, int64_t m, int64_t n) {
    const int8_t *a = (const int8_t *)L->A + m * L->K;
    const int8_t *b = (const int8_t *)L->B + n * L->K;
    int64_t s = 0;
    for (int64_t k = 0; k < L->K; ++k) s += (int64_t)a[k] * (int64_t)b[k];
    return s;
}

static double dot_f(const olayer_t *L, int64_t m, int64_t n, int64_t k0, int64_t k1) {
    double s = 0.0;
    for (int64_t k = k0; k < k1; ++k)
        s += elem(L, L->A, m * L->K + k) * elem(L, L->B, n * L->K + k);
    return s;
}

/* Steps (1)-(5) for one output element.  *acc_out receives the int32
 * accumulator in int8 mode. */
/* MXFP4 weights: B holds two E2M1 codes per byte (k = 2j in the low nibble
 * of byte j, k = 2j + 1 in the high nibble), row n at B + n*K/2; sb is
 * reinterpreted as E8M0 bytes [N][K/32].  A is bf16.  The sum is exact in
 * fp64 unless its terms span more than 53 bits of magnitude. */
static double dot_mx(const olayer_t *L, int64_t m, int64_t n) {
    const uint16_t *a = (const uint16_t *)L->A + m * L->K;
    const uint8_t *b = (const uint8_t *)L->B + n * (L->K / 2);
    const uint8_t *sc = (const uint8_t *)L->sb + n * (L->K / 32);
    double s = 0.0;
    for (int64_t k = 0; k < L->K; ++k) {
        const uint8_t byte = b[k / 2];
        const uint8_t code = (k & 1) ? (byte >> 4) : (byte & 15);
        s += oracle_bf16_to_f64(a[k]) * oracle_e2m1_to_f64(code) * oracle_e8m0_to_f64(sc[k / 32]);
    }
    return s;
}

static int one(const olayer_t *L, int64_t m, int64_t n, double *r_out, int32_t *acc_out) {
    double y;
    if (L->quant == OQ_MXFP4) {
        y = dot_mx(L, m, n);
    } else if (L->quant == OQ_W8A8_INT8) {
        int64_t s = dot_i8(L, m, n);
        if (s > INT32_MAX || s < INT32_MIN) return O_INT32_OVERFLOW;
        if (acc_out) *acc_out = (int32_t)s;
        y = (double)s * (double)L->sa[m] * (double)L->sb[n];
    } else if (L->quant == OQ_BLOCK_FP8) {
        /* per 128-wide K block: exact partial sum, then its two scales;
         * sa is [M][K/128], sb is [N/128][K/128] */
        int64_t KB = L->K / 128;
        y = 0.0;
        for (int64_t kb = 0; kb < KB; ++kb) {
            double p = dot_f(L, m, n, kb * 128, kb * 128 + 128);
            y += (double)L->sa[m * KB + kb] * (double)L->sb[(n / 128) * KB + kb] * p;
        }
    } else {
        y = dot_f(L, m, n, 0, L->K);
        if (L->quant == OQ_FP8_DYNAMIC) y = y * (double)L->sa[m] * (double)L->sb[n];
    }
    if (L->bias) y += dec16(L->quant, L->bias[n]);
    y = oracle_act(L->act, y);
    y = y * L->alpha;
    if (L->residual) y += dec16(L->quant, L->residual[m * L->N + n]);
    *r_out = y;
    return O_OK;
}

static int check(const olayer_t *L) {
    tables_init();
    if (L->M < 0 || L->N < 0 || L->K < 0) return O_BAD_ARG;
    if (L->quant < OQ_BF16 || L->quant > OQ_MXFP4) return O_BAD_ARG;
    if (L->act < OA_NONE || L->act > OA_SILU) return O_BAD_ARG;
    if ((L->quant == OQ_FP8_DYNAMIC || L->quant == OQ_W8A8_INT8 || L->quant == OQ_BLOCK_FP8) &&
        (!L->sa || !L->sb)) return O_BAD_ARG;
    if (L->quant == OQ_BLOCK_FP8 && (L->K % 128 != 0 || L->N % 128 != 0)) return O_BAD_ARG;
    if (L->quant == OQ_MXFP4 && (!L->sb || L->K % 32 != 0)) return O_BAD_ARG;
    return O_OK;
}

/* Full output: out[M][N] fp64 and, in int8 mode, acc[M][N] int32 (may be
 * NULL).  Rows are spread over nthreads OpenMP threads (<= 0: default). */
int oracle_linear(const void *A, const void *B, const float *sa, const float *sb,
                  double alpha, const uint16_t *bias, const uint16_t *residual,
                  int64_t M, int64_t N, int64_t K, int quant, int act,
                  double *out, int32_t *acc, int nthreads) {
    olayer_t L = {A, B, sa, sb, bias, residual, alpha, M, N, K, quant, act};
    int rc = check(&L);
    if (rc) return rc;
    int status = O_OK;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            int32_t a32 = 0;
            int r = one(&L, m, n, &out[m * N + n], &a32);
            if (acc) acc[m * N + n] = a32;
            if (r) {
#pragma omp atomic write
                status = r;
            }
        }
    }
    return status;
}

/* Selected elements only: out[i] = r[idx_m[i], idx_n[i]] (and acc[i] in int8
 * mode), for checking full-size problems at sampled positions. */
int oracle_linear_at(const void *A, const void *B, const float *sa, const float *sb,
                     double alpha, const uint16_t *bias, const uint16_t *residual,
                     int64_t M, int64_t N, int64_t K, int quant, int act,
                     const int64_t *idx_m, const int64_t *idx_n, int64_t count,
                     double *out, int32_t *acc, int nthreads) {
    olayer_t L = {A, B, sa, sb, bias, residual, alpha, M, N, K, quant, act};
    int rc = check(&L);
    if (rc) return rc;
    for (int64_t i = 0; i < count; ++i)
        if (idx_m[i] < 0 || idx_m[i] >= M || idx_n[i] < 0 || idx_n[i] >= N) return O_BAD_ARG;
    int status = O_OK;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < count; ++i) {
        int32_t a32 = 0;
        int r = one(&L, idx_m[i], idx_n[i], &out[i], &a32);
        if (acc) acc[i] = a32;
        if (r) {
#pragma omp atomic write
            status = r;
        }
    }
    return status;
}

/* The three-kernel unfused path of the pages' decoder-block example, stage by
 * stage, each stage from its own input so the GPU's stages can be checked
 * one at a time (the opacity-barrier section: GEMM output materialised,
 * re-read for bias + GELU, materialised again, re-read for the residual).
 *   stage 2:  u = GELU(t + bias[n])          (t: the stored GEMM output)
 *   stage 3:  o = alpha * u + residual[m,n]  (u: the stored stage-2 output)
 * Inputs and outputs are 16-bit codes of the given quant mode's float type;
 * outputs are fp64 (the reference value before the final narrowing). */
int oracle_unfused_stage2(const uint16_t *t, const uint16_t *bias, int64_t M, int64_t N,
                          int quant, int act, double *u) {
    tables_init();
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double y = dec16(quant, t[m * N + n]);
            if (bias) y += dec16(quant, bias[n]);
            u[m * N + n] = oracle_act(act, y);
        }
    return O_OK;
}

int oracle_unfused_stage3(const uint16_t *u, const uint16_t *residual, double alpha,
                          int64_t M, int64_t N, int quant, double *o) {
    tables_init();
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double y = dec16(quant, u[m * N + n]) * alpha;
            if (residual) y += dec16(quant, residual[m * N + n]);
            o[m * N + n] = y;
        }
    return O_OK;
}

/* ------------------------------------------------- dynamic quantization */
/*
 * Dynamic activation quantization: the step right before the layer, which
 * produces its A operand and activation scales at run time.  The pages name
 * it but do not spell it out: "helion-vllm-linear-backend" (section "Одно
 * ядро вместо трёх вариантов") gives FP8_Dynamic a per-token activation
 * scale, W8A8_INT8 the same scaling in int8, and Block_FP8 1x128 activation
 * blocks; the section on prologue/epilogue strategies of "Совместная работа
 * Helion и TorchInductor" lists quantization among the input-side (prologue)
 * transforms.  Readings taken here, for every group g of values (a row for
 * the per-token kinds, a 1x128 block of a row for the block kind):
 *
 *   amax_g  = max |x| over the group                 (exact)
 *   s_g     = amax_g / QMAX   in binary32, QMAX = 448 (e4m3) or 127 (int8)
 *             (s_g = 1 when amax_g == 0, so an all-zero group maps to 0)
 *   v       = x / s_g          in binary32
 *   e4m3:     q = the E4M3FN code nearest to v, ties to the even code,
 *             |v| >= 448 saturating to +-448; the sign is kept (a negative
 *             v that rounds to zero gives -0, code 0x80)
 *   int8:     q = v rounded to the nearest integer, ties to even, clamped
 *             to [-127, 127]
 *
 * The scale and v are computed in binary32 because that is the precision in
 * which the kernel takes the same decisions; the rounding of v to a code is
 * done here by searching the exact decoded values, not by bit tricks.
 * Inputs must be finite.
 */
enum { ODQ_FP8_TOKEN = 0, ODQ_INT8_TOKEN = 1, ODQ_FP8_BLOCK = 2 };

/* E4M3FN code nearest to v (RNE, saturating, sign kept). */
uint8_t oracle_f32_to_e4m3_rne(float v) {
    static double val[127]; /* values of the positive finite codes 0x00..0x7E */
    static int init = 0;
    if (!init) {
        for (int c = 0; c < 127; ++c) val[c] = oracle_e4m3_to_f64((uint8_t)c);
        init = 1;
    }
    const uint8_t sign = signbit(v) ? 0x80 : 0x00;
    const double a = fabs((double)v);
    int c;
    if (a >= val[126]) {
        c = 126;
    } else {
        int lo = 0; /* largest code with val <= a */
        while (lo + 1 < 127 && val[lo + 1] <= a) ++lo;
        const double dlo = a - val[lo], dhi = val[lo + 1] - a; /* both exact */
        if (dlo < dhi) c = lo;
        else if (dhi < dlo) c = lo + 1;
        else c = (lo & 1) ? lo + 1 : lo; /* tie: the even mantissa */
    }
    return (uint8_t)(sign | c);
}

int oracle_dynamic_quant(const uint16_t *X, int64_t M, int64_t K, int x_fp16, int kind,
                         void *Q, float *scales) {
    if (!X || !Q || !scales || M < 0 || K < 1 || kind < 0 || kind > 2) return O_BAD_ARG;
    if (kind == ODQ_FP8_BLOCK && K % 128) return O_BAD_ARG;
    tables_init();
    const int64_t glen = kind == ODQ_FP8_BLOCK ? 128 : K; /* group length */
    const int64_t ngroups = M * (K / glen);
    const float qmax = kind == ODQ_INT8_TOKEN ? 127.0f : 448.0f;
    for (int64_t gi = 0; gi < ngroups; ++gi) {
        const int64_t base = gi * glen; /* groups tile each row in order */
        float amax = 0.0f;
        for (int64_t k = 0; k < glen; ++k) {
            const float x = (float)dec16(x_fp16 ? OQ_FP16 : OQ_BF16, X[base + k]);
            if (fabsf(x) > amax) amax = fabsf(x);
        }
        const float s = amax > 0.0f ? amax / qmax : 1.0f;
        scales[gi] = s;
        for (int64_t k = 0; k < glen; ++k) {
            const float x = (float)dec16(x_fp16 ? OQ_FP16 : OQ_BF16, X[base + k]);
            const float v = x / s;
            if (kind == ODQ_INT8_TOKEN) {
                float r = rintf(v);
                if (r > 127.0f) r = 127.0f;
                if (r < -127.0f) r = -127.0f;
                ((int8_t *)Q)[base + k] = (int8_t)r;
            } else {
                ((uint8_t *)Q)[base + k] = oracle_f32_to_e4m3_rne(v);
            }
        }
    }
    return O_OK;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
