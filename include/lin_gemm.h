/*
 * lin_gemm.h -- C ABI of the MI355X (gfx950) scaled linear layer with a fused
 * epilogue.
 *
 *   C[m,n] = act( s(m,n) * sum_k A[m,k] * B[n,k]  +  bias[n] ) * alpha
 *            + residual[m,n]
 *
 * where s(m,n) is 1 (bf16 / fp16), sa[m] * sb[n] (FP8 dynamic, W8A8 int8),
 * or applied per 128-wide K block as sa[m,kb] * sb[n/128,kb] (block FP8).
 * Bias, activation, alpha, residual and the narrowing to a 16-bit float all
 * happen on the fp32 (or int32) accumulator in registers, before the one
 * store of C; no intermediate tensor is written to device memory.
 *
 * Sources, restated:
 *  - "Совместная работа Helion и TorchInductor: слияние операторов"
 *    (gurufy.ru): the epilogue-fusion section (bias, residual, GELU/SiLU and
 *    the fp32 -> 16-bit narrowing applied to the accumulator before the
 *    store), the extensible-epilogue kernel listing (fp32 accumulator over
 *    the K loop; bias broadcast over rows; activation code 1 = ReLU,
 *    2 = GELU in its tanh form; masked 16-bit store) and the custom-op
 *    wrapper in the TorchInductor-integration section (checks the inner
 *    dimension, allocates the output, launches one kernel over a ceil-div
 *    grid).
 *  - "helion-vllm-linear-backend" (aixai.ru): the scaled-GEMM formats of the
 *    section "Одно ядро вместо трёх вариантов" (FP8_Dynamic per-token x
 *    per-channel, W8A8_INT8 with the same scaling, Block_FP8 with 1x128
 *    activation and 128x128 weight scale blocks) and the split-K / swap-AB
 *    variants for small M of the section "Зачем трогать линейные слои",
 *    chosen per shape from a table (sections "Одно ядро вместо трёх
 *    вариантов" and "Гибридный диспатч").
 *
 * Layouts.  All matrices and scale arrays are dense, row-major, contiguous
 * and 16-byte aligned device memory owned by the caller:
 *   A        [M][K]  bf16 | fp16 | e4m3 (OCP E4M3FN) | int8, per quant mode
 *   B        [N][K]  same element type as A (the weight, K contiguous)
 *   bias     [N]     bf16 (fp16 in LIN_Q_FP16), or NULL
 *   residual [M][N]  bf16 (fp16 in LIN_Q_FP16), or NULL
 *   C        [M][N]  bf16 (fp16 in LIN_Q_FP16); with LIN_ACT_RAW_ACC:
 *                    int32 (LIN_Q_W8A8_INT8) or fp32 (other modes)
 *   scales->a  fp32 [M] (FP8 dynamic, int8) or [M][K/128] (block FP8)
 *   scales->b  fp32 [N] (FP8 dynamic, int8) or [N/128][K/128] (block FP8)
 *
 * LIN_Q_MXFP4 (4-bit weights; the pages list INT4 / NVFP4 weight formats in
 * "helion-vllm-linear-backend", section "Зачем трогать линейные слои", and
 * define none, so the gfx950-native OCP MX v1.0 MXFP4 format is used): A is
 * bf16 [M][K]; B is [N][K/2] bytes, two E2M1 codes per byte, the even K
 * index in the low nibble; scales->b points to E8M0 bytes [N][K/32] (one
 * power-of-two scale 2^(e-127) per 32 consecutive K values of a row, codes
 * 1..254) and scales->a is unused.  K % 256 == 0; any M (decode kernels up
 * to 32 tokens, tile kernels beyond).  C = act(sum_k A[m,k] * e2m1(B[n,k]) *
 * 2^(e[n,k/32]-127) + bias) * alpha + residual, in bf16.
 *
 * Streams and errors.  lin_gemm_run enqueues on `stream` (a hipStream_t;
 * NULL = the null stream) and returns without waiting.  The status it
 * returns covers argument checks and launch errors only; a fault inside a
 * kernel surfaces at the next synchronisation.  Nothing throws across this
 * ABI.  lin_gemm_last_error() gives a human-readable detail for the last
 * failing call on a handle.
 *
 * Handles.  A handle owns its split-K workspace and arrival counters
 * (device memory, grown on demand, freed by lin_gemm_destroy) and the
 * shape-keyed variant table.  Calls that share a handle must not run
 * concurrently on different streams (they share the workspace); use one
 * handle per stream.  Warm each shape up once before capturing calls into a
 * hipGraph, so no allocation happens during capture.  A buffer that grows
 * is replaced, not freed: the old one stays allocated until
 * lin_gemm_destroy, so graphs captured before the growth remain valid.
 */
#ifndef LIN_GEMM_H
#define LIN_GEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct lin_gemm_ctx *lin_gemm_t;

/* Quant modes (the formats of the linear-backend write-up, plus plain
 * 16-bit floats). */
enum lin_quant {
    LIN_Q_BF16 = 0,
    LIN_Q_FP16 = 1,
    LIN_Q_FP8_DYNAMIC = 2, /* e4m3 A, B; sa per token [M], sb per channel [N] */
    LIN_Q_W8A8_INT8 = 3,   /* int8 A, B; same scaling; int32 accumulator     */
    LIN_Q_BLOCK_FP8 = 4,   /* e4m3; sa [M][K/128], sb [N/128][K/128]         */
    LIN_Q_MXFP4 = 5        /* bf16 A; 4-bit B with E8M0 block scales (below) */
};

/* Activations.  1 and 2 keep the codes of the epilogue listing. */
enum lin_act {
    LIN_ACT_NONE = 0,
    LIN_ACT_RELU = 1,
    LIN_ACT_GELU_TANH = 2,  /* 0.5 y (1 + tanh(sqrt(2/pi) (y + 0.044715 y^3))) */
    LIN_ACT_SILU = 3,       /* y / (1 + exp(-y)) */
    LIN_ACT_RAW_ACC = 255   /* test hook: store the raw accumulator (int32 for
                               int8, fp32 otherwise); no scales, no epilogue */
};

enum lin_status {
    LIN_OK = 0,
    LIN_ERR_INVALID_ARG = -1, /* null pointer, bad code, negative size       */
    LIN_ERR_UNSUPPORTED = -2, /* valid but outside what the kernels handle   */
    LIN_ERR_HIP = -3,         /* a HIP runtime call failed                   */
    LIN_ERR_OOM = -4,         /* workspace allocation failed                 */
    LIN_ERR_CONFIG = -5       /* variant table file unreadable / malformed   */
};

typedef struct {
    const float *a; /* activation scales (see the layouts above)          */
    const float *b; /* weight scales                                       */
    float alpha;    /* multiplier applied after the activation (1 = none)  */
} lin_scales_t;

/* Create a handle.  config_path names a variant-table file (see
 * lin_gemm_describe for the variant syntax); NULL or "" uses the built-in
 * table, and the environment variable LIN_GEMM_CONFIG, if set, is read when
 * config_path is NULL.  Returns LIN_ERR_CONFIG (and no handle) if a named
 * file cannot be read or parsed. */
int lin_gemm_create(lin_gemm_t *out, const char *config_path);

/* Run one layer call.  scales may be NULL for LIN_Q_BF16 / LIN_Q_FP16
 * (alpha = 1); it and scales->a / scales->b are required for the quantised
 * modes.
 * Requirements (else LIN_ERR_UNSUPPORTED): N >= 1, K >= 1; K % 8 == 0 for
 * bf16/fp16 and K % 16 == 0 for e4m3/int8 (16-byte rows); block FP8 also
 * needs K % 128 == 0 and N % 128 == 0; int8 needs K <= 131071 so that the
 * int32 accumulator cannot overflow (127 * 127 * K < 2^31).  M == 0 is a
 * no-op that returns LIN_OK.  Unknown quant / activation codes, a NULL
 * handle, A, B or C, or negative sizes give LIN_ERR_INVALID_ARG. */
int lin_gemm_run(lin_gemm_t h, const void *A, const void *B, const lin_scales_t *scales,
                 const void *bias, const void *residual, void *C, int64_t M, int64_t N,
                 int64_t K, int quant_mode, int activation, void *stream);

/* lin_gemm_run for callers that cannot allocate device memory: code under
 * hipGraph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, checks, variant choice, kernels and results as
 * lin_gemm_run, but the split-K partials and arrival counters live in a
 * static device array of the library (64 MiB of partials and 65536 counters
 * per device, held from the first such call on a device until the process
 * ends) instead of handle buffers; nothing is allocated or freed, and the
 * handle's own buffers are not touched.  A call whose chosen variant needs
 * more partials or counters than that gets LIN_ERR_UNSUPPORTED before
 * anything is enqueued (lin_gemm_describe names the variant; a forced
 * smaller split, or lin_gemm_run, avoids it).  Counters and the atomic
 * reduction's accumulator are cleared by a fill kernel at the start of each
 * call that uses them.  Every call on a device shares that one array: calls
 * that overlap in time on one device (two streams, two host threads, or a
 * graph replay alongside an eager call) race on it and give wrong results;
 * calls ordered on one stream do not. */
int lin_gemm_run_noalloc(lin_gemm_t h, const void *A, const void *B, const lin_scales_t *scales,
                         const void *bias, const void *residual, void *C, int64_t M, int64_t N,
                         int64_t K, int quant_mode, int activation, void *stream);

/* Release the handle and its device workspace.  NULL is accepted. */
int lin_gemm_destroy(lin_gemm_t h);

/* Static text for a status code. */
const char *lin_gemm_strerror(int status);

/* Detail for the last failing call on h (empty string if none).  The
 * pointer stays valid until the next call on h. */
const char *lin_gemm_last_error(lin_gemm_t h);

/* Force a variant for every following lin_gemm_run on h (testing and the
 * offline sweep); NULL or "" returns to the table.  Spec syntax, e.g.
 *   "tile bm=128 bn=128"   "decode swap=1 split=4 reduce=lastwg waves=4"
 * Returns LIN_ERR_CONFIG if the spec does not parse or names a shape that
 * is not compiled.  A variant that does not apply to a later call's sizes
 * or quant mode (for example a decode shape compiled only with staged
 * activations, forced at a token count those builds do not cover) makes
 * that call fail, with LIN_ERR_UNSUPPORTED and no kernel launched. */
int lin_gemm_set_force(lin_gemm_t h, const char *spec);

/* Write into buf (NUL-terminated, at most buflen bytes) the variant that
 * lin_gemm_run would use for this shape, in the spec syntax above. */
int lin_gemm_describe(lin_gemm_t h, int quant_mode, int64_t M, int64_t N, int64_t K,
                      char *buf, int buflen);

/* The three-kernel unfused path of the decoder-block example (measurement
 * only; bf16 / fp16): T = A*B^T, U = act(T + bias), C = alpha*U + residual,
 * with T and U written to and re-read from the caller's [M][N] buffers.
 * Same requirements as lin_gemm_run in LIN_Q_BF16 / LIN_Q_FP16. */
int lin_gemm_run_unfused(lin_gemm_t h, const void *A, const void *B, const void *bias,
                         const void *residual, void *C, void *T, void *U, int64_t M,
                         int64_t N, int64_t K, float alpha, int quant_mode, int activation,
                         void *stream);

/* Measurement only (like lin_gemm_run_unfused): a plain streaming read of
 * `bytes` bytes of device memory at src, the HBM read rate that the weight
 * stream of a decode call is measured against.  The section "Зачем трогать
 * линейные слои" of "helion-vllm-linear-backend" describes small-M linear
 * layers as bound by reading the weight; this gives the rate a kernel that
 * does nothing but read reaches for the same byte count.  grid workgroups
 * of 256 threads (0 = 1024), each thread keeping `unroll` (4, 8 or 16)
 * 16-byte loads in flight; consecutive threads read consecutive 16-byte
 * chunks.  sink: 256 ints of caller device memory, written only in the
 * practically impossible case that the XOR of the data equals one fixed
 * value.  bytes % 16 == 0, src 16-byte aligned (else LIN_ERR_UNSUPPORTED);
 * bytes == 0 is a no-op.  Enqueued on `stream`; no allocation. */
int lin_gemm_stream_read(lin_gemm_t h, const void *src, int64_t bytes, int grid, int unroll,
                         int *sink, void *stream);

/* Dynamic activation quantization: the step that produces A and the
 * activation scales of the quantised modes from 16-bit activations at run
 * time.  "helion-vllm-linear-backend", section "Одно ядро вместо трёх
 * вариантов": per-token scales for FP8_Dynamic and W8A8_INT8, 1x128
 * activation blocks for Block_FP8; the prologue/epilogue section of
 * "Совместная работа Helion и TorchInductor" counts quantization among the
 * input-side transforms.  For each group g (a row, or a 1x128 block of a
 * row):  s_g = max|x| / QMAX in binary32 (QMAX = 448 for e4m3, 127 for
 * int8; s_g = 1 if the group is all zero), and code = x / s_g (binary32,
 * correctly rounded) rounded to nearest, ties to even, saturated to
 * [-QMAX, QMAX].  Inputs must be finite (NaN / Inf give unspecified codes). */
enum lin_dq_kind {
    LIN_DQ_FP8_TOKEN = 0,  /* e4m3 codes, scales [M]        (LIN_Q_FP8_DYNAMIC) */
    LIN_DQ_INT8_TOKEN = 1, /* int8 codes, scales [M]        (LIN_Q_W8A8_INT8)   */
    LIN_DQ_FP8_BLOCK = 2   /* e4m3 codes, scales [M][K/128] (LIN_Q_BLOCK_FP8)   */
};

/* Quantize X[M][K] (bf16 if x_dtype == LIN_Q_BF16, fp16 if LIN_Q_FP16) into
 * Q[M][K] (one byte per value) and scales (fp32, layout per kind).  All
 * three are caller-owned device buffers, 16-byte aligned.  K must be a
 * positive multiple of 16 (of 128 for LIN_DQ_FP8_BLOCK), else
 * LIN_ERR_UNSUPPORTED; M == 0 is a no-op.  Enqueued on `stream`; no
 * allocation. */
int lin_gemm_quantize(lin_gemm_t h, const void *X, int x_dtype, int64_t M, int64_t K, int kind,
                      void *Q, float *scales, void *stream);

/* The layer on 16-bit activations X[M][K], quantized on the fly as
 * lin_gemm_quantize does.  quant_mode is LIN_Q_FP8_DYNAMIC, LIN_Q_W8A8_INT8
 * or LIN_Q_BLOCK_FP8 (else LIN_ERR_INVALID_ARG); sb is the weight scale
 * array of that mode; other arguments and requirements as in lin_gemm_run.
 * For bf16 X and up to 16 tokens, when the shape's decode variant asks for
 * the quantization prologue ("dq=1" in the variant spec) and its LDS fits,
 * one kernel does both: the workgroup quantizes X into LDS and the K loop
 * reads the codes from there (the prologue fusion of the input-side
 * transforms the pages describe).  Otherwise lin_gemm_quantize runs into
 * handle-owned staging (grown on demand, like the split-K workspace) and
 * lin_gemm_run follows.  Both forms give the same codes and scales, and the
 * same output bits for the same variant. */
int lin_gemm_run_dynamic(lin_gemm_t h, const void *X, int x_dtype, const void *B,
                         const float *sb, float alpha, const void *bias, const void *residual,
                         void *C, int64_t M, int64_t N, int64_t K, int quant_mode,
                         int activation, void *stream);

/* Grouped layer for a mixture of experts: E experts, the M token rows
 * sorted by expert, expert x owning rows [offsets[x], offsets[x+1]) of A,
 * residual and C, each multiplied by its own weight with its own scales and
 * bias -- every segment is exactly lin_gemm_run on its rows with its
 * expert's operands.  "helion-vllm-linear-backend" names a mixture-of-experts
 * backend among its next steps (section "Что дальше") and defines
 * none; this is the plain reading: a grouped product with per-expert
 * weights, the per-token scales following their rows.
 * Layouts (dense, contiguous, caller-owned device memory, 16-byte aligned):
 *   A, residual, C, scales->a  as lin_gemm_run with M rows in expert order
 *   B         [E][N][K] (per quant mode; [E][N][K/2] bytes for MXFP4)
 *   scales->b [E][N] (FP8 dynamic, int8), [E][N/128][K/128] (block FP8),
 *             [E][N][K/32] E8M0 bytes (MXFP4)
 *   bias      [E][N] or NULL
 *   offsets   int32 [E+1] in device memory (4-byte aligned), non-decreasing
 *             from 0 to M.  The kernel reads it: it may be produced on the
 *             same stream just before.  Values are clamped into [0, M] and a
 *             segment whose end is below its start is empty, so a malformed
 *             array gives wrong rows but no out-of-bounds access; rows no
 *             segment covers are left unwritten.
 * max_rows is an upper bound on any expert's row count that the caller
 * knows (0 = M; for top-k routing over distinct experts, the token count).
 * It only shapes the launch, through the typical segment length
 * L = min(max_rows, ceil(M / E)); any segment lengths give the right
 * result.  L <= 4 (decode): the decode kernels (swap orientation, no
 * split-K) run rows in chunks of up to 16 tokens (32 when L > 16), each
 * chunk streaming its expert's weight; the grid holds min(E, M) rows of
 * workgroups, each serving one expert that has rows, and as many chunk
 * slots as a segment of L rows needs, and a workgroup loops over the
 * further chunks of a longer segment; a forced "decode" variant keeps this
 * path for any L.  L > 4: the tile kernels take every 64-row tile (256 when
 * L > 256) of every segment; a forced "tile" variant from
 * lin_gemm_set_force picks 64x128 (1x4 waves), 128x128 (2x2) or 256x256
 * (2x4); its split factor is ignored (grouped launches do not split K).  Requirements: those of lin_gemm_run for N and K per mode
 * (MXFP4: K % 256 == 0; no limit on M), E <= 65535, M < 2^31.  E == 0 or
 * M == 0 is a no-op.  No allocation; enqueued on `stream`. */
int lin_gemm_run_grouped(lin_gemm_t h, const void *A, const void *B, const lin_scales_t *scales,
                         const void *bias, const void *residual, void *C, const int32_t *offsets,
                         int64_t E, int64_t M, int64_t N, int64_t K, int64_t max_rows,
                         int quant_mode, int activation, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LIN_GEMM_H */
