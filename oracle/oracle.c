/*
 * CPU oracle for the decode-step matrix-vector product y = W·x with Q8_0
 * block-quantized weights and with bf16 or f16 weights.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the plain, slow, obviously correct
 * statement of what the GPU path must compute. Only the test suite, the smoke
 * check and the CPU-baseline leg of the benchmark may build, load or call it.
 * It shares no code, header, table or helper with the HIP library, and it
 * includes nothing but the C standard library and POSIX threads.
 *
 * Sources (cited by page title and section):
 *   [P]  "Filling in the blanks: Inference using Phobos", section "Fast Decode":
 *        a decode step touches each weight exactly once, for one fused
 *        multiply-add (two flops) per weight; a Q8_0 block is 32 int8 values that carry their own scale; the
 *        block products and sums stay in int8/int32 (4-way int8 dot); one
 *        quantization of an activation serves all its consumers; projections of
 *        one input run as one launch; the matmul also adds the residual.
 *   [H]  "One level down: #002 the same compiler on a GPU", sections "Emitting
 *        for a GPU" (the bf16 gate+up matvec, rows of 16-byte chunks; at
 *        decode the normalization and the activation are each fused with the
 *        projection after them), "The numerical contract" (bf16 weights and
 *        activations, f32 accumulators) and "The bench" (the same engine in f16).
 *   [P]  section "Q4_K_M" also names a block's RMS normalization and gated MLP;
 *        section "PrismML Ternary-Bonsai" the PTQ1_0 ternary format (128
 *        weights in 28 bytes, a Hadamard-rotated activation shared by the
 *        projections that read it; its footnote 11 names the rotation's origin).
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - weight and activation block scales are IEEE binary16;
 *   - the activation block scale is d = fl32(max|x| / 127); the codes are
 *     q = rint(fl32(x / d)) with ties to even, using the f32 d, and the stored
 *     scale is binary16(d) rounded to nearest even; an all-zero block gets
 *     d = 0, q = 0;
 *   - the residual is added once, after the whole dot;
 *   - a small batch is the Q8_0 GEMV once per activation vector;
 *   - RMS normalization: h = fl32(fl32(x * r) * gamma) with r = 1/sqrt(ss/K +
 *     eps) formed in f64 and rounded once to f32, ss = sum of x^2 in f64;
 *   - gated activation: a = silu(gate) * up = gate * up / (1 + exp(-gate)),
 *     formed in f64 and rounded once to f32.
 *   - PTQ1_0: the block layout, rotation and activation blocking stated at the
 *     PTQ1_0 section below.
 *
 * Precision: every Q8_0 block term isum·dw·dx is exact in f64 (20 + 11 + 11
 * significant bits); every bf16 product is exact in f64 (8 + 8 bits), every
 * f16 product too (11 + 11 bits). Sums are
 * taken in f64 in ascending index order. The quantizer works in f32, the
 * precision in which the method takes that integer decision.
 *
 * Parity pins (all in tests/test_oracle.py): the binary16 and bf16 decoders
 * against numpy's own casts over all 65536 bit patterns; the binary16 encoder
 * against numpy's cast; the quantizer against an independent numpy float32
 * quantizer and against closed forms (constant, one-hot, zero and tie
 * blocks); the block integer sums against Python-integer brute force and
 * closed forms; the GEMVs against exact rational arithmetic on tiny shapes,
 * against a numpy f64 matmul of the dequantized operands, and against closed
 * forms and invariants; the batched GEMV against an exact integer matmul at
 * unit scales and vector by vector against the single-vector GEMV; the RMS
 * normalization against an exactly rounded sum of squares (math.fsum) and
 * closed forms (constant vectors, scale invariance, gamma linearity, eps
 * dominating); the gated activation against an independent numpy f64
 * evaluation and closed forms (zero gate or up, saturated gates, the
 * silu(g) - silu(-g) = g identity). tests/test_oracle_mutants.py plants
 * mistakes in copies of this file; each must fail a pin.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>

#define ORC_QBLOCK 32

/* ---- number formats -------------------------------------------------------
 * IEEE 754 binary16: sign (1 bit), biased exponent e (5 bits, bias 15),
 * fraction f (10 bits). e = 0: subnormal, value f·2^-24. e = 31: inf / NaN.
 * Otherwise (1024 + f)·2^(e - 25).
 */
double orc_f16_value(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return sign ? -v : v;
}

/* bf16: the upper half of an IEEE binary32. Sign (1), biased exponent e
 * (8 bits, bias 127), fraction f (7 bits). e = 0: subnormal f·2^-133.
 * e = 255: inf / NaN. Otherwise (128 + f)·2^(e - 134). */
double orc_bf16_value(uint16_t u)
{
    int sign = (u >> 15) & 1;
    int e = (u >> 7) & 0xff;
    int f = u & 0x7f;
    double v;
    if (e == 0)
        v = ldexp((double)f, -133);
    else if (e == 255)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + f), e - 134);
    return sign ? -v : v;
}

/* Round a binary32 value to binary16 bits, to nearest with ties to even.
 * The value is exact in double; scaling by a power of two is exact, and
 * nearbyint() rounds to nearest even in the default rounding mode. */
uint16_t orc_f32_to_f16(float value)
{
    double a = fabs((double)value);
    uint16_t sign = signbit(value) ? 0x8000 : 0;
    if (isnan(value))
        return (uint16_t)(sign | 0x7e00);
    if (a >= 65520.0) /* half-way between 65504 and 2^16 rounds (to even) up */
        return (uint16_t)(sign | 0x7c00);
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: quantum 2^-24; a result of 1024 is the smallest
         * normal, whose encoding is the same integer */
        double q = nearbyint(ldexp(a, 24));
        return (uint16_t)(sign | (uint16_t)q);
    }
    int ex;
    frexp(a, &ex);        /* a = m·2^ex, m in [0.5, 1): a in [2^(ex-1), 2^ex) */
    int E = ex - 1;       /* unbiased exponent, -14..15 */
    double q = nearbyint(ldexp(a, 10 - E)); /* significand in units of 2^(E-10): 1024..2048 */
    /* q == 2048 carries into the exponent field, which the addition does */
    return (uint16_t)(sign | (uint16_t)(((E + 15) << 10) + ((int)q - 1024)));
}

/* ---- activation quantization ([P] Fast Decode: quantize an activation once
 * into the same block format as the weights) ------------------------------ */
void orc_quantize_blocks(const float *x, int64_t K, int64_t block, int8_t *qx, uint16_t *dx)
{
    for (int64_t b = 0; b < K / block; ++b) {
        const float *xb = x + b * block;
        float amax = 0.0f;
        for (int64_t i = 0; i < block; ++i) {
            float a = fabsf(xb[i]);
            if (a > amax)
                amax = a;
        }
        float d = amax / 127.0f;
        if (d == 0.0f) {
            for (int64_t i = 0; i < block; ++i)
                qx[b * block + i] = 0;
            dx[b] = 0;
            continue;
        }
        for (int64_t i = 0; i < block; ++i) {
            float t = xb[i] / d;
            float r = rintf(t);
            if (r > 127.0f)
                r = 127.0f;
            if (r < -127.0f)
                r = -127.0f;
            qx[b * block + i] = (int8_t)r;
        }
        dx[b] = orc_f32_to_f16(d);
    }
}

/* Q8_0: blocks of 32 values */
void orc_quantize_act(const float *x, int64_t K, int8_t *qx, uint16_t *dx)
{
    orc_quantize_blocks(x, K, ORC_QBLOCK, qx, dx);
}

/* ---- neighbour steps folded into a projection's prologue ([H] Emitting for a
 * GPU: for decode, two kernels each merge a neighbour step into the next
 * projection, one the normalization and one the activation; [P] Q4_K_M: a norm used inside
 * the fused kernels). The pages name these steps without formulas; the
 * readings here are the standard ones of the models the pages run.
 *
 * RMS normalization: h_i = (x_i * r) * gamma_i in f32, r = f32(1 / sqrt(ss/K
 * + eps)) with ss = sum x_i^2 and r's expression in f64 (each f32 square is
 * exact in f64). The f32 vector h is then quantized by orc_quantize_act. */
void orc_rmsnorm(const float *x, const float *gamma, float eps, int64_t K, float *h)
{
    double ss = 0.0;
    for (int64_t i = 0; i < K; ++i)
        ss += (double)x[i] * (double)x[i];
    const float r = (float)(1.0 / sqrt(ss / (double)K + (double)eps));
    for (int64_t i = 0; i < K; ++i) {
        const float t = x[i] * r;
        h[i] = t * gamma[i];
    }
}

/* Gated activation of the MLP: gu holds gate (first K values) then up (next
 * K); a_i = silu(gate_i) * up_i = gate_i * up_i / (1 + exp(-gate_i)), in f64,
 * rounded once to f32. */
void orc_silu_mul(const float *gu, int64_t K, float *a)
{
    for (int64_t i = 0; i < K; ++i) {
        const double g = (double)gu[i], u = (double)gu[K + i];
        a[i] = (float)((g * u) / (1.0 + exp(-g)));
    }
}

/* ---- block integer dot ([P] Fast Decode: block products and sums kept in integers) */
void orc_block_isums(const int8_t *qw, const int8_t *qx, int64_t N, int64_t K, int32_t *isum)
{
    int64_t nb = K / ORC_QBLOCK;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t b = 0; b < nb; ++b) {
            int32_t s = 0;
            for (int i = 0; i < ORC_QBLOCK; ++i)
                s += (int32_t)qw[n * K + b * ORC_QBLOCK + i] * (int32_t)qx[b * ORC_QBLOCK + i];
            isum[n * nb + b] = s;
        }
}

/* ---- Q8_0 GEMV: y[n] = sum_b isum[n][b]·f16(dw[n][b])·f16(dx[b]) (+ r[n]).
 * S[n] = sum over elements of |w·x| with w, x dequantized (+ |r[n]|): the
 * magnitude the tolerance is relative to. ----------------------------------- */
void orc_q8_gemv(const int8_t *qw, const uint16_t *dw, const int8_t *qx, const uint16_t *dx,
                 const float *residual, int64_t N, int64_t K, double *y, double *S)
{
    int64_t nb = K / ORC_QBLOCK;
    for (int64_t n = 0; n < N; ++n) {
        double acc = 0.0, mag = 0.0;
        for (int64_t b = 0; b < nb; ++b) {
            int32_t s = 0, sa = 0;
            for (int i = 0; i < ORC_QBLOCK; ++i) {
                int32_t p = (int32_t)qw[n * K + b * ORC_QBLOCK + i] * (int32_t)qx[b * ORC_QBLOCK + i];
                s += p;
                sa += p < 0 ? -p : p;
            }
            double scale = orc_f16_value(dw[n * nb + b]) * orc_f16_value(dx[b]);
            acc += (double)s * scale;
            mag += (double)sa * fabs(scale);
        }
        if (residual) {
            acc += (double)residual[n];
            mag += fabs((double)residual[n]);
        }
        y[n] = acc;
        S[n] = mag;
    }
}

/* ---- bf16 GEMV ([H] The numerical contract): y[n] = sum_k bf(w[n][k])·bf(x[k])
 * (+ r[n]); S[n] = sum_k |bf(w)·bf(x)| (+ |r[n]|). ------------------------- */
void orc_bf16_gemv(const uint16_t *w, const uint16_t *x, const float *residual, int64_t N,
                   int64_t K, double *y, double *S)
{
    for (int64_t n = 0; n < N; ++n) {
        double acc = 0.0, mag = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double p = orc_bf16_value(w[n * K + k]) * orc_bf16_value(x[k]);
            acc += p;
            mag += fabs(p);
        }
        if (residual) {
            acc += (double)residual[n];
            mag += fabs((double)residual[n]);
        }
        y[n] = acc;
        S[n] = mag;
    }
}

/* ---- f16 GEMV ([H] The bench: the same engine in f16): y[n] =
 * sum_k f16(w[n][k])·f16(x[k]) (+ r[n]); each product exact in f64. --------- */
void orc_f16_gemv(const uint16_t *w, const uint16_t *x, const float *residual, int64_t N, int64_t K,
                  double *y, double *S)
{
    for (int64_t n = 0; n < N; ++n) {
        double acc = 0.0, mag = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double p = orc_f16_value(w[n * K + k]) * orc_f16_value(x[k]);
            acc += p;
            mag += fabs(p);
        }
        if (residual) {
            acc += (double)residual[n];
            mag += fabs((double)residual[n]);
        }
        y[n] = acc;
        S[n] = mag;
    }
}

/* ---- small-batch Q8_0 GEMV: B activation vectors against one weight matrix.
 * By definition this is the Q8_0 GEMV once per vector b ([P] Fast Decode: the
 * per-token product; a batch only lets one weight pass serve B tokens):
 * qx int8 [B][K], dx [B][K/32], residual f32 [B][N] or NULL, y and S [B][N]. */
void orc_q8_gemv_batch(const int8_t *qw, const uint16_t *dw, const int8_t *qx, const uint16_t *dx,
                       const float *residual, int64_t N, int64_t K, int64_t B, double *y, double *S)
{
    int64_t nb = K / ORC_QBLOCK;
    for (int64_t b = 0; b < B; ++b)
        orc_q8_gemv(qw, dw, qx + b * K, dx + b * nb, residual ? residual + b * N : NULL, N, K, y + b * N,
                    S + b * N);
}

/* ---- PTQ1_0 ternary blocks ([P] PrismML Ternary-Bonsai: weights -1, 0 or +1;
 * 128 weights in 28 bytes; a Hadamard rotation of the activation, which evens out
 * large values across each block; one rotation per input serves every projection
 * that consumes that input). The pages give no byte
 * layout; the readings (listed in the design notes) are:
 *   - a block is 26 bytes of base-3 digits followed by its binary16 scale s
 *     (2 bytes, little-endian); weight i (0..127) of the block is
 *     s * (digit_i - 1), digit_i being digit i % 5, least significant first, of
 *     byte i / 5 (byte 25 holds weights 125..127); a row is K/128 blocks;
 *   - the rotation of each 128-value block of x is H x / sqrt(128), H the
 *     Sylvester-ordered Hadamard matrix, H[i][j] = (-1)^popcount(i & j); each
 *     output is the f64 sum over j in ascending order, divided by sqrt(128) in
 *     f64 and rounded once to f32;
 *   - the rotated activation is quantized with the quantizer above in blocks
 *     of 128 values, one scale per weight block;
 *   - y[n] = sum_b isum(n, b) * f16(s[n][b]) * f16(dx[b]) (+ r[n]), with
 *     isum(n, b) = sum_i t[n][128b + i] * q[128b + i] exact (|isum| <= 16256);
 *     every term is exact in f64 (14 + 11 + 11 significant bits). */
#define ORC_PTQ1_BLOCK 128
#define ORC_PTQ1_BYTES 28
#define ORC_PTQ1_TRIT_BYTES 26

/* binary16 scale bits of the block at blk (little-endian, after the trits) */
uint16_t orc_ptq1_scale(const uint8_t *blk)
{
    return (uint16_t)(blk[ORC_PTQ1_TRIT_BYTES] | (blk[ORC_PTQ1_TRIT_BYTES + 1] << 8));
}

/* trit (-1, 0, +1) of weight i of the block at blk */
int orc_ptq1_trit(const uint8_t *blk, int i)
{
    int v = blk[i / 5];
    for (int k = 0; k < i % 5; ++k)
        v /= 3;
    return v % 3 - 1;
}

/* the blocks' trits and scale bits, for checking the packing */
void orc_ptq1_decode(const uint8_t *w, int64_t nblocks, int8_t *t, uint16_t *s)
{
    for (int64_t b = 0; b < nblocks; ++b) {
        const uint8_t *blk = w + b * ORC_PTQ1_BYTES;
        for (int i = 0; i < ORC_PTQ1_BLOCK; ++i)
            t[b * ORC_PTQ1_BLOCK + i] = (int8_t)orc_ptq1_trit(blk, i);
        s[b] = orc_ptq1_scale(blk);
    }
}

static int orc_parity(unsigned v)
{
    int p = 0;
    for (; v; v >>= 1)
        p ^= (int)(v & 1u);
    return p;
}

void orc_hadamard128(const float *x, int64_t K, float *out)
{
    const double norm = sqrt((double)ORC_PTQ1_BLOCK);
    for (int64_t b = 0; b < K / ORC_PTQ1_BLOCK; ++b)
        for (int i = 0; i < ORC_PTQ1_BLOCK; ++i) {
            double acc = 0.0;
            for (int j = 0; j < ORC_PTQ1_BLOCK; ++j) {
                const double v = (double)x[b * ORC_PTQ1_BLOCK + j];
                acc += orc_parity((unsigned)(i & j)) ? -v : v;
            }
            out[b * ORC_PTQ1_BLOCK + i] = (float)(acc / norm);
        }
}

/* the activation of a PTQ1_0 projection: rotated, then quantized per 128 values */
void orc_ptq1_activation(const float *x, int64_t K, float *rot, int8_t *qx, uint16_t *dx)
{
    orc_hadamard128(x, K, rot);
    orc_quantize_blocks(rot, K, ORC_PTQ1_BLOCK, qx, dx);
}

void orc_ptq1_gemv(const uint8_t *w, const int8_t *qx, const uint16_t *dx, const float *residual, int64_t N,
                   int64_t K, double *y, double *S)
{
    const int64_t nb = K / ORC_PTQ1_BLOCK;
    for (int64_t n = 0; n < N; ++n) {
        double acc = 0.0, mag = 0.0;
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t *blk = w + (n * nb + b) * ORC_PTQ1_BYTES;
            int32_t s = 0, sa = 0;
            for (int i = 0; i < ORC_PTQ1_BLOCK; ++i) {
                int32_t p = (int32_t)orc_ptq1_trit(blk, i) * (int32_t)qx[b * ORC_PTQ1_BLOCK + i];
                s += p;
                sa += p < 0 ? -p : p;
            }
            double scale = orc_f16_value(orc_ptq1_scale(blk)) * orc_f16_value(dx[b]);
            acc += (double)s * scale;
            mag += (double)sa * fabs(scale);
        }
        if (residual) {
            acc += (double)residual[n];
            mag += fabs((double)residual[n]);
        }
        y[n] = acc;
        S[n] = mag;
    }
}

/* ---- row-partitioned threading (same per-row arithmetic, so identical
 * results to the single-threaded calls) ------------------------------------ */
typedef struct {
    int bf16; /* 0: Q8_0, 1: bf16, 2: f16, 3: PTQ1_0 */
    const void *w;
    const uint16_t *dw;
    const void *x;
    const uint16_t *dx;
    const float *residual;
    int64_t n0, n1, K;
    double *y, *S;
} orc_job;

static void *orc_run_job(void *arg)
{
    orc_job *j = (orc_job *)arg;
    int64_t rows = j->n1 - j->n0;
    if (rows <= 0)
        return NULL;
    const float *r = j->residual ? j->residual + j->n0 : NULL;
    if (j->bf16 == 1)
        orc_bf16_gemv((const uint16_t *)j->w + j->n0 * j->K, (const uint16_t *)j->x, r, rows, j->K,
                      j->y + j->n0, j->S + j->n0);
    else if (j->bf16 == 2)
        orc_f16_gemv((const uint16_t *)j->w + j->n0 * j->K, (const uint16_t *)j->x, r, rows, j->K,
                     j->y + j->n0, j->S + j->n0);
    else if (j->bf16 == 3)
        orc_ptq1_gemv((const uint8_t *)j->w + j->n0 * (j->K / ORC_PTQ1_BLOCK) * ORC_PTQ1_BYTES,
                      (const int8_t *)j->x, j->dx, r, rows, j->K, j->y + j->n0, j->S + j->n0);
    else
        orc_q8_gemv((const int8_t *)j->w + j->n0 * j->K, j->dw + j->n0 * (j->K / ORC_QBLOCK),
                    (const int8_t *)j->x, j->dx, r, rows, j->K, j->y + j->n0, j->S + j->n0);
    return NULL;
}

static int orc_run_threads(orc_job proto, int64_t N, int nthreads)
{
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 1024)
        nthreads = 1024;
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    orc_job *jobs = (orc_job *)calloc((size_t)nthreads, sizeof(orc_job));
    if (!th || !jobs) {
        free(th);
        free(jobs);
        return -1;
    }
    int started = 0, rc = 0;
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = proto;
        jobs[t].n0 = N * t / nthreads;
        jobs[t].n1 = N * (t + 1) / nthreads;
        if (pthread_create(&th[t], NULL, orc_run_job, &jobs[t]) != 0) {
            orc_run_job(&jobs[t]);
            rc = 1;
            th[t] = 0;
        } else {
            ++started;
        }
    }
    for (int t = 0; t < nthreads; ++t)
        if (th[t])
            pthread_join(th[t], NULL);
    free(th);
    free(jobs);
    (void)started;
    return rc;
}

int orc_q8_gemv_mt(const int8_t *qw, const uint16_t *dw, const int8_t *qx, const uint16_t *dx,
                   const float *residual, int64_t N, int64_t K, double *y, double *S, int nthreads)
{
    orc_job p = {0, qw, dw, qx, dx, residual, 0, 0, K, y, S};
    return orc_run_threads(p, N, nthreads);
}

int orc_bf16_gemv_mt(const uint16_t *w, const uint16_t *x, const float *residual, int64_t N,
                     int64_t K, double *y, double *S, int nthreads)
{
    orc_job p = {1, w, NULL, x, NULL, residual, 0, 0, K, y, S};
    return orc_run_threads(p, N, nthreads);
}

int orc_f16_gemv_mt(const uint16_t *w, const uint16_t *x, const float *residual, int64_t N,
                    int64_t K, double *y, double *S, int nthreads)
{
    orc_job p = {2, w, NULL, x, NULL, residual, 0, 0, K, y, S};
    return orc_run_threads(p, N, nthreads);
}

int orc_ptq1_gemv_mt(const uint8_t *w, const int8_t *qx, const uint16_t *dx, const float *residual, int64_t N,
                     int64_t K, double *y, double *S, int nthreads)
{
    orc_job p = {3, w, NULL, qx, dx, residual, 0, 0, K, y, S};
    return orc_run_threads(p, N, nthreads);
}
