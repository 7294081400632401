/*
 * q8gemv — decode-step matrix-vector products y = W·x on AMD Instinct MI355X
 * (CDNA4, gfx950), for Q8_0 block-quantized weights and for bf16 weights.
 *
 * Sources (by page title and section):
 *   [P] "Filling in the blanks: Inference using Phobos", section "Fast Decode":
 *       a decode step touches each weight exactly once, for one fused
 *       multiply-add (two flops) per weight; a Q8_0 block is 32 int8 values carrying their own scale;
 *       block products and sums stay in integers; one quantization of an
 *       activation serves all its consumers; the projections of one input run
 *       as one launch; the matmul also adds the residual.
 *   [H] "One level down: #002 the same compiler on a GPU", sections "Emitting
 *       for a GPU" (gate and up computed in one go; a weight row read as
 *       16-byte chunks of eight bf16; the last row index guards the tail) and
 *       "The numerical contract" (bf16 weights and activations, f32
 *       accumulators).
 *   [T] "Filling in the blanks: Inference using Phobos", section "PrismML
 *       Ternary-Bonsai": ternary weights (-1, 0, +1), 128 of them in 28 bytes
 *       (PTQ1_0), with the activation rotated by a Hadamard transform, which
 *       evens out large values across the block; one rotation per input
 *       serves every projection that consumes that input.
 *
 * Conventions for every entry point:
 *   - Data pointers are DEVICE pointers owned by the caller. The exceptions
 *     are the `parts` array of gemv_stacked and the descriptors of
 *     q8_decode_stack, host memory read during the call only, and the
 *     weight packing call q8_pack_tile16, which works on host memory.
 *   - `stream` is a hipStream_t (NULL = the null stream). Work is enqueued
 *     asynchronously; nothing is synchronized, allocated or freed, and no
 *     environment variable is read. The library holds no mutable global
 *     state apart from q8_decode_stack_static's per-device workspace, so the
 *     other calls are thread-safe and may be captured into a HIP graph.
 *   - Q8_0 data is stored as two planes: codes int8 [N][K] row-major and scale
 *     bits (IEEE binary16) [N][K/32] row-major; scale b of row n covers codes
 *     32b..32b+31 of that row. A quantized activation is codes int8 [K] plus
 *     binary16 scale bits [K/32].
 *   - bf16 data is the upper 16 bits of an IEEE binary32, stored as uint16.
 *   - All validation happens on the host before anything is enqueued; on any
 *     error nothing is written. N == 0 is a valid empty call (returns Q8G_OK
 *     and enqueues nothing). K == 0 gives y = 0 (+ residual).
 *   - Alignment: weight planes (`qw`, `w`), `qx`, bf16 `x` and f32 `x` need
 *     16-byte alignment; scale planes 2 bytes; `y` and `residual` 4 bytes.
 *   - Aliasing: `y` may be the same pointer as `residual` (each element is read
 *     once, then written once, by the same lane). No other overlap between an
 *     output and any other argument is allowed (Q8G_ERR_OVERLAP).
 *   - NaN or Inf inputs and binary16 overflow of a scale are outside the
 *     contract: results are unspecified but nothing faults.
 */
#ifndef Q8GEMV_H
#define Q8GEMV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    Q8G_OK = 0,
    Q8G_ERR_NULL = 1,    /* a required pointer is NULL */
    Q8G_ERR_SHAPE = 2,   /* negative size, K not a multiple of 32 (Q8_0) or 8 (bf16), size overflow */
    Q8G_ERR_ALIGN = 3,   /* a pointer is not aligned as stated above */
    Q8G_ERR_ARG = 4,     /* bad enum value or part count */
    Q8G_ERR_LAUNCH = 5,  /* the HIP runtime refused the kernel launch */
    Q8G_ERR_OVERLAP = 6  /* an output overlaps an input or another output */
} q8g_status;

/* Q8G_Q8_0_F32: Q8_0 weights with an f32 activation that the launch itself
 * quantizes (exactly as q8_quantize_act) before the dot products; K <= 16384. */
/* Q8G_F16: IEEE binary16 weights and activation, f32 accumulation. */
/* Q8G_PTQ1_0: PTQ1_0 ternary weights against a rotated, quantized activation
 * (see the PTQ1_0 section below). */
typedef enum { Q8G_Q8_0 = 0, Q8G_BF16 = 1, Q8G_Q8_0_F32 = 2, Q8G_F16 = 3, Q8G_PTQ1_0 = 4 } q8g_dtype;

/* Quantize an activation once into the Q8_0 block format ([P] Fast Decode).
 * For each block b of 32 consecutive values of x (f32 [K]):
 *   d = fl32(max_i |x_i| / 127)            (one IEEE f32 division)
 *   d == 0: codes 0, scale bits 0
 *   else:   q_i = rint(fl32(x_i / d))      (round half to even; |q_i| <= 127)
 *           dx[b] = binary16(d)            (round to nearest even, subnormals kept)
 * The f32 d quantizes; the binary16 d is what the dot products use.
 * K % 32 == 0. qx: int8 [K]; dx: uint16 [K/32]. Neither may overlap x. */
q8g_status q8_quantize_act(const float *x, int8_t *qx, uint16_t *dx, int64_t K, void *stream);

/* Q8_0 GEMV ([P] Fast Decode):
 *   isum[n][b] = sum_{i<32} qw[n][32b+i] * qx[32b+i]          (exact int32)
 *   y[n] = sum_b float(isum[n][b]) * (f16(dw[n][b]) * f16(dx[b]))  (f32 accumulate)
 *          (+ residual[n], added once after the dot; residual may be NULL)
 * qw int8 [N][K], dw uint16 [N][K/32], qx int8 [K], dx uint16 [K/32],
 * residual f32 [N] or NULL, y f32 [N]. K % 32 == 0. */
q8g_status q8_gemv(const int8_t *qw, const uint16_t *dw, const int8_t *qx, const uint16_t *dx,
                   const float *residual, float *y, int64_t N, int64_t K, void *stream);

/* bf16 GEMV ([H] The numerical contract):
 *   y[n] = sum_k f32(w[n][k]) * f32(x[k])   (f32 accumulate) (+ residual[n])
 * w uint16 (bf16) [N][K], x uint16 (bf16) [K], residual f32 [N] or NULL,
 * y f32 [N]. K % 8 == 0 (a row is whole 16-byte chunks, [H] Emitting for a GPU). */
q8g_status bf16_gemv(const uint16_t *w, const uint16_t *x, const float *residual, float *y,
                     int64_t N, int64_t K, void *stream);

/* f16 GEMV ([H] The bench: the same engine in f16, where f16 is the native
 * 16-bit format): y[n] = sum_k f32(w[n][k]) * f32(x[k]) (f32 accumulate)
 * (+ residual[n]), w and x IEEE binary16 bits. Every product of two binary16
 * values is exact in f32. Same layout and rules as bf16_gemv. */
q8g_status f16_gemv(const uint16_t *w, const uint16_t *x, const float *residual, float *y,
                    int64_t N, int64_t K, void *stream);

/* Small-batch Q8_0 GEMV: B activation vectors share one pass over the weights.
 * [P] Fast Decode sets the two ends: decode reads each weight once per token
 * (memory-bound), prompt processing reuses each weight once per prompt token
 * and belongs on the matrix units. For 1 <= B <= Q8G_BATCH_MAX, each weight
 * byte read serves B outputs, and the block sums run on the matrix cores:
 *   y[b][n] = sum_blk float(isum(n, b, blk)) * (f16(dw[n][blk]) * f16(dx[b][blk]))
 *             (+ residual[b][n]),   isum(n, b, blk) = sum_{i<32} qw[n][32 blk+i] * qx[b][32 blk+i]
 * i.e. q8_gemv once per vector b. qw int8 [N][K], dw uint16 [N][K/32] as for
 * q8_gemv; qx int8 [B][K] and dx uint16 [B][K/32] row-major (B activations
 * quantized by one q8_quantize_act call over B*K values); residual f32 [B][N]
 * or NULL (may equal y); y f32 [B][N]. K % 32 == 0 and K <= 2^27; B == 0 or
 * N == 0 enqueues nothing; B > Q8G_BATCH_MAX gives Q8G_ERR_SHAPE. The f32 accumulation order
 * differs from q8_gemv's, so results agree with it within the tolerance of the
 * f32 sum, not bit for bit. */
#define Q8G_BATCH_MAX 16
q8g_status q8_gemv_batch(const int8_t *qw, const uint16_t *dw, const int8_t *qx, const uint16_t *dx,
                         const float *residual, float *y, int64_t N, int64_t K, int64_t B, void *stream);

/* ---- weight layout of the small-batch GEMV ----------------------------------
 * [P] GPU Performance Heisenbugs: decode weights stored eight columns side by
 * side, so a warp's loads span full 128-byte lines. Q8G_LAYOUT_ROWS is the plain [N][K]
 * codes and [N][K/32] scales of q8_gemv_batch. Q8G_LAYOUT_TILE16 groups 16 rows:
 *   codes: tile t (rows 16t..16t+15) and step s (columns 64s..64s+63) form one
 *          1024-byte unit at byte (t * S + s) * 1024, S = ceil(K / 64); inside
 *          it, row j's columns 64s + 16c .. 64s + 16c + 15 are the 16 bytes at
 *          16 * (16c + j) (c = 0..3);
 *   scales: block b of tile t holds its 16 rows' binary16 scale bits side by
 *          side at element (t * K/32 + b) * 16 + j;
 *   rows past N (up to the next multiple of 16) and columns past K (up to the
 *   next multiple of 64) are zero. q8_tile16_sizes gives the sizes. */
typedef enum { Q8G_LAYOUT_ROWS = 0, Q8G_LAYOUT_TILE16 = 1 } q8g_layout;

/* q8_gemv_batch with the weights in the given layout (qw, dw device pointers in
 * that layout; every other argument and rule as for q8_gemv_batch). The results
 * are identical, bit for bit, in both layouts: only the weight addresses differ.
 * Q8G_ERR_ARG for an unknown layout. */
q8g_status q8_gemv_batch_layout(int layout, const int8_t *qw, const uint16_t *dw, const int8_t *qx,
                                const uint16_t *dx, const float *residual, float *y, int64_t N, int64_t K, int64_t B,
                                void *stream);

/* Bytes of the Q8G_LAYOUT_TILE16 codes and scales of an N x K matrix (K % 32 == 0).
 * Pure host query. */
q8g_status q8_tile16_sizes(int64_t N, int64_t K, int64_t *code_bytes, int64_t *scale_bytes);

/* Rewrite row-layout Q8_0 weights (qw int8 [N][K], dw uint16 [N][K/32]) into
 * Q8G_LAYOUT_TILE16 (qw_tiled, dw_tiled of the sizes above, padding written as
 * zero). HOST pointers, unlike every other call: weights are packed once, when
 * they are loaded, and then copied to the device. Synchronous; the outputs may
 * not overlap the inputs or each other. */
q8g_status q8_pack_tile16(const int8_t *qw, const uint16_t *dw, int64_t N, int64_t K, int8_t *qw_tiled,
                          uint16_t *dw_tiled);

/* Launch configuration q8_gemv_batch picks for N rows: how many waves split the K
 * range of one 16-row tile, and how many 64-column weight steps each wave keeps
 * in flight. Pure host query; nothing is enqueued. */
q8g_status q8g_batch_config(int64_t N, int *k_split, int *steps_in_flight);

/* Launch form q8_gemv_batch_layout picks for an N x K matrix in the tiled layout
 * whose scales are 16-byte aligned: *streams = 1 when each wave streams whole
 * 16-row tiles back to back with one staging of the activation (more than 2048
 * tiles and K of 8 or 16 64-column steps: 448 < K <= 512 or 960 < K <= 1024),
 * 0 when the launch takes the shape q8g_batch_config reports. Same outputs
 * either way. Pure host query; Q8G_ERR_SHAPE for N < 0, K < 0 or K % 32 != 0,
 * Q8G_ERR_NULL for a null streams. */
q8g_status q8g_batch_tiled_streams(int64_t N, int64_t K, int *streams);

/* One matrix of a stacked projection. */
typedef struct {
    const void *w;         /* Q8_0: int8 codes [n][K]; bf16 / f16: uint16 [n][K];
                              PTQ1_0: blocks uint8 [n][K/128 * 28] */
    const uint16_t *dw;    /* Q8_0: binary16 scale bits [n][K/32]; other kinds: ignored (may be NULL) */
    int64_t n;             /* output rows of this part (>= 0) */
    float *y;              /* f32 [n] */
    const float *residual; /* f32 [n] or NULL; may equal y */
} q8g_part;

/* Stacked projection ([P] Fast Decode: the projections of one input run as
 * one launch; [H] Emitting for a GPU: gate and up in one go). One launch computes
 * every part against the shared input: Q8_0 takes x = int8 codes [K] and
 * dx = binary16 scale bits [K/32]; bf16 and f16 take x = bf16 / f16 [K] and
 * ignore dx;
 * Q8G_Q8_0_F32 takes x = f32 [K] (16-byte aligned, K <= 16384), quantizes it
 * inside the launch, and ignores dx ([P] Fast Decode: one quantization of the
 * activation serves all its consumers; here, all the parts of the launch).
 * Q8G_PTQ1_0 takes x = the rotated codes int8 [K] and dx = binary16 scale
 * bits [K/128] of ptq1_rotate_quantize_act ([T]: one rotation per input for
 * all the projections that consume it), with the rules of ptq1_gemv.
 * Part p's result is identical, bit for bit, to q8_gemv / bf16_gemv /
 * ptq1_gemv called on that part alone (for Q8G_Q8_0_F32: to q8_quantize_act
 * then q8_gemv). 1 <= nparts <= 4. */
q8g_status gemv_stacked(q8g_dtype dtype, const q8g_part *parts, int nparts, const void *x,
                        const uint16_t *dx, int64_t K, void *stream);

/* ---- PTQ1_0 ternary weights ([T]) ----------------------------------------
 * The pages fix the weight values (-1, 0, +1), the block size (128 weights in
 * 28 bytes) and the rotation of the activation by a Hadamard transform; the
 * layout below is this library's reading of the rest.
 * Block (28 bytes, 128 weights):
 *   bytes 0..25  base-3 digits, five per byte, least significant digit first:
 *                weight i (0..127) is digit (i mod 5) of byte floor(i / 5), and
 *                its trit is digit - 1 (byte 25 holds weights 125..127; its
 *                digits 3 and 4 belong to no weight and are ignored);
 *   bytes 26..27 the block scale s, IEEE binary16 bits, little-endian;
 *   weight i of the block = s * trit_i.
 * A row of K weights (K % 128 == 0) is K/128 blocks back to back, rows
 * contiguous: w uint8 [N][K/128 * 28]. */
#define Q8G_PTQ1_BLOCK 128
#define Q8G_PTQ1_BYTES 28
#define Q8G_PTQ1_MAX_K 65536
#define Q8G_PTQ1_MAX_ROWS (1 << 30)

/* Rotate an activation and quantize it for PTQ1_0 weights ([T]: one rotation
 * per input). For each block b of 128 consecutive values of x (f32 [K]):
 *   r_i = fl32( (sum_{j<128} (-1)^popcount(i & j) * x_{128b+j}) / sqrt(128) )
 *         (the sum in f64 in ascending j, sqrt(128) the nearest f64, the
 *         quotient correctly rounded in f64, then rounded once to f32),
 *   then the 128 values r are quantized as q8_quantize_act quantizes a block,
 *   over 128 values instead of 32: d = fl32(max |r| / 127), q_i = rint(fl32(r_i / d)),
 *   dx[b] = binary16(d); d == 0 gives codes 0 and scale bits 0.
 * x f32 [K] (4-byte aligned); rot f32 [K] (4-byte aligned) or NULL: the values r;
 * qx int8 [K]; dx uint16 [K/128]. K % 128 == 0 (K == 0: nothing is enqueued).
 * No output may overlap x or another output. */
q8g_status ptq1_rotate_quantize_act(const float *x, float *rot, int8_t *qx, uint16_t *dx, int64_t K, void *stream);

/* PTQ1_0 GEMV ([T]):
 *   isum[n][b] = sum_{i<128} trit(n, b, i) * qx[128b+i]            (exact int32, |isum| <= 16256)
 *   y[n] = sum_b float(isum[n][b]) * (f16(s[n][b]) * f16(dx[b]))   (f32 accumulate)
 *          (+ residual[n], added once after the dot; residual may be NULL)
 * w uint8 [N][K/128 * 28] (4-byte aligned); qx int8 [K] (16-byte aligned) and
 * dx uint16 [K/128] from ptq1_rotate_quantize_act; residual f32 [N] or NULL
 * (may equal y); y f32 [N]. K % 128 == 0, K <= Q8G_PTQ1_MAX_K,
 * N <= Q8G_PTQ1_MAX_ROWS. K == 0 gives y = residual (or 0). */
q8g_status ptq1_gemv(const uint8_t *w, const int8_t *qx, const uint16_t *dx, const float *residual, float *y,
                     int64_t N, int64_t K, void *stream);

/* ---- neighbour steps folded into the projection --------------------------
 * [H] Emitting for a GPU: for decode, two kernels each merge a neighbour step
 * into the next projection, one the normalization and one the activation.
 * [P] Q4_K_M names the operations of a block's forward pass: RMS
 * normalization before the attention and MLP projections, and the gated MLP.
 * The values that get quantized are formed in f32 exactly as follows:
 *   RMS normalization (x, gamma f32 [K], eps >= 0 finite):
 *     ss = sum_i x_i^2 in f64 (every square exact), summed in an order that
 *          depends on K only;
 *     r  = fl32(1 / sqrt(ss / K + eps)) in f64, rounded once;
 *     h_i = fl32(fl32(x_i * r) * gamma_i).
 *   Gated activation (gu f32 [2K] = gate [K] then up [K]):
 *     a_i = fl32(gate_i * up_i / (1 + exp(-gate_i))) in f64, rounded once.
 * h or a is then quantized exactly as q8_quantize_act quantizes x. */

/* Quantize RMSnorm(x) * gamma. K % 32 == 0, K <= 16384 (one workgroup holds
 * the row). x, gamma f32 [K] 16-byte aligned; qx int8 [K] 16-byte aligned;
 * dx uint16 [K/32]. Outputs may not overlap the inputs or each other. */
q8g_status q8_rmsnorm_quantize_act(const float *x, const float *gamma, float eps, int8_t *qx, uint16_t *dx,
                                   int64_t K, void *stream);

/* Quantize silu(gate) * up. gu f32 [2K] 16-byte aligned; qx, dx as above;
 * K % 32 == 0. */
q8g_status q8_silu_mul_quantize_act(const float *gu, int8_t *qx, uint16_t *dx, int64_t K, void *stream);

/* The same two steps for B vectors in one launch (the inputs of q8_gemv_batch):
 * vector b is row b of x f32 [B][K] (gamma shared) or of gu f32 [B][2K] (gate
 * then up: the layout q8_gemv_batch writes for a stacked gate+up matrix), and
 * row b of qx int8 [B][K] and dx uint16 [B][K/32]. Each vector is normalized and
 * quantized on its own, exactly as the single-vector call does it.
 * 0 <= B <= 65535; B == 0 enqueues nothing. */
q8g_status q8_rmsnorm_quantize_act_batch(const float *x, const float *gamma, float eps, int8_t *qx, uint16_t *dx,
                                         int64_t K, int64_t B, void *stream);
q8g_status q8_silu_mul_quantize_act_batch(const float *gu, int8_t *qx, uint16_t *dx, int64_t K, int64_t B,
                                          void *stream);

/* Stacked Q8_0 projection of RMSnorm(x) * gamma: one launch normalizes and
 * quantizes x in every workgroup, then runs the dot products. K <= 16384.
 * Part p's result is identical, bit for bit, to q8_rmsnorm_quantize_act then
 * q8_gemv on that part; no output may overlap x or gamma. */
q8g_status gemv_stacked_rmsnorm(const q8g_part *parts, int nparts, const float *x, const float *gamma,
                                float eps, int64_t K, void *stream);

/* Q8_0 GEMV of silu(gate) * up: y = W · a (+ residual), a formed and
 * quantized inside the launch from gu f32 [2K]. K <= 16384. Identical, bit for
 * bit, to q8_silu_mul_quantize_act then q8_gemv; y may not overlap gu. */
q8g_status q8_gemv_silu_mul(const int8_t *qw, const uint16_t *dw, const float *gu, const float *residual,
                            float *y, int64_t N, int64_t K, void *stream);

/* Gate+up projection with the gated activation and its quantization in the
 * epilogue ([H] Emitting for a GPU: gate and up computed in one go; [P] Fast
 * Decode: quantize the activation once, here where it is produced). For F
 * gate rows and the F matching up rows (Q8_0, K columns each):
 *   g = W_gate · x, u = W_up · x     (each row exactly as gemv_stacked computes it)
 *   a = silu(g) * u, quantized       (exactly as q8_silu_mul_quantize_act)
 * qa int8 [F] and da uint16 [F/32] are the quantized input of the down
 * projection: bit-identical to gemv_stacked over (gate, up) followed by
 * q8_silu_mul_quantize_act on [g | u]. No f32 g or u is written.
 * F % 32 == 0 (one workgroup owns 32 gate and 32 up rows); K % 32 == 0.
 * qw_* int8 [F][K] and dw_* uint16 [F][K/32] as for q8_gemv (the two may be the
 * halves of one stacked [2F][K] matrix); qa 16-byte aligned; outputs may not
 * overlap any input or each other. */
q8g_status q8_gateup_silu_quantize(const int8_t *qw_gate, const uint16_t *dw_gate, const int8_t *qw_up,
                                   const uint16_t *dw_up, int64_t F, const int8_t *qx, const uint16_t *dx,
                                   int64_t K, int8_t *qa, uint16_t *da, void *stream);

/* The same with RMSnorm(x) * gamma as the input (x, gamma f32 [K], K <= 16384),
 * normalized and quantized in the prologue exactly as q8_rmsnorm_quantize_act:
 * the whole MLP front of a decode step (normalize, gate and up, activate,
 * quantize) in one launch, bit-identical to q8_rmsnorm_quantize_act, then
 * gemv_stacked, then q8_silu_mul_quantize_act. */
q8g_status q8_gateup_rmsnorm_silu_quantize(const int8_t *qw_gate, const uint16_t *dw_gate, const int8_t *qw_up,
                                           const uint16_t *dw_up, int64_t F, const float *x, const float *gamma,
                                           float eps, int64_t K, int8_t *qa, uint16_t *da, void *stream);

/* Gate+up projection with the gated activation in the epilogue, written in f32
 * ([H] Emitting for a GPU: the activation fused with the projection; [P]
 * Q4_K_M: the gated MLP): for F gate rows and the F matching up rows,
 *   a[j] = silu(g[j]) * u[j]         (f32, exactly as q8_silu_mul_quantize_act forms it)
 * with g, u as gemv_stacked computes them. a f32 [F] (4-byte aligned) is the
 * input of an f32-input down projection (gemv_stacked with Q8G_Q8_0_F32
 * parts), which quantizes it in its prologue: the codes it forms are
 * bit-identical to those of q8_gateup_silu_quantize. Without the quantization,
 * a workgroup needs only matching gate and up rows, not a whole 32-value block
 * of a, so the launch spreads over more workgroups. F % 32 == 0, K % 32 == 0;
 * weights and activation as for q8_gateup_silu_quantize; a may not overlap
 * any input. Q8G_ERR_NULL if a is NULL (F > 0). */
q8g_status q8_gateup_silu(const int8_t *qw_gate, const uint16_t *dw_gate, const int8_t *qw_up, const uint16_t *dw_up,
                          int64_t F, const int8_t *qx, const uint16_t *dx, int64_t K, float *a, void *stream);

/* The same with RMSnorm(x) * gamma as the input (x, gamma f32 [K], K <= 16384),
 * normalized and quantized in the prologue exactly as q8_rmsnorm_quantize_act. */
q8g_status q8_gateup_rmsnorm_silu(const int8_t *qw_gate, const uint16_t *dw_gate, const int8_t *qw_up,
                                  const uint16_t *dw_up, int64_t F, const float *x, const float *gamma, float eps,
                                  int64_t K, float *a, void *stream);

/* ---- a whole decode step in one launch ------------------------------------
 * [P] Fast Decode describes the decode pass as one replayed unit in which each
 * activation is quantized a single time and reused, projections with a common
 * input run together, and the residual joins the product's output.
 * q8_decode_stack runs a sequence of stacked Q8_0 projections as ONE
 * cooperative launch, in order: projection i reads its input only after every
 * workgroup has finished projection i-1 (a device-wide barrier), while the
 * weights of projection i, which depend on no activation, are fetched during
 * that barrier. The input of projection i is quantized once, by the
 * workgroups of projection i-1, with the arithmetic of q8_quantize_act, and
 * each output row is computed with the same instructions as gemv_stacked, so
 * every output is bit-identical to q8_quantize_act + gemv_stacked on the same
 * inputs. An input or residual may be an earlier projection's output (a real
 * decode chain): such a projection waits until those outputs are visible and
 * reads and quantizes its input itself. */
typedef struct {
    const float *x;     /* f32 [K] input of this projection (16-byte aligned) */
    int8_t *qx;         /* optional: the quantized codes int8 [K] are also written here (or NULL) */
    uint16_t *dx;       /* optional: binary16 scale bits [K/32] written here (or NULL) */
    int64_t K;          /* 32 <= K <= Q8G_STACK_MAX_K, K % 32 == 0 */
    int32_t nparts;     /* 1..4 */
    int32_t reserved;   /* must be 0 */
    q8g_part parts[4];  /* as for gemv_stacked; unused slots ignored */
} q8g_stack_op;

#define Q8G_STACK_MAX_K 16384
/* projections of one launch (their descriptors are staged on chip) */
#define Q8G_STACK_MAX_OPS 256
/* uint32 words of the synchronization workspace: a barrier count, an error
 * word, 16 barrier counters and two areas for a quantized input of up to
 * Q8G_STACK_MAX_K values. */
#define Q8G_STACK_SYNC_WORDS 20480
/* word of the workspace that is nonzero if a launch gave up waiting (its
 * outputs are then incomplete; zero the workspace before the next launch). */
#define Q8G_STACK_ERR_WORD 16

/* Run nops projections in order in one launch.
 * ops:     host array of nops <= Q8G_STACK_MAX_OPS descriptors, validated here
 *          (same rules as gemv_stacked per op; no output may overlap any
 *          weight or scale of any op, the input or residual of the same or an
 *          earlier op, or another output; an output may be a later op's input
 *          or residual).
 * ops_dev: device copy of the same nops descriptors (same bytes), read by the
 *          kernel; the caller keeps it alive until the launch completes.
 * sync:    device workspace of Q8G_STACK_SYNC_WORDS uint32 (64-byte aligned),
 *          zero-filled by the caller before its first use; it carries a barrier
 *          count between launches, so launches sharing it must be ordered (one
 *          stream) and run on one device.
 * The launch needs one resident workgroup per compute unit (cooperative
 * launch, at most 1024 compute units); if the device cannot guarantee that,
 * Q8G_ERR_LAUNCH is returned and nothing runs. */
q8g_status q8_decode_stack(const q8g_stack_op *ops, const q8g_stack_op *ops_dev, int nops, uint32_t *sync,
                           void *stream);

/* ---- the same step for callers that cannot allocate ------------------------
 * For callers that may not call hipMalloc or any allocating routine: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation. q8_decode_stack_static is q8_decode_stack without the `sync`
 * argument: its synchronization workspace is a static device array of
 * Q8G_STACK_SYNC_WORDS uint32 inside the library (one copy per device, held
 * until the process ends). Each call enqueues a small kernel that clears that
 * array, then the same launch as q8_decode_stack, so outputs are bit-identical
 * to q8_decode_stack's and no state carries over from one call to the next.
 * Nothing is allocated or freed.
 * status: NULL, or a device uint32 (4-byte aligned) that the launch sets to 1
 *         if it gave up waiting (its outputs are then incomplete); the library
 *         never clears it.
 * Limits: those of q8_decode_stack (Q8G_STACK_MAX_K, one workgroup per compute
 * unit on at most 1024 compute units, at most 256 devices); beyond them the
 * call returns an error and enqueues nothing.
 * All calls on one device share its array: calls that overlap in time on one
 * device (other streams, other threads) race on it and must not be issued. */
q8g_status q8_decode_stack_static(const q8g_stack_op *ops, const q8g_stack_op *ops_dev, int nops, uint32_t *status,
                                  void *stream);

/* Launch configuration the library picks for a GEMV over n_total rows of K
 * (all parts of a stacked call together): output rows per wave (for
 * Q8G_PTQ1_0: rows per wave step) and waves per workgroup. Pure host query; nothing is enqueued. Lets a profiler's per-kernel
 * statistics be matched to the calls that produced them. */
q8g_status q8g_gemv_config(q8g_dtype dtype, int64_t n_total, int64_t K, int *rows_per_wave,
                           int *waves_per_group);

/* A static, human-readable name for a status code. */
const char *q8g_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* Q8GEMV_H */
