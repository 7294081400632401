// Decode-step GEMV kernels for CDNA4 (gfx950) and the C ABI around them.
//
// What is computed is stated in include/q8gemv.h, after "Filling in the blanks:
// Inference using Phobos" (section Fast Decode) and "One level down: #002 the
// same compiler on a GPU" (sections Emitting for a GPU, The numerical contract).
//
// Design (MI355X, wave64):
//  * The work is a matrix-vector product: every weight byte is read once and
//    used for one multiply-add, about 2 ops per byte, so the bound is HBM
//    bandwidth and there is no dense contraction for MFMA to speed up.
//  * A wave owns R consecutive output rows. For each row it streams the row
//    in 1 KiB chunks: lane l loads bytes [16l, 16l+16) of the chunk with one
//    global_load_dwordx4, so each load instruction of the wave covers 1 KiB
//    of contiguous memory. The activation slice that lane l needs is the same
//    for every row, so it is loaded once per chunk and kept in registers.
//  * Q8_0: a 32-byte block spans lanes 2j and 2j+1. Each lane forms its half
//    with four v_dot4c_i32_i8; one DPP quad_perm add joins the halves, so
//    every block yields one exact int32 sum. The even lane of the pair scales
//    it by dw*dx (exact in f32: 11 + 11 significant bits) with one fma into
//    its f32 accumulator; the odd lane adds zero.
//  * bf16: a lane's 16 bytes are eight bf16 weights; bf16 -> f32 is a shift or
//    a mask, the products are exact in f32, and a chunk's eight products are
//    summed into a chunk partial before it joins the lane accumulator, so no
//    f32 chain grows beyond eight terms plus one per chunk.
//  * The R row sums of a wave are reduced together by a butterfly: exchanges
//    at lane distance 1, 2, 4 and 8 (DPP) and 16 and 32 (the permlane swaps),
//    none through the LDS crossbar. While two or more rows remain per lane, each
//    step keeps half of them and adds the partner's copy of that half, so R
//    rows cost R-1 exchanges plus the six of a single sum. The tree always
//    pairs lanes at distance 1, 2, 4, ..., 32, so a row's bits do not depend on
//    R, on its slot in the wave, or on whether it sits in a stacked launch.
//  * Rows past the last one are masked (no load, no store): the pages report a
//    tail that wrote rows beyond the output.
//  * Weights and weight scales are read once per call, so they are loaded
//    with the nontemporal hint; the activation, shared by every wave, is not.
//  * No atomics and no scratch; LDS holds only the quantized activation of the
//    f32-input kinds (and the reduction slots of the epilogue kind), so results
//    depend on the shape only.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemv_device.hpp"
#include "ptq1.hpp"
#include "q8gemv.h"

namespace {

using namespace q8g;

constexpr int kMaxParts = 4;

// Q8: x = int8 codes + binary16 scales; BF16: x = bf16; Q8F32: x = f32, quantized
// by every workgroup into LDS before use (one launch instead of two); F16:
// binary16 weights and activation. Q8NORM and Q8SILU are Q8F32 with a neighbour
// step folded into the prologue ("One level down: #002 the same compiler on a
// GPU", section Emitting for a GPU: for decode, two kernels each merge a
// neighbour step into the next projection, the normalization and the activation):
// Q8NORM quantizes (x * r) * gamma, r = 1/sqrt(mean(x^2) + eps); Q8SILU takes
// x = [gate | up] (2K values) and quantizes silu(gate) * up.
enum class Dt { Q8, BF16, Q8F32, F16, Q8NORM, Q8SILU };

// f32 activation quantized inside the launch
constexpr bool is_fused(Dt dt) { return dt == Dt::Q8F32 || dt == Dt::Q8NORM || dt == Dt::Q8SILU; }

// 16-bit float weights (no block scales), two bytes per element
constexpr bool is_16bit(Dt dt) { return dt == Dt::BF16 || dt == Dt::F16; }

constexpr int kMaxFusedK = 16384;  // LDS bytes for the codes of a fused launch
constexpr int64_t kMaxBatchVectors = 65535;  // vectors of one batched neighbour-step launch (grid dimension)

// ---- neighbour-step prologues ------------------------------------------------
// The quantization decision is taken on f32 values, so the oracle and every
// launch shape must form the same f32 values. The gated activation is one f64
// expression rounded once. The normalization's sum of squares is formed in f64
// (every f32 square is exact there) in an order that depends on K only: each
// 32-value block by its 8 lanes (4 values each, then exchanges at distance 1, 2
// and 4), then the block sums by every wave alike (lane l takes blocks l, l+64,
// ..., then exchanges at distance 1..32). Every lane of a group, and every
// wave, ends with the same bits, because IEEE addition is commutative.
__device__ __forceinline__ double sq4(const float4 &v)
{
    return (((double)v.x * v.x + (double)v.y * v.y) + (double)v.z * v.z) + (double)v.w * v.w;
}

// v + (the f64 v of the lane at xor distance M): both halves through the same
// 32-bit lane pairing (lane_pair), so each result half comes from one lane; the
// sum has the same bits in both lanes
template <int M>
__device__ __forceinline__ double xsum64(double v)
{
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    int alo, blo, ahi, bhi;
    lane_pair<M>((int)(uint32_t)u, alo, blo);
    lane_pair<M>((int)(uint32_t)(u >> 32), ahi, bhi);
    const double a = __builtin_bit_cast(double, ((uint64_t)(uint32_t)ahi << 32) | (uint32_t)alo);
    const double b = __builtin_bit_cast(double, ((uint64_t)(uint32_t)bhi << 32) | (uint32_t)blo);
    return a + b;
}

__device__ __forceinline__ double block_sum8(double p)
{
    p = xsum64<1>(p);
    p = xsum64<2>(p);
    p = xsum64<4>(p);
    return p;
}

// sum of nb block partials in LDS, the same bits in every lane of every wave
__device__ __forceinline__ double blocks_total(const double *s_bss, int64_t nb, int lane)
{
    double t = 0.0;
    for (int64_t b = lane; b < nb; b += kWave) t += s_bss[b];
    t = xsum64<1>(t);
    t = xsum64<2>(t);
    t = xsum64<4>(t);
    t = xsum64<8>(t);
    t = xsum64<16>(t);
    t = xsum64<32>(t);
    return t;
}

__device__ __forceinline__ float rms_scale(double ss, int64_t K, float eps)
{
    return (float)(1.0 / sqrt(ss / (double)K + (double)eps));
}

__device__ __forceinline__ float silu_mul(float g, float u)
{
    const double gd = g, ud = u;
    return (float)((gd * ud) / (1.0 + exp(-gd)));
}

// the f32 values that get quantized: Q8F32 x; Q8NORM (x * r) * gamma; Q8SILU
// silu(gate) * up (v = gate, v2 = up)
template <Dt DT>
__device__ __forceinline__ float4 prologue_value(const float4 &v, const float4 &v2, float r)
{
    if constexpr (DT == Dt::Q8NORM) {
        return make_float4((v.x * r) * v2.x, (v.y * r) * v2.y, (v.z * r) * v2.z, (v.w * r) * v2.w);
    } else if constexpr (DT == Dt::Q8SILU) {
        return make_float4(silu_mul(v.x, v2.x), silu_mul(v.y, v2.y), silu_mul(v.z, v2.z), silu_mul(v.w, v2.w));
    } else {
        return v;
    }
}


// Stacked parts. The kernel receives them as separate scalar arguments (see
// PARTS_PARAMS): an aggregate argument selected by a row-dependent index gets
// copied to scratch memory, while separate arguments stay in SGPRs. Parts are
// contiguous in the stacked row space; unused trailing slots have
// end = INT64_MAX so that no row selects them.
struct Parts {
    const void *w[kMaxParts];
    const uint16_t *dw[kMaxParts];
    float *y[kMaxParts];
    const float *res[kMaxParts];
    int64_t end[kMaxParts];
};

#define PARTS_PARAMS                                                                                   \
    const void *w0, const void *w1, const void *w2, const void *w3, const uint16_t *dw0,               \
        const uint16_t *dw1, const uint16_t *dw2, const uint16_t *dw3, float *y0, float *y1, float *y2, \
        float *y3, const float *r0, const float *r1, const float *r2, const float *r3, int64_t e0,     \
        int64_t e1, int64_t e2

// Row g of the stacked operand: which part, and its local index.
struct RowRef {
    const char *w;
    const uint16_t *dw;
    float *y;
    const float *res;
};

#define LOCATE(g, row_bytes, nb, out)                                                              \
    do {                                                                                           \
        int64_t local_ = (g);                                                                      \
        RowRef r_{static_cast<const char *>(w0), dw0, y0, r0};                                     \
        if ((g) >= e0) {                                                                           \
            local_ = (g) - e0;                                                                     \
            r_ = RowRef{static_cast<const char *>(w1), dw1, y1, r1};                               \
        }                                                                                          \
        if ((g) >= e1) {                                                                           \
            local_ = (g) - e1;                                                                     \
            r_ = RowRef{static_cast<const char *>(w2), dw2, y2, r2};                               \
        }                                                                                          \
        if ((g) >= e2) {                                                                           \
            local_ = (g) - e2;                                                                     \
            r_ = RowRef{static_cast<const char *>(w3), dw3, y3, r3};                               \
        }                                                                                          \
        r_.w += local_ * (row_bytes);                                                              \
        if (r_.dw) r_.dw += local_ * (nb);                                                         \
        r_.y += local_;                                                                            \
        if (r_.res) r_.res += local_;                                                              \
        (out) = r_;                                                                                \
    } while (0)

// ---- batches of row-chunk items ------------------------------------------------
// A wave's R rows times C chunks are visited chunk-major (chunk c of rows 0..R-1,
// then chunk c+1), so every row sees its chunks in ascending order, which is the
// order of its f32 accumulation. Items are loaded kBatch at a time with all of a
// batch's loads in flight together, and the next batch is requested before the
// current one is consumed: a multi-chunk row costs about one memory round trip,
// not one per chunk.
constexpr int kBatch = 4;
static_assert(kBatch == 4, "a batch holds 4 items (a multiple of R)");

struct Batch {
    int4 w[kBatch];      // weight bytes of item j (16 per lane)
    uint16_t s[kBatch];  // Q8_0: the weight block scale bits of item j
    int4 x[kBatch];      // activation bytes of item j's chunk (items with j % R == 0)
    uint16_t xs[kBatch]; // Q8_0: the activation block scale bits of that chunk
};

// Items j = 0..kBatch-1 of the batch starting at chunk c0: chunk c0 + j / R of
// row j % R. Lanes past the row end load offset 0 (always in bounds) and are
// masked when the batch is consumed. With XG the activation is read from
// global memory here as well; otherwise it is read from LDS when consumed.
//
// ALL: items past the row's last chunk re-read that chunk and are skipped when
// consumed, so every load is issued unconditionally (nchunk >= 1) and the
// compiler can count the loads in flight. A load under a condition, even a
// wave-uniform one, makes the wait for the loads issued before it assume the
// condition was false, i.e. wait for these loads as well. Used for every batch
// after the first (the row loop), and for the first batch of the f32-input
// kinds, whose activation quantization then overlaps the weights in flight. The
// first batch of the other kinds has nothing to overlap with and skips those
// items (the re-reads cost them time).
template <Dt DT, int R, bool XG, bool ALL>
__device__ __forceinline__ void load_batch(const RowRef (&rows)[R], const char *__restrict__ x,
                                           const uint16_t *__restrict__ dx, int64_t c0, int64_t nchunk,
                                           int64_t row_bytes, int64_t lane_off, Batch &b)
{
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
        const bool real = c0 + j / R < nchunk;  // wave-uniform
        if (ALL || real) {
            const int64_t c = real ? c0 + j / R : nchunk - 1;
            const int r = j % R;
            const int64_t off = c * kChunk + lane_off;
            const int64_t o = off < row_bytes ? off : 0;
            b.w[j] = load16_stream(rows[r].w + o);
            if constexpr (!is_16bit(DT)) b.s[j] = load_u16_stream(rows[r].dw + (o >> 5));
            if constexpr (XG) {
                if (r == 0) {
                    b.x[j] = load16(x + o);
                    if constexpr (DT == Dt::Q8) b.xs[j] = dx[o >> 5];
                }
            }
        }
    }
}

// The accumulators as they stand, before anything that follows: an empty
// volatile asm that reads and writes them. A scheduling barrier orders the
// machine instructions only; arithmetic can be placed after a later load before
// that, which keeps the batch it reads live across the load.
template <int R>
__device__ __forceinline__ void settle(float (&acc)[R])
{
#pragma unroll
    for (int r = 0; r < R; ++r) asm volatile("" : "+v"(acc[r]));
}

// Consume a batch. Q8_0: one exact int32 block sum per item (v_dot4 + one DPP
// add), scaled by dw*dx (exact in f32) with one fma; the odd lane of each block
// pair and lanes past the row end add zero. bf16: eight exact products summed
// into a chunk partial, then added to the row's accumulator (f16 the same).
template <Dt DT, int R, bool XG>
__device__ __forceinline__ void compute_batch(const Batch &b, const int8_t *__restrict__ s_qx,
                                              const float *__restrict__ s_dx, int64_t c0, int64_t nchunk,
                                              int64_t row_bytes, int64_t lane_off, float even, float (&acc)[R])
{
    int4 xq = make_int4(0, 0, 0, 0);
    float xs = 0.0f;
    float xf[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
        const int64_t c = c0 + j / R;
        const int r = j % R;
        if (c < nchunk) {
            if (r == 0) {
                const int64_t off = c * kChunk + lane_off;
                const bool active = off < row_bytes;
                const int64_t o = active ? off : 0;
                if constexpr (is_16bit(DT)) {
                    if constexpr (DT == Dt::BF16)
                        bf16_unpack(b.x[j], xf);
                    else
                        f16_unpack(b.x[j], xf);
#pragma unroll
                    for (int i = 0; i < 8; ++i) xf[i] = active ? xf[i] : 0.0f;
                } else if constexpr (XG) {
                    xq = b.x[j];
                    xs = active ? f16_bits_to_f32(b.xs[j]) * even : 0.0f;
                } else {
                    xq = *reinterpret_cast<const int4 *>(s_qx + o);
                    xs = active ? s_dx[o >> 5] * even : 0.0f;
                }
            }
            if constexpr (DT == Dt::BF16) {
                acc[r] += bf16_chunk_dot(b.w[j], xf);
            } else if constexpr (DT == Dt::F16) {
                acc[r] += f16_chunk_dot(b.w[j], xf);
            } else {
                const int s = q8_block_sum(b.w[j], xq);  // the block's exact int32 sum
                acc[r] = __builtin_fmaf((float)s, f16_bits_to_f32(b.s[j]) * xs, acc[r]);
            }
        }
    }
}

// Reduce the R row sums of a wave and write them (+ residual, added once).
// Row i is written by lane lane_of<R>(i); the loop index is a compile-time
// constant, so every row pointer stays a scalar (no indexed private array).
// PRES: some part has a residual, prefetched into res (without PRES no part has one)
template <int R, bool PRES>
__device__ __forceinline__ void reduce_and_store(float (&acc)[R], const RowRef (&rows)[R], const bool (&valid)[R],
                                                 const float (&res)[R], int lane)
{
    const float total = wave_reduce_rows<R>(acc, lane);
#pragma unroll
    for (int i = 0; i < R; ++i)
        if (valid[i] && lane == lane_of<R>(i)) *rows[i].y = PRES && rows[i].res ? total + res[i] : total;
}

// y[rows] = W[rows] · x (+ residual) for the R rows owned by each wave.
// Q8F32: x is f32; the workgroup first requests x (its loads return before the
// weight loads issued after them: one wave's loads complete in issue order),
// then its first weight batch, then quantizes x into LDS (the arithmetic of
// q8_quantize_act) while the weights are in flight. Per row, the arithmetic and
// its order are the same for all three kinds, so a Q8F32 launch is
// bit-identical to q8_quantize_act followed by a Q8 launch.
//
// EPI (nonzero): the gate+up projection with the gated activation in the
// epilogue (parts 0 and 1 are gate and up, F = n_total / 2 rows each). A
// workgroup owns P = R * WAVES / 2 gate rows P*b.. (its first WAVES / 2 waves)
// and the same up rows (the other half), and forms a = silu(gate) * up from the
// rows' f32 results as q8_silu_mul_quantize_act forms it. EPI 1 (R = 4, 16
// waves, P = 32): a is quantized as one Q8_0 block, written as the 32 codes
// qa[32b..] and the scale da[b]. EPI 2: a itself is written, in f32, to part
// 0's output (y0[P*b + j]); nothing else is written.
// XP: f32 activation passes requested before the weights (1 when one pass of
// 4 values per thread covers K, 2 when two do, else 4; values past them are
// read after the weights are requested). Loads of passes past K are clamped duplicates, so
// their number is chosen by the launch rather than fixed.
template <Dt DT, int R, int WAVES, int EPI = 0, bool PRES = false, int XP = 4>
__global__ __launch_bounds__(WAVES *kWave) void gemv_kernel(PARTS_PARAMS, const void *__restrict__ xv,
                                                            const uint16_t *__restrict__ dx,
                                                            const float *__restrict__ aux, float eps,
                                                            int64_t K, int64_t n_total, int8_t *__restrict__ qa,
                                                            uint16_t *__restrict__ da)
{
    static_assert(EPI != 1 || (R == 4 && WAVES == 16), "the quantizing epilogue needs 32 gate and 32 up rows");
    static_assert(EPI == 0 || (WAVES % 2 == 0 && R * WAVES / 2 <= 32), "gate and up waves in equal numbers");
    static_assert(!(EPI && PRES), "the epilogue kinds have no residual");
    constexpr int P = R * WAVES / 2;  // EPI: gate+up row pairs per workgroup
    constexpr bool FUSED = is_fused(DT);
    constexpr bool TWO = DT == Dt::Q8NORM || DT == Dt::Q8SILU;  // a second f32 input per value
    constexpr int kThreadsPerGroup = WAVES * kWave;
    constexpr int kXPasses = XP;  // f32 activation passes requested before the weights
    __shared__ __align__(16) int8_t s_qx[FUSED ? kMaxFusedK : 16];
    __shared__ float s_dx[FUSED ? kMaxFusedK / 32 : 4];
    __shared__ double s_bss[DT == Dt::Q8NORM ? kMaxFusedK / 32 : 1];

    const int lane = threadIdx.x & (kWave - 1);
    // wave-uniform by construction; readfirstlane lets the compiler keep the
    // row bookkeeping and the part table in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t row0 = !EPI               ? ((int64_t)blockIdx.x * WAVES + wave) * R
                         : wave < WAVES / 2 ? P * (int64_t)blockIdx.x + R * wave
                                            : n_total / 2 + P * (int64_t)blockIdx.x + R * (wave - WAVES / 2);
    const bool has_rows = row0 < n_total;  // wave-uniform
    if (!FUSED && !has_rows) return;

    const int64_t row_bytes = is_16bit(DT) ? 2 * K : K;
    const int64_t nb = K / 32;
    const int64_t nchunk = (row_bytes + kChunk - 1) / kChunk;
    constexpr int CB = kBatch / R;  // chunks per batch
    const char *x = static_cast<const char *>(xv);
    const int64_t lane_off = (int64_t)lane * 16;

    // the second input of a value: gamma (Q8NORM) or up (Q8SILU, the upper half of x)
    const float *x2 = DT == Dt::Q8NORM ? aux : static_cast<const float *>(xv) + K;
    float4 xin[kXPasses], xin2[kXPasses];
    if constexpr (FUSED) {
        // Every lane loads, past-the-end lanes from the last 4 values (K >= 32 here:
        // the host runs K == 0 as the Q8 kind). A load under a lane condition would
        // be waited for at the branch join, before any weight load is issued.
        const float *xf = static_cast<const float *>(xv);
#pragma unroll
        for (int p = 0; p < kXPasses; ++p) {
            const int64_t e = (int64_t)threadIdx.x * 4 + (int64_t)p * 4 * kThreadsPerGroup;
            const int64_t ec = e < K ? e : K - 4;
            xin[p] = *reinterpret_cast<const float4 *>(xf + ec);
            if constexpr (TWO) xin2[p] = *reinterpret_cast<const float4 *>(x2 + ec);
        }
    }

    RowRef rows[R];
    bool valid[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        valid[r] = row0 + r < n_total;
        LOCATE(valid[r] ? row0 + r : (has_rows ? row0 : 0), row_bytes, nb, rows[r]);
    }

    // PRES (launches where some part has a residual): the residuals are requested
    // before the weights (one wave's loads complete in issue order), so the final
    // store does not wait for one more memory round trip. Every lane loads (a load
    // under a condition would be waited for at the branch join); a row without a
    // residual reads the first word of the activation instead (just requested, so
    // cached; its value is unused), or its own output element when K == 0 and
    // there is no activation. The address goes through a vector register so that
    // this stays a vector load, counted with the other loads (a uniform address
    // would become a scalar load, whose wait the compiler merges with the LDS
    // waits of the quantization; a volatile load is waited for at once). Without
    // a residual the launch keeps the registers this costs (the output heads are
    // sensitive to occupancy).
    float res[R];
#pragma unroll
    for (int r = 0; r < R; ++r) res[r] = 0.0f;
    if constexpr (PRES) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float *dummy = K > 0 ? static_cast<const float *>(xv) : rows[r].y;
            uint64_t a = reinterpret_cast<uint64_t>(rows[r].res ? rows[r].res : dummy);
            asm("" : "+v"(a));
            res[r] = *reinterpret_cast<const __attribute__((address_space(1))) float *>(a);
        }
    }

    Batch cur, nxt;
    if constexpr (FUSED) {
        // K >= 32 here and a wave without rows has row 0's table, so the first batch
        // is requested unconditionally (such a wave reads row 0 and leaves after the
        // quantization): a condition here would make the quantization's wait for
        // the activation include these loads
        load_batch<DT, R, false, true>(rows, x, dx, 0, nchunk, row_bytes, lane_off, cur);
    } else {
        if (has_rows && nchunk > 0) load_batch<DT, R, true, false>(rows, x, dx, 0, nchunk, row_bytes, lane_off, cur);
    }

    if constexpr (FUSED) {
        const float *xf = static_cast<const float *>(xv);
        // Q8NORM: block sums of squares for every block, then their total
        float r = 1.0f;
        if constexpr (DT == Dt::Q8NORM) {
#pragma unroll
            for (int p = 0; p < kXPasses; ++p) {
                const int64_t e = (int64_t)threadIdx.x * 4 + (int64_t)p * 4 * kThreadsPerGroup;
                if (e - (int64_t)(threadIdx.x & 7) * 4 < K) {  // the 8-lane group of this block is in range
                    const double b = block_sum8(sq4(xin[p]));
                    if ((lane & 7) == 0) s_bss[e >> 5] = b;
                }
            }
            for (int64_t e = (int64_t)threadIdx.x * 4 + (int64_t)kXPasses * 4 * kThreadsPerGroup; e < K;
                 e += 4 * kThreadsPerGroup) {
                const double b = block_sum8(sq4(*reinterpret_cast<const float4 *>(xf + e)));
                if ((lane & 7) == 0) s_bss[e >> 5] = b;
            }
            __syncthreads();
            r = rms_scale(blocks_total(s_bss, nb, lane), K, eps);
        }
#pragma unroll
        for (int p = 0; p < kXPasses; ++p) {
            const int64_t e = (int64_t)threadIdx.x * 4 + (int64_t)p * 4 * kThreadsPerGroup;
            if (e - (int64_t)(threadIdx.x & 7) * 4 < K) {  // the 8-lane group of this block is in range
                float d;
                const uint32_t packed = quantize4(prologue_value<DT>(xin[p], xin2[p], r), &d);
                if (e < K) {
                    *reinterpret_cast<uint32_t *>(s_qx + e) = packed;
                    if ((lane & 7) == 0) s_dx[e >> 5] = f16_bits_to_f32(scale_bits(d));
                }
            }
        }
        for (int64_t e = (int64_t)threadIdx.x * 4 + (int64_t)kXPasses * 4 * kThreadsPerGroup; e < K;
             e += 4 * kThreadsPerGroup) {
            const float4 v = *reinterpret_cast<const float4 *>(xf + e);
            const float4 v2 = TWO ? *reinterpret_cast<const float4 *>(x2 + e) : v;
            float d;
            const uint32_t packed = quantize4(prologue_value<DT>(v, v2, r), &d);
            *reinterpret_cast<uint32_t *>(s_qx + e) = packed;
            if ((lane & 7) == 0) s_dx[e >> 5] = f16_bits_to_f32(scale_bits(d));
        }
        __syncthreads();
        if (!has_rows) return;
    }

    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.0f;
    const float even = (lane & 1) ? 0.0f : 1.0f;  // Q8_0: the even lane of a pair applies the scale

    // Rows of several batches: two batches a trip, cur and nxt taking turns, in a
    // straight-line body, so no register copy (which would wait for the loads just
    // issued) stands between a batch's request and its use. The loads are
    // unconditional (a partial batch re-reads its last chunk), so the wait before
    // each compute counts only the batch it consumes, and a scheduling barrier
    // keeps a batch's requests ahead of the compute that precedes them in program
    // order, so that the other batch stays in flight in full.
    int64_t c0 = 0;
    for (; c0 + 2 * CB < nchunk; c0 += 2 * CB) {
        load_batch<DT, R, !FUSED, true>(rows, x, dx, c0 + CB, nchunk, row_bytes, lane_off, nxt);
        __builtin_amdgcn_sched_barrier(0);
        compute_batch<DT, R, !FUSED>(cur, s_qx, s_dx, c0, nchunk, row_bytes, lane_off, even, acc);
        settle(acc);
        load_batch<DT, R, !FUSED, true>(rows, x, dx, c0 + 2 * CB, nchunk, row_bytes, lane_off, cur);
        __builtin_amdgcn_sched_barrier(0);
        compute_batch<DT, R, !FUSED>(nxt, s_qx, s_dx, c0 + CB, nchunk, row_bytes, lane_off, even, acc);
    }
    // the row's last one or two batches (cur holds chunk c0 on)
    if (c0 + CB < nchunk) {
        load_batch<DT, R, !FUSED, true>(rows, x, dx, c0 + CB, nchunk, row_bytes, lane_off, nxt);
        __builtin_amdgcn_sched_barrier(0);
        compute_batch<DT, R, !FUSED>(cur, s_qx, s_dx, c0, nchunk, row_bytes, lane_off, even, acc);
        compute_batch<DT, R, !FUSED>(nxt, s_qx, s_dx, c0 + CB, nchunk, row_bytes, lane_off, even, acc);
    } else if (c0 < nchunk) {
        compute_batch<DT, R, !FUSED>(cur, s_qx, s_dx, c0, nchunk, row_bytes, lane_off, even, acc);
    }
    if constexpr (EPI) {
        // s_gu[0..P-1]: gate rows P*b.., s_gu[P..2P-1]: the same up rows
        __shared__ __align__(16) float s_gu[2 * P];
        const float total = wave_reduce_rows<R>(acc, lane);
#pragma unroll
        for (int i = 0; i < R; ++i)
            if (lane == lane_of<R>(i)) s_gu[(wave < WAVES / 2 ? 0 : P) + R * (wave % (WAVES / 2)) + i] = total;
        __syncthreads();
        if constexpr (EPI == 2) {
            // a[P*b + j] = silu(gate) * up: wave 0's first row is gate row P*b, so its
            // output pointer is a + P*b
            if (wave == 0 && lane < P) rows[0].y[lane] = silu_mul(s_gu[lane], s_gu[P + lane]);
        } else if (wave == 0) {
            // one value per lane (lanes 32..63 repeat 0..31): a = silu(gate) * up, then
            // the block's quantization with quantize4's arithmetic (max |a| over the
            // 32 lanes, d = fl32(max / 127), q = rint(fl32(a / d)))
            const int j = lane & 31;
            const float a = silu_mul(s_gu[j], s_gu[32 + j]);
            float m = fabsf(a);
            m = xmax<1>(m);
            m = xmax<2>(m);
            m = xmax<4>(m);
            m = xmax<8>(m);
            m = xmax<16>(m);
            const float d = m / 127.0f;
            float q = 0.0f;
            if (d != 0.0f) q = fminf(fmaxf(__builtin_rintf(a / d), -127.0f), 127.0f);
            if (lane < 32) {
                qa[32 * (int64_t)blockIdx.x + j] = (int8_t)(int)q;
                if (lane == 0) da[blockIdx.x] = scale_bits(d);
            }
        }
    } else {
        reduce_and_store<R, PRES>(acc, rows, valid, res, lane);
    }
}

// One 8-lane group per 32-value block; each lane quantizes 4 values.
__global__ __launch_bounds__(256) void quantize_kernel(const float *__restrict__ x, int8_t *__restrict__ qx,
                                                       uint16_t *__restrict__ dx, int64_t K)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    const bool active = e < K;  // K % 32 == 0: whole groups are in or out
    const float4 v = active ? *reinterpret_cast<const float4 *>(x + e) : make_float4(0.f, 0.f, 0.f, 0.f);
    float d;
    const uint32_t packed = quantize4(v, &d);
    if (!active) return;
    *reinterpret_cast<uint32_t *>(qx + e) = packed;
    if ((lane & 7) == 0) dx[e >> 5] = scale_bits(d);
}

// Quantize silu(gate) * up (gu = [gate | up], K values each): the Q8SILU
// prologue as its own launch. Vector v = blockIdx.y of a batch: gu [v][2K],
// qx [v][K], dx [v][K/32].
__global__ __launch_bounds__(256) void silu_quantize_kernel(const float *__restrict__ gu, int8_t *__restrict__ qx,
                                                            uint16_t *__restrict__ dx, int64_t K)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t v = blockIdx.y;
    gu += v * 2 * K;
    qx += v * K;
    dx += v * (K / 32);
    const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    const bool active = e < K;
    const float4 g = active ? *reinterpret_cast<const float4 *>(gu + e) : make_float4(0.f, 0.f, 0.f, 0.f);
    const float4 u = active ? *reinterpret_cast<const float4 *>(gu + K + e) : make_float4(0.f, 0.f, 0.f, 0.f);
    float d;
    const uint32_t packed = quantize4(prologue_value<Dt::Q8SILU>(g, u, 1.0f), &d);
    if (!active) return;
    *reinterpret_cast<uint32_t *>(qx + e) = packed;
    if ((lane & 7) == 0) dx[e >> 5] = scale_bits(d);
}

// Quantize (x * r) * gamma with the Q8NORM prologue's arithmetic and order, as
// one workgroup of kNormThreads per vector (K <= kMaxFusedK): block sums of
// squares, their total, then the values. Vector v = blockIdx.x of a batch:
// x [v][K], qx [v][K], dx [v][K/32]; gamma is shared.
constexpr int kNormThreads = 1024;
__global__ __launch_bounds__(kNormThreads) void norm_quantize_kernel(const float *__restrict__ x,
                                                                     const float *__restrict__ gamma, float eps,
                                                                     int8_t *__restrict__ qx,
                                                                     uint16_t *__restrict__ dx, int64_t K)
{
    __shared__ double s_bss[kMaxFusedK / 32];
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t v = blockIdx.x;
    x += v * K;
    qx += v * K;
    dx += v * (K / 32);
    for (int64_t e = (int64_t)threadIdx.x * 4; e < K; e += 4 * kNormThreads) {
        const double b = block_sum8(sq4(*reinterpret_cast<const float4 *>(x + e)));
        if ((lane & 7) == 0) s_bss[e >> 5] = b;
    }
    __syncthreads();
    const float r = rms_scale(blocks_total(s_bss, K / 32, lane), K, eps);
    for (int64_t e = (int64_t)threadIdx.x * 4; e < K; e += 4 * kNormThreads) {
        const float4 xe = *reinterpret_cast<const float4 *>(x + e);
        const float4 g = *reinterpret_cast<const float4 *>(gamma + e);
        float d;
        const uint32_t packed = quantize4(prologue_value<Dt::Q8NORM>(xe, g, r), &d);
        *reinterpret_cast<uint32_t *>(qx + e) = packed;
        if ((lane & 7) == 0) dx[e >> 5] = scale_bits(d);
    }
}

// ---- host side ---------------------------------------------------------------

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlap(const void *a, int64_t abytes, const void *b, int64_t bbytes)
{
    if (!a || !b || abytes <= 0 || bbytes <= 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

constexpr int64_t kMaxElems = (int64_t)1 << 60;

template <Dt DT, int R, int WAVES, int EPI = 0, bool PRES = false, int XP = 4>
hipError_t launch_gemv(const Parts &p, const void *x, const uint16_t *dx, const float *aux, float eps, int64_t K,
                       int64_t n_total, hipStream_t s, int8_t *qa = nullptr, uint16_t *da = nullptr)
{
    const int64_t rows_per_block = (int64_t)R * WAVES;
    // EPI: one workgroup per R * WAVES / 2 gate rows and the matching up rows
    const int64_t blocks = EPI ? n_total / rows_per_block : (n_total + rows_per_block - 1) / rows_per_block;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    Parts pc = p;
    const void *xc = x;
    const uint16_t *dxc = dx;
    const float *auxc = aux;
    float epsc = eps;
    int64_t kc = K, nc = n_total;
    int8_t *qac = qa;
    uint16_t *dac = da;
    void *args[] = {&pc.w[0],   &pc.w[1],   &pc.w[2],   &pc.w[3],   &pc.dw[0],  &pc.dw[1], &pc.dw[2],
                    &pc.dw[3],  &pc.y[0],   &pc.y[1],   &pc.y[2],   &pc.y[3],   &pc.res[0], &pc.res[1],
                    &pc.res[2], &pc.res[3], &pc.end[0], &pc.end[1], &pc.end[2], &xc,       &dxc,
                    &auxc,      &epsc,      &kc,        &nc,        &qac,       &dac};
    const void *fn = reinterpret_cast<const void *>(&gemv_kernel<DT, R, WAVES, EPI, PRES, XP>);
    return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(WAVES * kWave), args, 0, s);
}

// Launch configuration by shape (measured on MI355X over the decode shapes):
// rows per wave R as many as keep at least ~8 waves per compute unit busy (at
// most 2 for bf16); 4 waves per workgroup, except fused launches over fewer
// than 32768 rows, where 8 waves share the activation quantization.
constexpr int kWavesPerGroup = 4;
constexpr int64_t kFusedWideRows = 32768;

int rows_per_wave(int64_t n_total)
{
    const int64_t target_waves = 256 * 8;
    if (n_total >= 4 * target_waves) return 4;
    if (n_total >= 2 * target_waves) return 2;
    return 1;
}

struct Config {
    int rows;
    int waves;
};

Config pick_config(q8g_dtype dt, int64_t n_total)
{
    Config c{rows_per_wave(n_total), kWavesPerGroup};
    if (dt == Q8G_BF16 || dt == Q8G_F16) {
        // 16-bit rows are twice as long: two rows per wave already keep 4 KiB in flight
        if (c.rows > 2) c.rows = 2;
    }
    if (dt == Q8G_Q8_0_F32) c.waves = n_total < kFusedWideRows ? 8 : 4;
    return c;
}

// the f32 input and its neighbour step of a fused launch
struct Prologue {
    const float *aux;  // Q8NORM: gamma [K]
    float eps;         // Q8NORM: added to the mean square
};

// activation passes of an f32-input launch: one when it covers K
constexpr bool one_pass(int64_t K, int threads) { return K <= 4 * (int64_t)threads; }
constexpr bool two_passes(int64_t K, int threads) { return K <= 8 * (int64_t)threads; }

template <Dt DT, int R, int W, bool PRES>
hipError_t launch_xp(const Parts &p, const void *x, const uint16_t *dx, Prologue pr, int64_t K, int64_t n_total,
                     hipStream_t s)
{
    if constexpr (is_fused(DT)) {
        if (one_pass(K, W * kWave))
            return launch_gemv<DT, R, W, 0, PRES, 1>(p, x, dx, pr.aux, pr.eps, K, n_total, s);
        if (two_passes(K, W * kWave))
            return launch_gemv<DT, R, W, 0, PRES, 2>(p, x, dx, pr.aux, pr.eps, K, n_total, s);
    }
    return launch_gemv<DT, R, W, 0, PRES, 4>(p, x, dx, pr.aux, pr.eps, K, n_total, s);
}

template <Dt DT, int R, int W>
hipError_t launch_res(bool pres, const Parts &p, const void *x, const uint16_t *dx, Prologue pr, int64_t K,
                      int64_t n_total, hipStream_t s)
{
    return pres ? launch_xp<DT, R, W, true>(p, x, dx, pr, K, n_total, s)
                : launch_xp<DT, R, W, false>(p, x, dx, pr, K, n_total, s);
}

template <Dt DT, int W>
hipError_t dispatch_rows(int rows, const Parts &p, const void *x, const uint16_t *dx, Prologue pr, int64_t K,
                         int64_t n_total, hipStream_t s)
{
    const bool pres = p.res[0] || p.res[1] || p.res[2] || p.res[3];
    switch (rows) {
    case 4: return launch_res<DT, 4, W>(pres, p, x, dx, pr, K, n_total, s);
    case 2: return launch_res<DT, 2, W>(pres, p, x, dx, pr, K, n_total, s);
    default: return launch_res<DT, 1, W>(pres, p, x, dx, pr, K, n_total, s);
    }
}

template <Dt DT>
hipError_t dispatch_gemv(Config c, const Parts &p, const void *x, const uint16_t *dx, Prologue pr, int64_t K,
                         int64_t n_total, hipStream_t s)
{
    if constexpr (is_fused(DT)) {
        if (c.waves == 8) return dispatch_rows<DT, 8>(c.rows, p, x, dx, pr, K, n_total, s);
    }
    return dispatch_rows<DT, kWavesPerGroup>(c.rows, p, x, dx, pr, K, n_total, s);
}

// Launch kinds: the public dtypes, and the two neighbour-step prologues (f32
// input, Q8_0 weights) reached through their own entry points.
constexpr int kKindNorm = 100;  // x f32 [K] and gamma f32 [K]
constexpr int kKindSilu = 101;  // x = [gate | up] f32 [2K]

// Validate parts and the shared input, build the kernel's part table.
q8g_status prepare(int dt, const q8g_part *parts, int nparts, const void *x, const uint16_t *dx, int64_t K,
                   Parts &out, int64_t &n_total, const float *aux = nullptr)
{
    if (dt != Q8G_Q8_0 && dt != Q8G_BF16 && dt != Q8G_Q8_0_F32 && dt != Q8G_F16 && dt != kKindNorm &&
        dt != kKindSilu)
        return Q8G_ERR_ARG;
    if (!parts) return Q8G_ERR_NULL;
    if (nparts < 1 || nparts > kMaxParts) return Q8G_ERR_ARG;
    if (K < 0 || K > kMaxElems) return Q8G_ERR_SHAPE;
    const bool fused = dt == Q8G_Q8_0_F32 || dt == kKindNorm || dt == kKindSilu;  // x is f32, quantized in the launch
    const bool q8 = dt == Q8G_Q8_0 || fused;  // Q8_0 weights (codes + scales)
    if (q8 ? (K % 32) : (K % 8)) return Q8G_ERR_SHAPE;
    if (fused && K > kMaxFusedK) return Q8G_ERR_SHAPE;
    n_total = 0;
    for (int i = 0; i < nparts; ++i) {
        if (parts[i].n < 0 || parts[i].n > kMaxElems) return Q8G_ERR_SHAPE;
        if (parts[i].n > 0 && K > 0 && parts[i].n > kMaxElems / K) return Q8G_ERR_SHAPE;
        n_total += parts[i].n;
        if (n_total > kMaxElems) return Q8G_ERR_SHAPE;
    }
    for (int i = 0; i < kMaxParts; ++i) {
        out.w[i] = nullptr;
        out.dw[i] = nullptr;
        out.y[i] = nullptr;
        out.res[i] = nullptr;
        out.end[i] = INT64_MAX;
    }
    if (n_total == 0) return Q8G_OK;
    // with K == 0 no weight or activation byte is read, so those may be NULL
    if (K > 0 && (!x || (q8 && !fused && !dx) || (dt == kKindNorm && !aux))) return Q8G_ERR_NULL;
    if (!aligned(x, 16) || (q8 && !fused && !aligned(dx, 2)) || (dt == kKindNorm && !aligned(aux, 16)))
        return Q8G_ERR_ALIGN;
    if (fused) dx = nullptr;  // not read

    const int64_t xbytes = dt == kKindSilu ? 8 * K : fused ? 4 * K : (q8 ? K : 2 * K);
    const int64_t auxbytes = dt == kKindNorm ? 4 * K : 0;
    const int64_t dxbytes = (q8 && !fused) ? (K / 32) * 2 : 0;
    int64_t begin = 0;
    int slot = 0;
    for (int i = 0; i < nparts; ++i) {
        const q8g_part &pt = parts[i];
        if (pt.n == 0) continue;
        if (!pt.y || (K > 0 && (!pt.w || (q8 && !pt.dw)))) return Q8G_ERR_NULL;
        if (!aligned(pt.w, 16) || !aligned(pt.y, 4) || (pt.residual && !aligned(pt.residual, 4)) ||
            (q8 && !aligned(pt.dw, 2)))
            return Q8G_ERR_ALIGN;
        out.w[slot] = pt.w;
        out.dw[slot] = q8 ? pt.dw : nullptr;
        out.y[slot] = pt.y;
        out.res[slot] = pt.residual;
        begin += pt.n;
        out.end[slot] = begin;
        ++slot;
    }
    // every output against every input and every other output
    for (int i = 0; i < nparts; ++i) {
        const q8g_part &a = parts[i];
        if (a.n == 0) continue;
        const int64_t ybytes = a.n * 4;
        if (overlap(a.y, ybytes, x, xbytes) || overlap(a.y, ybytes, dx, dxbytes) ||
            overlap(a.y, ybytes, aux, auxbytes))
            return Q8G_ERR_OVERLAP;
        for (int j = 0; j < nparts; ++j) {
            const q8g_part &b = parts[j];
            if (b.n == 0) continue;
            const int64_t wbytes = b.n * (q8 ? K : 2 * K);
            const int64_t dwbytes = q8 ? b.n * (K / 32) * 2 : 0;
            if (overlap(a.y, ybytes, b.w, wbytes) || overlap(a.y, ybytes, q8 ? b.dw : nullptr, dwbytes))
                return Q8G_ERR_OVERLAP;
            // the residual may be exactly y of the same part, nothing else
            if (b.residual && !(i == j && b.residual == a.y) && overlap(a.y, ybytes, b.residual, b.n * 4))
                return Q8G_ERR_OVERLAP;
            if (i != j && overlap(a.y, ybytes, b.y, b.n * 4)) return Q8G_ERR_OVERLAP;
        }
    }
    return Q8G_OK;
}

q8g_status run(int dt, const q8g_part *parts, int nparts, const void *x, const uint16_t *dx, int64_t K,
               void *stream, Prologue pr = Prologue{nullptr, 0.0f})
{
    Parts p;
    int64_t n_total = 0;
    const q8g_status st = prepare(dt, parts, nparts, x, dx, K, p, n_total, pr.aux);
    if (st != Q8G_OK || n_total == 0) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    // with K == 0 no activation is read: the f32-input kinds run as the Q8 kind
    // (their kernels assume K >= 32)
    if (K == 0 && (dt == Q8G_Q8_0_F32 || dt == kKindNorm || dt == kKindSilu)) dt = Q8G_Q8_0;
    // the neighbour-step kinds launch like the fused f32-input kind
    const Config c = pick_config(dt == kKindNorm || dt == kKindSilu ? Q8G_Q8_0_F32 : (q8g_dtype)dt, n_total);
    const hipError_t e = dt == Q8G_Q8_0       ? dispatch_gemv<Dt::Q8>(c, p, x, dx, pr, K, n_total, s)
                         : dt == Q8G_Q8_0_F32 ? dispatch_gemv<Dt::Q8F32>(c, p, x, nullptr, pr, K, n_total, s)
                         : dt == kKindNorm    ? dispatch_gemv<Dt::Q8NORM>(c, p, x, nullptr, pr, K, n_total, s)
                         : dt == kKindSilu    ? dispatch_gemv<Dt::Q8SILU>(c, p, x, nullptr, pr, K, n_total, s)
                         : dt == Q8G_F16      ? dispatch_gemv<Dt::F16>(c, p, x, nullptr, pr, K, n_total, s)
                                              : dispatch_gemv<Dt::BF16>(c, p, x, dx, pr, K, n_total, s);
    return e == hipSuccess ? Q8G_OK : Q8G_ERR_LAUNCH;
}

bool eps_ok(float eps) { return eps >= 0.0f && eps <= 3.4e38f; }  // finite, not negative (NaN fails)

// Launch shape of the f32 silu(gate) * up epilogue (EPI 2): R rows per wave,
// W waves, R * W / 2 gate+up row pairs per workgroup (a divisor of 32).
// Measured on MI355X over the 0.8B MLP (F = 3584, K = 1024): R = 4, W = 8
// (16 pairs, 224 workgroups) 4.0 us; R = 4, W = 4 4.1; R = 2, W = 8 4.4;
// R = 2, W = 16 5.0; R = 1, W = 8 6.3.
constexpr int kSiluRows = 4, kSiluWaves = 8;
static_assert(32 % (kSiluRows * kSiluWaves / 2) == 0, "row pairs per workgroup divide 32");

template <Dt DT, int R, int W, int EPI>
hipError_t launch_epi(const Parts &p, const void *x, const uint16_t *dx, const float *gamma, float eps, int64_t K,
                      int64_t F, hipStream_t s, int8_t *qa, uint16_t *da)
{
    if constexpr (is_fused(DT))
        if (one_pass(K, W * kWave)) return launch_gemv<DT, R, W, EPI, false, 1>(p, x, dx, gamma, eps, K, 2 * F, s, qa, da);
    return launch_gemv<DT, R, W, EPI, false, 4>(p, x, dx, gamma, eps, K, 2 * F, s, qa, da);
}

// Gate+up projection (F rows each, Q8_0) with a = silu(gate) * up formed in the
// epilogue: quantized there (qa, da; a == nullptr) or written in f32 (a; qa and
// da nullptr). kind: Q8G_Q8_0 (x = codes + dx) or kKindNorm (x f32, normalized
// with gamma and eps in the prologue).
q8g_status gateup_silu(int kind, const int8_t *qg, const uint16_t *dg, const int8_t *qu, const uint16_t *du, int64_t F,
                       const void *x, const uint16_t *dx, const float *gamma, float eps, int8_t *qa, uint16_t *da,
                       float *a, int64_t K, void *stream)
{
    if (F < 0 || F % 32 || F > kMaxElems / 2 || K < 0 || K % 32 || K > kMaxElems) return Q8G_ERR_SHAPE;
    if (K > 0 && F > kMaxElems / K) return Q8G_ERR_SHAPE;
    if (kind == kKindNorm && (K > kMaxFusedK)) return Q8G_ERR_SHAPE;
    if (kind == kKindNorm && !eps_ok(eps)) return Q8G_ERR_ARG;
    if (F == 0) return Q8G_OK;
    const bool f32_out = a != nullptr;
    if (!f32_out && (!qa || !da)) return Q8G_ERR_NULL;
    if (K > 0 && (!qg || !dg || !qu || !du || !x || (kind == Q8G_Q8_0 && !dx) || (kind == kKindNorm && !gamma)))
        return Q8G_ERR_NULL;
    if (!aligned(qg, 16) || !aligned(qu, 16) || !aligned(dg, 2) || !aligned(du, 2) || !aligned(x, 16) ||
        (!f32_out && (!aligned(qa, 16) || !aligned(da, 2))) || (f32_out && !aligned(a, 4)) ||
        (kind == Q8G_Q8_0 && !aligned(dx, 2)) || (kind == kKindNorm && !aligned(gamma, 16)))
        return Q8G_ERR_ALIGN;
    const int64_t wbytes = F * K, dwbytes = F * (K / 32) * 2;
    const int64_t xbytes = kind == kKindNorm ? 4 * K : K;
    const int64_t dxbytes = kind == Q8G_Q8_0 ? (K / 32) * 2 : 0;
    const int64_t gbytes = kind == kKindNorm ? 4 * K : 0;
    const int64_t qabytes = F, dabytes = (F / 32) * 2, abytes = 4 * F;
    const void *ins[6] = {qg, dg, qu, du, x, kind == Q8G_Q8_0 ? static_cast<const void *>(dx) : gamma};
    const int64_t inbytes[6] = {wbytes, dwbytes, wbytes, dwbytes, xbytes, kind == Q8G_Q8_0 ? dxbytes : gbytes};
    for (int i = 0; i < 6; ++i) {
        if (f32_out && overlap(a, abytes, ins[i], inbytes[i])) return Q8G_ERR_OVERLAP;
        if (!f32_out && (overlap(qa, qabytes, ins[i], inbytes[i]) || overlap(da, dabytes, ins[i], inbytes[i])))
            return Q8G_ERR_OVERLAP;
    }
    if (!f32_out && overlap(qa, qabytes, da, dabytes)) return Q8G_ERR_OVERLAP;

    Parts p;
    for (int i = 0; i < kMaxParts; ++i) {
        p.w[i] = nullptr;
        p.dw[i] = nullptr;
        p.y[i] = nullptr;
        p.res[i] = nullptr;
        p.end[i] = INT64_MAX;
    }
    p.w[0] = qg;
    p.dw[0] = dg;
    p.end[0] = F;
    p.w[1] = qu;
    p.dw[1] = du;
    p.end[1] = 2 * F;
    p.y[0] = a;  // EPI 2 writes a through part 0's output; EPI 1 writes no f32 output
    const hipStream_t s = static_cast<hipStream_t>(stream);
    // with K == 0 no activation is read: gate = up = 0, a = 0
    const bool norm = kind == kKindNorm && K > 0;
    const void *xq = kind == Q8G_Q8_0 ? x : nullptr;
    const uint16_t *dxq = kind == Q8G_Q8_0 ? dx : nullptr;
    constexpr int SR = kSiluRows, SW = kSiluWaves;
    const hipError_t e =
        f32_out ? (norm ? launch_epi<Dt::Q8NORM, SR, SW, 2>(p, x, nullptr, gamma, eps, K, F, s, nullptr, nullptr)
                        : launch_epi<Dt::Q8, SR, SW, 2>(p, xq, dxq, nullptr, 0.0f, K, F, s, nullptr, nullptr))
                : (norm ? launch_epi<Dt::Q8NORM, 4, 16, 1>(p, x, nullptr, gamma, eps, K, F, s, qa, da)
                        : launch_epi<Dt::Q8, 4, 16, 1>(p, xq, dxq, nullptr, 0.0f, K, F, s, qa, da));
    return e == hipSuccess ? Q8G_OK : Q8G_ERR_LAUNCH;
}

}  // namespace

extern "C" {

q8g_status q8_quantize_act(const float *x, int8_t *qx, uint16_t *dx, int64_t K, void *stream)
{
    if (K < 0 || K > kMaxElems || K % 32) return Q8G_ERR_SHAPE;
    if (K == 0) return Q8G_OK;
    if (!x || !qx || !dx) return Q8G_ERR_NULL;
    if (!aligned(x, 16) || !aligned(qx, 16) || !aligned(dx, 2)) return Q8G_ERR_ALIGN;
    if (overlap(qx, K, x, 4 * K) || overlap(dx, K / 16, x, 4 * K) || overlap(qx, K, dx, K / 16))
        return Q8G_ERR_OVERLAP;
    const int64_t threads = K / 4;
    const int64_t blocks = (threads + 255) / 256;
    if (blocks > 0x7FFFFFFF) return Q8G_ERR_SHAPE;
    const float *xc = x;
    int8_t *qc = qx;
    uint16_t *dc = dx;
    int64_t kc = K;
    void *args[] = {&xc, &qc, &dc, &kc};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&quantize_kernel), dim3((unsigned)blocks),
                                         dim3(256), args, 0, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? Q8G_OK : Q8G_ERR_LAUNCH;
}

q8g_status q8_gemv(const int8_t *qw, const uint16_t *dw, const int8_t *qx, const uint16_t *dx,
                   const float *residual, float *y, int64_t N, int64_t K, void *stream)
{
    if (N < 0) return Q8G_ERR_SHAPE;
    const q8g_part part = {qw, dw, N, y, residual};
    return run(Q8G_Q8_0, &part, 1, qx, dx, K, stream);
}

q8g_status bf16_gemv(const uint16_t *w, const uint16_t *x, const float *residual, float *y, int64_t N, int64_t K,
                     void *stream)
{
    if (N < 0) return Q8G_ERR_SHAPE;
    const q8g_part part = {w, nullptr, N, y, residual};
    return run(Q8G_BF16, &part, 1, x, nullptr, K, stream);
}

q8g_status f16_gemv(const uint16_t *w, const uint16_t *x, const float *residual, float *y, int64_t N, int64_t K,
                    void *stream)
{
    if (N < 0) return Q8G_ERR_SHAPE;
    const q8g_part part = {w, nullptr, N, y, residual};
    return run(Q8G_F16, &part, 1, x, nullptr, K, stream);
}

q8g_status gemv_stacked(q8g_dtype dtype, const q8g_part *parts, int nparts, const void *x, const uint16_t *dx,
                        int64_t K, void *stream)
{
    if (dtype == Q8G_PTQ1_0) return q8g::ptq1_stacked(parts, nparts, static_cast<const int8_t *>(x), dx, K, stream);
    if (dtype != Q8G_Q8_0 && dtype != Q8G_BF16 && dtype != Q8G_Q8_0_F32 && dtype != Q8G_F16) return Q8G_ERR_ARG;
    return run(dtype, parts, nparts, x, dx, K, stream);
}

q8g_status q8_rmsnorm_quantize_act_batch(const float *x, const float *gamma, float eps, int8_t *qx, uint16_t *dx,
                                         int64_t K, int64_t B, void *stream)
{
    if (K < 0 || K > kMaxFusedK || K % 32 || B < 0 || B > kMaxBatchVectors) return Q8G_ERR_SHAPE;
    if (!eps_ok(eps)) return Q8G_ERR_ARG;
    if (K == 0 || B == 0) return Q8G_OK;
    if (!x || !gamma || !qx || !dx) return Q8G_ERR_NULL;
    if (!aligned(x, 16) || !aligned(gamma, 16) || !aligned(qx, 16) || !aligned(dx, 2)) return Q8G_ERR_ALIGN;
    const int64_t xb = 4 * K * B, qb = K * B, db = (K / 16) * B;
    if (overlap(qx, qb, x, xb) || overlap(qx, qb, gamma, 4 * K) || overlap(dx, db, x, xb) ||
        overlap(dx, db, gamma, 4 * K) || overlap(qx, qb, dx, db))
        return Q8G_ERR_OVERLAP;
    const float *xc = x, *gc = gamma;
    float ec = eps;
    int8_t *qc = qx;
    uint16_t *dc = dx;
    int64_t kc = K;
    void *args[] = {&xc, &gc, &ec, &qc, &dc, &kc};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&norm_quantize_kernel), dim3((unsigned)B),
                                         dim3(kNormThreads), args, 0, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? Q8G_OK : Q8G_ERR_LAUNCH;
}

q8g_status q8_rmsnorm_quantize_act(const float *x, const float *gamma, float eps, int8_t *qx, uint16_t *dx, int64_t K,
                                   void *stream)
{
    return q8_rmsnorm_quantize_act_batch(x, gamma, eps, qx, dx, K, 1, stream);
}

q8g_status q8_silu_mul_quantize_act_batch(const float *gu, int8_t *qx, uint16_t *dx, int64_t K, int64_t B,
                                          void *stream)
{
    if (K < 0 || K % 32 || B < 0 || B > kMaxBatchVectors) return Q8G_ERR_SHAPE;
    if (B > 0 && K > kMaxElems / 2 / B) return Q8G_ERR_SHAPE;
    if (K == 0 || B == 0) return Q8G_OK;
    if (!gu || !qx || !dx) return Q8G_ERR_NULL;
    if (!aligned(gu, 16) || !aligned(qx, 16) || !aligned(dx, 2)) return Q8G_ERR_ALIGN;
    const int64_t gb = 8 * K * B, qb = K * B, db = (K / 16) * B;
    if (overlap(qx, qb, gu, gb) || overlap(dx, db, gu, gb) || overlap(qx, qb, dx, db)) return Q8G_ERR_OVERLAP;
    const int64_t blocks = (K / 4 + 255) / 256;
    if (blocks > 0x7FFFFFFF) return Q8G_ERR_SHAPE;
    const float *gc = gu;
    int8_t *qc = qx;
    uint16_t *dc = dx;
    int64_t kc = K;
    void *args[] = {&gc, &qc, &dc, &kc};
    const hipError_t e =
        hipLaunchKernel(reinterpret_cast<const void *>(&silu_quantize_kernel), dim3((unsigned)blocks, (unsigned)B),
                        dim3(256), args, 0, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? Q8G_OK : Q8G_ERR_LAUNCH;
}

q8g_status q8_silu_mul_quantize_act(const float *gu, int8_t *qx, uint16_t *dx, int64_t K, void *stream)
{
    return q8_silu_mul_quantize_act_batch(gu, qx, dx, K, 1, stream);
}

q8g_status gemv_stacked_rmsnorm(const q8g_part *parts, int nparts, const float *x, const float *gamma, float eps,
                                int64_t K, void *stream)
{
    if (!eps_ok(eps)) return Q8G_ERR_ARG;
    return run(kKindNorm, parts, nparts, x, nullptr, K, stream, Prologue{gamma, eps});
}

q8g_status q8_gemv_silu_mul(const int8_t *qw, const uint16_t *dw, const float *gu, const float *residual, float *y,
                            int64_t N, int64_t K, void *stream)
{
    if (N < 0) return Q8G_ERR_SHAPE;
    const q8g_part part = {qw, dw, N, y, residual};
    return run(kKindSilu, &part, 1, gu, nullptr, K, stream);
}

q8g_status q8_gateup_silu_quantize(const int8_t *qw_gate, const uint16_t *dw_gate, const int8_t *qw_up,
                                   const uint16_t *dw_up, int64_t F, const int8_t *qx, const uint16_t *dx, int64_t K,
                                   int8_t *qa, uint16_t *da, void *stream)
{
    return gateup_silu(Q8G_Q8_0, qw_gate, dw_gate, qw_up, dw_up, F, qx, dx, nullptr, 0.0f, qa, da, nullptr, K, stream);
}

q8g_status q8_gateup_rmsnorm_silu_quantize(const int8_t *qw_gate, const uint16_t *dw_gate, const int8_t *qw_up,
                                           const uint16_t *dw_up, int64_t F, const float *x, const float *gamma,
                                           float eps, int64_t K, int8_t *qa, uint16_t *da, void *stream)
{
    return gateup_silu(kKindNorm, qw_gate, dw_gate, qw_up, dw_up, F, x, nullptr, gamma, eps, qa, da, nullptr, K,
                       stream);
}

q8g_status q8_gateup_silu(const int8_t *qw_gate, const uint16_t *dw_gate, const int8_t *qw_up, const uint16_t *dw_up,
                          int64_t F, const int8_t *qx, const uint16_t *dx, int64_t K, float *a, void *stream)
{
    if (!a && F > 0) return Q8G_ERR_NULL;
    return gateup_silu(Q8G_Q8_0, qw_gate, dw_gate, qw_up, dw_up, F, qx, dx, nullptr, 0.0f, nullptr, nullptr, a, K,
                       stream);
}

q8g_status q8_gateup_rmsnorm_silu(const int8_t *qw_gate, const uint16_t *dw_gate, const int8_t *qw_up,
                                  const uint16_t *dw_up, int64_t F, const float *x, const float *gamma, float eps,
                                  int64_t K, float *a, void *stream)
{
    if (!a && F > 0) return Q8G_ERR_NULL;
    return gateup_silu(kKindNorm, qw_gate, dw_gate, qw_up, dw_up, F, x, nullptr, gamma, eps, nullptr, nullptr, a, K,
                       stream);
}

q8g_status q8g_gemv_config(q8g_dtype dtype, int64_t n_total, int64_t K, int *rows, int *waves)
{
    if (dtype == Q8G_PTQ1_0) {
        if (!rows || !waves) return Q8G_ERR_NULL;
        return q8g::ptq1_config(n_total, K, rows, waves);
    }
    if (dtype != Q8G_Q8_0 && dtype != Q8G_BF16 && dtype != Q8G_Q8_0_F32 && dtype != Q8G_F16) return Q8G_ERR_ARG;
    if (n_total < 0 || K < 0) return Q8G_ERR_SHAPE;
    if (!rows || !waves) return Q8G_ERR_NULL;
    const Config c = pick_config(dtype, n_total);
    *rows = c.rows;
    *waves = c.waves;
    return Q8G_OK;
}

const char *q8g_status_str(int status)
{
    switch (status) {
    case Q8G_OK: return "ok";
    case Q8G_ERR_NULL: return "a required pointer is NULL";
    case Q8G_ERR_SHAPE: return "invalid shape (negative size, K not a multiple of the block, or overflow)";
    case Q8G_ERR_ALIGN: return "misaligned pointer";
    case Q8G_ERR_ARG: return "invalid argument (dtype or part count)";
    case Q8G_ERR_LAUNCH: return "kernel launch failed";
    case Q8G_ERR_OVERLAP: return "an output overlaps an input or another output";
    default: return "unknown status";
    }
}

}  // extern "C"
