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
//    at lane distance 1 and 2 (DPP quad_perm), 4, 8 and 16 (ds_swizzle in xor
//    mode) and 32 (ds_bpermute). While two or more rows remain per lane, each
//    step keeps half of them and adds the partner's copy of that half, so R
//    rows cost R-1 exchanges plus the six of a single sum. The tree always
//    pairs lanes at distance 1, 2, 4, ..., 32, so a row's bits do not depend on
//    R, on its slot in the wave, or on whether it sits in a stacked launch.
//  * Rows past the last one are masked (no load, no store): the pages report a
//    tail that wrote rows beyond the output.
//  * Weights and weight scales are read once per call, so they are loaded
//    with the nontemporal hint; the activation, shared by every wave, is not.
//  * No atomics, no LDS staging, no scratch: results depend on the shape only.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemv_device.hpp"
#include "q8gemv.h"

namespace {

using namespace q8g;

constexpr int kMaxParts = 4;

// Q8: x = int8 codes + binary16 scales; BF16: x = bf16; Q8F32: x = f32, quantized
// by every workgroup into LDS before use (one launch instead of two).
enum class Dt { Q8, BF16, Q8F32 };

constexpr int kMaxFusedK = 16384;  // LDS bytes for the codes of a fused launch

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

// Q8_0 arithmetic of one chunk for R rows, given this lane's weight codes and
// scale bits, its activation codes and its activation scale (0 on odd and on
// inactive lanes): one exact int32 block sum per row, scaled by dw*dx, one fma.
template <int R>
__device__ __forceinline__ void q8_chunk_compute(const int4 (&wv)[R], const uint16_t (&ws)[R], const int4 &xq,
                                                 float xs, float (&acc)[R])
{
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int s = q8_block_sum(wv[r], xq);  // the block's exact int32 sum
        acc[r] = __builtin_fmaf((float)s, f16_bits_to_f32(ws[r]) * xs, acc[r]);
    }
}

template <bool SCALES, int R>
__device__ __forceinline__ void chunk_load(const RowRef (&rows)[R], int64_t off, int4 (&wv)[R], uint16_t (&ws)[R])
{
#pragma unroll
    for (int r = 0; r < R; ++r) wv[r] = load16_stream(rows[r].w + off);
    if constexpr (SCALES) {
#pragma unroll
        for (int r = 0; r < R; ++r) ws[r] = load_u16_stream(rows[r].dw + (off >> 5));
    }
}

// One 1 KiB chunk of R rows: lane l covers bytes [off, off+16) of each row.
// Inactive lanes (ragged tail) load in-bounds data and contribute zero.
template <Dt DT, int R>
__device__ __forceinline__ void chunk_step(const RowRef (&rows)[R], const void *__restrict__ xv,
                                           const uint16_t *__restrict__ dx, int64_t off, bool active,
                                           float even, float (&acc)[R])
{
    int4 wv[R];
    uint16_t ws[R];
    chunk_load<DT == Dt::Q8>(rows, off, wv, ws);
    const int4 xq = load16(static_cast<const char *>(xv) + off);
    if constexpr (DT == Dt::Q8) {
        const float xs = active ? f16_bits_to_f32(dx[off >> 5]) * even : 0.0f;
        q8_chunk_compute<R>(wv, ws, xq, xs, acc);
    } else {
        float xf[8];
        bf16_unpack(xq, xf);
#pragma unroll
        for (int i = 0; i < 8; ++i) xf[i] = active ? xf[i] : 0.0f;
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] += bf16_chunk_dot(wv[r], xf);
    }
}

// Reduce the R row sums of a wave and write them (+ residual, added once).
// Row i is written by lane lane_of<R>(i); the loop index is a compile-time
// constant, so every row pointer stays a scalar (no indexed private array).
template <int R>
__device__ __forceinline__ void reduce_and_store(float (&acc)[R], const RowRef (&rows)[R], const bool (&valid)[R],
                                                 int lane)
{
    const float total = wave_reduce_rows<R>(acc, lane);
#pragma unroll
    for (int i = 0; i < R; ++i)
        if (valid[i] && lane == lane_of<R>(i)) *rows[i].y = rows[i].res ? total + *rows[i].res : total;
}

// y[rows] = W[rows] · x (+ residual) for the R rows owned by each wave.
template <Dt DT, int R, int WAVES>
__global__ __launch_bounds__(WAVES *kWave) void gemv_kernel(PARTS_PARAMS, const void *__restrict__ xv,
                                                            const uint16_t *__restrict__ dx,
                                                            int64_t K, int64_t n_total)
{
    const int lane = threadIdx.x & (kWave - 1);
    // wave-uniform by construction; readfirstlane lets the compiler keep the
    // row bookkeeping and the part table in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t row0 = ((int64_t)blockIdx.x * WAVES + wave) * R;
    if (row0 >= n_total) return;  // wave-uniform

    const int64_t row_bytes = DT == Dt::Q8 ? K : 2 * K;
    const int64_t nb = K / 32;

    RowRef rows[R];
    bool valid[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        valid[r] = row0 + r < n_total;
        LOCATE(valid[r] ? row0 + r : row0, row_bytes, nb, rows[r]);
    }

    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.0f;

    // Q8_0: only the even lane of a block pair applies the block scale.
    const float even = (lane & 1) ? 0.0f : 1.0f;

    // Whole 1 KiB chunks need no masking. All loads of a chunk are issued
    // before any of them is consumed, with no branch in between, so a wave
    // keeps R+1 16-byte loads (and R+1 scale loads) in flight per chunk.
    const int64_t full = row_bytes / kChunk;
    for (int64_t c = 0; c < full; ++c)
        chunk_step<DT, R>(rows, xv, dx, c * kChunk + (int64_t)lane * 16, true, even, acc);
    // Ragged tail (K not a multiple of the chunk): lanes past the row end
    // load from offset 0 of their row (always in bounds) and contribute zero.
    if (full * kChunk < row_bytes) {
        const int64_t off = full * kChunk + (int64_t)lane * 16;
        const bool active = off < row_bytes;
        chunk_step<DT, R>(rows, xv, dx, active ? off : 0, active, even, acc);
    }

    reduce_and_store<R>(acc, rows, valid, lane);
}

// y = Q8_0 W · quantize(x) (+ residual) with x in f32: every workgroup issues
// its first chunk of weight loads, then quantizes x into LDS (the arithmetic
// of q8_quantize_act) while they are in flight, then proceeds as gemv_kernel
// does with the codes read from LDS. Bit-identical to q8_quantize_act followed
// by the Q8 gemv_kernel.
template <int R, int WAVES>
__global__ __launch_bounds__(WAVES *kWave) void gemv_q8_f32x_kernel(PARTS_PARAMS, const void *__restrict__ xv,
                                                                    const uint16_t *__restrict__ unused,
                                                                    int64_t K, int64_t n_total)
{
    __shared__ __align__(16) int8_t s_qx[kMaxFusedK];
    __shared__ float s_dx[kMaxFusedK / 32];
    (void)unused;
    const float *x = static_cast<const float *>(xv);
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t row0 = ((int64_t)blockIdx.x * WAVES + wave) * R;
    const bool has_rows = row0 < n_total;  // wave-uniform; waves without rows still quantize
    const int64_t nb = K / 32;

    RowRef rows[R];
    bool valid[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        valid[r] = row0 + r < n_total;
        LOCATE(valid[r] ? row0 + r : (has_rows ? row0 : 0), K, nb, rows[r]);
    }
    const int64_t nchunk = (K + kChunk - 1) / kChunk;
    int4 wv[R];
    uint16_t ws[R];
    const int64_t off0 = (int64_t)lane * 16;
    const bool active0 = off0 < K;
    if (has_rows && nchunk > 0) chunk_load<true>(rows, active0 ? off0 : 0, wv, ws);

    for (int64_t e = (int64_t)threadIdx.x * 4; e < K; e += 4 * WAVES * kWave) {
        const float4 v = *reinterpret_cast<const float4 *>(x + e);
        float d;
        const uint32_t packed = quantize4(v, &d);
        *reinterpret_cast<uint32_t *>(s_qx + e) = packed;
        if ((lane & 7) == 0) s_dx[e >> 5] = f16_bits_to_f32(scale_bits(d));
    }
    __syncthreads();
    if (!has_rows) return;

    const float even = (lane & 1) ? 0.0f : 1.0f;
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.0f;
    for (int64_t c = 0; c < nchunk; ++c) {
        const int64_t off = c * kChunk + off0;
        const bool active = off < K;
        const int64_t o = active ? off : 0;
        if (c > 0) chunk_load<true>(rows, o, wv, ws);
        const int4 xq = *reinterpret_cast<const int4 *>(s_qx + o);
        const float xs = active ? s_dx[o >> 5] * even : 0.0f;
        q8_chunk_compute<R>(wv, ws, xq, xs, acc);
    }
    reduce_and_store<R>(acc, rows, valid, lane);
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

// ---- host side ---------------------------------------------------------------

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlap(const void *a, int64_t abytes, const void *b, int64_t bbytes)
{
    if (!a || !b || abytes <= 0 || bbytes <= 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

constexpr int64_t kMaxElems = (int64_t)1 << 60;

struct Input {
    const void *p;
    int64_t bytes;
};

template <Dt DT, int R, int WAVES>
hipError_t launch_gemv(const Parts &p, const void *x, const uint16_t *dx, int64_t K, int64_t n_total,
                       hipStream_t s)
{
    const int64_t rows_per_block = (int64_t)R * WAVES;
    const int64_t blocks = (n_total + rows_per_block - 1) / rows_per_block;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    Parts pc = p;
    const void *xc = x;
    const uint16_t *dxc = dx;
    int64_t kc = K, nc = n_total;
    void *args[] = {&pc.w[0],   &pc.w[1],   &pc.w[2],   &pc.w[3],   &pc.dw[0],  &pc.dw[1], &pc.dw[2],
                    &pc.dw[3],  &pc.y[0],   &pc.y[1],   &pc.y[2],   &pc.y[3],   &pc.res[0], &pc.res[1],
                    &pc.res[2], &pc.res[3], &pc.end[0], &pc.end[1], &pc.end[2], &xc,       &dxc,
                    &kc,        &nc};
    const void *fn;
    if constexpr (DT == Dt::Q8F32)
        fn = reinterpret_cast<const void *>(&gemv_q8_f32x_kernel<R, WAVES>);
    else
        fn = reinterpret_cast<const void *>(&gemv_kernel<DT, R, WAVES>);
    return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(WAVES * kWave), args, 0, s);
}

// Rows per wave: as many as keep at least ~8 waves per CU in flight.
constexpr int kWavesPerGroup = 4;
constexpr int kWavesPerFusedGroup = 8;  // fewer, larger groups: each one quantizes x

int rows_per_wave(int64_t n_total)
{
    const int64_t target_waves = 256 * 8;
    if (n_total >= 4 * target_waves) return 4;
    if (n_total >= 2 * target_waves) return 2;
    return 1;
}

template <Dt DT>
hipError_t dispatch_gemv(const Parts &p, const void *x, const uint16_t *dx, int64_t K, int64_t n_total,
                         hipStream_t s)
{
    constexpr int W = DT == Dt::Q8F32 ? kWavesPerFusedGroup : kWavesPerGroup;
    switch (rows_per_wave(n_total)) {
    case 4: return launch_gemv<DT, 4, W>(p, x, dx, K, n_total, s);
    case 2: return launch_gemv<DT, 2, W>(p, x, dx, K, n_total, s);
    default: return launch_gemv<DT, 1, W>(p, x, dx, K, n_total, s);
    }
}

// Validate parts and the shared input, build the kernel's part table.
q8g_status prepare(q8g_dtype dt, const q8g_part *parts, int nparts, const void *x, const uint16_t *dx, int64_t K,
                   Parts &out, int64_t &n_total)
{
    if (dt != Q8G_Q8_0 && dt != Q8G_BF16 && dt != Q8G_Q8_0_F32) return Q8G_ERR_ARG;
    if (!parts) return Q8G_ERR_NULL;
    if (nparts < 1 || nparts > kMaxParts) return Q8G_ERR_ARG;
    if (K < 0 || K > kMaxElems) return Q8G_ERR_SHAPE;
    const bool q8 = dt != Q8G_BF16;          // Q8_0 weights (codes + scales)
    const bool fused = dt == Q8G_Q8_0_F32;   // x is f32, quantized in the launch
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
    if (K > 0 && (!x || (q8 && !fused && !dx))) return Q8G_ERR_NULL;
    if (!aligned(x, 16) || (q8 && !fused && !aligned(dx, 2))) return Q8G_ERR_ALIGN;
    if (fused) dx = nullptr;  // not read

    const int64_t xbytes = fused ? 4 * K : (q8 ? K : 2 * K);
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
        if (overlap(a.y, ybytes, x, xbytes) || overlap(a.y, ybytes, dx, dxbytes)) return Q8G_ERR_OVERLAP;
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

q8g_status run(q8g_dtype dt, const q8g_part *parts, int nparts, const void *x, const uint16_t *dx, int64_t K,
               void *stream)
{
    Parts p;
    int64_t n_total = 0;
    const q8g_status st = prepare(dt, parts, nparts, x, dx, K, p, n_total);
    if (st != Q8G_OK || n_total == 0) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e = dt == Q8G_Q8_0       ? dispatch_gemv<Dt::Q8>(p, x, dx, K, n_total, s)
                         : dt == Q8G_Q8_0_F32 ? dispatch_gemv<Dt::Q8F32>(p, x, nullptr, K, n_total, s)
                                              : dispatch_gemv<Dt::BF16>(p, x, dx, K, n_total, s);
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

q8g_status gemv_stacked(q8g_dtype dtype, const q8g_part *parts, int nparts, const void *x, const uint16_t *dx,
                        int64_t K, void *stream)
{
    return run(dtype, parts, nparts, x, dx, K, stream);
}

q8g_status q8g_gemv_config(q8g_dtype dtype, int64_t n_total, int64_t K, int *rows, int *waves)
{
    if (dtype != Q8G_Q8_0 && dtype != Q8G_BF16 && dtype != Q8G_Q8_0_F32) return Q8G_ERR_ARG;
    if (n_total < 0 || K < 0) return Q8G_ERR_SHAPE;
    if (!rows || !waves) return Q8G_ERR_NULL;
    *rows = rows_per_wave(n_total);
    *waves = dtype == Q8G_Q8_0_F32 ? kWavesPerFusedGroup : kWavesPerGroup;
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
