// PTQ1_0 ternary decode GEMV for CDNA4 (gfx950) and its C ABI.
//
// What is computed is stated in include/q8gemv.h, after "Filling in the blanks:
// Inference using Phobos", section PrismML Ternary-Bonsai: weights -1, 0 or +1,
// 128 of them in 28 bytes, against an activation rotated by a Hadamard
// transform; one rotation per input serves every projection that consumes it.
//
// Design (MI355X, wave64):
//  * Rotation: one workgroup per 128-value block, one output per thread. Each
//    output is the f64 sum of the block's inputs with the signs of its
//    Hadamard row, in ascending index order (128 dependent adds, about a
//    microsecond), divided by sqrt(128) and rounded once to f32; the block is
//    then quantized with the arithmetic of q8_quantize_act over 128 values.
//    The f64 sum in index order is the definition itself, so the rotated
//    values and codes do not depend on how the work is split.
//  * GEMV: a base-3 byte holds five weights, so at HBM speed (about 11 weight
//    bytes per clock per compute unit) the decode, not the memory, is the
//    limit: a compute unit issues 64 lane operations per clock, about six per
//    weight byte. Per weight byte this kernel spends one v_perm (it forms the
//    table address), one 8-byte LDS read and two v_dot4:
//      - a table in LDS maps each byte value to the trits of its five digits:
//        digits 0-3 as four int8 and digit 4 as one int8. It is held 32 times,
//        8 bytes per copy side by side, one copy per lane of a half-wave, so
//        the lanes of one LDS cycle never share a bank; one v_perm places the
//        weight byte at bits 8-15 and the lane's copy offset at bits 0-7;
//      - two lanes share a block: half 0 takes trit bytes 0-12, half 1 trit
//        bytes 13-25 and the scale. Each reads 16 bytes per step (block bytes
//        0-15, or 12-27 shifted down by one byte with v_alignbyte), so a lane
//        holds 4 registers per step in flight;
//      - a lane pair owns one block column c of the matrix for the whole
//        launch. Each half's 65 activation codes are packed once into
//        registers as the table entries need them: codes 5q..5q+3 in one
//        dword and code 5q+4 in another, for each of its 13 trit bytes q;
//      - a wave covers C consecutive block columns of R = 32 / C rows per
//        step, so each load instruction reads R runs of C * 28 contiguous
//        bytes; W waves cover the nb block columns of a row, and a workgroup
//        holds G such groups of W waves (up to 16 waves).
//    Small per-lane state (26 activation registers, 4 per step in flight,
//    74 VGPRs in all) leaves the table as the occupancy limit: two workgroups
//    per compute unit (10 waves at K = 5120), whose table reads and weight
//    loads wait while the other waves compute.
//  * The two halves' int32 sums are joined (one DPP add) into the block's
//    exact sum; times f16(s) * f16(dx) (exact in f32: 11 + 11 significant
//    bits) it is the block's term, formed by half 1. The C lanes of a row are summed
//    by a butterfly at lane distances 1, 2, ..., C/2; the W wave partials of
//    a row go through LDS and are added in wave order, then the residual.
//    C and W depend on K only, so a row's bits do not depend on N, on the
//    tiling or on the row's part in a stacked call.
//  * Each wave keeps four steps of weights in flight. Loads are unconditional
//    except in the last steps (rows past the part's end re-read its last row
//    and are masked), so the compiler can count them; no load goes past the
//    group's rows, and the barriers wait for LDS only, not for loads.
//  * No atomics and no scratch; LDS holds the table and the wave partials.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "gemv_device.hpp"
#include "ptq1.hpp"
#include "q8gemv.h"

namespace q8g {
namespace {

constexpr int kPtqBlock = Q8G_PTQ1_BLOCK;  // weights per block
constexpr int kPtqBytes = Q8G_PTQ1_BYTES;  // bytes per block
constexpr int kTritBytes = 26;             // bytes of base-3 digits per block
constexpr int kHalfBytes = kTritBytes / 2; // trit bytes per lane: two lanes share a block
constexpr int kLutCopies = 32;             // table copies, one per lane of a half-wave
constexpr int kLutStride = 8 * kLutCopies; // bytes per byte value: its entry in every copy
constexpr int kLutBytes = 256 * kLutStride;
constexpr int kMaxWaves = 16;              // waves per workgroup
constexpr int kWaveCap = 8;                // waves per workgroup the launch shape aims for
constexpr int kTargetGroups = 512;         // two workgroups per compute unit
constexpr int kMaxPartialBytes = 16384;    // LDS for wave partials per workgroup
constexpr int kMaxSteps = 1 << 16;         // wave steps per group
constexpr int64_t kMaxRows = Q8G_PTQ1_MAX_ROWS;  // rows per part: row indexes stay 32-bit
constexpr int kMaxCols = kMaxWaves * kWave / 2;  // block columns: one per lane pair of 16 waves
constexpr int64_t kMaxK = (int64_t)kMaxCols * kPtqBlock;
static_assert(kMaxK == Q8G_PTQ1_MAX_K, "the largest K is one block column per lane pair of 16 waves");


// Table entry of byte value v (0..255): the trits (digit - 1) of its base-3
// digits 0..3 as four int8 (digit k in byte k), and of digit 4 as an int8 in
// byte 0 of the second word. Digit k of v is floor(v / 3^k) mod 3, also for the
// byte values 243..255 that a valid block never holds.
__device__ __forceinline__ uint2 lut_entry(int v)
{
    uint32_t lo = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        lo |= (uint32_t)(uint8_t)(int8_t)(v % 3 - 1) << (8 * k);
        v /= 3;
    }
    return make_uint2(lo, (uint32_t)(uint8_t)(int8_t)(v % 3 - 1));
}

// ---- rotation and quantization ------------------------------------------------

__global__ __launch_bounds__(kPtqBlock) void rotate_kernel(const float *__restrict__ x, float *__restrict__ rot,
                                                           int8_t *__restrict__ qx, uint16_t *__restrict__ dx,
                                                           double root)
{
    __shared__ double xs[kPtqBlock];
    __shared__ float wmax[2];
    const int i = threadIdx.x;
    const int64_t base = (int64_t)blockIdx.x * kPtqBlock;
    xs[i] = (double)x[base + i];
    __syncthreads();
    // row i of the Sylvester Hadamard matrix: sign (-1)^popcount(i & j)
    double acc = 0.0;
#pragma unroll 16
    for (int j = 0; j < kPtqBlock; ++j) {
        const double v = xs[j];
        acc += (__builtin_popcount(i & j) & 1) ? -v : v;
    }
    const float r = (float)(acc / root);  // f64 quotient, correctly rounded, then once to f32
    float m = fabsf(r);
    m = xmax<1>(m);
    m = xmax<2>(m);
    m = xmax<4>(m);
    m = xmax<8>(m);
    m = xmax<16>(m);
    m = xmax<32>(m);
    if ((i & 63) == 0) wmax[i >> 6] = m;
    __syncthreads();
    m = fmaxf(wmax[0], wmax[1]);
    const float d = m / 127.0f;  // correctly rounded f32 division
    int8_t q = 0;
    if (d != 0.0f) {
        float t = __builtin_rintf(r / d);  // round half to even
        t = fminf(fmaxf(t, -127.0f), 127.0f);
        q = (int8_t)(int)t;
    }
    qx[base + i] = q;
    if (rot) rot[base + i] = r;
    if (i == 0) dx[blockIdx.x] = scale_bits(d);
}

// ---- the GEMV -------------------------------------------------------------------

// Stacked parts as separate scalar arguments. Each workgroup works on one part:
// workgroups [b_{p-1}, b_p) cover part p (b0 = 0), so the part is the same for
// every lane of a workgroup and is picked once, with scalar selects.
#define PTQ_PARTS_PARAMS                                                                                   \
    const uint8_t *w0, const uint8_t *w1, const uint8_t *w2, const uint8_t *w3, float *y0, float *y1,     \
        float *y2, float *y3, const float *r0, const float *r1, const float *r2, const float *r3, int n0, \
        int n1, int n2, int n3, int b1, int b2, int b3

// v_perm selector: byte 0 from src1 byte 0 (the copy offset), byte 1 from
// src0 byte B (the weight byte), bytes 2 and 3 zero.
template <int B>
constexpr uint32_t addr_sel()
{
    return 0x0C0C0000u | ((uint32_t)(4 + B) << 8);
}

// Exact int32 sum of one lane's 13 trit bytes (in w[0..3], byte q at w[q / 4]
// byte q % 4) against its packed activation codes.
__device__ __forceinline__ int half_isum(const uint32_t (&w)[4], const uint32_t (&ax)[kHalfBytes],
                                         const uint32_t (&ay)[kHalfBytes], uint32_t copy_off, const uint8_t *lut)
{
    int a0 = 0, a1 = 0;
#pragma unroll
    for (int q = 0; q < kHalfBytes; ++q) {
        constexpr uint32_t sel[4] = {addr_sel<0>(), addr_sel<1>(), addr_sel<2>(), addr_sel<3>()};
        const uint32_t addr = __builtin_amdgcn_perm(w[q >> 2], copy_off, sel[q & 3]);
        const uint2 e = *reinterpret_cast<const uint2 *>(lut + addr);
        a0 = __builtin_amdgcn_sdot4((int)e.x, (int)ax[q], a0, false);
        a1 = __builtin_amdgcn_sdot4((int)e.y, (int)ay[q], a1, false);
    }
    return a0 + a1;
}

// Sum over the L lanes of a row (lane bits 0 .. log2(L) - 1), in every lane.
template <int L>
__device__ __forceinline__ float row_sum(float v)
{
    if constexpr (L >= 2) v = xsum<1>(v);
    if constexpr (L >= 4) v = xsum<2>(v);
    if constexpr (L >= 8) v = xsum<4>(v);
    if constexpr (L >= 16) v = xsum<8>(v);
    if constexpr (L >= 32) v = xsum<16>(v);
    if constexpr (L >= 64) v = xsum<32>(v);
    return v;
}

constexpr int kDepth = 4;          // wave steps whose weights are in flight while one is consumed
constexpr int kRing = kDepth + 1;  // weight buffers per lane

typedef int v4i_a4 __attribute__((ext_vector_type(4), aligned(4)));

// Workgroup = G groups of W waves over rows of one part; group g owns
// rows_per_group consecutive rows starting at (workgroup index within the
// part) * G * rows_per_group + g * rows_per_group. Lane l: half h = l & 1 of
// block column j = (l / 2) % C of row slot l / (2C).
template <int C>
__global__ __launch_bounds__(kMaxWaves *kWave) void gemv_kernel(PTQ_PARTS_PARAMS, const int8_t *__restrict__ qx,
                                                                const uint16_t *__restrict__ dx, int nb, int W,
                                                                int steps)
{
    constexpr int R = kWave / (2 * C);  // rows per wave step
    __shared__ __attribute__((aligned(16))) uint8_t lut[kLutBytes];
    __shared__ uint2 stage[256];
    extern __shared__ float partial[];  // [G * rows_per_group][W]

    // this workgroup's part (uniform)
    const int bi = blockIdx.x;
    const int part = (bi >= b1) + (bi >= b2) + (bi >= b3);
    const uint8_t *wp = part == 0 ? w0 : part == 1 ? w1 : part == 2 ? w2 : w3;
    float *yp = part == 0 ? y0 : part == 1 ? y1 : part == 2 ? y2 : y3;
    const float *rp = part == 0 ? r0 : part == 1 ? r1 : part == 2 ? r2 : r3;
    const int np = part == 0 ? n0 : part == 1 ? n1 : part == 2 ? n2 : n3;
    const int bp = bi - (part == 0 ? 0 : part == 1 ? b1 : part == 2 ? b2 : b3);

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x >> 6;
    const int G = blockDim.x / (kWave * W);
    const int g = wave / W, wg = wave - g * W;
    const uint32_t h = lane & 1;                     // 0: trit bytes 0-12; 1: bytes 13-25 and the scale
    const int c = wg * C + ((lane >> 1) & (C - 1));  // block column of this lane
    const int rs = lane / (2 * C);                   // row slot within a step
    const bool col_ok = c < nb;
    const int cl = col_ok ? c : nb - 1;              // clamped: always a valid column to read
    const int rows_per_group = steps * R;
    const uint32_t row_bytes = (uint32_t)nb * kPtqBytes;
    const int wg_row0 = bp * G * rows_per_group;
    const int grp_row0 = wg_row0 + g * rows_per_group;
    // half 0 reads block bytes 0-15, half 1 bytes 12-27 (then drops its first byte)
    const uint8_t *lane_base = wp + (uint32_t)cl * kPtqBytes + 12 * h;

    // the lane's 16 bytes at step s (rows past the part's end re-read its last row)
    auto blk_at = [&](int s) {
        const int r = min(grp_row0 + s * R + rs, np - 1);
        const v4i_a4 v = __builtin_nontemporal_load(
            reinterpret_cast<const v4i_a4 *>(lane_base + (uint64_t)(uint32_t)r * row_bytes));
        return v;
    };

    // the column's 128 activation codes and scale: requested first, so that
    // waiting for them leaves the weight loads below in flight
    uint32_t raw[32];
    {
        const int4 *q4 = reinterpret_cast<const int4 *>(qx + (int64_t)cl * kPtqBlock);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int4 v = q4[i];
            raw[4 * i] = (uint32_t)v.x;
            raw[4 * i + 1] = (uint32_t)v.y;
            raw[4 * i + 2] = (uint32_t)v.z;
            raw[4 * i + 3] = (uint32_t)v.w;
        }
    }
    const uint16_t dxbits = dx[cl];

    // the first steps' weights are requested before the table is built
    v4i_a4 b[kRing];  // step t lives in b[t % kRing]
#pragma unroll
    for (int j = 0; j < kDepth; ++j) b[j] = blk_at(j < steps ? j : steps - 1);

    // table: the 256 entries computed once into a staging area (computed, not
    // loaded: a load here would have to wait for the weight loads above, which
    // were issued first), then copied with consecutive 16-byte writes (two copies
    // each), which touch every bank once per pass
    for (int v = threadIdx.x; v < 256; v += blockDim.x) stage[v] = lut_entry(v);
    lds_barrier();
    for (int e = threadIdx.x; e < kLutBytes / 16; e += blockDim.x) {
        const uint2 t = stage[e / (kLutStride / 16)];
        *reinterpret_cast<uint4 *>(lut + 16 * e) = make_uint4(t.x, t.y, t.x, t.y);
    }

    // this half's codes (weights 65h .. 65h + 64), packed for the table entries:
    // codes 5q..5q+3 and code 5q+4 of its trit byte q
    uint32_t ax[kHalfBytes], ay[kHalfBytes];
    {
        uint32_t hs[18], sh[17];
#pragma unroll
        for (int i = 0; i < 18; ++i) {
            const uint32_t lo = i < 32 ? raw[i] : 0u, hi = 16 + i < 32 ? raw[16 + i] : 0u;
            hs[i] = h ? hi : lo;  // codes from 64h
        }
#pragma unroll
        for (int i = 0; i < 17; ++i) sh[i] = __builtin_amdgcn_alignbyte(hs[i + 1], hs[i], h);  // from 65h
#pragma unroll
        for (int q = 0; q < kHalfBytes; ++q) {
            const int o = 5 * q, o4 = o + 4;
            ax[q] = (o & 3) ? __builtin_amdgcn_alignbyte(sh[(o >> 2) + 1], sh[o >> 2], o & 3) : sh[o >> 2];
            ay[q] = sh[o4 >> 2] >> (8 * (o4 & 3));
        }
        // half 1, byte 12 is block byte 25: its digits 3 and 4 belong to no weight
        if (h) {
            ax[kHalfBytes - 1] &= 0x00FFFFFFu;
            ay[kHalfBytes - 1] = 0;
        }
    }
    const float dxf = f16_bits_to_f32(dxbits);
    const uint32_t copy_off = (uint32_t)(lane & (kLutCopies - 1)) * 8;
    const uint32_t term_mask = (h && col_ok) ? 0xFFFFFFFFu : 0u;
    const bool leader = (lane & (2 * C - 1)) == 0;  // the lane that stores a row's wave partial
    lds_barrier();

    // one step: this half's block sum, joined with the other half's; the half
    // holding the scale forms the block's term; the row's terms are summed
    auto consume = [&](const v4i_a4 &k, int s) {
        const uint32_t d[5] = {(uint32_t)k.x, (uint32_t)k.y, (uint32_t)k.z, (uint32_t)k.w, 0u};
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = __builtin_amdgcn_alignbyte(d[i + 1], d[i], h);
        int isum = half_isum(w, ax, ay, copy_off, lut);
        isum += xchg_int<1>(isum);                                          // the block's exact sum
        const float sd = f16_bits_to_f32((uint16_t)(w[3] >> 8)) * dxf;      // exact (half 1)
        // half 0 (its scale bits are trit bytes) and columns past nb contribute +0
        float t = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, (float)isum * sd) & term_mask);
        t = row_sum<2 * C>(t);
        // rows past the part's end have slots too (the finalize skips them)
        if (leader) partial[(grp_row0 - wg_row0 + s * R + rs) * W + wg] = t;
    };
    // Each step first requests the weights of step s + kDepth into the buffer
    // consumed last, then consumes step s; the empty asm keeps the compiler from
    // sinking the request below the step's work.
    int s0 = 0;
    for (; s0 + kRing + kDepth <= steps; s0 += kRing) {  // every request is a step of this group
#pragma unroll
        for (int j = 0; j < kRing; ++j) {
            b[(j + kDepth) % kRing] = blk_at(s0 + j + kDepth);
            asm volatile("" ::: "memory");
            consume(b[j], s0 + j);
        }
    }
    for (; s0 < steps; s0 += kRing) {  // the last steps: requests past the group's end re-read its last step
#pragma unroll
        for (int j = 0; j < kRing; ++j) {
            b[(j + kDepth) % kRing] = blk_at(min(s0 + j + kDepth, steps - 1));
            asm volatile("" ::: "memory");
            if (s0 + j < steps) consume(b[j], s0 + j);
        }
    }

    // the W wave partials of each row in wave order, then the residual (no global
    // memory access inside the step loop, whose loads stay in flight)
    lds_barrier();
    const int wg_rows = G * rows_per_group;
    for (int i = threadIdx.x; i < wg_rows; i += blockDim.x) {
        const int r = wg_row0 + i;
        if (r >= np) break;
        float t = partial[i * W];
        for (int w = 1; w < W; ++w) t += partial[i * W + w];
        yp[r] = rp ? t + rp[r] : t;
    }
}

// K == 0: y = residual (or 0) for n rows
__global__ __launch_bounds__(256) void fill_kernel(float *__restrict__ y, const float *__restrict__ res, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) y[i] = res ? res[i] : 0.0f;
}

// ---- host side ------------------------------------------------------------------

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlap(const void *a, int64_t abytes, const void *b, int64_t bbytes)
{
    if (!a || !b || abytes <= 0 || bbytes <= 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

constexpr int64_t kMaxElems = (int64_t)1 << 60;

struct PtqConfig {
    int C;      // block columns per wave
    int W;      // waves per row group
    int G;      // row groups per workgroup
    int steps;  // wave steps per group (R rows each)
};

// C: the largest share of useful lanes first (nb / (W * C)), then in the order
// 8, 16, 4, 32, 2, 1 (runs of 224 or 448 contiguous bytes per row and a short
// butterfly first). W = ceil(nb / C) <= 16; G groups make up to 8 waves (W
// when W > 8): two such workgroups share a compute unit's LDS, and measured on
// MI355X, 8-wave workgroups beat 12- and 16-wave ones on the decode shapes.
// Steps: enough rows per group that about 512 workgroups cover all rows,
// within the LDS of the partials.
PtqConfig ptq_pick(int64_t nb, int64_t n_total)
{
    static const int pref[] = {8, 16, 4, 32, 2, 1};
    PtqConfig c{};
    double best = -1.0;
    for (int C : pref) {
        const int64_t W = (nb + C - 1) / C;
        if (W > kMaxWaves) continue;
        const double util = (double)nb / (double)(W * C);
        if (util > best + 1e-12) {
            best = util;
            c.C = C;
            c.W = (int)W;
        }
    }
    c.G = c.W < kWaveCap ? kWaveCap / c.W : 1;
    const int64_t per_step = (int64_t)c.G * (kWave / (2 * c.C));  // rows of one workgroup step
    int64_t steps = (n_total + kTargetGroups * per_step - 1) / (kTargetGroups * per_step);
    if (steps < 1) steps = 1;
    if (steps > kMaxSteps) steps = kMaxSteps;
    const int64_t cap = kMaxPartialBytes / (per_step * c.W * 4);
    if (steps > cap) steps = cap < 1 ? 1 : cap;
    c.steps = (int)steps;
    return c;
}

int64_t rows_per_block(const PtqConfig &c) { return (int64_t)c.G * (kWave / (2 * c.C)) * c.steps; }

struct PtqParts {
    const uint8_t *w[4];
    float *y[4];
    const float *res[4];
    int n[4];
    int bend[4];  // cumulative workgroup counts
};

template <int C>
hipError_t launch_c(const PtqParts &p, const int8_t *qx, const uint16_t *dx, int nb, const PtqConfig &c,
                    int blocks, hipStream_t s)
{
    PtqParts pc = p;
    const int8_t *qc = qx;
    const uint16_t *dc = dx;
    int nbc = nb, wc = c.W, sc = c.steps;
    void *args[] = {&pc.w[0], &pc.w[1],   &pc.w[2],   &pc.w[3],   &pc.y[0], &pc.y[1], &pc.y[2],
                    &pc.y[3], &pc.res[0], &pc.res[1], &pc.res[2], &pc.res[3], &pc.n[0], &pc.n[1],
                    &pc.n[2], &pc.n[3],   &pc.bend[0], &pc.bend[1], &pc.bend[2], &qc, &dc,
                    &nbc,     &wc,        &sc};
    const size_t dyn = (size_t)rows_per_block(c) * c.W * sizeof(float);
    return hipLaunchKernel(reinterpret_cast<const void *>(&gemv_kernel<C>), dim3((unsigned)blocks),
                           dim3(c.G * c.W * kWave), args, dyn, s);
}

hipError_t launch_gemv(PtqParts p, int nparts, const int8_t *qx, const uint16_t *dx, int nb, int64_t n_total,
                       hipStream_t s)
{
    const PtqConfig c = ptq_pick(nb, n_total);
    const int64_t rpb = rows_per_block(c);
    int64_t blocks = 0;
    for (int i = 0; i < 4; ++i) {
        if (i < nparts) blocks += (p.n[i] + rpb - 1) / rpb;
        if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
        p.bend[i] = i < nparts ? (int)blocks : 0x7FFFFFFF;
    }
    switch (c.C) {
    case 1: return launch_c<1>(p, qx, dx, nb, c, (int)blocks, s);
    case 2: return launch_c<2>(p, qx, dx, nb, c, (int)blocks, s);
    case 4: return launch_c<4>(p, qx, dx, nb, c, (int)blocks, s);
    case 8: return launch_c<8>(p, qx, dx, nb, c, (int)blocks, s);
    case 16: return launch_c<16>(p, qx, dx, nb, c, (int)blocks, s);
    default: return launch_c<32>(p, qx, dx, nb, c, (int)blocks, s);
    }
}

}  // namespace

q8g_status ptq1_stacked(const q8g_part *parts, int nparts, const int8_t *qx, const uint16_t *dx, int64_t K,
                        void *stream)
{
    if (!parts) return Q8G_ERR_NULL;
    if (nparts < 1 || nparts > 4) return Q8G_ERR_ARG;
    if (K < 0 || K % kPtqBlock || K > kMaxK) return Q8G_ERR_SHAPE;
    const int64_t nb = K / kPtqBlock;
    const int64_t row_bytes = nb * kPtqBytes;
    int64_t n_total = 0;
    for (int i = 0; i < nparts; ++i) {
        if (parts[i].n < 0 || parts[i].n > kMaxRows) return Q8G_ERR_SHAPE;
        n_total += parts[i].n;
    }
    if (n_total == 0) return Q8G_OK;
    if (K > 0 && (!qx || !dx)) return Q8G_ERR_NULL;
    if (!aligned(qx, 16) || !aligned(dx, 2)) return Q8G_ERR_ALIGN;
    const int64_t xbytes = K, dxbytes = nb * 2;
    PtqParts p{};
    int slot = 0;
    for (int i = 0; i < nparts; ++i) {
        const q8g_part &pt = parts[i];
        if (pt.n == 0) continue;
        if (!pt.y || (K > 0 && !pt.w)) return Q8G_ERR_NULL;
        if (!aligned(pt.w, 4) || !aligned(pt.y, 4) || (pt.residual && !aligned(pt.residual, 4)))
            return Q8G_ERR_ALIGN;
        p.w[slot] = static_cast<const uint8_t *>(pt.w);
        p.y[slot] = pt.y;
        p.res[slot] = pt.residual;
        p.n[slot] = (int)pt.n;
        ++slot;
    }
    for (int i = 0; i < nparts; ++i) {
        const q8g_part &a = parts[i];
        if (a.n == 0) continue;
        const int64_t ybytes = a.n * 4;
        if (overlap(a.y, ybytes, qx, xbytes) || overlap(a.y, ybytes, dx, dxbytes)) return Q8G_ERR_OVERLAP;
        for (int j = 0; j < nparts; ++j) {
            const q8g_part &b = parts[j];
            if (b.n == 0) continue;
            if (overlap(a.y, ybytes, b.w, b.n * row_bytes)) return Q8G_ERR_OVERLAP;
            if (b.residual && !(i == j && b.residual == a.y) && overlap(a.y, ybytes, b.residual, b.n * 4))
                return Q8G_ERR_OVERLAP;
            if (i != j && overlap(a.y, ybytes, b.y, b.n * 4)) return Q8G_ERR_OVERLAP;
        }
    }
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (K == 0) {
        for (int i = 0; i < slot; ++i) {
            float *y = p.y[i];
            const float *res = p.res[i];
            int64_t nn = p.n[i];
            void *args[] = {&y, &res, &nn};
            const hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&fill_kernel),
                                                 dim3((unsigned)((nn + 255) / 256)), dim3(256), args, 0, s);
            if (e != hipSuccess) return Q8G_ERR_LAUNCH;
        }
        return Q8G_OK;
    }
    const hipError_t e = launch_gemv(p, slot, qx, dx, (int)nb, n_total, s);
    return e == hipSuccess ? Q8G_OK : Q8G_ERR_LAUNCH;
}

q8g_status ptq1_config(int64_t n_total, int64_t K, int *rows_per_wave, int *waves_per_group)
{
    if (n_total < 0 || K <= 0 || K % kPtqBlock || K > kMaxK) return Q8G_ERR_SHAPE;
    const PtqConfig c = ptq_pick(K / kPtqBlock, n_total);
    if (rows_per_wave) *rows_per_wave = kWave / (2 * c.C);
    if (waves_per_group) *waves_per_group = c.G * c.W;
    return Q8G_OK;
}

}  // namespace q8g

extern "C" {

q8g_status ptq1_rotate_quantize_act(const float *x, float *rot, int8_t *qx, uint16_t *dx, int64_t K, void *stream)
{
    using namespace q8g;
    if (K < 0 || K > kMaxElems || K % kPtqBlock) return Q8G_ERR_SHAPE;
    if (K == 0) return Q8G_OK;
    if (!x || !qx || !dx) return Q8G_ERR_NULL;
    if (!aligned(x, 4) || !aligned(qx, 1) || !aligned(dx, 2) || (rot && !aligned(rot, 4))) return Q8G_ERR_ALIGN;
    const int64_t nb = K / kPtqBlock;
    if (overlap(qx, K, x, 4 * K) || overlap(dx, 2 * nb, x, 4 * K) || overlap(qx, K, dx, 2 * nb) ||
        overlap(rot, 4 * K, x, 4 * K) || overlap(rot, 4 * K, qx, K) || overlap(rot, 4 * K, dx, 2 * nb))
        return Q8G_ERR_OVERLAP;
    if (nb > 0x7FFFFFFF) return Q8G_ERR_SHAPE;
    const float *xc = x;
    float *rc = rot;
    int8_t *qc = qx;
    uint16_t *dc = dx;
    double root = sqrt((double)kPtqBlock);  // the f64 nearest to sqrt(128)
    void *args[] = {&xc, &rc, &qc, &dc, &root};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&rotate_kernel), dim3((unsigned)nb),
                                         dim3(kPtqBlock), args, 0, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? Q8G_OK : Q8G_ERR_LAUNCH;
}

q8g_status ptq1_gemv(const uint8_t *w, const int8_t *qx, const uint16_t *dx, const float *residual, float *y,
                     int64_t N, int64_t K, void *stream)
{
    if (N < 0) return Q8G_ERR_SHAPE;
    const q8g_part part = {w, nullptr, N, y, residual};
    return q8g::ptq1_stacked(&part, 1, qx, dx, K, stream);
}

}  // extern "C"
