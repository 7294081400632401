// A decode step of stacked Q8_0 projections in one cooperative launch
// (q8_decode_stack in include/q8gemv.h).
//
// "Filling in the blanks: Inference using Phobos", section Fast Decode, gives
// the launch-level recipe: replay the pass as a unit, quantize an activation
// once and share it, stack projections that read one input, fold the residual
// add into the matmul. On MI355X a kernel boundary costs about 1.6 us and a
// dependent projection of 2-8 MB takes 4-5 us as its own launch, so a token
// of 97 projections spent most of its time in launch ramp and tail. Here one
// workgroup per compute unit (1024 threads, 16 waves) stays resident for the
// whole token:
//
//  * Rows of projection i are split evenly over the workgroups; within a
//    workgroup, wave w >= 1 owns rows w-1, w-1+15, ... of that slice, whole rows
//    only, processed in groups of up to 4 with the standalone kernel's lane
//    layout, chunk order and butterfly reduction (gemv_device.hpp). So every
//    output is bit-identical to gemv_stacked.
//  * The weights of a projection depend on no activation, so as soon as a
//    workgroup has published projection i, each wave requests its first
//    kPrefetch 1 KiB items of projection i+1 and only then waits for the
//    other workgroups: the barrier wait overlaps the weight stream instead of
//    preceding it.
//  * Barrier: after its outputs are written, workgroup g stores the count of
//    projections it has finished (over all launches that used the workspace)
//    into its own 64-byte flag line; wave 0 of every workgroup polls all flag
//    lines. Wave 0 owns no weight rows: the loads of one wave complete in the
//    order they were issued, so polls from a wave with weight loads in flight
//    would wait for those first. Relaxed device-scope (sc1) stores and
//    loads only: no hot line, no L2 write-back or invalidate on the path.
//    Outputs are stored, and activations and residuals loaded, with the same
//    device-coherent accesses, so a projection that reads an earlier one's
//    output (a real decode chain) would see it.
//  * After the barrier each workgroup quantizes the f32 activation into LDS
//    (the same arithmetic as q8_quantize_act) and every wave reads its codes
//    from there.
//  * Every wait is bounded: a workgroup that polls too long raises the
//    workspace's error word and leaves; the others see it and leave too.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemv_device.hpp"
#include "q8gemv.h"

namespace {

using namespace q8g;

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kWorkWaves = kWaves - 1;  // wave 0 only synchronizes (see the barrier note)
constexpr int kPrefetch = 4;           // 1 KiB items per wave fetched ahead of the barrier
constexpr int kGroup = 4;              // rows reduced together
constexpr int kMaxGroups = 1024;       // workgroups the workspace has flag lines for
constexpr int kErrWord = Q8G_STACK_ERR_WORD;
constexpr int kFlagBase = 64;          // flag of workgroup g at kFlagBase + 16 g
constexpr long kSpinLimit = 1L << 22;  // polls before a wait is abandoned

static_assert(kFlagBase + 16 * kMaxGroups <= Q8G_STACK_SYNC_WORDS, "workspace too small");

__device__ __forceinline__ uint32_t ld_dev(const uint32_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(uint32_t *p, uint32_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev_f(const float *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev_f(float *p, float v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct Row {
    const char *w;
    const uint16_t *dw;
    float *y;
    const float *res;
};

// Row g of a stacked op (parts are contiguous in the stacked row space).
__device__ __forceinline__ Row locate_row(const q8g_stack_op *op, int64_t g, int64_t K)
{
    const int np = op->nparts;
    int64_t begin = 0;
    Row r{static_cast<const char *>(op->parts[0].w), op->parts[0].dw, op->parts[0].y, op->parts[0].residual};
    int64_t b0 = op->parts[0].n;
#pragma unroll
    for (int i = 1; i < 4; ++i) {
        if (i < np && g >= b0) {
            begin = b0;
            r = Row{static_cast<const char *>(op->parts[i].w), op->parts[i].dw, op->parts[i].y, op->parts[i].residual};
            b0 += op->parts[i].n;
        }
    }
    const int64_t local = g - begin;
    r.w += local * K;
    r.dw += local * (K / 32);
    r.y += local;
    if (r.res) r.res += local;
    return r;
}

__device__ __forceinline__ int64_t op_rows(const q8g_stack_op *op)
{
    int64_t n = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (i < op->nparts) n += op->parts[i].n;
    return n;
}

// This wave's rows of op: first row and count (rows are first + kWorkWaves j).
// Wave 0 owns none.
struct Slice {
    int64_t first;
    int64_t count;
};

__device__ __forceinline__ Slice wave_slice(int64_t n_total, int G, int g, int wave)
{
    const int64_t r0 = n_total * g / G, r1 = n_total * (g + 1) / G;
    const int64_t m = r1 - r0;
    const int work = wave - 1;
    if (work < 0) return Slice{r0, 0};
    const int64_t cnt = m > work ? (m - work + kWorkWaves - 1) / kWorkWaves : 0;
    return Slice{r0 + work, cnt};
}

// The items of a wave's first row group, in chunk-major order (chunk c of
// every row of the group, then chunk c+1): item k is chunk k / nr of row k % nr.
struct Prefetch {
    int4 w[kPrefetch];
    uint16_t s[kPrefetch];
};

__device__ __forceinline__ void issue_prefetch(const q8g_stack_op *op, Slice sl, int lane, Prefetch &pf)
{
    const int64_t K = op->K;
    const int nr = (int)(sl.count < kGroup ? sl.count : kGroup);
    const int64_t C = (K + kChunk - 1) / kChunk;
#pragma unroll
    for (int k = 0; k < kPrefetch; ++k) {
        if (nr > 0 && k < nr * C) {
            const int c = k / nr, r = k % nr;
            const Row row = locate_row(op, sl.first + (int64_t)r * kWorkWaves, K);
            const int64_t off = (int64_t)c * kChunk + lane * 16;
            const int64_t o = off < K ? off : 0;
            pf.w[k] = load16_stream(row.w + o);
            pf.s[k] = load_u16_stream(row.dw + (o >> 5));
        }
    }
}

__global__ __launch_bounds__(kThreads) void stack_kernel(const q8g_stack_op *__restrict__ ops, int nops,
                                                         uint32_t *__restrict__ sync)
{
    __shared__ __align__(16) int8_t s_qx[Q8G_STACK_MAX_K];
    __shared__ float s_dx[Q8G_STACK_MAX_K / 32];
    __shared__ int s_abort;

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int G = gridDim.x;
    const int g = blockIdx.x;
    const float even = (lane & 1) ? 0.0f : 1.0f;
    uint32_t *flags = sync + kFlagBase;

    if (threadIdx.x == 0) s_abort = 0;
    // Projections finished by earlier launches: after a completed launch every
    // flag line holds the same count, so each workgroup reads its own.
    const uint32_t done0 = ld_dev(flags + 16 * g);

    Prefetch cur;
    issue_prefetch(&ops[0], wave_slice(op_rows(&ops[0]), G, g, wave), lane, cur);

    for (int i = 0; i < nops; ++i) {
        const q8g_stack_op *op = &ops[i];
        const int64_t K = op->K;
        const int64_t n_total = op_rows(op);
        const Slice sl = wave_slice(n_total, G, g, wave);

        // wait until every workgroup has finished projection i-1
        if (i > 0 && wave == 0) {
            const uint32_t target = done0 + (uint32_t)i;
            for (long spin = 0;; ++spin) {
                bool ok = true;
                for (int w = lane; w < G; w += kWave) ok &= (int32_t)(ld_dev(flags + 16 * w) - target) >= 0;
                if (__all(ok)) break;
                if (ld_dev(sync + kErrWord) != 0 || spin > kSpinLimit) {
                    if (lane == 0) {
                        st_dev(sync + kErrWord, 1u);
                        s_abort = 1;
                    }
                    break;
                }
            }
        }
        __syncthreads();
        if (s_abort) return;

        // quantize the activation into LDS (same arithmetic as q8_quantize_act)
        for (int64_t e = (int64_t)threadIdx.x * 4; e < K; e += 4 * kThreads) {
            const float4 v = make_float4(ld_dev_f(op->x + e), ld_dev_f(op->x + e + 1), ld_dev_f(op->x + e + 2),
                                         ld_dev_f(op->x + e + 3));
            float d;
            const uint32_t packed = quantize4(v, &d);
            *reinterpret_cast<uint32_t *>(s_qx + e) = packed;
            const uint16_t bits = scale_bits(d);
            if ((lane & 7) == 0) {
                s_dx[e >> 5] = f16_bits_to_f32(bits);
                if (g == 0 && op->dx) op->dx[e >> 5] = bits;
            }
            if (g == 0 && op->qx) *reinterpret_cast<uint32_t *>(op->qx + e) = packed;
        }
        __syncthreads();

        // this wave's rows, in groups of kGroup; the first group's first
        // kPrefetch items are already in registers
        const int64_t C = (K + kChunk - 1) / kChunk;
        for (int64_t g0 = 0; g0 < sl.count; g0 += kGroup) {
            const int nr = (int)(sl.count - g0 < kGroup ? sl.count - g0 : kGroup);
            Row rows[kGroup];
#pragma unroll
            for (int r = 0; r < kGroup; ++r)
                rows[r] = locate_row(op, sl.first + (g0 + (r < nr ? r : 0)) * kWorkWaves, K);
            float acc[kGroup] = {0.0f, 0.0f, 0.0f, 0.0f};
            const int64_t nitems = nr * C;
            for (int64_t k0 = 0; k0 < nitems; k0 += kPrefetch) {
                int4 wv[kPrefetch];
                uint16_t ws[kPrefetch];
                const bool from_pf = g0 == 0 && k0 == 0;
#pragma unroll
                for (int k = 0; k < kPrefetch; ++k) {
                    if (from_pf) {
                        wv[k] = cur.w[k];
                        ws[k] = cur.s[k];
                    } else if (k0 + k < nitems) {
                        const int64_t kk = k0 + k;
                        const int c = (int)(kk / nr), r = (int)(kk % nr);
                        const Row rw = locate_row(op, sl.first + (g0 + r) * kWorkWaves, K);
                        const int64_t off = (int64_t)c * kChunk + lane * 16;
                        const int64_t o = off < K ? off : 0;
                        wv[k] = load16_stream(rw.w + o);
                        ws[k] = load_u16_stream(rw.dw + (o >> 5));
                    }
                }
#pragma unroll
                for (int k = 0; k < kPrefetch; ++k) {
                    const int64_t kk = k0 + k;
                    if (kk < nitems) {
                        const int c = (int)(kk / nr), r = (int)(kk % nr);
                        const int64_t off = (int64_t)c * kChunk + lane * 16;
                        const bool active = off < K;
                        const int64_t o = active ? off : 0;
                        const int4 xq = *reinterpret_cast<const int4 *>(s_qx + o);
                        const float xs = active ? s_dx[o >> 5] * even : 0.0f;
                        const int s = q8_block_sum(wv[k], xq);
#pragma unroll
                        for (int rr = 0; rr < kGroup; ++rr)
                            if (rr == r) acc[rr] = __builtin_fmaf((float)s, f16_bits_to_f32(ws[k]) * xs, acc[rr]);
                    }
                }
            }
            const float total = wave_reduce_rows<kGroup>(acc, lane);
#pragma unroll
            for (int r = 0; r < kGroup; ++r)
                if (r < nr && lane == lane_of<kGroup>(r))
                    st_dev_f(rows[r].y, rows[r].res ? total + ld_dev_f(rows[r].res) : total);
        }

        // publish: this workgroup's outputs of projection i are written. The
        // wait covers only this projection's stores: the next projection's
        // weights are requested after it, and arrive during the next barrier.
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (threadIdx.x == 0) st_dev(flags + 16 * g, done0 + (uint32_t)i + 1);
        if (i + 1 < nops) issue_prefetch(&ops[i + 1], wave_slice(op_rows(&ops[i + 1]), G, g, wave), lane, cur);
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

struct Span {
    const void *p;
    int64_t bytes;
};

q8g_status validate(const q8g_stack_op *ops, int nops)
{
    constexpr int64_t kMaxRows = (int64_t)1 << 40;
    for (int i = 0; i < nops; ++i) {
        const q8g_stack_op &op = ops[i];
        if (op.nparts < 1 || op.nparts > 4 || op.reserved != 0) return Q8G_ERR_ARG;
        if (op.K < 32 || op.K > Q8G_STACK_MAX_K || op.K % 32) return Q8G_ERR_SHAPE;
        if (!op.x) return Q8G_ERR_NULL;
        if (!aligned(op.x, 16) || (op.qx && !aligned(op.qx, 16)) || (op.dx && !aligned(op.dx, 2)))
            return Q8G_ERR_ALIGN;
        int64_t n = 0;
        for (int p = 0; p < op.nparts; ++p) {
            const q8g_part &pt = op.parts[p];
            if (pt.n < 0 || pt.n > kMaxRows) return Q8G_ERR_SHAPE;
            n += pt.n;
            if (pt.n == 0) continue;
            if (!pt.w || !pt.dw || !pt.y) return Q8G_ERR_NULL;
            if (!aligned(pt.w, 16) || !aligned(pt.dw, 2) || !aligned(pt.y, 4) ||
                (pt.residual && !aligned(pt.residual, 4)))
                return Q8G_ERR_ALIGN;
        }
        if (n < 1 || n > kMaxRows) return Q8G_ERR_SHAPE;
    }
    // outputs: each op's y planes, plus the optional code/scale copies
    for (int i = 0; i < nops; ++i) {
        const q8g_stack_op &a = ops[i];
        Span outs[6];
        int no = 0;
        for (int p = 0; p < a.nparts; ++p)
            if (a.parts[p].n) outs[no++] = Span{a.parts[p].y, a.parts[p].n * 4};
        if (a.qx) outs[no++] = Span{a.qx, a.K};
        if (a.dx) outs[no++] = Span{a.dx, a.K / 16};
        for (int o = 0; o < no; ++o) {
            for (int j = 0; j < nops; ++j) {
                const q8g_stack_op &b = ops[j];
                // weights and scales of every op are streamed ahead of the barriers
                for (int p = 0; p < b.nparts; ++p) {
                    const q8g_part &q = b.parts[p];
                    if (!q.n) continue;
                    if (overlap(outs[o].p, outs[o].bytes, q.w, q.n * b.K) ||
                        overlap(outs[o].p, outs[o].bytes, q.dw, q.n * (b.K / 32) * 2))
                        return Q8G_ERR_OVERLAP;
                    // an output may be a later op's residual (written before it is read), or be
                    // read as this op's own residual in place; anything else overlapping is a race
                    if (q.residual && overlap(outs[o].p, outs[o].bytes, q.residual, q.n * 4) && j <= i &&
                        !(j == i && q.residual == outs[o].p && q.n * 4 == outs[o].bytes))
                        return Q8G_ERR_OVERLAP;
                }
                // an output may feed a later op's input; not this op's or an earlier one's
                if (j <= i && overlap(outs[o].p, outs[o].bytes, b.x, b.K * 4)) return Q8G_ERR_OVERLAP;
            }
            // other outputs of any op
            for (int j = 0; j < nops; ++j) {
                const q8g_stack_op &b = ops[j];
                Span o2[6];
                int n2 = 0;
                for (int p = 0; p < b.nparts; ++p)
                    if (b.parts[p].n) o2[n2++] = Span{b.parts[p].y, b.parts[p].n * 4};
                if (b.qx) o2[n2++] = Span{b.qx, b.K};
                if (b.dx) o2[n2++] = Span{b.dx, b.K / 16};
                for (int q = 0; q < n2; ++q) {
                    if (j == i && q == o) continue;
                    if (overlap(outs[o].p, outs[o].bytes, o2[q].p, o2[q].bytes)) return Q8G_ERR_OVERLAP;
                }
            }
        }
    }
    return Q8G_OK;
}

}  // namespace

extern "C" q8g_status q8_decode_stack(const q8g_stack_op *ops, const q8g_stack_op *ops_dev, int nops,
                                      uint32_t *sync, void *stream)
{
    if (nops < 0) return Q8G_ERR_ARG;
    if (nops == 0) return Q8G_OK;
    if (!ops || !ops_dev || !sync) return Q8G_ERR_NULL;
    if (!aligned(ops_dev, 8) || !aligned(sync, 64)) return Q8G_ERR_ALIGN;
    const q8g_status st = validate(ops, nops);
    if (st != Q8G_OK) return st;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return Q8G_ERR_LAUNCH;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return Q8G_ERR_LAUNCH;
    if (cus < 1 || cus > kMaxGroups) return Q8G_ERR_LAUNCH;
    const q8g_stack_op *o = ops_dev;
    int n = nops;
    uint32_t *s = sync;
    void *args[] = {&o, &n, &s};
    const hipError_t e = hipLaunchCooperativeKernel(reinterpret_cast<const void *>(&stack_kernel), dim3(cus),
                                                    dim3(kThreads), args, 0, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? Q8G_OK : Q8G_ERR_LAUNCH;
}
