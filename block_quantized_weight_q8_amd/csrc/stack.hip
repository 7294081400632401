// A decode step of stacked Q8_0 projections in one cooperative launch
// (q8_decode_stack in include/q8gemv.h).
//
// "Filling in the blanks: Inference using Phobos", section Fast Decode: a
// decode pass is replayed as one unit, each activation is quantized once and
// reused, and projections that read one input are stacked. On MI355X a kernel
// boundary costs about 1.6 us, and a dependent projection of 2-8 MB run as its
// own launch takes 2.9-3.6 us, most of it latency. Here one workgroup per
// compute unit (1024 threads) stays resident for the whole token, and the
// per-projection critical path is cut to one barrier plus one read:
//
//  * Roles. Wave 0 of every workgroup synchronizes; waves 1-15 compute. One
//    wave's loads complete in issue order, so a wave with weight loads in
//    flight would see its barrier polls and input reads queue behind them.
//  * Weights. The rows of projection i are split evenly over the workgroups
//    and, within one, into contiguous blocks per compute wave. A compute wave
//    processes its rows in groups of R (1, 2 or 4) rows, chunk-major, in
//    batches of four 1 KiB items, with the lane layout, chunk order and
//    butterfly reduction of the standalone kernel (gemv_device.hpp), so every
//    output is bit-identical to gemv_stacked. Weights depend on no activation:
//    as soon as a wave has computed projection i it requests the first batch
//    of projection i+1, which then arrives during the barrier. For the layer
//    projections of a decode stack that batch is a wave's whole share; longer
//    shares stream with two batches in flight.
//  * The input of projection i+1 is quantized once: the workgroup that owns
//    32-value block b (b = g, g + G, ...) quantizes it after it has computed
//    its rows of projection i and publishes the 32 codes and the scale as nine
//    8-byte words, each carrying the barrier's tag in its upper half (an
//    8-byte store is single-copy atomic, so a word is either old or whole).
//  * Barrier: 16 counters, 256 bytes apart; workgroup g adds one to counter
//    g % 16 (a device-scope atomic) and wave 0 polls the 16 counters. Counters
//    on separate lines keep same-line atomics to 16 per line; one counter per
//    workgroup, or all of them on one line, measured slower (the atomics to one
//    line serialize at about 15 ns each).
//  * After the barrier wave 0 reads the published blocks (device-coherent
//    loads, all issued before one wait; a word whose tag is not yet the
//    barrier's is read again) and any residual of the workgroup's rows into
//    LDS; the compute waves then read codes, scales and residuals from there.
//  * An input or residual that is an earlier projection's output (a chained
//    projection) is not published: before that barrier every wave waits until
//    its own stores are acknowledged, and after it every workgroup reads the
//    f32 input with device-coherent loads and quantizes it into LDS.
//  * The workspace carries the number of barriers completed so far (T). The
//    counters only grow: barrier j of a launch is passed when counter c holds
//    (T + j + 1) times the number of workgroups that add to it; its tag is
//    T + j + 1. Workgroup 0 stores the new T after the last barrier, when every
//    workgroup has read the old one.
//  * Every wait is bounded: a workgroup that polls too long raises the error
//    word and leaves; the others see it and leave too.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "gemv_device.hpp"
#include "q8gemv.h"

namespace {

using namespace q8g;

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kWork = kWaves - 1;  // compute waves 1..15; wave 0 synchronizes
constexpr int kB = 4;              // 1 KiB items per batch
constexpr int kMaxOps = Q8G_STACK_MAX_OPS;
constexpr int kMaxGroups = 1024;   // workgroups (compute units) supported
constexpr int kCounters = 16;
constexpr int kTotalWord = 0;      // barriers completed by earlier launches
constexpr int kErrWord = Q8G_STACK_ERR_WORD;
constexpr int kCounterBase = 64;   // counter c at word kCounterBase + 64 c
constexpr int kBlockWords = 9;     // 8-byte words of one published block
constexpr int kMaxBlocks = Q8G_STACK_MAX_K / 32;
constexpr int kAreaBase = kCounterBase + 64 * kCounters;  // in uint32 words, 256-byte aligned
// u64 words of one area: the bulk read takes 16-byte pairs and may reach one word past the last block
constexpr int kAreaU64 = kMaxBlocks * kBlockWords + 2;
constexpr int kAreaWords = (2 * kAreaU64 + 63) / 64 * 64;
constexpr int kResMax = 2048;       // residual rows per workgroup staged in LDS
constexpr int kXPass = Q8G_STACK_MAX_K / (4 * kThreads);  // f32 passes of 4 values per thread
constexpr long kSpinLimit = 1L << 20;  // polls (each a memory round trip) before a wait is abandoned

static_assert(kAreaBase + 2 * kAreaWords <= Q8G_STACK_SYNC_WORDS, "workspace too small");
static_assert(kAreaBase % 64 == 0 && kAreaWords % 64 == 0, "areas 256-byte aligned");

// Every global access through a pointer taken from a descriptor in LDS is made
// through an address-space-1 pointer: from a generic pointer the compiler emits
// FLAT instructions, which count against the LDS counter as well, so that every
// LDS access would wait for all weight loads in flight.
#define GLOBAL __attribute__((address_space(1)))

template <typename T>
__device__ __forceinline__ GLOBAL T *gptr(T *p)
{
    return (GLOBAL T *)p;
}

// relaxed device-scope (sc1) accesses: coherent across the compute units of all XCDs
__device__ __forceinline__ uint32_t ld_dev(const uint32_t *p)
{
    return __hip_atomic_load(gptr(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(uint32_t *p, uint32_t v)
{
    __hip_atomic_store(gptr(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_dev64(const uint64_t *p)
{
    return __hip_atomic_load(gptr(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev64(uint64_t *p, uint64_t v)
{
    __hip_atomic_store(gptr(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev_f(const float *p)
{
    return __hip_atomic_load(gptr(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev_f(float *p, float v)
{
    __hip_atomic_store(gptr(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void arrive(uint32_t *p)
{
    __hip_atomic_fetch_add(gptr(p), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// weights: read once, nontemporal
__device__ __forceinline__ int4 ld_w16(const char *p)
{
    const v4i v = __builtin_nontemporal_load((const GLOBAL v4i *)p);
    return make_int4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint16_t ld_ws(const uint16_t *p) { return __builtin_nontemporal_load(gptr(p)); }

// inputs from before the launch, and the optional code / scale outputs
typedef float v4f __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 ld_f4(const float *p)
{
    const v4f v = *(const GLOBAL v4f *)p;
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float ld_f(const float *p) { return *gptr(p); }
__device__ __forceinline__ void st_u32(int8_t *p, uint32_t v) { *gptr(reinterpret_cast<uint32_t *>(p)) = v; }
__device__ __forceinline__ void st_u16(uint16_t *p, uint16_t v) { *gptr(p) = v; }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kPairs = 8;  // 16-byte loads per lane per pass over a published input

// 16 bytes at base + off, bypassing the caches that another compute unit's stores do
// not update (device scope, sc1). Issued only; wait_loads() waits for it.
__device__ __forceinline__ void load16_dev(const uint64_t *base, uint32_t off, u32x4 &v)
{
    asm volatile("global_load_dwordx4 %0, %1, %2 sc1" : "=v"(v) : "v"(off), "s"(base) : "memory");
}

// Wait for every load of this wave; the values become visible to the compiler only here.
template <int N>
__device__ __forceinline__ void wait_loads(u32x4 (&v)[N])
{
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int k = 0; k < N; ++k) asm volatile("" : "+v"(v[k]));
}

// What a workgroup keeps of an op besides its descriptor: the row ends of the
// parts and its own slice of rows, worked out once per launch (64-bit divisions
// are long instruction sequences).
struct OpInfo {
    int64_t end[3];  // cumulative row ends of parts 0..2 (INT64_MAX past the last part)
    int64_t n;       // rows of all parts
    int64_t r0;      // first row of this workgroup's slice
    int32_t m;       // rows of the slice
    int32_t rw;      // rows per compute wave: ceil(m / kWork)
    int32_t R;       // rows per group: 1, 2 or 4
    int32_t C;       // 1 KiB chunks per row
    int32_t bpg;     // batches per group
    int32_t chained; // the input or a residual overlaps an earlier op's output
    int32_t has_res; // some part has a residual
    int32_t pad;
};

struct RowPtr {
    const char *w;
    const uint16_t *dw;
    float *y;
    const float *res;
};

// Row `row` of op `op` (stacked parts are contiguous in the row space).
__device__ __forceinline__ RowPtr locate(const q8g_stack_op &op, const OpInfo &oi, int64_t row)
{
    int p = 0;
    int64_t begin = 0;
    if (row >= oi.end[0]) { p = 1; begin = oi.end[0]; }
    if (row >= oi.end[1]) { p = 2; begin = oi.end[1]; }
    if (row >= oi.end[2]) { p = 3; begin = oi.end[2]; }
    const q8g_part &pt = op.parts[p];
    const int64_t local = row - begin;
    RowPtr r;
    r.w = static_cast<const char *>(pt.w) + local * op.K;
    r.dw = pt.dw + local * (op.K / 32);
    r.y = pt.y + local;
    r.res = pt.residual ? pt.residual + local : nullptr;
    return r;
}

// A compute wave's share of an op: rows [first, first + count), processed in
// groups of R rows; a group is `bpg` batches of kB items, chunk-major.
struct Share {
    int64_t first;   // first row (in the op's row space)
    int64_t slice0;  // first row of the workgroup's slice (residuals are staged from there)
    int count;       // rows of this wave
    int R;           // rows per group: 1, 2 or 4
    int C;           // 1 KiB chunks per row
    int bpg;         // batches per group
    int nbatch;      // batches of this wave
};

__device__ __forceinline__ Share share_of(const OpInfo &oi, int wave)
{
    const int w = wave - 1;
    Share s;
    s.slice0 = oi.r0;
    s.first = oi.r0 + (int64_t)w * oi.rw;
    int cnt = oi.m - w * oi.rw;
    s.count = cnt < 0 ? 0 : (cnt > oi.rw ? oi.rw : cnt);
    s.R = oi.R;
    s.C = oi.C;
    s.bpg = oi.bpg;
    const int groups = s.R == 4 ? (s.count + 3) >> 2 : (s.R == 2 ? (s.count + 1) >> 1 : s.count);
    s.nbatch = groups * s.bpg;
    return s;
}

// a wave-uniform value kept in scalar registers
__device__ __forceinline__ int64_t uni64(int64_t v)
{
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}
template <typename T>
__device__ __forceinline__ T *uni_ptr(T *p)
{
    return reinterpret_cast<T *>(uni64(reinterpret_cast<int64_t>(p)));
}
__device__ __forceinline__ int uni32(int v) { return __builtin_amdgcn_readfirstlane(v); }

struct WBatch {
    int4 w[kB];
    uint16_t s[kB];
};

// Batch t of a share: group q = t / bpg, chunks u * (kB / R) .. of rows q R .. q R + R - 1.
// Every load is issued: a row slot past the share reads the group's first row, a chunk
// past the row reads the row's last chunk, a lane past the row end reads offset 0.
template <int R>
__device__ __forceinline__ void load_batch(const q8g_stack_op &op, const OpInfo &oi, const Share &s, int t,
                                           int64_t lane_off, WBatch &b)
{
    const int q = t / s.bpg, u = t % s.bpg;
    const int64_t K = op.K;
    const int nr = s.count - q * R;  // rows of this group (>= 1)
    const char *rw[R];
    const uint16_t *rd[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const RowPtr p = locate(op, oi, s.first + (int64_t)q * R + (r < nr ? r : 0));
        rw[r] = uni_ptr(p.w);  // wave-uniform: scalar registers
        rd[r] = uni_ptr(p.dw);
    }
#pragma unroll
    for (int j = 0; j < kB; ++j) {
        const int r = j % R;
        int c = u * (kB / R) + j / R;
        if (c >= s.C) c = s.C - 1;
        const int64_t off = (int64_t)c * kChunk + lane_off;
        const int64_t o = off < K ? off : 0;
        b.w[j] = ld_w16(rw[r] + o);
        b.s[j] = ld_ws(rd[r] + (o >> 5));
    }
}

template <int R>
__device__ __forceinline__ void compute_batch(const WBatch &b, const Share &s, int t, int64_t K, int64_t lane_off,
                                              float even, const int8_t *s_qx, const float *s_dx, float (&acc)[R])
{
    const int u = t % s.bpg;
#pragma unroll
    for (int j = 0; j < kB; ++j) {
        const int r = j % R;
        const int c = u * (kB / R) + j / R;
        if (c < s.C) {
            const int64_t off = (int64_t)c * kChunk + lane_off;
            const bool active = off < K;
            const int64_t o = active ? off : 0;
            const int4 xq = *reinterpret_cast<const int4 *>(s_qx + o);
            const float xs = active ? s_dx[o >> 5] * even : 0.0f;
            const int sum = q8_block_sum(b.w[j], xq);
            acc[r] = __builtin_fmaf((float)sum, f16_bits_to_f32(b.s[j]) * xs, acc[r]);
        }
    }
}

template <int R>
__device__ __forceinline__ void settle(float (&acc)[R])
{
#pragma unroll
    for (int r = 0; r < R; ++r) asm volatile("" : "+v"(acc[r]));
}

// After batch t: if it closes its group, reduce the group's rows and store them
// (+ the residual, added once), then clear the accumulators.
template <int R>
__device__ __forceinline__ void finish(const q8g_stack_op &op, const OpInfo &oi, const Share &s, int t, int lane,
                                       const float *s_res, bool res_staged, float (&acc)[R])
{
    if (t % s.bpg != s.bpg - 1) return;
    const int q = t / s.bpg;
    const int nr = s.count - q * R;
    const float total = wave_reduce_rows<R>(acc, lane);
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (r < nr && lane == lane_of<R>(r)) {
            const int64_t row = s.first + (int64_t)q * R + r;
            const RowPtr p = locate(op, oi, row);
            // each branch stores on its own: a join after the global load would make
            // the compiler wait for every load in flight (the next batch's too)
            if (!p.res)
                st_dev_f(p.y, total);
            else if (res_staged)
                st_dev_f(p.y, total + s_res[row - s.slice0]);
            else
                st_dev_f(p.y, total + ld_dev_f(p.res));
        }
        acc[r] = 0.0f;
    }
}

// A compute wave's work on one op; `cur` holds batch 0 on entry.
template <int R>
__device__ __forceinline__ void run_share(const q8g_stack_op &op, const OpInfo &oi, const Share &s, int lane,
                                          const int8_t *s_qx, const float *s_dx, const float *s_res, bool res_staged,
                                          WBatch &cur, WBatch &nxt)
{
    const int64_t K = op.K;
    const int64_t lane_off = (int64_t)lane * 16;
    const float even = (lane & 1) ? 0.0f : 1.0f;
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.0f;
    const int nb = s.nbatch;
    int t = 0;
    // two batches a trip, cur and nxt taking turns (as in the standalone kernel):
    // each batch's loads are requested one batch ahead of its compute
    for (; t + 2 < nb; t += 2) {
        load_batch<R>(op, oi, s, t + 1, lane_off, nxt);
        __builtin_amdgcn_sched_barrier(0);
        compute_batch<R>(cur, s, t, K, lane_off, even, s_qx, s_dx, acc);
        settle(acc);
        finish<R>(op, oi, s, t, lane, s_res, res_staged, acc);
        load_batch<R>(op, oi, s, t + 2, lane_off, cur);
        __builtin_amdgcn_sched_barrier(0);
        compute_batch<R>(nxt, s, t + 1, K, lane_off, even, s_qx, s_dx, acc);
        settle(acc);
        finish<R>(op, oi, s, t + 1, lane, s_res, res_staged, acc);
    }
    if (t + 1 < nb) {
        load_batch<R>(op, oi, s, t + 1, lane_off, nxt);
        __builtin_amdgcn_sched_barrier(0);
        compute_batch<R>(cur, s, t, K, lane_off, even, s_qx, s_dx, acc);
        settle(acc);
        finish<R>(op, oi, s, t, lane, s_res, res_staged, acc);
        compute_batch<R>(nxt, s, t + 1, K, lane_off, even, s_qx, s_dx, acc);
        finish<R>(op, oi, s, t + 1, lane, s_res, res_staged, acc);
    } else if (t < nb) {
        compute_batch<R>(cur, s, t, K, lane_off, even, s_qx, s_dx, acc);
        finish<R>(op, oi, s, t, lane, s_res, res_staged, acc);
    }
}

__device__ __forceinline__ void issue_first(const q8g_stack_op &op, const OpInfo &oi, const Share &s, int lane,
                                            WBatch &b)
{
    if (s.nbatch == 0) return;
    const int64_t lane_off = (int64_t)lane * 16;
    if (s.R == 4)
        load_batch<4>(op, oi, s, 0, lane_off, b);
    else if (s.R == 2)
        load_batch<2>(op, oi, s, 0, lane_off, b);
    else
        load_batch<1>(op, oi, s, 0, lane_off, b);
}

// On-chip state of a workgroup.
struct Smem {
    q8g_stack_op ops[kMaxOps];
    OpInfo info[kMaxOps];
    __attribute__((aligned(16))) int8_t qx[Q8G_STACK_MAX_K];
    float dx[Q8G_STACK_MAX_K / 32];
    float res[kResMax];
    uint8_t pub[64];
    int abort;
    int res_ok;
    uint32_t T;
};

// Quantize values e..e+3 of op's input (an aligned group of 8 lanes holds one
// 32-value block) into LDS; workgroup 0 also writes the optional codes and scales.
__device__ __forceinline__ void quantize_store(const q8g_stack_op &op, int64_t e, const float4 &v, int g, int lane,
                                               Smem &sm)
{
    float d;
    const uint32_t packed = quantize4(v, &d);
    *reinterpret_cast<uint32_t *>(sm.qx + e) = packed;
    const uint16_t bits = scale_bits(d);
    if ((lane & 7) == 0) {
        sm.dx[e >> 5] = f16_bits_to_f32(bits);
        if (g == 0 && op.dx) st_u16(op.dx + (e >> 5), bits);
    }
    if (g == 0 && op.qx) st_u32(op.qx + e, packed);
}

// Quantize an f32 input into LDS with every thread of the workgroup (the
// arithmetic of q8_quantize_act); workgroup 0 also writes the optional codes and
// scales. COHERENT: the input is an earlier op's output of this launch.
template <bool COHERENT>
__device__ __forceinline__ void quantize_input(const q8g_stack_op &op, int g, int lane, Smem &sm)
{
    const int64_t K = op.K;
    for (int64_t e = (int64_t)threadIdx.x * 4; e < K; e += 4 * kThreads) {
        float4 v;
        if constexpr (COHERENT) {
            const uint64_t a = ld_dev64(reinterpret_cast<const uint64_t *>(op.x + e));
            const uint64_t c = ld_dev64(reinterpret_cast<const uint64_t *>(op.x + e + 2));
            v = make_float4(__builtin_bit_cast(float, (uint32_t)a), __builtin_bit_cast(float, (uint32_t)(a >> 32)),
                            __builtin_bit_cast(float, (uint32_t)c), __builtin_bit_cast(float, (uint32_t)(c >> 32)));
        } else {
            v = ld_f4(op.x + e);
        }
        quantize_store(op, e, v, g, lane, sm);
    }
}

// Residuals of op i's rows of this workgroup into LDS (wave 0).
__device__ __forceinline__ void stage_residuals(const q8g_stack_op &op, const OpInfo &oi, int G, int g, int lane,
                                                bool coherent, Smem &sm)
{
    const bool ok = oi.m <= kResMax;
    if (ok && oi.has_res)
        for (int j = lane; j < oi.m; j += kWave) {
            const RowPtr p = locate(op, oi, oi.r0 + j);
            sm.res[j] = p.res ? (coherent ? ld_dev_f(p.res) : ld_f(p.res)) : 0.0f;
        }
    if (lane == 0) sm.res_ok = ok ? 1 : 0;
}

__device__ __forceinline__ Share uniform_share(const Share &s)
{
    Share u;
    u.first = uni64(s.first);
    u.slice0 = uni64(s.slice0);
    u.count = uni32(s.count);
    u.R = uni32(s.R);
    u.C = uni32(s.C);
    u.bpg = uni32(s.bpg);
    u.nbatch = uni32(s.nbatch);
    return u;
}

// Waves 1..15: the rows of every op. The barriers match sync_role's one for one.
__device__ void compute_role(int nops, int G, int g, int wave, int lane, Smem &sm)
{
    WBatch cur, nxt;
    // op 0: the weights are requested after this thread's input values, so that the
    // quantization waits only for the input (every load is issued, past-the-end ones
    // at the last four values: K >= 32)
    {
        const q8g_stack_op &op = sm.ops[0];
        const int64_t K = op.K;
        float4 xin[kXPass];
#pragma unroll
        for (int p = 0; p < kXPass; ++p) {
            const int64_t e = (int64_t)threadIdx.x * 4 + (int64_t)p * 4 * kThreads;
            xin[p] = ld_f4(op.x + (e < K ? e : K - 4));
        }
        issue_first(op, sm.info[0], uniform_share(share_of(sm.info[0], wave)), lane, cur);
#pragma unroll
        for (int p = 0; p < kXPass; ++p) {
            const int64_t e = (int64_t)threadIdx.x * 4 + (int64_t)p * 4 * kThreads;
            if (e < K) quantize_store(op, e, xin[p], g, lane, sm);
        }
    }
    lds_barrier();
    for (int i = 0; i < nops; ++i) {
        const q8g_stack_op &op = sm.ops[i];
        const OpInfo &oi = sm.info[i];
        const bool last = i + 1 == nops;
        const bool next_chained = !last && sm.info[i + 1].chained;
        const Share s = uniform_share(share_of(oi, wave));
        const bool staged = sm.res_ok != 0;
        if (s.R == 4)
            run_share<4>(op, oi, s, lane, sm.qx, sm.dx, sm.res, staged, cur, nxt);
        else if (s.R == 2)
            run_share<2>(op, oi, s, lane, sm.qx, sm.dx, sm.res, staged, cur, nxt);
        else
            run_share<1>(op, oi, s, lane, sm.qx, sm.dx, sm.res, staged, cur, nxt);
        if (next_chained) {
            // the next op reads an output: this wave's stores are acknowledged before
            // the workgroup arrives at the barrier
            __builtin_amdgcn_s_waitcnt(0);
        } else if (!last) {
            const q8g_stack_op &on = sm.ops[i + 1];
            issue_first(on, sm.info[i + 1], uniform_share(share_of(sm.info[i + 1], wave)), lane, cur);
        }
        lds_barrier();  // this workgroup has finished op i
        if (last) return;
        lds_barrier();  // wave 0 has passed the barrier and staged the next input
        if (sm.abort) return;
        if (next_chained) {
            const q8g_stack_op &on = sm.ops[i + 1];
            quantize_input<true>(on, g, lane, sm);
            lds_barrier();
            issue_first(on, sm.info[i + 1], uniform_share(share_of(sm.info[i + 1], wave)), lane, cur);
        }
    }
}

// Wave 0: publishes each next input, arrives at and waits for each barrier, and
// stages the next input and residuals in LDS.
__device__ void sync_role(int nops, int G, int g, int lane, uint32_t *sync, uint32_t *status, Smem &sm)
{
    uint32_t *counters = sync + kCounterBase;
    uint64_t *areas = reinterpret_cast<uint64_t *>(sync + kAreaBase);
    const uint32_t T = sm.T;
    quantize_input<false>(sm.ops[0], g, lane, sm);
    stage_residuals(sm.ops[0], sm.info[0], G, g, lane, false, sm);
    lds_barrier();
    for (int i = 0; i < nops; ++i) {
        const bool last = i + 1 == nops;
        const bool next_chained = !last && sm.info[i + 1].chained;
        const int64_t Kn = last ? 0 : sm.ops[i + 1].K;
        const int64_t nbn = Kn / 32;                // blocks of the next input
        const uint32_t tag = T + (uint32_t)i + 1u;  // tag of barrier i
        // the f32 values of the next input's blocks this workgroup owns (b = g + G m;
        // lanes 0-31 hold block m = 0, lanes 32-63 block m = 1), requested while the
        // compute waves work
        float xv = 0.0f;
        if (!last && !next_chained) {
            const int64_t b = g + (int64_t)G * (lane >> 5);
            if (b < nbn) xv = ld_f(sm.ops[i + 1].x + 32 * b + (lane & 31));
        }
        lds_barrier();  // this workgroup has finished op i
        if (last) return;

        const q8g_stack_op &on = sm.ops[i + 1];
        uint64_t *area = areas + (size_t)((i + 1) & 1) * (kAreaWords / 2);
        if (!next_chained) {
            // quantize and publish this workgroup's blocks of the next input
            for (int64_t m0 = 0; g + (int64_t)G * m0 < nbn; m0 += 2) {
                const int64_t b = g + (int64_t)G * (m0 + (lane >> 5));
                const bool have = b < nbn;
                float v = xv;
                if (m0 > 0) v = have ? ld_f(on.x + 32 * b + (lane & 31)) : 0.0f;
                // the quantizer of q8_quantize_act over the block's 32 values, one per lane
                float mx = fabsf(v);
                mx = xmax<1>(mx);
                mx = xmax<2>(mx);
                mx = xmax<4>(mx);
                mx = xmax<8>(mx);
                mx = xmax<16>(mx);
                const float d = mx / 127.0f;
                float q = 0.0f;
                if (d != 0.0f) q = fminf(fmaxf(__builtin_rintf(v / d), -127.0f), 127.0f);
                sm.pub[lane] = (uint8_t)(int8_t)(int)q;
                const uint16_t bits = scale_bits(d);
                // lanes 32 h + j (j < 8) store code word j of block h, lane 32 h + 8 its scale
                const int j = lane & 31, h = lane >> 5;
                if (have && j <= 8) {
                    const uint32_t payload = j < 8 ? *reinterpret_cast<const uint32_t *>(sm.pub + 32 * h + 4 * j)
                                                   : (uint32_t)bits;
                    st_dev64(area + kBlockWords * b + j, ((uint64_t)tag << 32) | payload);
                    if (j < 8 && on.qx) st_u32(on.qx + 32 * b + 4 * j, payload);
                    if (j == 8 && on.dx) st_u16(on.dx + b, bits);
                }
            }
        } else {
            __builtin_amdgcn_s_waitcnt(0);
        }
        if (lane == 0) arrive(counters + 64 * (g % kCounters));
        // wait until every workgroup has arrived at barrier i
        bool abort = false;
        {
            const int c = lane & (kCounters - 1);
            const uint32_t per = (uint32_t)((G - c + kCounters - 1) / kCounters);
            const uint32_t want = (T + (uint32_t)i + 1u) * per;
            for (long spin = 0;; ++spin) {
                const uint32_t v = ld_dev(counters + 64 * c);
                if (__all((int32_t)(v - want) >= 0)) break;
                if ((spin & 63) == 63 && (ld_dev(sync + kErrWord) != 0 || spin > kSpinLimit)) {
                    abort = true;
                    break;
                }
            }
        }
        if (!abort && !next_chained) {
            // the published blocks: 16-byte pairs of words, all requested before one
            // wait; the pass is read again while some word's tag is not yet this barrier's
            const int nwords = kBlockWords * (int)nbn;
            for (int p0 = 0; p0 < nwords && !abort; p0 += 2 * kWave * kPairs) {
                bool done = false;
                for (long spin = 0; !done; ++spin) {
                    u32x4 v[kPairs];
#pragma unroll
                    for (int k = 0; k < kPairs; ++k) {
                        const int w = p0 + 2 * (lane + kWave * k);
                        load16_dev(area, 8u * (uint32_t)(w < nwords ? w : 0), v[k]);
                    }
                    wait_loads(v);
                    bool ok = true;
#pragma unroll
                    for (int k = 0; k < kPairs; ++k) {
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const int w = p0 + 2 * (lane + kWave * k) + h;
                            if (w < nwords) {
                                const uint32_t payload = h ? v[k].z : v[k].x;
                                const uint32_t wtag = h ? v[k].w : v[k].y;
                                ok &= wtag == tag;
                                const int b = w / kBlockWords;
                                const int jw = w - b * kBlockWords;
                                if (jw < 8)
                                    *reinterpret_cast<uint32_t *>(sm.qx + 32 * b + 4 * jw) = payload;
                                else
                                    sm.dx[b] = f16_bits_to_f32((uint16_t)payload);
                            }
                        }
                    }
                    done = __all(ok);
                    if (!done && (spin & 63) == 63 && (ld_dev(sync + kErrWord) != 0 || spin > kSpinLimit)) {
                        abort = true;
                        break;
                    }
                }
            }
        }
        if (!abort) {
            stage_residuals(on, sm.info[i + 1], G, g, lane, true, sm);
            // workgroup 0 records this launch's barriers once every workgroup has passed
            // the last one (each read the old count before its first arrival)
            if (g == 0 && lane == 0 && i + 2 == nops) st_dev(sync + kTotalWord, T + (uint32_t)nops - 1u);
        } else if (lane == 0) {
            st_dev(sync + kErrWord, 1u);
            if (status) st_dev(status, 1u);
            sm.abort = 1;
        }
        lds_barrier();  // the next input is staged (or the launch gives up)
        if (sm.abort) return;
        if (next_chained) {
            quantize_input<true>(on, g, lane, sm);
            lds_barrier();
        }
    }
}

// chained0..3: bit i set when op i's input or a residual overlaps an earlier op's
// output (found on the host, where the descriptors are validated)
__global__ __launch_bounds__(kThreads) void stack_kernel(const q8g_stack_op *__restrict__ ops, int nops,
                                                         uint32_t *__restrict__ sync, uint32_t *__restrict__ status,
                                                         uint64_t chained0, uint64_t chained1, uint64_t chained2,
                                                         uint64_t chained3)
{
    __shared__ Smem sm;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int G = gridDim.x;
    const int g = blockIdx.x;

    // descriptors into LDS, per-op row ends, chained ops
    static_assert(sizeof(q8g_stack_op) % 8 == 0, "descriptors are copied in 8-byte words");
    {
        const GLOBAL uint64_t *src = gptr(reinterpret_cast<const uint64_t *>(ops));
        uint64_t *dst = reinterpret_cast<uint64_t *>(sm.ops);
        const int n8 = nops * (int)(sizeof(q8g_stack_op) / 8);
        for (int k = threadIdx.x; k < n8; k += kThreads) dst[k] = src[k];
    }
    if (threadIdx.x == 0) {
        sm.abort = 0;
        sm.T = ld_dev(sync + kTotalWord);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < nops; i += kThreads) {
        const q8g_stack_op &o = sm.ops[i];
        OpInfo oi;
        int64_t e = 0;
        for (int q = 0; q < 4; ++q) {
            e += q < o.nparts ? o.parts[q].n : 0;
            if (q < 3) oi.end[q] = q + 1 < o.nparts ? e : INT64_MAX;
        }
        oi.n = e;
        oi.r0 = e * g / G;
        oi.m = (int32_t)(e * (g + 1) / G - oi.r0);
        oi.rw = (oi.m + kWork - 1) / kWork;
        oi.R = oi.rw >= 4 ? 4 : (oi.rw >= 2 ? 2 : 1);
        oi.C = (int32_t)((o.K + kChunk - 1) / kChunk);
        const int cpb = kB / oi.R;  // chunks per batch
        oi.bpg = (oi.C + cpb - 1) / cpb;
        oi.pad = 0;
        const uint64_t word = (i >> 6) == 0 ? chained0 : (i >> 6) == 1 ? chained1 : (i >> 6) == 2 ? chained2 : chained3;
        oi.chained = (int32_t)((word >> (i & 63)) & 1u);
        bool hr = false;
        for (int q = 0; q < o.nparts; ++q) hr = hr || (o.parts[q].n > 0 && o.parts[q].residual);
        oi.has_res = hr ? 1 : 0;
        sm.info[i] = oi;
    }
    __syncthreads();
    if (wave == 0)
        sync_role(nops, G, g, lane, sync, status, sm);
    else
        compute_role(nops, G, g, wave, lane, sm);
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
    if (nops > kMaxOps) return Q8G_ERR_ARG;
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

// whether [p, p + bytes) overlaps an output (y, qx, dx) of op o
bool hits_output(const q8g_stack_op &o, const void *p, int64_t bytes)
{
    if (overlap(p, bytes, o.qx, o.K) || overlap(p, bytes, o.dx, o.K / 16)) return true;
    for (int q = 0; q < o.nparts; ++q)
        if (overlap(p, bytes, o.parts[q].y, o.parts[q].n * 4)) return true;
    return false;
}

// Bit i: op i reads an earlier op's output (its input or a residual), so the barrier
// before it must order that output's stores.
void chained_mask(const q8g_stack_op *ops, int nops, uint64_t (&mask)[4])
{
    mask[0] = mask[1] = mask[2] = mask[3] = 0;
    for (int i = 1; i < nops; ++i) {
        const q8g_stack_op &o = ops[i];
        bool ch = false;
        for (int j = 0; j < i && !ch; ++j) {
            ch = hits_output(ops[j], o.x, o.K * 4);
            for (int q = 0; q < o.nparts && !ch; ++q) ch = hits_output(ops[j], o.parts[q].residual, o.parts[q].n * 4);
        }
        if (ch) mask[i >> 6] |= 1ull << (i & 63);
    }
}

// One cooperative launch of stack_kernel over the workspace `sync` (checks done).
q8g_status launch_stack(const q8g_stack_op *ops, const q8g_stack_op *ops_dev, int nops, uint32_t *sync,
                        uint32_t *status, hipStream_t stream)
{
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return Q8G_ERR_LAUNCH;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return Q8G_ERR_LAUNCH;
    if (cus < 1 || cus > kMaxGroups) return Q8G_ERR_LAUNCH;
    const q8g_stack_op *o = ops_dev;
    int n = nops;
    uint32_t *s = sync;
    uint32_t *st = status;
    uint64_t m[4];
    chained_mask(ops, nops, m);
    void *args[] = {&o, &n, &s, &st, &m[0], &m[1], &m[2], &m[3]};
    const hipError_t e = hipLaunchCooperativeKernel(reinterpret_cast<const void *>(&stack_kernel), dim3(cus),
                                                    dim3(kThreads), args, 0, stream);
    return e == hipSuccess ? Q8G_OK : Q8G_ERR_LAUNCH;
}

// whether [p, p + bytes) overlaps any input or output of any op
bool touches_any(const q8g_stack_op *ops, int nops, const void *p, int64_t bytes)
{
    for (int i = 0; i < nops; ++i) {
        const q8g_stack_op &a = ops[i];
        if (overlap(p, bytes, a.x, a.K * 4) || overlap(p, bytes, a.qx, a.K) || overlap(p, bytes, a.dx, a.K / 16))
            return true;
        for (int q = 0; q < a.nparts; ++q) {
            const q8g_part &pt = a.parts[q];
            if (overlap(p, bytes, pt.w, pt.n * a.K) || overlap(p, bytes, pt.dw, pt.n * (a.K / 32) * 2) ||
                overlap(p, bytes, pt.y, pt.n * 4) || overlap(p, bytes, pt.residual, pt.n * 4))
                return true;
        }
    }
    return false;
}

q8g_status check_call(const q8g_stack_op *ops, const q8g_stack_op *ops_dev, int nops)
{
    if (nops < 0) return Q8G_ERR_ARG;
    if (nops == 0) return Q8G_OK;
    if (!ops || !ops_dev) return Q8G_ERR_NULL;
    if (!aligned(ops_dev, 8)) return Q8G_ERR_ALIGN;
    return validate(ops, nops);
}

}  // namespace

extern "C" q8g_status q8_decode_stack(const q8g_stack_op *ops, const q8g_stack_op *ops_dev, int nops,
                                      uint32_t *sync, void *stream)
{
    const q8g_status st = check_call(ops, ops_dev, nops);
    if (st != Q8G_OK || nops == 0) return st;
    if (!sync) return Q8G_ERR_NULL;
    if (!aligned(sync, 64)) return Q8G_ERR_ALIGN;
    return launch_stack(ops, ops_dev, nops, sync, nullptr, static_cast<hipStream_t>(stream));
}

// ---- the same step for callers that cannot allocate --------------------------
// The synchronization workspace lives in this file-scope array instead of a
// caller buffer. In host code `scratch` is only a stand-in for the symbol: its
// device address (one per device) comes from hipGetSymbolAddress, taken once per
// device with that device current, and only that address is passed to kernels.
static __device__ __align__(256) uint32_t scratch[Q8G_STACK_SYNC_WORDS];

namespace {

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
uint32_t *g_scratch[kMaxDevices];  // device address of `scratch` on each device, once taken

q8g_status scratch_on(int dev, uint32_t **out)
{
    if (dev < 0 || dev >= kMaxDevices) return Q8G_ERR_LAUNCH;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return Q8G_ERR_LAUNCH;
        g_scratch[dev] = static_cast<uint32_t *>(p);
    }
    *out = g_scratch[dev];
    return Q8G_OK;
}

// zero n words (a kernel, not a memset node, so that a captured graph replays it faithfully)
__global__ __launch_bounds__(1024) void zero_words(uint32_t *__restrict__ p, int n)
{
    for (int i = blockIdx.x * 1024 + threadIdx.x; i < n; i += gridDim.x * 1024) p[i] = 0u;
}

}  // namespace

extern "C" q8g_status q8_decode_stack_static(const q8g_stack_op *ops, const q8g_stack_op *ops_dev, int nops,
                                             uint32_t *status, void *stream)
{
    const q8g_status st = check_call(ops, ops_dev, nops);
    if (st != Q8G_OK || nops == 0) return st;
    if (status && !aligned(status, 4)) return Q8G_ERR_ALIGN;
    if (status && touches_any(ops, nops, status, 4)) return Q8G_ERR_OVERLAP;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return Q8G_ERR_LAUNCH;
    uint32_t *ws = nullptr;
    const q8g_status sst = scratch_on(dev, &ws);
    if (sst != Q8G_OK) return sst;
    // every call starts from a cleared workspace: no state carries over between calls
    const hipStream_t s = static_cast<hipStream_t>(stream);
    uint32_t *p = ws;
    int n = Q8G_STACK_SYNC_WORDS;
    void *zargs[] = {&p, &n};
    if (hipLaunchKernel(reinterpret_cast<const void *>(&zero_words), dim3((n + 1023) / 1024), dim3(1024), zargs, 0, s) !=
        hipSuccess)
        return Q8G_ERR_LAUNCH;
    return launch_stack(ops, ops_dev, nops, ws, status, s);
}
