// Small-batch Q8_0 decode GEMV on the matrix cores (q8_gemv_batch in
// include/q8gemv.h): B <= 16 activation vectors share one pass over the
// weights, so each weight byte read from HBM serves B outputs.
//
// What is computed is the Q8_0 product of "Filling in the blanks: Inference
// using Phobos", section Fast Decode (32 int8 codes per block with their own
// scale, block math in integers), once per activation vector:
//   y[b][n] = sum_blk isum(n, b, blk) * (f16(dw[n][blk]) * f16(dx[b][blk])) (+ residual[b][n]).
// With B vectors the work is a skinny dense contraction, so the integer block
// sums come from v_mfma_i32_16x16x64_i8 rather than from per-lane dot4:
//
//  * One MFMA tile is 16 activation vectors (M, zero beyond B) x 16 weight rows
//    (N) x 64 k (two Q8_0 blocks). Operand lane l holds 16 contiguous bytes:
//    row l % 16, k group l / 16 (groups 0-1 are the first block, 2-3 the
//    second), so a wave's weight load is 16 rows x 64 contiguous bytes.
//  * Each block needs its own exact int32 sum before its scales apply, so a
//    step issues two MFMAs on the same weight operand, the first with the
//    activation groups of the second block zeroed and the second with those of
//    the first block zeroed. The MFMA work doubles; it stays far below the
//    matrix cores' rate, and the weight stream is what bounds the kernel.
//  * Lane l of the result holds vectors 4(l/16)..+3 of weight row l % 16, so
//    a lane applies one weight scale and four activation scales per block,
//    as float(isum) * (dw * dx) accumulated in f32 (the product of two
//    binary16 values is exact in f32, and so is float(isum)).
//  * The activation codes and scales of a tile of TK columns are copied
//    into LDS with direct global-to-LDS loads (gfx950 global_load_lds): no
//    registers hold them in flight and no wave waits on them before its
//    weight stream is requested. Each lane picks its own source address, so
//    the copy lays the codes out XOR-swizzled (16-byte chunk c of vector b at
//    position c ^ b within its group of 16), which makes the 16 vectors' reads
//    of one k group hit distinct banks, and gathers the scales transposed to
//    [block][vector], so a lane reads its four vectors' scales in one load.
//  * Each wave also copies its 16 rows' weight scales for the tile into LDS
//    (two rows' 64-byte scale runs per load). Loading them per step instead
//    would make every step's load touch 16 rows' scale lines for 4 useful
//    bytes each: on MI355X that kept the address unit waiting on the L1 cache
//    and held the kernel to well under half of the HBM rate.
//  * Weights stream through registers in a rolling window of P steps per
//    wave; the steady-state loop issues unconditionally, so the compiler keeps
//    the window in flight instead of waiting for every load.
//  * S waves of a workgroup may split the K range of one 16-row tile (16 or 4
//    for matrices with few tiles, so that enough waves exist); their partial
//    sums are added in a fixed order through LDS.
//  * Weight layouts ("Filling in the blanks", section GPU Performance
//    Heisenbugs: decode weights stored eight columns side by side, so a
//    warp's loads span full 128-byte lines). In the row layout a step's operand load is 16
//    rows x 64 bytes, 16 cache lines per KiB, half of each line used by the
//    step. The tiled layout (Q8G_LAYOUT_TILE16, written once by
//    q8_pack_tile16) stores each 16-row x 64-column step operand as one
//    contiguous KiB in the lane order of the load (lane l reads bytes
//    [16l, 16l + 16)), and each block's 16 row scales side by side, so a step
//    covers 8 full 128-byte lines. Only addresses differ: both layouts compute
//    every output with the same instructions in the same order.
//  * Output heads in the tiled layout (many tiles, K of 8 or 16 steps) run a
//    persistent form (stream_kernel): one 8-wave workgroup per compute unit
//    stages the activation once, and each wave streams its tiles back to back
//    with one window of loads across tile boundaries. Same arithmetic, same bits.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemv_device.hpp"
#include "q8gemv.h"

namespace {

using namespace q8g;

constexpr int kBatchMax = Q8G_BATCH_MAX;  // MFMA M dimension
constexpr int kTileRows = 16;             // weight rows per tile (MFMA N dimension)
constexpr int kStepK = 64;                // k per MFMA step (two Q8_0 blocks)
constexpr int64_t kMaxElems = (int64_t)1 << 60;
constexpr int64_t kMaxK = (int64_t)1 << 27;  // 16 rows x K bytes of a tile addressed with 32-bit offsets
// 16-row tile counts that select the launch shape (MI355X has 256 compute units)
constexpr int64_t kWideSplitTiles = 256;  // up to this many: 16 waves per tile, one workgroup per unit
constexpr int64_t kSplitTiles = 2048;     // up to this many: 4 waves per tile

// Launch shape: W waves per workgroup, S of them splitting the K range of one
// 16-row tile (W / S tiles per workgroup), P weight steps in flight per wave,
// TK activation columns staged in LDS at a time.
//
// LDS: [16 zero bytes][activation scales: TK/32 blocks x 16 vectors, one dword
//      each][codes: 16 vectors x TK bytes, XOR-swizzled][weight scales: per
//      tile, the S split waves' regions of 16 rows x their blocks, one dword
//      each]. The zero slot is what a lane reads for an operand group that must
//      be zero (another block's half of a step, a vector past B); it also keeps
//      every direct-load destination away from LDS offset 0.
template <int W_, int S_, int P_, int TK_>
struct Shape {
    static constexpr int W = W_, S = S_, P = P_, TK = TK_;
    static constexpr int kThreads = W * kWave;
    static constexpr int kTiles = W / S;
    static constexpr int kDxOff = 16;
    static constexpr int kCodesOff = kDxOff + (TK / 32) * kBatchMax * 4;
    static constexpr int kWscOff = kCodesOff + kBatchMax * TK;
    static constexpr int kWscTile = kTileRows * (TK / 32) * 4;
    static constexpr int kLds = kWscOff + kTiles * kWscTile;
    static_assert(W % S == 0 && W >= 1 && W <= 16, "whole tiles per workgroup");
    static_assert(TK % kStepK == 0 && (TK / 16) % 16 == 0, "tile of whole steps and chunk groups");
    static_assert(kCodesOff % 16 == 0, "16-byte aligned code area");
    static_assert(kThreads * 4 * 4 <= kBatchMax * TK, "partials fit in the code area");
    static_assert(kLds <= 160 * 1024, "LDS per workgroup");
};
// Matrices with few 16-row tiles (the decode stack's narrow projections): 16
// waves split each tile's K range, so that the launch spreads over enough
// compute units, and a 4096-column staging tile covers K <= 4096 in one pass.
using WideSplitShape = Shape<16, 16, 2, 4096>;
// A few hundred to a few thousand tiles: 4 waves per tile, small workgroups so
// that four fit on a compute unit and the launch runs in one round.
using SplitShape = Shape<4, 4, 4, 1024>;
// Many tiles (output heads): each wave streams whole rows of K with 8 steps in
// flight; small staging tiles keep four workgroups per compute unit.
using WholeShape = Shape<4, 1, 8, 1024>;

__device__ __forceinline__ v4i as_v4i(const int4 &v) { return v4i{v.x, v.y, v.z, v.w}; }

// s_waitcnt with vmcnt <= vm (vm < 64; 63 waits for nothing) and lgkmcnt <= lgkm
// (lgkm < 16), expcnt left alone. The barriers below are bare s_barrier
// instructions, and on gfx950 the compiler puts no wait in front of one, so a
// wave's own LDS writes (lgkmcnt) and direct global-to-LDS copies (vmcnt) are
// waited for here before other waves may read them.
template <int vm, int lgkm>
__device__ __forceinline__ void wait_counts()
{
    static_assert(vm >= 0 && vm < 64 && lgkm >= 0 && lgkm < 16, "counter range");
    __builtin_amdgcn_s_waitcnt((vm & 0xF) | ((vm >> 4) << 14) | (0x7 << 4) | (lgkm << 8));
}

// Direct copies of the activation codes and scales of columns [k0, k0 + kt)
// into LDS, requested by every wave of the workgroup (one wave's loads
// complete in issue order, so these are older than any weight request that
// follows). Codes: LDS chunk position p -> vector p / rowc16, chunk
// (p % rowc16) ^ vector; positions past the real chunks copy chunk 0 of their
// vector and are never read. Scales: LDS dword t -> block t / 16, vector t % 16
// (vectors past B copy vector B-1; their outputs are never stored).
template <class SH>
__device__ __forceinline__ void stage_activation(uint8_t *s_lds, const int8_t *__restrict__ qx,
                                                 const uint16_t *__restrict__ dx, int64_t K, int64_t k0, int kt,
                                                 int B, int wave, int lane)
{
    constexpr int W = SH::W;
    uint8_t *const s_codes = s_lds + SH::kCodesOff;
    const int64_t nb = K / 32;
    const int nbt = kt / 32;
    const int cpv = kt / 16;
    const int rowc16 = (cpv + 15) & ~15;
    const int code_pos = B * rowc16;
    for (int p0 = wave * kWave; p0 < code_pos; p0 += W * kWave) {
        const int p = p0 + lane;
        const int b = p / rowc16, c = (p - b * rowc16) ^ (b & 15);
        const int bb = b < B ? b : B - 1;
        const int cc = c < cpv ? c : 0;
        if (p < code_pos)
            __builtin_amdgcn_global_load_lds(qx + (int64_t)bb * K + k0 + 16 * cc, s_codes + 16 * p0, 16, 0, 0);
    }
    const int dx_pos = nbt * kBatchMax;
    for (int p0 = wave * kWave; p0 < dx_pos; p0 += W * kWave) {
        const int t = p0 + lane;
        const int blk = t / kBatchMax, b = t - blk * kBatchMax;
        const int bb = b < B ? b : B - 1;
        if (t < dx_pos)
            __builtin_amdgcn_global_load_lds(dx + (int64_t)bb * nb + k0 / 32 + blk, s_lds + SH::kDxOff + 4 * p0, 2,
                                             0, 0);
    }
}

template <class SH, bool TILED>
__global__ __launch_bounds__(SH::kThreads) void batch_kernel(const int8_t *__restrict__ qw,
                                                            const uint16_t *__restrict__ dw,
                                                            const int8_t *__restrict__ qx,
                                                            const uint16_t *__restrict__ dx,
                                                            const float *residual, float *y, int64_t N, int64_t K,
                                                            int B)
{
    constexpr int S = SH::S, P = SH::P, TK = SH::TK;
    __shared__ __align__(16) uint8_t s_lds[SH::kLds];
    uint8_t *const s_codes = s_lds + SH::kCodesOff;
    const float *const s_dxf = reinterpret_cast<const float *>(s_lds + SH::kDxOff);

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int tile = wave / S, split = wave % S;
    const int j = lane & 15;  // weight row in the tile / activation vector of the operand
    const int q = lane >> 4;  // 16-byte k group of a step
    const int64_t row0 = ((int64_t)blockIdx.x * SH::kTiles + tile) * kTileRows;  // wave-uniform
    const int64_t row = row0 + j;
    const bool row_ok = row < N;
    const int64_t nb = K / 32;
    // a wave-uniform base and a 32-bit lane offset in [0, 16) rows (rows of at
    // most 2^27 bytes; larger K is refused on the host). Rows past N re-read
    // row N-1; a tile wholly past N (in the last workgroup) re-reads it too.
    const int64_t rbase = row0 < N ? row0 : N - 1;
    const int jr = (int)((row_ok ? row : N - 1) - rbase);
    const int8_t *wbase = qw + rbase * K;
    const uint32_t woff = (uint32_t)jr * (uint32_t)K;
    // tiled layout: tile tg's step st is the KiB at (tg * steps_row + st) * 1024; a
    // tile wholly past N (in the last workgroup) re-reads the last tile
    const int64_t ntiles = (N + kTileRows - 1) / kTileRows;
    const int64_t tg = row0 / kTileRows < ntiles ? row0 / kTileRows : ntiles - 1;
    const int64_t steps_row = (K + kStepK - 1) / kStepK;
    const int8_t *tbase = qw + tg * steps_row * 1024 + 16 * lane;

    if (threadIdx.x == 0) *reinterpret_cast<uint4 *>(s_lds) = make_uint4(0u, 0u, 0u, 0u);  // the zero slot

    // The residuals of the four outputs this lane stores are requested before
    // anything else, so the store at the end waits for no further memory round
    // trip (the first barrier's wait covers them). Every lane loads, clamped into
    // [B][N]; the values of rows past N and vectors past B are never stored. The
    // branch is uniform and nothing reads the values before the end, so no wait
    // is placed at its join.
    float res[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (residual) {
        const int64_t rr = row_ok ? row : N - 1;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int b = 4 * q + r < B ? 4 * q + r : B - 1;
            res[r] = residual[(int64_t)b * N + rr];
        }
    }

    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int64_t k0 = 0; k0 < K; k0 += TK) {
        const int kt = (int)(K - k0 < TK ? K - k0 : TK);  // multiple of 32
        const int nbt = kt / 32;
        const int cpv = kt / 16;              // 16-byte chunks per vector
        const int rowc16 = (cpv + 15) & ~15;  // LDS chunks per vector (whole groups of 16)
        const int steps = (kt + kStepK - 1) / kStepK;
        const int s_begin = steps * split / S, s_end = steps * (split + 1) / S;

        // 1. direct copies of the activation into LDS, requested first
        stage_activation<SH>(s_lds, qx, dx, K, k0, kt, B, wave, lane);
        const int dx_pos = nbt * kBatchMax;
        //    Weight scales of this wave's rows and steps, into its region of the
        //    tile's area: LDS dword t -> row t / nbw, block t % nbw of the
        //    wave's blocks (rows past N read row N-1; a missing second block of
        //    the last step reads the first, and its product is zero).
        const int nbw = 2 * (s_end - s_begin);
        const int64_t blk0 = k0 / 32 + 2 * s_begin;
        uint8_t *const s_wsc = s_lds + SH::kWscOff + tile * SH::kWscTile + kTileRows * 4 * (2 * s_begin);
        for (int p0 = 0; p0 < kTileRows * nbw; p0 += kWave) {
            const int t = p0 + lane;
            const int r = t / nbw, bo = t - r * nbw;
            const int64_t rr = row0 + r < N ? row0 + r : N - 1;
            const int64_t bk = blk0 + bo < nb ? blk0 + bo : blk0;
            // tiled: block bk of tile tg holds its 16 rows' scales side by side (rows
            // past N are padding inside the tile)
            const uint16_t *src = TILED ? dw + (tg * nb + bk) * kTileRows + r : dw + rr * nb + bk;
            if (t < kTileRows * nbw) __builtin_amdgcn_global_load_lds(src, s_wsc + 4 * p0, 2, 0, 0);
        }

        // 2. the first window of weights (one load per step). Steps past the
        //    wave's share re-read its last step, so every issue is unconditional.
        int4 wv[P];
        auto issue = [&](int p, int st) {
            if (TILED) {
                // a missing second block reads the tile's zero padding
                wv[p] = load16_stream(tbase + (k0 / kStepK + st) * 1024);
            } else {
                const bool hi = st * kStepK + 32 < kt;  // the step's second block exists
                wv[p] = load16_stream(wbase + (woff + ((q < 2 || hi) ? (uint32_t)(k0 + st * kStepK + 16 * q) : 0u)));
            }
        };
        const int last = s_end > s_begin ? s_end - 1 : s_begin;
#pragma unroll
        for (int p = 0; p < P; ++p) issue(p, s_begin + p < s_end ? s_begin + p : last);

        // 3. the copies are older than the P weight loads: wait for them (and
        //    for the zero slot's LDS store) only, then a bare barrier; a full
        //    __syncthreads would also wait for the weights
        wait_counts<P, 0>();
        __builtin_amdgcn_s_barrier();
        //    the staged activation scale bits to f32, in place, once per tile;
        //    the rewritten words are complete before the barrier
        for (int t = threadIdx.x; t < dx_pos; t += SH::kThreads) {
            uint32_t *v = reinterpret_cast<uint32_t *>(s_lds + SH::kDxOff) + t;
            *v = __builtin_bit_cast(uint32_t, f16_bits_to_f32((uint16_t)*v));
        }
        wait_counts<63, 0>();
        __builtin_amdgcn_s_barrier();

        auto consume = [&](int p, int st) {
            const bool hi = st * kStepK + 32 < kt;
            const v4i zero = {0, 0, 0, 0};
            // operand groups 0-1 feed the first block's MFMA, 2-3 the second's;
            // a lane whose group belongs to the other block (or to a vector
            // past B, or to a missing second block) reads the zero slot
            const int c = 4 * st + q;  // the lane's 16-byte chunk of vector j
            const uint32_t at = SH::kCodesOff + 16u * (uint32_t)(j * rowc16 + (c ^ j));
            const bool lo_ok = j < B && q < 2, hi_ok = j < B && q >= 2 && hi;
            const v4i a_lo = *reinterpret_cast<const v4i *>(s_lds + (lo_ok ? at : 0u));
            const v4i a_hi = *reinterpret_cast<const v4i *>(s_lds + (hi_ok ? at : 0u));
            const v4i w = as_v4i(wv[p]);
            const v4i i0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a_lo, w, zero, 0, 0, 0);
            const v4i i1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a_hi, w, zero, 0, 0, 0);
            const int blk = 2 * st;  // within the tile
            const float4 x0 = *reinterpret_cast<const float4 *>(s_dxf + blk * kBatchMax + 4 * q);
            const float4 x1 = hi ? *reinterpret_cast<const float4 *>(s_dxf + (blk + 1) * kBatchMax + 4 * q)
                                 : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            const uint2 ws = *reinterpret_cast<const uint2 *>(s_wsc + 4 * (j * nbw + 2 * (st - s_begin)));
            const float w0 = f16_bits_to_f32((uint16_t)ws.x), w1 = f16_bits_to_f32((uint16_t)ws.y);
            acc[0] = __builtin_fmaf((float)i0[0], w0 * x0.x, acc[0]);
            acc[1] = __builtin_fmaf((float)i0[1], w0 * x0.y, acc[1]);
            acc[2] = __builtin_fmaf((float)i0[2], w0 * x0.z, acc[2]);
            acc[3] = __builtin_fmaf((float)i0[3], w0 * x0.w, acc[3]);
            acc[0] = __builtin_fmaf((float)i1[0], w1 * x1.x, acc[0]);
            acc[1] = __builtin_fmaf((float)i1[1], w1 * x1.y, acc[1]);
            acc[2] = __builtin_fmaf((float)i1[2], w1 * x1.z, acc[2]);
            acc[3] = __builtin_fmaf((float)i1[3], w1 * x1.w, acc[3]);
            // one step at a time: the empty asm makes this step's sums exist here,
            // so the compiler cannot sink them to the end of the window and keep
            // every MFMA result of the window live (registers, and so waves per
            // SIMD, are what a memory-bound loop needs)
            asm volatile("" : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]));
        };

        // 4. steady state: a whole window is consumed while the next is requested
        int s0 = s_begin;
        for (; s0 + P < s_end; s0 += P) {
#pragma unroll
            for (int p = 0; p < P; ++p) {
                consume(p, s0 + p);
                const int nx = s0 + P + p;
                issue(p, nx < s_end ? nx : s_end - 1);
            }
        }
        // the last window: consumed, nothing more requested
#pragma unroll
        for (int p = 0; p < P; ++p)
            if (s0 + p < s_end) consume(p, s0 + p);
        __syncthreads();  // the next tile's copies overwrite the staging area
    }


    if constexpr (S > 1) {
        // partial sums of the S waves of a tile, added in split order
        float *part = reinterpret_cast<float *>(s_codes);
#pragma unroll
        for (int r = 0; r < 4; ++r) part[(wave * kWave + lane) * 4 + r] = acc[r];
        __syncthreads();
        if (split != 0) return;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float t = part[(wave * kWave + lane) * 4 + r];
#pragma unroll
            for (int k = 1; k < S; ++k) t += part[((wave + k) * kWave + lane) * 4 + r];
            acc[r] = t;
        }
    }
    if (!row_ok) return;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int b = 4 * q + r;
        if (b < B) y[(int64_t)b * N + row] = residual ? acc[r] + res[r] : acc[r];
    }
}

// Many tiles, K <= TK, tiled layout: the whole-row shape made persistent. Each
// workgroup stages the activation once; each wave then streams its own tiles
// (every GW-th tile from its global wave index, GW waves in all) back to back,
// with one rolling window of P steps that runs across tile boundaries, so a
// wave's requests never drain between tiles. A tile's 16 x nb weight scales
// are nb * 32 contiguous bytes in the tiled layout: lane l < 2 nb requests
// bytes [16 l, 16 l + 16) one tile ahead, and the wave writes them to its own
// LDS area when the tile's first step is consumed (one wave's LDS accesses
// complete in order, so no barrier is needed). The residuals are requested one
// tile ahead as well. Every step runs the batched kernel's arithmetic in the
// same order, so the outputs equal its outputs bit for bit. Eight waves per
// workgroup and about eight per compute unit: measured on MI355X for the
// 151936 x 1024 head at 16 vectors, more waves per unit (two workgroups on
// one unit, or sixteen-wave workgroups) and four-wave workgroups were slower.
using StreamShape = Shape<8, 1, 8, 1024>;
constexpr int kStreamScaleBytes = kTileRows * (StreamShape::TK / 32) * 2;  // one tile's scales
constexpr int kStreamLds = StreamShape::kWscOff + StreamShape::W * kStreamScaleBytes;
static_assert(kStreamLds <= 160 * 1024, "LDS per workgroup");

template <int STEPS, bool RES>
__global__ __launch_bounds__(StreamShape::kThreads) void stream_kernel(const int8_t *__restrict__ qw,
                                                                       const uint16_t *__restrict__ dw,
                                                                       const int8_t *__restrict__ qx,
                                                                       const uint16_t *__restrict__ dx,
                                                                       const float *residual, float *y, int64_t N,
                                                                       int64_t K, int B, int ntiles)
{
    using SH = StreamShape;
    constexpr int W = SH::W, P = SH::P;
    static_assert(STEPS % P == 0 && STEPS * kStepK <= SH::TK, "whole windows per tile, one staging pass");
    __shared__ __align__(16) uint8_t s_lds[kStreamLds];
    const float *const s_dxf = reinterpret_cast<const float *>(s_lds + SH::kDxOff);

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int j = lane & 15;  // weight row in the tile / activation vector of the operand
    const int q = lane >> 4;  // 16-byte k group of a step
    const int gw = blockIdx.x * W + wave, GW = gridDim.x * W;
    const int nt = gw < ntiles ? (ntiles - 1 - gw) / GW + 1 : 0;  // this wave's tiles
    const int kt = (int)K;                                         // (STEPS - 1) * 64 < K <= STEPS * 64
    const int nb = kt / 32;
    const int rowc16 = (kt / 16 + 15) & ~15;
    uint8_t *const s_wsc = s_lds + SH::kWscOff + wave * kStreamScaleBytes;
    const uint16_t *const s_ws16 = reinterpret_cast<const uint16_t *>(s_wsc);
    auto tile_of = [&](int i) { return gw + i * GW; };  // the wave's tile i (i < nt)

    if (threadIdx.x == 0) *reinterpret_cast<uint4 *>(s_lds) = make_uint4(0u, 0u, 0u, 0u);  // the zero slot
    stage_activation<SH>(s_lds, qx, dx, K, 0, kt, B, wave, lane);

    // Requests are unconditional, with clamped addresses: lanes past a tile's
    // scale bytes re-read its first chunk, residuals of vectors past B and rows
    // past N read clamped elements (never stored), requests past the wave's
    // last tile re-read it, and a wave without tiles requests the last tile's
    // first steps. So every path issues the same loads in the same order after
    // the copies above, and the compiler's wait counts keep the window in flight.
    const int sl = lane < 2 * nb ? lane : 0;
    auto tile_scales = [&](int t) {
        return *reinterpret_cast<const int4 *>(dw + (int64_t)t * nb * kTileRows + 8 * sl);
    };
    auto tile_residuals = [&](int t, float (&r)[4]) {
        const int64_t row = (int64_t)t * kTileRows + j;
        const int64_t rr = row < N ? row : N - 1;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int b = 4 * q + k < B ? 4 * q + k : B - 1;
            r[k] = residual[(int64_t)b * N + rr];
        }
    };
    auto weights = [&](int t, int st) {
        return load16_stream(qw + ((int64_t)t * STEPS + st) * 1024 + 16 * lane);
    };

    const int t0 = nt > 0 ? gw : ntiles - 1;
    int4 wv[P];
    int4 sc = tile_scales(t0);
    float res_nx[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (RES) tile_residuals(t0, res_nx);
#pragma unroll
    for (int p = 0; p < P; ++p) wv[p] = weights(t0, p);

    // the copies are older than the weight window: wait for them only, then a
    // bare barrier
    wait_counts<P + 1 + (RES ? 4 : 0), 0>();
    __builtin_amdgcn_s_barrier();
    const int dx_pos = nb * kBatchMax;
    for (int t = threadIdx.x; t < dx_pos; t += SH::kThreads) {
        uint32_t *v = reinterpret_cast<uint32_t *>(s_lds + SH::kDxOff) + t;
        *v = __builtin_bit_cast(uint32_t, f16_bits_to_f32((uint16_t)*v));
    }
    wait_counts<63, 0>();
    __builtin_amdgcn_s_barrier();

    for (int i = 0; i < nt; ++i) {
        // tile i: its scales into the wave's area (its earlier reads are
        // complete: one wave's LDS accesses run in order); the next tile's
        // scales and residuals requested
        if (lane < 2 * nb) *reinterpret_cast<int4 *>(s_wsc + 16 * lane) = sc;
        float res[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) res[k] = res_nx[k];
        const bool more = i + 1 < nt;
        const int t = tile_of(i), tn = tile_of(more ? i + 1 : i);
        sc = tile_scales(tn);
        if (RES) tile_residuals(tn, res_nx);

        float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int st = 0; st < STEPS; ++st) {
            const int p = st % P;
            const bool hi = st * kStepK + 32 < kt;
            const v4i zero = {0, 0, 0, 0};
            const int c = 4 * st + q;
            const uint32_t at = SH::kCodesOff + 16u * (uint32_t)(j * rowc16 + (c ^ j));
            const bool lo_ok = j < B && q < 2, hi_ok = j < B && q >= 2 && hi;
            const v4i a_lo = *reinterpret_cast<const v4i *>(s_lds + (lo_ok ? at : 0u));
            const v4i a_hi = *reinterpret_cast<const v4i *>(s_lds + (hi_ok ? at : 0u));
            const v4i w = as_v4i(wv[p]);
            const v4i i0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a_lo, w, zero, 0, 0, 0);
            const v4i i1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a_hi, w, zero, 0, 0, 0);
            const int blk = 2 * st;
            const float4 x0 = *reinterpret_cast<const float4 *>(s_dxf + blk * kBatchMax + 4 * q);
            const float4 x1 = hi ? *reinterpret_cast<const float4 *>(s_dxf + (blk + 1) * kBatchMax + 4 * q)
                                 : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            // a missing second block reads the first block's scale; its product is zero
            const float w0 = f16_bits_to_f32(s_ws16[blk * kTileRows + j]);
            const float w1 = f16_bits_to_f32(s_ws16[(hi ? blk + 1 : blk) * kTileRows + j]);
            acc[0] = __builtin_fmaf((float)i0[0], w0 * x0.x, acc[0]);
            acc[1] = __builtin_fmaf((float)i0[1], w0 * x0.y, acc[1]);
            acc[2] = __builtin_fmaf((float)i0[2], w0 * x0.z, acc[2]);
            acc[3] = __builtin_fmaf((float)i0[3], w0 * x0.w, acc[3]);
            acc[0] = __builtin_fmaf((float)i1[0], w1 * x1.x, acc[0]);
            acc[1] = __builtin_fmaf((float)i1[1], w1 * x1.y, acc[1]);
            acc[2] = __builtin_fmaf((float)i1[2], w1 * x1.z, acc[2]);
            acc[3] = __builtin_fmaf((float)i1[3], w1 * x1.w, acc[3]);
            asm volatile("" : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]));
            // the step P ahead: in this tile, or the next (past the last tile, its
            // last step again)
            if (st + P < STEPS) {
                wv[p] = weights(t, st + P);
            } else {
                wv[p] = weights(tn, more ? st + P - STEPS : STEPS - 1);
            }
        }
        const int64_t row = (int64_t)t * kTileRows + j;
        if (row < N) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int b = 4 * q + k;
                if (b < B) y[(int64_t)b * N + row] = RES ? acc[k] + res[k] : acc[k];
            }
        }
    }
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlap(const void *a, int64_t abytes, const void *b, int64_t bbytes)
{
    if (!a || !b || abytes <= 0 || bbytes <= 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

template <class SH>
hipError_t launch(bool tiled, const int8_t *qw, const uint16_t *dw, const int8_t *qx, const uint16_t *dx,
                  const float *residual, float *y, int64_t N, int64_t K, int B, hipStream_t s)
{
    const int64_t tiles = (N + kTileRows - 1) / kTileRows;
    const int64_t groups = (tiles + SH::kTiles - 1) / SH::kTiles;
    void *args[] = {&qw, &dw, &qx, &dx, &residual, &y, &N, &K, &B};
    const void *fn = tiled ? reinterpret_cast<const void *>(&batch_kernel<SH, true>)
                           : reinterpret_cast<const void *>(&batch_kernel<SH, false>);
    return hipLaunchKernel(fn, dim3((unsigned)groups), dim3(SH::kThreads), args, 0, s);
}

// The persistent streaming form serves the tiled layout of matrices with many
// tiles whose K fits one staging pass (output heads of the small models); its
// tile scales are read as 16-byte chunks, so dw must be 16-byte aligned.
constexpr int kStreamWavesPerUnit = 8;  // waves per compute unit the tile split aims for
constexpr int kUnits = 256;             // compute units of an MI355X

bool stream_shape(int64_t N, int64_t K)
{
    const int64_t tiles = (N + kTileRows - 1) / kTileRows;
    const int64_t steps = (K + kStepK - 1) / kStepK;
    return tiles > kSplitTiles && (steps == 8 || steps == 16) && tiles * steps <= (int64_t)INT32_MAX;
}

bool stream_fits(bool tiled, const uint16_t *dw, int64_t N, int64_t K)
{
    return tiled && stream_shape(N, K) && aligned(dw, 16);
}

// Every wave takes ceil(tiles / waves) or one tile fewer: the number of waves is
// the fewest that give each at most ceil(tiles / (kUnits * kStreamWavesPerUnit))
// tiles, rounded up to whole workgroups.
int64_t stream_groups(int64_t tiles)
{
    const int64_t target = (int64_t)kUnits * kStreamWavesPerUnit;
    const int64_t per_wave = (tiles + target - 1) / target;
    const int64_t waves = (tiles + per_wave - 1) / per_wave;
    return (waves + StreamShape::W - 1) / StreamShape::W;
}

q8g_status launch_stream(const int8_t *qw, const uint16_t *dw, const int8_t *qx, const uint16_t *dx,
                         const float *residual, float *y, int64_t N, int64_t K, int B, hipStream_t s)
{
    int ntiles = (int)((N + kTileRows - 1) / kTileRows);
    void *args[] = {&qw, &dw, &qx, &dx, &residual, &y, &N, &K, &B, &ntiles};
    const bool r = residual != nullptr;
    const void *fn = (K + kStepK - 1) / kStepK == 16
                         ? (r ? reinterpret_cast<const void *>(&stream_kernel<16, true>)
                              : reinterpret_cast<const void *>(&stream_kernel<16, false>))
                         : (r ? reinterpret_cast<const void *>(&stream_kernel<8, true>)
                              : reinterpret_cast<const void *>(&stream_kernel<8, false>));
    const hipError_t e =
        hipLaunchKernel(fn, dim3((unsigned)stream_groups(ntiles)), dim3(StreamShape::kThreads), args, 0, s);
    return e == hipSuccess ? Q8G_OK : Q8G_ERR_LAUNCH;
}

// bytes of the tiled codes and scales of an N x K matrix (rows padded to whole
// 16-row tiles, each row's codes to whole 64-byte steps)
int64_t tile16_code_bytes(int64_t N, int64_t K)
{
    return (N + kTileRows - 1) / kTileRows * kTileRows * ((K + kStepK - 1) / kStepK * kStepK);
}
int64_t tile16_scale_bytes(int64_t N, int64_t K) { return (N + kTileRows - 1) / kTileRows * kTileRows * (K / 32) * 2; }

q8g_status batch_run(int layout, const int8_t *qw, const uint16_t *dw, const int8_t *qx, const uint16_t *dx,
                     const float *residual, float *y, int64_t N, int64_t K, int64_t B, void *stream)
{
    if (layout != Q8G_LAYOUT_ROWS && layout != Q8G_LAYOUT_TILE16) return Q8G_ERR_ARG;
    const bool tiled = layout == Q8G_LAYOUT_TILE16;
    if (N < 0 || K < 0 || B < 0 || B > kBatchMax || N > kMaxElems || K > kMaxElems) return Q8G_ERR_SHAPE;
    if (K % 32 || K > kMaxK) return Q8G_ERR_SHAPE;
    if (N > 0 && K > 0 && N > kMaxElems / K) return Q8G_ERR_SHAPE;
    if ((N + kTileRows - 1) / kTileRows > (int64_t)INT32_MAX) return Q8G_ERR_SHAPE;
    if (N == 0 || B == 0) return Q8G_OK;
    if (!y || (K > 0 && (!qw || !dw || !qx || !dx))) return Q8G_ERR_NULL;
    if (!aligned(qw, 16) || !aligned(qx, 16) || !aligned(dw, 2) || !aligned(dx, 2) || !aligned(y, 4) ||
        (residual && !aligned(residual, 4)))
        return Q8G_ERR_ALIGN;
    const int64_t ybytes = B * N * 4;
    const int64_t wbytes = tiled ? tile16_code_bytes(N, K) : N * K;
    const int64_t dwbytes = tiled ? tile16_scale_bytes(N, K) : N * (K / 32) * 2;
    if (overlap(y, ybytes, qw, wbytes) || overlap(y, ybytes, dw, dwbytes) || overlap(y, ybytes, qx, B * K) ||
        overlap(y, ybytes, dx, B * (K / 32) * 2))
        return Q8G_ERR_OVERLAP;
    // the residual may be y itself (each element is read, then written, by one lane)
    if (residual && residual != y && overlap(y, ybytes, residual, ybytes)) return Q8G_ERR_OVERLAP;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t tiles = (N + kTileRows - 1) / kTileRows;
    if (stream_fits(tiled, dw, N, K)) return launch_stream(qw, dw, qx, dx, residual, y, N, K, (int)B, s);
    const hipError_t e =
        tiles <= kWideSplitTiles ? launch<WideSplitShape>(tiled, qw, dw, qx, dx, residual, y, N, K, (int)B, s)
        : tiles <= kSplitTiles   ? launch<SplitShape>(tiled, qw, dw, qx, dx, residual, y, N, K, (int)B, s)
                                 : launch<WholeShape>(tiled, qw, dw, qx, dx, residual, y, N, K, (int)B, s);
    return e == hipSuccess ? Q8G_OK : Q8G_ERR_LAUNCH;
}

}  // namespace

extern "C" q8g_status q8_gemv_batch(const int8_t *qw, const uint16_t *dw, const int8_t *qx, const uint16_t *dx,
                                    const float *residual, float *y, int64_t N, int64_t K, int64_t B, void *stream)
{
    return batch_run(Q8G_LAYOUT_ROWS, qw, dw, qx, dx, residual, y, N, K, B, stream);
}

extern "C" q8g_status q8_gemv_batch_layout(int layout, const int8_t *qw, const uint16_t *dw, const int8_t *qx,
                                           const uint16_t *dx, const float *residual, float *y, int64_t N, int64_t K,
                                           int64_t B, void *stream)
{
    return batch_run(layout, qw, dw, qx, dx, residual, y, N, K, B, stream);
}

extern "C" q8g_status q8_tile16_sizes(int64_t N, int64_t K, int64_t *code_bytes, int64_t *scale_bytes)
{
    if (N < 0 || K < 0 || K % 32 || K > kMaxK || N > kMaxElems || (N > 0 && K > 0 && N > kMaxElems / K))
        return Q8G_ERR_SHAPE;
    if (!code_bytes || !scale_bytes) return Q8G_ERR_NULL;
    *code_bytes = tile16_code_bytes(N, K);
    *scale_bytes = tile16_scale_bytes(N, K);
    return Q8G_OK;
}

extern "C" q8g_status q8_pack_tile16(const int8_t *qw, const uint16_t *dw, int64_t N, int64_t K, int8_t *qw_tiled,
                                     uint16_t *dw_tiled)
{
    if (N < 0 || K < 0 || K % 32 || K > kMaxK || N > kMaxElems || (N > 0 && K > 0 && N > kMaxElems / K))
        return Q8G_ERR_SHAPE;
    if (N == 0 || K == 0) return Q8G_OK;
    if (!qw || !dw || !qw_tiled || !dw_tiled) return Q8G_ERR_NULL;
    const int64_t cb = tile16_code_bytes(N, K), sb = tile16_scale_bytes(N, K);
    if (overlap(qw_tiled, cb, qw, N * K) || overlap(qw_tiled, cb, dw, N * (K / 32) * 2) ||
        overlap(dw_tiled, sb, qw, N * K) || overlap(dw_tiled, sb, dw, N * (K / 32) * 2) ||
        overlap(qw_tiled, cb, dw_tiled, sb))
        return Q8G_ERR_OVERLAP;
    const int64_t tiles = (N + kTileRows - 1) / kTileRows, steps = (K + kStepK - 1) / kStepK, nb = K / 32;
    for (int64_t t = 0; t < tiles; ++t)
        for (int64_t st = 0; st < steps; ++st) {
            int8_t *o = qw_tiled + (t * steps + st) * 1024;
            for (int q = 0; q < 4; ++q)
                for (int j = 0; j < kTileRows; ++j)
                    for (int b = 0; b < 16; ++b) {
                        const int64_t row = t * kTileRows + j, col = st * kStepK + 16 * q + b;
                        o[16 * (16 * q + j) + b] = row < N && col < K ? qw[row * K + col] : 0;
                    }
        }
    for (int64_t t = 0; t < tiles; ++t)
        for (int64_t blk = 0; blk < nb; ++blk)
            for (int j = 0; j < kTileRows; ++j) {
                const int64_t row = t * kTileRows + j;
                dw_tiled[(t * nb + blk) * kTileRows + j] = row < N ? dw[row * nb + blk] : (uint16_t)0;
            }
    return Q8G_OK;
}

extern "C" q8g_status q8g_batch_config(int64_t N, int *k_split, int *steps_in_flight)
{
    if (N < 0) return Q8G_ERR_SHAPE;
    if (!k_split || !steps_in_flight) return Q8G_ERR_NULL;
    const int64_t tiles = (N + kTileRows - 1) / kTileRows;
    *k_split = tiles <= kWideSplitTiles ? WideSplitShape::S : tiles <= kSplitTiles ? SplitShape::S : WholeShape::S;
    *steps_in_flight = tiles <= kWideSplitTiles ? WideSplitShape::P : tiles <= kSplitTiles ? SplitShape::P
                                                                                          : WholeShape::P;
    return Q8G_OK;
}

extern "C" q8g_status q8g_batch_tiled_streams(int64_t N, int64_t K, int *streams)
{
    if (N < 0 || K < 0 || K % 32 || N > kMaxElems || K > kMaxK) return Q8G_ERR_SHAPE;
    if (!streams) return Q8G_ERR_NULL;
    *streams = stream_shape(N, K) ? 1 : 0;
    return Q8G_OK;
}
