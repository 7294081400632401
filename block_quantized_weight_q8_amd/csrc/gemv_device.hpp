// Device building blocks shared by the standalone GEMV kernels and the
// persistent decode-step kernel, so that both compute every output row with
// the same instructions in the same order (and therefore the same bits).
//
// Row layout per wave (wave64): a row is streamed in 1 KiB chunks; lane l owns
// bytes [16l, 16l+16) of every chunk. For Q8_0 a 32-byte block spans lanes 2j
// and 2j+1 ("Filling in the blanks: Inference using Phobos", section Fast
// Decode: a block of 32 int8 values carries its own scale; block products and
// sums stay in integers). For bf16 a lane's 16 bytes are eight values ("One
// level down: #002 the same compiler on a GPU", section Emitting for a GPU:
// rows read as 16-byte chunks of eight bf16).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q8g {

constexpr int kWave = 64;
constexpr int kChunk = 1024;  // bytes of one row covered by one wave-wide 16-byte load

typedef int v4i __attribute__((ext_vector_type(4)));

// ---- cross-lane exchange with the lane at xor distance D --------------------
// All in VALU lane-crossing forms, none through the LDS crossbar (ds_swizzle and
// ds_bpermute, which these replaced, each cost a round trip on the critical
// path of every reduction): DPP for 1, 2, 4 and 8, the gfx950 permlane swaps for
// 16 and 32. Every form was checked on the GPU against lane i ^ D.
template <int D>
__device__ __forceinline__ int xchg_int(int v)
{
    static_assert(D == 1 || D == 2 || D == 4 || D == 8, "xchg: xor distance 1, 2, 4 or 8");
    if constexpr (D == 1) {
        return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
    } else if constexpr (D == 2) {
        return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
    } else if constexpr (D == 4) {
        // row_half_mirror (lane 7 - i within 8), then quad_perm [3,2,1,0]: (i ^ 3) ^ 7 = i ^ 4
        const int m = __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);
        return __builtin_amdgcn_update_dpp(0, m, 0x1B, 0xF, 0xF, false);
    } else {
        return __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false);  // row_ror:8 = i ^ 8 in 16
    }
}

// the value of the lane at xor distance D (1, 2, 4 or 8)
template <int D>
__device__ __forceinline__ float xchg(float v)
{
    return __builtin_bit_cast(float, xchg_int<D>(__builtin_bit_cast(int, v)));
}

// {a, b} = {this lane's v, the v of the lane at xor distance D}, in an order that may
// differ between lanes, for combining with a commutative operation (a + b, max):
// at 16 and 32 a permlane swap of v with itself returns the two values, one per
// result (odd rows / the upper half take them in the other order), so no lane
// select is needed; a + b and max(a, b) have the same bits in both orders.
template <int D>
__device__ __forceinline__ void lane_pair(int v, int &a, int &b)
{
    if constexpr (D == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        a = (int)r[0];
        b = (int)r[1];
    } else if constexpr (D == 32) {
        const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        a = (int)r[0];
        b = (int)r[1];
    } else {
        a = v;
        b = xchg_int<D>(v);
    }
}

// v + (v of the lane at xor distance D), the same bits in both lanes
template <int D>
__device__ __forceinline__ float xsum(float v)
{
    int a, b;
    lane_pair<D>(__builtin_bit_cast(int, v), a, b);
    return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}

// max(v, v of the lane at xor distance D)
template <int D>
__device__ __forceinline__ float xmax(float v)
{
    int a, b;
    lane_pair<D>(__builtin_bit_cast(int, v), a, b);
    return fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}

// Keep half of v[0..CNT) (the upper half when `upper`), add the partner's copy
// of that half; the result is in v[0..CNT/2).
template <int D, int CNT>
__device__ __forceinline__ void halve(float *v, bool upper)
{
#pragma unroll
    for (int j = 0; j < CNT / 2; ++j) {
        const float keep = upper ? v[j + CNT / 2] : v[j];
        const float send = upper ? v[j] : v[j + CNT / 2];
        v[j] = keep + xchg<D>(send);
    }
}

// Sum R per-lane values over the wave (butterfly: while two or more rows remain
// per lane, each step keeps half of them and adds the partner's copy of that
// half). The tree always pairs lanes at distance 1, 2, 4, ..., 32, so a row's
// total does not depend on R or on the row's slot. Returns, in every lane, the
// total of row row_of<R>(lane).
template <int R>
__device__ __forceinline__ float wave_reduce_rows(float (&v)[R], int lane)
{
    static_assert(R == 1 || R == 2 || R == 4 || R == 8, "R must be 1, 2, 4 or 8");
    if constexpr (R >= 2) halve<1, R>(v, lane & 1);
    if constexpr (R >= 4) halve<2, R / 2>(v, lane & 2);
    if constexpr (R >= 8) halve<4, R / 4>(v, lane & 4);
    float s = v[0];
    if constexpr (R < 2) s = xsum<1>(s);
    if constexpr (R < 4) s = xsum<2>(s);
    if constexpr (R < 8) s = xsum<4>(s);
    s = xsum<8>(s);
    s = xsum<16>(s);
    s = xsum<32>(s);
    return s;
}

template <int R>
__device__ __forceinline__ int row_of(int lane)
{
    if constexpr (R == 1) return 0;
    if constexpr (R == 2) return lane & 1;
    if constexpr (R == 4) return ((lane & 1) << 1) | ((lane >> 1) & 1);
    return ((lane & 1) << 2) | (((lane >> 1) & 1) << 1) | ((lane >> 2) & 1);
}

// The first lane whose wave_reduce_rows<R> result is row i (row_of<R> is a bit
// reversal of the low lane bits, so it is its own inverse).
template <int R>
__device__ __forceinline__ constexpr int lane_of(int i)
{
    if constexpr (R == 1) return 0;
    if constexpr (R == 2) return i;
    if constexpr (R == 4) return ((i & 1) << 1) | ((i >> 1) & 1);
    return ((i & 1) << 2) | (((i >> 1) & 1) << 1) | ((i >> 2) & 1);
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

// Plain 16-byte load (data other waves reuse: the activation).
__device__ __forceinline__ int4 load16(const void *p) { return *reinterpret_cast<const int4 *>(p); }

// Streaming 16-byte load (weights: read once per call, so marked nontemporal).
__device__ __forceinline__ int4 load16_stream(const void *p)
{
    const v4i v = __builtin_nontemporal_load(reinterpret_cast<const v4i *>(p));
    return make_int4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint16_t load_u16_stream(const uint16_t *p) { return __builtin_nontemporal_load(p); }

// Q8_0: one lane's half block (16 codes) against the activation codes, joined
// with the partner lane into the block's exact int32 sum (in both lanes).
__device__ __forceinline__ int q8_block_sum(const int4 &w, const int4 &x)
{
    int s = __builtin_amdgcn_sdot4(w.x, x.x, 0, false);
    s = __builtin_amdgcn_sdot4(w.y, x.y, s, false);
    s = __builtin_amdgcn_sdot4(w.z, x.z, s, false);
    s = __builtin_amdgcn_sdot4(w.w, x.w, s, false);
    return s + xchg_int<1>(s);
}

// bf16: eight products of one lane's 16 bytes, summed into one chunk partial.
// bf16 -> f32 is exact: the low value is (word << 16), the high (word & ~0xFFFF).
__device__ __forceinline__ void bf16_unpack(const int4 &v, float (&f)[8])
{
    const uint32_t w[4] = {(uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __builtin_bit_cast(float, w[i] << 16);
        f[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xFFFF0000u);
    }
}

__device__ __forceinline__ float bf16_chunk_dot(const int4 &wv, const float (&xf)[8])
{
    const uint32_t ww[4] = {(uint32_t)wv.x, (uint32_t)wv.y, (uint32_t)wv.z, (uint32_t)wv.w};
    float part = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        part = __builtin_fmaf(__builtin_bit_cast(float, ww[i] << 16), xf[2 * i], part);
        part = __builtin_fmaf(__builtin_bit_cast(float, ww[i] & 0xFFFF0000u), xf[2 * i + 1], part);
    }
    return part;
}

// f16 ("One level down", The bench: the same engine in f16): eight binary16
// values per lane, converted exactly to f32; each product of two binary16
// values is exact in f32 (11 + 11 significant bits).
__device__ __forceinline__ void f16_unpack(const int4 &v, float (&f)[8])
{
    const uint32_t w[4] = {(uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = f16_bits_to_f32((uint16_t)(w[i] & 0xFFFFu));
        f[2 * i + 1] = f16_bits_to_f32((uint16_t)(w[i] >> 16));
    }
}

__device__ __forceinline__ float f16_chunk_dot(const int4 &wv, const float (&xf)[8])
{
    float wf[8];
    f16_unpack(wv, wf);
    float part = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) part = __builtin_fmaf(wf[i], xf[i], part);
    return part;
}

// Activation quantization of four consecutive values of one 32-value block
// held by an aligned group of 8 lanes ("Filling in the blanks", Fast Decode:
// quantize an activation once into the weights' block format):
//   d = fl32(max|x| / 127); q = rint(fl32(x / d)) (ties to even); d == 0 -> 0.
// Returns the four codes packed little-endian; *d_out receives d (f32).
__device__ __forceinline__ uint32_t quantize4(const float4 &v, float *d_out)
{
    float m = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    m = xmax<1>(m);
    m = xmax<2>(m);
    m = xmax<4>(m);
    const float d = m / 127.0f;  // correctly rounded f32 division
    *d_out = d;
    uint32_t packed = 0;
    if (d != 0.0f) {
        const float t[4] = {v.x / d, v.y / d, v.z / d, v.w / d};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float q = __builtin_rintf(t[i]);  // round half to even
            q = fminf(fmaxf(q, -127.0f), 127.0f);
            packed |= ((uint32_t)(uint8_t)(int8_t)(int)q) << (8 * i);
        }
    }
    return packed;
}

__device__ __forceinline__ uint16_t scale_bits(float d) { return d != 0.0f ? f32_to_f16_bits(d) : (uint16_t)0; }

// A barrier among the workgroup's waves that waits only for this wave's own LDS
// operations, not for its global loads in flight: gfx950 puts no wait in front of
// a bare s_barrier, and __syncthreads (a fence) would also wait for the weights a
// wave has requested ahead of use. The empty asm statements keep the compiler
// from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt 63 (no wait), expcnt 7 (no wait), lgkmcnt 0
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

}  // namespace q8g
