// Device-side helpers shared by the gfx950 kernels of libnq.
//
// Storage types: fp32 is `float`; bf16 is carried as its 16-bit pattern
// (`uint16_t`).  Every fp32 -> bf16 conversion rounds to nearest-even.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nqk {

typedef uint16_t bf16_bits;

__device__ __forceinline__ float bf16_to_f32(uint32_t h16) { return __uint_as_float(h16 << 16); }

// Round to nearest-even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

template <typename T> struct Elt;

template <> struct Elt<float> {
    static constexpr int bytes = 4;
    __device__ __forceinline__ static float load(const float *p, int64_t i) { return p[i]; }
    __device__ __forceinline__ static void store(float *p, int64_t i, float v) { p[i] = v; }
    // Value that `store` would keep.
    __device__ __forceinline__ static float stored(float v) { return v; }
};

template <> struct Elt<bf16_bits> {
    static constexpr int bytes = 2;
    __device__ __forceinline__ static float load(const bf16_bits *p, int64_t i)
    {
        return bf16_to_f32(p[i]);
    }
    __device__ __forceinline__ static void store(bf16_bits *p, int64_t i, float v)
    {
        p[i] = (bf16_bits)f32_to_bf16(v);
    }
    __device__ __forceinline__ static float stored(float v) { return bf16_to_f32(f32_to_bf16(v)); }
};

// Loads 32 consecutive elements starting at p (16-byte aligned) as fp32.
template <typename T> __device__ __forceinline__ void load32_f32(const T *p, float *v);

template <> __device__ __forceinline__ void load32_f32<float>(const float *p, float *v)
{
    const uint4 *q = reinterpret_cast<const uint4 *>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint4 d = q[i];
        v[4 * i + 0] = __uint_as_float(d.x);
        v[4 * i + 1] = __uint_as_float(d.y);
        v[4 * i + 2] = __uint_as_float(d.z);
        v[4 * i + 3] = __uint_as_float(d.w);
    }
}

template <> __device__ __forceinline__ void load32_f32<bf16_bits>(const bf16_bits *p, float *v)
{
    const uint4 *q = reinterpret_cast<const uint4 *>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint4 d = q[i];
        uint32_t w[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[8 * i + 2 * j + 0] = __uint_as_float(w[j] << 16);
            v[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
        }
    }
}

// Code j (0..31) of a 32-element lane chunk held in BITS words (LSB-first
// bit stream; codes of 3, 5 and 6 bits may straddle two words).
template <int BITS>
__device__ __forceinline__ uint32_t code_at(const uint32_t *w, int j)
{
    const int bit = j * BITS;
    const int wi = bit >> 5, sh = bit & 31;
    uint32_t q = w[wi] >> sh;
    if (sh + BITS > 32) q |= w[wi + 1] << (32 - sh);
    return q & ((1u << BITS) - 1u);
}

// v from lane (lane ^ OFF) of the wave, without the LDS pipe: DPP quad
// permutes for 1 and 2, DPP row rotations for 4 and 8 (a rotation by 8
// inside a 16-lane row is the xor; for 4 the lanes pick a rotation by 4 or
// by 12), gfx950's v_permlane16_swap / v_permlane32_swap for 16 and 32.
// A swap of a register with itself leaves, in the first result, the lower
// row (half) of each pair twice and, in the second, the upper one twice.
template <int OFF>
__device__ __forceinline__ float xor_lane(float v, int lane)
{
    const int iv = __float_as_int(v);
    int r;
    if constexpr (OFF == 1) r = __builtin_amdgcn_mov_dpp(iv, 0xB1, 0xF, 0xF, true);   // [1,0,3,2]
    else if constexpr (OFF == 2) r = __builtin_amdgcn_mov_dpp(iv, 0x4E, 0xF, 0xF, true);  // [2,3,0,1]
    else if constexpr (OFF == 4) {
        const int a = __builtin_amdgcn_update_dpp(0, iv, 0x124, 0xF, 0xF, false);   // row_ror:4
        const int b = __builtin_amdgcn_update_dpp(0, iv, 0x12C, 0xF, 0xF, false);   // row_ror:12
        r = (lane & 4) ? a : b;
    } else if constexpr (OFF == 8) {
        r = __builtin_amdgcn_update_dpp(0, iv, 0x128, 0xF, 0xF, false);             // row_ror:8
    } else if constexpr (OFF == 16) {
        const auto s = __builtin_amdgcn_permlane16_swap(iv, iv, false, false);
        r = (lane & 16) ? (int)s[0] : (int)s[1];
    } else {
        static_assert(OFF == 32, "lane exchange distance");
        const auto s = __builtin_amdgcn_permlane32_swap(iv, iv, false, false);
        r = (lane & 32) ? (int)s[0] : (int)s[1];
    }
    return __int_as_float(r);
}

// One step (distance OFF = 16 or 32) of a transposed lane reduction: lanes
// without bit OFF keep a and add it from lane ^ OFF, lanes with it keep b and
// add it from lane ^ OFF -- one swap of the two registers.  The sum of each
// lane's pair is the same as keep + partner (addition commutes).
template <int OFF>
__device__ __forceinline__ float swap_sum(float a, float b)
{
    static_assert(OFF == 16 || OFF == 32, "swap distance");
    const auto s = OFF == 32 ? __builtin_amdgcn_permlane32_swap(__float_as_int(a), __float_as_int(b), false, false)
                             : __builtin_amdgcn_permlane16_swap(__float_as_int(a), __float_as_int(b), false, false);
    return __int_as_float((int)s[0]) + __int_as_float((int)s[1]);
}

__device__ __forceinline__ float pick(bool c, float a, float b)
{
    // c ? a : b, written with integer masks so that it stays a register select
    const int m = -(int)c;
    return __int_as_float((__float_as_int(a) & m) | (__float_as_int(b) & ~m));
}


}  // namespace nqk
