// Floating-point quantization modes on gfx950: MXFP4, MXFP8 and NVFP4.
//
// Method: "Quantization" page of the nuvec documentation, section
// "Floating-point formats" (every weight a small float, one uint8 scale
// code per group, no biases; dequantize gives bf16; a product comes out in
// x's dtype) and section "Mixture of experts" (an NVFP4 expert may carry one
// fp32 global scale).  The encodings are the public format definitions:
// OCP Microscaling Formats v1.0 -- blocks of 32 elements sharing an E8M0
// scale 2^(s - 127) (s = 255: NaN), elements FP4 E2M1 or FP8 E4M3 -- and
// NVFP4 -- blocks of 16 E2M1 elements sharing an E4M3 scale.  Codes are
// packed LSB-first into uint32 words like the affine codes.
//
// Every kernel takes 32-element chunks: one MX block, or two NVFP4 blocks.
//   quantize    MX: s = clamp(biased exponent of max|w| - emax, 0, 254)
//               (emax 2 for E2M1, 8 for E4M3; an all-zero block gets 0),
//               element = round(ldexp(w, 127 - s)).  NVFP4: s =
//               e4m3(fp32(max|w| / 6)), element = round(fp32(w / S)) with S
//               the decoded scale (zero codes when S is 0).  round: nearest
//               value, ties to the even code, saturating at the largest
//               magnitude, sign kept.
//   dequantize  S * E in fp32 (exact), rounded to bf16 (NaN -> 0x7fc0) or
//               kept in fp32.
//   products    the hardware conversions v_cvt_scalef32_pk_{bf16,f32}_{fp4,fp8}
//               with scale 1 (exact) turn elements into bf16 or fp32 pairs;
//               the matrix-vector kernel dots them with x per group and
//               scales each group sum in fp32, the tiled kernels write
//               bf16(S * E) tiles to LDS for bf16 MFMA (MX modes: the same
//               conversions with the power-of-two scale S give bf16(S * E)
//               in one instruction per pair).  A global scale multiplies the
//               fp32 result.
#include <algorithm>
#include <type_traits>

#include "nq_device.h"
#include "nq_internal.h"
#include "nq_tiles.h"

namespace nqk {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

template <int MODE> struct Fp;
template <> struct Fp<FP_MXFP4> {
    static constexpr int bits = 4, gs = 32, emax = 2;
    static constexpr bool fp8 = false, e8m0 = true;
};
template <> struct Fp<FP_MXFP8> {
    static constexpr int bits = 8, gs = 32, emax = 8;
    static constexpr bool fp8 = true, e8m0 = true;
};
template <> struct Fp<FP_NVFP4> {
    static constexpr int bits = 4, gs = 16, emax = 2;
    static constexpr bool fp8 = false, e8m0 = false;
};

constexpr uint32_t kQuietNan = 0x7fc00000u;

// ---------------------------------------------------------------- decoding
// E2M1: sign bit 3, exponent bits 2:1 (bias 1), mantissa bit 0; exponent 0
// is subnormal (m * 0.5).
__device__ __forceinline__ float e2m1_value(uint32_t c)
{
    const uint32_t mag = c & 7u;
    const uint32_t b = mag >= 2u ? (((mag >> 1) + 126u) << 23) | ((mag & 1u) << 22)
                                 : (mag ? 0x3f000000u : 0u);
    return __uint_as_float(b | ((c & 8u) << 28));
}

// E4M3 (OCP): sign bit 7, exponent bits 6:3 (bias 7), mantissa bits 2:0;
// exponent 0 is subnormal (m * 2^-9); S.1111.111 is NaN.
// Both magnitudes are formed and selected, and the sign is or-ed in, so
// that the conversion is straight-line code (no branch around the NaN or
// subnormal cases inside the kernels' loops).
__device__ __forceinline__ float e4m3_value(uint32_t c)
{
    const uint32_t e = (c >> 3) & 15u, m = c & 7u;
    const float normal = __uint_as_float(((e + 120u) << 23) | (m << 20));
    const float subnormal = (float)m * 0x1p-9f;
    const float mag = e ? normal : subnormal;
    const float v = __uint_as_float(__float_as_uint(mag) | ((c & 0x80u) << 24));
    return (c & 0x7fu) == 0x7fu ? __uint_as_float(kQuietNan) : v;
}

// E8M0: 2^(s - 127); s = 0 is the fp32 subnormal 2^-127; s = 255 is NaN.
__device__ __forceinline__ float e8m0_value(uint32_t s)
{
    return __uint_as_float(s == 255u ? kQuietNan : s == 0u ? 0x00400000u : s << 23);
}

template <int MODE>
__device__ __forceinline__ float scale_value(uint32_t s)
{
    return Fp<MODE>::e8m0 ? e8m0_value(s) : e4m3_value(s);
}

template <int MODE>
__device__ __forceinline__ float elem_value(uint32_t c)
{
    return Fp<MODE>::fp8 ? e4m3_value(c) : e2m1_value(c);
}

// ---------------------------------------------------------------- encoding
// Nearest E2M1 value, ties to the even code, saturating at 6: the code is
// the number of decision points below |v| (strict where the tie goes down).
__device__ __forceinline__ uint32_t e2m1_code(float v)
{
    const float a = fabsf(v);
    const uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                       (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                       (uint32_t)(a > 5.0f);
    return c | ((__float_as_uint(v) >> 28) & 8u);
}

// Nearest E4M3 value, ties to the even code, saturating at 448.  Below 2^-6
// the spacing is 2^-9 (codes 0..8); above, the fp32 mantissa is rounded to 3
// bits (a carry moves into the exponent) and the exponent rebased.
__device__ __forceinline__ uint32_t e4m3_code(float v)
{
    const float a = fabsf(v);
    uint32_t c;
    if (a < 0x1p-6f) {
        c = (uint32_t)rintf(a * 512.0f);
    } else {
        uint32_t u = __float_as_uint(a);
        u += 0x7ffffu + ((u >> 20) & 1u);
        c = min((u >> 20) - (120u << 3), 0x7eu);
    }
    return c | ((__float_as_uint(v) >> 24) & 0x80u);
}

template <int MODE>
__device__ __forceinline__ uint32_t elem_code(float v)
{
    return Fp<MODE>::fp8 ? e4m3_code(v) : e2m1_code(v);
}

// ---------------------------------------------------------------- element pairs
// Elements 2p and 2p + 1 of a chunk's code words as bf16 or fp32 pairs (the
// scaled conversions with scale 1: exact for these formats).
template <int MODE>
__device__ __forceinline__ bf16x2_t pair_bf16(const uint32_t *wd, int p)
{
    if constexpr (Fp<MODE>::fp8) {
        const uint32_t w = wd[p >> 1];
        return (p & 1) ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)
                       : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
    } else {
        const uint32_t w = wd[p >> 2];
        switch (p & 3) {   // the byte select is an immediate
        case 0: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0);
        case 1: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1);
        case 2: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2);
        default: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3);
        }
    }
}

// Elements 2p and 2p + 1 times a power-of-two scale S, as bf16 pairs, by the
// scaled conversions (exact: a power of two times an E2M1 or E4M3 value).
template <int MODE>
__device__ __forceinline__ bf16x2_t pair_bf16_scaled(const uint32_t *wd, int p, float S)
{
    if constexpr (Fp<MODE>::fp8) {
        const uint32_t w = wd[p >> 1];
        return (p & 1) ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, S, true)
                       : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, S, false);
    } else {
        const uint32_t w = wd[p >> 2];
        switch (p & 3) {
        case 0: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, S, 0);
        case 1: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, S, 1);
        case 2: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, S, 2);
        default: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, S, 3);
        }
    }
}

template <int MODE>
__device__ __forceinline__ f32x2_t pair_f32(const uint32_t *wd, int p)
{
    if constexpr (Fp<MODE>::fp8) {
        const uint32_t w = wd[p >> 1];
        return (p & 1) ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, true)
                       : __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, false);
    } else {
        const uint32_t w = wd[p >> 2];
        switch (p & 3) {
        case 0: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
        case 1: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
        case 2: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
        default: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
        }
    }
}

// ---------------------------------------------------------------- quantize
template <int MODE, typename WT>
__global__ void __launch_bounds__(256) fp_quantize_kernel(const WT *__restrict__ w, int64_t chunks,
                                                          uint32_t *__restrict__ codes,
                                                          uint8_t *__restrict__ scales)
{
    constexpr int BITS = Fp<MODE>::bits, GS = Fp<MODE>::gs, NG = 32 / GS;
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= chunks) return;
    float v[32];
    load32_f32<WT>(w + c * 32, v);
    uint32_t q[32];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < GS; ++j) amax = fmaxf(amax, fabsf(v[g * GS + j]));
        uint32_t s;
        if constexpr (Fp<MODE>::e8m0) {
            s = (uint32_t)min(max((int)(__float_as_uint(amax) >> 23) - Fp<MODE>::emax, 0), 254);
            const int sh = 127 - (int)s;
#pragma unroll
            for (int j = 0; j < GS; ++j) q[g * GS + j] = elem_code<MODE>(ldexpf(v[g * GS + j], sh));
        } else {
            s = e4m3_code(amax / 6.0f);
            const float S = e4m3_value(s);
#pragma unroll
            for (int j = 0; j < GS; ++j) q[g * GS + j] = S == 0.0f ? 0u : e2m1_code(v[g * GS + j] / S);
        }
        scales[c * NG + g] = (uint8_t)s;
    }
    uint32_t wd[BITS];
#pragma unroll
    for (int i = 0; i < BITS; ++i) wd[i] = 0u;
#pragma unroll
    for (int j = 0; j < 32; ++j) wd[j * BITS / 32] |= q[j] << ((j * BITS) % 32);
    uint4 *dst = reinterpret_cast<uint4 *>(codes + c * BITS);
#pragma unroll
    for (int i = 0; i < BITS / 4; ++i) dst[i] = make_uint4(wd[4 * i], wd[4 * i + 1], wd[4 * i + 2], wd[4 * i + 3]);
}

// ---------------------------------------------------------------- dequantize
// A wave's 64 chunks are one contiguous run of the output: each lane puts
// its piece (64 or 128 bytes) into LDS and the wave stores the run with
// every instruction writing 1 KB contiguous.  Lane pieces sit 16 bytes
// apart beyond their length (stride P + 1 uint4), which keeps the 16-byte
// writes of 16 lanes on distinct banks.
template <int MODE, typename OT>
__global__ void __launch_bounds__(256) fp_dequantize_kernel(const uint32_t *__restrict__ codes,
                                                            const uint8_t *__restrict__ scales,
                                                            int64_t chunks, OT *__restrict__ out)
{
    constexpr int BITS = Fp<MODE>::bits, GS = Fp<MODE>::gs, NG = 32 / GS;
    constexpr int P = 32 * (int)sizeof(OT) / 16;   // uint4 pieces per lane
    __shared__ uint4 stage[4][64 * (P + 1)];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t cw = ((int64_t)blockIdx.x * 4 + wave) * 64;   // the wave's first chunk
    if (cw >= chunks) return;
    const int64_t c = min(cw + lane, chunks - 1);
    uint32_t wd[BITS];
    const uint4 *src = reinterpret_cast<const uint4 *>(codes + c * BITS);
#pragma unroll
    for (int i = 0; i < BITS / 4; ++i) {
        const uint4 t = src[i];
        wd[4 * i] = t.x, wd[4 * i + 1] = t.y, wd[4 * i + 2] = t.z, wd[4 * i + 3] = t.w;
    }
    // S * E in fp32 (exact) from the hardware pair conversion; a NaN scale
    // makes its whole group NaN, a NaN element (E4M3 only) its own value;
    // every NaN leaves as the canonical quiet NaN
    float o[32];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        const float S = scale_value<MODE>(scales[c * NG + g]);
        const bool snan = S != S;
#pragma unroll
        for (int q = 0; q < GS / 2; ++q) {
            const int pi = g * (GS / 2) + q;
            const f32x2_t e = pair_f32<MODE>(wd, pi);
            float v0 = S * e[0], v1 = S * e[1];
            if constexpr (Fp<MODE>::fp8) {
                v0 = v0 != v0 ? __uint_as_float(kQuietNan) : v0;
                v1 = v1 != v1 ? __uint_as_float(kQuietNan) : v1;
            }
            o[2 * pi] = snan ? __uint_as_float(kQuietNan) : v0;
            o[2 * pi + 1] = snan ? __uint_as_float(kQuietNan) : v1;
        }
    }
    uint4 *st = stage[wave];
    if constexpr (std::is_same<OT, float>::value) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            st[lane * (P + 1) + i] = make_uint4(__float_as_uint(o[4 * i]), __float_as_uint(o[4 * i + 1]),
                                                __float_as_uint(o[4 * i + 2]), __float_as_uint(o[4 * i + 3]));
    } else {
        // hardware round-to-nearest-even packing (the canonical NaN stays 0x7fc0)
        uint32_t h[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const f32x2_t v = {o[2 * i], o[2 * i + 1]};
            h[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
            st[lane * (P + 1) + i] = make_uint4(h[4 * i], h[4 * i + 1], h[4 * i + 2], h[4 * i + 3]);
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // store instruction u writes uint4 j = 64 u + lane of the wave's run
    const int64_t valid = min((int64_t)64, chunks - cw) * P;   // uint4 of the run inside the output
    uint4 *dst = reinterpret_cast<uint4 *>(out + cw * 32);
#pragma unroll
    for (int u = 0; u < P; ++u) {
        const int j = 64 * u + lane;
        if (j < valid) dst[j] = st[(j / P) * (P + 1) + j % P];
    }
}

// ---------------------------------------------------------------- matrix-vector
// A wave owns RW consecutive weight rows and MR activation vectors; lane L
// takes the 32-element chunks L, L + 64, ... of K.  Per chunk and group it
// forms the dot product of the group's elements with x (bf16 pairs through
// v_dot2_f32_bf16, or fp32 fused multiply-adds, in element order), then adds
// scale * sum to its running sum; the 64 lanes' sums are added by a xor
// butterfly.  A vector's arithmetic is the same for any MR, RW or launch
// chunk, so every row equals its one-row product bit for bit.
struct FpGemvParams {
    const void *x;
    void *y;
    const uint32_t *codes;
    const uint8_t *scales;
    const float *gscale;     // per expert (or the only matrix); null: 1
    const uint32_t *idx;     // expert of each item; null: one weight matrix
    int64_t vpi, cpi;        // vectors per item, MR-chunks per item
    int64_t n, k, e;
    int64_t y0;              // first (item, chunk) index of this launch
    // grouped gather: workgroup row c runs chunk c of the table built by the
    // grouping pass (uint4 {expert, first, count, 0} over perm); chunks past
    // *nchunks do nothing
    const uint4 *chunks;
    const uint32_t *perm, *nchunks;
};

__device__ __forceinline__ float wave_sum(float v, int lane)
{
    v = swap_sum<32>(v, v);
    v = swap_sum<16>(v, v);
    v += xor_lane<8>(v, lane);
    v += xor_lane<4>(v, lane);
    v += xor_lane<2>(v, lane);
    v += xor_lane<1>(v, lane);
    return v;
}

template <int MODE, typename XT, int MR, int RW>
__global__ void __launch_bounds__(256) fp_gemv_kernel(FpGemvParams p)
{
    constexpr int BITS = Fp<MODE>::bits, GS = Fp<MODE>::gs, NG = 32 / GS;
    constexpr bool kBf16 = std::is_same<XT, bf16_bits>::value;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t yb = p.y0 + blockIdx.y;
    const int64_t row0 = ((int64_t)blockIdx.x * 4 + wave) * RW;
    if (row0 >= p.n) return;
    // the chunk's vectors (rows of x and y) and their expert
    int64_t vec[MR];
    int mr;
    uint32_t ex;
    if (p.chunks) {
        if (yb >= *p.nchunks) return;   // uniform over the workgroup
        const uint4 ch = p.chunks[yb];
        ex = ch.x, mr = (int)ch.z;
#pragma unroll
        for (int i = 0; i < MR; ++i) vec[i] = p.perm[ch.y + min(i, mr - 1)];
    } else {
        const int64_t item = yb / p.cpi, v0 = (yb % p.cpi) * MR;
        mr = (int)min((int64_t)MR, p.vpi - v0);
        ex = p.idx ? p.idx[item] : 0u;
#pragma unroll
        for (int i = 0; i < MR; ++i) vec[i] = item * p.vpi + v0 + min(i, mr - 1);
    }
    XT *y = reinterpret_cast<XT *>(p.y);
    if ((int64_t)ex >= p.e) {   // no such expert: zero rows
        if (lane < RW && row0 + lane < p.n)
            for (int i = 0; i < mr; ++i) Elt<XT>::store(y, vec[i] * p.n + row0 + lane, 0.0f);
        return;
    }
    const int64_t wpr = p.k * BITS / 32, gpr = p.k / GS, chunks = p.k / 32;
    const uint32_t *codes = p.codes + (int64_t)ex * p.n * wpr;
    const uint8_t *scales = p.scales + (int64_t)ex * p.n * gpr;
    const XT *x = reinterpret_cast<const XT *>(p.x);

    float acc[MR][RW];
#pragma unroll
    for (int i = 0; i < MR; ++i)
#pragma unroll
        for (int r = 0; r < RW; ++r) acc[i][r] = 0.0f;

    // U chunks per pass (their loads issued together); a lane still adds its
    // chunks in increasing order
    constexpr int U = 2;
    for (int64_t c0 = lane; c0 < chunks; c0 += 64 * U) {
        uint32_t wd[U][RW][BITS];
        uint32_t sc[U][RW][NG];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t c = c0 + 64 * u < chunks ? c0 + 64 * u : c0;
#pragma unroll
            for (int r = 0; r < RW; ++r) {
                const int64_t row = min(row0 + r, p.n - 1);
                const uint4 *src = reinterpret_cast<const uint4 *>(codes + row * wpr + c * BITS);
#pragma unroll
                for (int i = 0; i < BITS / 4; ++i) {
                    const uint4 t = src[i];
                    wd[u][r][4 * i] = t.x, wd[u][r][4 * i + 1] = t.y, wd[u][r][4 * i + 2] = t.z,
                    wd[u][r][4 * i + 3] = t.w;
                }
#pragma unroll
                for (int g = 0; g < NG; ++g) sc[u][r][g] = scales[row * gpr + c * NG + g];
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
        const int64_t c = c0 + 64 * u;
        if (c >= chunks) break;
#pragma unroll
        for (int i = 0; i < MR; ++i) {
            const XT *xr = x + vec[i] * p.k + c * 32;
            uint32_t xw[kBf16 ? 16 : 32];
            const uint4 *xs = reinterpret_cast<const uint4 *>(xr);
#pragma unroll
            for (int t = 0; t < (kBf16 ? 4 : 8); ++t) {
                const uint4 u = xs[t];
                xw[4 * t] = u.x, xw[4 * t + 1] = u.y, xw[4 * t + 2] = u.z, xw[4 * t + 3] = u.w;
            }
#pragma unroll
            for (int r = 0; r < RW; ++r)
#pragma unroll
                for (int g = 0; g < NG; ++g) {
                    float s = 0.0f;
#pragma unroll
                    for (int q = 0; q < GS / 2; ++q) {
                        const int pi = g * (GS / 2) + q;   // element pair of the chunk
                        if constexpr (kBf16) {
                            s = __builtin_amdgcn_fdot2_f32_bf16(pair_bf16<MODE>(wd[u][r], pi),
                                                                __builtin_bit_cast(bf16x2_t, xw[pi]), s, false);
                        } else {
                            const f32x2_t e = pair_f32<MODE>(wd[u][r], pi);
                            s = fmaf(__uint_as_float(xw[2 * pi]), e[0], s);
                            s = fmaf(__uint_as_float(xw[2 * pi + 1]), e[1], s);
                        }
                    }
                    acc[i][r] = fmaf(scale_value<MODE>(sc[u][r][g]), s, acc[i][r]);
                }
        }
        }
    }
    const float gsc = p.gscale ? p.gscale[ex] : 1.0f;
#pragma unroll
    for (int i = 0; i < MR; ++i)
#pragma unroll
        for (int r = 0; r < RW; ++r) {
            const float t = wave_sum(acc[i][r], lane);
            if (lane == 0 && i < mr && row0 + r < p.n) Elt<XT>::store(y, vec[i] * p.n + row0 + r, t * gsc);
        }
}

// One bf16 activation row (decode), K at most 64 U lane chunks: persistent
// waves.  Lane L keeps its x chunks L + 64 u in registers; wave w of W takes
// the weight rows w, w + W, ... and issues the next row's code and scale
// loads before the current row's arithmetic.  Per row the arithmetic is
// fp_gemv_kernel's (chunks in increasing order, the same dot products,
// scaling and butterfly), so the bits are the same.
template <int MODE, int U>
__global__ void __launch_bounds__(256) fp_gemv_stream_kernel(FpGemvParams p)
{
    constexpr int BITS = Fp<MODE>::bits, GS = Fp<MODE>::gs, NG = 32 / GS;
    // x goes through LDS once per workgroup (16-byte pieces), then each
    // lane keeps its chunks in registers; the first row's loads are issued
    // before, so that their latency covers the staging
    __shared__ uint4 xl[64 * U * 4];
    const int lane = threadIdx.x & 63;
    const int64_t W = (int64_t)gridDim.x * 4;
    int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t wpr = p.k * BITS / 32, gpr = p.k / GS, chunks = p.k / 32;
    struct RowLd {
        uint32_t wd[U][BITS];
        uint32_t sc[U][NG];
    };
    auto load = [&](int64_t r, RowLd &l) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t c = min((int64_t)lane + 64 * u, chunks - 1);
            const uint4 *src = reinterpret_cast<const uint4 *>(p.codes + r * wpr + c * BITS);
#pragma unroll
            for (int i = 0; i < BITS / 4; ++i) {
                const uint4 t = src[i];
                l.wd[u][4 * i] = t.x, l.wd[u][4 * i + 1] = t.y, l.wd[u][4 * i + 2] = t.z, l.wd[u][4 * i + 3] = t.w;
            }
#pragma unroll
            for (int g = 0; g < NG; ++g) l.sc[u][g] = p.scales[r * gpr + c * NG + g];
        }
    };
    const float gsc = p.gscale ? p.gscale[0] : 1.0f;
    bf16_bits *y = static_cast<bf16_bits *>(p.y);
    // The next row's loads are unconditional (past the last row they re-read
    // it), so the loop is straight-line and the wait before a row's
    // arithmetic leaves the next row's loads in flight.  Results wait in
    // lane j (iteration j mod 64) and are stored 64 at a time, so no store
    // sits between a row's loads and their wait.
    RowLd cur, nxt;
    load(min(row, p.n - 1), cur);
    const uint4 *xg = static_cast<const uint4 *>(p.x);
    for (int i = threadIdx.x; i < (int)chunks * 4; i += 256) xl[i] = xg[i];
    __syncthreads();
    if (row >= p.n) return;
    uint32_t xw[U][16];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int c = (int)min((int64_t)lane + 64 * u, chunks - 1);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint4 v = xl[c * 4 + t];
            xw[u][4 * t] = v.x, xw[u][4 * t + 1] = v.y, xw[u][4 * t + 2] = v.z, xw[u][4 * t + 3] = v.w;
        }
    }
    const int64_t row0 = row;
    float res = 0.0f;
    for (int j = 0; row < p.n; row += W, ++j) {
        load(min(row + W, p.n - 1), nxt);
        float acc = 0.0f;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if ((int64_t)lane + 64 * u >= chunks) break;
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                float s = 0.0f;
#pragma unroll
                for (int q = 0; q < GS / 2; ++q) {
                    const int pi = g * (GS / 2) + q;
                    s = __builtin_amdgcn_fdot2_f32_bf16(pair_bf16<MODE>(cur.wd[u], pi),
                                                        __builtin_bit_cast(bf16x2_t, xw[u][pi]), s, false);
                }
                acc = fmaf(scale_value<MODE>(cur.sc[u][g]), s, acc);
            }
        }
        const float t = wave_sum(acc, lane) * gsc;
        res = lane == (j & 63) ? t : res;
        if ((j & 63) == 63 || row + W >= p.n) {   // uniform over the wave
            const int64_t r = row0 + ((int64_t)(j & ~63) + lane) * W;
            if (lane <= (j & 63)) Elt<bf16_bits>::store(y, r, res);
        }
        cur = nxt;
    }
}

// Sum of V values over the 64 lanes, every value through the same pairwise
// tree as wave_sum (xor 32, 16, ..., 1; own value plus the partner's): at
// each step a lane keeps half of its values and sends the other half.
// Afterwards lane L holds value L >> (6 - log2 V).
template <int V, int OFF = 32>
__device__ __forceinline__ float wave_sum_many(float (&v)[V], int lane)
{
    if constexpr (OFF == 0) {
        return v[0];
    } else if constexpr (V > 1) {
        const bool upper = (lane & OFF) != 0;
        float h[V / 2];
#pragma unroll
        for (int i = 0; i < V / 2; ++i) {
            if constexpr (OFF >= 16) {
                h[i] = swap_sum<OFF>(v[i], v[i + V / 2]);
            } else {
                const float send = pick(upper, v[i], v[i + V / 2]);
                const float keep = pick(upper, v[i + V / 2], v[i]);
                h[i] = keep + xor_lane<OFF>(send, lane);
            }
        }
        return wave_sum_many<V / 2, OFF / 2>(h, lane);
    } else {
        float one[1];
        if constexpr (OFF >= 16) one[0] = swap_sum<OFF>(v[0], v[0]);
        else one[0] = v[0] + xor_lane<OFF>(v[0], lane);
        return wave_sum_many<1, OFF / 2>(one, lane);
    }
}

// Grouped gather, bf16 x, K = 2048 (one lane chunk per lane): workgroup row
// c runs chunk c of the grouping table (up to 8 vectors of one expert).
// Each wave keeps the chunk's 8 activation chunks in registers and streams
// weight rows w, w + W, ... of the expert (the next row's loads issued
// before the current row's arithmetic); the 8 sums of a row go through
// wave_sum_many, and lane L keeps (vector L / 8, row slot L % 8) so that
// eight rows leave in one store instruction.  Per vector the arithmetic is
// fp_gemv_kernel's, so every row keeps its one-row bits.
template <int MODE>
__global__ void __launch_bounds__(256) fp_gather_stream_kernel(FpGemvParams p)
{
    constexpr int BITS = Fp<MODE>::bits, GS = Fp<MODE>::gs, NG = 32 / GS, MR = 8;
    __shared__ uint4 xl[MR * 256];   // the chunk's 8 activation rows (2048 bf16 each)
    const int lane = threadIdx.x & 63;
    const int64_t cidx = blockIdx.y;
    if (cidx >= *p.nchunks) return;   // uniform over the workgroup
    const uint4 ch = p.chunks[cidx];
    const uint32_t ex = ch.x;
    const int cnt = max((int)ch.z, 1);   // chunks hold at least one vector
    const int64_t W = (int64_t)gridDim.x * 4;
    int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const bool live = (int64_t)ex < p.e;               // ex >= e: zero rows
    const int64_t wpr = p.k * BITS / 32, gpr = p.k / GS;
    const uint32_t *codes = p.codes + (int64_t)(live ? ex : 0u) * p.n * wpr;
    const uint8_t *scales = p.scales + (int64_t)(live ? ex : 0u) * p.n * gpr;
    struct RowLd {
        uint32_t wd[BITS];
        uint32_t sc[NG];
    };
    auto load = [&](int64_t r, RowLd &l) {
        const uint4 *src = reinterpret_cast<const uint4 *>(codes + r * wpr + lane * BITS);
#pragma unroll
        for (int i = 0; i < BITS / 4; ++i) {
            const uint4 t = src[i];
            l.wd[4 * i] = t.x, l.wd[4 * i + 1] = t.y, l.wd[4 * i + 2] = t.z, l.wd[4 * i + 3] = t.w;
        }
#pragma unroll
        for (int g = 0; g < NG; ++g) l.sc[g] = scales[r * gpr + lane * NG + g];
    };
    // the first row's loads go out before the activation staging, whose
    // latency they cover
    RowLd cur, nxt;
    if (live) load(min(row, p.n - 1), cur);
    {
        // x rows of the chunk through LDS, once per workgroup
        const bf16_bits *xg = static_cast<const bf16_bits *>(p.x);
        for (int t = threadIdx.x; t < MR * 256; t += 256) {
            const int i = t >> 8;
            xl[t] = reinterpret_cast<const uint4 *>(xg + (int64_t)p.perm[ch.y + min(i, cnt - 1)] * 2048)[t & 255];
        }
        __syncthreads();
    }
    if (row >= p.n) return;
    bf16_bits *y = static_cast<bf16_bits *>(p.y);
    const int myv = lane >> 3;                         // the vector this lane stores
    const int64_t yrow = (int64_t)p.perm[ch.y + min(myv, cnt - 1)];
    if (!live) {
        for (int64_t r = row + (lane & 7) * W; r < p.n; r += 8 * W)
            if (myv < cnt) Elt<bf16_bits>::store(y, yrow * p.n + r, 0.0f);
        return;
    }
    uint32_t xw[MR][16];
#pragma unroll
    for (int i = 0; i < MR; ++i) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint4 v = xl[i * 256 + lane * 4 + t];
            xw[i][4 * t] = v.x, xw[i][4 * t + 1] = v.y, xw[i][4 * t + 2] = v.z, xw[i][4 * t + 3] = v.w;
        }
    }
    const float gsc = p.gscale ? p.gscale[ex] : 1.0f;
    const int64_t row0 = row;
    float res = 0.0f;
    for (int j = 0; row < p.n; row += W, ++j) {
        load(min(row + W, p.n - 1), nxt);
        float acc[MR];
#pragma unroll
        for (int i = 0; i < MR; ++i) acc[i] = 0.0f;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const float S = scale_value<MODE>(cur.sc[g]);
            float sg[MR];
#pragma unroll
            for (int i = 0; i < MR; ++i) sg[i] = 0.0f;
#pragma unroll
            for (int q = 0; q < GS / 2; ++q) {
                const int pi = g * (GS / 2) + q;
                const bf16x2_t e = pair_bf16<MODE>(cur.wd, pi);
#pragma unroll
                for (int i = 0; i < MR; ++i)
                    sg[i] = __builtin_amdgcn_fdot2_f32_bf16(e, __builtin_bit_cast(bf16x2_t, xw[i][pi]), sg[i], false);
            }
#pragma unroll
            for (int i = 0; i < MR; ++i) acc[i] = fmaf(S, sg[i], acc[i]);
        }
        const float t = wave_sum_many<MR>(acc, lane) * gsc;   // lane L: vector L / 8
        res = (lane & 7) == (j & 7) ? t : res;
        if ((j & 7) == 7 || row + W >= p.n) {              // uniform over the wave
            const int64_t r = row0 + (int64_t)((j & ~7) + (lane & 7)) * W;
            if ((lane & 7) <= (j & 7) && myv < cnt) Elt<bf16_bits>::store(y, yrow * p.n + r, res);
        }
        cur = nxt;
    }
}

// ---------------------------------------------------------------- tiled (bf16 MFMA)
constexpr int kFpLdG = 72;   // LDS row stride (elements) of the gather tiles

// Grouped gather on matrix cores (bf16 x, K a multiple of 64): workgroup
// (b, c) multiplies chunk c of the grouping table (up to 32 activation
// vectors of one expert, gathered through perm) by the expert's weight rows
// [128 b, 128 b + 128).  Per K step of 64 the 32 x rows and the 128 weight
// rows (as bf16(S * E), exact) are staged in LDS -- thread t stages 8
// elements of x row t / 8 and 32 weights of row t / 2 -- and wave w runs
// one 32 x 32 block (its 32 weight rows) with v_mfma_f32_32x32x16_bf16; the
// next step's loads are issued before the MFMAs.  Each weight tile is
// converted once for all the chunk's vectors.
template <int MODE, int NW>
__global__ void __launch_bounds__(64 * NW) fp_gather_mfma_kernel(FpGemvParams p)
{
    constexpr int BITS = Fp<MODE>::bits, GS = Fp<MODE>::gs, NG = 32 / GS;
    constexpr int TN = 32 * NW, NT = 64 * NW, XP = (256 + NT - 1) / NT;   // weight rows, threads, x pieces a thread
    __shared__ __attribute__((aligned(16))) bf16_bits xs[32 * kFpLdG];
    __shared__ __attribute__((aligned(16))) bf16_bits ws[TN * kFpLdG];
    const int64_t cidx = blockIdx.y;
    if (cidx >= *p.nchunks) return;   // uniform over the workgroup
    const uint4 ch = p.chunks[cidx];
    const uint32_t ex = ch.x;
    const int cnt = max((int)ch.z, 1);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t n0 = (int64_t)blockIdx.x * TN;
    bf16_bits *y = static_cast<bf16_bits *>(p.y);
    if ((int64_t)ex >= p.e) {   // no such expert: zero rows
        for (int t = tid; t < 32 * TN; t += NT) {
            const int i = t / TN;
            const int64_t col = n0 + t % TN;
            if (i < (int)ch.z && col < p.n) y[(int64_t)p.perm[ch.y + i] * p.n + col] = 0;
        }
        return;
    }
    const int64_t wpr = p.k * BITS / 32, gpr = p.k / GS;
    const uint32_t *codes = p.codes + (int64_t)ex * p.n * wpr;
    const uint8_t *scales = p.scales + (int64_t)ex * p.n * gpr;
    const bf16_bits *x = static_cast<const bf16_bits *>(p.x);
    // x loader: pieces q = tid + NT j of the 32 x 8 pieces of 8 elements
    int64_t xrow[XP];
#pragma unroll
    for (int j = 0; j < XP; ++j) xrow[j] = (int64_t)p.perm[ch.y + min(min(tid + NT * j, 255) >> 3, cnt - 1)];
    const int wrl = tid >> 1, whalf = tid & 1;               // weight loader: row, 32-element half
    const int64_t wr = n0 + wrl, wrc = min(wr, p.n - 1);
    const int nsteps = (int)(p.k / 64);
    struct Ld {
        uint4 x[XP];
        uint4 c[BITS / 4];
        uint32_t s[NG];
    };
    auto load = [&](int step, Ld &l) {
        const int64_t k0 = (int64_t)step * 64;
#pragma unroll
        for (int j = 0; j < XP; ++j)
            if (tid + NT * j < 256)
                l.x[j] = *reinterpret_cast<const uint4 *>(x + xrow[j] * p.k + k0 + 8 * ((tid + NT * j) & 7));
        const int64_t e0 = k0 + 32 * whalf;
        const uint4 *csrc = reinterpret_cast<const uint4 *>(codes + wrc * wpr + e0 * BITS / 32);
#pragma unroll
        for (int u = 0; u < BITS / 4; ++u) l.c[u] = csrc[u];
#pragma unroll
        for (int g = 0; g < NG; ++g) l.s[g] = scales[wrc * gpr + e0 / GS + g];
    };
    auto store = [&](const Ld &l) {
#pragma unroll
        for (int j = 0; j < XP; ++j) {
            const int q = tid + NT * j;
            if (q < 256) *reinterpret_cast<uint4 *>(xs + (q >> 3) * kFpLdG + 8 * (q & 7)) = l.x[j];
        }
        uint32_t wd[BITS];
#pragma unroll
        for (int u = 0; u < BITS / 4; ++u)
            wd[4 * u] = l.c[u].x, wd[4 * u + 1] = l.c[u].y, wd[4 * u + 2] = l.c[u].z, wd[4 * u + 3] = l.c[u].w;
        uint32_t o[16];
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const float S = scale_value<MODE>(l.s[g]);
#pragma unroll
            for (int q = 0; q < GS / 2; ++q) {
                const int pi = g * (GS / 2) + q;
                if constexpr (Fp<MODE>::e8m0) {
                    o[pi] = __builtin_bit_cast(uint32_t, pair_bf16_scaled<MODE>(wd, pi, S));
                } else {
                    const f32x2_t e = pair_f32<MODE>(wd, pi);
                    const f32x2_t v = {S * e[0], S * e[1]};
                    o[pi] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
                }
            }
        }
        uint4 *wdst = reinterpret_cast<uint4 *>(ws + wrl * kFpLdG + 32 * whalf);
#pragma unroll
        for (int u = 0; u < 4; ++u)
            wdst[u] = wr < p.n ? make_uint4(o[4 * u], o[4 * u + 1], o[4 * u + 2], o[4 * u + 3])
                               : make_uint4(0u, 0u, 0u, 0u);
    };

    f32x16_t acc = {};
    Ld cur, nxt;
    if (nsteps > 0) load(0, cur);
    for (int step = 0; step < nsteps; ++step) {
        store(cur);
        __syncthreads();
        if (step + 1 < nsteps) load(step + 1, nxt);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int kk = ks * 16 + 8 * (lane >> 5);
            const bf16x8_t a = *reinterpret_cast<const bf16x8_t *>(xs + (lane & 31) * kFpLdG + kk);
            const bf16x8_t b = *reinterpret_cast<const bf16x8_t *>(ws + (wave * 32 + (lane & 31)) * kFpLdG + kk);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
        }
        __syncthreads();
        cur = nxt;
    }
    // lane l holds weight row (column of y) l % 32 of the wave's block and
    // vectors 8 (v / 4) + 4 (l / 32) + v % 4
    const float gsc = p.gscale ? p.gscale[ex] : 1.0f;
    const int64_t col = n0 + wave * 32 + (lane & 31);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int i = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (i < (int)ch.z && col < p.n)
            y[(int64_t)p.perm[ch.y + i] * p.n + col] = (bf16_bits)f32_to_bf16(acc[v] * gsc);
    }
}

// 128 x 128 tiles of y, four waves of 64 x 64 (2 x 2 blocks of
// v_mfma_f32_32x32x16_bf16), K steps of 64.  Thread t stages row t / 2 of
// the x tile and of the weight tile, 32 elements at k = 32 (t % 2): x as it
// is, the weights as bf16(S * E) (exact: an E2M1 or E4M3 value times a power
// of two or an E4M3 scale).  The next step's loads are issued before the
// current step's MFMAs.  Rows past m or n stage zeros; K is a multiple of 64.
struct FpTiledParams {
    const bf16_bits *x;
    bf16_bits *y;
    const uint32_t *codes;
    const uint8_t *scales;
    const float *gscale;
    int64_t m, n, k;
};

constexpr int kFpTM = 128, kFpTN = 128, kFpBK = 64, kFpLd = kFpBK + 8;

template <int MODE>
__global__ void __launch_bounds__(256) fp_tiled_kernel(FpTiledParams p)
{
    constexpr int BITS = Fp<MODE>::bits, GS = Fp<MODE>::gs, NG = 32 / GS;
    __shared__ __attribute__((aligned(16))) bf16_bits xs[kFpTM * kFpLd];
    __shared__ __attribute__((aligned(16))) bf16_bits ws[kFpTN * kFpLd];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    int tm, tn;
    if (!xcd_panel_tile(blockIdx.x, (int)((p.m + kFpTM - 1) / kFpTM), (int)((p.n + kFpTN - 1) / kFpTN), tm, tn))
        return;
    const int64_t m0 = (int64_t)tm * kFpTM, n0 = (int64_t)tn * kFpTN;
    const int lrow = tid >> 1, lhalf = tid & 1;
    const int64_t xm = m0 + lrow, wr = n0 + lrow;
    const int64_t xmc = min(xm, p.m - 1), wrc = min(wr, p.n - 1);
    const int64_t wpr = p.k * BITS / 32, gpr = p.k / GS;
    const int nsteps = (int)(p.k / kFpBK);

    struct Ld {
        uint4 x[4];
        uint4 c[BITS / 4];
        uint32_t s[NG];
    };
    auto load = [&](int step, Ld &l) {
        const int64_t e0 = (int64_t)step * kFpBK + 32 * lhalf;
        const uint4 *xsrc = reinterpret_cast<const uint4 *>(p.x + xmc * p.k + e0);
#pragma unroll
        for (int u = 0; u < 4; ++u) l.x[u] = xsrc[u];
        const uint4 *csrc = reinterpret_cast<const uint4 *>(p.codes + wrc * wpr + e0 * BITS / 32);
#pragma unroll
        for (int u = 0; u < BITS / 4; ++u) l.c[u] = csrc[u];
#pragma unroll
        for (int g = 0; g < NG; ++g) l.s[g] = p.scales[wrc * gpr + e0 / GS + g];
    };
    auto store = [&](const Ld &l) {
        uint4 *xd = reinterpret_cast<uint4 *>(xs + lrow * kFpLd + 32 * lhalf);
#pragma unroll
        for (int u = 0; u < 4; ++u) xd[u] = xm < p.m ? l.x[u] : make_uint4(0u, 0u, 0u, 0u);
        uint32_t wd[BITS];
#pragma unroll
        for (int u = 0; u < BITS / 4; ++u)
            wd[4 * u] = l.c[u].x, wd[4 * u + 1] = l.c[u].y, wd[4 * u + 2] = l.c[u].z, wd[4 * u + 3] = l.c[u].w;
        uint32_t o[16];
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const float S = scale_value<MODE>(l.s[g]);
#pragma unroll
            for (int q = 0; q < GS / 2; ++q) {
                const int pi = g * (GS / 2) + q;
                if constexpr (Fp<MODE>::e8m0) {
                    o[pi] = __builtin_bit_cast(uint32_t, pair_bf16_scaled<MODE>(wd, pi, S));
                } else {
                    const f32x2_t e = pair_f32<MODE>(wd, pi);
                    const f32x2_t v = {S * e[0], S * e[1]};
                    o[pi] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
                }
            }
        }
        uint4 *wdst = reinterpret_cast<uint4 *>(ws + lrow * kFpLd + 32 * lhalf);
#pragma unroll
        for (int u = 0; u < 4; ++u)
            wdst[u] = wr < p.n ? make_uint4(o[4 * u], o[4 * u + 1], o[4 * u + 2], o[4 * u + 3])
                               : make_uint4(0u, 0u, 0u, 0u);
    };

    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_t{};

    Ld cur, nxt;
    if (nsteps > 0) load(0, cur);
    for (int step = 0; step < nsteps; ++step) {
        store(cur);
        __syncthreads();
        if (step + 1 < nsteps) load(step + 1, nxt);
#pragma unroll
        for (int ks = 0; ks < kFpBK / 16; ++ks) {
            const int kk = ks * 16 + 8 * (lane >> 5);
            bf16x8_t a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                a[i] = *reinterpret_cast<const bf16x8_t *>(xs + (wm * 64 + i * 32 + (lane & 31)) * kFpLd + kk);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                b[j] = *reinterpret_cast<const bf16x8_t *>(ws + (wn * 64 + j * 32 + (lane & 31)) * kFpLd + kk);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
        cur = nxt;
    }

    const float gsc = p.gscale ? *p.gscale : 1.0f;
    // D layout of the 32x32 MFMA: lane l holds column l % 32 and rows
    // 8 (v / 4) + 4 (l / 32) + v % 4.
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t col = n0 + wn * 64 + j * 32 + (lane & 31);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t row = m0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                if (row < p.m && col < p.n) p.y[row * p.n + col] = (bf16_bits)f32_to_bf16(acc[i][j][v] * gsc);
            }
        }
}

// ---------------------------------------------------------------- weights as stored
// y[m, c] = x[m, i] . (g w_hat)[i, c] for a quantized matrix w_hat [ni, nc]
// whose groups run along c (the derivative for the activations with the
// forward weights).  Few rows: the rows of w_hat are cut into ranges that
// depend only on (ni, nc); workgroup (b, r) covers the 64 lane chunks
// [64 b, 64 b + 64) of a row (32 columns each) over range r, wave w taking
// the range's rows w, w + 4, ... in increasing order; per row a lane forms
// x[m, i] * S once and adds it times each element to its 32 column sums.
// The waves' sums are added in LDS in wave order, and a second kernel adds
// the ranges in order, so a row's bits do not depend on the other rows.
struct FpNtParams {
    const void *x;
    void *y;
    float *part;
    const uint32_t *codes;
    const uint8_t *scales;
    const float *gscale;
    int64_t m0, mr, ni, nc, rows_per_range;
    int ranges;
};

template <int MODE, typename XT, int MR>
__global__ void __launch_bounds__(256) fp_nt_partial_kernel(FpNtParams p)
{
    constexpr int BITS = Fp<MODE>::bits, GS = Fp<MODE>::gs, NG = 32 / GS, U = 4;
    __shared__ float red[3][MR][64 * 33];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t chunks = p.nc / 32, chunk = (int64_t)blockIdx.x * 64 + lane;
    const bool ok = chunk < chunks;
    const int64_t cc = ok ? chunk : 0;
    const int64_t i0 = (int64_t)blockIdx.y * p.rows_per_range, i1 = min(i0 + p.rows_per_range, p.ni);
    const int64_t wpr = p.nc * BITS / 32, gpr = p.nc / GS;
    const XT *x = static_cast<const XT *>(p.x);
    float acc[MR][32];
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int j = 0; j < 32; ++j) acc[m][j] = 0.0f;
    for (int64_t ib = i0 + wave; ib < i1; ib += 4 * U) {
        // U rows' loads first (rows past the range re-read its last row and
        // are not added)
        uint32_t wd[U][BITS];
        uint32_t sc[U][NG];
        float xv[U][MR];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = min(ib + 4 * u, i1 - 1);
            const uint4 *src = reinterpret_cast<const uint4 *>(p.codes + i * wpr + cc * BITS);
#pragma unroll
            for (int q = 0; q < BITS / 4; ++q) {
                const uint4 t = src[q];
                wd[u][4 * q] = t.x, wd[u][4 * q + 1] = t.y, wd[u][4 * q + 2] = t.z, wd[u][4 * q + 3] = t.w;
            }
#pragma unroll
            for (int g = 0; g < NG; ++g) sc[u][g] = p.scales[i * gpr + cc * NG + g];
#pragma unroll
            for (int m = 0; m < MR; ++m) xv[u][m] = Elt<XT>::load(x, (p.m0 + min((int64_t)m, p.mr - 1)) * p.ni + i);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (ib + 4 * u >= i1) break;   // uniform over the wave
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const float S = scale_value<MODE>(sc[u][g]);
                float xs[MR];
#pragma unroll
                for (int m = 0; m < MR; ++m) xs[m] = xv[u][m] * S;
#pragma unroll
                for (int q = 0; q < GS / 2; ++q) {
                    const int pi = g * (GS / 2) + q;
                    const f32x2_t e = pair_f32<MODE>(wd[u], pi);
#pragma unroll
                    for (int m = 0; m < MR; ++m) {
                        acc[m][2 * pi] = fmaf(xs[m], e[0], acc[m][2 * pi]);
                        acc[m][2 * pi + 1] = fmaf(xs[m], e[1], acc[m][2 * pi + 1]);
                    }
                }
            }
        }
    }
    if (wave > 0) {
#pragma unroll
        for (int m = 0; m < MR; ++m)
#pragma unroll
            for (int j = 0; j < 32; ++j) red[wave - 1][m][lane * 33 + j] = acc[m][j];
    }
    __syncthreads();
    if (wave == 0 && ok) {
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            if (m >= p.mr) break;
            float o[32];
#pragma unroll
            for (int j = 0; j < 32; ++j)
                o[j] = ((acc[m][j] + red[0][m][lane * 33 + j]) + red[1][m][lane * 33 + j]) + red[2][m][lane * 33 + j];
            uint4 *dst = reinterpret_cast<uint4 *>(p.part + ((int64_t)blockIdx.y * kFpNtRows + m) * p.nc + chunk * 32);
#pragma unroll
            for (int t = 0; t < 8; ++t)
                dst[t] = make_uint4(__float_as_uint(o[4 * t]), __float_as_uint(o[4 * t + 1]),
                                    __float_as_uint(o[4 * t + 2]), __float_as_uint(o[4 * t + 3]));
        }
    }
}

// y[m0 + m, c] = g * sum over the ranges of part[r][m][c]: workgroup (b, m)
// takes 16 columns; thread (part q, column j) adds the ranges of part q
// (consecutive, increasing) and the 16 part sums are added in part order in
// LDS.  The order depends only on the number of ranges.
constexpr int kFpNtRedParts = 16;

template <typename XT>
__global__ void __launch_bounds__(256) fp_nt_reduce_kernel(FpNtParams p)
{
    __shared__ float ps[kFpNtRedParts][16];
    const int j = threadIdx.x & 15, q = threadIdx.x >> 4;
    const int64_t col = (int64_t)blockIdx.x * 16 + j;
    const int m = blockIdx.y;
    const int per = (p.ranges + kFpNtRedParts - 1) / kFpNtRedParts;
    const int r0 = min(q * per, p.ranges), r1 = min(r0 + per, p.ranges);
    const int64_t stride = (int64_t)kFpNtRows * p.nc;
    const float *src = p.part + (int64_t)m * p.nc + min(col, p.nc - 1);
    float s = 0.0f;
    int r = r0;
    for (; r + 8 <= r1; r += 8) {
        float v[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) v[t] = src[(int64_t)(r + t) * stride];
#pragma unroll
        for (int t = 0; t < 8; ++t) s += v[t];
    }
    for (; r < r1; ++r) s += src[(int64_t)r * stride];
    ps[q][j] = s;
    __syncthreads();
    if (q == 0 && col < p.nc) {
        float t = ps[0][j];
#pragma unroll
        for (int u = 1; u < kFpNtRedParts; ++u) t += ps[u][j];
        const float g = p.gscale ? *p.gscale : 1.0f;
        Elt<XT>::store(static_cast<XT *>(p.y), (p.m0 + m) * p.nc + col, t * g);
    }
}

// Many bf16 rows: 128 x 128 tiles of y with bf16 MFMA, K steps of 64 rows i
// of w_hat; thread t stages 32 elements of x row t / 2 and the 16 columns
// 16 (t % 8) .. + 15 of w_hat rows 2 (t / 8) and 2 (t / 8) + 1, converted to
// bf16(S * E) and written down LDS columns, two rows per 4-byte write, so
// that a B operand reads 8 consecutive i of one column.  Column c starts at
// c * 72 + 16 ((c / 16) % 8) elements, which puts the 64 writes of a wave
// instruction (8 row pairs x 8 column groups) on distinct banks and keeps a
// B-operand read phase (16 columns) on one shift.  ni is a multiple of 64.
__device__ __forceinline__ int fp_nt_wcol(int c) { return c * 72 + 16 * ((c >> 4) & 7); }

template <int MODE>
__global__ void __launch_bounds__(256) fp_tiled_nt_kernel(FpNtParams p)
{
    constexpr int BITS = Fp<MODE>::bits, GS = Fp<MODE>::gs;
    __shared__ __attribute__((aligned(16))) bf16_bits xs[2][128 * 72];
    __shared__ __attribute__((aligned(16))) bf16_bits ws[2][128 * 72 + 128];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    int tm, tn;
    if (!xcd_panel_tile(blockIdx.x, (int)((p.mr + 127) / 128), (int)((p.nc + 127) / 128), tm, tn)) return;
    const int64_t m0 = (int64_t)tm * 128, c0 = (int64_t)tn * 128;
    const int lrow = tid >> 1, lhalf = tid & 1;
    // rows past mr read row mr - 1 and columns past nc column 0: their
    // products land only in outputs that are not stored
    const int64_t xmc = min(m0 + lrow, p.mr - 1);
    // weights: thread t takes rows 2 (t / 8) and 2 (t / 8) + 1 of the step
    // and the 16 columns from 16 (t % 8), inside one scale group (GS is 16
    // or 32), and writes the two rows' values of a column as one 4-byte word
    const int wrow = 2 * (tid >> 3), wcol = 16 * (tid & 7);
    const int64_t cb = c0 + wcol;
    const int64_t cbc = cb < p.nc ? cb : 0;
    const int64_t wpr = p.nc * BITS / 32, gpr = p.nc / GS;
    const bf16_bits *x = static_cast<const bf16_bits *>(p.x);
    const int nsteps = (int)(p.ni / 64);
    constexpr int NW = 16 * BITS / 32;   // code words of a row's 16 columns
    struct Ld {
        uint4 x[4];
        uint32_t c[2][NW];
        uint32_t s[2];
    };
    auto load = [&](int step, Ld &l) {
        const int64_t i0 = (int64_t)step * 64;
        const uint4 *xsrc = reinterpret_cast<const uint4 *>(x + xmc * p.ni + i0 + 32 * lhalf);
#pragma unroll
        for (int u = 0; u < 4; ++u) l.x[u] = xsrc[u];
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int64_t i = i0 + wrow + r;
            const uint32_t *csrc = p.codes + i * wpr + cbc * BITS / 32;
            if constexpr (NW == 4) {
                const uint4 d = *reinterpret_cast<const uint4 *>(csrc);
                l.c[r][0] = d.x, l.c[r][1] = d.y, l.c[r][2] = d.z, l.c[r][3] = d.w;
            } else {
                const uint2 d = *reinterpret_cast<const uint2 *>(csrc);
                l.c[r][0] = d.x, l.c[r][1] = d.y;
            }
            l.s[r] = p.scales[i * gpr + cbc / GS];
        }
    };
    auto store = [&](const Ld &l, auto bufc) {
        constexpr int B = decltype(bufc)::value;
        uint4 *xd = reinterpret_cast<uint4 *>(xs[B] + lrow * 72 + 32 * lhalf);
#pragma unroll
        for (int u = 0; u < 4; ++u) xd[u] = make_uint4(l.x[u].x, l.x[u].y, l.x[u].z, l.x[u].w);
        // bf16 pairs of adjacent columns of each row, regrouped by one
        // v_perm_b32 per word into the two rows of one column
        uint32_t h[2][8];
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            uint32_t wd[BITS] = {};   // the first NW words hold the 16 codes
#pragma unroll
            for (int j = 0; j < NW; ++j) wd[j] = l.c[r][j];
            const float S = scale_value<MODE>(l.s[r]);
#pragma unroll
            for (int pi = 0; pi < 8; ++pi) {
                if constexpr (Fp<MODE>::e8m0) {
                    h[r][pi] = __builtin_bit_cast(uint32_t, pair_bf16_scaled<MODE>(wd, pi, S));
                } else {
                    const f32x2_t e = pair_f32<MODE>(wd, pi);
                    const f32x2_t v = {S * e[0], S * e[1]};
                    h[r][pi] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
                }
            }
        }
#pragma unroll
        for (int pi = 0; pi < 8; ++pi) {
            *reinterpret_cast<uint32_t *>(&ws[B][fp_nt_wcol(wcol + 2 * pi) + wrow]) =
                __builtin_amdgcn_perm(h[1][pi], h[0][pi], 0x05040100u);
            *reinterpret_cast<uint32_t *>(&ws[B][fp_nt_wcol(wcol + 2 * pi + 1) + wrow]) =
                __builtin_amdgcn_perm(h[1][pi], h[0][pi], 0x07060302u);
        }
    };
    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_t{};
    auto mfmas = [&](auto bufc) {
        constexpr int B = decltype(bufc)::value;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int kk = ks * 16 + 8 * (lane >> 5);
            bf16x8_t a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                a[i] = *reinterpret_cast<const bf16x8_t *>(xs[B] + (wm * 64 + i * 32 + (lane & 31)) * 72 + kk);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                b[j] = *reinterpret_cast<const bf16x8_t *>(ws[B] + fp_nt_wcol(wn * 64 + j * 32 + (lane & 31)) + kk);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    };
    tile_pipeline<Ld>(nsteps, load, store, mfmas);
    const float gsc = p.gscale ? *p.gscale : 1.0f;
    bf16_bits *y = static_cast<bf16_bits *>(p.y);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t col = c0 + wn * 64 + j * 32 + (lane & 31);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t row = m0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                if (row < p.mr && col < p.nc) y[row * p.nc + col] = (bf16_bits)f32_to_bf16(acc[i][j][v] * gsc);
            }
        }
}

// ---------------------------------------------------------------- launchers
namespace {

template <template <int> class F, typename... A>
hipError_t by_mode(int mode, A &&...a)
{
    switch (mode) {
    case FP_MXFP4: return F<FP_MXFP4>::run(a...);
    case FP_MXFP8: return F<FP_MXFP8>::run(a...);
    default: return F<FP_NVFP4>::run(a...);
    }
}

template <int MODE> struct QuantRun {
    static hipError_t run(const void *w, int w_dt, int64_t chunks, uint32_t *codes, uint8_t *scales,
                          hipStream_t stream)
    {
        const dim3 grid((unsigned)((chunks + 255) / 256));
        if (w_dt == DT_BF16)
            fp_quantize_kernel<MODE, bf16_bits><<<grid, 256, 0, stream>>>(
                static_cast<const bf16_bits *>(w), chunks, codes, scales);
        else
            fp_quantize_kernel<MODE, float><<<grid, 256, 0, stream>>>(static_cast<const float *>(w),
                                                                       chunks, codes, scales);
        return hipGetLastError();
    }
};

template <int MODE> struct DequantRun {
    static hipError_t run(const uint32_t *codes, const uint8_t *scales, int64_t chunks, void *out,
                          int out_dt, hipStream_t stream)
    {
        const dim3 grid((unsigned)((chunks + 255) / 256));   // 4 waves of 64 chunks
        if (out_dt == DT_BF16)
            fp_dequantize_kernel<MODE, bf16_bits><<<grid, 256, 0, stream>>>(codes, scales, chunks,
                                                                             static_cast<bf16_bits *>(out));
        else
            fp_dequantize_kernel<MODE, float><<<grid, 256, 0, stream>>>(codes, scales, chunks,
                                                                         static_cast<float *>(out));
        return hipGetLastError();
    }
};

template <int MODE, typename XT, int MR, int RW>
hipError_t gemv_mr_rw(const FpQmmLaunch &a, hipStream_t stream)
{
    FpGemvParams p;
    p.x = a.x, p.y = a.y, p.codes = a.codes, p.scales = a.scales, p.gscale = a.gscale, p.idx = a.idx;
    p.vpi = a.vpi, p.cpi = (a.vpi + MR - 1) / MR;
    p.n = a.n, p.k = a.k, p.e = a.idx || a.chunks ? a.e : 1;
    p.chunks = a.chunks, p.perm = a.perm, p.nchunks = a.nchunks;
    const int64_t total = a.chunks ? a.max_chunks : a.items * p.cpi;
    for (p.y0 = 0; p.y0 < total; p.y0 += 65535) {   // grid.y is at most 65535
        const dim3 grid((unsigned)((a.n + 4 * RW - 1) / (4 * RW)), (unsigned)std::min<int64_t>(65535, total - p.y0));
        fp_gemv_kernel<MODE, XT, MR, RW><<<grid, 256, 0, stream>>>(p);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

// Weight rows per wave: the most of 4, 2, 1 whose workgroup count along n
// fills its last round of 256 compute units best (a whole number of
// workgroups per CU; an uneven count leaves some CUs a round longer).  One
// x load serves RW rows; RW never changes a row's arithmetic.
inline int fp_gemv_rows_per_wave(int64_t n)
{
    int best = 4;
    double best_fill = 0.0;
    for (int rw : {4, 2, 1}) {
        const int64_t g = (n + 4 * rw - 1) / (4 * rw);
        const double fill = (double)g / (double)(((g + 255) / 256) * 256);
        if (fill > best_fill + 1e-9) best = rw, best_fill = fill;
    }
    return best;
}

template <int MODE, typename XT, int MR>
hipError_t gemv_mr(const FpQmmLaunch &a, hipStream_t stream)
{
    switch (fp_gemv_rows_per_wave(a.n)) {
    case 1: return gemv_mr_rw<MODE, XT, MR, 1>(a, stream);
    case 2: return gemv_mr_rw<MODE, XT, MR, 2>(a, stream);
    default: return gemv_mr_rw<MODE, XT, MR, 4>(a, stream);
    }
}

// Workgroups of a kernel that stay resident together on one CU (at most
// `cap`), and the device's CU count; asked once per kernel.
template <typename K>
int64_t resident_grid(K kernel, int cap)
{
    static const int64_t total = [&] {
        int per = 1, dev = 0, cus = 256;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, 256, 0) != hipSuccess || per < 1) per = 1;
        if (hipGetDevice(&dev) == hipSuccess)
            (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        return (int64_t)std::min(per, cap) * cus;
    }();
    return total;
}

// One bf16 row, one weight matrix, K at most 256 lane chunks: the
// streaming kernel on a whole number of workgroups per CU that stay
// resident together (at most 4).
template <int MODE, int U>
hipError_t gemv_stream(const FpQmmLaunch &a, hipStream_t stream)
{
    FpGemvParams p = {};
    p.x = a.x, p.y = a.y, p.codes = a.codes, p.scales = a.scales, p.gscale = a.gscale;
    p.n = a.n, p.k = a.k, p.e = 1;
    const int64_t wgs = std::min<int64_t>((a.n + 3) / 4, resident_grid(fp_gemv_stream_kernel<MODE, U>, 4));
    fp_gemv_stream_kernel<MODE, U><<<dim3((unsigned)wgs), 256, 0, stream>>>(p);
    return hipGetLastError();
}

// Grouped gather with bf16 x and K = 2048: the streaming gather kernel,
// about 32 weight rows per wave.
template <int MODE>
hipError_t gather_stream(const FpQmmLaunch &a, hipStream_t stream)
{
    FpGemvParams p = {};
    p.x = a.x, p.y = a.y, p.codes = a.codes, p.scales = a.scales, p.gscale = a.gscale;
    p.n = a.n, p.k = a.k, p.e = a.e;
    p.chunks = a.chunks, p.perm = a.perm, p.nchunks = a.nchunks;
    const dim3 grid((unsigned)((a.n + 127) / 128), (unsigned)a.max_chunks);
    fp_gather_stream_kernel<MODE><<<grid, 256, 0, stream>>>(p);
    return hipGetLastError();
}

// Grouped gather on matrix cores: 128 weight rows per workgroup, one
// workgroup row per chunk of up to 32 vectors.
template <int MODE>
hipError_t gather_mfma(const FpQmmLaunch &a, hipStream_t stream)
{
    FpGemvParams p = {};
    p.x = a.x, p.y = a.y, p.codes = a.codes, p.scales = a.scales, p.gscale = a.gscale;
    p.n = a.n, p.k = a.k, p.e = a.e;
    p.chunks = a.chunks, p.perm = a.perm, p.nchunks = a.nchunks;
    constexpr int NW = 4;   // measured: 2 waves 73 us, 4 waves 48 us, 8 waves 57 us (512 rows, 32 experts)
    fp_gather_mfma_kernel<MODE, NW><<<dim3((unsigned)((a.n + 32 * NW - 1) / (32 * NW)), (unsigned)a.max_chunks),
                                      64 * NW, 0, stream>>>(p);
    return hipGetLastError();
}

template <int MODE> struct QmmRun {
    static hipError_t run(const FpQmmLaunch &a, hipStream_t stream)
    {
        if (a.chunks && a.mfma) return gather_mfma<MODE>(a, stream);
        if (a.chunks && a.x_dt == DT_BF16 && a.k == 2048 && a.max_chunks <= 65535)
            return gather_stream<MODE>(a, stream);
        if (!a.tiled && !a.idx && !a.chunks && a.vpi == 1 && a.items == 1 && a.x_dt == DT_BF16 && a.k > 0 &&
            a.k <= 256 * 32) {
            const int64_t c = a.k / 32;
            if (c <= 64) return gemv_stream<MODE, 1>(a, stream);
            if (c <= 128) return gemv_stream<MODE, 2>(a, stream);
            return gemv_stream<MODE, 4>(a, stream);
        }
        if (a.tiled) {
            FpTiledParams p;
            p.x = static_cast<const bf16_bits *>(a.x), p.y = static_cast<bf16_bits *>(a.y);
            p.codes = a.codes, p.scales = a.scales, p.gscale = a.gscale;
            p.m = a.vpi, p.n = a.n, p.k = a.k;
            const int64_t tiles = ((a.n + kFpTN - 1) / kFpTN) * ((a.vpi + kFpTM - 1) / kFpTM);
            const unsigned blocks = xcd_panel_blocks(tiles);
            if (blocks == 0) return hipErrorInvalidValue;
            fp_tiled_kernel<MODE><<<dim3(blocks), 256, 0, stream>>>(p);
            return hipGetLastError();
        }
        const int64_t v = a.chunks ? kGroupChunk : a.vpi;
        if (a.x_dt == DT_BF16) {
            if (v <= 1) return gemv_mr<MODE, bf16_bits, 1>(a, stream);
            if (v <= 2) return gemv_mr<MODE, bf16_bits, 2>(a, stream);
            if (v <= 4) return gemv_mr<MODE, bf16_bits, 4>(a, stream);
            return gemv_mr<MODE, bf16_bits, 8>(a, stream);
        }
        if (v <= 1) return gemv_mr<MODE, float, 1>(a, stream);
        if (v <= 2) return gemv_mr<MODE, float, 2>(a, stream);
        if (v <= 4) return gemv_mr<MODE, float, 4>(a, stream);
        return gemv_mr<MODE, float, 8>(a, stream);
    }
};

}  // namespace

hipError_t launch_fp_quantize(const void *w, int w_dt, int64_t n, int64_t k, int mode, uint32_t *codes,
                              uint8_t *scales, hipStream_t stream)
{
    return by_mode<QuantRun>(mode, w, w_dt, n * (k / 32), codes, scales, stream);
}

hipError_t launch_fp_dequantize(const uint32_t *codes, const uint8_t *scales, int64_t n, int64_t k, int mode,
                                void *out, int out_dt, hipStream_t stream)
{
    return by_mode<DequantRun>(mode, codes, scales, n * (k / 32), out, out_dt, stream);
}

int fp_nt_ranges(int64_t ni, int64_t nc)
{
    if (ni <= 0) return 1;
    const int64_t cblocks = (nc / 32 + 63) / 64;
    int64_t r = std::max<int64_t>(1, std::min<int64_t>((512 + cblocks - 1) / std::max<int64_t>(cblocks, 1), (ni + 3) / 4));
    r = std::min<int64_t>(r, 65535);
    const int64_t per = (ni + r - 1) / r;
    return (int)((ni + per - 1) / per);
}

size_t fp_nt_ws_bytes(int64_t ni, int64_t nc)
{
    return (size_t)fp_nt_ranges(ni, nc) * kFpNtRows * (size_t)nc * 4;
}

namespace {
template <int MODE> struct NtRun {
    static hipError_t run(const FpNtLaunch &a, hipStream_t stream)
    {
        FpNtParams p = {};
        p.x = a.x, p.y = a.y, p.codes = a.codes, p.scales = a.scales, p.gscale = a.gscale;
        p.ni = a.ni, p.nc = a.nc;
        if (a.tiled) {
            p.mr = a.m;
            const int64_t tiles = ((a.nc + 127) / 128) * ((a.m + 127) / 128);
            const unsigned blocks = xcd_panel_blocks(tiles);
            if (blocks == 0) return hipErrorInvalidValue;
            fp_tiled_nt_kernel<MODE><<<dim3(blocks), 256, 0, stream>>>(p);
            return hipGetLastError();
        }
        p.part = static_cast<float *>(a.workspace);
        p.ranges = fp_nt_ranges(a.ni, a.nc);
        p.rows_per_range = (a.ni + p.ranges - 1) / p.ranges;
        const dim3 pgrid((unsigned)((a.nc / 32 + 63) / 64), (unsigned)p.ranges);
        for (int64_t m0 = 0; m0 < a.m; m0 += kFpNtRows) {
            p.m0 = m0, p.mr = std::min<int64_t>(kFpNtRows, a.m - m0);
            // the chunk's row count as a template argument (a row's arithmetic is the same either way)
            if (a.x_dt == DT_BF16) {
                if (p.mr == 1) fp_nt_partial_kernel<MODE, bf16_bits, 1><<<pgrid, 256, 0, stream>>>(p);
                else fp_nt_partial_kernel<MODE, bf16_bits, kFpNtRows><<<pgrid, 256, 0, stream>>>(p);
            } else {
                if (p.mr == 1) fp_nt_partial_kernel<MODE, float, 1><<<pgrid, 256, 0, stream>>>(p);
                else fp_nt_partial_kernel<MODE, float, kFpNtRows><<<pgrid, 256, 0, stream>>>(p);
            }
            hipError_t err = hipGetLastError();
            if (err != hipSuccess) return err;
            const dim3 rgrid((unsigned)((a.nc + 15) / 16), (unsigned)p.mr);
            if (a.x_dt == DT_BF16) fp_nt_reduce_kernel<bf16_bits><<<rgrid, 256, 0, stream>>>(p);
            else fp_nt_reduce_kernel<float><<<rgrid, 256, 0, stream>>>(p);
            if ((err = hipGetLastError()) != hipSuccess) return err;
        }
        return hipSuccess;
    }
};
}  // namespace

hipError_t launch_fp_qmm_nt(const FpNtLaunch &a, hipStream_t stream)
{
    return by_mode<NtRun>(a.mode, a, stream);
}

hipError_t launch_fp_qmm(const FpQmmLaunch &a, hipStream_t stream)
{
    return by_mode<QmmRun>(a.mode, a, stream);
}

}  // namespace nqk
