// Group-wise affine quantize and dequantize kernels for gfx950.
//
// Method: "Quantization" page of the nuvec documentation, section "Affine":
// rows are cut into groups of group_size values, each group keeps one scale
// and one bias, values become `bits`-bit codes packed into uint32 words and
// w ~ scale * code + bias.  Scale/bias selection (min/max), rounding and bit
// order follow the contract stated in include/nq.h.
//
// Both kernels are bandwidth-bound streams: one lane owns 32 consecutive
// elements of a row (one lane chunk, always inside one group), reads them with
// 16-byte loads and writes `bits` words of codes.  A group of 32/64/128
// values spans 1/2/4 adjacent lanes, which exchange min/max with xor
// shuffles.  The file is built with -ffp-contract=off: every fp32 step below
// rounds once, as written, which is what makes quantize bit-exact.
#include <math.h>

#include "nq_device.h"
#include "nq_internal.h"

namespace nqk {

template <int BITS>
__device__ __forceinline__ void store_words(uint32_t *dst, const uint32_t *wd)
{
    if constexpr (BITS % 4 == 0) {
#pragma unroll
        for (int i = 0; i < BITS / 4; ++i)
            reinterpret_cast<uint4 *>(dst)[i] =
                make_uint4(wd[4 * i], wd[4 * i + 1], wd[4 * i + 2], wd[4 * i + 3]);
    } else if constexpr (BITS % 2 == 0) {
#pragma unroll
        for (int i = 0; i < BITS / 2; ++i)
            reinterpret_cast<uint2 *>(dst)[i] = make_uint2(wd[2 * i], wd[2 * i + 1]);
    } else {
#pragma unroll
        for (int i = 0; i < BITS; ++i) dst[i] = wd[i];
    }
}

template <int BITS>
__device__ __forceinline__ void load_words(const uint32_t *src, uint32_t *wd)
{
    if constexpr (BITS % 4 == 0) {
#pragma unroll
        for (int i = 0; i < BITS / 4; ++i) {
            uint4 d = reinterpret_cast<const uint4 *>(src)[i];
            wd[4 * i] = d.x, wd[4 * i + 1] = d.y, wd[4 * i + 2] = d.z, wd[4 * i + 3] = d.w;
        }
    } else if constexpr (BITS % 2 == 0) {
#pragma unroll
        for (int i = 0; i < BITS / 2; ++i) {
            uint2 d = reinterpret_cast<const uint2 *>(src)[i];
            wd[2 * i] = d.x, wd[2 * i + 1] = d.y;
        }
    } else {
#pragma unroll
        for (int i = 0; i < BITS; ++i) wd[i] = src[i];
    }
}

// One lane per 32-element chunk; chunks are numbered row-major over [n, k/32].
template <int BITS, typename WT>
__global__ void __launch_bounds__(256)
quantize_kernel(const WT *__restrict__ w, int64_t chunks, int64_t k, int gs,
                uint32_t *__restrict__ codes, WT *__restrict__ scales, WT *__restrict__ biases)
{
    // A wave's 64 chunks are one contiguous run of w, moved into LDS by
    // direct-to-LDS loads that each cover 1 KB of the run (16 bytes every 64
    // or 128 per instruction if each lane loaded its own chunk).  Instruction
    // i, lane l takes the run's 16-byte piece 64 i + kPPC (l % kCPI) + l / kCPI
    // into LDS slot 64 i + l, so that piece q of chunk c sits in slot
    // 64 (c / kCPI) + kCPI q + c % kCPI: a lane's q-th read and its 15
    // neighbours' touch 16 consecutive slots (bf16; two such runs for f32).
    constexpr int kPPC = kLaneChunk * (int)sizeof(WT) / 16;   // pieces per chunk: 4 (bf16), 8 (f32)
    constexpr int kCPI = 64 / kPPC;                           // chunks per load instruction
    constexpr int kEPP = 16 / (int)sizeof(WT);                // elements per piece
    __shared__ uint4 stage[4][64 * kPPC];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t c0 = (int64_t)blockIdx.x * blockDim.x + wave * 64;   // the wave's first chunk
    const int64_t c = c0 + lane;
    const bool valid = c < chunks;
    const int lanes_per_group = gs / kLaneChunk;   // 1, 2 or 4, adjacent lanes
    const float top = (float)((1u << BITS) - 1u);

    if (c0 >= chunks) return;   // the whole wave is past the end (no barriers here)
    float v[kLaneChunk];
    {
        // pieces past the end of w re-read its last piece (the lanes they
        // reach are past the end too, and their groups hold no valid lane)
        const int64_t last_piece = min((chunks - c0) * kPPC, (int64_t)64 * kPPC) - 1;
        const WT *run = w + c0 * kLaneChunk;
#pragma unroll
        for (int i = 0; i < kPPC; ++i) {
            const int64_t piece = min((int64_t)(64 * i + kPPC * (lane % kCPI) + lane / kCPI), last_piece);
            __builtin_amdgcn_global_load_lds((const void *)(run + piece * kEPP),
                                             (__attribute__((address_space(3))) void *)(stage[wave] + 64 * i),
                                             16, 0, 0);
        }
        __builtin_amdgcn_s_waitcnt(0xf70);   // vmcnt(0): this wave's pieces are in LDS
        asm volatile("" ::: "memory");
#pragma unroll
        for (int q = 0; q < kPPC; ++q) {
            const uint4 d = stage[wave][64 * (lane / kCPI) + kCPI * q + lane % kCPI];
            const uint32_t u[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if constexpr (sizeof(WT) == 2) {
                    v[kEPP * q + 2 * j] = __uint_as_float(u[j] << 16);
                    v[kEPP * q + 2 * j + 1] = __uint_as_float(u[j] & 0xffff0000u);
                } else {
                    v[kEPP * q + j] = __uint_as_float(u[j]);
                }
            }
        }
    }
    // Three-input hardware min and max (weights are finite by contract; the
    // sign of a zero extreme is dropped below, so ties between -0 and +0 do
    // not matter).
    float mn = v[0], mx = v[0];
#pragma unroll
    for (int j = 1; j + 1 < kLaneChunk; j += 2) {
        asm("v_min3_f32 %0, %1, %2, %3" : "=v"(mn) : "v"(mn), "v"(v[j]), "v"(v[j + 1]));
        asm("v_max3_f32 %0, %1, %2, %3" : "=v"(mx) : "v"(mx), "v"(v[j]), "v"(v[j + 1]));
    }
    asm("v_min_f32 %0, %1, %2" : "=v"(mn) : "v"(mn), "v"(v[kLaneChunk - 1]));
    asm("v_max_f32 %0, %1, %2" : "=v"(mx) : "v"(mx), "v"(v[kLaneChunk - 1]));
    // A group's lanes are all valid or all invalid (k is a multiple of gs).
    for (int off = 1; off < lanes_per_group; off <<= 1) {
        const float omn = __shfl_xor(mn, off);
        const float omx = __shfl_xor(mx, off);
        mn = omn < mn ? omn : mn;
        mx = omx > mx ? omx : mx;
    }
    if (!valid) return;

    mn = mn + 0.0f;   // -0 -> +0, so the result does not depend on the order
    mx = mx + 0.0f;
    const float range = mx - mn;
    float scale = range / top;   // IEEE division (correctly rounded)
    scale = scale + 0.0f;
    const float s = Elt<WT>::stored(scale);
    const float b = Elt<WT>::stored(mn);

    // A row is k / gs whole groups of lanes_per_group chunks, so chunk c
    // belongs to group c / lanes_per_group (row-major over [n, k / gs]).
    if ((c & (lanes_per_group - 1)) == 0) {
        const int64_t gi = c >> (lanes_per_group == 4 ? 2 : lanes_per_group - 1);
        Elt<WT>::store(scales, gi, scale);
        Elt<WT>::store(biases, gi, mn);
    }

    // Code = clamp(rint(t), 0, top) with t = (v - b) / s rounded once (IEEE
    // division; 0 when s is 0).  No division runs per element: with r within
    // 1 ulp of 1 / s (v_rcp_f32), t0 = (v - b) * r is within
    // 4.0000003 u |t0| of t (u = 2^-24).  Where t0 is more than
    // 2^-21 (1 + |t0|) from the nearest half-integer, t lies strictly inside
    // the same unit interval as t0, so rint(t) = rint(t0).  Elements nearer
    // a half-integer (a few in 10^4 for spread values), and every element
    // of a group whose scale is 0 or outside [2^-120, 2^120] (where r or t0
    // could leave the normal range), take the division itself.
    // The margin test's value is a non-negative float or NaN, so comparing
    // its bits as unsigned integers orders it as a float with NaN above all:
    // one running maximum per lane says whether any element failed.
    // Up to 7 bits the fast codes need no clamp: 0 <= v - b <= max - min, so
    // 0 <= t0 <= top (1 + 2^-9 + 4 u) (the stored scale is at most 2^-9 below
    // (max - min) / top), which rounds to at most top.
    const bool s_ok = s >= 0x1p-120f && s <= 0x1p120f;
    const float r = __builtin_amdgcn_rcpf(s_ok ? s : 1.0f);
    constexpr float kMargin = 0.5f - 0x1p-20f;
    constexpr bool kClampFast = BITS == 8;
    auto margin = [](float t0, float m) { return fmaf(fabsf(t0), 0x1p-21f, fabsf(t0 - m)); };
    auto clamp = [&](float t) {
        float o;   // [0, top] in one instruction (the codes are finite)
        asm("v_med3_f32 %0, %1, 0, %2" : "=v"(o) : "v"(t), "v"(top));
        return o;
    };
    float tq[kLaneChunk];
    uint32_t worst = s_ok ? 0u : 0xffffffffu;
#pragma unroll
    for (int j = 0; j < kLaneChunk; ++j) {
        const float t0 = (v[j] - b) * r;
        tq[j] = rintf(t0);
        worst = max(worst, __float_as_uint(margin(t0, tq[j])));
    }
    if (worst >= __float_as_uint(kMargin)) {
#pragma unroll
        for (int j = 0; j < kLaneChunk; ++j) {
            const float d = v[j] - b;
            const float t0 = d * r;
            if (!(s_ok && margin(t0, rintf(t0)) < kMargin)) tq[j] = s != 0.0f ? clamp(rintf(d / s)) : 0.0f;
        }
    }
    uint32_t wd[BITS];
#pragma unroll
    for (int i = 0; i < BITS; ++i) wd[i] = 0u;
#pragma unroll
    for (int j = 0; j < kLaneChunk; ++j) {
        const uint32_t q = (uint32_t)(kClampFast ? clamp(tq[j]) : tq[j]);
        const int bit = j * BITS;
        wd[bit >> 5] |= q << (bit & 31);
        if ((bit & 31) + BITS > 32) wd[(bit >> 5) + 1] |= q >> (32 - (bit & 31));
    }
    store_words<BITS>(codes + c * BITS, wd);
}

template <int BITS, typename ST, typename OT>
__global__ void __launch_bounds__(256)
dequantize_kernel(const uint32_t *__restrict__ codes, const ST *__restrict__ scales,
                  const ST *__restrict__ biases, int64_t chunks, int64_t k, int gs,
                  OT *__restrict__ out)
{
    // A lane's 32 outputs are 16-byte pieces; a wave's 64 chunks are one
    // contiguous run of the output.  The pieces go through LDS so that store
    // instruction i writes pieces 64 i .. 64 i + 63 of the run: 1 KB
    // contiguous per instruction instead of 16 bytes every 64 or 128.
    constexpr int kPieces = kLaneChunk * (int)sizeof(OT) / 16;   // 4 (bf16) or 8 (f32)
    constexpr int kStride = kPieces + 1;                         // padded LDS row, in pieces
    __shared__ uint4 stage[4][64 * kStride];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t c0 = (int64_t)blockIdx.x * blockDim.x + wave * 64;   // the wave's first chunk
    const int64_t c = min(c0 + lane, chunks - 1);                       // past the end: a valid chunk, not stored
    const int64_t chunks_per_row = k / kLaneChunk;
    const int64_t row = c / chunks_per_row;
    const int64_t cir = c - row * chunks_per_row;
    const int64_t gi = row * (k / gs) + cir * kLaneChunk / gs;
    const float s = Elt<ST>::load(scales, gi);
    const float b = Elt<ST>::load(biases, gi);
    uint32_t wd[BITS];
    load_words<BITS>(codes + c * BITS, wd);
    float v[kLaneChunk];
#pragma unroll
    for (int j = 0; j < kLaneChunk; ++j) v[j] = fmaf(s, (float)code_at<BITS>(wd, j), b);
    uint4 *st = stage[wave] + lane * kStride;
    if constexpr (sizeof(OT) == 4) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            st[i] = make_uint4(__float_as_uint(v[4 * i]), __float_as_uint(v[4 * i + 1]),
                               __float_as_uint(v[4 * i + 2]), __float_as_uint(v[4 * i + 3]));
    } else {
        // v_cvt_pk_bf16_f32: round to nearest even, the rounding of f32_to_bf16
        // for every finite value (the values here are finite)
        typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
        typedef float f32x2_v __attribute__((ext_vector_type(2)));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t pk[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x2_v f = {v[8 * i + 2 * j], v[8 * i + 2 * j + 1]};
                pk[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_v));
            }
            st[i] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
        }
    }
    __builtin_amdgcn_wave_barrier();   // the wave's LDS writes before its reads (one wave, no workgroup barrier)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    uint4 *dst = reinterpret_cast<uint4 *>(out + c0 * kLaneChunk);
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
        const int q = i * 64 + lane;          // piece q of the run: chunk q / kPieces, piece q % kPieces
        const int ch = q / kPieces, pc = q % kPieces;
        if (c0 + ch < chunks) dst[q] = stage[wave][ch * kStride + pc];
    }
}

namespace {

template <typename WT>
hipError_t quantize_bits(const void *w, int64_t n, int64_t k, int gs, int bits, uint32_t *codes,
                         void *scales, void *biases, hipStream_t stream)
{
    const int64_t chunks = n * (k / kLaneChunk);
    const dim3 block(256);
    const dim3 grid((unsigned)((chunks + 255) / 256));
    const WT *wp = static_cast<const WT *>(w);
    WT *sp = static_cast<WT *>(scales), *bp = static_cast<WT *>(biases);
    switch (bits) {
#define NQ_Q(B)                                                                            \
    case B:                                                                                \
        quantize_kernel<B, WT><<<grid, block, 0, stream>>>(wp, chunks, k, gs, codes, sp, bp); \
        break;
        NQ_Q(1) NQ_Q(2) NQ_Q(3) NQ_Q(4) NQ_Q(5) NQ_Q(6) NQ_Q(8)
#undef NQ_Q
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename ST, typename OT>
hipError_t dequantize_bits(const uint32_t *codes, const void *scales, const void *biases,
                           int64_t n, int64_t k, int gs, int bits, void *out, hipStream_t stream)
{
    const int64_t chunks = n * (k / kLaneChunk);
    const dim3 block(256);
    const dim3 grid((unsigned)((chunks + 255) / 256));
    const ST *sp = static_cast<const ST *>(scales), *bp = static_cast<const ST *>(biases);
    OT *op = static_cast<OT *>(out);
    switch (bits) {
#define NQ_D(B)                                                                                 \
    case B:                                                                                     \
        dequantize_kernel<B, ST, OT><<<grid, block, 0, stream>>>(codes, sp, bp, chunks, k, gs, op); \
        break;
        NQ_D(1) NQ_D(2) NQ_D(3) NQ_D(4) NQ_D(5) NQ_D(6) NQ_D(8)
#undef NQ_D
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(const void *w, int w_dt, int64_t n, int64_t k, int gs, int bits,
                           uint32_t *codes, void *scales, void *biases, hipStream_t stream)
{
    if (w_dt == DT_F32) return quantize_bits<float>(w, n, k, gs, bits, codes, scales, biases, stream);
    return quantize_bits<bf16_bits>(w, n, k, gs, bits, codes, scales, biases, stream);
}

hipError_t launch_dequantize(const uint32_t *codes, const void *scales, const void *biases,
                             int sb_dt, int64_t n, int64_t k, int gs, int bits, void *out,
                             int out_dt, hipStream_t stream)
{
    if (sb_dt == DT_F32) {
        if (out_dt == DT_F32)
            return dequantize_bits<float, float>(codes, scales, biases, n, k, gs, bits, out, stream);
        return dequantize_bits<float, bf16_bits>(codes, scales, biases, n, k, gs, bits, out, stream);
    }
    if (out_dt == DT_F32)
        return dequantize_bits<bf16_bits, float>(codes, scales, biases, n, k, gs, bits, out, stream);
    return dequantize_bits<bf16_bits, bf16_bits>(codes, scales, biases, n, k, gs, bits, out, stream);
}

}  // namespace nqk
