// Matrix-vector family of quantized products for gfx950: decode GEMV (1 row),
// few-row GEMV (up to 8 rows per launch chunk), split-K and the per-row
// mixture-of-experts gather.  All four are one kernel.
//
// Method: "Quantization" page of the nuvec documentation -- section "Affine"
// (w ~ scale * code + bias per group; the product is x times the transposed
// weights), section "Products on the GPU" (matrix-vector kernels for few rows,
// split-K for a small output with a long inner dimension, row-exact products
// whose rows equal their one-row products bit for bit) and section "Mixture
// of experts" (each row multiplied by the weights of its own expert, without
// gathering them).
//
// Work decomposition (all of it fixed by n, k, bits, group size and dtypes):
//   - K is walked in steps of 2048 elements; in a step lane L of a wave owns
//     the 32-element lane chunk [2048*t + 32*L, +32), i.e. `bits` consecutive
//     code words, which always lie inside one group.
//   - A wave owns RW consecutive output rows (weight rows) and accumulates
//     MR activation rows at once; each weight word is read once for all MR
//     rows.
//   - Split-K: the `ksplit` (<= 8) waves of a workgroup take the steps t = s,
//     s + ksplit, ...; their per-wave sums are added in LDS in wave order.
//   - Per lane chunk the group factorisation is used:
//         sum_k x_k (s q_k + b) = s * sum_k x_k q_k + b * sum_k x_k,
//     so the dequantized weight is never formed.
//   - The 64 lane partials are combined by a fixed xor butterfly.
// Nothing in a row's arithmetic depends on MR, on the other rows or on the
// launch chunking, so every row of a batched call is bit-equal to its
// one-row call.  There are no atomics; results are run-to-run identical.
//
// 4-bit codes with bf16 activations use v_dot2_f32_bf16: two codes are turned
// into the bf16 pair (128 + q_a, 128 + q_b) with one and-or (128 + q is exact
// in bf16 for q < 128), dotted with the matching activation pair, and the
// 128 * sum(x) offset is removed once per lane chunk.  Other cases convert
// codes to fp32 and use fp32 FMAs.
#include <algorithm>

#include "nq_device.h"
#include "nq_internal.h"

namespace nqk {

template <typename XT, typename ST>
struct GemvParams {
    const XT *x;
    XT *y;
    const uint32_t *codes;
    const ST *scales;
    const ST *biases;
    const uint32_t *idx;
    int64_t rows_per_item, k, n, e;
    int64_t words_per_row, groups_per_row;
    int64_t item0;          // first item of this launch (items are split over launches)
    int gs, ksplit, steps, chunks_per_item, qrows;   // qrows: row groups per workgroup
};

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c)
{
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), c, false);
}

template <int BITS>
__device__ __forceinline__ void load_chunk_words(const uint32_t *src, uint32_t *wd)
{
    if constexpr (BITS % 4 == 0) {
#pragma unroll
        for (int i = 0; i < BITS / 4; ++i) {
            typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
            u32x4_t d = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(src) + i);
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

template <int BITS, int RW>
struct Stage {
    uint32_t cw[RW][BITS];
    float s[RW], b[RW];
};

template <int BITS, typename XT, typename ST, int MR, int RW>
__global__ void __launch_bounds__(512) gemv_kernel(GemvParams<XT, ST> p)
{
    constexpr bool kMagic = (BITS == 4) && (sizeof(XT) == 2);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int S = p.ksplit;
    const int sl = wave % S;            // K slice of this wave
    const int q = wave / S;             // row group of this wave inside the workgroup
    const int64_t n0 = ((int64_t)blockIdx.x * p.qrows + q) * RW;

    const int64_t item = p.item0 + blockIdx.y / p.chunks_per_item;
    const int64_t r0 = (int64_t)(blockIdx.y % p.chunks_per_item) * MR;
    const int mrows = (int)min((int64_t)MR, p.rows_per_item - r0);
    const XT *xb = p.x + (item * p.rows_per_item + r0) * p.k;
    XT *yb = p.y + (item * p.rows_per_item + r0) * p.n;

    bool live = true;
    int64_t slab = 0;
    if (p.idx) {
        const uint32_t ex = p.idx[item];
        if ((int64_t)ex >= p.e) live = false;
        else slab = ex;
    }
    const uint32_t *cb = p.codes + slab * p.n * p.words_per_row;
    const ST *sb = p.scales + slab * p.n * p.groups_per_row;
    const ST *bb = p.biases + slab * p.n * p.groups_per_row;

    float acc[MR][RW];
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int r = 0; r < RW; ++r) acc[m][r] = 0.0f;

    auto load_stage = [&](int t, Stage<BITS, RW> &st) {
        const int64_t e0 = (int64_t)t * kStepElems + lane * kLaneChunk;
        const bool on = e0 < p.k;
        const int64_t g = on ? e0 / p.gs : 0;
#pragma unroll
        for (int r = 0; r < RW; ++r) {
            const int64_t nr = n0 + r;
            if (on && nr < p.n) {
                load_chunk_words<BITS>(cb + nr * p.words_per_row + e0 * BITS / 32, st.cw[r]);
                st.s[r] = Elt<ST>::load(sb, nr * p.groups_per_row + g);
                st.b[r] = Elt<ST>::load(bb, nr * p.groups_per_row + g);
            } else {
#pragma unroll
                for (int i = 0; i < BITS; ++i) st.cw[r][i] = 0u;
                st.s[r] = 0.0f;
                st.b[r] = 0.0f;
            }
        }
    };

    auto compute_stage = [&](int t, const Stage<BITS, RW> &st) {
        const int64_t e0 = (int64_t)t * kStepElems + lane * kLaneChunk;
        if (e0 >= p.k) return;
        const XT *xl = xb + e0;
        float X[MR];
        float D[MR][RW];
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            X[m] = 0.0f;
#pragma unroll
            for (int r = 0; r < RW; ++r) D[m][r] = 0.0f;
        }
        if constexpr (kMagic) {
            constexpr uint32_t kOnes = 0x3f803f80u;   // bf16 pair (1, 1)
#pragma unroll
            for (int j = 0; j < 4; ++j) {             // word j: elements 8j .. 8j+7
                uint32_t xp[MR][4];
#pragma unroll
                for (int m = 0; m < MR; ++m) {
                    uint4 xv = make_uint4(0u, 0u, 0u, 0u);
                    if (m < mrows) xv = *reinterpret_cast<const uint4 *>(xl + m * p.k + 8 * j);
                    // pairs (x0,x4) (x1,x5) (x2,x6) (x3,x7), matching the code pairs below
                    xp[m][0] = __builtin_amdgcn_perm(xv.z, xv.x, 0x05040100u);
                    xp[m][1] = __builtin_amdgcn_perm(xv.z, xv.x, 0x07060302u);
                    xp[m][2] = __builtin_amdgcn_perm(xv.w, xv.y, 0x05040100u);
                    xp[m][3] = __builtin_amdgcn_perm(xv.w, xv.y, 0x07060302u);
                    X[m] = dot2_bf16(xv.x, kOnes, X[m]);
                    X[m] = dot2_bf16(xv.y, kOnes, X[m]);
                    X[m] = dot2_bf16(xv.z, kOnes, X[m]);
                    X[m] = dot2_bf16(xv.w, kOnes, X[m]);
                }
#pragma unroll
                for (int r = 0; r < RW; ++r) {
                    const uint32_t w = st.cw[r][j];
                    // bf16 pairs (128 + q_i, 128 + q_{i+4}), i = 0..3
                    const uint32_t q0 = (w & 0x000f000fu) | 0x43004300u;
                    const uint32_t q1 = ((w >> 4) & 0x000f000fu) | 0x43004300u;
                    const uint32_t q2 = ((w >> 8) & 0x000f000fu) | 0x43004300u;
                    const uint32_t q3 = ((w >> 12) & 0x000f000fu) | 0x43004300u;
#pragma unroll
                    for (int m = 0; m < MR; ++m) {
                        D[m][r] = dot2_bf16(xp[m][0], q0, D[m][r]);
                        D[m][r] = dot2_bf16(xp[m][1], q1, D[m][r]);
                        D[m][r] = dot2_bf16(xp[m][2], q2, D[m][r]);
                        D[m][r] = dot2_bf16(xp[m][3], q3, D[m][r]);
                    }
                }
            }
#pragma unroll
            for (int m = 0; m < MR; ++m)
#pragma unroll
                for (int r = 0; r < RW; ++r) D[m][r] = fmaf(-128.0f, X[m], D[m][r]);
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {             // elements 8j .. 8j+7
                float xf[MR][8];
#pragma unroll
                for (int m = 0; m < MR; ++m) {
                    if constexpr (sizeof(XT) == 2) {
                        uint4 xv = make_uint4(0u, 0u, 0u, 0u);
                        if (m < mrows) xv = *reinterpret_cast<const uint4 *>(xl + m * p.k + 8 * j);
                        const uint32_t d[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            xf[m][2 * i] = __uint_as_float(d[i] << 16);
                            xf[m][2 * i + 1] = __uint_as_float(d[i] & 0xffff0000u);
                        }
                    } else {
                        uint4 a = make_uint4(0u, 0u, 0u, 0u), b = a;
                        if (m < mrows) {
                            a = *reinterpret_cast<const uint4 *>(xl + m * p.k + 8 * j);
                            b = *reinterpret_cast<const uint4 *>(xl + m * p.k + 8 * j + 4);
                        }
                        xf[m][0] = __uint_as_float(a.x), xf[m][1] = __uint_as_float(a.y);
                        xf[m][2] = __uint_as_float(a.z), xf[m][3] = __uint_as_float(a.w);
                        xf[m][4] = __uint_as_float(b.x), xf[m][5] = __uint_as_float(b.y);
                        xf[m][6] = __uint_as_float(b.z), xf[m][7] = __uint_as_float(b.w);
                    }
#pragma unroll
                    for (int i = 0; i < 8; ++i) X[m] += xf[m][i];
                }
#pragma unroll
                for (int r = 0; r < RW; ++r) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const float qf = (float)code_at<BITS>(st.cw[r], 8 * j + i);
#pragma unroll
                        for (int m = 0; m < MR; ++m) D[m][r] = fmaf(xf[m][i], qf, D[m][r]);
                    }
                }
            }
        }
#pragma unroll
        for (int m = 0; m < MR; ++m)
#pragma unroll
            for (int r = 0; r < RW; ++r) {
                acc[m][r] = fmaf(st.s[r], D[m][r], acc[m][r]);
                acc[m][r] = fmaf(st.b[r], X[m], acc[m][r]);
            }
    };

    if (live) {
        Stage<BITS, RW> cur, nxt;
        int t = sl;
        if (t < p.steps) load_stage(t, cur);
        for (; t < p.steps; t += S) {
            if (t + S < p.steps) load_stage(t + S, nxt);
            compute_stage(t, cur);
            cur = nxt;
        }
    }

    // Fixed xor butterfly: every lane ends with the same, order-fixed total.
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int r = 0; r < RW; ++r) {
            float v = acc[m][r];
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
            acc[m][r] = v;
        }

    // Lane m*RW + r holds output (m, r).
    float mine = 0.0f;
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int r = 0; r < RW; ++r)
            if (lane == m * RW + r) mine = acc[m][r];

    const int mi = lane / RW, ri = lane % RW;
    const bool writer = lane < MR * RW && mi < mrows && n0 + ri < p.n;
    if (S == 1) {
        if (writer) Elt<XT>::store(yb, (int64_t)mi * p.n + n0 + ri, mine);
        return;
    }
    __shared__ float part[8 * MR * RW];
    if (lane < MR * RW) part[wave * MR * RW + lane] = mine;
    __syncthreads();
    if (sl == 0 && writer) {
        float tot = part[(q * S) * MR * RW + lane];
        for (int s2 = 1; s2 < S; ++s2) tot += part[(q * S + s2) * MR * RW + lane];
        Elt<XT>::store(yb, (int64_t)mi * p.n + n0 + ri, tot);
    }
}

namespace {

constexpr int kMaxGridY = 65535;

template <int BITS, typename XT, typename ST, int MR>
hipError_t gemv_mr(const GemvLaunch &a, hipStream_t stream)
{
    constexpr int RW = 4;
    if (a.rows_per_wave != RW) return hipErrorInvalidValue;
    GemvParams<XT, ST> p;
    p.x = static_cast<const XT *>(a.x);
    p.y = static_cast<XT *>(a.y);
    p.codes = a.codes;
    p.scales = static_cast<const ST *>(a.scales);
    p.biases = static_cast<const ST *>(a.biases);
    p.idx = a.idx;
    p.rows_per_item = a.rows_per_item;
    p.k = a.k;
    p.n = a.n;
    p.e = a.e;
    p.words_per_row = a.k * BITS / 32;
    p.groups_per_row = a.k / a.gs;
    p.gs = a.gs;
    p.ksplit = a.ksplit;
    p.steps = (int)((a.k + kStepElems - 1) / kStepElems);
    p.chunks_per_item = (int)((a.rows_per_item + MR - 1) / MR);
    p.qrows = a.ksplit >= 4 ? 1 : 4 / a.ksplit;
    const int threads = 64 * a.ksplit * p.qrows;
    const int64_t rows_per_block = (int64_t)p.qrows * RW;
    const unsigned gx = (unsigned)((a.n + rows_per_block - 1) / rows_per_block);
    const int64_t items_per_launch = std::max<int64_t>(1, kMaxGridY / p.chunks_per_item);
    for (int64_t i0 = 0; i0 < a.items; i0 += items_per_launch) {
        const int64_t cnt = std::min(items_per_launch, a.items - i0);
        p.item0 = i0;
        gemv_kernel<BITS, XT, ST, MR, RW>
            <<<dim3(gx, (unsigned)(cnt * p.chunks_per_item)), dim3(threads), 0, stream>>>(p);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

template <int BITS, typename XT, typename ST>
hipError_t gemv_bits(const GemvLaunch &a, hipStream_t stream)
{
    const int64_t mr = std::min<int64_t>(a.rows_per_item, 8);
    if (mr <= 1) return gemv_mr<BITS, XT, ST, 1>(a, stream);
    if (mr <= 2) return gemv_mr<BITS, XT, ST, 2>(a, stream);
    if (mr <= 4) return gemv_mr<BITS, XT, ST, 4>(a, stream);
    return gemv_mr<BITS, XT, ST, 8>(a, stream);
}

template <typename XT, typename ST>
hipError_t gemv_dt(const GemvLaunch &a, hipStream_t stream)
{
    switch (a.bits) {
    case 4: return gemv_bits<4, XT, ST>(a, stream);
    case 8: return gemv_bits<8, XT, ST>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_gemv(const GemvLaunch &a, hipStream_t stream)
{
    if (a.ksplit < 1 || a.ksplit > 8) return hipErrorInvalidValue;
    if (a.x_dt == DT_F32) {
        if (a.sb_dt == DT_F32) return gemv_dt<float, float>(a, stream);
        return gemv_dt<float, bf16_bits>(a, stream);
    }
    if (a.sb_dt == DT_F32) return gemv_dt<bf16_bits, float>(a, stream);
    return gemv_dt<bf16_bits, bf16_bits>(a, stream);
}

}  // namespace nqk
