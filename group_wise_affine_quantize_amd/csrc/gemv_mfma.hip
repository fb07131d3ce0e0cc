// Matrix-vector family of quantized products on gfx950 matrix cores: few
// activation rows (a launch chunk of up to 32) times the quantized weights,
// for bf16 activations and 4- or 8-bit codes (the routing takes it for
// 4-bit codes only; see gemv_mfma_family).
//
// Method: "Quantization" page of the nuvec documentation -- section "Affine"
// (w ~ scale * code + bias per group; the product is x times the transposed
// weights), section "Products on the GPU" (matrix-vector kernels for few
// rows; split-K for a small output with a long inner dimension; row-exact
// products whose rows equal their one-row products bit for bit) and section
// "Mixture of experts" (each row multiplied by its own expert's weights in
// place).
//
// Per element (activation row m, weight row n) and group g:
//     G = sum_{k in g} x[m, k] * q[n, k]      (matrix cores, fp32)
//     X = sum_{k in g} x[m, k]                (matrix cores, fp32)
//     acc = fma(s[n, g], G, acc);  acc = fma(b[n, g], X, acc)
// in increasing g inside a K slice; the K slices' sums are added in slice
// order.  Codes enter the matrix cores exactly as bf16: 4-bit codes as the
// pairs (128 + q_i, 128 + q_{i+4}) built with one v_and_or_b32 each (then
// G = D - 128 X), 8-bit codes as their byte values.  No element's arithmetic
// depends on the other rows of its launch, on the chunking or on the route
// (plain, batched, per-row gather, grouped gather, left indices), so every
// row has the bits of its one-row product.
//
// Work decomposition (fixed by n, k, group size and the plan's K split S):
//   - A wave owns 32 consecutive weight rows (the B columns of
//     v_mfma_f32_32x32x16_bf16) and one K slice; its A rows are the chunk's
//     activation rows (rows past the chunk are zero).
//   - K is walked in steps of 64: in step s lane (c = l % 32, h = l / 32)
//     holds, for weight row c and activation row c, the 32 elements
//     k = 64 s + 32 h .. + 32 (groups of 64 or more), or the two runs
//     64 s + 16 h .. + 16 and 64 s + 32 + 16 h .. + 16 (groups of 32), so
//     every MFMA's sixteen k lie in one group.
//   - Slice sl takes the units (groups of 128 or steps of 64) from
//     sl * U / S to (sl + 1) * U / S.
#include <algorithm>
#include <type_traits>

#include "nq_device.h"
#include "nq_internal.h"

namespace nqk {

typedef __bf16 mf_bf16x8_t __attribute__((ext_vector_type(8)));
typedef float mf_f32x16_t __attribute__((ext_vector_type(16)));

template <typename ST>
struct MfmaGemvParams {
    const bf16_bits *x;
    bf16_bits *y;
    const uint32_t *codes;
    const ST *scales;
    const ST *biases;
    const uint32_t *idx;
    int64_t rows_per_item, k, n, e;
    int64_t words_per_row, groups_per_row;
    int64_t item0;
    const uint4 *chunks;
    const uint32_t *perm;
    const uint32_t *nchunks;
    const uint32_t *lhs;
    int64_t x_items, lhs_l;
    int gs, ksplit, chunks_per_item, qrows, units;
};

// One K step of a lane, as loaded: raw code words (4 per 4-bit step, 8 per
// 8-bit step, MFMA j using words j or 2j, 2j + 1), the activation row's 32
// elements (16 dwords, MFMA j using dwords 4j .. 4j + 3) and the raw scale /
// bias bits of the step's groups (two for 32-wide groups).
template <int BITS>
struct MfStage {
    uint32_t c[BITS];
    uint32_t x[16];
    uint32_t s[2], b[2];
};

template <typename ST>
__device__ __forceinline__ uint32_t mf_raw(const ST *p, int64_t i)
{
    if constexpr (sizeof(ST) == 2) return (uint32_t)p[i];
    else return __float_as_uint(p[i]);
}

template <typename ST>
__device__ __forceinline__ float mf_f32(uint32_t v)
{
    if constexpr (sizeof(ST) == 2) return __uint_as_float(v << 16);
    else return __uint_as_float(v);
}

// B operand of MFMA j: 4-bit, the pairs (128 + q_i, 128 + q_{i+4}) of code
// word j (element order 0 4 1 5 2 6 3 7); 8-bit, the bf16 values of the
// eight codes of words 2j, 2j + 1 in order.
template <int BITS>
__device__ __forceinline__ mf_bf16x8_t mf_b_operand(const uint32_t *c, int j)
{
    uint4 o;
    if constexpr (BITS == 4) {
        const uint32_t w = c[j];
        o.x = (w & 0x000f000fu) | 0x43004300u;
        o.y = ((w >> 4) & 0x000f000fu) | 0x43004300u;
        o.z = ((w >> 8) & 0x000f000fu) | 0x43004300u;
        o.w = ((w >> 12) & 0x000f000fu) | 0x43004300u;
    } else {
        const uint32_t w0 = c[2 * j], w1 = c[2 * j + 1];
        const float f0 = (float)(w0 & 0xffu), f1 = (float)((w0 >> 8) & 0xffu);
        const float f2 = (float)((w0 >> 16) & 0xffu), f3 = (float)(w0 >> 24);
        const float f4 = (float)(w1 & 0xffu), f5 = (float)((w1 >> 8) & 0xffu);
        const float f6 = (float)((w1 >> 16) & 0xffu), f7 = (float)(w1 >> 24);
        o.x = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
        o.y = __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
        o.z = __builtin_amdgcn_perm(__float_as_uint(f5), __float_as_uint(f4), 0x07060302u);
        o.w = __builtin_amdgcn_perm(__float_as_uint(f7), __float_as_uint(f6), 0x07060302u);
    }
    return __builtin_bit_cast(mf_bf16x8_t, o);
}

// A operand of MFMA j: the activation row's eight elements of that MFMA, in
// the order of the B operand (4-bit: 0 4 1 5 2 6 3 7; 8-bit: as stored).
template <int BITS>
__device__ __forceinline__ mf_bf16x8_t mf_a_operand(const uint32_t *x, int j)
{
    const uint32_t d0 = x[4 * j], d1 = x[4 * j + 1], d2 = x[4 * j + 2], d3 = x[4 * j + 3];
    uint4 o;
    if constexpr (BITS == 4) {
        o.x = __builtin_amdgcn_perm(d2, d0, 0x05040100u);   // (x0, x4)
        o.y = __builtin_amdgcn_perm(d2, d0, 0x07060302u);   // (x1, x5)
        o.z = __builtin_amdgcn_perm(d3, d1, 0x05040100u);   // (x2, x6)
        o.w = __builtin_amdgcn_perm(d3, d1, 0x07060302u);   // (x3, x7)
    } else {
        o = make_uint4(d0, d1, d2, d3);
    }
    return __builtin_bit_cast(mf_bf16x8_t, o);
}

template <int I, int N, typename F>
__device__ __forceinline__ void static_for_mf(F &&f)
{
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for_mf<I + 1, N>(f);
    }
}

template <int BITS, typename ST, int VB, int D, int GS>
__global__ void __launch_bounds__(512) gemv_mfma_kernel(MfmaGemvParams<ST> p)
{
    constexpr int MR = 8 * VB;       // activation rows per launch chunk
    constexpr int NV = 4 * VB;       // accumulator values per lane
    constexpr bool kG32 = GS == 32;
    constexpr int kUps = GS >= 128 ? GS / 64 : 1;   // steps per K unit (and per group when GS >= 64)
    static_assert((D + 1) % kUps == 0, "a round of steps starts on a group boundary");
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int S = p.ksplit;
    const int sl = wave % S;
    const int q = wave / S;
    const int c = lane & 31, h = lane >> 5;
    const int64_t n0 = ((int64_t)blockIdx.x * p.qrows + q) * 32;

    // ---- launch chunk: activation rows, output rows, expert slab (as in the
    // ---- VALU kernels of this family)
    bool live = true;
    int64_t slab = 0;
    int mrows;
    uint32_t first = 0;
    const bf16_bits *xb = p.x;
    bf16_bits *yb = p.y;
    if (p.chunks) {
        if (blockIdx.y >= *p.nchunks) return;   // uniform over the workgroup
        const uint4 ch = p.chunks[blockIdx.y];
        if ((int64_t)ch.x >= p.e) live = false;
        else slab = ch.x;
        first = ch.y;
        mrows = (int)ch.z;
    } else {
        const int64_t item = p.item0 + blockIdx.y / p.chunks_per_item;
        const int64_t r0 = (int64_t)(blockIdx.y % p.chunks_per_item) * MR;
        mrows = (int)min((int64_t)MR, p.rows_per_item - r0);
        int64_t xi = item;
        if (p.lhs) {
            xi = p.lhs[item];
            if (xi >= p.x_items) live = false, xi = 0;   // a zero row; x is never read
        }
        xb = p.x + (xi * p.rows_per_item + r0) * p.k;
        yb = p.y + (item * p.rows_per_item + r0) * p.n;
        if (p.idx) {
            const uint32_t ex = p.idx[item];
            if ((int64_t)ex >= p.e) live = false;
            else slab = ex;
        }
    }
    // this lane's activation row (row c of the chunk; rows past it read row
    // 0 and are zeroed before use)
    const bool xon = c < mrows;
    const int mm = xon ? c : 0;
    const bf16_bits *xrow;
    if (p.chunks) {
        int64_t v = p.perm[first + mm];
        if (p.lhs) {
            const int64_t xi = p.lhs[v / p.lhs_l];
            v = (xi < p.x_items ? xi : 0) * p.lhs_l + v % p.lhs_l;
        }
        xrow = p.x + v * p.k;
    } else {
        xrow = xb + (int64_t)mm * p.k;
    }
    const int64_t wr = min(n0 + c, p.n - 1);   // weight row (rows past n read row n - 1)
    const uint32_t *crow = p.codes + (slab * p.n + wr) * p.words_per_row;
    const ST *srow = p.scales + (slab * p.n + wr) * p.groups_per_row;
    const ST *brow = p.biases + (slab * p.n + wr) * p.groups_per_row;

    // ---- this wave's K slice, in steps of 64
    const int u0 = (int)((int64_t)sl * p.units / S), u1 = (int)((int64_t)(sl + 1) * p.units / S);
    const int s0 = u0 * kUps, ns = (u1 - u0) * kUps;

    auto load = [&](int s, MfStage<BITS> &st) {
        const int64_t kk = (int64_t)(s0 + min(s, max(ns - 1, 0))) * 64;   // past the slice: its last step
        if constexpr (!kG32) {
            const int64_t e0 = kk + 32 * h;
            const uint4 *cs = reinterpret_cast<const uint4 *>(crow + e0 * BITS / 32);
#pragma unroll
            for (int i = 0; i < BITS / 4; ++i) {
                const uint4 v = cs[i];
                st.c[4 * i] = v.x, st.c[4 * i + 1] = v.y, st.c[4 * i + 2] = v.z, st.c[4 * i + 3] = v.w;
            }
            // only lanes of the chunk's rows read activations (the others
            // feed zeros and fetch nothing)
            if (xon) {
                const uint4 *xs = reinterpret_cast<const uint4 *>(xrow + e0);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint4 v = xs[i];
                    st.x[4 * i] = v.x, st.x[4 * i + 1] = v.y, st.x[4 * i + 2] = v.z, st.x[4 * i + 3] = v.w;
                }
            } else {
#pragma unroll
                for (int i = 0; i < 16; ++i) st.x[i] = 0u;
            }
            const int64_t g = e0 / GS;
            st.s[0] = mf_raw(srow, g);
            st.b[0] = mf_raw(brow, g);
        } else {
#pragma unroll
            for (int r = 0; r < 2; ++r) {   // run r: k = kk + 32 r + 16 h .. + 16 (group 2 s + r)
                const int64_t e0 = kk + 32 * r + 16 * h;
                if constexpr (BITS == 4) {
                    const uint2 v = *reinterpret_cast<const uint2 *>(crow + e0 / 8);
                    st.c[2 * r] = v.x, st.c[2 * r + 1] = v.y;
                } else {
                    const uint4 v = *reinterpret_cast<const uint4 *>(crow + e0 / 4);
                    st.c[4 * r] = v.x, st.c[4 * r + 1] = v.y, st.c[4 * r + 2] = v.z, st.c[4 * r + 3] = v.w;
                }
                if (xon) {
                    const uint4 *xs = reinterpret_cast<const uint4 *>(xrow + e0);
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        const uint4 v = xs[i];
                        st.x[8 * r + 4 * i] = v.x, st.x[8 * r + 4 * i + 1] = v.y;
                        st.x[8 * r + 4 * i + 2] = v.z, st.x[8 * r + 4 * i + 3] = v.w;
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 8; ++i) st.x[8 * r + i] = 0u;
                }
                st.s[r] = mf_raw(srow, e0 / 32);
                st.b[r] = mf_raw(brow, e0 / 32);
            }
        }
    };

    float acc[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) acc[v] = 0.0f;
    mf_f32x16_t dq = {}, dx = {};   // running group sums: x * codes, x
    const mf_bf16x8_t ones = __builtin_bit_cast(mf_bf16x8_t, make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u));

    // one group's sums into the accumulators (values v < NV: rows
    // 8 (v / 4) + 4 h + v % 4)
    auto finish_group = [&](uint32_t sraw, uint32_t braw) {
        const float sc = mf_f32<ST>(sraw), bi = mf_f32<ST>(braw);
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const float X = dx[v];
            const float G = BITS == 4 ? fmaf(-128.0f, X, dq[v]) : dq[v];
            acc[v] = fmaf(sc, G, acc[v]);
            acc[v] = fmaf(bi, X, acc[v]);
        }
    };

    // MFMA j of a step; FRESH starts a group's sums.  Lanes of rows past the
    // chunk feed zeros.
    auto mfma = [&](const MfStage<BITS> &st, int j, auto fresh) {
        constexpr bool FRESH = decltype(fresh)::value;
        const mf_bf16x8_t a = mf_a_operand<BITS>(st.x, j);   // zeros past the chunk's rows
        const mf_bf16x8_t bq = mf_b_operand<BITS>(st.c, j);
        const mf_f32x16_t z = {};
        dq = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bq, FRESH ? z : dq, 0, 0, 0);
        dx = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, ones, FRESH ? z : dx, 0, 0, 0);
    };
    using yes = std::true_type;
    using no = std::false_type;

    // step number i of a round (rounds start on group boundaries)
    auto compute = [&](auto ii, const MfStage<BITS> &st) {
        constexpr int I = decltype(ii)::value;
        if constexpr (kG32) {
            mfma(st, 0, yes{});
            mfma(st, 1, no{});
            finish_group(st.s[0], st.b[0]);
            mfma(st, 2, yes{});
            mfma(st, 3, no{});
            finish_group(st.s[1], st.b[1]);
        } else {
            if constexpr (I % kUps == 0) mfma(st, 0, yes{});
            else mfma(st, 0, no{});
            mfma(st, 1, no{});
            mfma(st, 2, no{});
            mfma(st, 3, no{});
            if constexpr ((I + 1) % kUps == 0) finish_group(st.s[0], st.b[0]);
        }
    };

    // steps in rounds of D + 1: every load of a round is issued before the
    // first of its steps is computed; loads past the slice re-read its last
    // step and are not computed
    if (live && ns > 0) {
        MfStage<BITS> st[D + 1];
#pragma unroll
        for (int i = 0; i < D; ++i) load(i, st[i]);
        for (int base = 0; base < ns; base += D + 1) {
            static_for_mf<0, D + 1>([&](auto ii) {
                constexpr int I = decltype(ii)::value;
                const int s = base + I;
                load(s + D, st[(I + D) % (D + 1)]);
                __builtin_amdgcn_sched_barrier(0);
                if (s < ns) compute(ii, st[I]);
                __builtin_amdgcn_sched_barrier(0);
            });
        }
    }

    // ---- slices added in slice order, then stored (rows past the chunk and
    // ---- past n are not stored)
    auto store = [&](const float *vals) {
        const bool col_ok = n0 + c < p.n;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int m = 8 * (v >> 2) + 4 * h + (v & 3);
            if (col_ok && m < mrows) {
                bf16_bits *yr = p.chunks ? p.y + (int64_t)p.perm[first + m] * p.n : yb + (int64_t)m * p.n;
                Elt<bf16_bits>::store(yr, n0 + c, vals[v]);
            }
        }
    };
    if (S == 1) {
        store(acc);
        return;
    }
    extern __shared__ float part[];   // [wave][NV][64]
#pragma unroll
    for (int v = 0; v < NV; ++v) part[(wave * NV + v) * 64 + lane] = acc[v];
    __syncthreads();
    if (sl != 0) return;
    float tot[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        tot[v] = part[((q * S) * NV + v) * 64 + lane];
        for (int s2 = 1; s2 < S; ++s2) tot[v] += part[((q * S + s2) * NV + v) * 64 + lane];
    }
    store(tot);
}

namespace {

constexpr int kMfMaxGridY = 65535;

template <int BITS, typename ST, int VB>
hipError_t gemv_mfma_run(const GemvLaunch &a, hipStream_t stream)
{
    MfmaGemvParams<ST> p;
    p.x = static_cast<const bf16_bits *>(a.x);
    p.y = static_cast<bf16_bits *>(a.y);
    p.codes = a.codes;
    p.scales = static_cast<const ST *>(a.scales);
    p.biases = static_cast<const ST *>(a.biases);
    p.idx = a.idx;
    p.chunks = reinterpret_cast<const uint4 *>(a.chunks);
    p.perm = a.perm;
    p.nchunks = a.nchunks;
    p.lhs = a.lhs;
    p.x_items = a.x_items;
    p.lhs_l = a.lhs_l;
    p.rows_per_item = a.rows_per_item;
    p.k = a.k;
    p.n = a.n;
    p.e = a.e;
    p.words_per_row = a.k * BITS / 32;
    p.groups_per_row = a.k / a.gs;
    p.gs = a.gs;
    p.ksplit = a.ksplit;
    p.units = (int)(a.gs >= 128 ? a.k / a.gs : a.k / 64);
    constexpr int MR = 8 * VB;
    p.chunks_per_item = (int)((a.rows_per_item + MR - 1) / MR);
    // row groups per workgroup: 8 waves when the split allows it
    p.qrows = a.ksplit >= 8 ? 1 : 8 / a.ksplit;
    const int threads = 64 * a.ksplit * p.qrows;
    const size_t lds = a.ksplit > 1 ? (size_t)threads / 64 * 4 * VB * 64 * sizeof(float) : 0;
    const int64_t rows_per_block = (int64_t)p.qrows * 32;
    const unsigned gx = (unsigned)((a.n + rows_per_block - 1) / rows_per_block);
    constexpr int D = 3;
    auto go = [&](dim3 grid) {
        switch (a.gs) {
        case 32: gemv_mfma_kernel<BITS, ST, VB, D, 32><<<grid, dim3(threads), lds, stream>>>(p); break;
        case 64: gemv_mfma_kernel<BITS, ST, VB, D, 64><<<grid, dim3(threads), lds, stream>>>(p); break;
        default: gemv_mfma_kernel<BITS, ST, VB, D, 128><<<grid, dim3(threads), lds, stream>>>(p); break;
        }
        return hipGetLastError();
    };
    if (a.chunks) {
        if (a.max_chunks > kMfMaxGridY) return hipErrorInvalidValue;
        p.item0 = 0;
        return go(dim3(gx, (unsigned)a.max_chunks));
    }
    const int64_t items_per_launch = std::max<int64_t>(1, kMfMaxGridY / p.chunks_per_item);
    for (int64_t i0 = 0; i0 < a.items; i0 += items_per_launch) {
        const int64_t cnt = std::min(items_per_launch, a.items - i0);
        p.item0 = i0;
        if (hipError_t err = go(dim3(gx, (unsigned)(cnt * p.chunks_per_item)))) return err;
    }
    return hipSuccess;
}

template <int BITS, typename ST>
hipError_t gemv_mfma_rows(const GemvLaunch &a, hipStream_t stream)
{
    // launch chunks of up to 8, 16 or 32 rows (the chunking never changes a
    // row's arithmetic)
    const int64_t rows = a.chunks ? a.max_rows : a.rows_per_item;
    if (rows <= 8) return gemv_mfma_run<BITS, ST, 1>(a, stream);
    if (rows <= 16) return gemv_mfma_run<BITS, ST, 2>(a, stream);
    return gemv_mfma_run<BITS, ST, 4>(a, stream);
}

}  // namespace

bool gemv_mfma_family(int64_t n, int64_t k, int gs, int bits, int x_dt)
{
    // Measured choice (the arithmetic differs, so it is made by shape only):
    // 4-bit codes with k <= 4096 below the streaming shapes take the matrix
    // cores (the 32-vector chunks of the row-exact expert gather: 76.6 us
    // against 104 us at 512 x [32, 1408, 2048]); a long K over few weight rows
    // splits better in the VALU kernels' 2048-wide steps (split-K [4, 14336]
    // x [1024, 14336]: 7.8 us against 41 us), and 8-bit codes lose on this
    // kernel's B-operand loads, which spread each instruction over 32 weight
    // rows (x [8, 4096] x [4096, 4096]: 12.4 us VALU against 16.4 us).
    if (x_dt != DT_BF16 || bits != 4 || k < 64 || k % 64 != 0 || k > 4096) return false;
    if (gs != 32 && gs != 64 && gs != 128) return false;
    return n < 8 * 1024;
}

hipError_t launch_gemv_mfma(const GemvLaunch &a, hipStream_t stream)
{
    if (a.ksplit < 1 || a.ksplit > 8) return hipErrorInvalidValue;
    if (a.bits == 4) {
        if (a.sb_dt == DT_F32) return gemv_mfma_rows<4, float>(a, stream);
        return gemv_mfma_rows<4, bf16_bits>(a, stream);
    }
    if (a.sb_dt == DT_F32) return gemv_mfma_rows<8, float>(a, stream);
    return gemv_mfma_rows<8, bf16_bits>(a, stream);
}

}  // namespace nqk
