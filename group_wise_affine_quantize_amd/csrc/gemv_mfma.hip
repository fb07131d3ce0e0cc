// Matrix-vector family of quantized products on gfx950 matrix cores: few
// activation rows times the quantized weights, for bf16 activations.  Two
// kernels: gemv_mfma_kernel (launch chunks of up to 32 rows, 32 weight rows
// per wave; the routing takes it for 4-bit codes, see gemv_mfma_family) and
// gemv_band_kernel (8-bit codes; bands of 16 weight rows staged whole in
// LDS, see gemv_band_family).
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
typedef float mf_f32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

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

// ---------------------------------------------------------------------------
// 8-bit codes: one band of 16 weight rows per workgroup, staged whole in LDS.
//
// Per element (activation row m, weight row n), group g and K quarter w:
//     G = sum_{k in g} x[m, k] * q[n, k]     (v_mfma_f32_16x16x32_bf16, fp32)
//     X = sum_{k in g} x[m, k]               (the same instruction against ones)
//     acc_w = fma(s[n, g], G, acc_w);  acc_w = fma(b[n, g], X, acc_w)
// in increasing g inside quarter w (of the four equal K quarters), and
// y = ((acc_0 + acc_1) + acc_2) + acc_3.  The codes enter the matrix cores
// as their exact bf16 values.  Inside a group, MFMA j of lane group h takes
// k = 32 j + 8 h .. + 8 of the quarter: every instruction's 32 k lie in one
// group.  Nothing depends on the other rows of the launch chunk (up to 8
// activation rows; MFMA rows 8..15 are computed and not stored), so every
// row keeps the bits of its one-row product on every route.
//
// Work decomposition: workgroup (band, launch chunk); its 4 waves take the K
// quarters.  Each wave issues all of its loads at once, as direct-to-LDS
// loads of whole 16-byte chunks: the codes of its 16 rows (every
// instruction 1 KB of consecutive chunks, a row's quarter in 256-byte
// stages), the chunk's activations of its quarter and the quarter's scales
// and biases.  Chunk q of row r is written to slot q ^ (r mod 16) of its
// stage, so the B-operand reads (16 rows of one chunk column) and the
// A-operand reads spread over all banks.  Stage t is computed after a
// counted wait for its own loads; later stages stay in flight.
constexpr int kBandRows = 16;        // weight rows per workgroup (MFMA columns)
constexpr int kBandVectors = 8;      // activation rows per launch chunk
constexpr int kBandStageK = 256;     // K per stage
constexpr int kBandMaxK = 4096;

template <typename ST, int GPQ>
constexpr int band_sb_loads() { return (kBandRows * GPQ * (int)sizeof(ST) + 255) / 256; }

template <typename ST, int GS, int NST, bool SBLDS>
__global__ void __launch_bounds__(256) gemv_band_kernel(MfmaGemvParams<ST> p)
{
    constexpr int KQ = NST * kBandStageK;            // K per wave (quarter)
    constexpr int RBS = kBandStageK;                 // code bytes per row and stage (8-bit)
    constexpr int CPS = RBS / 16;                    // 16-byte chunks per row and stage
    constexpr int NIC = kBandRows * RBS / 1024;      // code loads per stage
    constexpr int XCS = kBandStageK * 2 / 16;        // activation chunks per row and stage
    constexpr int NIX = kBandVectors * XCS / 64;     // activation loads per stage
    constexpr int GPQ = KQ / GS;                     // groups per quarter
    constexpr int SBW = (int)sizeof(ST) / 2;         // scale words (16-bit) per group
    constexpr int NSB = band_sb_loads<ST, GPQ>();    // scale (and bias) loads
    constexpr int L = NIC + NIX;
    static_assert(CPS >= kBandRows, "the swizzle stays inside a stage");
    static_assert((NST - 1) * L < 64, "vmcnt");
    static_assert(GPQ * (int)sizeof(ST) >= 4, "scale runs of whole dwords");
    __shared__ __attribute__((aligned(16))) uint8_t c_lds[4][kBandRows * KQ];
    __shared__ __attribute__((aligned(16))) uint8_t x_lds[4][kBandVectors * KQ * 2];
    __shared__ __attribute__((aligned(16))) uint8_t s_lds[4][NSB * 256];
    __shared__ __attribute__((aligned(16))) uint8_t b_lds[4][NSB * 256];
    __shared__ mf_f32x4_t part[3][64];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t n0 = (int64_t)blockIdx.x * kBandRows;
    const int64_t k0 = (int64_t)wave * KQ;
    const int c = lane & 15, h = lane >> 4;

    // ---- launch chunk (as in the kernel above)
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
        const int64_t r0 = (int64_t)(blockIdx.y % p.chunks_per_item) * kBandVectors;
        mrows = (int)min((int64_t)kBandVectors, p.rows_per_item - r0);
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
    auto x_row = [&](int r) -> const bf16_bits * {   // r < mrows
        if (p.chunks) {
            int64_t v = p.perm[first + r];
            if (p.lhs) {
                const int64_t xi = p.lhs[v / p.lhs_l];
                v = (xi < p.x_items ? xi : 0) * p.lhs_l + v % p.lhs_l;
            }
            return p.x + v * p.k;
        }
        return xb + (int64_t)r * p.k;
    };

    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (live) {
#if defined(__HIP_DEVICE_COMPILE__)
        // scales and biases of the quarter (4-byte aligned rows): lane t of
        // load i -> row t / DPR, dword t % DPR
        if constexpr (SBLDS) {
            constexpr int DPR = GPQ * (int)sizeof(ST) / 4;
#pragma unroll
            for (int i = 0; i < NSB; ++i) {
                const int t = i * 64 + lane;
                const int r = min(t / DPR, kBandRows - 1), d = t % DPR;
                const int64_t row = slab * p.n + min(n0 + r, p.n - 1);
                const int64_t off = row * p.groups_per_row + k0 / GS + d * (4 / (int)sizeof(ST));
                __builtin_amdgcn_global_load_lds((const void *)(p.scales + off), (lds_void_t *)&s_lds[wave][i * 256], 4, 0, 0);
                __builtin_amdgcn_global_load_lds((const void *)(p.biases + off), (lds_void_t *)&b_lds[wave][i * 256], 4, 0, 0);
            }
        }
        // activation rows of this lane's loads (rows past the chunk read row 0)
        const bf16_bits *xsrc[NIX];
#pragma unroll
        for (int i = 0; i < NIX; ++i) {
            const int r = (i * 64 + lane) / XCS;
            xsrc[i] = x_row(r < mrows ? r : 0) + k0;
        }
        const uint8_t *csrc = reinterpret_cast<const uint8_t *>(p.codes) + k0;
#pragma unroll
        for (int st = 0; st < NST; ++st) {
#pragma unroll
            for (int i = 0; i < NIC; ++i) {
                const int t = i * 64 + lane;
                const int r = t / CPS, sl = t % CPS;
                const int q = sl ^ (r & (kBandRows - 1));   // the chunk that goes to slot sl
                const int64_t row = slab * p.n + min(n0 + r, p.n - 1);
                __builtin_amdgcn_global_load_lds((const void *)(csrc + row * p.words_per_row * 4 + (int64_t)(st * CPS + q) * 16),
                                                 (lds_void_t *)&c_lds[wave][st * kBandRows * RBS + i * 1024], 16, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < NIX; ++i) {
                const int t = i * 64 + lane;
                const int r = t / XCS, sl = t % XCS;
                const int q = sl ^ (r & (kBandRows - 1));
                __builtin_amdgcn_global_load_lds((const void *)(xsrc[i] + (int64_t)(st * XCS + q) * 8),
                                                 (lds_void_t *)&x_lds[wave][st * kBandVectors * XCS * 16 + i * 1024], 16, 0, 0);
            }
        }
#else
        (void)x_row;
#endif
        mf_f32x4_t dq = {}, dx = {};
        const uint32_t onew = 0x3f803f80u;
        const mf_bf16x8_t ones = __builtin_bit_cast(mf_bf16x8_t, make_uint4(onew, onew, onew, onew));
        const int xr = c & (kBandVectors - 1);   // MFMA rows 8..15 repeat rows 0..7 (not stored)
        const uint16_t *ss = reinterpret_cast<const uint16_t *>(&s_lds[wave][0]);
        const uint16_t *bs = reinterpret_cast<const uint16_t *>(&b_lds[wave][0]);
        static_for_mf<0, NST>([&](auto stt) {
            constexpr int ST_ = decltype(stt)::value;
            constexpr int after = (NST - 1 - ST_) * L;   // loads issued after this stage's
            __builtin_amdgcn_s_waitcnt((after & 15) | ((after >> 4) << 14) | (0x7 << 4) | (0xf << 8));
            asm volatile("" ::: "memory");
            const uint8_t *cs = &c_lds[wave][ST_ * kBandRows * RBS];
            const uint8_t *xs = &x_lds[wave][ST_ * kBandVectors * XCS * 16];
            constexpr int NJ = kBandStageK / 32;
            uint2 braw[NJ];
            uint4 araw[NJ];
#pragma unroll
            for (int j = 0; j < NJ; ++j) {   // all of the stage's operands first
                const int byte = 32 * j + 8 * h;
                braw[j] = *reinterpret_cast<const uint2 *>(cs + c * RBS + 16 * ((byte >> 4) ^ c) + (byte & 15));
                araw[j] = *reinterpret_cast<const uint4 *>(xs + xr * XCS * 16 + 16 * ((4 * j + h) ^ xr));
            }
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int kk = ST_ * kBandStageK + 32 * j;   // inside the quarter
                const uint2 w = braw[j];
                const float f0 = (float)(w.x & 0xffu), f1 = (float)((w.x >> 8) & 0xffu);
                const float f2 = (float)((w.x >> 16) & 0xffu), f3 = (float)(w.x >> 24);
                const float f4 = (float)(w.y & 0xffu), f5 = (float)((w.y >> 8) & 0xffu);
                const float f6 = (float)((w.y >> 16) & 0xffu), f7 = (float)(w.y >> 24);
                uint4 b;
                b.x = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
                b.y = __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
                b.z = __builtin_amdgcn_perm(__float_as_uint(f5), __float_as_uint(f4), 0x07060302u);
                b.w = __builtin_amdgcn_perm(__float_as_uint(f7), __float_as_uint(f6), 0x07060302u);
                const mf_bf16x8_t av = __builtin_bit_cast(mf_bf16x8_t, araw[j]);
                const mf_bf16x8_t bv = __builtin_bit_cast(mf_bf16x8_t, b);
                const bool fresh = (kk % GS) == 0;
                const mf_f32x4_t z = {};
                dq = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, fresh ? z : dq, 0, 0, 0);
                dx = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, ones, fresh ? z : dx, 0, 0, 0);
                if ((kk + 32) % GS == 0) {
                    const int gi = kk / GS;
                    uint32_t sr, br;
                    if constexpr (!SBLDS) {   // read in place: the same values
                        const int64_t at = (slab * p.n + min(n0 + c, p.n - 1)) * p.groups_per_row + (k0 + kk) / GS;
                        sr = sizeof(ST) == 2 ? (uint32_t)reinterpret_cast<const uint16_t *>(p.scales)[at] << 16
                                             : reinterpret_cast<const uint32_t *>(p.scales)[at];
                        br = sizeof(ST) == 2 ? (uint32_t)reinterpret_cast<const uint16_t *>(p.biases)[at] << 16
                                             : reinterpret_cast<const uint32_t *>(p.biases)[at];
                    } else if constexpr (SBW == 1) {
                        sr = (uint32_t)ss[c * GPQ + gi] << 16;
                        br = (uint32_t)bs[c * GPQ + gi] << 16;
                    } else {
                        sr = reinterpret_cast<const uint32_t *>(ss)[c * GPQ + gi];
                        br = reinterpret_cast<const uint32_t *>(bs)[c * GPQ + gi];
                    }
                    const float sc = __uint_as_float(sr), bi = __uint_as_float(br);
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        acc[v] = fmaf(sc, dq[v], acc[v]);
                        acc[v] = fmaf(bi, dx[v], acc[v]);
                    }
                }
            }
        });
    }
    // the quarters added in quarter order
    if (wave > 0) part[wave - 1][lane] = mf_f32x4_t{acc[0], acc[1], acc[2], acc[3]};
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w2 = 0; w2 < 3; ++w2) {
        const mf_f32x4_t o = part[w2][lane];
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[v] += o[v];
    }
    // lane (c, h) holds rows 4 h + v of column c
    const bool col_ok = n0 + c < p.n;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int m = 4 * h + v;
        if (col_ok && m < mrows) {
            bf16_bits *yr = p.chunks ? p.y + (int64_t)p.perm[first + m] * p.n : yb + (int64_t)m * p.n;
            Elt<bf16_bits>::store(yr, n0 + c, acc[v]);
        }
    }
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

namespace {

template <typename ST, int GS, int NST, bool SBLDS>
hipError_t gemv_band_run(const GemvLaunch &a, hipStream_t stream)
{
    MfmaGemvParams<ST> p{};
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
    p.words_per_row = a.k / 4;
    p.groups_per_row = a.k / a.gs;
    p.gs = a.gs;
    p.ksplit = 4;
    p.chunks_per_item = (int)((a.rows_per_item + kBandVectors - 1) / kBandVectors);
    const unsigned gx = (unsigned)((a.n + kBandRows - 1) / kBandRows);
    if (a.chunks) {
        if (a.max_chunks > kMfMaxGridY) return hipErrorInvalidValue;
        p.item0 = 0;
        gemv_band_kernel<ST, GS, NST, SBLDS><<<dim3(gx, (unsigned)a.max_chunks), dim3(256), 0, stream>>>(p);
        return hipGetLastError();
    }
    const int64_t items_per_launch = std::max<int64_t>(1, kMfMaxGridY / p.chunks_per_item);
    for (int64_t i0 = 0; i0 < a.items; i0 += items_per_launch) {
        const int64_t cnt = std::min(items_per_launch, a.items - i0);
        p.item0 = i0;
        gemv_band_kernel<ST, GS, NST, SBLDS><<<dim3(gx, (unsigned)(cnt * p.chunks_per_item)), dim3(256), 0, stream>>>(p);
        if (hipError_t err = hipGetLastError()) return err;
    }
    return hipSuccess;
}

template <typename ST, int GS, bool SBLDS>
hipError_t gemv_band_stages(const GemvLaunch &a, hipStream_t stream)
{
    switch (a.k / (4 * kBandStageK)) {
    case 1: return gemv_band_run<ST, GS, 1, SBLDS>(a, stream);
    case 2: return gemv_band_run<ST, GS, 2, SBLDS>(a, stream);
    case 3: return gemv_band_run<ST, GS, 3, SBLDS>(a, stream);
    default: return gemv_band_run<ST, GS, 4, SBLDS>(a, stream);
    }
}

// Scales and biases go to LDS as dwords when both start on a 4-byte
// boundary (the rest of each row's run is then aligned too); otherwise the
// kernel reads them in place.  The values, and so the results, are the same.
template <typename ST, int GS>
hipError_t gemv_band_sb(const GemvLaunch &a, hipStream_t stream)
{
    if ((((uintptr_t)a.scales | (uintptr_t)a.biases) & 3) == 0) return gemv_band_stages<ST, GS, true>(a, stream);
    return gemv_band_stages<ST, GS, false>(a, stream);
}

template <typename ST>
hipError_t gemv_band_gs(const GemvLaunch &a, hipStream_t stream)
{
    switch (a.gs) {
    case 32: return gemv_band_sb<ST, 32>(a, stream);
    case 64: return gemv_band_sb<ST, 64>(a, stream);
    default: return gemv_band_sb<ST, 128>(a, stream);
    }
}

}  // namespace

bool gemv_band_family(int64_t n, int64_t k, int gs, int bits, int x_dt)
{
    // Measured choice, by shape only: 8-bit codes with bf16 activations, K
    // in whole quarters of 256-wide stages up to 4096, below the streaming
    // one-row shapes (x [8, 4096] x [4096, 4096] 8-bit g128: 7.1 us against
    // 11.9 us for the matrix-vector VALU kernel).
    if (x_dt != DT_BF16 || bits != 8 || k < 4 * kBandStageK || k % (4 * kBandStageK) != 0 || k > kBandMaxK)
        return false;
    if (gs != 32 && gs != 64 && gs != 128) return false;
    return n < 8 * 1024;
}

hipError_t launch_gemv_band(const GemvLaunch &a, hipStream_t stream)
{
    if (!gemv_band_family(a.n, a.k, a.gs, a.bits, a.x_dt)) return hipErrorInvalidValue;
    if (a.sb_dt == DT_F32) return gemv_band_gs<float>(a, stream);
    return gemv_band_gs<bf16_bits>(a, stream);
}

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
