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
// 4-bit codes with bf16 activations use v_dot2_f32_bf16.  A code word is split
// into its even and odd nibbles (one and, one shift and and), and each byte
// pair becomes the bf16 pair (128 + q_a, 128 + q_b) with one v_perm_b32 that
// takes the 0x43 exponent bytes from a register (128 + q is exact in bf16 for
// q < 128): 7 VALU operations per 8 codes.  The activations are paired in the
// same order ((x0,x2) (x4,x6) (x1,x3) (x5,x7) per word) and the
// 128 * sum(x) offset is removed once per lane chunk.  For one or two
// activation rows the pairs and chunk sums are prepared once per workgroup in
// LDS.  8-bit codes with bf16 activations are exact in bf16 too: each code
// word becomes two bf16 pairs (v_cvt_f32_ubyte and the high halves), made
// once per weight row and dotted with the activations' own bf16 pairs by
// every activation row.  Other cases convert codes to fp32 and use fp32 FMAs.
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
    // Grouped gather: when `chunks` is set, workgroup row y runs chunk y of
    // the table (uint4 {expert, first, count, 0}: activation vectors
    // perm[first .. first + count) all use that expert); chunks past
    // *nchunks do nothing.
    const uint4 *chunks;
    const uint32_t *perm;
    const uint32_t *nchunks;
    // left indices: vector r * lhs_l + j reads x row lhs[r] * lhs_l + j
    const uint32_t *lhs;
    int64_t x_items, lhs_l;
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

// One K step of a wave's work, as loaded: raw scale/bias storage bits
// (converted only when used, so no conversion forces an early wait on the
// load), raw code words and, for few activation rows read directly, the
// lane's activations.  Scales and biases are loaded before the codes, so they
// have arrived whenever the codes have.
template <int BITS, int RW, int XW>
struct Stage {
    uint32_t s[RW], b[RW];
    uint4 xr[XW > 0 ? XW : 1];
    uint32_t cw[RW][BITS];
};

template <typename T>
__device__ __forceinline__ uint32_t load_raw(const T *p, int64_t i)
{
    if constexpr (sizeof(T) == 2) return (uint32_t)p[i];
    else return __float_as_uint(p[i]);
}

template <typename T>
__device__ __forceinline__ float raw_to_f32(uint32_t v)
{
    if constexpr (sizeof(T) == 2) return __uint_as_float(v << 16);
    else return __uint_as_float(v);
}

// Sum of V values over the 64 lanes (V a power of two <= 64).  At each xor
// step a lane keeps half of its values and sends the other half, so every
// value goes through the same pairwise tree (xor 32, 16, ..., 1) as a plain
// butterfly, with V - 1 + 6 - log2(V) exchanges instead of 6 V.  Afterwards
// lane L holds value L >> (6 - log2 V).
template <int V, int OFF = 32>
__device__ __forceinline__ float wave_reduce_transposed(float (&v)[V], int lane)
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
        return wave_reduce_transposed<V / 2, OFF / 2>(h, lane);
    } else {
        float r;
        if constexpr (OFF >= 16) r = swap_sum<OFF>(v[0], v[0]);
        else r = v[0] + xor_lane<OFF>(v[0], lane);
        float one[1] = {r};
        return wave_reduce_transposed<1, OFF / 2>(one, lane);
    }
}

template <int V>
constexpr int ilog2() { return V <= 1 ? 0 : 1 + ilog2<V / 2>(); }

// ---- arithmetic of one 32-element lane chunk, shared by every variant so
// ---- that a row's bits never depend on which variant ran it.

// Activation pairs of one code word (8 bf16 in dwords d0..d3 = (x1:x0)
// (x3:x2) (x5:x4) (x7:x6)), in the order of the code pairs below.
__device__ __forceinline__ void x_pairs_word(uint4 d, uint32_t *xp)
{
    xp[0] = __builtin_amdgcn_perm(d.y, d.x, 0x05040100u);   // (x0, x2)
    xp[1] = __builtin_amdgcn_perm(d.w, d.z, 0x05040100u);   // (x4, x6)
    xp[2] = __builtin_amdgcn_perm(d.y, d.x, 0x07060302u);   // (x1, x3)
    xp[3] = __builtin_amdgcn_perm(d.w, d.z, 0x07060302u);   // (x5, x7)
}

// Sum of the 8 activations of a word, accumulated onto X.
__device__ __forceinline__ float x_sum_word(uint4 d, float X)
{
    constexpr uint32_t kOnes = 0x3f803f80u;   // bf16 pair (1, 1)
    X = dot2_bf16(d.x, kOnes, X);
    X = dot2_bf16(d.y, kOnes, X);
    X = dot2_bf16(d.z, kOnes, X);
    return dot2_bf16(d.w, kOnes, X);
}

// D += sum over the 8 codes of a 4-bit word of x_i * (128 + q_i).
__device__ __forceinline__ float word_dot_magic(uint32_t w, const uint32_t *xp, uint32_t mag, float D)
{
    const uint32_t lo = w & 0x0f0f0f0fu;          // q0 q2 q4 q6
    const uint32_t hi = (w >> 4) & 0x0f0f0f0fu;   // q1 q3 q5 q7
    D = dot2_bf16(xp[0], __builtin_amdgcn_perm(mag, lo, 0x04010400u), D);   // (q0, q2)
    D = dot2_bf16(xp[1], __builtin_amdgcn_perm(mag, lo, 0x04030402u), D);   // (q4, q6)
    D = dot2_bf16(xp[2], __builtin_amdgcn_perm(mag, hi, 0x04010400u), D);   // (q1, q3)
    return dot2_bf16(xp[3], __builtin_amdgcn_perm(mag, hi, 0x04030402u), D); // (q5, q7)
}

// 1- and 2-bit codes with bf16 activations use the same (128 + q) pairs:
// shifting a code word right by `bits` * i and masking every byte down to its
// low `bits` bits leaves one code per byte, codes i, i + 32 / (4 bits), ...
// (a stride of 8 at 1 bit, 4 at 2 bits), and two v_perm_b32 turn the four
// bytes into two bf16 pairs.  The activation pairs follow that order.

// Activation pairs of a lane chunk (32 bf16 in d[0..3]) in the order of the
// code pairs of chunk_dot_magic<BITS>.
template <int BITS>
__device__ __forceinline__ void x_pairs_chunk(const uint4 *d, uint32_t *xp)
{
    if constexpr (BITS == 4) {
#pragma unroll
        for (int j = 0; j < 4; ++j) x_pairs_word(d[j], xp + 4 * j);
    } else {
        uint32_t v[16];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[4 * j] = d[j].x, v[4 * j + 1] = d[j].y, v[4 * j + 2] = d[j].z, v[4 * j + 3] = d[j].w;
        // element e of the chunk is half e % 2 of dword e / 2
        auto pair = [&](int a, int b) -> uint32_t {   // (x_a, x_b), a % 2 == b % 2
            return __builtin_amdgcn_perm(v[b >> 1], v[a >> 1], (a & 1) ? 0x07060302u : 0x05040100u);
        };
        constexpr int kWordCodes = 32 / BITS;      // codes per word: 16 or 32
        constexpr int kStride = kWordCodes / 4;    // code stride inside a byte lane: 4 or 8
#pragma unroll
        for (int h = 0; h < BITS; ++h)             // word h of the chunk
#pragma unroll
            for (int i = 0; i < kStride; ++i) {
                const int c0 = h * kWordCodes + i;
                xp[2 * (h * kStride + i)] = pair(c0, c0 + kStride);
                xp[2 * (h * kStride + i) + 1] = pair(c0 + 2 * kStride, c0 + 3 * kStride);
            }
    }
}

// D += sum over the lane chunk's 32 codes (words cw[0 .. BITS)) of x * (128 + q).
template <int BITS>
__device__ __forceinline__ float chunk_dot_magic(const uint32_t *cw, const uint32_t *xp, uint32_t mag, float D)
{
    if constexpr (BITS == 4) {
#pragma unroll
        for (int j = 0; j < 4; ++j) D = word_dot_magic(cw[j], xp + 4 * j, mag, D);
    } else {
        constexpr uint32_t kMask = BITS == 1 ? 0x01010101u : 0x03030303u;
        constexpr int kStride = 8 / BITS;
#pragma unroll
        for (int h = 0; h < BITS; ++h)
#pragma unroll
            for (int i = 0; i < kStride; ++i) {
                const uint32_t b = (cw[h] >> (BITS * i)) & kMask;   // codes i, i + s, i + 2 s, i + 3 s
                D = dot2_bf16(xp[2 * (h * kStride + i)], __builtin_amdgcn_perm(mag, b, 0x04010400u), D);
                D = dot2_bf16(xp[2 * (h * kStride + i) + 1], __builtin_amdgcn_perm(mag, b, 0x04030402u), D);
            }
    }
    return D;
}

// The fp32 activations of a lane chunk's word j (8 values).
template <typename XT>
__device__ __forceinline__ void x_f32_word(const uint4 *xw, int j, float *xf)
{
    if constexpr (sizeof(XT) == 2) {
        const uint4 d = xw[j];
        const uint32_t v[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            xf[2 * i] = __uint_as_float(v[i] << 16);
            xf[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
        }
    } else {
        const uint4 a = xw[2 * j], b = xw[2 * j + 1];
        xf[0] = __uint_as_float(a.x), xf[1] = __uint_as_float(a.y);
        xf[2] = __uint_as_float(a.z), xf[3] = __uint_as_float(a.w);
        xf[4] = __uint_as_float(b.x), xf[5] = __uint_as_float(b.y);
        xf[6] = __uint_as_float(b.z), xf[7] = __uint_as_float(b.w);
    }
}

// LDS image of the staged activations: for activation row m, step t, word j
// (0..3 of the lane chunk) and lane L, the 4 pairs of that word; then the
// chunk sums.  Sized MR * steps * (4 * 64 * 16 + 64 * 4) bytes.
constexpr int kStageBytesPerStep = 4 * 64 * 16 + 64 * 4;

template <int BITS, typename XT, typename ST, int MR, int RW, int STX>
__global__ void __launch_bounds__(512) gemv_kernel(GemvParams<XT, ST> p)
{
    constexpr bool kMagic = (BITS == 1 || BITS == 2 || BITS == 4) && (sizeof(XT) == 2);
    constexpr bool kBytePairs = (BITS == 8) && (sizeof(XT) == 2);
    static_assert(STX == 0 || (kMagic && BITS == 4), "staged activations hold bf16 pairs for 4-bit codes");
    // without staging, activations travel with the codes when they are few
    constexpr int kXW = (STX == 0 && MR <= 2) ? MR * (kLaneChunk * (int)sizeof(XT) / 16) : 0;
    constexpr int kXWR = kLaneChunk * (int)sizeof(XT) / 16;   // 16-byte pieces per row chunk
    extern __shared__ uint4 lds_x[];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform per wave
    const int S = p.ksplit;
    const int sl = wave % S;            // K slice of this wave
    const int q = wave / S;             // row group of this wave inside the workgroup
    const int64_t n0 = ((int64_t)blockIdx.x * p.qrows + q) * RW;

    bool live = true;
    int64_t slab = 0;
    int mrows;
    const XT *xb;   // activation row 0 of this chunk (rows are contiguous unless grouped)
    XT *yb;
    uint32_t first = 0;   // grouped: the chunk's first position in perm
    if (p.chunks) {
        if (blockIdx.y >= *p.nchunks) return;   // uniform over the workgroup
        const uint4 ch = p.chunks[blockIdx.y];
        if ((int64_t)ch.x >= p.e) live = false;
        else slab = ch.x;
        first = ch.y;
        mrows = (int)ch.z;
        xb = p.x;
        yb = p.y;
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
    // activation rows of the chunk (rows past the chunk's repeat its last),
    // computed once and kept in scalar registers: they are the same for the
    // whole workgroup
    const XT *xr[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        const int mm = min(m, mrows - 1);
        int64_t v = 0;
        if (p.chunks) {
            v = p.perm[first + mm];
            if (p.lhs) {
                // rows with lhs >= x_items are in the zero bucket and never
                // read x; they point at item 0 all the same
                const int64_t xi = p.lhs[v / p.lhs_l];
                v = (xi < p.x_items ? xi : 0) * p.lhs_l + v % p.lhs_l;
            }
        }
        const XT *r = p.chunks ? p.x + v * p.k : xb + (int64_t)mm * p.k;
        const uint64_t u = reinterpret_cast<uint64_t>(r);
        const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
        const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
        xr[m] = reinterpret_cast<const XT *>(((uint64_t)hi << 32) | lo);
    }
    auto x_row = [&](int m) -> const XT * {
        if constexpr (MR == 1) return xr[0];
        else if constexpr (MR == 2) return m == 0 ? xr[0] : xr[1];
        else return xr[m];   // m is a constant after unrolling here
    };
    auto y_row = [&](int m) -> XT * {
        return p.chunks ? p.y + (int64_t)p.perm[first + m] * p.n : yb + (int64_t)m * p.n;
    };
    const uint32_t *cb = p.codes + slab * p.n * p.words_per_row;
    const ST *sb = p.scales + slab * p.n * p.groups_per_row;
    const ST *bb = p.biases + slab * p.n * p.groups_per_row;

    // Rows past n and lanes past k read row 0 / element 0 of the slab (always
    // in bounds) and are masked when used.
    const uint32_t *crow[RW];
    int64_t srow[RW];
#pragma unroll
    for (int r = 0; r < RW; ++r) {
        const int64_t nr = min(n0 + r, p.n - 1);
        crow[r] = cb + nr * p.words_per_row;
        srow[r] = nr * p.groups_per_row;
    }
    constexpr uint32_t kMag = 0x43434343u;   // bf16 exponent bytes of 128 + q

    // ---- staged activations: loads first, then (after this wave's first codes
    // ---- are in flight) pairs and sums into LDS.
    constexpr int kStageChunks = STX;   // chunks of 32 activations per thread
    uint4 sx[kStageChunks > 0 ? kStageChunks : 1][4];
    const int nstage = MR * p.steps * 64;
    if constexpr (STX > 0) {
#pragma unroll
        for (int i = 0; i < kStageChunks; ++i) {
            const int c = min((int)threadIdx.x + i * (int)blockDim.x, nstage - 1);
            const int m = c / (p.steps * 64), rem = c % (p.steps * 64);
            const int64_t e0 = (int64_t)(rem >> 6) * kStepElems + (rem & 63) * kLaneChunk;
            const uint4 *src = reinterpret_cast<const uint4 *>(x_row(m) + (e0 < p.k ? e0 : 0));
#pragma unroll
            for (int j = 0; j < 4; ++j) sx[i][j] = src[j];
        }
    }

    float acc[MR][RW];
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int r = 0; r < RW; ++r) acc[m][r] = 0.0f;

    auto load_stage = [&](int t, Stage<BITS, RW, kXW> &st) {
        const int64_t e0 = (int64_t)t * kStepElems + lane * kLaneChunk;
        const bool on = t < p.steps && e0 < p.k;
        const int64_t ec = on ? e0 : 0;
        const int64_t g = ec / p.gs;
#pragma unroll
        for (int r = 0; r < RW; ++r) {
            st.s[r] = load_raw(sb, srow[r] + g);
            st.b[r] = load_raw(bb, srow[r] + g);
        }
        if constexpr (kXW > 0) {
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                const uint4 *xs = reinterpret_cast<const uint4 *>(x_row(m) + ec);
#pragma unroll
                for (int i = 0; i < kXWR; ++i) st.xr[m * kXWR + i] = xs[i];
            }
        }
#pragma unroll
        for (int r = 0; r < RW; ++r) load_chunk_words<BITS>(crow[r] + ec * BITS / 32, st.cw[r]);
    };

    auto compute_stage = [&](int t, const Stage<BITS, RW, kXW> &st) {
        const int64_t e0 = (int64_t)t * kStepElems + lane * kLaneChunk;
        if (e0 >= p.k) return;
        float X[MR];
        float T[MR][RW];   // magic: sum x (128 + q) - 128 X; else sum x q
        if constexpr (kMagic) {
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                uint32_t xp[16];
                if constexpr (STX > 0) {
                    const uint4 *base = lds_x + (int64_t)((m * p.steps + t) * 4) * 64 + lane;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint4 v = base[j * 64];
                        xp[4 * j] = v.x, xp[4 * j + 1] = v.y, xp[4 * j + 2] = v.z, xp[4 * j + 3] = v.w;
                    }
                    const float *sums = reinterpret_cast<const float *>(lds_x + MR * p.steps * 256);
                    X[m] = sums[(m * p.steps + t) * 64 + lane];
                } else {
                    X[m] = 0.0f;
                    uint4 d[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        if constexpr (kXW > 0) d[j] = st.xr[m * kXWR + j];
                        else d[j] = reinterpret_cast<const uint4 *>(x_row(m) + e0)[j];
                        X[m] = x_sum_word(d[j], X[m]);
                    }
                    x_pairs_chunk<BITS>(d, xp);
                }
#pragma unroll
                for (int r = 0; r < RW; ++r) {
                    const float D = chunk_dot_magic<BITS>(st.cw[r], xp, kMag, 0.0f);
                    T[m][r] = fmaf(-128.0f, X[m], D);
                }
            }
        } else if constexpr (kBytePairs) {
            // 8-bit codes are exact in bf16: each weight row's 32 codes become
            // 16 bf16 pairs once (v_cvt_f32_ubyte, then the high halves), and
            // every activation row takes 16 dot2 against its own bf16 pairs
            uint32_t qp[RW][16];
#pragma unroll
            for (int r = 0; r < RW; ++r)
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const uint32_t w = st.cw[r][j];
                    const float f0 = (float)(w & 0xffu), f1 = (float)((w >> 8) & 0xffu);
                    const float f2 = (float)((w >> 16) & 0xffu), f3 = (float)(w >> 24);
                    qp[r][2 * j] = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
                    qp[r][2 * j + 1] = __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
                }
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                uint32_t xd[16];
                X[m] = 0.0f;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    uint4 d;
                    if constexpr (kXW > 0) d = st.xr[m * kXWR + j];
                    else d = reinterpret_cast<const uint4 *>(x_row(m) + e0)[j];
                    xd[4 * j] = d.x, xd[4 * j + 1] = d.y, xd[4 * j + 2] = d.z, xd[4 * j + 3] = d.w;
                    X[m] = x_sum_word(d, X[m]);
                }
#pragma unroll
                for (int r = 0; r < RW; ++r) {
                    float D = 0.0f;
#pragma unroll
                    for (int u = 0; u < 16; ++u) D = dot2_bf16(xd[u], qp[r][u], D);
                    T[m][r] = D;
                }
            }
        } else {
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                X[m] = 0.0f;
#pragma unroll
                for (int r = 0; r < RW; ++r) T[m][r] = 0.0f;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {             // elements 8j .. 8j+7
                float xf[MR][8];
#pragma unroll
                for (int m = 0; m < MR; ++m) {
                    if constexpr (kXW > 0) {
                        x_f32_word<XT>(st.xr + m * kXWR, j, xf[m]);
                    } else {
                        x_f32_word<XT>(reinterpret_cast<const uint4 *>(x_row(m) + e0), j, xf[m]);
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
                        for (int m = 0; m < MR; ++m) T[m][r] = fmaf(xf[m][i], qf, T[m][r]);
                    }
                }
            }
        }
#pragma unroll
        for (int r = 0; r < RW; ++r) {
            const bool rv = n0 + r < p.n;
            const float sc = rv ? raw_to_f32<ST>(st.s[r]) : 0.0f;
            const float bi = rv ? raw_to_f32<ST>(st.b[r]) : 0.0f;
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                acc[m][r] = fmaf(sc, T[m][r], acc[m][r]);
                acc[m][r] = fmaf(bi, X[m], acc[m][r]);
            }
        }
    };

    // Groups of kGroup steps: every load of a group is issued before the
    // first of them is used.  Steps past the end read a dummy in-bounds
    // address and are not computed.
    constexpr int kGroup = 2;
    int t0 = sl;
    // A wave with no step to do (k == 0, where the inputs may be empty and
    // their pointers null, or a slice past the last step) loads nothing.
    const bool work = live && t0 < p.steps;
    Stage<BITS, RW, kXW> st[kGroup];
    if (work) {
#pragma unroll
        for (int u = 0; u < kGroup; ++u) load_stage(t0 + u * S, st[u]);
    }
    if constexpr (STX > 0) {
        // pairs and sums of the staged activations (the loads above were issued first)
        float *sums = reinterpret_cast<float *>(lds_x + MR * p.steps * 256);
#pragma unroll
        for (int i = 0; i < kStageChunks; ++i) {
            const int c = (int)threadIdx.x + i * (int)blockDim.x;
            if (c < nstage) {
                const int mt = c >> 6, ln = c & 63;
                float Xs = 0.0f;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    uint32_t xp[4];
                    x_pairs_word(sx[i][j], xp);
                    Xs = x_sum_word(sx[i][j], Xs);
                    lds_x[(mt * 4 + j) * 64 + ln] = make_uint4(xp[0], xp[1], xp[2], xp[3]);
                }
                sums[mt * 64 + ln] = Xs;
            }
        }
        __syncthreads();
    }
    if (work) {
        for (;;) {
#pragma unroll
            for (int u = 0; u < kGroup; ++u)
                if (t0 + u * S < p.steps) compute_stage(t0 + u * S, st[u]);
            t0 += kGroup * S;
            if (t0 >= p.steps) break;
#pragma unroll
            for (int u = 0; u < kGroup; ++u) load_stage(t0 + u * S, st[u]);
        }
    }

    // Fixed-order reduction over the 64 lanes; lane L then holds output
    // v = L >> kShift, i.e. (m, r) = (v / RW, v % RW).
    constexpr int V = MR * RW;
    constexpr int kShift = 6 - ilog2<V>();
    float vals[V];
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int r = 0; r < RW; ++r) vals[m * RW + r] = acc[m][r];
    const float mine = wave_reduce_transposed<V>(vals, lane);
    const int vi = lane >> kShift;
    const bool leader = (lane & ((1 << kShift) - 1)) == 0;
    const int mi = vi / RW, ri = vi % RW;
    const bool writer = leader && mi < mrows && n0 + ri < p.n;
    if (S == 1) {
        if (writer) Elt<XT>::store(y_row(mi), n0 + ri, mine);
        return;
    }
    __shared__ float part[8 * V];
    if (leader) part[wave * V + vi] = mine;
    __syncthreads();
    if (sl == 0 && writer) {
        float tot = part[(q * S) * V + vi];
        for (int s2 = 1; s2 < S; ++s2) tot += part[(q * S + s2) * V + vi];
        Elt<XT>::store(y_row(mi), n0 + ri, tot);
    }
}

// ---------------------------------------------------------------------------
// One activation row of bf16 activations (any code width), K in at most
// kStreamMaxSteps steps and not split: a streaming form of the kernel above.
// Every wave keeps the activation pairs and chunk sums of all its steps in
// registers and walks NR weight rows spaced by the wave count W (rows
// w, w + W, w + 2W, ...: at any moment the waves read one contiguous band of
// the weights), loading rows kStreamDepth ahead of the one it computes.  The
// row loop is straight-line code (lanes past k compute on clamped data and a
// select drops the result), so the only waits are the counted ones for the
// row about to be used.  Per lane and row the arithmetic is that of
// gemv_kernel (same lane chunks, same operation order) and the lane sums take
// the same xor tree, so every row has the bits gemv_kernel gives it.  Rows
// past n read row n - 1 and are not stored.
constexpr int kStreamMaxSteps = 4;
constexpr int kStreamDepth = 3;
constexpr int kStreamWaves = 4;   // waves per workgroup

template <int BITS, int STEPS>
struct StreamStage {
    uint32_t s[STEPS], b[STEPS];
    uint32_t c[STEPS][BITS];
};

// Per-step activations held by a wave: 1-, 2- and 4-bit codes, the pairs in
// code-pair order; 8-bit codes, the bf16 pairs as stored; other widths, fp32
// values.
template <int BITS>
struct StreamX {
    static constexpr int kWords = BITS == 1 || BITS == 2 || BITS == 4 || BITS == 8 ? 16 : 32;
    uint32_t v[kWords];
};

template <int BITS, typename ST, int STEPS, int NR>
__global__ void __launch_bounds__(64 * kStreamWaves) gemv_stream_kernel(GemvParams<bf16_bits, ST> p)
{
    const int lane = threadIdx.x & 63;
    const int64_t w = (int64_t)blockIdx.x * kStreamWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t nw = (int64_t)gridDim.x * kStreamWaves;
    constexpr uint32_t kMag = 0x43434343u;

    // activations and chunk sums of every step, in gemv_kernel's order
    StreamX<BITS> xs[STEPS];
    float X[STEPS];
    bool on[STEPS];
    int64_t e0[STEPS], g0[STEPS];
#pragma unroll
    for (int t = 0; t < STEPS; ++t) {
        const int64_t e = (int64_t)t * kStepElems + lane * kLaneChunk;
        on[t] = e < p.k;
        e0[t] = on[t] ? e : 0;
        g0[t] = e0[t] / p.gs;
        const uint4 *src = reinterpret_cast<const uint4 *>(p.x + e0[t]);
        X[t] = 0.0f;
        if constexpr (BITS == 1 || BITS == 2 || BITS == 4) {
            uint4 d[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                d[j] = src[j];
                X[t] = x_sum_word(d[j], X[t]);
            }
            x_pairs_chunk<BITS>(d, xs[t].v);
        } else if constexpr (BITS == 8) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint4 d = src[j];
                xs[t].v[4 * j] = d.x, xs[t].v[4 * j + 1] = d.y, xs[t].v[4 * j + 2] = d.z, xs[t].v[4 * j + 3] = d.w;
                X[t] = x_sum_word(d, X[t]);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float xf[8];
                x_f32_word<bf16_bits>(src, j, xf);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    xs[t].v[8 * j + i] = __float_as_uint(xf[i]);
                    X[t] += xf[i];
                }
            }
        }
    }

    auto row_of = [&](int i) -> int64_t { return min(w + (int64_t)i * nw, p.n - 1); };
    auto load = [&](int i, StreamStage<BITS, STEPS> &st) {
        const int64_t r = row_of(i);
        const uint32_t *crow = p.codes + r * p.words_per_row;
#pragma unroll
        for (int t = 0; t < STEPS; ++t) {
            st.s[t] = load_raw(p.scales, r * p.groups_per_row + g0[t]);
            st.b[t] = load_raw(p.biases, r * p.groups_per_row + g0[t]);
        }
#pragma unroll
        for (int t = 0; t < STEPS; ++t) load_chunk_words<BITS>(crow + e0[t] * BITS / 32, st.c[t]);
    };
    auto compute = [&](const StreamStage<BITS, STEPS> &st) -> float {
        float a = 0.0f;
#pragma unroll
        for (int t = 0; t < STEPS; ++t) {
            float T;
            if constexpr (BITS == 1 || BITS == 2 || BITS == 4) {
                const float D = chunk_dot_magic<BITS>(st.c[t], xs[t].v, kMag, 0.0f);
                T = fmaf(-128.0f, X[t], D);
            } else if constexpr (BITS == 8) {
                float D = 0.0f;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const uint32_t cw = st.c[t][j];
                    const float f0 = (float)(cw & 0xffu), f1 = (float)((cw >> 8) & 0xffu);
                    const float f2 = (float)((cw >> 16) & 0xffu), f3 = (float)(cw >> 24);
                    D = dot2_bf16(xs[t].v[2 * j], __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u), D);
                    D = dot2_bf16(xs[t].v[2 * j + 1], __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u), D);
                }
                T = D;
            } else {
                T = 0.0f;
#pragma unroll
                for (int i = 0; i < kLaneChunk; ++i)
                    T = fmaf(__uint_as_float(xs[t].v[i]), (float)code_at<BITS>(st.c[t], i), T);
            }
            float an = fmaf(raw_to_f32<ST>(st.s[t]), T, a);
            an = fmaf(raw_to_f32<ST>(st.b[t]), X[t], an);
            a = pick(on[t], an, a);
        }
        return a;
    };

    constexpr int V = NR <= 8 ? 8 : 16;
    float acc[V];
    StreamStage<BITS, STEPS> st[kStreamDepth + 1];
#pragma unroll
    for (int i = 0; i < kStreamDepth && i < NR; ++i) load(i, st[i]);
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        if (i + kStreamDepth < NR) load(i + kStreamDepth, st[(i + kStreamDepth) % (kStreamDepth + 1)]);
        __builtin_amdgcn_sched_barrier(0);   // keep the prefetch ahead of the arithmetic
        acc[i] = compute(st[i % (kStreamDepth + 1)]);
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = NR; i < V; ++i) acc[i] = 0.0f;
    const float mine = wave_reduce_transposed<V>(acc, lane);
    constexpr int kShift = 6 - ilog2<V>();
    const int vi = lane >> kShift;
    const int64_t row = w + (int64_t)vi * nw;
    if ((lane & ((1 << kShift) - 1)) == 0 && vi < NR && row < p.n) Elt<bf16_bits>::store(p.y, row, mine);
}

// Launch shape of the streaming kernel for n rows on `cus` compute units:
// a whole number of workgroups per compute unit (an uneven count leaves some
// units with twice the rows), and rows per wave the smallest of 8, 10, ..., 16
// that covers n.
struct StreamShape {
    int64_t groups;
    int nr;
};

StreamShape stream_shape(int64_t n, int cus)
{
    const int64_t per_cu = (n + (int64_t)cus * kStreamWaves * 16 - 1) / ((int64_t)cus * kStreamWaves * 16);
    StreamShape sh;
    sh.groups = std::max<int64_t>(1, per_cu) * cus;
    const int64_t need = (n + sh.groups * kStreamWaves - 1) / (sh.groups * kStreamWaves);
    sh.nr = need <= 8 ? 8 : (int)((need + 1) / 2 * 2);
    return sh;
}

// ---------------------------------------------------------------------------
// Grouping pass of the grouped gather ("Mixture of experts" section: a
// grouped kernel reads each expert's weights once for the rows that chose
// it).  One workgroup sorts the activation vectors v = r * l + j by expert
// bucket b = min(ids[r], e) (bucket e: ids past the last expert, whose rows
// are zero) with a stable counting sort -- within a bucket in increasing v,
// so the result never depends on timing -- and cuts every bucket into
// chunks of at most `chunk` vectors.  Workspace layout (uint32):
// perm[V], nchunks, padding to 16 bytes, then the chunk table as uint4
// {bucket, first position in perm, count, 0}.
constexpr int kGroupThreads = 1024;

__device__ void block_exclusive_scan(uint32_t *a, int n, uint32_t *part, uint32_t *total)
{
    // a[0..n) in LDS, scanned in place; part: kGroupThreads scratch words
    const int t = threadIdx.x;
    const int seg = (n + kGroupThreads - 1) / kGroupThreads;
    const int lo = min(n, t * seg), hi = min(n, lo + seg);
    uint32_t sum = 0;
    for (int i = lo; i < hi; ++i) sum += a[i];
    part[t] = sum;
    __syncthreads();
    for (int off = 1; off < kGroupThreads; off <<= 1) {   // inclusive Hillis-Steele
        const uint32_t v = t >= off ? part[t - off] : 0u;
        __syncthreads();
        part[t] += v;
        __syncthreads();
    }
    uint32_t run = t ? part[t - 1] : 0u;
    if (t == kGroupThreads - 1) *total = part[t];
    for (int i = lo; i < hi; ++i) {
        const uint32_t c = a[i];
        a[i] = run;
        run += c;
    }
    __syncthreads();
}

__global__ void __launch_bounds__(kGroupThreads)
gather_group_kernel(const uint32_t *ids, const uint32_t *lhs, int64_t x_items, int64_t rows, int64_t l, int e,
                    uint32_t *ws, int64_t v_total, uint32_t chunk)
{
    extern __shared__ uint4 sh4[];   // bucket[1024], part[1024], count[e+1], chunk offset[e+1], totals[2]
    uint32_t *sh = reinterpret_cast<uint32_t *>(sh4);
    const int nb = e + 1;
    uint32_t *bk = sh, *part = sh + kGroupThreads, *cnt = part + kGroupThreads, *coff = cnt + nb;
    uint32_t *totals = coff + nb;
    uint32_t *perm = ws, *nchunks = ws + v_total;
    uint4 *table = reinterpret_cast<uint4 *>(ws + ((v_total + 1 + 3) & ~(int64_t)3));
    const int t = threadIdx.x;
    auto bucket = [&](int64_t v) -> uint32_t {
        const int64_t r = v / l;
        return lhs && (int64_t)lhs[r] >= x_items ? (uint32_t)e : min(ids[r], (uint32_t)e);
    };

    for (int b = t; b < nb; b += kGroupThreads) cnt[b] = 0;
    __syncthreads();
    for (int64_t v = t; v < v_total; v += kGroupThreads) atomicAdd(&cnt[bucket(v)], 1u);
    __syncthreads();
    for (int b = t; b < nb; b += kGroupThreads) coff[b] = (cnt[b] + chunk - 1) / chunk;
    __syncthreads();
    block_exclusive_scan(coff, nb, part, &totals[1]);   // first chunk of each bucket
    // chunk table, before cnt turns into offsets
    for (int b = t; b < nb; b += kGroupThreads) {
        const uint32_t c = cnt[b];
        for (uint32_t i = 0; i * chunk < c; ++i)
            table[coff[b] + i] = make_uint4((uint32_t)b, 0u, min(chunk, c - i * chunk), 0u);
    }
    block_exclusive_scan(cnt, nb, part, &totals[0]);    // first position of each bucket
    for (int b = t; b < nb; b += kGroupThreads) {
        const uint32_t c = (b + 1 < nb ? cnt[b + 1] : (uint32_t)v_total) - cnt[b];
        for (uint32_t i = 0; i * chunk < c; ++i) table[coff[b] + i].y = cnt[b] + i * chunk;
    }
    if (t == 0) *nchunks = totals[1];
    // stable placement, kGroupThreads vectors at a time: a vector's rank is
    // the number of earlier vectors of its bucket in the same batch
    for (int64_t v0 = 0; v0 < v_total; v0 += kGroupThreads) {
        const int64_t v = v0 + t;
        const uint32_t b = v < v_total ? bucket(v) : 0xffffffffu;
        bk[t] = b;
        __syncthreads();
        if (v < v_total) {
            // 16-byte reads of the earlier buckets (every lane of a wave
            // reads the same address at a time: broadcasts)
            const uint4 *bk4 = reinterpret_cast<const uint4 *>(bk);
            uint32_t rank = 0;
            for (int u = 0; u < (t >> 2); ++u) {
                const uint4 q = bk4[u];
                rank += (q.x == b) + (q.y == b) + (q.z == b) + (q.w == b);
            }
            for (int u = t & ~3; u < t; ++u) rank += bk[u] == b;
            perm[cnt[b] + rank] = (uint32_t)v;
        }
        __syncthreads();
        if (v < v_total) atomicAdd(&cnt[b], 1u);   // the batch's count per bucket (an exact sum)
        __syncthreads();
    }
}

// The same grouping for up to kGroupSmallBuckets buckets (e < 256): each
// wave ranks its 64 vectors by bucket with ballots (one pass per distinct
// bucket in the wave), per-wave counts go to a [wave][bucket] table whose
// prefix over the waves gives every vector's position; one wave scans the
// bucket sizes with shuffles.  Same stable order, same table.
constexpr int kGroupSmallBuckets = 256;
constexpr int kGroupWaves = kGroupThreads / 64;

__global__ void __launch_bounds__(kGroupThreads)
gather_group_small_kernel(const uint32_t *ids, const uint32_t *lhs, int64_t x_items, int64_t l, int e, uint32_t *ws,
                          int64_t v_total, uint32_t chunk)
{
    __shared__ uint32_t wc[kGroupWaves][kGroupSmallBuckets];   // per-wave counts, then positions
    __shared__ uint32_t hist[kGroupSmallBuckets];
    __shared__ uint32_t start[kGroupSmallBuckets];              // next position of each bucket
    __shared__ uint32_t coff[kGroupSmallBuckets + 1];           // first chunk of each bucket
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int nb = e + 1;
    uint32_t *perm = ws, *nchunks = ws + v_total;
    uint4 *table = reinterpret_cast<uint4 *>(ws + ((v_total + 1 + 3) & ~(int64_t)3));
    const uint64_t lanes_below = (lane ? ~0ull >> (64 - lane) : 0ull);
    auto bucket = [&](int64_t v) -> uint32_t {
        if (v >= v_total) return 0xffffffffu;
        const int64_t r = v / l;
        return lhs && (int64_t)lhs[r] >= x_items ? (uint32_t)e : min(ids[r], (uint32_t)e);
    };
    // For every distinct bucket among this wave's valid lanes (in lane
    // order of first appearance): fn(bucket, lanes holding it).
    auto match = [&](uint32_t b, auto fn) {
        uint64_t active = __ballot(b != 0xffffffffu);
        while (active) {
            const int leader = __ffsll((long long)active) - 1;
            const uint32_t lb = (uint32_t)__builtin_amdgcn_readlane((int)b, leader);
            const uint64_t m = __ballot(b == lb) & active;
            fn(lb, m, leader);
            active &= ~m;
        }
    };

    // the bucket sizes in hist -> start[b] (first position), coff[b] (first
    // chunk), coff[nb] and *nchunks (the chunk count)
    auto scan = [&] {
        if (w != 0) return;
        // exclusive scans of the bucket sizes and chunk counts; lane i holds
        // buckets 4 i .. 4 i + 3
        uint32_t h[4], cn[4], sh = 0, sc = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int b = 4 * lane + j;
            h[j] = b < nb ? hist[b] : 0u;
            cn[j] = (h[j] + chunk - 1) / chunk;
            sh += h[j];
            sc += cn[j];
        }
        uint32_t ih = sh, ic = sc;   // inclusive over lanes
        for (int off = 1; off < 64; off <<= 1) {
            const uint32_t a = __shfl_up(ih, off), c2 = __shfl_up(ic, off);
            if (lane >= off) ih += a, ic += c2;
        }
        uint32_t ph = ih - sh, pc = ic - sc;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int b = 4 * lane + j;
            if (b < nb) start[b] = ph, coff[b] = pc;
            ph += h[j];
            pc += cn[j];
        }
        if (lane == 63) {
            coff[nb] = ic;
            *nchunks = ic;
        }
    };
    // chunk table: entry j belongs to the last bucket whose first chunk is <= j
    auto write_table = [&] {
        const uint32_t total = coff[nb];
        for (uint32_t j = t; j < total; j += kGroupThreads) {
            int lo = 0, hi = nb;   // coff[lo] <= j < coff[hi]
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (coff[mid] <= j) lo = mid;
                else hi = mid;
            }
            const uint32_t i = j - coff[lo];
            table[j] = make_uint4((uint32_t)lo, start[lo] + i * chunk, min(chunk, hist[lo] - i * chunk), 0u);
        }
    };

    if (v_total <= kGroupThreads) {   // uniform
        // One round: a single pass over the ids gives each wave's count per
        // bucket and each vector's rank among the earlier lanes of its wave
        // with the same bucket; the bucket sizes are the waves' counts
        // summed, and a vector goes to start[b] + (the earlier waves' count
        // in b) + its rank -- the positions of the general path below.
        for (int i = t; i < kGroupWaves * kGroupSmallBuckets; i += kGroupThreads) (&wc[0][0])[i] = 0;
        __syncthreads();
        const uint32_t b = bucket(t);
        uint32_t rank = 0;
        match(b, [&](uint32_t lb, uint64_t m, int leader) {
            if (b == lb) rank = (uint32_t)__popcll(m & lanes_below);
            if (lane == leader) wc[w][lb] = (uint32_t)__popcll(m);
        });
        __syncthreads();
        for (int bb = t; bb < nb; bb += kGroupThreads) {
            uint32_t run = 0;
            for (int w2 = 0; w2 < kGroupWaves; ++w2) {
                const uint32_t cnt = wc[w2][bb];
                wc[w2][bb] = run;
                run += cnt;
            }
            hist[bb] = run;
        }
        __syncthreads();
        scan();
        __syncthreads();
        write_table();
        if (b != 0xffffffffu) perm[start[b] + wc[w][b] + rank] = (uint32_t)t;
        return;
    }

    for (int b = t; b < nb; b += kGroupThreads) hist[b] = 0;
    __syncthreads();
    for (int64_t v0 = 0; v0 < v_total; v0 += kGroupThreads) {
        const uint32_t b = bucket(v0 + t);
        match(b, [&](uint32_t lb, uint64_t m, int leader) {
            if (lane == leader) atomicAdd(&hist[lb], (uint32_t)__popcll(m));
        });
    }
    __syncthreads();
    scan();
    __syncthreads();
    write_table();
    __syncthreads();
    // stable placement, kGroupThreads vectors a round
    for (int64_t v0 = 0; v0 < v_total; v0 += kGroupThreads) {
        for (int i = t; i < kGroupWaves * kGroupSmallBuckets; i += kGroupThreads) (&wc[0][0])[i] = 0;
        __syncthreads();
        const uint32_t b = bucket(v0 + t);
        uint32_t rank = 0;
        match(b, [&](uint32_t lb, uint64_t m, int leader) {
            if (b == lb) rank = (uint32_t)__popcll(m & lanes_below);
            if (lane == leader) wc[w][lb] = (uint32_t)__popcll(m);
        });
        __syncthreads();
        for (int bb = t; bb < nb; bb += kGroupThreads) {
            uint32_t run = start[bb];
            for (int w2 = 0; w2 < kGroupWaves; ++w2) {
                const uint32_t cnt = wc[w2][bb];
                wc[w2][bb] = run;
                run += cnt;
            }
            start[bb] = run;
        }
        __syncthreads();
        if (b != 0xffffffffu) perm[wc[w][b] + rank] = (uint32_t)(v0 + t);
        __syncthreads();
    }
}

int64_t gather_group_max_chunks(int64_t vectors, int64_t e, int chunk)
{
    return (vectors + chunk - 1) / chunk + e + 1;
}

size_t gather_group_ws_bytes(int64_t vectors, int64_t e, int chunk)
{
    return (size_t)(((vectors + 1 + 3) & ~(int64_t)3) + 4 * gather_group_max_chunks(vectors, e, chunk)) * 4;
}

hipError_t launch_gather_groups(const uint32_t *ids, const uint32_t *lhs, int64_t x_items, int64_t rows,
                                int64_t l, int64_t e, int chunk,
                                void *ws, hipStream_t stream)
{
    if (e + 1 <= kGroupSmallBuckets) {
        gather_group_small_kernel<<<1, kGroupThreads, 0, stream>>>(ids, lhs, x_items, l, (int)e,
                                                                   static_cast<uint32_t *>(ws),
                                                                   rows * l, (uint32_t)chunk);
        return hipGetLastError();
    }
    const size_t lds = (size_t)(2 * (e + 1) + 2 * kGroupThreads + 2) * 4;
    gather_group_kernel<<<1, kGroupThreads, lds, stream>>>(ids, lhs, x_items, rows, l, (int)e,
                                                           static_cast<uint32_t *>(ws), rows * l,
                                                           (uint32_t)chunk);
    return hipGetLastError();
}

namespace {

constexpr int kMaxGridY = 65535;
constexpr int kMaxStageBytes = 64 * 1024;

template <int BITS, typename XT, typename ST, int MR, int RW, int STX>
hipError_t gemv_run(const GemvLaunch &a, hipStream_t stream)
{
    GemvParams<XT, ST> p;
    p.x = static_cast<const XT *>(a.x);
    p.y = static_cast<XT *>(a.y);
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
    p.steps = (int)((a.k + kStepElems - 1) / kStepElems);
    p.chunks_per_item = (int)((a.rows_per_item + MR - 1) / MR);
    p.qrows = a.ksplit >= 4 ? 1 : 4 / a.ksplit;
    const int threads = 64 * a.ksplit * p.qrows;
    const size_t lds = STX > 0 ? (size_t)MR * p.steps * kStageBytesPerStep : 0;
    const int64_t rows_per_block = (int64_t)p.qrows * RW;
    const unsigned gx = (unsigned)((a.n + rows_per_block - 1) / rows_per_block);
    if (a.chunks) {   // grouped gather: one launch over the whole chunk table
        if (a.max_chunks > kMaxGridY) return hipErrorInvalidValue;
        p.item0 = 0;
        gemv_kernel<BITS, XT, ST, MR, RW, STX>
            <<<dim3(gx, (unsigned)a.max_chunks), dim3(threads), lds, stream>>>(p);
        return hipGetLastError();
    }
    const int64_t items_per_launch = std::max<int64_t>(1, kMaxGridY / p.chunks_per_item);
    for (int64_t i0 = 0; i0 < a.items; i0 += items_per_launch) {
        const int64_t cnt = std::min(items_per_launch, a.items - i0);
        p.item0 = i0;
        gemv_kernel<BITS, XT, ST, MR, RW, STX>
            <<<dim3(gx, (unsigned)(cnt * p.chunks_per_item)), dim3(threads), lds, stream>>>(p);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

template <int BITS, typename ST, int STEPS, int NR>
hipError_t gemv_stream_run(const GemvLaunch &a, int64_t groups, hipStream_t stream)
{
    GemvParams<bf16_bits, ST> p{};
    p.x = static_cast<const bf16_bits *>(a.x);
    p.y = static_cast<bf16_bits *>(a.y);
    p.codes = a.codes;
    p.scales = static_cast<const ST *>(a.scales);
    p.biases = static_cast<const ST *>(a.biases);
    p.k = a.k;
    p.n = a.n;
    p.words_per_row = a.k * BITS / 32;
    p.groups_per_row = a.k / a.gs;
    p.gs = a.gs;
    gemv_stream_kernel<BITS, ST, STEPS, NR><<<dim3((unsigned)groups), dim3(64 * kStreamWaves), 0, stream>>>(p);
    return hipGetLastError();
}

template <int BITS, typename ST, int STEPS>
hipError_t gemv_stream_nr(const GemvLaunch &a, hipStream_t stream)
{
    int dev = 0, cus = 0;
    if (hipError_t err = hipGetDevice(&dev)) return err;
    if (hipError_t err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) return err;
    const StreamShape sh = stream_shape(a.n, std::max(cus, 1));
    switch (sh.nr) {
    case 16: return gemv_stream_run<BITS, ST, STEPS, 16>(a, sh.groups, stream);
    case 14: return gemv_stream_run<BITS, ST, STEPS, 14>(a, sh.groups, stream);
    case 12: return gemv_stream_run<BITS, ST, STEPS, 12>(a, sh.groups, stream);
    case 10: return gemv_stream_run<BITS, ST, STEPS, 10>(a, sh.groups, stream);
    default: return gemv_stream_run<BITS, ST, STEPS, 8>(a, sh.groups, stream);
    }
}

// The streaming kernel serves a plain one-row product (no gather) with
// enough weight rows to give every wave 8 or more, K unsplit.
bool gemv_stream_fits(const GemvLaunch &a)
{
    const int64_t steps = (a.k + kStepElems - 1) / kStepElems;
    return a.x_dt == DT_BF16 && a.items == 1 && a.rows_per_item == 1 && !a.idx &&
           !a.chunks && !a.lhs && a.ksplit == 1 && a.rows_per_wave == 0 && steps >= 1 &&
           steps <= kStreamMaxSteps && a.n >= 8 * 1024;
}

template <int BITS, typename ST>
hipError_t gemv_stream(const GemvLaunch &a, hipStream_t stream)
{
    switch ((a.k + kStepElems - 1) / kStepElems) {
    case 1: return gemv_stream_nr<BITS, ST, 1>(a, stream);
    case 2: return gemv_stream_nr<BITS, ST, 2>(a, stream);
    case 3: return gemv_stream_nr<BITS, ST, 3>(a, stream);
    default: return gemv_stream_nr<BITS, ST, 4>(a, stream);
    }
}

// Rows per wave: 2 for one or two activation rows (more waves, shorter
// per-wave work), else 4 (more reuse of the activations).  It does not
// change any row's arithmetic.
template <int BITS, typename XT, typename ST, int MR>
hipError_t gemv_mr(const GemvLaunch &a, hipStream_t stream)
{
    constexpr int RW = MR <= 2 ? 2 : 4;
    if constexpr (MR == 1 && sizeof(XT) == 2) {
        if (gemv_stream_fits(a)) return gemv_stream<BITS, ST>(a, stream);
    }
    if (a.rows_per_wave != 0 && a.rows_per_wave != RW) return hipErrorInvalidValue;
    if constexpr (BITS == 4 && sizeof(XT) == 2 && MR <= 2) {
        const int steps = (int)((a.k + kStepElems - 1) / kStepElems);
        const int threads = 64 * a.ksplit * (a.ksplit >= 4 ? 1 : 4 / a.ksplit);
        const int chunks = MR * steps * 64;
        if (steps > 0 && (size_t)MR * steps * kStageBytesPerStep <= kMaxStageBytes) {
            if (chunks <= threads) return gemv_run<BITS, XT, ST, MR, RW, 1>(a, stream);
            if (chunks <= 2 * threads) return gemv_run<BITS, XT, ST, MR, RW, 2>(a, stream);
            if (chunks <= 4 * threads) return gemv_run<BITS, XT, ST, MR, RW, 4>(a, stream);
        }
    }
    return gemv_run<BITS, XT, ST, MR, RW, 0>(a, stream);
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
    case 1: return gemv_bits<1, XT, ST>(a, stream);
    case 2: return gemv_bits<2, XT, ST>(a, stream);
    case 3: return gemv_bits<3, XT, ST>(a, stream);
    case 4: return gemv_bits<4, XT, ST>(a, stream);
    case 5: return gemv_bits<5, XT, ST>(a, stream);
    case 6: return gemv_bits<6, XT, ST>(a, stream);
    case 8: return gemv_bits<8, XT, ST>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_gemv(const GemvLaunch &a, hipStream_t stream)
{
    if (a.ksplit < 1 || a.ksplit > 8) return hipErrorInvalidValue;
    if (gemv_mfma_family(a.n, a.k, a.gs, a.bits, a.x_dt)) return launch_gemv_mfma(a, stream);
    // the 8-bit matrix-core family takes the plan's own split; an explicit
    // plan with another split runs the VALU kernels
    if (gemv_band_family(a.n, a.k, a.gs, a.bits, a.x_dt) && a.ksplit == kBandKsplit && a.rows_per_wave == 0)
        return launch_gemv_band(a, stream);
    if (a.x_dt == DT_F32) {
        if (a.sb_dt == DT_F32) return gemv_dt<float, float>(a, stream);
        return gemv_dt<float, bf16_bits>(a, stream);
    }
    if (a.sb_dt == DT_F32) return gemv_dt<bf16_bits, float>(a, stream);
    return gemv_dt<bf16_bits, bf16_bits>(a, stream);
}

}  // namespace nqk
