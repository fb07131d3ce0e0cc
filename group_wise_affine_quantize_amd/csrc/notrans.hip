// Products with the weights as stored (transpose = false), and the
// derivatives of quantized products for the scales and biases.
//
// Method: "Quantization" page of the nuvec documentation -- section "Affine"
// (the quantized_matmul flag: x times the weights as stored instead of their
// transpose; the weights' groups then run along the output columns) and
// section "Training through quantized weights" (affine products can be
// differentiated in x and, in affine mode, in the scales and biases; the
// derivative in x is dy times the weights as stored, i.e. this file's
// product with the forward weights, whose rows are the forward outputs).
//
// Notation: the quantized matrix has ni rows of nc columns, grouped along the
// columns: codes [ni, nc*bits/32], scales and biases [ni, nc/gs];
// y[m, c] = sum_i x[m, i] * w_hat[i, c], w_hat = fmaf(s, q, b) in fp32.
#include <algorithm>

#include "nq_device.h"
#include "nq_internal.h"
#include "nq_tiles.h"

namespace nqk {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------------------
// Few activation rows.  Lane L of a workgroup owns the 32 columns
// [2048 bx + 32 L, +32) -- `bits` consecutive code words of every row, read
// coalesced, all in one group; the four waves take the rows i0 + w,
// i0 + w + 4, ... of the workgroup's row range.  Per row, with the row's
// scale s and bias b of that group, the lane adds (x s) q to each column's
// sum and x b to one sum shared by its 32 columns (sum_i x (s q + b) split
// in two), in increasing i;
// waves 1-3 hand their sums to wave 0 through LDS (added in wave order), and
// the workgroup's partial sums go to the workspace.  A second kernel adds the
// row ranges' partials in range order.  The row ranges depend only on ni and
// nc, and nothing in a row's arithmetic depends on the other rows, so every
// row is bit-equal to its one-row product.

template <typename XT, typename ST>
struct NtParams {
    const XT *x;
    const uint32_t *codes;
    const ST *scales;
    const ST *biases;
    float *part;   // [nsplit][MR][nc]
    int64_t m0, ni, nc, words_per_row, groups_per_row, rows_per_split;
    int mrows, lg_gs;
};

constexpr int kNtWaves = 4;

// A lane's 32 codes of a row: `bits` words, 16-, 8- or 4-byte aligned as the
// width allows (every row starts on such a boundary: nc is a multiple of 32).
template <int BITS>
__device__ __forceinline__ void load_run(const uint32_t *src, uint32_t *w)
{
    if constexpr (BITS % 4 == 0) {
#pragma unroll
        for (int u = 0; u < BITS / 4; ++u) {
            const uint4 d = reinterpret_cast<const uint4 *>(src)[u];
            w[4 * u] = d.x, w[4 * u + 1] = d.y, w[4 * u + 2] = d.z, w[4 * u + 3] = d.w;
        }
    } else if constexpr (BITS % 2 == 0) {
#pragma unroll
        for (int u = 0; u < BITS / 2; ++u) {
            const uint2 d = reinterpret_cast<const uint2 *>(src)[u];
            w[2 * u] = d.x, w[2 * u + 1] = d.y;
        }
    } else {
#pragma unroll
        for (int u = 0; u < BITS; ++u) w[u] = src[u];
    }
}

// The 32 codes of a lane's run as fp32 values.  4-bit words are split into
// their even and odd nibbles (kept opaque to the compiler) so that each code
// is one v_cvt_f32_ubyte; 8-bit codes are bytes already.  The values are the
// codes exactly, whichever way they are converted.
template <int BITS>
__device__ __forceinline__ void codes_f32(const uint32_t *w, float *q)
{
    if constexpr (BITS == 4) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            uint32_t lo, hi;
            asm("v_and_b32 %0, 0x0f0f0f0f, %1" : "=v"(lo) : "v"(w[u]));
            asm("v_and_b32 %0, 0x0f0f0f0f, %1" : "=v"(hi) : "v"(w[u] >> 4));
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                q[8 * u + 2 * b] = (float)((lo >> (8 * b)) & 0xffu);
                q[8 * u + 2 * b + 1] = (float)((hi >> (8 * b)) & 0xffu);
            }
        }
    } else if constexpr (BITS == 8) {
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int b = 0; b < 4; ++b) q[4 * u + b] = (float)((w[u] >> (8 * b)) & 0xffu);
    } else {
#pragma unroll
        for (int j = 0; j < kLaneChunk; ++j) q[j] = (float)code_at<BITS>(w, j);
    }
}

// Rows a wave loads before it computes any of them (its rows i, i + 4, ...).
constexpr int kNtUnroll = 4;

template <int BITS, typename XT, typename ST, int MR>
__global__ void __launch_bounds__(64 * kNtWaves) qmm_nt_partial_kernel(NtParams<XT, ST> p)
{
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t c0 = (int64_t)blockIdx.x * kStepElems + lane * kLaneChunk;
    const bool cv = c0 < p.nc;   // nc is a multiple of 32: then c0 + 32 <= nc
    const int64_t cc = cv ? c0 : 0;
    const int64_t g = cc >> p.lg_gs;
    const int64_t i0 = (int64_t)blockIdx.y * p.rows_per_split;
    const int64_t i1 = min(p.ni, i0 + p.rows_per_split);
    float acc[MR][kLaneChunk], bsum[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        bsum[m] = 0.0f;
#pragma unroll
        for (int j = 0; j < kLaneChunk; ++j) acc[m][j] = 0.0f;
    }
    // kNtUnroll rows per pass, all their loads first; rows past i1 read row
    // i1 - 1 and take x = 0 (adding exactly nothing)
    for (int64_t ib = i0 + wave; ib < i1; ib += kNtUnroll * kNtWaves) {
        uint32_t w[kNtUnroll][BITS];
        float s[kNtUnroll], b[kNtUnroll], xv[kNtUnroll][MR];
#pragma unroll
        for (int u = 0; u < kNtUnroll; ++u) {
            const int64_t iu = ib + (int64_t)u * kNtWaves;
            const bool ok = iu < i1;
            const int64_t i = ok ? iu : i1 - 1;
            load_run<BITS>(p.codes + i * p.words_per_row + (cc / kLaneChunk) * BITS, w[u]);
            s[u] = Elt<ST>::load(p.scales, i * p.groups_per_row + g);
            b[u] = Elt<ST>::load(p.biases, i * p.groups_per_row + g);
#pragma unroll
            for (int m = 0; m < MR; ++m)
                xv[u][m] = ok ? Elt<XT>::load(p.x, (p.m0 + min(m, p.mrows - 1)) * p.ni + i) : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < kNtUnroll; ++u) {
            float xs[MR];
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                xs[m] = xv[u][m] * s[u];
                bsum[m] = fmaf(xv[u][m], b[u], bsum[m]);
            }
            float qf[kLaneChunk];
            codes_f32<BITS>(w[u], qf);
#pragma unroll
            for (int j = 0; j < kLaneChunk; ++j)
#pragma unroll
                for (int m = 0; m < MR; ++m) acc[m][j] = fmaf(xs[m], qf[j], acc[m][j]);
        }
    }
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int j = 0; j < kLaneChunk; ++j) acc[m][j] += bsum[m];
    __shared__ float red[kNtWaves - 1][MR][kLaneChunk][64];
    if (wave > 0) {
#pragma unroll
        for (int m = 0; m < MR; ++m)
#pragma unroll
            for (int j = 0; j < kLaneChunk; ++j) red[wave - 1][m][j][lane] = acc[m][j];
    }
    __syncthreads();
    if (wave != 0 || !cv) return;
#pragma unroll
    for (int w2 = 0; w2 < kNtWaves - 1; ++w2)
#pragma unroll
        for (int m = 0; m < MR; ++m)
#pragma unroll
            for (int j = 0; j < kLaneChunk; ++j) acc[m][j] += red[w2][m][j][lane];
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        if (m >= p.mrows) break;
        float4 *dst = reinterpret_cast<float4 *>(p.part + ((int64_t)blockIdx.y * MR + m) * p.nc + c0);
#pragma unroll
        for (int j = 0; j < kLaneChunk / 4; ++j)
            dst[j] = make_float4(acc[m][4 * j], acc[m][4 * j + 1], acc[m][4 * j + 2], acc[m][4 * j + 3]);
    }
}

// y[m0 + m, c] = the row ranges' partials, added in a fixed order: a
// workgroup takes 64 outputs, and its thread q * 64 + t adds the ranges of
// part q (of kNtRedParts equal parts) of output t in increasing order; the
// part sums are then added in part order.
constexpr int kNtRedCols = 64;
constexpr int kNtRedParts = 16;

template <typename XT, int MR>
__global__ void __launch_bounds__(kNtRedCols * kNtRedParts)
qmm_nt_reduce_kernel(const float *part, XT *y, int64_t m0, int mrows, int64_t nc, int nsplit)
{
    const int t = threadIdx.x & (kNtRedCols - 1), qt = threadIdx.x / kNtRedCols;
    const int64_t idx = (int64_t)blockIdx.x * kNtRedCols + t;
    const bool ok = idx < (int64_t)mrows * nc;
    const int64_t m = ok ? idx / nc : 0, c = ok ? idx % nc : 0;
    const int per = (nsplit + kNtRedParts - 1) / kNtRedParts;
    const int s0 = min(nsplit, qt * per), s1 = min(nsplit, s0 + per);
    float sum = 0.0f;
    int sp = s0;
    for (; sp + 8 <= s1; sp += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = part[((int64_t)(sp + u) * MR + m) * nc + c];
#pragma unroll
        for (int u = 0; u < 8; ++u) sum += v[u];
    }
    for (; sp < s1; ++sp) sum += part[((int64_t)sp * MR + m) * nc + c];
    __shared__ float qs[kNtRedParts - 1][kNtRedCols];
    if (qt > 0) qs[qt - 1][t] = sum;
    __syncthreads();
    if (qt == 0 && ok) {
#pragma unroll
        for (int q = 0; q < kNtRedParts - 1; ++q) sum += qs[q][t];
        Elt<XT>::store(y, (m0 + m) * nc + c, sum);
    }
}

// ---------------------------------------------------------------------------
// Many rows (bf16 x): 128 x 128 tiles of y with bf16 MFMA, as the tiled
// product with the transposed weights, but the weight tile of a K step (64
// rows i of 128 columns c) is dequantized from the rows as stored and written
// to LDS transposed, [c][i], so that the B operands read 8 consecutive i of
// one column.  Each thread dequantizes 32 columns of one row (a run of
// codes that starts on a word) into round_bf16(fmaf(s, q, b)).  The tiles are
// double buffered in LDS and a step's global loads are issued two steps
// ahead, so they are in flight while the matrix cores run.

template <typename ST>
struct NtTiledParams {
    const bf16_bits *x;   // [m, ni]
    bf16_bits *y;         // [m, nc]
    const uint32_t *codes;
    const ST *scales;
    const ST *biases;
    int64_t m, ni, nc, words_per_row, groups_per_row;
    int lg_gs;
};

constexpr int kNtTM = 128, kNtTN = 128, kNtBK = 64, kNtLd = kNtBK + 8;
// Column c of the transposed weight tile starts at c * kNtLd + 16 * ((c / 16) % 8)
// elements.  With the plain stride the writes of a wave all fall in the same
// few LDS banks: a column start is 36 c dwords, i.e. the same bank for every
// 16 columns.  The shift, 8 dwords per 16 columns, spreads them: the 4-byte
// writes of a wave (8 row pairs x 8 groups of 16 columns) land in 64
// distinct banks, the 2-byte writes (16 rows x 4 groups of 32 columns) in 32
// distinct dwords; and the 16 columns one B-operand read phase touches share
// a shift, so the reads stay conflict-free.
__device__ __forceinline__ int nt_wcol(int c) { return c * kNtLd + 16 * ((c >> 4) & 7); }
constexpr int kNtWsElems = kNtTN * kNtLd + 128;

template <int BITS, typename ST>
__global__ void __launch_bounds__(256) tiled_nt_kernel(NtTiledParams<ST> p)
{
    // two LDS buffers for the x and weight tiles: step j is staged into
    // buffer j % 2 while the MFMAs of step j - 1 read the other one
    __shared__ __attribute__((aligned(16))) bf16_bits xs[2][kNtTM * kNtLd];
    __shared__ __attribute__((aligned(16))) bf16_bits ws[2][kNtWsElems];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    int tm, tn;
    if (!xcd_panel_tile(blockIdx.x, (int)((p.m + kNtTM - 1) / kNtTM), (int)((p.nc + kNtTN - 1) / kNtTN), tm, tn))
        return;
    const int64_t m0 = (int64_t)tm * kNtTM;
    const int64_t c0 = (int64_t)tn * kNtTN;
    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_t{};

    const int lrow = tid >> 1, lhalf = tid & 1;          // x loader: one row, 32 elements
    const int64_t xm = m0 + lrow;
    // Weight loader.  Widths 2, 4 and 8 (PAIR): thread t takes rows
    // 2 (t / 8) and 2 (t / 8) + 1 of the step and the 16 columns from
    // 16 (t % 8), and writes the two rows' values of a column into LDS as one
    // 4-byte word.  Other widths: row t / 4, the 32 columns from 32 (t % 4),
    // 2-byte writes.  Either way a thread's columns lie inside one group and
    // its codes start on a word boundary.
    constexpr bool PAIR = BITS == 2 || BITS == 4 || BITS == 8;
    constexpr int NR = PAIR ? 2 : 1;                      // rows per thread
    constexpr int NCOL = PAIR ? 16 : 32;                  // columns per thread
    constexpr int NW = NCOL * BITS / 32;                  // code words per row
    const int wrow = PAIR ? 2 * (tid >> 3) : tid >> 2;
    const int wcol = PAIR ? 16 * (tid & 7) : 32 * (tid & 3);
    const int64_t cb = c0 + wcol;
    const bool wv_ok = cb < p.nc;                         // nc % 32 == 0: then cb + NCOL <= nc
    const int64_t g = (wv_ok ? cb : 0) >> p.lg_gs;

    // One K step's global data for this thread: 32 activations, the codes of
    // its rows and the raw storage bits of their scales and biases
    // (converted only when used, so that no conversion waits on the load
    // early).
    struct Ld {
        uint4 x[4];
        uint32_t raw[NR][NW];
        uint32_t s[NR], b[NR];
    };
    // Rows past m read row m - 1 and columns past nc read column 0: their
    // products land only in outputs past m or nc, which are never stored.
    const int64_t xmc = min(xm, p.m - 1);
    const int64_t cbc = wv_ok ? cb : 0;
    auto raw_of = [](const ST *a, int64_t i) -> uint32_t {
        if constexpr (sizeof(ST) == 2) return (uint32_t)a[i];
        else return __float_as_uint(a[i]);
    };
    auto f32_of = [](uint32_t v) -> float { return sizeof(ST) == 2 ? __uint_as_float(v << 16) : __uint_as_float(v); };
    auto load = [&](int step, Ld &l) {
        const int64_t i0 = (int64_t)step * kNtBK;
        const uint4 *src = reinterpret_cast<const uint4 *>(p.x + xmc * p.ni + i0 + 32 * lhalf);
#pragma unroll
        for (int u = 0; u < 4; ++u) l.x[u] = src[u];
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const int64_t i = i0 + wrow + r;
            l.s[r] = raw_of(p.scales, i * p.groups_per_row + g);
            l.b[r] = raw_of(p.biases, i * p.groups_per_row + g);
            const uint32_t *src = p.codes + i * p.words_per_row + ((cbc * BITS) >> 5);
            if constexpr (NW == 4) {
                const uint4 d = *reinterpret_cast<const uint4 *>(src);
                l.raw[r][0] = d.x, l.raw[r][1] = d.y, l.raw[r][2] = d.z, l.raw[r][3] = d.w;
            } else if constexpr (NW == 2) {
                const uint2 d = *reinterpret_cast<const uint2 *>(src);
                l.raw[r][0] = d.x, l.raw[r][1] = d.y;
            } else if constexpr (NW == 1) {
                l.raw[r][0] = *src;
            } else {
                load_run<BITS>(src, l.raw[r]);
            }
        }
    };
    typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
    typedef float f32x2_v __attribute__((ext_vector_type(2)));
    // dequantize a step's weights, round_bf16(fmaf(s, q, b)), and write them
    // with its activations into LDS buffer B (the weights transposed)
    auto stage = [&](const Ld &l, auto bufc) {
        constexpr int B = decltype(bufc)::value;
        uint4 *xd = reinterpret_cast<uint4 *>(xs[B] + lrow * kNtLd + 32 * lhalf);
#pragma unroll
        for (int u = 0; u < 4; ++u) xd[u] = make_uint4(l.x[u].x, l.x[u].y, l.x[u].z, l.x[u].w);
        // v_cvt_pk_bf16_f32: round to nearest even, as f32_to_bf16 for finite values
        if constexpr (PAIR) {
            float q0[kLaneChunk], q1[kLaneChunk];
            uint32_t w0[BITS] = {}, w1[BITS] = {};   // the first NW words hold the 16 codes
#pragma unroll
            for (int j = 0; j < NW; ++j) w0[j] = l.raw[0][j], w1[j] = l.raw[1][j];
            codes_f32<BITS>(w0, q0);
            codes_f32<BITS>(w1, q1);
            const float s0 = f32_of(l.s[0]), b0 = f32_of(l.b[0]);
            const float s1 = f32_of(l.s[1]), b1 = f32_of(l.b[1]);
#pragma unroll
            for (int u = 0; u < NCOL; ++u) {
                const f32x2_v f = {fmaf(s0, q0[u], b0), fmaf(s1, q1[u], b1)};
                *reinterpret_cast<uint32_t *>(&ws[B][nt_wcol(wcol + u) + wrow]) =
                    __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_v));
            }
        } else {
            const float sc = f32_of(l.s[0]), bi = f32_of(l.b[0]);
            float qf[kLaneChunk];
            codes_f32<BITS>(l.raw[0], qf);
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const f32x2_v f = {fmaf(sc, qf[2 * u], bi), fmaf(sc, qf[2 * u + 1], bi)};
                const uint32_t pk = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_v));
                ws[B][nt_wcol(wcol + 2 * u) + wrow] = (bf16_bits)(pk & 0xffffu);
                ws[B][nt_wcol(wcol + 2 * u + 1) + wrow] = (bf16_bits)(pk >> 16);
            }
        }
    };
    auto mfmas = [&](auto bufc) {
        constexpr int B = decltype(bufc)::value;
#pragma unroll
        for (int ks = 0; ks < kNtBK / 16; ++ks) {
            const int kk = ks * 16 + 8 * (lane >> 5);
            bf16x8_t a[2], bo[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                a[i] = *reinterpret_cast<const bf16x8_t *>(xs[B] + (wm * 64 + i * 32 + (lane & 31)) * kNtLd + kk);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                bo[j] = *reinterpret_cast<const bf16x8_t *>(ws[B] + nt_wcol(wn * 64 + j * 32 + (lane & 31)) + kk);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], bo[j], acc[i][j], 0, 0, 0);
        }
    };

    tile_pipeline<Ld>((int)(p.ni / kNtBK), load, stage, mfmas);   // ni is a multiple of 64
    // D layout: lane l holds column l % 32 and rows 8 (v / 4) + 4 (l / 32) + v % 4
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t col = c0 + wn * 64 + j * 32 + (lane & 31);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t row = m0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                if (row < p.m && col < p.nc) p.y[row * p.nc + col] = (bf16_bits)f32_to_bf16(acc[i][j][v]);
            }
        }
}

// ---------------------------------------------------------------------------
// Derivatives for the scales and biases of the product with the transposed
// weights (codes [n, k*bits/32]):
//   ds[c, g] = sum_m dy[m, c] * sum_{k in g} x[m, k] q[c, k]
//   db[c, g] = sum_m dy[m, c] * sum_{k in g} x[m, k]
// A wave owns RW weight rows c; in K step t lane L owns the 32 columns
// [2048 t + 32 L, +32) (inside one group).  For every activation row m the
// lane forms sum x q and sum x over its columns and adds dy[m, c] times them,
// in increasing m; the gs / 32 lanes of a group are then added by a fixed xor
// tree, and the group's first lane stores.

template <typename XT, typename GT>
struct GradParams {
    const XT *x;    // [m, k]
    const XT *dy;   // [m, n]
    const uint32_t *codes;
    GT *ds;         // [n, k/gs]
    GT *db;
    int64_t m, k, n, words_per_row, groups_per_row;
    int lg_gs, steps;
};

constexpr int kGradRows = 4;   // weight rows per wave

template <int OFF>
__device__ __forceinline__ float xor_sum(float v)
{
    // v + v from lane (lane ^ OFF), OFF in {1, 2}: DPP quad permutes
    const int iv = __float_as_int(v);
    const int r = OFF == 1 ? __builtin_amdgcn_mov_dpp(iv, 0xB1, 0xF, 0xF, true)
                           : __builtin_amdgcn_mov_dpp(iv, 0x4E, 0xF, 0xF, true);
    return v + __int_as_float(r);
}

template <int BITS, typename XT, typename GT, bool VEC>
__global__ void __launch_bounds__(256) grad_sb_kernel(GradParams<XT, GT> p)
{
    // VEC: x and the codes are 16-byte aligned, so a lane's 32 activations
    // and its run of codes are read with 16-byte loads (same values)
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t r0 = ((int64_t)blockIdx.x * 4 + wave) * kGradRows;
    const int lpg = 1 << (p.lg_gs - 5);   // lanes per group: 1, 2 or 4
    for (int t = 0; t < p.steps; ++t) {
        const int64_t e0 = (int64_t)t * kStepElems + lane * kLaneChunk;
        const bool on = e0 < p.k;
        const int64_t ec = on ? e0 : 0;
        // the codes of this step, as fp32 values, for all activation rows
        float qf[kGradRows][kLaneChunk];
#pragma unroll
        for (int r = 0; r < kGradRows; ++r) {
            const int64_t c = min(r0 + r, p.n - 1);
            const uint32_t *src = p.codes + c * p.words_per_row + (ec / kLaneChunk) * BITS;
            uint32_t w[BITS];
            if constexpr (VEC) {
                load_run<BITS>(src, w);
            } else {
#pragma unroll
                for (int u = 0; u < BITS; ++u) w[u] = src[u];
            }
            codes_f32<BITS>(w, qf[r]);
        }
        float as[kGradRows], ab[kGradRows];
#pragma unroll
        for (int r = 0; r < kGradRows; ++r) as[r] = ab[r] = 0.0f;
        for (int64_t m = 0; m < p.m; ++m) {
            float xf[kLaneChunk];
            float X = 0.0f;
            if constexpr (VEC) {
                load32_f32<XT>(p.x + m * p.k + ec, xf);
            } else {
#pragma unroll
                for (int j = 0; j < kLaneChunk; ++j) xf[j] = Elt<XT>::load(p.x, m * p.k + ec + j);
            }
#pragma unroll
            for (int j = 0; j < kLaneChunk; ++j) X += xf[j];
#pragma unroll
            for (int r = 0; r < kGradRows; ++r) {
                float T = 0.0f;
#pragma unroll
                for (int j = 0; j < kLaneChunk; ++j) T = fmaf(xf[j], qf[r][j], T);
                const float d = Elt<XT>::load(p.dy, m * p.n + min(r0 + r, p.n - 1));
                as[r] = fmaf(d, T, as[r]);
                ab[r] = fmaf(d, X, ab[r]);
            }
        }
#pragma unroll
        for (int r = 0; r < kGradRows; ++r) {
            if (lpg >= 2) as[r] = xor_sum<1>(as[r]), ab[r] = xor_sum<1>(ab[r]);
            if (lpg >= 4) as[r] = xor_sum<2>(as[r]), ab[r] = xor_sum<2>(ab[r]);
            if (on && (lane & (lpg - 1)) == 0 && r0 + r < p.n) {
                const int64_t o = (r0 + r) * p.groups_per_row + (e0 >> p.lg_gs);
                Elt<GT>::store(p.ds, o, as[r]);
                Elt<GT>::store(p.db, o, ab[r]);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Launchers

namespace {

int lg_of(int gs) { return gs == 32 ? 5 : gs == 64 ? 6 : 7; }

template <int BITS, typename XT, typename ST, int MR>
hipError_t qmm_nt_run(const NtLaunch &a, hipStream_t stream)
{
    NtParams<XT, ST> p;
    p.x = static_cast<const XT *>(a.x);
    p.codes = a.codes;
    p.scales = static_cast<const ST *>(a.scales);
    p.biases = static_cast<const ST *>(a.biases);
    p.part = static_cast<float *>(a.workspace);
    p.ni = a.ni;
    p.nc = a.nc;
    p.words_per_row = a.nc * BITS / 32;
    p.groups_per_row = a.nc / a.gs;
    p.lg_gs = lg_of(a.gs);
    const int nsplit = qmm_nt_splits(a.ni, a.nc);
    p.rows_per_split = (a.ni + nsplit - 1) / nsplit;
    const unsigned gx = (unsigned)((a.nc + kStepElems - 1) / kStepElems);
    for (int64_t m0 = 0; m0 < a.m; m0 += MR) {
        p.m0 = m0;
        p.mrows = (int)std::min<int64_t>(MR, a.m - m0);
        qmm_nt_partial_kernel<BITS, XT, ST, MR><<<dim3(gx, (unsigned)nsplit), dim3(64 * kNtWaves), 0, stream>>>(p);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
        const int64_t outs = (int64_t)p.mrows * a.nc;
        qmm_nt_reduce_kernel<XT, MR><<<dim3((unsigned)((outs + kNtRedCols - 1) / kNtRedCols)),
                                      dim3(kNtRedCols * kNtRedParts), 0, stream>>>(
            p.part, static_cast<XT *>(a.y), m0, p.mrows, a.nc, nsplit);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    return hipSuccess;
}

template <int BITS, typename ST>
hipError_t tiled_nt_run(const NtLaunch &a, hipStream_t stream)
{
    NtTiledParams<ST> p;
    p.x = static_cast<const bf16_bits *>(a.x);
    p.y = static_cast<bf16_bits *>(a.y);
    p.codes = a.codes;
    p.scales = static_cast<const ST *>(a.scales);
    p.biases = static_cast<const ST *>(a.biases);
    p.m = a.m;
    p.ni = a.ni;
    p.nc = a.nc;
    p.words_per_row = a.nc * BITS / 32;
    p.groups_per_row = a.nc / a.gs;
    p.lg_gs = lg_of(a.gs);
    if (a.ni % kNtBK != 0) return hipErrorInvalidValue;
    const int64_t tiles = ((a.nc + kNtTN - 1) / kNtTN) * ((a.m + kNtTM - 1) / kNtTM);
    const unsigned blocks = xcd_panel_blocks(tiles);
    if (blocks == 0) return hipErrorInvalidValue;
    tiled_nt_kernel<BITS, ST><<<dim3(blocks), dim3(256), 0, stream>>>(p);
    return hipGetLastError();
}

template <int BITS, typename XT, typename ST>
hipError_t nt_bits(const NtLaunch &a, hipStream_t stream)
{
    if (a.tiled) {
        if constexpr (sizeof(XT) == 2) return tiled_nt_run<BITS, ST>(a, stream);
        else return hipErrorInvalidValue;
    }
    // one activation row per pass for single-row calls (the same arithmetic per row)
    if (a.m == 1) return qmm_nt_run<BITS, XT, ST, 1>(a, stream);
    return qmm_nt_run<BITS, XT, ST, kNtRowsPerChunk>(a, stream);
}

template <typename XT, typename ST>
hipError_t nt_dt(const NtLaunch &a, hipStream_t stream)
{
    switch (a.bits) {
    case 1: return nt_bits<1, XT, ST>(a, stream);
    case 2: return nt_bits<2, XT, ST>(a, stream);
    case 3: return nt_bits<3, XT, ST>(a, stream);
    case 4: return nt_bits<4, XT, ST>(a, stream);
    case 5: return nt_bits<5, XT, ST>(a, stream);
    case 6: return nt_bits<6, XT, ST>(a, stream);
    case 8: return nt_bits<8, XT, ST>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

template <int BITS, typename XT, typename GT>
hipError_t grad_run(const GradLaunch &a, hipStream_t stream)
{
    GradParams<XT, GT> p;
    p.x = static_cast<const XT *>(a.x);
    p.dy = static_cast<const XT *>(a.dy);
    p.codes = a.codes;
    p.ds = static_cast<GT *>(a.ds);
    p.db = static_cast<GT *>(a.db);
    p.m = a.m;
    p.k = a.k;
    p.n = a.n;
    p.words_per_row = a.k * BITS / 32;
    p.groups_per_row = a.k / a.gs;
    p.lg_gs = lg_of(a.gs);
    p.steps = (int)((a.k + kStepElems - 1) / kStepElems);
    const unsigned gx = (unsigned)((a.n + 4 * kGradRows - 1) / (4 * kGradRows));
    if ((((uintptr_t)a.x | (uintptr_t)a.codes) & 15) == 0)
        grad_sb_kernel<BITS, XT, GT, true><<<dim3(gx), dim3(256), 0, stream>>>(p);
    else
        grad_sb_kernel<BITS, XT, GT, false><<<dim3(gx), dim3(256), 0, stream>>>(p);
    return hipGetLastError();
}

template <typename XT, typename GT>
hipError_t grad_dt(const GradLaunch &a, hipStream_t stream)
{
    switch (a.bits) {
    case 1: return grad_run<1, XT, GT>(a, stream);
    case 2: return grad_run<2, XT, GT>(a, stream);
    case 3: return grad_run<3, XT, GT>(a, stream);
    case 4: return grad_run<4, XT, GT>(a, stream);
    case 5: return grad_run<5, XT, GT>(a, stream);
    case 6: return grad_run<6, XT, GT>(a, stream);
    case 8: return grad_run<8, XT, GT>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

int qmm_nt_splits(int64_t ni, int64_t nc)
{
    // about 512 workgroups, and at least 16 rows (4 per wave) per range
    const int64_t col_blocks = (nc + kStepElems - 1) / kStepElems;
    const int64_t want = std::max<int64_t>(1, (512 + col_blocks - 1) / col_blocks);
    const int64_t most = std::max<int64_t>(1, (ni + 15) / 16);
    return (int)std::min<int64_t>(std::min(want, most), 65535);
}

size_t qmm_nt_ws_bytes(int64_t ni, int64_t nc)
{
    return (size_t)qmm_nt_splits(ni, nc) * kNtRowsPerChunk * (size_t)nc * sizeof(float);
}

hipError_t launch_qmm_nt(const NtLaunch &a, hipStream_t stream)
{
    if (a.x_dt == DT_F32) {
        if (a.sb_dt == DT_F32) return nt_dt<float, float>(a, stream);
        return nt_dt<float, bf16_bits>(a, stream);
    }
    if (a.sb_dt == DT_F32) return nt_dt<bf16_bits, float>(a, stream);
    return nt_dt<bf16_bits, bf16_bits>(a, stream);
}

hipError_t launch_grad_sb(const GradLaunch &a, hipStream_t stream)
{
    if (a.x_dt == DT_F32) {
        if (a.g_dt == DT_F32) return grad_dt<float, float>(a, stream);
        return grad_dt<float, bf16_bits>(a, stream);
    }
    if (a.g_dt == DT_F32) return grad_dt<bf16_bits, float>(a, stream);
    return grad_dt<bf16_bits, bf16_bits>(a, stream);
}

}  // namespace nqk
