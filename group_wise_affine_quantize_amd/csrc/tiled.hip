// Tiled quantized product for many rows on gfx950 matrix cores.
//
// Method: "Quantization" page of the nuvec documentation, sections "Affine"
// (w ~ scale * code + bias per group, product x times the transposed
// weights) and "Products on the GPU" (tiled kernels for many rows).
//
// y[m, n] = sum_k x[m, k] * w_hat[n, k] with x, y in bf16 and fp32
// accumulation.  Each workgroup owns a TM x TN tile of y.  Per K step of 32
// elements (one 32-code chunk per weight row, inside one group) it stages the
// x tile in LDS, dequantizes the weight tile into LDS as bf16 -- the value of
// the stand-alone dequantize, round_bf16(fmaf(scale, code, bias)) -- and
// runs v_mfma_f32_32x32x16_bf16 over it.  Four waves split the tile 2 x 2.
#include <type_traits>

#include "nq_device.h"
#include "nq_internal.h"

namespace nqk {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

template <typename ST>
struct TiledParams {
    const bf16_bits *x;
    bf16_bits *y;
    const uint32_t *codes;
    const ST *scales;
    const ST *biases;
    int64_t m, n, k, words_per_row, groups_per_row;
    int gs, lg_gs;   // group size and its base-2 logarithm
};

constexpr int kTM = 128, kTN = 128, kBK = 32, kPad = 8, kLd = kBK + kPad;

template <int BITS, typename ST>
__global__ void __launch_bounds__(256) tiled_kernel(TiledParams<ST> p)
{
    __shared__ __attribute__((aligned(16))) bf16_bits xs[kTM * kLd];
    __shared__ __attribute__((aligned(16))) bf16_bits ws[kTN * kLd];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t m0 = (int64_t)blockIdx.y * kTM;
    const int64_t n0 = (int64_t)blockIdx.x * kTN;

    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    const int lrow = tid >> 1, lhalf = tid & 1;   // loader: one row, 16 elements
    const int64_t xm = m0 + lrow, wr = n0 + lrow;

    for (int64_t k0 = 0; k0 < p.k; k0 += kBK) {
        // x tile: 16 bf16 (two 16-byte loads) per thread
        uint4 xa = make_uint4(0u, 0u, 0u, 0u), xb = xa;
        if (xm < p.m) {
            const uint4 *src = reinterpret_cast<const uint4 *>(p.x + xm * p.k + k0 + 16 * lhalf);
            xa = src[0];
            xb = src[1];
        }
        // weight tile: 16 codes of one row, dequantized to bf16
        uint32_t outw[8];
        if (wr < p.n) {
            const int64_t e0 = k0 + 16 * lhalf;
            const float s = Elt<ST>::load(p.scales, wr * p.groups_per_row + e0 / p.gs);
            const float b = Elt<ST>::load(p.biases, wr * p.groups_per_row + e0 / p.gs);
            // the 16 codes start at bit e0 * BITS of the row: 16 bits into a
            // word for odd widths and odd halves.  Load the (BITS + 1) / 2
            // words they touch (no more: all inside the row) and realign.
            constexpr int NW = (BITS + 1) / 2;
            const int64_t bit0 = e0 * BITS;
            const uint32_t *src = p.codes + wr * p.words_per_row + (bit0 >> 5);
            const uint32_t sh = (uint32_t)(bit0 & 31);
            uint32_t raw[NW], cw[NW];
#pragma unroll
            for (int i = 0; i < NW; ++i) raw[i] = src[i];
#pragma unroll
            for (int i = 0; i < NW; ++i) cw[i] = __builtin_amdgcn_alignbit(i + 1 < NW ? raw[i + 1] : 0u, raw[i], sh);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float v0 = fmaf(s, (float)code_at<BITS>(cw, 2 * i), b);
                const float v1 = fmaf(s, (float)code_at<BITS>(cw, 2 * i + 1), b);
                outw[i] = f32_to_bf16(v0) | (f32_to_bf16(v1) << 16);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) outw[i] = 0u;
        }
        __syncthreads();   // previous step's MFMA reads are done
        uint4 *xd = reinterpret_cast<uint4 *>(xs + lrow * kLd + 16 * lhalf);
        xd[0] = xa;
        xd[1] = xb;
        uint4 *wd = reinterpret_cast<uint4 *>(ws + lrow * kLd + 16 * lhalf);
        wd[0] = make_uint4(outw[0], outw[1], outw[2], outw[3]);
        wd[1] = make_uint4(outw[4], outw[5], outw[6], outw[7]);
        __syncthreads();

#pragma unroll
        for (int ks = 0; ks < kBK / 16; ++ks) {
            const int kk = ks * 16 + 8 * (lane >> 5);
            bf16x8_t a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int row = wm * 64 + i * 32 + (lane & 31);
                a[i] = *reinterpret_cast<const bf16x8_t *>(xs + row * kLd + kk);
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int row = wn * 64 + j * 32 + (lane & 31);
                b[j] = *reinterpret_cast<const bf16x8_t *>(ws + row * kLd + kk);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    }

    // D layout of the 32x32 MFMA: lane l holds column l % 32 and rows
    // 8 * (v / 4) + 4 * (l / 32) + v % 4 for v = 0..15.
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t col = n0 + wn * 64 + j * 32 + (lane & 31);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t row = m0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                if (row < p.m && col < p.n) p.y[row * p.n + col] = (bf16_bits)f32_to_bf16(acc[i][j][v]);
            }
        }
}

// ---------------------------------------------------------------------------
// 256 x 256 tiles for large products (K a multiple of 64).
//
// Four waves; wave w owns weight rows [64 w, 64 w + 64) of the tile (two
// 32-column MFMA blocks) and all 256 rows of x (eight 32-row blocks):
// 16 v_mfma_f32_32x32x16_bf16 accumulators.  Per K block of 64:
//   - x (256 x 64 bf16 = 32 KB) goes straight from global memory into an LDS
//     buffer (global_load_lds_dwordx4), double buffered.  In LDS a row is 8
//     16-byte chunks; chunk c of row r sits at position c ^ ((r / 2) % 8), so
//     the 16 rows one 16-lane pass of a 128-bit operand read touches land in
//     16 distinct 16-byte bank groups (64 banks).
//   - each wave dequantizes only its own 64 weight rows, straight into
//     B-operand registers: lane (n = l % 32, h = l / 32) holds, for k16 step
//     j, the 8 codes k = 32 h + 8 j + 0..7 of weight row n, i.e. one 4-bit
//     code word (two 8-bit ones), converted as round_bf16(fmaf(s, q, b)) --
//     the value of the stand-alone dequantize.  The A operand uses the same
//     k assignment: x[m][32 h + 8 j + 0..7].
//   - codes, scales and biases reach the B-operand lanes through wave-private
//     LDS rings (two stages each; a codes stage is 128 bytes of each of the
//     wave's rows, 4 K blocks at 4 bits and 2 at 8 bits, swizzled like x; a
//     scale/bias stage is 8 groups of each row).  The rings are filled by
//     ordinary loads whose every instruction covers whole 128-byte row
//     segments (the B-operand layout would touch 32 rows per instruction and
//     use 16 or 2 bytes of each), kept in registers for two blocks to hide
//     their latency, then written with ds_write.
//   - B operands of the next block are dequantized during the MFMAs of the
//     current one (rolling, one register set); A operands are read one k16
//     step ahead, across block boundaries too.
// Tile order is XCD-aware: workgroups go to the 8 XCDs round-robin, and XCD
// x takes the x-th eighth of the column-major tile list, i.e. a band of
// weight columns: each XCD's L2 sees an eighth of the weights (instead of
// all of them, as with row-major bands of x), which measured faster.

constexpr int kBM = 256, kBN = 256, kBK2 = 64;
// Ring geometry in LDS (bytes)
constexpr int kCodeRowBytes = 128;                    // per row per stage
constexpr int kCodeStageBytes = 64 * kCodeRowBytes;   // one wave's 64 rows: 8 KB
constexpr int kSbGroups = 8;                          // groups per row per stage
template <typename ST>
constexpr int sb_row_bytes() { return kSbGroups * (int)sizeof(ST); }
template <typename ST>
constexpr int sb_stage_bytes() { return 2 * 64 * sb_row_bytes<ST>(); }   // scales, then biases

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi)
{
    const f32x2_t f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

__device__ __forceinline__ uint32_t u4_at(const uint4 &v, int i)
{
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;   // i is a constant after unrolling
}

// A lane's codes of one K block (32 codes) with its scale and bias.
template <int BITS>
struct CodeRegs {
    uint4 w[BITS / 4];
    uint32_t s, b;          // raw scale / bias storage bits
};

// Codes of k16 step j (8 of the lane's 32) -> one B operand of 8 bf16.
template <int BITS, typename ST>
__device__ __forceinline__ bf16x8_t dequant_step(const CodeRegs<BITS> &c, int j)
{
    const float s = sizeof(ST) == 2 ? __uint_as_float(c.s << 16) : __uint_as_float(c.s);
    const float b = sizeof(ST) == 2 ? __uint_as_float(c.b << 16) : __uint_as_float(c.b);
    float v[8];
    if constexpr (BITS == 4) {
        const uint32_t w = u4_at(c.w[0], j);
        // lo holds codes 0, 2, 4, 6 and hi codes 1, 3, 5, 7 in its four bytes;
        // the masks are kept opaque so that each code is one
        // v_cvt_f32_ubyte{0..3} instead of a bit-field extract plus a convert
        uint32_t lo, hi;
        asm("v_and_b32 %0, 0x0f0f0f0f, %1" : "=v"(lo) : "v"(w));
        asm("v_and_b32 %0, 0x0f0f0f0f, %1" : "=v"(hi) : "v"(w >> 4));
        v[0] = (float)(lo & 0xffu), v[1] = (float)(hi & 0xffu);
        v[2] = (float)((lo >> 8) & 0xffu), v[3] = (float)((hi >> 8) & 0xffu);
        v[4] = (float)((lo >> 16) & 0xffu), v[5] = (float)((hi >> 16) & 0xffu);
        v[6] = (float)(lo >> 24), v[7] = (float)(hi >> 24);
    } else {
        const uint32_t w0 = u4_at(c.w[j / 2], 2 * (j % 2));
        const uint32_t w1 = u4_at(c.w[j / 2], 2 * (j % 2) + 1);
        v[0] = (float)(w0 & 0xffu), v[1] = (float)((w0 >> 8) & 0xffu);
        v[2] = (float)((w0 >> 16) & 0xffu), v[3] = (float)(w0 >> 24);
        v[4] = (float)(w1 & 0xffu), v[5] = (float)((w1 >> 8) & 0xffu);
        v[6] = (float)((w1 >> 16) & 0xffu), v[7] = (float)(w1 >> 24);
    }
    uint4 o;
    o.x = pack_bf16(fmaf(s, v[0], b), fmaf(s, v[1], b));
    o.y = pack_bf16(fmaf(s, v[2], b), fmaf(s, v[3], b));
    o.z = pack_bf16(fmaf(s, v[4], b), fmaf(s, v[5], b));
    o.w = pack_bf16(fmaf(s, v[6], b), fmaf(s, v[7], b));
    return __builtin_bit_cast(bf16x8_t, o);
}

template <int BITS, typename ST>
__global__ void __launch_bounds__(256) tiled256_kernel(TiledParams<ST> p, int tiles_m, int tiles_n,
                                                       int per_xcd)
{
    constexpr int kSbRow = sb_row_bytes<ST>();
    // Separate LDS arrays (two x buffers, the rings), so that the compiler
    // sees that what a wave reads never aliases the x buffer that
    // direct-to-LDS loads are filling, and adds no wait for them.
    __shared__ uint4 x_lds0[kBM * 8];                                   // 256 rows x 128 B
    __shared__ uint4 x_lds1[kBM * 8];
    __shared__ uint4 code_lds[4 * 2 * kCodeStageBytes / 16];            // [wave][stage] 8 KB
    __shared__ uint32_t sb_lds[4 * 2 * sb_stage_bytes<ST>() / 4];       // [wave][stage][s|b]

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int xcd = blockIdx.x % 8, j_local = blockIdx.x / 8;
    const int t = xcd * per_xcd + j_local;
    if (j_local >= per_xcd || t >= tiles_m * tiles_n) return;
    const int64_t m0 = (int64_t)(t % tiles_m) * kBM;
    const int64_t n0 = (int64_t)(t / tiles_m) * kBN;
    const int nr = lane & 31, h = lane >> 5;
    const int nk = (int)(p.k / kBK2);
    const uint32_t wpr = (uint32_t)p.words_per_row, gpr = (uint32_t)p.groups_per_row;
    const uint32_t wrow0 = (uint32_t)(n0 + wave * 64);   // this wave's first weight row

    // Ring geometry.  Codes: kCB K blocks per stage, filled in kCB slices of
    // 64 / kCB rows (kCodeLd 16-byte loads per lane).  Scales and biases:
    // 2^lg_sb K blocks per stage (8 groups), filled in 4 slices of 16 rows
    // (kSbLd 4-byte loads per lane per array).
    constexpr int kCB = 16 / BITS;
    constexpr int kCodeLd = BITS / 2;
    constexpr int kSbLanesPerRow = kSbRow / 4;
    constexpr int kSbLd = 16 * kSbLanesPerRow / 64;
    constexpr uint32_t kPerDword = 4 / sizeof(ST);
    const int lg_sb = p.lg_gs - 3;
    const int last_code_stage = (nk - 1) / kCB;
    const int last_sb_stage = (int)((gpr - 1) / kSbGroups);

    // x loader: instruction i of wave w fills LDS rows 64 w + 8 i .. + 8; lane
    // l writes position l % 8 of row 64 w + 8 i + l / 8, i.e. chunk
    // (l % 8) ^ ((row / 2) % 8) of that row of x
    uint32_t xoff[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = wave * 64 + i * 8 + (lane >> 3);
        const int c = (lane & 7) ^ ((r >> 1) & 7);
        xoff[i] = (uint32_t)min(m0 + r, p.m - 1) * (uint32_t)p.k + (uint32_t)(8 * c);
    }
    auto x_buf = [&](int buf) { return buf ? x_lds1 : x_lds0; };   // buf is a constant
    auto load_x = [&](int buf, int kb) {
        const bf16_bits *xg = p.x + (uint32_t)(kb * kBK2);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            __builtin_amdgcn_global_load_lds(xg + xoff[i], (lds_void *)(x_buf(buf) + (wave * 64 + i * 8) * 8),
                                             16, 0, 0);
    };

    // Codes slice q of stage T: load l of a lane covers ring row
    // r = q * 64 / kCB + 8 l + lane / 8, ring position lane % 8, holding
    // 16-byte chunk (lane % 8) ^ ((r / 2) % 8) of the row's 128 stage bytes.
    // Stages past the last re-read the last stage (their ring buffer is not
    // read again); chunks past a row's end re-read its last chunk.
    struct CodeSlice { uint4 v[kCodeLd]; };
    auto code_slice_load = [&](int T, int q) {
        CodeSlice d;
        const uint32_t w0 = (uint32_t)min(T, last_code_stage) * (kCodeRowBytes / 4);
#pragma unroll
        for (int l = 0; l < kCodeLd; ++l) {
            const int r = q * (64 / kCB) + 8 * l + (lane >> 3);
            const int c = (lane & 7) ^ ((r >> 1) & 7);
            const uint32_t row = min(wrow0 + (uint32_t)r, (uint32_t)p.n - 1);
            const uint32_t in_row = min(w0 + (uint32_t)(4 * c), wpr - 4);
            d.v[l] = *reinterpret_cast<const uint4 *>(p.codes + row * wpr + in_row);
        }
        return d;
    };
    auto code_slice_store = [&](int T, int q, CodeSlice d) {
        const int base = (wave * 2 + (T & 1)) * (kCodeStageBytes / 16) + q * (64 / kCB) * 8;
#pragma unroll
        for (int l = 0; l < kCodeLd; ++l) code_lds[base + l * 64 + lane] = d.v[l];
    };

    // Scale/bias slice q of stage U: 16 rows; load l of a lane covers ring
    // row 16 q + (64 l + lane) / kSbLanesPerRow, dword lane % kSbLanesPerRow.
    struct SbSlice { uint32_t s[kSbLd], b[kSbLd]; };
    auto sb_slice_load = [&](int U, int q) {
        SbSlice d;
        const uint32_t g = min((uint32_t)(min(U, last_sb_stage) * kSbGroups) +
                                   (uint32_t)(lane % kSbLanesPerRow) * kPerDword,
                               gpr - kPerDword);
#pragma unroll
        for (int l = 0; l < kSbLd; ++l) {
            const int r = 16 * q + (64 * l + lane) / kSbLanesPerRow;
            const uint32_t off = min(wrow0 + (uint32_t)r, (uint32_t)p.n - 1) * gpr + g;
            d.s[l] = *reinterpret_cast<const uint32_t *>(p.scales + off);
            d.b[l] = *reinterpret_cast<const uint32_t *>(p.biases + off);
        }
        return d;
    };
    auto sb_slice_store = [&](int U, int q, SbSlice d) {
        const int base = (wave * 2 + (U & 1)) * (sb_stage_bytes<ST>() / 4) + 16 * q * kSbRow / 4;
#pragma unroll
        for (int l = 0; l < kSbLd; ++l) {
            sb_lds[base + l * 64 + lane] = d.s[l];
            sb_lds[base + 64 * kSbRow / 4 + l * 64 + lane] = d.b[l];
        }
    };
    // Slice t: codes slice t % kCB of stage t / kCB + 1, scale slice
    // min(t % 2^lg_sb, 3) of stage t / 2^lg_sb + 1 (slices 4.. of a stage
    // rewrite slice 3 with the same bytes).  Block kb writes slice kb + 3
    // (loaded during block kb - 1).
    auto code_slice_of = [&](int tt, int &T, int &q) { T = tt / kCB + 1; q = tt % kCB; };
    auto sb_slice_of = [&](int tt, int &U, int &q) {
        U = (tt >> lg_sb) + 1;
        q = min(tt & ((1 << lg_sb) - 1), 3);
    };

    // a lane's codes, scale and bias of K block kb, from the rings (indexed
    // straight off the LDS arrays, so the compiler can tell which array each
    // read touches)
    auto read_codes = [&](int kb, int cb, CodeRegs<BITS> &c) {
        const int row = cb * 32 + nr;
        const int base = (wave * 2 + ((kb / kCB) & 1)) * (kCodeStageBytes / 16) + row * 8;
#pragma unroll
        for (int i = 0; i < BITS / 4; ++i) {
            const int chunk = ((kb % kCB) * 2 + h) * (BITS / 4) + i;
            c.w[i] = code_lds[base + (chunk ^ ((row >> 1) & 7))];
        }
        const int ss = kb >> lg_sb;
        const int g = ((kb * kBK2 + 32 * h) >> p.lg_gs) - ss * kSbGroups;
        const int sbase = (wave * 2 + (ss & 1)) * (sb_stage_bytes<ST>() / 4) + row * (kSbRow / 4);
        if constexpr (sizeof(ST) == 2) {
            const int sh = 16 * (g & 1);
            c.s = (sb_lds[sbase + (g >> 1)] >> sh) & 0xffffu;
            c.b = (sb_lds[sbase + 64 * kSbRow / 4 + (g >> 1)] >> sh) & 0xffffu;
        } else {
            c.s = sb_lds[sbase + g];
            c.b = sb_lds[sbase + 64 * kSbRow / 4 + g];
        }
    };

    f32x16_t acc[8][2];        // first written by the first MFMA (zero C operand)
    bf16x8_t bop[2][2][4];     // B operands: [K block parity][column block][k16 step]
    bf16x8_t a[2][8];          // A operands: [k16 step parity][row block]
    // ring slices in flight, by the parity of the block that writes them
    CodeSlice csl0, csl1;
    SbSlice ssl0, ssl1;

    // A operand of row block rb, k16 step j, from x buffer buf, into the
    // register set of step j's parity
    auto read_a = [&](int buf, int j, int rb) {
        const int c = 4 * h + j, r = rb * 32 + nr;
        a[j & 1][rb] = __builtin_bit_cast(bf16x8_t, x_buf(buf)[r * 8 + (c ^ ((r >> 1) & 7))]);
    };

    CodeRegs<BITS> cr[2][2];   // codes of the next blocks: [K block parity][column block]

    // Prologue: x blocks 0 and 1; ring stage 0, from which blocks 0 and 1
    // are read before any other slice is written (at 8 bits stage 2 shares
    // stage 0's buffer); block 0's B operands; slices 0..2 (written by
    // blocks -3..-1); slice 3, which block 0 writes; block 0's first A
    // operands.
    load_x(0, 0);
    load_x(1, min(1, nk - 1));
#pragma unroll
    for (int q = 0; q < kCB; ++q) code_slice_store(0, q, code_slice_load(0, q));
#pragma unroll
    for (int q = 0; q < 4; ++q) sb_slice_store(0, q, sb_slice_load(0, q));
    read_codes(0, 0, cr[0][0]);
    read_codes(0, 1, cr[0][1]);
    read_codes(1, 0, cr[1][0]);
    read_codes(1, 1, cr[1][1]);
#pragma unroll
    for (int tt = 0; tt < 3; ++tt) {
        int T, q;
        code_slice_of(tt, T, q);
        code_slice_store(T, q, code_slice_load(T, q));
        sb_slice_of(tt, T, q);
        sb_slice_store(T, q, sb_slice_load(T, q));
    }
    {
        int T, q;
        code_slice_of(3, T, q);
        csl0 = code_slice_load(T, q);
        sb_slice_of(3, T, q);
        ssl0 = sb_slice_load(T, q);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        bop[0][0][j] = dequant_step<BITS, ST>(cr[0][0], j);
        bop[0][1][j] = dequant_step<BITS, ST>(cr[0][1], j);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#pragma unroll
    for (int rb = 0; rb < 8; ++rb) read_a(0, 0, rb);

    // One K block (PAR = kb % 2 at compile time: x buffer, B-operand set,
    // code and slice registers).  Step j runs its 16 MFMAs, reads the next
    // step's A operands into the other A set, and dequantizes step j of the
    // next block into the other B set -- registers last read by MFMAs a
    // whole step (A) or block (B) earlier, never by MFMAs that may still be
    // queued.  One barrier per block, before the last step: every wave has
    // then read all of this block's A operands and waited for its x loads of
    // the next block, so that x is visible (its first A operands are read
    // under the last step's MFMAs) and this block's x buffer is free for x
    // two blocks ahead.  Right after the barrier no load into LDS is in
    // flight, and the rings are read (codes of block kb + 2) and then
    // written (slice kb + 3, loaded in the previous block's first step)
    // before x is requested: a slice goes into a stage buffer whose previous
    // stage was last read before it, at the latest just before in the same
    // step, and is first read at least one block later.  Prefetches past the
    // last block re-read the last one, into buffers nothing reads any more
    // (or with the same bytes); the operands prepared during the last block
    // go unused.
    constexpr int kRingLoads = kCodeLd + 2 * kSbLd;   // ring loads per block (after x)
    auto block = [&](int kb, auto par, auto first) {
        constexpr int PAR = decltype(par)::value;
        constexpr bool FIRST = decltype(first)::value;
        const f32x16_t zero = {};
        // Step j.  The B operands are double-buffered by block for a measured
        // reason: rewriting a B register in place right after the MFMAs that
        // read it (the usual rolling scheme) gave corrupted products on this
        // GPU whenever the write was scheduled within a few instructions of
        // those MFMAs, from one run to the next -- the matrix core reads its
        // operands after issue, and nothing stalls the write.
        auto step = [&](int j, int nbuf, int nj, auto issue) {
            issue();
#pragma unroll
            for (int rb = 0; rb < 8; ++rb) {
                const bool init = FIRST && j == 0;
                acc[rb][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j & 1][rb], bop[PAR][0][j], init ? zero : acc[rb][0], 0, 0, 0);
                acc[rb][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j & 1][rb], bop[PAR][1][j], init ? zero : acc[rb][1], 0, 0, 0);
                read_a(nbuf, nj, rb);
            }
            bop[PAR ^ 1][0][j] = dequant_step<BITS, ST>(cr[PAR ^ 1][0], j);
            bop[PAR ^ 1][1][j] = dequant_step<BITS, ST>(cr[PAR ^ 1][1], j);
            // spread the VALU over the MFMAs: per row block, its two MFMAs
            // and six VALU operations
#pragma unroll
            for (int rb = 0; rb < 8; ++rb) {
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);   // VALU
            }
            __builtin_amdgcn_sched_barrier(0);
        };
        // step 0 also loads slice kb + 4 (written by the next block)
        step(0, PAR, 1, [&] {
            CodeSlice &csl = PAR ? csl0 : csl1;
            SbSlice &ssl = PAR ? ssl0 : ssl1;
            int T, q;
            code_slice_of(kb + 4, T, q);
            csl = code_slice_load(T, q);
            sb_slice_of(kb + 4, T, q);
            ssl = sb_slice_load(T, q);
        });
        step(1, PAR, 2, [] {});
        step(2, PAR, 3, [] {});
        // Wait for x of the next block (issued in the previous block's last
        // step; only this block's ring loads were issued after it), then
        // the barrier.  __syncthreads() would wait for every load; the memory
        // clobbers keep the compiler from moving memory accesses across.
        // s_waitcnt: vmcnt in bits 3:0 and 15:14, lgkmcnt (11:8) and
        // expcnt (6:4) zero.
        __builtin_amdgcn_s_waitcnt(kRingLoads & 15 | (kRingLoads >> 4) << 14);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        step(3, PAR ^ 1, 0, [&] {
            read_codes(kb + 2, 0, cr[PAR][0]);
            read_codes(kb + 2, 1, cr[PAR][1]);
            const CodeSlice &csl = PAR ? csl1 : csl0;
            const SbSlice &ssl = PAR ? ssl1 : ssl0;
            int T, q;
            code_slice_of(kb + 3, T, q);
            code_slice_store(T, q, csl);
            sb_slice_of(kb + 3, T, q);
            sb_slice_store(T, q, ssl);
            load_x(PAR, min(kb + 2, nk - 1));
        });
    };
    block(0, std::integral_constant<int, 0>{}, std::true_type{});
    int kb = 1;
    for (; kb + 1 < nk; kb += 2) {
        block(kb, std::integral_constant<int, 1>{}, std::false_type{});
        block(kb + 1, std::integral_constant<int, 0>{}, std::false_type{});
    }
    if (kb < nk) block(kb, std::integral_constant<int, 1>{}, std::false_type{});
    // the last block's prefetches must land before the workgroup's LDS is
    // handed to another workgroup
    __builtin_amdgcn_s_waitcnt(0);

    // epilogue: lane l holds column l % 32 and rows 8 (v / 4) + 4 (l / 32) + v % 4
    // of each 32 x 32 block; offsets from the tile corner are 32-bit
    bf16_bits *yt = p.y + m0 * p.n + n0 + wave * 64;
    const bool full = m0 + kBM <= p.m && n0 + kBN <= p.n;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
        const bool col_ok = full || n0 + wave * 64 + cb * 32 + nr < p.n;
#pragma unroll
        for (int rb = 0; rb < 8; ++rb)
#pragma unroll
            for (int v = 0; v < 16; v += 2) {
                const uint32_t pk = pack_bf16(acc[rb][cb][v], acc[rb][cb][v + 1]);
                const int rl = rb * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
                const uint32_t off = (uint32_t)rl * (uint32_t)p.n + (uint32_t)(cb * 32 + nr);
                if (full) {
                    yt[off] = (bf16_bits)(pk & 0xffffu);
                    yt[off + (uint32_t)p.n] = (bf16_bits)(pk >> 16);
                } else if (col_ok) {
                    if (m0 + rl < p.m) yt[off] = (bf16_bits)(pk & 0xffffu);
                    if (m0 + rl + 1 < p.m) yt[off + (uint32_t)p.n] = (bf16_bits)(pk >> 16);
                }
            }
    }
}

// ---------------------------------------------------------------------------
// Grouped matrix-core gather ("Mixture of experts" section: a grouped kernel
// reads each expert's weights once for the rows that chose it).  A
// workgroup computes a 32 x (32 CB) tile of y: the up to 32 activation
// vectors of one chunk (all of one expert, gathered through perm) against
// 32 CB weight rows of that expert.  Its CB x KS waves form KS groups that
// take consecutive equal ranges of K blocks (64 wide); in a group, wave w
// owns 32 weight rows.  Each wave runs v_mfma_f32_32x32x16_bf16 over its K
// blocks, and the groups' partial tiles are added in LDS in group order.
// Many small workgroups of equal work keep every SIMD equally loaded.
//
// Activations: each K block of the chunk (32 rows x 128 bytes) goes global
// -> LDS with direct-to-LDS loads (8 lanes per 128-byte row segment; the CB
// waves of a group share the loading) into a ring of D LDS arrays per group,
// and the group's waves read their A operands from there.  Row r's 16-byte
// chunk q sits in slot q ^ ((r / 2) % 8), so the operand reads (16 lanes =
// rows c .. c + 15 of one chunk column) cover all 64 banks once.
// Weights: lane (c = l % 32, h = l / 32) loads the 32 codes of weight row c
// at k = 32 h .. 32 h + 31 of the block into a ring of D register sets, and
// dequantizes them into B operands as round_bf16(fmaf(s, q, b)); k16 step j
// takes k = 32 h + 8 j .. + 8 on both sides.  Scales and biases come in
// stages of 8 groups per row: one direct-to-LDS load per 16 bytes of a
// row's run (lanes 0-31 scales, 32-63 biases of the wave's 32 rows) into a
// wave-private two-stage LDS ring, one stage ahead; each block reads its
// group's pair from there.  (One scale and one bias load per lane and block
// would touch 16 cache lines each for 2 bytes a lane; those narrow loads
// cost more than all the rest of the traffic.)  Where the ring does not
// fit (scales or biases not 16-byte aligned, or a K range that is not a
// whole number of stages) each block loads its own pair with its codes:
// the same values, so the same results.
//
// Schedule of block kb (ring index kb % D): wait until this wave's LDS loads
// of block kb have landed; barrier over the workgroup when CB > 1 (then all
// 32 rows of block kb are in LDS, and every wave has finished reading block
// kb - 1); load block kb + D - 1 into the LDS array block kb - 1 used,
// compute block kb, load the weights of block kb + D into the register set
// block kb used.  The wait counts the loads issued after the ones it waits
// for, from this fixed issue order, so the later blocks stay in flight; the
// compiler keeps the order (memory clobbers and scheduling barriers around
// each block's loads).

template <typename ST>
struct GatherParams {
    const bf16_bits *x;
    bf16_bits *y;
    const uint32_t *codes;
    const ST *scales;
    const ST *biases;
    const uint32_t *perm;
    const uint4 *chunks;
    const uint32_t *nchunks;
    const uint32_t *ids;
    const uint32_t *lhs;   // left indices or null: vector r * l + j reads x row lhs[r] * l + j
    int64_t n, k, e, words_per_row, groups_per_row, l, v_total, x_items;
    int lg_gs;
};

constexpr int kGatherRows = 32;      // activation vectors per chunk (MFMA rows)
constexpr int kGatherColWaves = 2;   // waves along N per K range (sharing the activations)
constexpr int kGatherDepth = 2;      // K blocks in flight per wave

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

// s_waitcnt with vmcnt = N and the other counters left at their maximum
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// In-workgroup grouping (gather_self_group_fits): every workgroup counts
// the vectors per bucket (expert id, ids past the last expert in bucket
// e), scans the counts into chunk offsets, and finds its chunk -- the
// blockIdx.y-th in bucket order, chunks of at most 32 vectors in increasing
// vector order within a bucket, exactly the separate grouping pass's table
// -- and the chunk's vectors, by ballots over its ids.  Returns false if
// the workgroup has no chunk.  ch = {bucket, -, count}; list[r] = vector r.
constexpr int kSelfGroupRounds = 16;

template <int NT>
__device__ bool gather_self_group(const uint32_t *ids, const uint32_t *lhs, int64_t x_items, int64_t l,
                                  int64_t v_total, int e, uint4 &ch, uint32_t *list)
{
    constexpr int NWV = NT / 64;
    __shared__ uint32_t gh[256], gst[256], gcoff[257], gw[NWV];
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const int nb = e + 1;
    const int rounds = (int)((v_total + NT - 1) / NT);
    const uint64_t below = lane ? ~0ull >> (64 - lane) : 0ull;
    uint32_t bk[kSelfGroupRounds];
    for (int b = t; b < nb; b += NT) gh[b] = 0;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kSelfGroupRounds; ++r) {
        bk[r] = 0xffffffffu;
        if (r < rounds) {   // uniform
            const int64_t v = (int64_t)r * NT + t;
            if (v < v_total) {
                const int64_t rr = v / l;   // rows with lhs past the x items: the zero bucket
                bk[r] = lhs && (int64_t)lhs[rr] >= x_items ? (uint32_t)e : min(ids[rr], (uint32_t)e);
            }
            // counts by LDS atomics (the sums do not depend on their order)
            if (bk[r] != 0xffffffffu) atomicAdd(&gh[bk[r]], 1u);
        }
    }
    __syncthreads();
    if (wv == 0) {
        // exclusive scans of the bucket sizes and chunk counts (lane i: buckets 4 i .. 4 i + 3)
        uint32_t hv[4], cn[4], sh = 0, sc = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int b = 4 * lane + j;
            hv[j] = b < nb ? gh[b] : 0u;
            cn[j] = (hv[j] + kGatherRows - 1) / kGatherRows;
            sh += hv[j];
            sc += cn[j];
        }
        uint32_t ih = sh, ic = sc;
        for (int off = 1; off < 64; off <<= 1) {
            const uint32_t a = __shfl_up(ih, off), c2 = __shfl_up(ic, off);
            if (lane >= off) ih += a, ic += c2;
        }
        uint32_t ph = ih - sh, pc = ic - sc;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int b = 4 * lane + j;
            if (b < nb) gst[b] = ph, gcoff[b] = pc;
            ph += hv[j];
            pc += cn[j];
        }
        if (lane == 63) gcoff[nb] = ic;
    }
    __syncthreads();
    const uint32_t j = blockIdx.y;
    if (j >= gcoff[nb]) return false;   // uniform
    int lo = 0, hi = nb;                // gcoff[lo] <= j < gcoff[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (gcoff[mid] <= j) lo = mid;
        else hi = mid;
    }
    const uint32_t bj = (uint32_t)lo, first = (j - gcoff[lo]) * kGatherRows;
    const uint32_t cnt = min((uint32_t)kGatherRows, gh[lo] - first);
    uint32_t run = 0;   // vectors of bucket bj in earlier rounds
#pragma unroll
    for (int r = 0; r < kSelfGroupRounds; ++r) {
        if (r < rounds) {   // uniform
            const uint64_t m = __ballot(bk[r] == bj);
            if (lane == 0) gw[wv] = (uint32_t)__popcll(m);
            __syncthreads();
            uint32_t before = run, all = 0;
#pragma unroll
            for (int w2 = 0; w2 < NWV; ++w2) {
                const uint32_t g = gw[w2];
                before += w2 < wv ? g : 0u;
                all += g;
            }
            if (bk[r] == bj) {
                const uint32_t rank = before + (uint32_t)__popcll(m & below) - first;
                if (rank < cnt) list[rank] = (uint32_t)((int64_t)r * NT + t);
            }
            run += all;
            __syncthreads();
        }
    }
    ch = make_uint4(bj, 0u, cnt, 0u);
    return true;
}

template <int BITS, typename ST, int CB, int KS, int D, bool SBR, bool SELF>
__global__ void __launch_bounds__(64 * CB * KS) gather_mfma_kernel(GatherParams<ST> p)
{
    static_assert(D >= 2 && D <= 4, "ring depth");
    static_assert(CB == 1 || CB == 2 || CB == 4, "column waves per group");
    static_assert(CB * KS <= 16, "workgroup size");
    constexpr int NX = 4 / CB;                  // activation loads per wave and block (8 rows each)
    constexpr int NS = (int)sizeof(ST) / 2;     // scale/bias loads per wave and stage
    constexpr int CW = BITS / 4;                // 16-byte code loads per lane and block
    __shared__ uint4 xs0[KS][kGatherRows * 8], xs1[KS][kGatherRows * 8], xs2[KS][kGatherRows * 8],
        xs3[KS][kGatherRows * 8];
    // per wave, two stages of [NS][scales of 32 rows, biases of 32 rows] x 16 bytes
    __shared__ uint4 sb_lds[CB * KS][SBR ? 2 : 1][SBR ? NS * 64 : 1];
    __shared__ uint32_t vec_list[kGatherRows];
    uint4 ch;
    if constexpr (SELF) {
        if (!gather_self_group<64 * CB * KS>(p.ids, p.lhs, p.x_items, p.l, p.v_total, (int)p.e, ch, vec_list))
            return;
    } else {
        if (blockIdx.y >= *p.nchunks) return;   // uniform over the workgroup
        ch = p.chunks[blockIdx.y];
    }
    // vector r of the chunk (r < count)
    auto vec_at = [&](int r) -> uint32_t { return SELF ? vec_list[r] : p.perm[ch.y + r]; };
    const int lane = threadIdx.x & 63;
    const int wave_id = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int cbw = wave_id % CB, grp = wave_id / CB;
    const int c = lane & 31, h = lane >> 5;
    const int count = (int)ch.z;
    const int64_t n0 = ((int64_t)blockIdx.x * CB + cbw) * 32;
    const bool live = (int64_t)ch.x < p.e;
    // wave group grp takes the K blocks [kb0, kb0 + nk)
    const int nk = (int)(p.k / kBK2) / KS;
    const int kb0 = grp * nk;
    // the vector whose output row is this lane's A row (clamped; rows past
    // count are computed and not stored)
    const uint32_t vec_c = vec_at(min(c, count - 1));
    f32x16_t acc = f32x16_t{};
    if (live && nk > 0) {
        const int64_t slab = ch.x;
        // activation loads: rows r0 + 8 i + lane / 8 of the chunk, slot lane % 8
        const int r0 = cbw * (32 / CB);
        const bf16_bits *xsrc[NX];
#pragma unroll
        for (int i = 0; i < NX; ++i) {
            const int xr = r0 + 8 * i + (lane >> 3);
            int64_t xvec = vec_at(min(xr, count - 1));
            if (p.lhs) {   // the x row of vector xvec (zero-bucket rows never get here)
                const int64_t xi = p.lhs[xvec / p.l];
                xvec = (xi < p.x_items ? xi : 0) * p.l + xvec % p.l;
            }
            xsrc[i] = p.x + xvec * p.k + (int64_t)kb0 * kBK2 + 8 * ((lane & 7) ^ ((xr >> 1) & 7));
        }
        // this lane's codes: weight row c, k = 32 h .. 32 h + 31 of each block
        const int64_t wr = min(n0 + c, p.n - 1);
        const uint32_t *crow = p.codes + (slab * p.n + wr) * p.words_per_row + h * BITS + (int64_t)kb0 * 2 * BITS;
        // scale/bias stages: 8 groups, i.e. 2^(lg_gs - 3) blocks, from group g0
        const int64_t g0 = ((int64_t)kb0 * kBK2) >> p.lg_gs;
        const ST *srow = p.scales + (slab * p.n + wr) * p.groups_per_row + g0;
        const ST *brow = p.biases + (slab * p.n + wr) * p.groups_per_row + g0;
        const ST *sbsrc = h ? brow : srow;
        const int lg_sb = p.lg_gs - 3;
        const int nsb = ((nk * kBK2) >> p.lg_gs) >> 3;   // scale/bias stages
        uint4 *sbw = sb_lds[wave_id][0];
        CodeRegs<BITS> cw[D];
        // register loads per block, and all loads per block (the scale/bias
        // stage loads in between only make the counted waits stricter)
        constexpr int NW = CW + (SBR ? 0 : 2);
        constexpr int NB = NW + NX;
        auto ring = [&](auto s) -> uint4 * {
            constexpr int S = decltype(s)::value;
            if constexpr (S == 0) return xs0[grp];
            else if constexpr (S == 1) return xs1[grp];
            else if constexpr (S == 2) return xs2[grp];
            else return xs3[grp];
        };
        auto fence = [] {
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
        };
        auto load_x = [&](int kb, auto s) {
            asm volatile("" ::: "memory");
#pragma unroll
            for (int i = 0; i < NX; ++i)
                __builtin_amdgcn_global_load_lds((const void *)(xsrc[i] + (int64_t)kb * kBK2),
                                                 (lds_void *)(ring(s) + (r0 + 8 * i) * 8), 16, 0, 0);
            fence();
        };
        auto load_w = [&](int kb, int slot) {
            const uint4 *cs = reinterpret_cast<const uint4 *>(crow + (int64_t)kb * 2 * BITS);
#pragma unroll
            for (int i = 0; i < CW; ++i) cw[slot].w[i] = cs[i];
            if constexpr (!SBR) {
                const int gr = (kb * kBK2 + 32 * h) >> p.lg_gs;   // group, relative to g0
                if constexpr (sizeof(ST) == 2) {
                    cw[slot].s = srow[gr];
                    cw[slot].b = brow[gr];
                } else {
                    cw[slot].s = __float_as_uint(srow[gr]);
                    cw[slot].b = __float_as_uint(brow[gr]);
                }
            }
            fence();
        };
        // scale/bias stage t into ring buffer t % 2
        auto load_sb = [&](int t) {
            asm volatile("" ::: "memory");
#pragma unroll
            for (int j = 0; j < NS; ++j)
                __builtin_amdgcn_global_load_lds((const void *)(sbsrc + 8 * t + (16 / (int)sizeof(ST)) * j),
                                                 (lds_void *)(sbw + (t & 1) * (NS * 64) + j * 64), 16, 0, 0);
            fence();
        };
        // At the first block of scale/bias stage t >= 1, stage t + 1 goes
        // into the buffer stage t - 1 used (this wave's alone, and its reads
        // are done: the barrier before waited for this wave's LDS reads).
        auto stage_next = [&](int kb) {
            if constexpr (!SBR) return;
            const int t = kb >> lg_sb;
            if (kb > 0 && (kb & ((1 << lg_sb) - 1)) == 0 && t + 1 < nsb) load_sb(t + 1);
        };
        // This lane's scale and bias for block kb, read in one asm block that
        // waits for its own results: the compiler cannot tell the stage read
        // here from the one whose load may be in flight, and would wait for
        // every load this wave has in flight.  The counted waits already
        // cover this stage: its load is older than the activation loads of
        // the block that first uses it.
        const uint32_t sb_base = (uint32_t)(uintptr_t)(lds_void *)sbw + c * 16;
        auto read_sb = [&](int kb, CodeRegs<BITS> &w) {
            if constexpr (!SBR) return;   // loaded with the codes
            const int gr = (kb * kBK2 + 32 * h) >> p.lg_gs;   // group, relative to g0
            const int t = gr >> 3, e = gr & 7;
            const uint32_t sa = sb_base + (uint32_t)((t & 1) * (NS * 1024) + (e * (int)sizeof(ST) / 16) * 1024 +
                                                     (e * (int)sizeof(ST)) % 16);
            uint32_t sv, bv;
            if constexpr (sizeof(ST) == 2)
                asm volatile("ds_read_u16 %0, %2\n\tds_read_u16 %1, %2 offset:512\n\ts_waitcnt lgkmcnt(0)"
                             : "=&v"(sv), "=&v"(bv) : "v"(sa));
            else
                asm volatile("ds_read_b32 %0, %2\n\tds_read_b32 %1, %2 offset:512\n\ts_waitcnt lgkmcnt(0)"
                             : "=&v"(sv), "=&v"(bv) : "v"(sa));
            w.s = sv;
            w.b = bv;
        };
        auto barrier = [&] {
            // this wave's LDS reads are done (lgkmcnt 0); with CB > 1 the
            // waves of a group share the activation ring
            __builtin_amdgcn_s_waitcnt(0xc07f);
            asm volatile("" ::: "memory");
            if constexpr (CB > 1) __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        };
        auto compute = [&](auto s, int slot, int kb) {
            CodeRegs<BITS> &w = cw[slot];
            read_sb(kb, w);
            const uint4 *xb = ring(s);
            uint4 a[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) a[j] = xb[c * 8 + ((4 * h + j) ^ ((c >> 1) & 7))];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bf16x8_t bv = dequant_step<BITS, ST>(w, j);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a[j]), bv, acc,
                                                              0, 0, 0);
            }
        };
        // prologue: scale/bias stages 0 and 1, then in the steady-state
        // order W(0), X(j), W(j + 1) for j = 0 .. D - 2 (blocks past the end
        // are clamped; they are never computed)
        if constexpr (SBR) {
            load_sb(0);
            if (nsb > 1) load_sb(1);
        }
        load_w(0, 0);
        static_for<0, D - 1>([&](auto jj) {
            constexpr int J = decltype(jj)::value;
            load_x(min(J, nk - 1), std::integral_constant<int, J>{});
            load_w(min(J + 1, nk - 1), J + 1);
        });
        // Block kb: wait for this wave's activation loads of block kb (the
        // loads issued after them: the codes of block kb + 1 and those of
        // D - 2 later blocks), barrier, load the activations of block
        // kb + D - 1 into the buffer block kb - 1 used, start the next
        // scale/bias stage where due, compute, load the codes of block kb + D
        // into the register set block kb used.
        int base = 0;
        for (; base + 2 * D <= nk; base += D) {
            static_for<0, D>([&](auto dd) {
                constexpr int d = decltype(dd)::value;
                wait_vmcnt<NW + (D - 2) * NB>();
                barrier();
                load_x(base + d + D - 1, std::integral_constant<int, (d + D - 1) % D>{});
                stage_next(base + d);
                compute(dd, d, base + d);
                load_w(base + d + D, d);
            });
        }
        // the last D .. 2D - 1 blocks (or all of them when nk < D)
        static_for<0, 2 * D - 1>([&](auto dd) {
            constexpr int d = decltype(dd)::value;
            const int kb = base + d;
            if (kb < nk) {   // uniform
                if constexpr (d == 0) wait_vmcnt<NW + (D - 2) * NB>();
                else if constexpr (d < D) wait_vmcnt<(D - 1 - d) * NB>();
                else wait_vmcnt<0>();
                barrier();
                if constexpr (d == 0) load_x(min(kb + D - 1, nk - 1), std::integral_constant<int, D - 1>{});
                else if (kb + D - 1 < nk) load_x(kb + D - 1, std::integral_constant<int, (d + D - 1) % D>{});
                stage_next(kb);
                compute(std::integral_constant<int, d % D>{}, d % D, kb);
                if (kb + D < nk) load_w(kb + D, d % D);
            }
        });
    }
    if constexpr (KS > 1) {
        // the later groups' partial tiles are added in LDS, in group order
        __shared__ f32x16_t part[KS - 1][CB][64];
        if (grp > 0) part[grp - 1][cbw][lane] = acc;
        __syncthreads();
        if (grp > 0) return;
#pragma unroll
        for (int g2 = 0; g2 < KS - 1; ++g2) acc += part[g2][cbw][lane];
    }
    // D layout: lane l holds column l % 32 and rows 8 (v / 4) + 4 (l / 32) + v % 4
    const int64_t col = n0 + c;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int r = 8 * (v >> 2) + 4 * h + (v & 3);
        const uint32_t yv = __shfl(vec_c, r);
        if (r < count && col < p.n)
            p.y[(int64_t)yv * p.n + col] = (bf16_bits)(pack_bf16(acc[v], 0.0f) & 0xffffu);
    }
}

// The scale/bias ring needs K split into KS equal ranges that are whole
// numbers of stages (8 groups), and 16-byte aligned scales and biases (its
// loads move 16 bytes a lane).  Otherwise each block loads its own pair;
// the values, and so the results, are the same either way.
bool gather_sb_ring_fits(int ks, int64_t k, int gs, const void *scales, const void *biases)
{
    return gs >= 32 && (k / ks) % (8 * (int64_t)gs) == 0 &&
           (((uintptr_t)scales | (uintptr_t)biases) & 15) == 0;
}

template <int BITS, typename ST, int KS, bool SBR, bool SELF>
hipError_t gather_mfma_run(const GatherMfmaLaunch &a, hipStream_t stream)
{
    constexpr int CB = kGatherColWaves, D = kGatherDepth;
    GatherParams<ST> p;
    p.x = static_cast<const bf16_bits *>(a.x);
    p.y = static_cast<bf16_bits *>(a.y);
    p.codes = a.codes;
    p.scales = static_cast<const ST *>(a.scales);
    p.biases = static_cast<const ST *>(a.biases);
    p.perm = a.perm;
    p.chunks = reinterpret_cast<const uint4 *>(a.chunks);
    p.nchunks = a.nchunks;
    p.ids = a.ids;
    p.lhs = a.lhs;
    p.x_items = a.x_items;
    p.n = a.n;
    p.k = a.k;
    p.e = a.e;
    p.l = a.l;
    p.v_total = a.v_total;
    p.words_per_row = a.k * BITS / 32;
    p.groups_per_row = a.k / a.gs;
    p.lg_gs = a.gs == 32 ? 5 : a.gs == 64 ? 6 : 7;
    if (a.k % (kBK2 * KS) != 0 || a.max_chunks > 65535) return hipErrorInvalidValue;
    if (SELF && (!gather_self_group_fits(a.v_total, a.e) || a.v_total > (int64_t)kSelfGroupRounds * 64 * CB * KS ||
                 a.l <= 0))
        return hipErrorInvalidValue;
    if (SBR && !gather_sb_ring_fits(KS, a.k, a.gs, a.scales, a.biases)) return hipErrorInvalidValue;
    const unsigned gx = (unsigned)((a.n + 32 * CB - 1) / (32 * CB));
    gather_mfma_kernel<BITS, ST, CB, KS, D, SBR, SELF>
        <<<dim3(gx, (unsigned)a.max_chunks), dim3(64 * CB * KS), 0, stream>>>(p);
    return hipGetLastError();
}

template <int BITS, typename ST, bool SELF>
hipError_t gather_mfma_pick(const GatherMfmaLaunch &a, hipStream_t stream)
{
    // the K split depends on k alone: it fixes each row's summation order
    if (a.k % (2 * kBK2) == 0) {
        if (gather_sb_ring_fits(2, a.k, a.gs, a.scales, a.biases))
            return gather_mfma_run<BITS, ST, 2, true, SELF>(a, stream);
        return gather_mfma_run<BITS, ST, 2, false, SELF>(a, stream);
    }
    if (gather_sb_ring_fits(1, a.k, a.gs, a.scales, a.biases)) return gather_mfma_run<BITS, ST, 1, true, SELF>(a, stream);
    return gather_mfma_run<BITS, ST, 1, false, SELF>(a, stream);
}

template <int BITS, typename ST>
hipError_t gather_mfma_pick(const GatherMfmaLaunch &a, hipStream_t stream)
{
    if (a.self_group) return gather_mfma_pick<BITS, ST, true>(a, stream);
    return gather_mfma_pick<BITS, ST, false>(a, stream);
}

hipError_t launch_gather_mfma(const GatherMfmaLaunch &a, hipStream_t stream)
{
    if (a.bits != 4 && a.bits != 8) return hipErrorInvalidValue;
    if (a.sb_dt == DT_F32) {
        if (a.bits == 4) return gather_mfma_pick<4, float>(a, stream);
        return gather_mfma_pick<8, float>(a, stream);
    }
    if (a.bits == 4) return gather_mfma_pick<4, bf16_bits>(a, stream);
    return gather_mfma_pick<8, bf16_bits>(a, stream);
}

bool tiled_fits(int tile_m, int tile_n, int bits, int gs, int sb_dt, int64_t m, int64_t n, int64_t k)
{
    if (!tiled_supported(tile_m, tile_n, bits)) return false;
    if (tile_m != kBM) return true;
    // K in whole 64-blocks; 32-bit offsets; every row of scales and biases
    // starts on a 4-byte boundary (4-byte direct-to-LDS loads)
    const int64_t groups = k / gs;
    const bool sb_aligned = sb_dt == DT_F32 || groups % 2 == 0;
    return k % kBK2 == 0 && sb_aligned && m * k < ((int64_t)1 << 31) &&
           n * (k * bits / 32) < ((int64_t)1 << 31) && (m + kBM) * n < ((int64_t)1 << 31) &&
           n * groups < ((int64_t)1 << 31);
}

bool tiled_supported(int tile_m, int tile_n, int bits)
{
    const bool any_width = bits == 1 || bits == 2 || bits == 3 || bits == 4 || bits == 5 || bits == 6 || bits == 8;
    if (tile_m == kTM && tile_n == kTN) return any_width;
    return tile_m == kBM && tile_n == kBN && (bits == 4 || bits == 8);
}

namespace {
template <int BITS, typename ST>
hipError_t tiled_run(const TiledLaunch &a, hipStream_t stream)
{
    TiledParams<ST> p;
    p.x = static_cast<const bf16_bits *>(a.x);
    p.y = static_cast<bf16_bits *>(a.y);
    p.codes = a.codes;
    p.scales = static_cast<const ST *>(a.scales);
    p.biases = static_cast<const ST *>(a.biases);
    p.m = a.m;
    p.n = a.n;
    p.k = a.k;
    p.words_per_row = a.k * BITS / 32;
    p.groups_per_row = a.k / a.gs;
    p.gs = a.gs;
    p.lg_gs = a.gs == 32 ? 5 : a.gs == 64 ? 6 : 7;
    if constexpr (BITS == 4 || BITS == 8) {
        if (a.tile_m == kBM) {
            if (!tiled_fits(kBM, kBN, BITS, a.gs, a.sb_dt, a.m, a.n, a.k)) return hipErrorInvalidValue;
            const int tm = (int)((a.m + kBM - 1) / kBM), tn = (int)((a.n + kBN - 1) / kBN);
            const int per = (tm * tn + 7) / 8;
            tiled256_kernel<BITS, ST><<<dim3(8 * per), dim3(256), 0, stream>>>(p, tm, tn, per);
            return hipGetLastError();
        }
    } else if (a.tile_m != kTM) {
        return hipErrorInvalidValue;
    }
    const dim3 grid((unsigned)((a.n + kTN - 1) / kTN), (unsigned)((a.m + kTM - 1) / kTM));
    tiled_kernel<BITS, ST><<<grid, dim3(256), 0, stream>>>(p);
    return hipGetLastError();
}

template <typename ST>
hipError_t tiled_bits(const TiledLaunch &a, hipStream_t stream)
{
    switch (a.bits) {
    case 1: return tiled_run<1, ST>(a, stream);
    case 2: return tiled_run<2, ST>(a, stream);
    case 3: return tiled_run<3, ST>(a, stream);
    case 4: return tiled_run<4, ST>(a, stream);
    case 5: return tiled_run<5, ST>(a, stream);
    case 6: return tiled_run<6, ST>(a, stream);
    case 8: return tiled_run<8, ST>(a, stream);
    default: return hipErrorInvalidValue;
    }
}
}  // namespace

hipError_t launch_tiled(const TiledLaunch &a, hipStream_t stream)
{
    if (!tiled_supported(a.tile_m, a.tile_n, a.bits)) return hipErrorInvalidValue;
    if (a.sb_dt == DT_F32) return tiled_bits<float>(a, stream);
    return tiled_bits<bf16_bits>(a, stream);
}

}  // namespace nqk
