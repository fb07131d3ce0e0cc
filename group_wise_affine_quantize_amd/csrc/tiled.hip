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
    int gs;
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
            uint32_t cw[BITS / 2];
            const uint32_t *src = p.codes + wr * p.words_per_row + e0 * BITS / 32;
#pragma unroll
            for (int i = 0; i < BITS / 2; ++i) cw[i] = src[i];
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

bool tiled_supported(int tile_m, int tile_n, int bits)
{
    return tile_m == kTM && tile_n == kTN && (bits == 4 || bits == 8);
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
    const dim3 grid((unsigned)((a.n + kTN - 1) / kTN), (unsigned)((a.m + kTM - 1) / kTM));
    tiled_kernel<BITS, ST><<<grid, dim3(256), 0, stream>>>(p);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_tiled(const TiledLaunch &a, hipStream_t stream)
{
    if (!tiled_supported(a.tile_m, a.tile_n, a.bits)) return hipErrorInvalidValue;
    if (a.sb_dt == DT_F32) {
        if (a.bits == 4) return tiled_run<4, float>(a, stream);
        return tiled_run<8, float>(a, stream);
    }
    if (a.bits == 4) return tiled_run<4, bf16_bits>(a, stream);
    return tiled_run<8, bf16_bits>(a, stream);
}

}  // namespace nqk
