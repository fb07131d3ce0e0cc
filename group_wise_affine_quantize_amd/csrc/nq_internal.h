// Internal interface between the C-ABI layer (nq_api.hip) and the kernel
// translation units.  Launchers assume validated arguments and only enqueue.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nqk {

enum { DT_F32 = 0, DT_BF16 = 1 };

// Elements handled by one lane per K step of the matrix-vector family: one
// lane chunk is 32 codes = `bits` uint32 words, always inside one group.
constexpr int kLaneChunk = 32;
constexpr int kWave = 64;
constexpr int kStepElems = kLaneChunk * kWave;   // 2048 elements of K per wave step

hipError_t launch_quantize(const void *w, int w_dt, int64_t n, int64_t k, int gs, int bits,
                           uint32_t *codes, void *scales, void *biases, hipStream_t stream);

hipError_t launch_dequantize(const uint32_t *codes, const void *scales, const void *biases,
                             int sb_dt, int64_t n, int64_t k, int gs, int bits, void *out,
                             int out_dt, hipStream_t stream);

// One launch of the matrix-vector family over `items` independent products
// that share n, k and the quantization: item i multiplies rows_per_item
// consecutive rows of x (starting at row i * rows_per_item) with the weights
// of expert idx[i] (or the only weight matrix when idx is null), writing the
// same rows of y.  Items whose expert id is >= e produce zero rows.
//
// Grouped gather (chunks set): instead of items, the launch runs the chunk
// table a grouping pass built (launch_gather_groups); chunk c multiplies the
// activation vectors perm[first .. first + count) by expert `bucket`'s
// weights (bucket >= e: zero rows).
struct GemvLaunch {
    const void *x;
    void *y;
    const uint32_t *codes;
    const void *scales;
    const void *biases;
    const uint32_t *idx;     // null: plain product
    int x_dt, sb_dt;
    int64_t items, rows_per_item, k, n, e;
    int gs, bits;
    int ksplit, rows_per_wave;
    const uint32_t *perm = nullptr, *chunks = nullptr, *nchunks = nullptr;
    int64_t max_chunks = 0;
    int max_rows = 8;   // largest vector count of a chunk of the table
    // gather with left indices: vector r * l + j reads x row lhs[r] * l + j
    // (lhs[r] >= x_items gives a zero row)
    const uint32_t *lhs = nullptr;
    int64_t x_items = 0, lhs_l = 1;
};
hipError_t launch_gemv(const GemvLaunch &a, hipStream_t stream);

// The matrix-core arithmetic of the matrix-vector family: bf16 activations,
// 4-bit codes, k a multiple of 64 up to 4096, n below the streaming one-row
// shapes.  A function of the sizes and dtypes only, so a row's arithmetic
// never depends on how many rows share its call.
bool gemv_mfma_family(int64_t n, int64_t k, int gs, int bits, int x_dt);
hipError_t launch_gemv_mfma(const GemvLaunch &a, hipStream_t stream);

// The matrix-core arithmetic of the 8-bit matrix-vector family: bf16
// activations, k a multiple of 1024 up to 4096, n below the streaming
// one-row shapes; K in four fixed quarters (the plan's ksplit is 4).
bool gemv_band_family(int64_t n, int64_t k, int gs, int bits, int x_dt);
constexpr int kBandKsplit = 4;
hipError_t launch_gemv_band(const GemvLaunch &a, hipStream_t stream);

// Vectors per chunk of the grouped matrix-vector gather (that family's
// largest row count per launch chunk) and of the grouped matrix-core gather.
constexpr int kGroupChunk = 8;
constexpr int kGroupChunkMfma = 32;
// Workspace of the grouping pass over `vectors` activation vectors and e
// experts cut into chunks of `chunk`, and the chunk-table bound it implies.
size_t gather_group_ws_bytes(int64_t vectors, int64_t e, int chunk);
int64_t gather_group_max_chunks(int64_t vectors, int64_t e, int chunk);
// Groups the vectors r * l + j by expert ids[r] (one workgroup): perm,
// chunk count and chunk table into ws (layout in gemv.hip).
hipError_t launch_gather_groups(const uint32_t *ids, const uint32_t *lhs, int64_t x_items, int64_t rows,
                                int64_t l, int64_t e, int chunk,
                                void *ws, hipStream_t stream);

// Grouped matrix-core gather: chunk c of the table multiplies its (up to 32)
// bf16 activation vectors perm[first ..] by expert `bucket`'s weights (K a
// multiple of 64; bucket >= e: zero rows).
struct GatherMfmaLaunch {
    const void *x;
    void *y;
    const uint32_t *codes;
    const void *scales;
    const void *biases;
    const uint32_t *perm, *chunks, *nchunks;   // grouping tables (unless self_group)
    const uint32_t *ids;                       // expert ids (self_group)
    const uint32_t *lhs;                       // left indices, or null
    int64_t x_items;
    int sb_dt;
    int64_t n, k, e, max_chunks, l, v_total;
    int gs, bits;
    bool self_group;   // each workgroup groups the ids itself (gather_self_group_fits)
};
// Whether the matrix-core gather can group the vector ids by itself in
// every workgroup: few experts and few vectors.
inline bool gather_self_group_fits(int64_t vectors, int64_t e) { return e < 256 && vectors <= 2048; }
hipError_t launch_gather_mfma(const GatherMfmaLaunch &a, hipStream_t stream);

// Tiled bf16-MFMA product: y[m, n] = x[m, k] . w_hat[n, k]^T, x and y bf16.
struct TiledLaunch {
    const void *x;
    void *y;
    const uint32_t *codes;
    const void *scales;
    const void *biases;
    int sb_dt;
    int64_t m, n, k;
    int gs, bits;
    int tile_m, tile_n;
};
hipError_t launch_tiled(const TiledLaunch &a, hipStream_t stream);
bool tiled_supported(int tile_m, int tile_n, int bits);
// Whether a tile shape fits these sizes (the 256 x 256 kernel takes K in
// multiples of 64, rows of scales and biases that start on 4-byte boundaries,
// and uses 32-bit offsets).
bool tiled_fits(int tile_m, int tile_n, int bits, int gs, int sb_dt, int64_t m, int64_t n, int64_t k);

// Product with the weights as stored: y[m, c] = x[m, i] . w_hat[i, c], the
// quantized matrix [ni, nc] grouped along c.  Few rows: row ranges of the
// matrix give partial sums in the workspace (qmm_nt_ws_bytes), added by a
// second kernel, kNtRowsPerChunk activation rows per launch pair.  tiled:
// 128 x 128 bf16-MFMA tiles (x bf16, ni a multiple of 32), no workspace.
constexpr int kNtRowsPerChunk = 2;
struct NtLaunch {
    const void *x;
    void *y;
    const uint32_t *codes;
    const void *scales;
    const void *biases;
    void *workspace;
    int x_dt, sb_dt;
    int64_t m, ni, nc;
    int gs, bits;
    bool tiled;
};
int qmm_nt_splits(int64_t ni, int64_t nc);
size_t qmm_nt_ws_bytes(int64_t ni, int64_t nc);
hipError_t launch_qmm_nt(const NtLaunch &a, hipStream_t stream);

// Derivatives of sum(dy * (x . w_hat^T)) for the scales and biases of w:
// x [m, k], dy [m, n] (same dtype), codes [n, k*bits/32] -> ds, db [n, k/gs].
struct GradLaunch {
    const void *x;
    const void *dy;
    const uint32_t *codes;
    void *ds;
    void *db;
    int x_dt, g_dt;
    int64_t m, k, n;
    int gs, bits;
};
hipError_t launch_grad_sb(const GradLaunch &a, hipStream_t stream);

// ---- floating-point modes (fp.hip): element and scale formats per mode,
// codes packed like the affine codes, uint8 scale codes, no biases; K a
// multiple of 32 (one lane chunk: one MX block or two NVFP4 blocks).
enum { FP_MXFP4 = 1, FP_MXFP8 = 2, FP_NVFP4 = 3 };
inline int fp_mode_bits(int mode) { return mode == FP_MXFP8 ? 8 : 4; }
inline int fp_mode_group(int mode) { return mode == FP_NVFP4 ? 16 : 32; }

hipError_t launch_fp_quantize(const void *w, int w_dt, int64_t n, int64_t k, int mode, uint32_t *codes,
                              uint8_t *scales, hipStream_t stream);
hipError_t launch_fp_dequantize(const uint32_t *codes, const uint8_t *scales, int64_t n, int64_t k, int mode,
                                void *out, int out_dt, hipStream_t stream);
// items products of vpi vectors each: item i multiplies its vectors with
// expert idx[i]'s weights (idx null: the only weight matrix; idx[i] >= e:
// zero rows) and the expert's global scale (gscale null: 1).  tiled: one
// item, bf16 x, k a multiple of 64 (128 x 128 MFMA tiles); otherwise the
// matrix-vector kernel in chunks of up to 8 vectors.  chunks set: the
// matrix-vector kernel runs the grouping pass's chunk table instead
// (launch_gather_groups, kGroupChunk vectors per chunk, max_chunks rows).
struct FpQmmLaunch {
    const void *x;
    void *y;
    const uint32_t *codes;
    const uint8_t *scales;
    const float *gscale;
    const uint32_t *idx;
    int x_dt, mode;
    int64_t items, vpi, n, k, e;
    bool tiled;
    const uint32_t *perm = nullptr, *nchunks = nullptr;
    const uint4 *chunks = nullptr;
    int64_t max_chunks = 0;
    bool mfma = false;   // chunks of up to kGroupChunkMfma vectors on matrix cores (bf16 x, k % 64 == 0)
};
hipError_t launch_fp_qmm(const FpQmmLaunch &a, hipStream_t stream);

// Weights as stored in a floating-point mode: y[m, c] = x[m, i] . (g w_hat)[i, c],
// w_hat [ni, nc] with groups along c (nc a multiple of 32).  tiled: bf16 x,
// ni a multiple of 64 (128 x 128 MFMA tiles); otherwise row ranges fixed by
// (ni, nc) write fp32 partial sums to the workspace (fp_nt_ws_bytes), added
// in range order, kFpNtRows activation rows per launch pair.
constexpr int kFpNtRows = 2;
struct FpNtLaunch {
    const void *x;
    void *y;
    const uint32_t *codes;
    const uint8_t *scales;
    const float *gscale;
    void *workspace;
    int x_dt, mode;
    int64_t m, ni, nc;
    bool tiled;
};
int fp_nt_ranges(int64_t ni, int64_t nc);
size_t fp_nt_ws_bytes(int64_t ni, int64_t nc);
hipError_t launch_fp_qmm_nt(const FpNtLaunch &a, hipStream_t stream);

}  // namespace nqk
