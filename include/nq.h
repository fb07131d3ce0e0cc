/*
 * nq.h -- group-wise affine quantization and quantized matrix products on
 * AMD Instinct MI355X (gfx950).  C ABI of libnq.so.
 *
 * What the operations compute is defined by the "Quantization" page of the
 * nuvec documentation (hupe1980.github.io/nuvec/docs/quantization/):
 *   - section "Affine": each row of the weights w [n, k] is cut into groups of
 *     group_size (32, 64 or 128) consecutive values; each group keeps one scale
 *     and one bias, each value becomes a `bits`-bit code packed into uint32
 *     words, and w ~ scale * code + bias;
 *   - section "Affine", example: the product is x times the TRANSPOSED weights
 *     (quantized_matmul with transpose = true), dequantize returns the
 *     approximate weights;
 *   - section "Floating-point formats", example: the product comes out in x's
 *     dtype;
 *   - section "Products on the GPU": few rows run as matrix-vector products,
 *     many rows as tiled products, split-K serves a small output with a long
 *     inner dimension; in row-exact mode every row of a product of up to 8
 *     rows equals that row's one-row product bit for bit;
 *   - section "Mixture of experts": gather_qmm multiplies each row by the
 *     weights of the expert chosen for it, without gathering the weights.
 * The nuvec API index (docs.rs/nuvec) adds: scales are stored in the weights'
 * dtype (struct Quantized); the row-independence limit ROW_INDEPENDENT_ROWS
 * (constant; 8 rows per the section above); the choice of kernel depends only
 * on shapes, dtypes, options and the row-exact mode (section "Determinism",
 * "Routing is pure"); and results are bit-identical run to run (section
 * "Determinism").
 *
 * Conventions shared by every entry point:
 *   - Every array pointer is a DEVICE pointer owned by the caller.  The library
 *     never allocates, frees or synchronises; a call only validates its
 *     arguments and enqueues kernels on `stream` (0 = the null stream).
 *   - Arrays are dense and row-major.  Base pointers of x, w, codes, the
 *     output and the workspace must be 16-byte aligned; scales and biases
 *     must be aligned to their element size.
 *   - Layout of a quantized matrix of n rows and k columns (k a multiple of
 *     group_size): codes [n, k*bits/32] uint32, scales [n, k/group_size] and
 *     biases [n, k/group_size] in sb_dt.  Element j of a row occupies bits
 *     [j*bits, (j+1)*bits) of the row's little-endian bit stream (bit i of the
 *     stream is bit i%32 of word i/32): least significant bits first.
 *   - Every argument is checked before anything is enqueued.  On an error the
 *     call returns a non-zero nq_status, writes nothing, enqueues nothing, and
 *     nq_last_error() names the entry point and the reason (a thread-local
 *     string).  A launch failure reported by the HIP runtime is NQ_ERR_LAUNCH.
 *   - A call with an empty output (m == 0 or n == 0, rows == 0) returns NQ_OK
 *     and enqueues nothing.  k == 0 gives an all-zero product.
 *   - Outputs must not overlap any input or each other (NQ_ERR_ALIAS).
 *   - No float atomics are used: the same call on the same inputs gives the
 *     same bits, whatever else runs on the device.
 *   - Calls are reentrant across host threads and streams.
 */
#ifndef NQ_H
#define NQ_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    NQ_OK = 0,
    NQ_ERR_NULL = 1,      /* a required pointer is null */
    NQ_ERR_DTYPE = 2,     /* unknown dtype, or a dtype pair not supported */
    NQ_ERR_QUANT = 3,     /* group_size not in {32, 64, 128}, or bits not in {1, 2, 3, 4, 5,
                             6, 8} (every operation takes the same widths) */
    NQ_ERR_SHAPE = 4,     /* negative size, k % group_size != 0, bad expert count, size overflow */
    NQ_ERR_ALIGN = 5,     /* a base pointer is not aligned as documented above */
    NQ_ERR_ALIAS = 6,     /* an output overlaps an input or another output */
    NQ_ERR_WORKSPACE = 7, /* workspace null or smaller than the *_workspace_bytes figure */
    NQ_ERR_LAUNCH = 8,    /* the HIP runtime rejected a kernel launch */
    NQ_ERR_PLAN = 9       /* an explicit plan that does not fit the shapes */
} nq_status;

/* Dtype arguments are validated (NQ_ERR_DTYPE for any other value), so the
 * type holds every int32 value: compiled as C++ its underlying type is fixed
 * to int32_t (in C an enum of these constants is int-sized anyway), and
 * reading an unknown value is defined behaviour on both sides. */
#ifdef __cplusplus
typedef enum : int32_t { NQ_F32 = 0, NQ_BF16 = 1 } nq_dtype;
#else
typedef enum { NQ_F32 = 0, NQ_BF16 = 1 } nq_dtype;
#endif

/* Rows of a product that keep the bits of their one-row product in every
 * mode (nuvec API index, constant ROW_INDEPENDENT_ROWS). */
#define NQ_ROW_INDEPENDENT_ROWS 8

/* ---------------------------------------------------------------- quantize */

/* Quantize w [n, k] (w_dt) in groups of group_size along each row
 * ("Affine" section).  For each group: bias = the group minimum and
 * scale = (max - min) / (2^bits - 1), computed in fp32 and rounded to w_dt;
 * code = clamp(round_half_even((w - bias) / scale), 0, 2^bits - 1) with the
 * STORED scale and bias, or 0 when the stored scale is 0.
 * Outputs: codes [n, k*bits/32] uint32, scales and biases [n, k/group_size]
 * in w_dt.  Bit-exact with IEEE fp32 arithmetic (no contraction, correctly
 * rounded division, denormals kept).  Non-finite weights are outside the
 * contract. */
nq_status nq_quantize(const void *w, nq_dtype w_dt, int64_t n, int64_t k, int32_t group_size,
                      int32_t bits, uint32_t *codes, void *scales, void *biases,
                      hipStream_t stream);

/* Dequantize ("Affine" section, q.dequantize): w_out[r, j] =
 * round_to_out_dt(fmaf(scale, code, bias)) -- one fp32 fused multiply-add,
 * then round-to-nearest-even into out_dt.  w_out: [n, k] in out_dt (the
 * documented default is the scales' dtype; the caller passes it). */
nq_status nq_dequantize(const uint32_t *codes, const void *scales, const void *biases,
                        nq_dtype sb_dt, int64_t n, int64_t k, int32_t group_size, int32_t bits,
                        void *w_out, nq_dtype out_dt, hipStream_t stream);

/* ---------------------------------------------------------------- products */

/* Kernel families ("Products on the GPU" section).  NQ_ROUTE_GEMV is the
 * matrix-vector family for up to 8 rows per launch chunk; its K loop may be
 * cut into `ksplit` slices of whole 32-element lane chunks whose partial sums
 * are combined in a fixed order (split-K).  NQ_ROUTE_TILED is the tiled
 * matrix-core (bf16 MFMA) product for many rows, in 128 x 128 tiles or (for
 * k a multiple of 64) 256 x 256 tiles. */
typedef enum { NQ_ROUTE_GEMV = 1, NQ_ROUTE_TILED = 2 } nq_route;

typedef struct {
    int32_t route;          /* nq_route */
    int32_t ksplit;         /* GEMV: K slices per output row, 1..8 (1 = no split) */
    int32_t rows_per_wave;  /* GEMV: weight rows per 64-lane wavefront: 0 = chosen per
                               launch chunk (it never changes a row's bits), else the
                               value that chunk takes -- 2 for m <= 2, 4 for more --
                               or NQ_ERR_PLAN */
    int32_t tile_m;         /* TILED: rows of x per workgroup tile */
    int32_t tile_n;         /* TILED: weight rows per workgroup tile */
    int32_t reserved[3];    /* zero */
} nq_plan;

/* The kernel choice for a product y[m, n] = x[m, k] . w_hat[n, k]^T.  A pure
 * function of its arguments and the device generation.  With row_exact = 0,
 * m <= 8 takes the GEMV family and m > 8 the tiled family (x in bf16; fp32 x
 * stays on the GEMV family, which keeps fp32 activations).  With
 * row_exact = 1 every m takes the GEMV family in chunks of at most 8 rows.
 * The GEMV family's ksplit depends only on (n, k), never on m, which is
 * (with the fixed per-row arithmetic of that family) what makes its rows
 * independent of how many rows share a call. */
nq_status nq_qmm_plan(int64_t m, int64_t n, int64_t k, int32_t group_size, int32_t bits,
                      nq_dtype x_dt, nq_dtype sb_dt, int32_t row_exact, nq_plan *plan);

/* Workspace bytes a product needs (0 for every current plan; reserved for
 * cross-workgroup split-K). */
size_t nq_qmm_workspace_bytes(int64_t m, int64_t n, int64_t k, int32_t group_size,
                              int32_t bits, nq_dtype x_dt, nq_dtype sb_dt, int32_t row_exact);

/* y [m, n] (x_dt) = x [m, k] (x_dt) times the transposed dequantized
 * weights (codes/scales/biases of n rows and k columns, see above), fp32
 * accumulation ("Affine" example: x.quantized_matmul(&q, true)).  The kernel
 * is chosen by nq_qmm_plan(..., row_exact = 0).  Rows m < 8 of a call are
 * already bit-equal to their one-row calls, since the GEMV family keeps each
 * row's arithmetic fixed. */
nq_status nq_qmm(const void *x, nq_dtype x_dt, int64_t m, int64_t k, const uint32_t *codes,
                 const void *scales, const void *biases, nq_dtype sb_dt, int64_t n,
                 int32_t group_size, int32_t bits, void *y, void *workspace,
                 size_t workspace_bytes, hipStream_t stream);

/* As nq_qmm in row-exact mode ("Products on the GPU" section; nuvec API index,
 * with_row_exact): every row of y is bit-equal to nq_qmm on that row alone,
 * for any m (chunks of at most NQ_ROW_INDEPENDENT_ROWS rows of the GEMV
 * family). */
nq_status nq_qmm_row_exact(const void *x, nq_dtype x_dt, int64_t m, int64_t k,
                           const uint32_t *codes, const void *scales, const void *biases,
                           nq_dtype sb_dt, int64_t n, int32_t group_size, int32_t bits, void *y,
                           void *workspace, size_t workspace_bytes, hipStream_t stream);

/* As nq_qmm with an explicit plan (for tests and tuning).  NQ_ERR_PLAN if the
 * plan does not fit.  Row independence is only promised for plans returned by
 * nq_qmm_plan. */
nq_status nq_qmm_with_plan(const nq_plan *plan, const void *x, nq_dtype x_dt, int64_t m,
                           int64_t k, const uint32_t *codes, const void *scales,
                           const void *biases, nq_dtype sb_dt, int64_t n, int32_t group_size,
                           int32_t bits, void *y, void *workspace, size_t workspace_bytes,
                           hipStream_t stream);

/* A product over batch items that keeps each item's solo bits (nuvec API
 * index, section "Determinism", batch items of quantized products: each item
 * gets the bits of its product alone, the split of K counted per item).  x [batch, l, k]
 * (x_dt), y [batch, l, n] (x_dt), weights as for nq_qmm; item i of y is
 * bit-equal to nq_qmm(x[i]) with m = l, whatever batch is, because the
 * route is nq_qmm_plan(l, ...) (not of batch * l rows) and no kernel's
 * result for an element depends on the other rows of its launch.  Errors
 * and conventions as for nq_qmm, with m = batch * l; NQ_ERR_SHAPE if
 * batch * l overflows. */
nq_status nq_qmm_batched(const void *x, nq_dtype x_dt, int64_t batch, int64_t l, int64_t k,
                         const uint32_t *codes, const void *scales, const void *biases,
                         nq_dtype sb_dt, int64_t n, int32_t group_size, int32_t bits, void *y,
                         void *workspace, size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------- weights as stored, derivatives */

/* Workspace bytes nq_qmm_notrans / nq_qmm_notrans_row_exact need: 0 on the
 * tiled route (row_exact = 0, m > NQ_ROW_INDEPENDENT_ROWS, bf16 x, ni a
 * multiple of 64), else room for the partial sums of the matrix's row ranges
 * (a function of ni and nc only), fully rewritten by every call. */
size_t nq_qmm_notrans_workspace_bytes(int64_t m, int64_t ni, int64_t nc, int32_t group_size,
                                      int32_t bits, nq_dtype x_dt, int32_t row_exact);

/* The product with the weights as stored, x times w_hat ("Affine" example:
 * quantized_matmul with the transpose flag off).  The quantized matrix has
 * ni rows of nc columns grouped along the columns: codes [ni, nc*bits/32],
 * scales and biases [ni, nc/group_size] (what nq_quantize makes of an
 * [ni, nc] matrix).  x [m, ni] (x_dt); y [m, nc] (x_dt):
 * y[r, c] = sum_i x[r, i] * (s[i, c/gs] * q[i, c] + b[i, c/gs]), fp32
 * accumulation.  With the forward weights (ni = n, nc = k) and x = dy this is
 * the derivative for the activations of nq_qmm ("Training through quantized
 * weights").  Routes: see nq_qmm_notrans_workspace_bytes; the matrix-vector
 * route splits the rows i into ranges fixed by (ni, nc) and adds their
 * partial sums in range order, so rows are run-to-run identical and bit-equal
 * to their one-row calls.  Errors as nq_qmm, nc % group_size != 0 is
 * NQ_ERR_SHAPE, a missing or short workspace NQ_ERR_WORKSPACE. */
nq_status nq_qmm_notrans(const void *x, nq_dtype x_dt, int64_t m, int64_t ni, const uint32_t *codes,
                         const void *scales, const void *biases, nq_dtype sb_dt, int64_t nc,
                         int32_t group_size, int32_t bits, void *y, void *workspace,
                         size_t workspace_bytes, hipStream_t stream);

/* As nq_qmm_notrans, every row of y bit-equal to the call on that row alone
 * (always the matrix-vector route). */
nq_status nq_qmm_notrans_row_exact(const void *x, nq_dtype x_dt, int64_t m, int64_t ni,
                                   const uint32_t *codes, const void *scales, const void *biases,
                                   nq_dtype sb_dt, int64_t nc, int32_t group_size, int32_t bits, void *y,
                                   void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Derivatives of L = sum(dy * nq_qmm(x, w)) for the scales and biases of w
 * ("Training through quantized weights": affine products have derivative
 * rules for the activations, scales and biases; the codes have none).
 * x [m, k] and dy [m, n] in x_dt; codes [n, k*bits/32] (w's, 4-byte
 * aligned); dscales and dbiases [n, k/group_size] in g_dt:
 *   dscales[c, g] = sum_r dy[r, c] * sum_{kk in group g} x[r, kk] * q[c, kk]
 *   dbiases[c, g] = sum_r dy[r, c] * sum_{kk in group g} x[r, kk]
 * fp32 accumulation in a fixed order (run-to-run identical).  m == 0 writes
 * zeros.  x, dy and the outputs need only element alignment.  The outputs
 * must not overlap each other or any input (NQ_ERR_ALIAS).  The derivative
 * for x is nq_qmm_notrans(dy, w). */
nq_status nq_qmm_grad_scales_biases(const void *x, const void *dy, nq_dtype x_dt, int64_t m, int64_t k,
                                    const uint32_t *codes, int64_t n, int32_t group_size, int32_t bits,
                                    void *dscales, void *dbiases, nq_dtype g_dt, hipStream_t stream);

/* ---------------------------------------------------------------- mixture of experts */

/* Workspace bytes nq_gather_qmm and nq_gather_qmm_row_exact need for these
 * arguments: nonzero once experts are shared by several vectors (rows * l
 * >= 16 and >= 4 * e, e <= 4096), when the vectors are grouped by expert on
 * the device and each expert's weights are read once per chunk of vectors.
 * The workspace holds that grouping (a permutation of the vectors and a
 * chunk table) and is fully rewritten by every call. */
size_t nq_gather_qmm_workspace_bytes(int64_t rows, int64_t l, int64_t k, int64_t e, int64_t n,
                                     int32_t group_size, int32_t bits, nq_dtype x_dt,
                                     nq_dtype sb_dt, int32_t sorted_hint);

/* gather_qmm ("Mixture of experts" section): x [rows, l, k] (x_dt); stacked
 * expert weights codes [e, n, k*bits/32], scales and biases [e, n, k/gs];
 * rhs_idx [rows] uint32 (the expert of each row).  y [rows, l, n] (x_dt):
 * y[r, j, :] = x[r, j, :] times the transposed weights of expert rhs_idx[r].
 * Weights are indexed in place, never copied.  An id >= e gives an all-zero
 * row of y (the id is never used to address memory).  The ids need not be
 * sorted; sorted_hint is accepted and changes nothing.  The route is a pure
 * function of the sizes and dtypes: with a nonzero workspace size (see
 * above), bf16 x and k a multiple of 64, vectors are grouped by expert into
 * chunks of up to 32 and multiplied on the matrix cores (rows within the
 * product tolerance of the exact result, like nq_qmm's tiled rows);
 * otherwise every row is bit-equal to nq_qmm_row_exact of x[r] with expert
 * rhs_idx[r]'s weights.  NQ_ERR_WORKSPACE if the workspace is needed and
 * missing or short; it must not overlap any argument. */
nq_status nq_gather_qmm(const void *x, nq_dtype x_dt, int64_t rows, int64_t l, int64_t k,
                        const uint32_t *codes, const void *scales, const void *biases,
                        nq_dtype sb_dt, int64_t e, int64_t n, int32_t group_size, int32_t bits,
                        const uint32_t *rhs_idx, int32_t sorted_hint, void *y, void *workspace,
                        size_t workspace_bytes, hipStream_t stream);

/* For callers that cannot allocate -- code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc: nq_gather_qmm with its
 * workspace taken from a static array of NQ_NOALLOC_SCRATCH_BYTES (1 MiB) in
 * the library's own device memory, one per GPU, held until the process
 * ends.  Same arguments (minus the workspace), routes, results and errors
 * as nq_gather_qmm, and bit-identical outputs; NQ_ERR_WORKSPACE if the
 * grouping tables would need more than the array holds (a workspace size
 * above 1 MiB: about 160,000 vectors).  It calls no hipMalloc, hipFree or
 * other allocating routine; the array's address is looked up once per GPU
 * (hipGetSymbolAddress).  Every call on one GPU uses the same array and
 * leaves its tables in it: calls that overlap in time on one GPU (on other
 * streams or threads) race, and the caller must order them. */
#define NQ_NOALLOC_SCRATCH_BYTES (1u << 20)
nq_status nq_gather_qmm_noalloc(const void *x, nq_dtype x_dt, int64_t rows, int64_t l, int64_t k,
                                const uint32_t *codes, const void *scales, const void *biases,
                                nq_dtype sb_dt, int64_t e, int64_t n, int32_t group_size, int32_t bits,
                                const uint32_t *rhs_idx, int32_t sorted_hint, void *y, hipStream_t stream);

/* As nq_gather_qmm in row-exact mode ("Products on the GPU" section; nuvec
 * API index, with_row_exact): every row of y is bit-equal to
 * nq_qmm_row_exact of x[r] with expert rhs_idx[r]'s weights, whatever the
 * ids.  Grouped vectors (same workspace rule) run as chunks of up to 8
 * through the matrix-vector family, whose rows never depend on the chunk. */
nq_status nq_gather_qmm_row_exact(const void *x, nq_dtype x_dt, int64_t rows, int64_t l, int64_t k,
                                  const uint32_t *codes, const void *scales, const void *biases,
                                  nq_dtype sb_dt, int64_t e, int64_t n, int32_t group_size,
                                  int32_t bits, const uint32_t *rhs_idx, int32_t sorted_hint,
                                  void *y, void *workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/* gather_qmm with indices on both sides ("Mixture of experts" section: the
 * gathered product picks the activation batch and the expert per output
 * row).  x [x_items, l, k]; lhs_idx [rows] and rhs_idx [rows] uint32:
 *   y[r, j, :] = x[lhs_idx[r], j, :] times expert rhs_idx[r]'s transposed weights.
 * lhs_idx[r] >= x_items, like rhs_idx[r] >= e, gives an all-zero row of y
 * and is never used to address memory.  x_items >= 1 (NQ_ERR_SHAPE
 * otherwise); lhs_idx must be non-null (NQ_ERR_NULL), 4-byte aligned and
 * must not overlap y or the workspace.  row_exact != 0 takes the row-exact
 * mode of nq_gather_qmm_row_exact (each row bit-equal to nq_qmm_row_exact of
 * its x row with its expert's weights); otherwise the routes, the
 * workspace (nq_gather_qmm_workspace_bytes with these rows, l, k, e, n) and
 * the tolerance are those of nq_gather_qmm.  With lhs_idx[r] = r and
 * x_items = rows the results equal nq_gather_qmm's / _row_exact's bit for
 * bit. */
nq_status nq_gather_qmm_lhs(const void *x, nq_dtype x_dt, int64_t x_items, int64_t rows, int64_t l,
                            int64_t k, const uint32_t *codes, const void *scales, const void *biases,
                            nq_dtype sb_dt, int64_t e, int64_t n, int32_t group_size, int32_t bits,
                            const uint32_t *lhs_idx, const uint32_t *rhs_idx, int32_t sorted_hint,
                            int32_t row_exact, void *y, void *workspace, size_t workspace_bytes,
                            hipStream_t stream);

/* ---------------------------------------------------------------- floating-point modes */

/* Floating-point quantization modes ("Quantization" page, section
 * "Floating-point formats": every weight a small float, one uint8 scale code
 * per group, no biases; dequantize gives bf16; products in x's dtype).  The
 * page names the modes; their encodings are the public format definitions:
 *   NQ_MXFP4  OCP Microscaling Formats v1.0, MXFP4: groups of 32 FP4 E2M1
 *             elements (4-bit codes) sharing one E8M0 scale code s, value
 *             2^(s - 127) (s = 255: NaN).
 *   NQ_MXFP8  the same with FP8 E4M3 elements (8-bit codes; bias 7, largest
 *             value 448, S.1111.111 NaN, no infinities).
 *   NQ_NVFP4  groups of 16 E2M1 elements sharing one E4M3 scale code, and in
 *             products an optional fp32 global scale (section "Mixture of
 *             experts": one per expert).
 * Layout of a matrix of n rows and k columns: codes [n, k*bits/32] uint32,
 * packed LSB-first exactly like the affine codes (bits = 4 or 8); scales
 * [n, k/group] uint8.  k must be a multiple of 32 (NQ_ERR_SHAPE); an
 * unknown mode is NQ_ERR_QUANT.  A weight's value is S * E (S the decoded
 * scale, E the decoded element), times the global scale in products. */
typedef enum { NQ_MXFP4 = 1, NQ_MXFP8 = 2, NQ_NVFP4 = 3 } nq_fp_mode;

/* Quantize w [n, k] (w_dt) -- a reading of the formats' conversion rules,
 * every decision taken on fp32 values, bit-exact:
 *   MX: s = clamp(floor(log2(max |w| of the group)) - emax + 127, 0, 254),
 *       emax = 2 (E2M1) or 8 (E4M3), an all-zero group gets s = 0; each code
 *       is the element nearest to w * 2^(127 - s).
 *   NVFP4: s = the E4M3 code nearest to fp32(max |w| / 6); each code is the
 *       E2M1 element nearest to fp32(w / S), S the decoded scale; S = 0 gives
 *       zero codes.
 * "Nearest" breaks ties to the even code, saturates at the largest finite
 * magnitude (6 or 448) and keeps the value's sign (also for a zero).
 * Outputs codes and scales as laid out above.  Non-finite weights are
 * outside the contract. */
nq_status nq_fp_quantize(const void *w, nq_dtype w_dt, int64_t n, int64_t k, int32_t mode,
                         uint32_t *codes, uint8_t *scales, hipStream_t stream);

/* Dequantize: w_out[r, j] = S * E computed in fp32 (exact for these formats
 * unless it overflows to infinity), rounded to nearest even into out_dt
 * (bf16 is the page's default); a NaN scale or element gives the quiet NaN
 * 0x7fc0 (bf16) or 0x7fc00000 (fp32). */
nq_status nq_fp_dequantize(const uint32_t *codes, const uint8_t *scales, int64_t n, int64_t k,
                           int32_t mode, void *w_out, nq_dtype out_dt, hipStream_t stream);

/* y[m, n] = x[m, k] . (g * w_hat)^T in x's dtype with fp32 accumulation, g =
 * *global_scale (a device pointer to one fp32; NVFP4 only, else NQ_ERR_QUANT;
 * null: 1).  With m <= 8 or row_exact = 1 the matrix-vector kernel runs in
 * chunks of up to 8 rows, and every row is bit-equal to its one-row product;
 * otherwise (bf16 x, k a multiple of 64) 128 x 128 bf16-MFMA tiles, whose
 * B operands are bf16(S * E) (exact while |S * E| fits bf16; beyond -- only
 * with E8M0 scale codes near 2^127 -- an infinite operand makes its output
 * column non-finite, where the matrix-vector route stays finite).  Tolerance
 * as for the affine products. */
nq_status nq_fp_qmm(const void *x, nq_dtype x_dt, int64_t m, int64_t k, const uint32_t *codes,
                    const uint8_t *scales, const float *global_scale, int64_t n, int32_t mode,
                    int32_t row_exact, void *y, hipStream_t stream);

/* Workspace bytes of nq_fp_gather_qmm: nonzero once experts are shared by
 * several vectors (rows * l >= 16 and >= 4 * e, e <= 4096 -- the thresholds
 * of the "Mixture of experts" section), when the vectors are grouped by
 * expert on the device and each expert's weights are read once per chunk of
 * vectors (either route). */
size_t nq_fp_gather_qmm_workspace_bytes(int64_t rows, int64_t l, int64_t k, int64_t e, int64_t n);

/* gather_qmm in a floating-point mode ("Mixture of experts" section): x
 * [rows, l, k]; experts codes [e, n, k*bits/32] and scales [e, n, k/group];
 * global_scales [e] fp32 (NVFP4 only; null: 1); rhs_idx [rows] uint32.
 * y [rows, l, n]: y[r, j, :] = x[r, j, :] . (g[i] * w_hat[i])^T with i =
 * rhs_idx[r]; rhs_idx[r] >= e gives an all-zero row.  Routes: few vectors,
 * matrix-vector products per row; shared experts (see the workspace
 * function), the vectors grouped by expert on the device, then with
 * row_exact = 0, bf16 x and k a multiple of 64 bf16-MFMA tiles over chunks
 * of up to 32 vectors (the affine products' tolerance), otherwise the
 * matrix-vector kernel over chunks of up to 8.  With row_exact = 1 every
 * row is bit-equal to nq_fp_qmm(row_exact = 1) of x[r] with expert i's
 * weights and global scale.  workspace: at least
 * nq_fp_gather_qmm_workspace_bytes (16-byte aligned; NQ_ERR_WORKSPACE if
 * short). */
nq_status nq_fp_gather_qmm(const void *x, nq_dtype x_dt, int64_t rows, int64_t l, int64_t k,
                           const uint32_t *codes, const uint8_t *scales, const float *global_scales,
                           int64_t e, int64_t n, int32_t mode, const uint32_t *rhs_idx, int32_t row_exact,
                           void *y, void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Product with the weights as stored in a floating-point mode (the
 * "transpose = false" product; with the forward weights, dy . w_hat is the
 * derivative for the activations, "Training through quantized weights"):
 * y[m, c] = x[m, i] . (g * w_hat)[i, c] for a quantized matrix w_hat
 * [ni, nc] laid out as above with groups along nc (nc a multiple of 32);
 * g = *global_scale (NVFP4 only; null: 1); y in x's dtype.  Routes: with
 * row_exact = 0, m > 8, bf16 x and ni a multiple of 64, 128 x 128 bf16-MFMA
 * tiles (no workspace); otherwise row ranges of w_hat fixed by (ni, nc)
 * write fp32 partial sums to the workspace, added in range order, so every
 * row is bit-equal to its one-row product.  workspace: at least
 * nq_fp_qmm_notrans_workspace_bytes bytes (16-byte aligned; NQ_ERR_WORKSPACE
 * if short). */
size_t nq_fp_qmm_notrans_workspace_bytes(int64_t m, int64_t ni, int64_t nc, int32_t mode, nq_dtype x_dt,
                                         int32_t row_exact);
nq_status nq_fp_qmm_notrans(const void *x, nq_dtype x_dt, int64_t m, int64_t ni, const uint32_t *codes,
                            const uint8_t *scales, const float *global_scale, int64_t nc, int32_t mode,
                            int32_t row_exact, void *y, void *workspace, size_t workspace_bytes,
                            hipStream_t stream);

/* ---------------------------------------------------------------- errors */

/* A static description of a status code. */
const char *nq_status_string(nq_status s);

/* The message of the calling thread's last call ("" if it succeeded): the
 * entry point and the reason, e.g. "nq_qmm: k=500 is not a multiple of
 * group_size=64".  Valid until the thread's next call into the library. */
const char *nq_last_error(void);

/* Library version, "major.minor.patch". */
const char *nq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NQ_H */
