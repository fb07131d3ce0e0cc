// C-ABI entry points of libnq: argument validation, the pure kernel planner
// and dispatch to the kernel translation units.  See include/nq.h for the
// contract of every call.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "nq.h"
#include "nq_internal.h"

namespace {

thread_local std::string g_last_error;

nq_status fail(nq_status st, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

bool dtype_ok(int dt) { return dt == NQ_F32 || dt == NQ_BF16; }
int64_t dtype_bytes(int dt) { return dt == NQ_F32 ? 4 : 2; }

// Bit widths of the stand-alone quantize/dequantize kernels and of the
// product kernels ("an unsupported combination fails in the operation that
// uses it").
bool storage_bits_ok(int b) { return b == 1 || b == 2 || b == 3 || b == 4 || b == 5 || b == 6 || b == 8; }
bool product_bits_ok(int b) { return storage_bits_ok(b); }
bool group_ok(int gs) { return gs == 32 || gs == 64 || gs == 128; }

constexpr int64_t kMaxDim = (int64_t)1 << 31;
constexpr int64_t kMaxElems = (int64_t)1 << 40;

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned_to(const void *p, int64_t a) { return ((uintptr_t)p % (uintptr_t)a) == 0; }

struct Span {
    const void *p;
    int64_t bytes;
};

bool overlap(Span a, Span b)
{
    if (!a.p || !b.p || a.bytes <= 0 || b.bytes <= 0) return false;
    const uintptr_t a0 = (uintptr_t)a.p, a1 = a0 + (uintptr_t)a.bytes;
    const uintptr_t b0 = (uintptr_t)b.p, b1 = b0 + (uintptr_t)b.bytes;
    return a0 < b1 && b0 < a1;
}

nq_status check_quant(const char *op, int gs, int bits, bool product)
{
    if (!group_ok(gs)) return fail(NQ_ERR_QUANT, "%s: group_size=%d is not 32, 64 or 128", op, gs);
    if (product ? !product_bits_ok(bits) : !storage_bits_ok(bits))
        return fail(NQ_ERR_QUANT, "%s: bits=%d is not supported (%s)", op, bits,
                    "1, 2, 3, 4, 5, 6 or 8");
    return NQ_OK;
}

nq_status check_dims(const char *op, int64_t n, int64_t k, int gs)
{
    if (n < 0 || k < 0) return fail(NQ_ERR_SHAPE, "%s: negative size (n=%lld, k=%lld)", op,
                                    (long long)n, (long long)k);
    if (n >= kMaxDim || k >= kMaxDim || (k > 0 && n > kMaxElems / k))
        return fail(NQ_ERR_SHAPE, "%s: size too large (n=%lld, k=%lld)", op, (long long)n,
                    (long long)k);
    if (k % gs != 0)
        return fail(NQ_ERR_SHAPE, "%s: k=%lld is not a multiple of group_size=%d", op,
                    (long long)k, gs);
    return NQ_OK;
}

nq_status check_launch(const char *op, hipError_t err)
{
    if (err != hipSuccess)
        return fail(NQ_ERR_LAUNCH, "%s: kernel launch failed: %s", op, hipGetErrorString(err));
    return NQ_OK;
}

// The K split of the matrix-vector family.  A function of (n, k) only --
// never of the row count -- so that a row's arithmetic is the same however
// many rows share the call.  Enough waves are formed to keep every compute
// unit's memory pipeline busy: about 2048 waves (8 per CU on 256 CUs).
int gemv_ksplit(int64_t n, int64_t k, int gs, int bits, int x_dt)
{
    if (nqk::gemv_band_family(n, k, gs, bits, x_dt)) return nqk::kBandKsplit;   // four K quarters
    if (nqk::gemv_mfma_family(n, k, gs, bits, x_dt)) {
        // matrix-core waves own 32 weight rows; K units are groups of 128 or
        // steps of 64
        const int64_t units = gs >= 128 ? k / gs : k / 64;
        const int64_t base_waves = (n + 31) / 32;
        const int64_t want = (2048 + base_waves - 1) / std::max<int64_t>(base_waves, 1);
        return (int)std::max<int64_t>(1, std::min<int64_t>({want, units, 8}));
    }
    const int64_t steps = (k + nqk::kStepElems - 1) / nqk::kStepElems;
    if (steps <= 1) return 1;
    const int64_t base_waves = (n + 3) / 4;
    const int64_t want = (2048 + base_waves - 1) / std::max<int64_t>(base_waves, 1);
    return (int)std::max<int64_t>(1, std::min<int64_t>({want, steps, 8}));
}

nq_status make_plan(const char *op, int64_t m, int64_t n, int64_t k, int gs, int bits,
                    int x_dt, int sb_dt, int row_exact, nq_plan *plan)
{
    memset(plan, 0, sizeof *plan);
    const bool tiled = !row_exact && m > NQ_ROW_INDEPENDENT_ROWS && x_dt == NQ_BF16 &&
                       nqk::tiled_supported(128, 128, bits);
    (void)op;
    if (tiled) {
        plan->route = NQ_ROUTE_TILED;
        // 256 x 256 tiles when the product is large enough to fill them
        const bool big = m >= 128 && n >= 256 && nqk::tiled_fits(256, 256, bits, gs, sb_dt, m, n, k);
        plan->tile_m = big ? 256 : 128;
        plan->tile_n = big ? 256 : 128;
    } else {
        plan->route = NQ_ROUTE_GEMV;
        plan->ksplit = gemv_ksplit(n, k, gs, bits, x_dt);
        plan->rows_per_wave = 0;   // chosen per launch chunk; no effect on a row's bits
    }
    return NQ_OK;
}

nq_status check_plan(const char *op, const nq_plan *plan, int x_dt, int sb_dt, int gs, int bits,
                     int64_t m, int64_t n, int64_t k)
{
    if (!plan) return fail(NQ_ERR_NULL, "%s: plan is null", op);
    if (plan->route == NQ_ROUTE_GEMV) {
        if (plan->ksplit < 1 || plan->ksplit > 8)
            return fail(NQ_ERR_PLAN, "%s: ksplit=%d is not in [1, 8]", op, plan->ksplit);
        if (plan->rows_per_wave != 0 && plan->rows_per_wave != 2 && plan->rows_per_wave != 4)
            return fail(NQ_ERR_PLAN, "%s: rows_per_wave=%d is not supported (0, 2 or 4)", op,
                        plan->rows_per_wave);
        // the VALU kernels take 2 rows per wave for launch chunks of one or
        // two activation rows and 4 for more (the matrix-core forms ignore it)
        const int fit = std::min<int64_t>(m, 8) <= 2 ? 2 : 4;
        if (plan->rows_per_wave != 0 && plan->rows_per_wave != fit &&
            !nqk::gemv_mfma_family(n, k, gs, bits, x_dt))
            return fail(NQ_ERR_PLAN, "%s: rows_per_wave=%d does not fit m=%lld (%d)", op,
                        plan->rows_per_wave, (long long)m, fit);
        return NQ_OK;
    }
    if (plan->route == NQ_ROUTE_TILED) {
        if (x_dt != NQ_BF16) return fail(NQ_ERR_PLAN, "%s: the tiled route takes bf16 x", op);
        if (!nqk::tiled_supported(plan->tile_m, plan->tile_n, bits))
            return fail(NQ_ERR_PLAN, "%s: tile %dx%d is not supported", op, plan->tile_m,
                        plan->tile_n);
        if (!nqk::tiled_fits(plan->tile_m, plan->tile_n, bits, gs, sb_dt, m, n, k))
            return fail(NQ_ERR_PLAN, "%s: tile %dx%d does not fit m=%lld n=%lld k=%lld", op,
                        plan->tile_m, plan->tile_n, (long long)m, (long long)n, (long long)k);
        return NQ_OK;
    }
    return fail(NQ_ERR_PLAN, "%s: unknown route %d", op, plan->route);
}

struct QmmArgs {
    const void *x;
    int x_dt;
    int64_t m, k;
    const uint32_t *codes;
    const void *scales, *biases;
    int sb_dt;
    int64_t n;
    int gs, bits;
    void *y;
    void *ws;
    size_t ws_bytes;
};

nq_status check_qmm(const char *op, const QmmArgs &a, bool *empty)
{
    *empty = false;
    if (!dtype_ok(a.x_dt) || !dtype_ok(a.sb_dt))
        return fail(NQ_ERR_DTYPE, "%s: unknown dtype (x_dt=%d, sb_dt=%d)", op, a.x_dt, a.sb_dt);
    nq_status st = check_quant(op, a.gs, a.bits, true);
    if (st) return st;
    if (a.m < 0) return fail(NQ_ERR_SHAPE, "%s: negative m=%lld", op, (long long)a.m);
    if ((st = check_dims(op, a.n, a.k, a.gs))) return st;
    if (a.m >= kMaxDim || (a.k > 0 && a.m > kMaxElems / a.k) || (a.n > 0 && a.m > kMaxElems / a.n))
        return fail(NQ_ERR_SHAPE, "%s: m=%lld is too large", op, (long long)a.m);
    if (a.m == 0 || a.n == 0) {
        *empty = true;
        return NQ_OK;
    }
    if (!a.y) return fail(NQ_ERR_NULL, "%s: y is null", op);
    if (a.k > 0 && (!a.x || !a.codes || !a.scales || !a.biases))
        return fail(NQ_ERR_NULL, "%s: x, codes, scales and biases must be non-null", op);
    if (!aligned16(a.x) || !aligned16(a.codes) || !aligned16(a.y))
        return fail(NQ_ERR_ALIGN, "%s: x, codes and y must be 16-byte aligned", op);
    if (!aligned_to(a.scales, dtype_bytes(a.sb_dt)) || !aligned_to(a.biases, dtype_bytes(a.sb_dt)))
        return fail(NQ_ERR_ALIGN, "%s: scales and biases must be aligned to %lld bytes", op,
                    (long long)dtype_bytes(a.sb_dt));
    const Span y{a.y, a.m * a.n * dtype_bytes(a.x_dt)};
    const Span ins[4] = {{a.x, a.m * a.k * dtype_bytes(a.x_dt)},
                         {a.codes, a.n * (a.k * a.bits / 32) * 4},
                         {a.scales, a.n * (a.k / a.gs) * dtype_bytes(a.sb_dt)},
                         {a.biases, a.n * (a.k / a.gs) * dtype_bytes(a.sb_dt)}};
    static const char *names[4] = {"x", "codes", "scales", "biases"};
    for (int i = 0; i < 4; ++i)
        if (overlap(y, ins[i])) return fail(NQ_ERR_ALIAS, "%s: y overlaps %s", op, names[i]);
    return NQ_OK;
}

nq_status run_qmm(const char *op, const nq_plan &plan, const QmmArgs &a, hipStream_t stream)
{
    if (plan.route == NQ_ROUTE_TILED) {
        nqk::TiledLaunch t;
        t.x = a.x;
        t.y = a.y;
        t.codes = a.codes;
        t.scales = a.scales;
        t.biases = a.biases;
        t.sb_dt = a.sb_dt;
        t.m = a.m;
        t.n = a.n;
        t.k = a.k;
        t.gs = a.gs;
        t.bits = a.bits;
        t.tile_m = plan.tile_m;
        t.tile_n = plan.tile_n;
        return check_launch(op, nqk::launch_tiled(t, stream));
    }
    nqk::GemvLaunch g;
    g.x = a.x;
    g.y = a.y;
    g.codes = a.codes;
    g.scales = a.scales;
    g.biases = a.biases;
    g.idx = nullptr;
    g.x_dt = a.x_dt;
    g.sb_dt = a.sb_dt;
    g.items = 1;
    g.rows_per_item = a.m;
    g.k = a.k;
    g.n = a.n;
    g.e = 1;
    g.gs = a.gs;
    g.bits = a.bits;
    g.ksplit = plan.ksplit;
    g.rows_per_wave = plan.rows_per_wave;
    return check_launch(op, nqk::launch_gemv(g, stream));
}

nq_status qmm_common(const char *op, int row_exact, const nq_plan *forced, const QmmArgs &a,
                     hipStream_t stream)
{
    g_last_error.clear();
    bool empty = false;
    nq_status st = check_qmm(op, a, &empty);
    if (st || empty) return st;
    nq_plan plan;
    if (forced) {
        if ((st = check_plan(op, forced, a.x_dt, a.sb_dt, a.gs, a.bits, a.m, a.n, a.k))) return st;
        plan = *forced;
    } else {
        make_plan(op, a.m, a.n, a.k, a.gs, a.bits, a.x_dt, a.sb_dt, row_exact, &plan);
    }
    return run_qmm(op, plan, a, stream);
}

// ---- product with the weights as stored, derivatives

// Route of the product with the weights as stored: 128 x 128 MFMA tiles for
// many bf16 rows (the ranges of i a multiple of 64), else the matrix-vector
// pair, which keeps every row bit-equal to its one-row product.  A pure
// function of the sizes, dtypes and mode.
bool nt_tiled(int64_t m, int64_t ni, int x_dt, int row_exact)
{
    return !row_exact && m > NQ_ROW_INDEPENDENT_ROWS && x_dt == NQ_BF16 && ni % 64 == 0;
}

nq_status qmm_nt_impl(const char *op, int row_exact, const void *x, nq_dtype x_dt, int64_t m,
                      int64_t ni, const uint32_t *codes, const void *scales, const void *biases,
                      nq_dtype sb_dt, int64_t nc, int32_t group_size, int32_t bits, void *y,
                      void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    g_last_error.clear();
    if (!dtype_ok(x_dt) || !dtype_ok(sb_dt))
        return fail(NQ_ERR_DTYPE, "%s: unknown dtype (x_dt=%d, sb_dt=%d)", op, (int)x_dt, (int)sb_dt);
    nq_status st = check_quant(op, group_size, bits, true);
    if (st) return st;
    if (m < 0 || ni < 0) return fail(NQ_ERR_SHAPE, "%s: negative size (m=%lld, ni=%lld)", op,
                                     (long long)m, (long long)ni);
    if ((st = check_dims(op, ni, nc, group_size))) return st;
    if (m >= kMaxDim || (ni > 0 && m > kMaxElems / ni) || (nc > 0 && m > kMaxElems / nc))
        return fail(NQ_ERR_SHAPE, "%s: m=%lld is too large", op, (long long)m);
    if (m == 0 || nc == 0) return NQ_OK;
    if (!y) return fail(NQ_ERR_NULL, "%s: y is null", op);
    if (ni > 0 && (!x || !codes || !scales || !biases))
        return fail(NQ_ERR_NULL, "%s: x, codes, scales and biases must be non-null", op);
    if (!aligned16(x) || !aligned16(codes) || !aligned16(y))
        return fail(NQ_ERR_ALIGN, "%s: x, codes and y must be 16-byte aligned", op);
    const int64_t sbb = dtype_bytes(sb_dt);
    if (!aligned_to(scales, sbb) || !aligned_to(biases, sbb))
        return fail(NQ_ERR_ALIGN, "%s: scales and biases must be aligned to %lld bytes", op, (long long)sbb);
    const Span sy{y, m * nc * dtype_bytes(x_dt)};
    const Span ins[4] = {{x, m * ni * dtype_bytes(x_dt)},
                         {codes, ni * (nc * bits / 32) * 4},
                         {scales, ni * (nc / group_size) * sbb},
                         {biases, ni * (nc / group_size) * sbb}};
    static const char *names[4] = {"x", "codes", "scales", "biases"};
    for (int i = 0; i < 4; ++i)
        if (overlap(sy, ins[i])) return fail(NQ_ERR_ALIAS, "%s: y overlaps %s", op, names[i]);
    nqk::NtLaunch a;
    a.x = x;
    a.y = y;
    a.codes = codes;
    a.scales = scales;
    a.biases = biases;
    a.workspace = workspace;
    a.x_dt = x_dt;
    a.sb_dt = sb_dt;
    a.m = m;
    a.ni = ni;
    a.nc = nc;
    a.gs = group_size;
    a.bits = bits;
    a.tiled = nt_tiled(m, ni, x_dt, row_exact);
    if (!a.tiled) {
        const size_t need = nqk::qmm_nt_ws_bytes(ni, nc);
        if (!workspace || workspace_bytes < need)
            return fail(NQ_ERR_WORKSPACE, "%s: needs a workspace of %zu bytes (got %zu)", op, need,
                        workspace ? workspace_bytes : (size_t)0);
        if (!aligned16(workspace)) return fail(NQ_ERR_ALIGN, "%s: workspace must be 16-byte aligned", op);
        const Span sw{workspace, (int64_t)need};
        if (overlap(sw, sy)) return fail(NQ_ERR_ALIAS, "%s: workspace overlaps y", op);
        for (int i = 0; i < 4; ++i)
            if (overlap(sw, ins[i])) return fail(NQ_ERR_ALIAS, "%s: workspace overlaps %s", op, names[i]);
    }
    return check_launch(op, nqk::launch_qmm_nt(a, stream));
}

// ---- floating-point modes
bool fp_mode_ok(int mode) { return mode == NQ_MXFP4 || mode == NQ_MXFP8 || mode == NQ_NVFP4; }

nq_status check_fp(const char *op, int mode, int64_t n, int64_t k)
{
    if (!fp_mode_ok(mode))
        return fail(NQ_ERR_QUANT, "%s: mode=%d is not NQ_MXFP4, NQ_MXFP8 or NQ_NVFP4", op, mode);
    if (n < 0 || k < 0) return fail(NQ_ERR_SHAPE, "%s: negative size (n=%lld, k=%lld)", op,
                                    (long long)n, (long long)k);
    if (n >= kMaxDim || k >= kMaxDim || (k > 0 && n > kMaxElems / k))
        return fail(NQ_ERR_SHAPE, "%s: size too large (n=%lld, k=%lld)", op, (long long)n,
                    (long long)k);
    if (k % 32 != 0)
        return fail(NQ_ERR_SHAPE, "%s: k=%lld is not a multiple of 32", op, (long long)k);
    return NQ_OK;
}

int64_t fp_code_bytes(int mode, int64_t n, int64_t k) { return n * (k * nqk::fp_mode_bits(mode) / 32) * 4; }
int64_t fp_scale_bytes(int mode, int64_t n, int64_t k) { return n * (k / nqk::fp_mode_group(mode)); }

nq_status check_global_scale(const char *op, int mode, const float *g)
{
    if (g && mode != NQ_NVFP4)
        return fail(NQ_ERR_QUANT, "%s: a global scale is only defined for NQ_NVFP4", op);
    if (g && !aligned_to(g, 4)) return fail(NQ_ERR_ALIGN, "%s: global scales must be 4-byte aligned", op);
    return NQ_OK;
}

}  // namespace

extern "C" {

size_t nq_qmm_notrans_workspace_bytes(int64_t m, int64_t ni, int64_t nc, int32_t group_size,
                                      int32_t bits, nq_dtype x_dt, int32_t row_exact)
{
    (void)group_size, (void)bits;
    if (m <= 0 || ni < 0 || nc <= 0 || nt_tiled(m, ni, x_dt, row_exact)) return 0;
    return nqk::qmm_nt_ws_bytes(ni, nc);
}

nq_status nq_qmm_notrans(const void *x, nq_dtype x_dt, int64_t m, int64_t ni, const uint32_t *codes,
                         const void *scales, const void *biases, nq_dtype sb_dt, int64_t nc,
                         int32_t group_size, int32_t bits, void *y, void *workspace,
                         size_t workspace_bytes, hipStream_t stream)
{
    return qmm_nt_impl("nq_qmm_notrans", 0, x, x_dt, m, ni, codes, scales, biases, sb_dt, nc, group_size,
                       bits, y, workspace, workspace_bytes, stream);
}

nq_status nq_qmm_notrans_row_exact(const void *x, nq_dtype x_dt, int64_t m, int64_t ni,
                                   const uint32_t *codes, const void *scales, const void *biases,
                                   nq_dtype sb_dt, int64_t nc, int32_t group_size, int32_t bits, void *y,
                                   void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    return qmm_nt_impl("nq_qmm_notrans_row_exact", 1, x, x_dt, m, ni, codes, scales, biases, sb_dt, nc,
                       group_size, bits, y, workspace, workspace_bytes, stream);
}

nq_status nq_qmm_grad_scales_biases(const void *x, const void *dy, nq_dtype x_dt, int64_t m, int64_t k,
                                    const uint32_t *codes, int64_t n, int32_t group_size, int32_t bits,
                                    void *dscales, void *dbiases, nq_dtype g_dt, hipStream_t stream)
{
    const char *op = "nq_qmm_grad_scales_biases";
    g_last_error.clear();
    if (!dtype_ok(x_dt) || !dtype_ok(g_dt))
        return fail(NQ_ERR_DTYPE, "%s: unknown dtype (x_dt=%d, g_dt=%d)", op, (int)x_dt, (int)g_dt);
    nq_status st = check_quant(op, group_size, bits, true);
    if (st) return st;
    if (m < 0) return fail(NQ_ERR_SHAPE, "%s: negative m=%lld", op, (long long)m);
    if ((st = check_dims(op, n, k, group_size))) return st;
    if (m >= kMaxDim || (k > 0 && m > kMaxElems / k) || (n > 0 && m > kMaxElems / n))
        return fail(NQ_ERR_SHAPE, "%s: m=%lld is too large", op, (long long)m);
    if (n == 0 || k == 0) return NQ_OK;
    if (!dscales || !dbiases || !codes)
        return fail(NQ_ERR_NULL, "%s: codes, dscales and dbiases must be non-null", op);
    if (m > 0 && (!x || !dy)) return fail(NQ_ERR_NULL, "%s: x and dy must be non-null", op);
    if (!aligned_to(x, dtype_bytes(x_dt)) || !aligned_to(dy, dtype_bytes(x_dt)) || !aligned_to(codes, 4))
        return fail(NQ_ERR_ALIGN, "%s: x, dy and codes must be aligned to their element size", op);
    const int64_t gb = dtype_bytes(g_dt);
    if (!aligned_to(dscales, gb) || !aligned_to(dbiases, gb))
        return fail(NQ_ERR_ALIGN, "%s: dscales and dbiases must be aligned to %lld bytes", op, (long long)gb);
    const int64_t G = k / group_size;
    const Span outs[2] = {{dscales, n * G * gb}, {dbiases, n * G * gb}};
    const Span ins[3] = {{x, m * k * dtype_bytes(x_dt)}, {dy, m * n * dtype_bytes(x_dt)},
                         {codes, n * (k * bits / 32) * 4}};
    static const char *onames[2] = {"dscales", "dbiases"}, *inames[3] = {"x", "dy", "codes"};
    if (overlap(outs[0], outs[1])) return fail(NQ_ERR_ALIAS, "%s: dscales overlaps dbiases", op);
    for (int o = 0; o < 2; ++o)
        for (int i = 0; i < 3; ++i)
            if (overlap(outs[o], ins[i]))
                return fail(NQ_ERR_ALIAS, "%s: %s overlaps %s", op, onames[o], inames[i]);
    nqk::GradLaunch a;
    a.x = x;
    a.dy = dy;
    a.codes = codes;
    a.ds = dscales;
    a.db = dbiases;
    a.x_dt = x_dt;
    a.g_dt = g_dt;
    a.m = m;
    a.k = k;
    a.n = n;
    a.gs = group_size;
    a.bits = bits;
    return check_launch(op, nqk::launch_grad_sb(a, stream));
}


nq_status nq_quantize(const void *w, nq_dtype w_dt, int64_t n, int64_t k, int32_t group_size,
                      int32_t bits, uint32_t *codes, void *scales, void *biases, hipStream_t stream)
{
    const char *op = "nq_quantize";
    g_last_error.clear();
    if (!dtype_ok(w_dt)) return fail(NQ_ERR_DTYPE, "%s: unknown dtype w_dt=%d", op, (int)w_dt);
    nq_status st = check_quant(op, group_size, bits, false);
    if (st) return st;
    if ((st = check_dims(op, n, k, group_size))) return st;
    if (n == 0 || k == 0) return NQ_OK;
    if (!w || !codes || !scales || !biases)
        return fail(NQ_ERR_NULL, "%s: w, codes, scales and biases must be non-null", op);
    if (!aligned16(w) || !aligned16(codes))
        return fail(NQ_ERR_ALIGN, "%s: w and codes must be 16-byte aligned", op);
    const int64_t eb = dtype_bytes(w_dt);
    if (!aligned_to(scales, eb) || !aligned_to(biases, eb))
        return fail(NQ_ERR_ALIGN, "%s: scales and biases must be aligned to %lld bytes", op,
                    (long long)eb);
    const Span sw{w, n * k * eb}, sc{codes, n * (k * bits / 32) * 4},
        ss{scales, n * (k / group_size) * eb}, sbi{biases, n * (k / group_size) * eb};
    if (overlap(sc, sw) || overlap(ss, sw) || overlap(sbi, sw))
        return fail(NQ_ERR_ALIAS, "%s: an output overlaps w", op);
    if (overlap(sc, ss) || overlap(sc, sbi) || overlap(ss, sbi))
        return fail(NQ_ERR_ALIAS, "%s: codes, scales and biases overlap", op);
    return check_launch(op, nqk::launch_quantize(w, w_dt, n, k, group_size, bits, codes, scales,
                                                 biases, stream));
}

nq_status nq_dequantize(const uint32_t *codes, const void *scales, const void *biases,
                        nq_dtype sb_dt, int64_t n, int64_t k, int32_t group_size, int32_t bits,
                        void *w_out, nq_dtype out_dt, hipStream_t stream)
{
    const char *op = "nq_dequantize";
    g_last_error.clear();
    if (!dtype_ok(sb_dt) || !dtype_ok(out_dt))
        return fail(NQ_ERR_DTYPE, "%s: unknown dtype (sb_dt=%d, out_dt=%d)", op, (int)sb_dt,
                    (int)out_dt);
    nq_status st = check_quant(op, group_size, bits, false);
    if (st) return st;
    if ((st = check_dims(op, n, k, group_size))) return st;
    if (n == 0 || k == 0) return NQ_OK;
    if (!w_out || !codes || !scales || !biases)
        return fail(NQ_ERR_NULL, "%s: codes, scales, biases and w_out must be non-null", op);
    if (!aligned16(w_out) || !aligned16(codes))
        return fail(NQ_ERR_ALIGN, "%s: codes and w_out must be 16-byte aligned", op);
    const int64_t sbb = dtype_bytes(sb_dt);
    if (!aligned_to(scales, sbb) || !aligned_to(biases, sbb))
        return fail(NQ_ERR_ALIGN, "%s: scales and biases must be aligned to %lld bytes", op,
                    (long long)sbb);
    const Span so{w_out, n * k * dtype_bytes(out_dt)};
    if (overlap(so, Span{codes, n * (k * bits / 32) * 4}) ||
        overlap(so, Span{scales, n * (k / group_size) * sbb}) ||
        overlap(so, Span{biases, n * (k / group_size) * sbb}))
        return fail(NQ_ERR_ALIAS, "%s: w_out overlaps an input", op);
    return check_launch(op, nqk::launch_dequantize(codes, scales, biases, sb_dt, n, k, group_size,
                                                   bits, w_out, out_dt, stream));
}

nq_status nq_qmm_plan(int64_t m, int64_t n, int64_t k, int32_t group_size, int32_t bits,
                      nq_dtype x_dt, nq_dtype sb_dt, int32_t row_exact, nq_plan *plan)
{
    const char *op = "nq_qmm_plan";
    g_last_error.clear();
    if (!plan) return fail(NQ_ERR_NULL, "%s: plan is null", op);
    if (!dtype_ok(x_dt) || !dtype_ok(sb_dt))
        return fail(NQ_ERR_DTYPE, "%s: unknown dtype (x_dt=%d, sb_dt=%d)", op, (int)x_dt, (int)sb_dt);
    nq_status st = check_quant(op, group_size, bits, true);
    if (st) return st;
    if (m < 0) return fail(NQ_ERR_SHAPE, "%s: negative m=%lld", op, (long long)m);
    if ((st = check_dims(op, n, k, group_size))) return st;
    return make_plan(op, m, n, k, group_size, bits, x_dt, sb_dt, row_exact, plan);
}

size_t nq_qmm_workspace_bytes(int64_t m, int64_t n, int64_t k, int32_t group_size, int32_t bits,
                              nq_dtype x_dt, nq_dtype sb_dt, int32_t row_exact)
{
    (void)m, (void)n, (void)k, (void)group_size, (void)bits, (void)x_dt, (void)sb_dt, (void)row_exact;
    return 0;
}

nq_status nq_qmm(const void *x, nq_dtype x_dt, int64_t m, int64_t k, const uint32_t *codes,
                 const void *scales, const void *biases, nq_dtype sb_dt, int64_t n,
                 int32_t group_size, int32_t bits, void *y, void *workspace,
                 size_t workspace_bytes, hipStream_t stream)
{
    const QmmArgs a{x, x_dt, m, k, codes, scales, biases, sb_dt, n, group_size, bits, y,
                    workspace, workspace_bytes};
    return qmm_common("nq_qmm", 0, nullptr, a, stream);
}

nq_status nq_qmm_row_exact(const void *x, nq_dtype x_dt, int64_t m, int64_t k,
                           const uint32_t *codes, const void *scales, const void *biases,
                           nq_dtype sb_dt, int64_t n, int32_t group_size, int32_t bits, void *y,
                           void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    const QmmArgs a{x, x_dt, m, k, codes, scales, biases, sb_dt, n, group_size, bits, y,
                    workspace, workspace_bytes};
    return qmm_common("nq_qmm_row_exact", 1, nullptr, a, stream);
}

nq_status nq_qmm_with_plan(const nq_plan *plan, const void *x, nq_dtype x_dt, int64_t m,
                           int64_t k, const uint32_t *codes, const void *scales,
                           const void *biases, nq_dtype sb_dt, int64_t n, int32_t group_size,
                           int32_t bits, void *y, void *workspace, size_t workspace_bytes,
                           hipStream_t stream)
{
    if (!plan) {
        g_last_error.clear();
        return fail(NQ_ERR_NULL, "nq_qmm_with_plan: plan is null");
    }
    const QmmArgs a{x, x_dt, m, k, codes, scales, biases, sb_dt, n, group_size, bits, y,
                    workspace, workspace_bytes};
    return qmm_common("nq_qmm_with_plan", 0, plan, a, stream);
}

// Batch items keep their solo bits (nuvec API index, section "Determinism":
// batch items of quantized products).  The route is the plan of one item; every
// kernel's arithmetic for an output element depends only on its own row of
// x and its weight row, so running that plan over all items at once gives
// each item the bits of the call on it alone.  Only the launch is cut where
// the 256-row tiles' 32-bit offsets would overflow.
nq_status nq_qmm_batched(const void *x, nq_dtype x_dt, int64_t batch, int64_t l, int64_t k,
                         const uint32_t *codes, const void *scales, const void *biases,
                         nq_dtype sb_dt, int64_t n, int32_t group_size, int32_t bits, void *y,
                         void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    const char *op = "nq_qmm_batched";
    g_last_error.clear();
    if (batch < 0 || l < 0)
        return fail(NQ_ERR_SHAPE, "%s: negative size (batch=%lld, l=%lld)", op, (long long)batch,
                    (long long)l);
    if (batch >= kMaxDim || l >= kMaxDim || (batch > 0 && l > kMaxDim / batch))
        return fail(NQ_ERR_SHAPE, "%s: batch*l is too large", op);
    const QmmArgs a{x, x_dt, batch * l, k, codes, scales, biases, sb_dt, n, group_size, bits, y,
                    workspace, workspace_bytes};
    bool empty = false;
    nq_status st = check_qmm(op, a, &empty);
    if (st || empty) return st;
    nq_plan plan;
    make_plan(op, l, n, k, group_size, bits, x_dt, sb_dt, 0, &plan);
    int64_t per_launch = batch;   // items per launch
    const int64_t xb = dtype_bytes(x_dt);
    if (plan.route == NQ_ROUTE_TILED &&
        !nqk::tiled_fits(plan.tile_m, plan.tile_n, bits, group_size, sb_dt, batch * l, n, k)) {
        while (per_launch > 1 && !nqk::tiled_fits(plan.tile_m, plan.tile_n, bits, group_size, sb_dt,
                                                   per_launch * l, n, k))
            per_launch = (per_launch + 1) / 2;
        // every launch's y starts 16-byte aligned
        int64_t unit = 1;
        while ((unit * l * n * xb) % 16) unit *= 2;
        if (per_launch < unit)
            return fail(NQ_ERR_SHAPE, "%s: items of l=%lld rows are too large to batch", op, (long long)l);
        per_launch -= per_launch % unit;
    }
    for (int64_t i0 = 0; i0 < batch; i0 += per_launch) {
        QmmArgs part = a;
        part.m = std::min(per_launch, batch - i0) * l;
        part.x = static_cast<const char *>(x) + i0 * l * k * xb;
        part.y = static_cast<char *>(y) + i0 * l * n * xb;
        if ((st = run_qmm(op, plan, part, stream))) return st;
    }
    return NQ_OK;
}

namespace {
// Gather routes ("Mixture of experts" section).  Once experts are shared by
// several vectors (at least 16 vectors, 4 per expert on average) the
// vectors are grouped by expert on the device and each expert's weights are
// read once per chunk: by the matrix-core kernel (bf16 x, K a multiple of
// 64; rows within the product tolerance), or in row-exact mode by the
// matrix-vector family, whose rows never depend on how many rows share a
// chunk.  Otherwise every row runs as its own matrix-vector product.  Pure
// functions of the sizes, dtypes and mode.
bool gather_shared(int64_t rows, int64_t l, int64_t k, int64_t e, int64_t n)
{
    const int64_t v = rows * l;
    return k > 0 && n > 0 && rows > 0 && l > 0 && e > 0 && e <= 4096 && v >= 16 && v >= 4 * e &&
           v < ((int64_t)1 << 31) && nqk::gather_group_max_chunks(v, e, nqk::kGroupChunk) <= 65535;
}

bool gather_mfma(int64_t rows, int64_t l, int64_t k, int64_t e, int64_t n, int x_dt, int bits,
                 int row_exact)
{
    return !row_exact && x_dt == NQ_BF16 && (bits == 4 || bits == 8) && k % 64 == 0 &&
           gather_shared(rows, l, k, e, n);
}

nq_status gather_impl(const char *op, int row_exact, const void *x, nq_dtype x_dt, int64_t rows,
                      int64_t l, int64_t k, const uint32_t *codes, const void *scales,
                      const void *biases, nq_dtype sb_dt, int64_t e, int64_t n, int32_t group_size,
                      int32_t bits, const uint32_t *lhs_idx, int64_t x_items, const uint32_t *rhs_idx,
                      void *y, void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    // lhs_idx null: output row r reads x item r (x has rows items)
    g_last_error.clear();
    if (!dtype_ok(x_dt) || !dtype_ok(sb_dt))
        return fail(NQ_ERR_DTYPE, "%s: unknown dtype (x_dt=%d, sb_dt=%d)", op, (int)x_dt, (int)sb_dt);
    nq_status st = check_quant(op, group_size, bits, true);
    if (st) return st;
    if (rows < 0 || l < 0 || e < 0)
        return fail(NQ_ERR_SHAPE, "%s: negative size (rows=%lld, l=%lld, e=%lld)", op,
                    (long long)rows, (long long)l, (long long)e);
    if ((st = check_dims(op, n, k, group_size))) return st;
    if (e >= kMaxDim || (e > 0 && n > kMaxElems / std::max<int64_t>(e, 1) / std::max<int64_t>(k, 1)))
        return fail(NQ_ERR_SHAPE, "%s: e=%lld is too large", op, (long long)e);
    if (rows >= kMaxDim || l >= kMaxDim || (rows > 0 && l > kMaxElems / rows) ||
        (rows * l > 0 && std::max<int64_t>(k, n) > kMaxElems / (rows * l)))
        return fail(NQ_ERR_SHAPE, "%s: rows*l is too large", op);
    if (lhs_idx && (x_items < 1 || x_items >= kMaxDim ||
                    (k > 0 && x_items > kMaxElems / std::max<int64_t>(l, 1) / k)))
        return fail(NQ_ERR_SHAPE, "%s: x_items=%lld must be positive and not too large", op,
                    (long long)x_items);
    if (!lhs_idx) x_items = rows;
    if (rows == 0 || l == 0 || n == 0) return NQ_OK;
    if (!y || !rhs_idx) return fail(NQ_ERR_NULL, "%s: y and rhs_idx must be non-null", op);
    if (k > 0 && (!x || (e > 0 && (!codes || !scales || !biases))))
        return fail(NQ_ERR_NULL, "%s: x, codes, scales and biases must be non-null", op);
    if (!aligned16(x) || !aligned16(codes) || !aligned16(y))
        return fail(NQ_ERR_ALIGN, "%s: x, codes and y must be 16-byte aligned", op);
    const int64_t sbb = dtype_bytes(sb_dt);
    if (!aligned_to(scales, sbb) || !aligned_to(biases, sbb) || !aligned_to(rhs_idx, 4) ||
        !aligned_to(lhs_idx, 4))
        return fail(NQ_ERR_ALIGN, "%s: scales, biases, rhs_idx or lhs_idx misaligned", op);
    const Span sy{y, rows * l * n * dtype_bytes(x_dt)};
    const Span ins[6] = {{x, x_items * l * k * dtype_bytes(x_dt)},
                         {codes, e * n * (k * bits / 32) * 4},
                         {scales, e * n * (k / group_size) * sbb},
                         {biases, e * n * (k / group_size) * sbb},
                         {rhs_idx, rows * 4},
                         {lhs_idx, lhs_idx ? rows * 4 : 0}};
    static const char *names[6] = {"x", "codes", "scales", "biases", "rhs_idx", "lhs_idx"};
    for (int i = 0; i < 6; ++i)
        if (overlap(sy, ins[i])) return fail(NQ_ERR_ALIAS, "%s: y overlaps %s", op, names[i]);

    const bool shared = gather_shared(rows, l, k, e, n);
    const bool mfma = gather_mfma(rows, l, k, e, n, x_dt, bits, row_exact);
    const int64_t v = rows * l;
    if (shared) {
        const size_t need = nqk::gather_group_ws_bytes(v, e, nqk::kGroupChunk);
        if (!workspace || workspace_bytes < need)
            return fail(NQ_ERR_WORKSPACE, "%s: the grouped route needs a workspace of %zu bytes (got %zu)",
                        op, need, workspace ? workspace_bytes : (size_t)0);
        if (!aligned16(workspace)) return fail(NQ_ERR_ALIGN, "%s: workspace must be 16-byte aligned", op);
        const Span sw{workspace, (int64_t)need};
        if (overlap(sw, sy)) return fail(NQ_ERR_ALIAS, "%s: workspace overlaps y", op);
        for (int i = 0; i < 6; ++i)
            if (overlap(sw, ins[i])) return fail(NQ_ERR_ALIAS, "%s: workspace overlaps %s", op, names[i]);
    }
    uint32_t *ws = static_cast<uint32_t *>(workspace);
    // chunks of 32 vectors for the matrix cores (either route), of 8 for the
    // VALU matrix-vector kernels
    const bool gemv_cores = nqk::gemv_mfma_family(n, k, group_size, bits, x_dt);
    const int chunk = (mfma || gemv_cores) ? nqk::kGroupChunkMfma : nqk::kGroupChunk;
    // the matrix-core route groups small id sets inside its own workgroups
    const bool self_group = mfma && nqk::gather_self_group_fits(v, e);
    if (shared && !self_group) {
        if (hipError_t err = nqk::launch_gather_groups(rhs_idx, lhs_idx, x_items, rows, l, e, chunk, workspace,
                                                       stream))
            return check_launch(op, err);
    }
    if (mfma) {
        nqk::GatherMfmaLaunch g;
        g.x = x;
        g.y = y;
        g.codes = codes;
        g.scales = scales;
        g.biases = biases;
        g.perm = ws;
        g.nchunks = ws + v;
        g.chunks = ws + ((v + 1 + 3) & ~(int64_t)3);
        g.ids = rhs_idx;
        g.lhs = lhs_idx;
        g.x_items = x_items;
        g.sb_dt = sb_dt;
        g.n = n;
        g.k = k;
        g.e = e;
        g.max_chunks = nqk::gather_group_max_chunks(v, e, chunk);
        g.l = l;
        g.v_total = v;
        g.gs = group_size;
        g.bits = bits;
        g.self_group = self_group;
        return check_launch(op, nqk::launch_gather_mfma(g, stream));
    }

    nqk::GemvLaunch g;
    g.x = x;
    g.y = y;
    g.codes = codes;
    g.scales = scales;
    g.biases = biases;
    g.idx = rhs_idx;
    g.x_dt = x_dt;
    g.sb_dt = sb_dt;
    g.items = rows;
    g.rows_per_item = l;
    g.k = k;
    g.n = n;
    g.e = e;
    g.gs = group_size;
    g.bits = bits;
    g.ksplit = gemv_ksplit(n, k, group_size, bits, x_dt);   // the plan nq_qmm_row_exact takes
    g.rows_per_wave = 0;
    g.lhs = lhs_idx;
    g.x_items = x_items;
    g.lhs_l = l;
    if (shared) {
        g.idx = nullptr;
        g.perm = ws;
        g.nchunks = ws + v;
        g.chunks = ws + ((v + 1 + 3) & ~(int64_t)3);
        g.max_chunks = nqk::gather_group_max_chunks(v, e, chunk);
        g.items = 1;
        g.rows_per_item = chunk;   // chunks of up to `chunk` vectors
        g.max_rows = chunk;
    }
    return check_launch(op, nqk::launch_gemv(g, stream));
}
}  // namespace

size_t nq_gather_qmm_workspace_bytes(int64_t rows, int64_t l, int64_t k, int64_t e, int64_t n,
                                     int32_t group_size, int32_t bits, nq_dtype x_dt,
                                     nq_dtype sb_dt, int32_t sorted_hint)
{
    (void)group_size, (void)bits, (void)x_dt, (void)sb_dt, (void)sorted_hint;
    if (rows < 0 || l < 0 || e < 0 || k < 0 || n < 0) return 0;
    if (!gather_shared(rows, l, k, e, n)) return 0;
    // enough for either grouped route (the matrix-vector one has more chunks)
    return nqk::gather_group_ws_bytes(rows * l, e, nqk::kGroupChunk);
}

nq_status nq_gather_qmm(const void *x, nq_dtype x_dt, int64_t rows, int64_t l, int64_t k,
                        const uint32_t *codes, const void *scales, const void *biases,
                        nq_dtype sb_dt, int64_t e, int64_t n, int32_t group_size, int32_t bits,
                        const uint32_t *rhs_idx, int32_t sorted_hint, void *y, void *workspace,
                        size_t workspace_bytes, hipStream_t stream)
{
    (void)sorted_hint;
    return gather_impl("nq_gather_qmm", 0, x, x_dt, rows, l, k, codes, scales, biases, sb_dt, e, n,
                       group_size, bits, nullptr, rows, rhs_idx, y, workspace, workspace_bytes, stream);
}

// ---- the gather for callers that cannot allocate

// The grouping tables of nq_gather_qmm_noalloc: one array per GPU, in the
// library's own device memory.  Host code never passes the array's name to
// a kernel or a copy (on the host it is only a stand-in for the device
// address); the address of each GPU's copy is taken once, with that GPU
// current, and kept.
static __device__ __align__(256) uint8_t scratch[NQ_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kScratchDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kScratchDevices];   // device address of `scratch`, per GPU

// The current GPU's copy of `scratch` (its address taken on first use).
nq_status scratch_of_current_device(const char *op, void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices)
        return fail(NQ_ERR_LAUNCH, "%s: no usable current device (%d)", op, dev);
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        const hipError_t err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (err != hipSuccess || !ptr)
            return fail(NQ_ERR_LAUNCH, "%s: hipGetSymbolAddress of the scratch array failed on device %d: %s",
                        op, dev, hipGetErrorString(err));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return NQ_OK;
}

}  // namespace

nq_status nq_gather_qmm_noalloc(const void *x, nq_dtype x_dt, int64_t rows, int64_t l, int64_t k,
                                const uint32_t *codes, const void *scales, const void *biases,
                                nq_dtype sb_dt, int64_t e, int64_t n, int32_t group_size, int32_t bits,
                                const uint32_t *rhs_idx, int32_t sorted_hint, void *y, hipStream_t stream)
{
    const char *op = "nq_gather_qmm_noalloc";
    g_last_error.clear();
    const size_t need = nq_gather_qmm_workspace_bytes(rows, l, k, e, n, group_size, bits, x_dt, sb_dt,
                                                      sorted_hint);
    if (need > NQ_NOALLOC_SCRATCH_BYTES)
        return fail(NQ_ERR_WORKSPACE,
                    "%s: the grouping tables of %lld x %lld vectors and %lld experts need %zu bytes, above "
                    "the %u-byte static scratch",
                    op, (long long)rows, (long long)l, (long long)e, need, (unsigned)NQ_NOALLOC_SCRATCH_BYTES);
    void *ws = nullptr;
    if (need) {
        // the grouping pass rewrites every table entry a later kernel reads,
        // so nothing in the array has to start at zero
        if (nq_status st = scratch_of_current_device(op, &ws)) return st;
    }
    return gather_impl(op, 0, x, x_dt, rows, l, k, codes, scales, biases, sb_dt, e, n, group_size, bits,
                       nullptr, rows, rhs_idx, y, ws, need ? (size_t)NQ_NOALLOC_SCRATCH_BYTES : 0, stream);
}

nq_status nq_gather_qmm_row_exact(const void *x, nq_dtype x_dt, int64_t rows, int64_t l, int64_t k,
                                  const uint32_t *codes, const void *scales, const void *biases,
                                  nq_dtype sb_dt, int64_t e, int64_t n, int32_t group_size,
                                  int32_t bits, const uint32_t *rhs_idx, int32_t sorted_hint,
                                  void *y, void *workspace, size_t workspace_bytes,
                                  hipStream_t stream)
{
    (void)sorted_hint;
    return gather_impl("nq_gather_qmm_row_exact", 1, x, x_dt, rows, l, k, codes, scales, biases,
                       sb_dt, e, n, group_size, bits, nullptr, rows, rhs_idx, y, workspace, workspace_bytes,
                       stream);
}

nq_status nq_gather_qmm_lhs(const void *x, nq_dtype x_dt, int64_t x_items, int64_t rows, int64_t l,
                            int64_t k, const uint32_t *codes, const void *scales, const void *biases,
                            nq_dtype sb_dt, int64_t e, int64_t n, int32_t group_size, int32_t bits,
                            const uint32_t *lhs_idx, const uint32_t *rhs_idx, int32_t sorted_hint,
                            int32_t row_exact, void *y, void *workspace, size_t workspace_bytes,
                            hipStream_t stream)
{
    (void)sorted_hint;
    const char *op = "nq_gather_qmm_lhs";
    if (!lhs_idx && rows > 0 && l > 0 && n > 0) {
        g_last_error.clear();
        return fail(NQ_ERR_NULL, "%s: lhs_idx must be non-null (nq_gather_qmm takes none)", op);
    }
    return gather_impl(op, row_exact ? 1 : 0, x, x_dt, rows, l, k, codes, scales, biases, sb_dt, e, n,
                       group_size, bits, lhs_idx, x_items, rhs_idx, y, workspace, workspace_bytes, stream);
}

nq_status nq_fp_quantize(const void *w, nq_dtype w_dt, int64_t n, int64_t k, int32_t mode,
                         uint32_t *codes, uint8_t *scales, hipStream_t stream)
{
    const char *op = "nq_fp_quantize";
    g_last_error.clear();
    if (!dtype_ok(w_dt)) return fail(NQ_ERR_DTYPE, "%s: unknown dtype w_dt=%d", op, (int)w_dt);
    nq_status st = check_fp(op, mode, n, k);
    if (st) return st;
    if (n == 0 || k == 0) return NQ_OK;
    if (!w || !codes || !scales) return fail(NQ_ERR_NULL, "%s: w, codes and scales must be non-null", op);
    if (!aligned16(w) || !aligned16(codes))
        return fail(NQ_ERR_ALIGN, "%s: w and codes must be 16-byte aligned", op);
    const Span sw{w, n * k * dtype_bytes(w_dt)}, sc{codes, fp_code_bytes(mode, n, k)},
        ss{scales, fp_scale_bytes(mode, n, k)};
    if (overlap(sc, sw) || overlap(ss, sw)) return fail(NQ_ERR_ALIAS, "%s: an output overlaps w", op);
    if (overlap(sc, ss)) return fail(NQ_ERR_ALIAS, "%s: codes and scales overlap", op);
    return check_launch(op, nqk::launch_fp_quantize(w, w_dt, n, k, mode, codes, scales, stream));
}

nq_status nq_fp_dequantize(const uint32_t *codes, const uint8_t *scales, int64_t n, int64_t k,
                           int32_t mode, void *w_out, nq_dtype out_dt, hipStream_t stream)
{
    const char *op = "nq_fp_dequantize";
    g_last_error.clear();
    if (!dtype_ok(out_dt)) return fail(NQ_ERR_DTYPE, "%s: unknown dtype out_dt=%d", op, (int)out_dt);
    nq_status st = check_fp(op, mode, n, k);
    if (st) return st;
    if (n == 0 || k == 0) return NQ_OK;
    if (!codes || !scales || !w_out)
        return fail(NQ_ERR_NULL, "%s: codes, scales and w_out must be non-null", op);
    if (!aligned16(codes) || !aligned16(w_out))
        return fail(NQ_ERR_ALIGN, "%s: codes and w_out must be 16-byte aligned", op);
    const Span so{w_out, n * k * dtype_bytes(out_dt)};
    if (overlap(so, Span{codes, fp_code_bytes(mode, n, k)}) || overlap(so, Span{scales, fp_scale_bytes(mode, n, k)}))
        return fail(NQ_ERR_ALIAS, "%s: w_out overlaps an input", op);
    return check_launch(op, nqk::launch_fp_dequantize(codes, scales, n, k, mode, w_out, out_dt, stream));
}

static nq_status fp_qmm_impl(const char *op, const void *x, nq_dtype x_dt, int64_t items, int64_t vpi,
                             int64_t k, const uint32_t *codes, const uint8_t *scales, const float *gscale,
                             int64_t e, int64_t n, int32_t mode, const uint32_t *idx, int32_t row_exact,
                             void *y, void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    g_last_error.clear();
    if (!dtype_ok(x_dt)) return fail(NQ_ERR_DTYPE, "%s: unknown dtype x_dt=%d", op, (int)x_dt);
    nq_status st = check_fp(op, mode, n, k);
    if (st) return st;
    if ((st = check_global_scale(op, mode, gscale))) return st;
    if (items < 0 || vpi < 0 || e < 1)
        return fail(NQ_ERR_SHAPE, "%s: bad sizes (rows=%lld, l=%lld, e=%lld)", op, (long long)items,
                    (long long)vpi, (long long)e);
    if (items >= kMaxDim || vpi >= kMaxDim || (vpi > 0 && items > kMaxDim / vpi) || e > 65536 ||
        (k > 0 && items * vpi > kMaxElems / std::max<int64_t>(k, n)) || e * n >= kMaxDim)
        return fail(NQ_ERR_SHAPE, "%s: size too large", op);
    if (items == 0 || vpi == 0 || n == 0) return NQ_OK;
    if (!y || (idx == nullptr && e != 1) || (k > 0 && (!x || !codes || !scales)))
        return fail(NQ_ERR_NULL, "%s: x, codes, scales, y (and rhs_idx) must be non-null", op);
    if (!aligned16(x) || !aligned16(codes) || !aligned16(y))
        return fail(NQ_ERR_ALIGN, "%s: x, codes and y must be 16-byte aligned", op);
    if (idx && !aligned_to(idx, 4)) return fail(NQ_ERR_ALIGN, "%s: rhs_idx must be 4-byte aligned", op);
    const int64_t xb = dtype_bytes(x_dt);
    const Span sy{y, items * vpi * n * xb};
    if (overlap(sy, Span{x, items * vpi * k * xb}) || overlap(sy, Span{codes, e * fp_code_bytes(mode, n, k)}) ||
        overlap(sy, Span{scales, e * fp_scale_bytes(mode, n, k)}) ||
        overlap(sy, Span{gscale, gscale ? (idx ? e : 1) * 4 : 0}) || overlap(sy, Span{idx, idx ? items * 4 : 0}))
        return fail(NQ_ERR_ALIAS, "%s: y overlaps an input", op);
    // gathered rows that share experts are grouped on the device, so that
    // each expert's weights are read once per chunk of vectors
    const bool grouped = idx && gather_shared(items, vpi, k, e, n);
    if (grouped) {
        const size_t need = nqk::gather_group_ws_bytes(items * vpi, e, nqk::kGroupChunk);
        if (!workspace || workspace_bytes < need)
            return fail(NQ_ERR_WORKSPACE, "%s: workspace of %zu bytes needed (got %zu)", op, need,
                        workspace ? workspace_bytes : (size_t)0);
        if (!aligned16(workspace)) return fail(NQ_ERR_ALIGN, "%s: workspace must be 16-byte aligned", op);
        const Span sw{workspace, (int64_t)need};
        if (overlap(sw, sy) || overlap(sw, Span{x, items * vpi * k * xb}) ||
            overlap(sw, Span{codes, e * fp_code_bytes(mode, n, k)}) ||
            overlap(sw, Span{scales, e * fp_scale_bytes(mode, n, k)}) || overlap(sw, Span{idx, items * 4}))
            return fail(NQ_ERR_ALIAS, "%s: the workspace overlaps an argument", op);
    }
    nqk::FpQmmLaunch a;
    a.x = x, a.y = y, a.codes = codes, a.scales = scales, a.gscale = gscale, a.idx = idx;
    a.x_dt = x_dt, a.mode = mode;
    a.items = items, a.vpi = vpi, a.n = n, a.k = k, a.e = e;
    a.tiled = idx == nullptr && !row_exact && vpi > NQ_ROW_INDEPENDENT_ROWS && x_dt == NQ_BF16 && k % 64 == 0 &&
              vpi <= (int64_t)65535 * 128;   // row tiles along grid.y
    if (grouped) {
        // matrix cores unless every row must keep its one-row bits
        a.mfma = !row_exact && x_dt == NQ_BF16 && k % 64 == 0;
        const int chunk = a.mfma ? nqk::kGroupChunkMfma : nqk::kGroupChunk;
        hipError_t err = nqk::launch_gather_groups(idx, nullptr, items, items, vpi, e, chunk, workspace, stream);
        if (err != hipSuccess) return check_launch(op, err);
        const int64_t v = items * vpi;
        uint32_t *ws = static_cast<uint32_t *>(workspace);
        a.perm = ws, a.nchunks = ws + v;
        a.chunks = reinterpret_cast<const uint4 *>(ws + ((v + 1 + 3) & ~(int64_t)3));
        a.max_chunks = nqk::gather_group_max_chunks(v, e, chunk);
    }
    return check_launch(op, nqk::launch_fp_qmm(a, stream));
}

nq_status nq_fp_qmm(const void *x, nq_dtype x_dt, int64_t m, int64_t k, const uint32_t *codes,
                    const uint8_t *scales, const float *global_scale, int64_t n, int32_t mode,
                    int32_t row_exact, void *y, hipStream_t stream)
{
    if (m < 0) {
        g_last_error.clear();
        return fail(NQ_ERR_SHAPE, "nq_fp_qmm: negative m=%lld", (long long)m);
    }
    return fp_qmm_impl("nq_fp_qmm", x, x_dt, 1, m, k, codes, scales, global_scale, 1, n, mode, nullptr,
                       row_exact, y, nullptr, 0, stream);
}

size_t nq_fp_gather_qmm_workspace_bytes(int64_t rows, int64_t l, int64_t k, int64_t e, int64_t n)
{
    if (rows < 0 || l < 0 || e < 0 || k < 0 || n < 0 || !gather_shared(rows, l, k, e, n)) return 0;
    return nqk::gather_group_ws_bytes(rows * l, e, nqk::kGroupChunk);
}

nq_status nq_fp_gather_qmm(const void *x, nq_dtype x_dt, int64_t rows, int64_t l, int64_t k,
                           const uint32_t *codes, const uint8_t *scales, const float *global_scales,
                           int64_t e, int64_t n, int32_t mode, const uint32_t *rhs_idx, int32_t row_exact,
                           void *y, void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (!rhs_idx && rows > 0 && l > 0 && n > 0) {
        g_last_error.clear();
        return fail(NQ_ERR_NULL, "nq_fp_gather_qmm: rhs_idx must be non-null");
    }
    return fp_qmm_impl("nq_fp_gather_qmm", x, x_dt, rows, l, k, codes, scales, global_scales, e, n, mode,
                       rhs_idx, row_exact, y, workspace, workspace_bytes, stream);
}

size_t nq_fp_qmm_notrans_workspace_bytes(int64_t m, int64_t ni, int64_t nc, int32_t mode, nq_dtype x_dt,
                                         int32_t row_exact)
{
    (void)mode;
    if (m <= 0 || ni < 0 || nc <= 0 || nc % 32 != 0) return 0;
    if (!row_exact && m > NQ_ROW_INDEPENDENT_ROWS && x_dt == NQ_BF16 && ni % 64 == 0) return 0;   // tiles
    return nqk::fp_nt_ws_bytes(ni, nc);
}

nq_status nq_fp_qmm_notrans(const void *x, nq_dtype x_dt, int64_t m, int64_t ni, const uint32_t *codes,
                            const uint8_t *scales, const float *global_scale, int64_t nc, int32_t mode,
                            int32_t row_exact, void *y, void *workspace, size_t workspace_bytes,
                            hipStream_t stream)
{
    const char *op = "nq_fp_qmm_notrans";
    g_last_error.clear();
    if (!dtype_ok(x_dt)) return fail(NQ_ERR_DTYPE, "%s: unknown dtype x_dt=%d", op, (int)x_dt);
    nq_status st = check_fp(op, mode, ni, nc);   // nc (the grouped axis) a multiple of 32
    if (st) return st;
    if ((st = check_global_scale(op, mode, global_scale))) return st;
    if (m < 0) return fail(NQ_ERR_SHAPE, "%s: negative m=%lld", op, (long long)m);
    if (m >= kMaxDim || (ni > 0 && m > kMaxElems / ni) || (nc > 0 && m > kMaxElems / nc))
        return fail(NQ_ERR_SHAPE, "%s: m=%lld is too large", op, (long long)m);
    if (m == 0 || nc == 0) return NQ_OK;
    if (!y || (ni > 0 && (!x || !codes || !scales)))
        return fail(NQ_ERR_NULL, "%s: x, codes, scales and y must be non-null", op);
    if (!aligned16(x) || !aligned16(codes) || !aligned16(y))
        return fail(NQ_ERR_ALIGN, "%s: x, codes and y must be 16-byte aligned", op);
    const int64_t xb = dtype_bytes(x_dt);
    const Span sy{y, m * nc * xb};
    if (overlap(sy, Span{x, m * ni * xb}) || overlap(sy, Span{codes, fp_code_bytes(mode, ni, nc)}) ||
        overlap(sy, Span{scales, fp_scale_bytes(mode, ni, nc)}) || overlap(sy, Span{global_scale, global_scale ? 4 : 0}))
        return fail(NQ_ERR_ALIAS, "%s: y overlaps an input", op);
    nqk::FpNtLaunch a;
    a.x = x, a.y = y, a.codes = codes, a.scales = scales, a.gscale = global_scale, a.workspace = workspace;
    a.x_dt = x_dt, a.mode = mode, a.m = m, a.ni = ni, a.nc = nc;
    a.tiled = !row_exact && m > NQ_ROW_INDEPENDENT_ROWS && x_dt == NQ_BF16 && ni % 64 == 0;
    if (!a.tiled) {
        const size_t need = nqk::fp_nt_ws_bytes(ni, nc);
        if (!workspace || workspace_bytes < need)
            return fail(NQ_ERR_WORKSPACE, "%s: workspace of %zu bytes needed (got %zu)", op, need,
                        workspace ? workspace_bytes : (size_t)0);
        if (!aligned16(workspace)) return fail(NQ_ERR_ALIGN, "%s: workspace must be 16-byte aligned", op);
        const Span sw{workspace, (int64_t)need};
        if (overlap(sw, sy) || overlap(sw, Span{x, m * ni * xb}) ||
            overlap(sw, Span{codes, fp_code_bytes(mode, ni, nc)}) || overlap(sw, Span{scales, fp_scale_bytes(mode, ni, nc)}))
            return fail(NQ_ERR_ALIAS, "%s: the workspace overlaps an argument", op);
    }
    return check_launch(op, nqk::launch_fp_qmm_nt(a, stream));
}

const char *nq_status_string(nq_status s)
{
    switch (s) {
    case NQ_OK: return "ok";
    case NQ_ERR_NULL: return "null pointer";
    case NQ_ERR_DTYPE: return "unsupported dtype";
    case NQ_ERR_QUANT: return "unsupported group size or bit width";
    case NQ_ERR_SHAPE: return "invalid shape";
    case NQ_ERR_ALIGN: return "misaligned pointer";
    case NQ_ERR_ALIAS: return "output overlaps an input";
    case NQ_ERR_WORKSPACE: return "workspace missing or too small";
    case NQ_ERR_LAUNCH: return "kernel launch failed";
    case NQ_ERR_PLAN: return "plan does not fit";
    }
    return "unknown status";
}

const char *nq_last_error(void) { return g_last_error.c_str(); }

const char *nq_version(void) { return "0.1.0"; }

}  // extern "C"
