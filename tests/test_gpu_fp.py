"""GPU parity of the floating-point modes (MXFP4, MXFP8, NVFP4) against the
CPU oracle (oracle/fp.py): quantize and dequantize bit for bit, products
within the affine products' tolerance, every element code exactly through
both product kernels, row independence, gathered products with global
scales, and the decode and prefill workload sizes."""
import numpy as np
import pytest
import torch

from gpu_helpers import assert_rows_close, bits_equal, dev, host, tolerance, values
from group_wise_affine_quantize_amd import _binding as B
from group_wise_affine_quantize_amd import synthetic
from oracle import fp as F

pytestmark = pytest.mark.gpu

MODES = ["mxfp4", "mxfp8", "nvfp4"]
# scale codes of moderate magnitude: E8M0 2^-7 .. 2^7, E4M3 0.125 .. 8
SCALES = {"mxfp4": (120, 134), "mxfp8": (120, 134), "nvfp4": (0x20, 0x50)}


def u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def codes_case(seed, lead, k, mode, finite=True):
    _, bits, gs, _ = F.mode_info(mode)
    return synthetic.random_fp_matrix(seed, lead, k, bits, gs, SCALES[mode], finite_bytes=finite)


# ---------------------------------------------------------------- storage ops
def _quantize_inputs(seed, n, k, dtype):
    rng = np.random.default_rng(seed)
    w = synthetic.normal(rng, (n, k), 1.0) * np.exp(rng.uniform(-6, 6, (n, 1))).astype(np.float32)
    # edge blocks: all zeros, minus zeros, tiny values, exact element values
    # at a fixed scale (ties after scaling), a huge value
    w[0, :32] = 0.0
    w[1, :32] = -0.0
    w[2, :32] = np.float32(1e-41)
    w[3, :32] = np.float32(np.ldexp(np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0] * 4), -3))
    w[4, :32] = np.float32(3e38) * np.sign(w[4, :32])
    w[5, 32:64] = np.float32(np.ldexp(np.arange(32) / 16.0, -130))
    if dtype == "bf16":
        return synthetic.to_bf16_bits(w)
    return w


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quantize_bit_exact(mode, dtype):
    w = _quantize_inputs(21, 37, 320, dtype)
    cq, sq = F.quantize(w, mode)
    c, s = B.nq_fp_quantize(dev(w), mode)
    assert np.array_equal(host(c), cq), mode
    assert np.array_equal(s.cpu().numpy(), sq), mode


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_dequantize_every_code_bit_exact(mode, out):
    # uniformly random words and every scale code, NaN ones included
    _, bits, gs, _ = F.mode_info(mode)
    words, _ = synthetic.random_fp_matrix(5, (64,), 512, bits, gs, (0, 255))
    scales = np.arange(64 * 512 // gs, dtype=np.int64).reshape(64, -1) % 256
    ref = F.dequantize(words, scales.astype(np.uint8), mode, 512, out)
    got = host(B.nq_fp_dequantize(dev(words), u8(scales), mode,
                                  out_dtype=torch.bfloat16 if out == "bf16" else torch.float32))
    if out == "bf16":
        assert np.array_equal(got, ref)
    else:
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


# ---------------------------------------------------------------- products
def _one_hot(k, dtype):
    x = np.eye(k, dtype=np.float32)
    return synthetic.to_bf16_bits(x) if dtype == "bf16" else x


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("route", ["gemv_f32", "gemv_bf16", "tiled"])
def test_products_pick_every_element_exactly(mode, route):
    # x one-hot rows: y[i, r] = w_hat[r, i], exact in bf16 and fp32, so every
    # element code (all 16, or all 254 finite 8-bit ones) and scale goes
    # through the kernel's conversion without rounding
    k, n = 128, 96
    words, scales = codes_case(6, (n,), k, mode)
    dtype = "f32" if route == "gemv_f32" else "bf16"
    x = _one_hot(k, dtype)
    exact = F.dequantize_f64(words, scales, mode, k).T          # [k, n]
    y = B.nq_fp_qmm(dev(x), dev(words), u8(scales), mode, row_exact=route != "tiled")
    got = values(host(y))
    assert np.array_equal(got, exact), (mode, route, np.argwhere(got != exact)[:4])


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("m,n,k,dtype,row_exact", [
    (1, 200, 320, "bf16", False),
    (3, 77, 96, "f32", False),
    (8, 128, 2048 + 96, "bf16", False),
    (40, 200, 320, "bf16", False),      # tiles, ragged m and n
    (130, 260, 448, "bf16", False),     # several tiles
    (700, 650, 256, "bf16", False),     # 6 x 6 tiles: a partial panel of tile rows, 36 tiles
    (40, 200, 96, "bf16", False),       # k not a multiple of 64: matrix-vector chunks
    (13, 150, 320, "bf16", True),
    (20, 64, 256, "f32", False),
])
def test_qmm_matches_oracle(mode, m, n, k, dtype, row_exact):
    rng_seed = 100 + m + n + k
    words, scales = codes_case(rng_seed, (n,), k, mode)
    _, x = synthetic.random_case(rng_seed, (1, k), (m, k), 1.0, dtype)
    ref = F.qmm_f64(x, words, scales, mode)
    y = B.nq_fp_qmm(dev(x), dev(words), u8(scales), mode, row_exact=row_exact)
    assert_rows_close(values(host(y)), ref, tolerance(y.dtype), (mode, m, n, k, dtype))


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rows_keep_their_one_row_bits(mode, dtype):
    words, scales = codes_case(8, (300,), 2048 + 320, mode)
    _, x = synthetic.random_case(9, (1, 2048 + 320), (13, 2048 + 320), 1.0, dtype)
    xs, cs, ss = dev(x), dev(words), u8(scales)
    full = B.nq_fp_qmm(xs, cs, ss, mode, row_exact=True)
    few = B.nq_fp_qmm(xs[:5], cs, ss, mode)
    for i in range(13):
        one = B.nq_fp_qmm(xs[i:i + 1], cs, ss, mode)
        assert bits_equal(full[i:i + 1], one), (mode, i)
        if i < 5:
            assert bits_equal(few[i:i + 1], one), (mode, i)


def test_nvfp4_global_scale():
    words, scales = codes_case(10, (200,), 320, "nvfp4")
    _, x = synthetic.random_case(10, (1, 320), (40, 320), 1.0, "bf16")
    g = np.float32(0.0371)
    gt = torch.tensor([g], dtype=torch.float32, device="cuda")
    for m in (1, 40):
        ref = F.qmm_f64(x[:m], words, scales, "nvfp4", g)
        y = B.nq_fp_qmm(dev(x[:m]), dev(words), u8(scales), "nvfp4", global_scale=gt)
        assert_rows_close(values(host(y)), ref, tolerance(y.dtype), m)


@pytest.mark.parametrize("mode", MODES)
def test_gather_rows_match_their_expert(mode):
    e, n, k, rows, l = 4, 96, 256, 10, 2
    words, scales = codes_case(12, (e, n), k, mode)
    _, x = synthetic.random_case(12, (1, k), (rows, l, k), 1.0, "bf16")
    idx = np.array([3, 0, 0, 1, 9, 2, 3, 3, 1, 0], np.uint32)          # 9: no such expert
    gsc = np.array([0.5, 1.25, 2.0, 0.75], np.float32) if mode == "nvfp4" else None
    gt = torch.from_numpy(gsc).cuda() if gsc is not None else None
    y = B.nq_fp_gather_qmm(dev(x), dev(words), u8(scales), mode, dev(idx), global_scales=gt,
                           row_exact=True)
    ref = F.gather_qmm_f64(x, words, scales, mode, idx, gsc)
    assert not values(host(y[4])).any()
    keep = [r for r in range(rows) if idx[r] < e]
    assert_rows_close(values(host(y[keep])), ref[keep], tolerance(y.dtype), mode)
    for r in keep:
        ex = int(idx[r])
        one = B.nq_fp_qmm(dev(x[r]), dev(words[ex]), u8(scales[ex]), mode,
                          global_scale=None if gt is None else gt[ex:ex + 1], row_exact=True)
        assert bits_equal(y[r], one), (mode, r)


def test_empty_and_zero_k():
    words, scales = codes_case(13, (64,), 64, "mxfp4")
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    assert B.nq_fp_qmm(x, dev(words), u8(scales), "mxfp4").shape == (0, 64)
    x0 = torch.ones((20, 0), dtype=torch.bfloat16, device="cuda")
    c0 = torch.zeros((64, 0), dtype=torch.int32, device="cuda")
    s0 = torch.zeros((64, 0), dtype=torch.uint8, device="cuda")
    for m in (1, 20):
        y = B.nq_fp_qmm(x0[:m], c0, s0, "mxfp4")
        torch.cuda.synchronize()
        assert not y.float().abs().sum().item()


# ---------------------------------------------------------------- workload sizes
@pytest.mark.parametrize("mode", MODES)
def test_decode_size(mode):
    # [1, 4096] . [14336, 4096]^T, all outputs against the oracle
    words, scales = codes_case(14, (14336,), 4096, mode)
    _, x = synthetic.random_case(14, (1, 4096), (1, 4096), 1.0, "bf16")
    y = B.nq_fp_qmm(dev(x), dev(words), u8(scales), mode)
    ref = F.qmm_f64(x, words, scales, mode)
    assert_rows_close(values(host(y)), ref, tolerance(y.dtype), mode)


def test_prefill_size_sampled_rows():
    # [2048, 4096] . [14336, 4096]^T in tiles; 16 sampled rows against the oracle
    mode = "mxfp4"
    words, scales = codes_case(15, (14336,), 4096, mode)
    _, x = synthetic.random_case(15, (1, 4096), (2048, 4096), 1.0, "bf16")
    y = B.nq_fp_qmm(dev(x), dev(words), u8(scales), mode)
    rows = np.random.default_rng(15).choice(2048, 16, replace=False)
    ref = F.qmm_f64(x[rows], words, scales, mode)
    assert_rows_close(values(host(y[torch.from_numpy(rows).cuda()])), ref, tolerance(y.dtype), mode)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("l", [1, 3])
def test_grouped_gather_rows_keep_their_bits(mode, l):
    # enough rows per expert for the device grouping (workspace in use)
    e, n, k, rows = 8, 96, 320, 48
    assert B.nq_fp_gather_qmm_workspace_bytes(rows, l, k, e, n) > 0
    words, scales = codes_case(16, (e, n), k, mode)
    _, x = synthetic.random_case(16, (1, k), (rows, l, k), 1.0, "bf16")
    idx = np.random.default_rng(16).integers(0, e + 2, size=rows).astype(np.uint32)   # some past e
    gsc = np.linspace(0.5, 2.0, e).astype(np.float32) if mode == "nvfp4" else None
    gt = torch.from_numpy(gsc).cuda() if gsc is not None else None
    y = B.nq_fp_gather_qmm(dev(x), dev(words), u8(scales), mode, dev(idx), global_scales=gt,
                           row_exact=True)
    ref = F.gather_qmm_f64(x, words, scales, mode, idx, gsc)
    yv = values(host(y))
    for r in range(rows):
        if idx[r] >= e:
            assert not yv[r].any(), r
    keep = [r for r in range(rows) if idx[r] < e]
    assert_rows_close(yv[keep], ref[keep], tolerance(y.dtype), mode)
    xs, ws, ss = dev(x), dev(words), u8(scales)
    for r in keep:
        ex = int(idx[r])
        one = B.nq_fp_qmm(xs[r], ws[ex], ss[ex], mode,
                          global_scale=None if gt is None else gt[ex:ex + 1], row_exact=True)
        assert bits_equal(y[r], one), (mode, r)


@pytest.mark.parametrize("mode", MODES)
def test_grouped_gather_moe_shape_streams(mode):
    # K = 2048 takes the streaming grouped kernel: 64 rows over 8 experts
    # (some past the last), every row bit-equal to its one-row product
    e, n, k, rows = 8, 200, 2048, 64
    words, scales = codes_case(17, (e, n), k, mode)
    _, x = synthetic.random_case(17, (1, k), (rows, 1, k), 1.0, "bf16")
    idx = np.random.default_rng(17).integers(0, e + 1, size=rows).astype(np.uint32)
    gsc = np.linspace(0.25, 4.0, e).astype(np.float32) if mode == "nvfp4" else None
    gt = torch.from_numpy(gsc).cuda() if gsc is not None else None
    y = B.nq_fp_gather_qmm(dev(x), dev(words), u8(scales), mode, dev(idx), global_scales=gt,
                           row_exact=True)
    ref = F.gather_qmm_f64(x, words, scales, mode, idx, gsc)
    yv = values(host(y))
    keep = [r for r in range(rows) if idx[r] < e]
    assert all(not yv[r].any() for r in range(rows) if idx[r] >= e)
    assert_rows_close(yv[keep], ref[keep], tolerance(y.dtype), mode)
    xs, ws, ss = dev(x), dev(words), u8(scales)
    for r in keep:
        ex = int(idx[r])
        one = B.nq_fp_qmm(xs[r], ws[ex], ss[ex], mode,
                          global_scale=None if gt is None else gt[ex:ex + 1], row_exact=True)
        assert bits_equal(y[r], one), (mode, r)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("n,k", [(8192 + 96, 2048 + 320), (9000, 1024)])
def test_long_decode_rows_keep_their_bits(mode, n, k):
    # long one-row products (the streaming decode kernel, several rows per
    # wave) equal the few-row kernel's rows (row-exact) bit for bit, and the
    # oracle
    words, scales = codes_case(19, (n,), k, mode)
    _, x = synthetic.random_case(19, (1, k), (3, k), 1.0, "bf16")
    xs, cs, ss = dev(x), dev(words), u8(scales)
    full = B.nq_fp_qmm(xs, cs, ss, mode, row_exact=True)
    for i in range(3):
        one = B.nq_fp_qmm(xs[i:i + 1], cs, ss, mode)
        assert bits_equal(full[i:i + 1], one), (mode, i)
    ref = F.qmm_f64(x[:1], words, scales, mode)
    assert_rows_close(values(host(full[:1])), ref, tolerance(full.dtype), mode)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("l,k", [(1, 320), (2, 448)])
def test_gather_matrix_core_route(mode, l, k):
    # shared experts, bf16 x, k % 64 == 0, row_exact off: MFMA tiles over
    # chunks of up to 32 vectors (ragged n, ids past the last expert)
    e, n, rows = 8, 200, 80
    words, scales = codes_case(20 + l, (e, n), k, mode)
    _, x = synthetic.random_case(20 + l, (1, k), (rows, l, k), 1.0, "bf16")
    idx = np.random.default_rng(20 + l).integers(0, e + 1, size=rows).astype(np.uint32)
    gsc = np.linspace(0.5, 3.0, e).astype(np.float32) if mode == "nvfp4" else None
    gt = torch.from_numpy(gsc).cuda() if gsc is not None else None
    y = B.nq_fp_gather_qmm(dev(x), dev(words), u8(scales), mode, dev(idx), global_scales=gt)
    ref = F.gather_qmm_f64(x, words, scales, mode, idx, gsc)
    yv = values(host(y))
    assert all(not yv[r].any() for r in range(rows) if idx[r] >= e)
    keep = [r for r in range(rows) if idx[r] < e]
    assert_rows_close(yv[keep], ref[keep], tolerance(y.dtype), mode)


def test_gather_matrix_core_moe_shape():
    # 512 rows over 32 NVFP4 experts [1408, 2048] with global scales; 24
    # sampled rows against the oracle
    mode, e, n, k, rows = "nvfp4", 32, 1408, 2048, 512
    words, scales = codes_case(22, (e, n), k, mode)
    _, x = synthetic.random_case(22, (1, k), (rows, 1, k), 1.0, "bf16")
    idx = np.random.default_rng(22).integers(0, e, size=rows).astype(np.uint32)
    gsc = np.linspace(0.5, 2.0, e).astype(np.float32)
    y = B.nq_fp_gather_qmm(dev(x), dev(words), u8(scales), mode, dev(idx),
                           global_scales=torch.from_numpy(gsc).cuda())
    pick = np.random.default_rng(22).choice(rows, 24, replace=False)
    ref = F.gather_qmm_f64(x[pick], words, scales, mode, idx[pick], gsc)
    assert_rows_close(values(host(y[torch.from_numpy(pick).cuda()])), ref, tolerance(y.dtype), mode)


# ---------------------------------------------------------------- weights as stored
@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("m,ni,nc,dtype,row_exact", [
    (1, 320, 224, "bf16", False),
    (3, 300, 96, "f32", False),                   # ragged row ranges
    (5, 448, 256, "bf16", True),
    (40, 320, 224, "bf16", False),                # tiles, ragged nc
    (130, 448, 96, "bf16", False),                # several row tiles, nc < one tile
    (700, 192, 640, "bf16", False),               # 6 x 5 tiles: a partial panel, 30 tiles
    (40, 64, 224, "bf16", False),                 # tiles, one K step
    (130, 128, 96, "bf16", False),                # tiles, two K steps
])
def test_notrans_matches_oracle(mode, m, ni, nc, dtype, row_exact):
    words, scales = codes_case(30 + m, (ni,), nc, mode)
    _, x = synthetic.random_case(30 + m, (1, ni), (m, ni), 1.0, dtype)
    g = 0.625 if mode == "nvfp4" else None
    gt = torch.tensor([g], dtype=torch.float32, device="cuda") if g else None
    y = B.nq_fp_qmm_notrans(dev(x), dev(words), u8(scales), mode, global_scale=gt, row_exact=row_exact)
    ref = F.qmm_nt_f64(x, words, scales, mode, g)
    assert_rows_close(values(host(y)), ref, tolerance(y.dtype), (mode, m, ni, nc))


@pytest.mark.parametrize("mode", MODES)
def test_notrans_rows_keep_their_bits(mode):
    words, scales = codes_case(40, (1000,), 512, mode)
    _, x = synthetic.random_case(40, (1, 1000), (7, 1000), 1.0, "bf16")
    xs, cs, ss = dev(x), dev(words), u8(scales)
    full = B.nq_fp_qmm_notrans(xs, cs, ss, mode, row_exact=True)
    for i in range(7):
        one = B.nq_fp_qmm_notrans(xs[i:i + 1], cs, ss, mode)
        assert bits_equal(full[i:i + 1], one), (mode, i)


def test_notrans_decode_size_and_empty_inner():
    # dx = dy [1, 14336] . W [14336, 4096] as stored (the decode weights' derivative)
    mode = "mxfp4"
    words, scales = codes_case(41, (14336,), 4096, mode)
    _, dy = synthetic.random_case(41, (1, 14336), (1, 14336), 1.0, "bf16")
    y = B.nq_fp_qmm_notrans(dev(dy), dev(words), u8(scales), mode)
    assert_rows_close(values(host(y)), F.qmm_nt_f64(dy, words, scales, mode), tolerance(y.dtype), mode)
    x0 = torch.ones((3, 0), dtype=torch.bfloat16, device="cuda")
    c0 = torch.zeros((0, 64 * 4 // 32), dtype=torch.int32, device="cuda")
    s0 = torch.zeros((0, 2), dtype=torch.uint8, device="cuda")
    y0 = B.nq_fp_qmm_notrans(x0, c0, s0, mode)
    torch.cuda.synchronize()
    assert y0.shape == (3, 64) and not y0.float().abs().sum().item()


@pytest.mark.parametrize("mode", ["mxfp4", "mxfp8"])
@pytest.mark.parametrize("route", ["gemv", "tiled"])
def test_products_extreme_scales_exact(mode, route):
    # one-hot rows pick w_hat[r, i] exactly, with E8M0 scale codes at the ends
    # of the range.  The matrix-vector route scales in fp32 after the group
    # sums and takes every code up to 2^127 (products that overflow bf16 are
    # +-inf in both); the tiles' B operands are bf16(S * E), so there the
    # codes stop where |S * E| still fits bf16 (an infinite B element would
    # make 0 * inf = NaN in the other outputs of its column)
    _, bits, gs, _ = F.mode_info(mode)
    k, n = 128, 64
    words, _ = synthetic.random_fp_matrix(50, (n,), k, bits, gs, (0, 0), finite_bytes=True)
    if route == "gemv":
        codes = np.array([0, 1, 2, 3, 60, 127, 200, 250, 252, 253, 254], np.uint8)
    else:
        top = 252 if mode == "mxfp4" else 245           # 6 * 2^125, 448 * 2^118 < bf16 max
        codes = np.array([0, 1, 2, 3, 60, 127, 200, top - 2, top - 1, top], np.uint8)
    scales = codes[np.arange(n * (k // gs)) % len(codes)].reshape(n, k // gs)
    x = _one_hot(k, "bf16")
    exact = F.dequantize(words, scales, mode, k, "bf16").T          # bf16(S * E), [k, n]
    y = B.nq_fp_qmm(dev(x), dev(words), u8(scales), mode, row_exact=route == "gemv")
    got = host(y)
    same = (got == exact) | ((got & 0x7FFF) == 0) & ((exact & 0x7FFF) == 0)   # +-0 alike
    assert same.all(), (mode, route, np.argwhere(~same)[:4], got[~same][:4], exact[~same][:4])
