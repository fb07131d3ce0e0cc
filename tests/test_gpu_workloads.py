"""The five benchmark workloads at full size, through the kernels the planner
picks for them (the launch configuration the benchmark times), against the
CPU oracle on the same seeded inputs.

  affine_f32_256x512  W f32 [256,512] ~ N(0,1), 4-bit g64, x f32 [4,512]
  decode_gemv         W [14336,4096] ~ N(0,0.02) 4-bit g64, x bf16 [1,4096]
  multirow_8bit       W [4096,4096] 8-bit g128, x bf16 [8,4096], batched and row-exact
  splitk              W [1024,14336] 4-bit g64, x bf16 [4,14336]
  prefill             W as decode_gemv, x bf16 [2048,4096] (sampled outputs)
  moe_gather          W [32,1408,2048] 4-bit g64, x bf16 [512,1,2048], ids in [0,32)
and the derivative rows of the benchmark at the decode weights (dx for 1 and
2048 rows, the scale and bias derivatives for 1 row).
"""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_helpers import assert_rows_close, bits_equal, dev, host, values
from group_wise_affine_quantize_amd import _binding as B
from group_wise_affine_quantize_amd import synthetic

pytestmark = pytest.mark.gpu

_cache = {}


def workload(name):
    if name not in _cache:
        wl = synthetic.WORKLOADS[name]
        d = synthetic.generate(name)
        d["q"] = O.quantize(d["w"], wl.group_size, wl.bits)
        d["wl"] = wl
        _cache[name] = d
    return _cache[name]


def quantize_on_gpu_and_check(d):
    wl = d["wl"]
    c, s, b = B.nq_quantize(dev(d["w"]), wl.group_size, wl.bits)
    torch.cuda.synchronize()
    cr, sr, br = d["q"]
    assert np.array_equal(host(c), cr)
    assert np.array_equal(host(s).view(np.uint8), sr.view(np.uint8))
    assert np.array_equal(host(b).view(np.uint8), br.view(np.uint8))
    return c, s, b


def plan_of(d, m, row_exact=False):
    wl = d["wl"]
    xdt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    n, k = wl.w_shape[-2], wl.w_shape[-1]
    return B.nq_qmm_plan(m, n, k, wl.group_size, wl.bits, xdt, xdt, row_exact)


def test_affine_f32_256x512():
    d = workload("affine_f32_256x512")
    wl = d["wl"]
    c, s, b = quantize_on_gpu_and_check(d)
    w_hat = B.nq_dequantize(c, s, b, wl.group_size, wl.bits)
    assert w_hat.shape == (256, 512) and w_hat.dtype == torch.float32
    assert np.array_equal(host(w_hat), O.dequantize(*d["q"], wl.group_size, wl.bits))
    y = B.nq_qmm(dev(d["x"]), c, s, b, wl.group_size, wl.bits)
    assert y.shape == (4, 256) and y.dtype == torch.float32
    assert_rows_close(host(y), O.qmm_f64(d["x"], *d["q"], wl.group_size, wl.bits), 1e-3)


def test_decode_gemv():
    d = workload("decode_gemv")
    wl = d["wl"]
    c, s, b = quantize_on_gpu_and_check(d)
    p = plan_of(d, 1)
    assert p.route == B.NQ_ROUTE_GEMV and p.ksplit == 1
    y = B.nq_qmm(dev(d["x"]), c, s, b, wl.group_size, wl.bits)
    assert y.shape == (1, 14336) and y.dtype == torch.bfloat16
    assert_rows_close(values(host(y)), O.qmm_f64(d["x"], *d["q"], wl.group_size, wl.bits), 1e-2)
    assert bits_equal(y, B.nq_qmm(dev(d["x"]), c, s, b, wl.group_size, wl.bits))


def test_multirow_8bit_batched_and_row_exact():
    d = workload("multirow_8bit")
    wl = d["wl"]
    c, s, b = quantize_on_gpu_and_check(d)
    xs = dev(d["x"])
    y = B.nq_qmm(xs, c, s, b, wl.group_size, wl.bits)
    y_ref = O.qmm_f64(d["x"], *d["q"], wl.group_size, wl.bits)
    assert_rows_close(values(host(y)), y_ref, 1e-2)
    yr = B.nq_qmm_row_exact(xs, c, s, b, wl.group_size, wl.bits)
    assert_rows_close(values(host(yr)), y_ref, 1e-2)
    for i in range(8):
        y1 = B.nq_qmm(xs[i:i + 1].contiguous(), c, s, b, wl.group_size, wl.bits)
        assert bits_equal(y1[0], yr[i]) and bits_equal(y1[0], y[i]), i


def test_splitk():
    d = workload("splitk")
    wl = d["wl"]
    c, s, b = quantize_on_gpu_and_check(d)
    p = plan_of(d, 4)
    assert p.route == B.NQ_ROUTE_GEMV and p.ksplit > 1
    xs = dev(d["x"])
    y = B.nq_qmm(xs, c, s, b, wl.group_size, wl.bits)
    assert_rows_close(values(host(y)), O.qmm_f64(d["x"], *d["q"], wl.group_size, wl.bits), 1e-2)
    yr = B.nq_qmm_row_exact(xs, c, s, b, wl.group_size, wl.bits)
    for i in range(4):
        y1 = B.nq_qmm(xs[i:i + 1].contiguous(), c, s, b, wl.group_size, wl.bits)
        assert bits_equal(y1[0], yr[i]) and bits_equal(y1[0], y[i]), i


def test_prefill_sampled():
    d = workload("prefill")
    wl = d["wl"]
    cr, sr, br = d["q"]
    c, s, b = dev(cr), dev(sr), dev(br)   # same weights as decode_gemv, checked there
    assert plan_of(d, 2048).route == B.NQ_ROUTE_TILED
    y = host(B.nq_qmm(dev(d["x"]), c, s, b, wl.group_size, wl.bits))
    assert y.shape == (2048, 14336)
    yv = values(y)
    assert np.all(np.isfinite(yv))
    rng = np.random.default_rng(7)
    # whole rows at tile edges and at random
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 255, 256, 1023, 2046, 2047],
                                     rng.integers(0, 2048, 7)]))
    y_ref = O.qmm_f64(d["x"][rows], cr, sr, br, wl.group_size, wl.bits)
    assert_rows_close(yv[rows], y_ref, 1e-2, "prefill rows")
    # scattered single outputs, including tile corners
    ms = np.concatenate([rng.integers(0, 2048, 20000), [0, 2047, 127, 128]])
    ns = np.concatenate([rng.integers(0, 14336, 20000), [14335, 0, 127, 128]])
    ref = O.qmm_sample_f64(d["x"], cr, sr, br, wl.group_size, wl.bits, ms, ns)
    scale = np.max(np.abs(y_ref))
    assert np.max(np.abs(yv[ms, ns] - ref)) <= 1e-2 * scale


def test_moe_gather():
    d = workload("moe_gather")
    wl = d["wl"]
    c, s, b = quantize_on_gpu_and_check(d)
    xs, ids = dev(d["x"]), dev(d["ids"])
    y_ref = O.gather_qmm_f64(d["x"], *d["q"], wl.group_size, wl.bits, d["ids"])
    yd = B.nq_gather_qmm(xs, c, s, b, wl.group_size, wl.bits, ids)     # matrix cores
    assert yd.shape == (512, 1, 1408) and yd.dtype == torch.bfloat16
    assert_rows_close(values(host(yd)), y_ref, 1e-2, "gather")
    y = B.nq_gather_qmm_row_exact(xs, c, s, b, wl.group_size, wl.bits, ids)
    assert_rows_close(values(host(y)), y_ref, 1e-2, "gather row-exact")
    outs = [B.nq_qmm(xs[r], c[e], s[e], b[e], wl.group_size, wl.bits)
            for r, e in enumerate(d["ids"].tolist())]
    torch.cuda.synchronize()
    for r in range(512):
        assert bits_equal(outs[r], y[r]), r


def test_derivatives_at_the_decode_weights():
    """The derivative rows of the benchmark at full size ("Training through
    quantized weights"): dx = dy times the decode weights as stored, for one
    row (partial sums and their ordered reduction) and for 2048 rows (tiles,
    sampled rows), and the scale and bias derivatives for one row."""
    d = workload("decode_gemv")
    wl = d["wl"]
    cr, sr, br = d["q"]
    c, s, b = dev(cr), dev(sr), dev(br)
    gs, bits = wl.group_size, wl.bits
    dy1 = synthetic.random_case(5, (1, 1), (1, 14336), 1.0, "f32", "bf16")[1]
    dx = B.nq_qmm_notrans(dev(dy1), c, s, b, gs, bits)
    assert dx.shape == (1, 4096) and dx.dtype == torch.bfloat16
    assert_rows_close(values(host(dx)), O.qmm_nt_f64(dy1, cr, sr, br, gs, bits), 1e-2, "dx decode")
    assert bits_equal(dx, B.nq_qmm_notrans_row_exact(dev(dy1), c, s, b, gs, bits))
    ds, db = B.nq_qmm_grad_scales_biases(dev(d["x"]), dev(dy1), c, gs, bits, out_dtype=torch.float32)
    ds_ref, db_ref = O.qmm_grad_sb_f64(d["x"], dy1, cr, gs, bits)
    assert ds.shape == (14336, 64)
    assert_rows_close(values(host(ds)), ds_ref, 1e-3, "dscales")
    assert_rows_close(values(host(db)), db_ref, 1e-3, "dbiases")
    dyp = synthetic.random_case(6, (1, 1), (2048, 14336), 1.0, "f32", "bf16")[1]
    dxp = values(host(B.nq_qmm_notrans(dev(dyp), c, s, b, gs, bits)))
    assert dxp.shape == (2048, 4096) and np.all(np.isfinite(dxp))
    rows = np.array([0, 127, 128, 1023, 2047])
    assert_rows_close(dxp[rows], O.qmm_nt_f64(dyp[rows], cr, sr, br, gs, bits), 1e-2, "dx prefill rows")
