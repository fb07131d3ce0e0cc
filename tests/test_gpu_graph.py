"""Captured HIP graphs of the product kernels (affine and floating-point
modes) replay the eager results bit for bit, replay after replay, with other eager work and synchronisations in
between (the benchmark times graph replays)."""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_helpers import bits_equal, dev
from group_wise_affine_quantize_amd import _binding as B
from group_wise_affine_quantize_amd import synthetic

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    gs, bits = 64, 4
    w, x = synthetic.random_case(11, (512, 2048 * 3), (20, 2048 * 3), 0.02, "bf16")
    c, s, b = (dev(a) for a in O.quantize(w, gs, bits))
    xs = dev(x)
    ids = dev(np.array([0, 1, 1, 0], np.uint32))
    wg, xg = synthetic.random_case(12, (2, 256, 1024), (4, 1, 1024), 0.02, "bf16")
    cg, sg, bg = (dev(a) for a in O.quantize(wg, gs, bits))
    xgs = dev(xg)

    # a long decode (the streaming kernel), a grouped gather with left
    # indices, the product with the weights as stored and the derivatives
    wl, xl = synthetic.random_case(13, (8192, 2048), (2, 2048), 0.02, "bf16")
    cl, sl, bl = (dev(a) for a in O.quantize(wl, gs, bits))
    xls = dev(xl)
    we, xe = synthetic.random_case(14, (3, 128, 1024), (64, 1, 1024), 0.02, "bf16")
    ce, se, be = (dev(a) for a in O.quantize(we, gs, bits))
    xes = dev(xe)
    rng = np.random.default_rng(5)
    ide = dev(rng.integers(0, 3, size=80, dtype=np.uint32))
    lhe = dev(rng.integers(0, 64, size=80, dtype=np.uint32))
    ws_g = torch.empty(B.nq_gather_qmm_workspace_bytes(80, 1, 1024, 3, 128, gs, bits, torch.bfloat16,
                                                       torch.bfloat16), dtype=torch.uint8, device="cuda")
    ws_nt = torch.empty(max(1, B.nq_qmm_notrans_workspace_bytes(1, 512, 2048 * 3, gs, bits, torch.bfloat16)),
                        dtype=torch.uint8, device="cuda")
    wf, sfp = synthetic.random_fp_matrix(18, (1024,), 2048, 4, 16, (0x20, 0x50))
    wf, sfp = dev(wf), torch.from_numpy(sfp).cuda()
    gfp = torch.tensor([0.75], dtype=torch.float32, device="cuda")
    xf = xs[:, :2048].contiguous()
    # floating-point gathers with shared experts: matrix-core and row-exact
    # routes behind the device grouping pass
    wfe, sfe = synthetic.random_fp_matrix(19, (4, 256), 2048, 4, 32, (120, 134))
    wfe, sfe = dev(wfe), torch.from_numpy(sfe).cuda()
    idf = dev(np.random.default_rng(19).integers(0, 5, size=20).astype(np.uint32))
    xfg = xf.view(20, 1, 2048)
    ws_f = torch.empty(B.nq_fp_gather_qmm_workspace_bytes(20, 1, 2048, 4, 256), dtype=torch.uint8,
                       device="cuda")
    # the weights as stored: dy [3, 1024] . W [1024, 2048] (row ranges, ordered adds)
    dyf = xs[:3, :1024].contiguous()
    ws_nf = torch.empty(B.nq_fp_qmm_notrans_workspace_bytes(3, 1024, 2048, "nvfp4", torch.bfloat16),
                        dtype=torch.uint8, device="cuda")
    dy = xs[:1, :512].contiguous()
    dy3 = xs[:3, :512].contiguous()

    outs = {
        "decode": torch.empty((1, 512), dtype=torch.bfloat16, device="cuda"),
        "few": torch.empty((5, 512), dtype=torch.bfloat16, device="cuda"),
        "exact": torch.empty((20, 512), dtype=torch.bfloat16, device="cuda"),
        "tiled": torch.empty((20, 512), dtype=torch.bfloat16, device="cuda"),
        "gather": torch.empty((4, 1, 256), dtype=torch.bfloat16, device="cuda"),
        "stream": torch.empty((1, 8192), dtype=torch.bfloat16, device="cuda"),
        "batched": torch.empty((2, 10, 512), dtype=torch.bfloat16, device="cuda"),
        "gather_lhs": torch.empty((80, 1, 128), dtype=torch.bfloat16, device="cuda"),
        "notrans": torch.empty((1, 2048 * 3), dtype=torch.bfloat16, device="cuda"),
        "dscales": torch.empty((512, 2048 * 3 // gs), dtype=torch.float32, device="cuda"),
        "dbiases": torch.empty((512, 2048 * 3 // gs), dtype=torch.float32, device="cuda"),
        "dequant": torch.empty((512, 2048 * 3), dtype=torch.bfloat16, device="cuda"),
        "fp_decode": torch.empty((1, 1024), dtype=torch.bfloat16, device="cuda"),
        "fp_few": torch.empty((5, 1024), dtype=torch.bfloat16, device="cuda"),
        "fp_tiled": torch.empty((20, 1024), dtype=torch.bfloat16, device="cuda"),
        "fp_dequant": torch.empty((1024, 2048), dtype=torch.bfloat16, device="cuda"),
        "fp_gather": torch.empty((20, 1, 256), dtype=torch.bfloat16, device="cuda"),
        "fp_gather_exact": torch.empty((20, 1, 256), dtype=torch.bfloat16, device="cuda"),
        "fp_notrans": torch.empty((3, 2048), dtype=torch.bfloat16, device="cuda"),
    }

    def launch():
        B.nq_qmm(xs[:1], c, s, b, gs, bits, y=outs["decode"])
        B.nq_qmm(xs[:5], c, s, b, gs, bits, y=outs["few"])
        B.nq_qmm_row_exact(xs, c, s, b, gs, bits, y=outs["exact"])
        B.nq_qmm(xs, c, s, b, gs, bits, y=outs["tiled"])
        B.nq_gather_qmm(xgs, cg, sg, bg, gs, bits, ids, y=outs["gather"])
        B.nq_qmm(xls[:1], cl, sl, bl, gs, bits, y=outs["stream"])
        B.nq_qmm_batched(xs.view(2, 10, -1), c, s, b, gs, bits, y=outs["batched"])
        B.nq_gather_qmm_lhs(xes, ce, se, be, gs, bits, lhe, ide, y=outs["gather_lhs"], workspace=ws_g)
        B.nq_qmm_notrans(dy, c, s, b, gs, bits, y=outs["notrans"], workspace=ws_nt)
        B.nq_qmm_grad_scales_biases(xs[:3], dy3, c, gs, bits, dscales=outs["dscales"], dbiases=outs["dbiases"])
        B.nq_dequantize(c, s, b, gs, bits, out=outs["dequant"])
        B.nq_fp_qmm(xf[:1], wf, sfp, "nvfp4", global_scale=gfp, y=outs["fp_decode"])
        B.nq_fp_qmm(xf[:5], wf, sfp, "nvfp4", y=outs["fp_few"])
        B.nq_fp_qmm(xf, wf, sfp, "nvfp4", global_scale=gfp, y=outs["fp_tiled"])
        B.nq_fp_dequantize(wf, sfp, "nvfp4", out=outs["fp_dequant"])
        B.nq_fp_gather_qmm(xfg, wfe, sfe, "mxfp4", idf, y=outs["fp_gather"], workspace=ws_f)
        B.nq_fp_gather_qmm(xfg, wfe, sfe, "mxfp4", idf, row_exact=True, y=outs["fp_gather_exact"],
                           workspace=ws_f)
        B.nq_fp_qmm_notrans(dyf, wf, sfp, "nvfp4", global_scale=gfp, y=outs["fp_notrans"], workspace=ws_nf)

    launch()
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in outs.items()}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        launch()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        launch()
    for rep in range(4):
        for v in outs.values():
            v.fill_(0)
        scratch = B.nq_qmm(xs[:3], c, s, b, gs, bits)     # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in outs.items():
            assert bits_equal(v, eager[k]), (rep, k)
        assert scratch.shape == (3, 512)


def test_graph_replays_match_eager_band():
    """The 8-bit matrix-core matrix-vector kernel (plain, row-exact and the
    grouped gather behind the grouping pass) under graph replay."""
    gs, bits = 128, 8
    w, x = synthetic.random_case(21, (4096, 2048), (11, 2048), 0.02, "bf16")
    c, s, b = (dev(a) for a in O.quantize(w, gs, bits))
    xs = dev(x)
    we, xe = synthetic.random_case(22, (3, 96, 1024), (40, 1, 1024), 0.02, "bf16")
    ce, se, be = (dev(a) for a in O.quantize(we, gs, bits))
    xes = dev(xe)
    ide = dev(np.random.default_rng(23).integers(0, 3, size=40, dtype=np.uint32))
    ws = torch.empty(B.nq_gather_qmm_workspace_bytes(40, 1, 1024, 3, 96, gs, bits, torch.bfloat16,
                                                     torch.bfloat16), dtype=torch.uint8, device="cuda")
    outs = {
        "few": torch.empty((8, 4096), dtype=torch.bfloat16, device="cuda"),
        "exact": torch.empty((11, 4096), dtype=torch.bfloat16, device="cuda"),
        "gather": torch.empty((40, 1, 96), dtype=torch.bfloat16, device="cuda"),
    }

    def launch():
        B.nq_qmm(xs[:8], c, s, b, gs, bits, y=outs["few"])
        B.nq_qmm_row_exact(xs, c, s, b, gs, bits, y=outs["exact"])
        B.nq_gather_qmm_row_exact(xes, ce, se, be, gs, bits, ide, y=outs["gather"], workspace=ws)

    launch()
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in outs.items()}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        launch()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        launch()
    for rep in range(4):
        for v in outs.values():
            v.fill_(0)
        scratch = B.nq_qmm(xs[:3], c, s, b, gs, bits)     # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in outs.items():
            assert bits_equal(v, eager[k]), (rep, k)
        assert scratch.shape == (3, 4096)
