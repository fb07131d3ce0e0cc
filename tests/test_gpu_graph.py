"""Captured HIP graphs of the product kernels replay the eager results bit
for bit, replay after replay, with other eager work and synchronisations in
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

    outs = {
        "decode": torch.empty((1, 512), dtype=torch.bfloat16, device="cuda"),
        "few": torch.empty((5, 512), dtype=torch.bfloat16, device="cuda"),
        "exact": torch.empty((20, 512), dtype=torch.bfloat16, device="cuda"),
        "tiled": torch.empty((20, 512), dtype=torch.bfloat16, device="cuda"),
        "gather": torch.empty((4, 1, 256), dtype=torch.bfloat16, device="cuda"),
    }

    def launch():
        B.nq_qmm(xs[:1], c, s, b, gs, bits, y=outs["decode"])
        B.nq_qmm(xs[:5], c, s, b, gs, bits, y=outs["few"])
        B.nq_qmm_row_exact(xs, c, s, b, gs, bits, y=outs["exact"])
        B.nq_qmm(xs, c, s, b, gs, bits, y=outs["tiled"])
        B.nq_gather_qmm(xgs, cg, sg, bg, gs, bits, ids, y=outs["gather"])

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
