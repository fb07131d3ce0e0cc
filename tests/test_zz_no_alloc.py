"""The gather entry point for callers that cannot allocate
(nq_gather_qmm_noalloc: its grouping tables in the library's static device
array) against nq_gather_qmm with a caller's workspace: bit-identical
outputs on two calls in a row, the second with a smaller input, on both
grouped routes that write the tables (the matrix-vector one for fp32
activations, the matrix-core one past the in-kernel grouping's size).
Collected last: it must also pass after every other test has used the GPU."""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_helpers import assert_rows_close, bits_equal, dev, host, tolerance, values
from group_wise_affine_quantize_amd import _binding as B
from group_wise_affine_quantize_amd import synthetic

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    torch.cuda.set_device(0)
    B.load_library()


def _case(seed, rows, e, n, k, x_dtype):
    w, _ = synthetic.random_case(seed, (e, n, k), (1, k), 0.02, "bf16")
    _, x = synthetic.random_case(seed + 1, (1, 1), (rows, 1, k), 1.0, "f32", x_dtype)
    ids = np.random.default_rng(seed).integers(0, e + 1, size=rows, dtype=np.uint32)   # e: zero rows
    c, s, b = O.quantize(w.reshape(e * n, k), 64, 4)
    c, s, b = (a.reshape(e, n, -1) for a in (c, s, b))
    return x, c, s, b, ids


@pytest.mark.parametrize("x_dtype,first,second", [("f32", (300, 8), (60, 8)),
                                                  ("bf16", (2600, 40), (1200, 300))])
def test_noalloc_gather_matches_workspace_gather(x_dtype, first, second):
    n, k = 192, 512
    for seed, (rows, e) in ((11, first), (12, second)):
        x, c, s, b, ids = _case(seed, rows, e, n, k, x_dtype)
        assert B.nq_gather_qmm_workspace_bytes(rows, 1, k, e, n, 64, 4, x_dtype == "bf16" and torch.bfloat16
                                               or torch.float32, torch.bfloat16) > 0   # a grouped route
        xs, cs, ss, bs, idx = dev(x), dev(c), dev(s), dev(b), dev(ids)
        y_ws = B.nq_gather_qmm(xs, cs, ss, bs, 64, 4, idx)
        y_na = B.nq_gather_qmm_noalloc(xs, cs, ss, bs, 64, 4, idx)
        torch.cuda.synchronize()
        assert bits_equal(y_ws, y_na), (x_dtype, rows, e)
        assert_rows_close(values(host(y_na)), O.gather_qmm_f64(x, c, s, b, 64, 4, ids), tolerance(y_na.dtype),
                          "noalloc gather")


def test_noalloc_gather_rejects_tables_past_the_scratch():
    rows, e, n, k = 200_000, 64, 64, 64
    need = B.nq_gather_qmm_workspace_bytes(rows, 1, k, e, n, 64, 4, torch.bfloat16, torch.bfloat16)
    assert need > (1 << 20)
    x = torch.zeros((rows, 1, k), dtype=torch.bfloat16, device="cuda")
    cs = torch.zeros((e, n, k // 8), dtype=torch.int32, device="cuda")
    ss = torch.zeros((e, n, 1), dtype=torch.bfloat16, device="cuda")
    ids = torch.zeros(rows, dtype=torch.int32, device="cuda")
    with pytest.raises(B.NQError) as ei:
        B.nq_gather_qmm_noalloc(x, cs, ss, ss, 64, 4, ids)
    assert ei.value.status == 7 and "static scratch" in ei.value.message   # NQ_ERR_WORKSPACE
