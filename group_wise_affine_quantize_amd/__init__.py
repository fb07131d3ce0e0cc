"""group_wise_affine_quantize_amd -- group-wise affine quantization and
quantized matrix products on MI355X (gfx950).

The work is done by the C-ABI library libnq.so (hand-written HIP kernels);
this package only marshals torch tensors into its calls.  Importing the
package loads nothing; the first call loads libnq.so and fails loudly if it
is missing.
"""
from ._binding import (  # noqa: F401
    NQ_ROW_INDEPENDENT_ROWS,
    NQError,
    library_path,
    load_library,
    nq_dequantize,
    nq_fp_dequantize,
    nq_fp_gather_qmm,
    nq_fp_gather_qmm_workspace_bytes,
    nq_fp_qmm,
    nq_fp_qmm_notrans,
    nq_fp_qmm_notrans_workspace_bytes,
    nq_fp_quantize,
    nq_gather_qmm,
    nq_gather_qmm_row_exact,
    nq_gather_qmm_lhs,
    nq_gather_qmm_workspace_bytes,
    nq_qmm,
    nq_qmm_batched,
    nq_qmm_grad_scales_biases,
    nq_qmm_notrans,
    nq_qmm_notrans_row_exact,
    nq_qmm_notrans_workspace_bytes,
    nq_qmm_plan,
    nq_qmm_row_exact,
    nq_qmm_with_plan,
    Plan,
    nq_qmm_workspace_bytes,
    nq_quantize,
)
