"""ctypes binding of libnq.so: argument marshalling only.

Every function here takes torch tensors on the GPU, checks that their dtypes
and shapes describe the call, and passes raw device pointers and the current
HIP stream to the C entry point of the same name (include/nq.h).  All
arithmetic happens in libnq's HIP kernels; there is no fallback of any kind.
If libnq.so was not built, the first call raises.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libnq.so"

NQ_ROW_INDEPENDENT_ROWS = 8
NQ_F32, NQ_BF16 = 0, 1
NQ_ROUTE_GEMV, NQ_ROUTE_TILED = 1, 2
NQ_MXFP4, NQ_MXFP8, NQ_NVFP4 = 1, 2, 3
# floating-point mode -> (C enum, bits per code, group size)
FP_MODES = {"mxfp4": (NQ_MXFP4, 4, 32), "mxfp8": (NQ_MXFP8, 8, 32), "nvfp4": (NQ_NVFP4, 4, 16)}

_lib = None


class NQError(RuntimeError):
    """A libnq call returned a non-zero status."""

    def __init__(self, status, message):
        super().__init__(f"[{status}] {message}")
        self.status = status
        self.message = message


class Plan(ctypes.Structure):
    _fields_ = [("route", ctypes.c_int32), ("ksplit", ctypes.c_int32),
                ("rows_per_wave", ctypes.c_int32), ("tile_m", ctypes.c_int32),
                ("tile_n", ctypes.c_int32), ("reserved", ctypes.c_int32 * 3)]

    def as_dict(self):
        return {"route": {1: "gemv", 2: "tiled"}.get(self.route, self.route),
                "ksplit": self.ksplit, "rows_per_wave": self.rows_per_wave,
                "tile_m": self.tile_m, "tile_n": self.tile_n}


def library_path():
    """libnq.so next to this file, or the build NQ_LIBRARY names (for
    instance the host-sanitizer build)."""
    return os.environ.get("NQ_LIBRARY") or os.path.join(HERE, _LIB_NAME)


_P, _I64, _I32, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
_SIGNATURES = {
    "nq_quantize": [_P, _I32, _I64, _I64, _I32, _I32, _P, _P, _P, _P],
    "nq_dequantize": [_P, _P, _P, _I32, _I64, _I64, _I32, _I32, _P, _I32, _P],
    "nq_qmm_plan": [_I64, _I64, _I64, _I32, _I32, _I32, _I32, _I32, ctypes.POINTER(Plan)],
    "nq_qmm_workspace_bytes": [_I64, _I64, _I64, _I32, _I32, _I32, _I32, _I32],
    "nq_qmm": [_P, _I32, _I64, _I64, _P, _P, _P, _I32, _I64, _I32, _I32, _P, _P, _SZ, _P],
    "nq_qmm_row_exact": [_P, _I32, _I64, _I64, _P, _P, _P, _I32, _I64, _I32, _I32, _P, _P, _SZ,
                         _P],
    "nq_qmm_with_plan": [ctypes.POINTER(Plan), _P, _I32, _I64, _I64, _P, _P, _P, _I32, _I64,
                         _I32, _I32, _P, _P, _SZ, _P],
    "nq_qmm_batched": [_P, _I32, _I64, _I64, _I64, _P, _P, _P, _I32, _I64, _I32, _I32, _P, _P, _SZ,
                       _P],
    "nq_gather_qmm_workspace_bytes": [_I64, _I64, _I64, _I64, _I64, _I32, _I32, _I32, _I32,
                                      _I32],
    "nq_gather_qmm": [_P, _I32, _I64, _I64, _I64, _P, _P, _P, _I32, _I64, _I64, _I32, _I32, _P,
                      _I32, _P, _P, _SZ, _P],
    "nq_gather_qmm_noalloc": [_P, _I32, _I64, _I64, _I64, _P, _P, _P, _I32, _I64, _I64, _I32, _I32, _P,
                              _I32, _P, _P],
    "nq_gather_qmm_row_exact": [_P, _I32, _I64, _I64, _I64, _P, _P, _P, _I32, _I64, _I64, _I32,
                                _I32, _P, _I32, _P, _P, _SZ, _P],
    "nq_gather_qmm_lhs": [_P, _I32, _I64, _I64, _I64, _I64, _P, _P, _P, _I32, _I64, _I64, _I32, _I32,
                          _P, _P, _I32, _I32, _P, _P, _SZ, _P],
    "nq_qmm_notrans_workspace_bytes": [_I64, _I64, _I64, _I32, _I32, _I32, _I32],
    "nq_qmm_notrans": [_P, _I32, _I64, _I64, _P, _P, _P, _I32, _I64, _I32, _I32, _P, _P, _SZ, _P],
    "nq_qmm_notrans_row_exact": [_P, _I32, _I64, _I64, _P, _P, _P, _I32, _I64, _I32, _I32, _P, _P,
                                 _SZ, _P],
    "nq_qmm_grad_scales_biases": [_P, _P, _I32, _I64, _I64, _P, _I64, _I32, _I32, _P, _P, _I32, _P],
    "nq_fp_quantize": [_P, _I32, _I64, _I64, _I32, _P, _P, _P],
    "nq_fp_dequantize": [_P, _P, _I64, _I64, _I32, _P, _I32, _P],
    "nq_fp_qmm": [_P, _I32, _I64, _I64, _P, _P, _P, _I64, _I32, _I32, _P, _P],
    "nq_fp_gather_qmm_workspace_bytes": [_I64, _I64, _I64, _I64, _I64],
    "nq_fp_gather_qmm": [_P, _I32, _I64, _I64, _I64, _P, _P, _P, _I64, _I64, _I32, _P, _I32, _P, _P,
                         _SZ, _P],
    "nq_fp_qmm_notrans_workspace_bytes": [_I64, _I64, _I64, _I32, _I32, _I32],
    "nq_fp_qmm_notrans": [_P, _I32, _I64, _I64, _P, _P, _P, _I64, _I32, _I32, _P, _P, _SZ, _P],
    "nq_status_string": [_I32],
    "nq_last_error": [],
    "nq_version": [],
}
_RESTYPES = {"nq_qmm_workspace_bytes": _SZ, "nq_gather_qmm_workspace_bytes": _SZ,
             "nq_qmm_notrans_workspace_bytes": _SZ, "nq_fp_gather_qmm_workspace_bytes": _SZ,
             "nq_fp_qmm_notrans_workspace_bytes": _SZ,
             "nq_status_string": ctypes.c_char_p, "nq_last_error": ctypes.c_char_p,
             "nq_version": ctypes.c_char_p}


def load_library(path=None):
    """Loads libnq.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    path = path or library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m group_wise_affine_quantize_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(path)
    for name, args in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = _RESTYPES.get(name, ctypes.c_int)
    _lib = lib
    return lib


def _check(status):
    if status != 0:
        lib = load_library()
        raise NQError(status, lib.nq_last_error().decode())


def _torch():
    import torch
    return torch


def _dt(t):
    torch = _torch()
    if t.dtype == torch.float32:
        return NQ_F32
    if t.dtype == torch.bfloat16:
        return NQ_BF16
    raise TypeError(f"libnq takes float32 or bfloat16 tensors, got {t.dtype}")


def _torch_dtype(dt):
    torch = _torch()
    return torch.float32 if dt == NQ_F32 else torch.bfloat16


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _empty(stream, shape, dtype, device):
    """A new output or workspace tensor.  With a caller's stream it is
    allocated under that stream, so the caching allocator ties the memory to
    the stream the kernels run on and does not hand it to other work while
    they may still use it."""
    torch = _torch()
    if stream is None:
        return torch.empty(shape, dtype=dtype, device=device)
    with torch.cuda.stream(stream):
        return torch.empty(shape, dtype=dtype, device=device)


def _contig(name, t):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def words_per_row(k, bits):
    return k * bits // 32


def nq_quantize(w, group_size, bits, codes=None, scales=None, biases=None, stream=None):
    """w [..., k] (f32 or bf16) -> (codes uint32-as-int32 [..., k*bits/32],
    scales [..., k/gs], biases [..., k/gs]) in w's dtype."""
    torch = _torch()
    lib = load_library()
    _contig("w", w)
    k = w.shape[-1]
    n = w.numel() // k if k else 0
    lead = tuple(w.shape[:-1])
    if codes is None:
        codes = _empty(stream, lead + (words_per_row(k, bits),), torch.int32, w.device)
    if scales is None:
        scales = _empty(stream, lead + (k // group_size if group_size else 0,), w.dtype, w.device)
    if biases is None:
        biases = _empty(stream, scales.shape, scales.dtype, scales.device)
    _check(lib.nq_quantize(_ptr(w), _dt(w), n, k, group_size, bits, _ptr(codes), _ptr(scales),
                           _ptr(biases), _stream(stream)))
    return codes, scales, biases


def nq_dequantize(codes, scales, biases, group_size, bits, out_dtype=None, out=None, stream=None):
    """-> w_hat [..., k] in out_dtype (default: the scales' dtype)."""
    torch = _torch()
    lib = load_library()
    for name, t in (("codes", codes), ("scales", scales), ("biases", biases)):
        _contig(name, t)
    k = scales.shape[-1] * group_size
    n = scales.numel() // scales.shape[-1] if scales.shape[-1] else 0
    out_dtype = out_dtype or scales.dtype
    if out is None:
        out = _empty(stream, tuple(scales.shape[:-1]) + (k,), out_dtype, scales.device)
    _check(lib.nq_dequantize(_ptr(codes), _ptr(scales), _ptr(biases), _dt(scales), n, k,
                             group_size, bits, _ptr(out), _dt(out), _stream(stream)))
    return out


def nq_qmm_plan(m, n, k, group_size, bits, x_dtype, sb_dtype, row_exact=False):
    torch = _torch()
    lib = load_library()
    plan = Plan()
    xd = NQ_F32 if x_dtype == torch.float32 else NQ_BF16
    sd = NQ_F32 if sb_dtype == torch.float32 else NQ_BF16
    _check(lib.nq_qmm_plan(m, n, k, group_size, bits, xd, sd, int(bool(row_exact)),
                           ctypes.byref(plan)))
    return plan


def nq_qmm_workspace_bytes(m, n, k, group_size, bits, x_dtype, sb_dtype, row_exact=False):
    torch = _torch()
    xd = NQ_F32 if x_dtype == torch.float32 else NQ_BF16
    sd = NQ_F32 if sb_dtype == torch.float32 else NQ_BF16
    return load_library().nq_qmm_workspace_bytes(m, n, k, group_size, bits, xd, sd,
                                                 int(bool(row_exact)))


def _qmm_call(entry, x, codes, scales, biases, group_size, bits, y, workspace, stream, plan=None):
    torch = _torch()
    lib = load_library()
    for name, t in (("x", x), ("codes", codes), ("scales", scales), ("biases", biases)):
        _contig(name, t)
    m, k = x.shape
    n = scales.shape[0]
    if scales.shape[1] * group_size != k or codes.shape != (n, words_per_row(k, bits)):
        raise ValueError("codes/scales shapes do not match x and the quantization")
    if y is None:
        y = _empty(stream, (m, n), x.dtype, x.device)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    args = [_ptr(x), _dt(x), m, k, _ptr(codes), _ptr(scales), _ptr(biases), _dt(scales), n,
            group_size, bits, _ptr(y), _ptr(workspace), ws_bytes, _stream(stream)]
    if plan is not None:
        _check(lib.nq_qmm_with_plan(ctypes.byref(plan), *args))
    else:
        _check(getattr(lib, entry)(*args))
    return y


def nq_qmm(x, codes, scales, biases, group_size, bits, y=None, workspace=None, stream=None):
    """y [m, n] = x [m, k] times the transposed dequantized weights, in x's dtype."""
    return _qmm_call("nq_qmm", x, codes, scales, biases, group_size, bits, y, workspace, stream)


def nq_qmm_row_exact(x, codes, scales, biases, group_size, bits, y=None, workspace=None,
                     stream=None):
    """nq_qmm whose every row is bit-equal to the one-row product."""
    return _qmm_call("nq_qmm_row_exact", x, codes, scales, biases, group_size, bits, y,
                     workspace, stream)


def nq_qmm_with_plan(plan, x, codes, scales, biases, group_size, bits, y=None, workspace=None,
                     stream=None):
    return _qmm_call(None, x, codes, scales, biases, group_size, bits, y, workspace, stream,
                     plan=plan)


def nq_qmm_batched(x, codes, scales, biases, group_size, bits, y=None, workspace=None,
                   stream=None):
    """x [batch, l, k] -> y [batch, l, n]: item i bit-equal to nq_qmm(x[i])."""
    torch = _torch()
    lib = load_library()
    for name, t in (("x", x), ("codes", codes), ("scales", scales), ("biases", biases)):
        _contig(name, t)
    batch, l, k = x.shape
    n = scales.shape[0]
    if scales.shape[1] * group_size != k or codes.shape != (n, words_per_row(k, bits)):
        raise ValueError("codes/scales shapes do not match x and the quantization")
    if y is None:
        y = _empty(stream, (batch, l, n), x.dtype, x.device)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.nq_qmm_batched(_ptr(x), _dt(x), batch, l, k, _ptr(codes), _ptr(scales),
                              _ptr(biases), _dt(scales), n, group_size, bits, _ptr(y),
                              _ptr(workspace), ws_bytes, _stream(stream)))
    return y


def nq_qmm_notrans_workspace_bytes(m, ni, nc, group_size, bits, x_dtype, row_exact=False):
    torch = _torch()
    xd = NQ_F32 if x_dtype == torch.float32 else NQ_BF16
    return load_library().nq_qmm_notrans_workspace_bytes(m, ni, nc, group_size, bits, xd,
                                                         int(bool(row_exact)))


def _notrans_call(entry, x, codes, scales, biases, group_size, bits, y, workspace, stream):
    torch = _torch()
    lib = load_library()
    for name, t in (("x", x), ("codes", codes), ("scales", scales), ("biases", biases)):
        _contig(name, t)
    m, ni = x.shape
    nc = scales.shape[1] * group_size
    if scales.shape[0] != ni or codes.shape != (ni, words_per_row(nc, bits)):
        raise ValueError("codes/scales shapes do not match x and the quantization")
    if y is None:
        y = _empty(stream, (m, nc), x.dtype, x.device)
    if workspace is None:
        need = lib.nq_qmm_notrans_workspace_bytes(m, ni, nc, group_size, bits, _dt(x),
                                                  int(entry.endswith("row_exact")))
        if need:
            workspace = _empty(stream, need, torch.uint8, x.device)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(getattr(lib, entry)(_ptr(x), _dt(x), m, ni, _ptr(codes), _ptr(scales), _ptr(biases),
                               _dt(scales), nc, group_size, bits, _ptr(y), _ptr(workspace),
                               ws_bytes, _stream(stream)))
    return y


def nq_qmm_notrans(x, codes, scales, biases, group_size, bits, y=None, workspace=None, stream=None):
    """y [m, nc] = x [m, ni] times the dequantized weights as stored ([ni, nc],
    grouped along nc): the transpose = false product.  With the forward
    weights and x = dy it is the derivative for the activations."""
    return _notrans_call("nq_qmm_notrans", x, codes, scales, biases, group_size, bits, y, workspace,
                         stream)


def nq_qmm_notrans_row_exact(x, codes, scales, biases, group_size, bits, y=None, workspace=None,
                             stream=None):
    """nq_qmm_notrans whose every row is bit-equal to the one-row product."""
    return _notrans_call("nq_qmm_notrans_row_exact", x, codes, scales, biases, group_size, bits, y,
                         workspace, stream)


def nq_qmm_grad_scales_biases(x, dy, codes, group_size, bits, out_dtype=None, dscales=None,
                              dbiases=None, stream=None):
    """Derivatives of sum(dy * nq_qmm(x, w)) for w's scales and biases:
    x [m, k], dy [m, n] (same dtype), codes [n, k*bits/32] -> (dscales,
    dbiases) [n, k/gs] in out_dtype (default: x's dtype)."""
    torch = _torch()
    lib = load_library()
    for name, t in (("x", x), ("dy", dy), ("codes", codes)):
        _contig(name, t)
    m, k = x.shape
    n = dy.shape[1]
    if dy.shape[0] != m or dy.dtype != x.dtype or codes.shape != (n, words_per_row(k, bits)):
        raise ValueError("x, dy and codes do not match")
    od = out_dtype or x.dtype
    if dscales is None:
        dscales = _empty(stream, (n, k // group_size), od, x.device)
    if dbiases is None:
        dbiases = _empty(stream, (n, k // group_size), od, x.device)
    _check(lib.nq_qmm_grad_scales_biases(_ptr(x), _ptr(dy), _dt(x), m, k, _ptr(codes), n, group_size,
                                         bits, _ptr(dscales), _ptr(dbiases), _dt(dscales),
                                         _stream(stream)))
    return dscales, dbiases


def nq_gather_qmm_workspace_bytes(rows, l, k, e, n, group_size, bits, x_dtype, sb_dtype,
                                  sorted_hint=False):
    torch = _torch()
    xd = NQ_F32 if x_dtype == torch.float32 else NQ_BF16
    sd = NQ_F32 if sb_dtype == torch.float32 else NQ_BF16
    return load_library().nq_gather_qmm_workspace_bytes(rows, l, k, e, n, group_size, bits, xd,
                                                        sd, int(bool(sorted_hint)))


def _gather_call(entry, x, codes, scales, biases, group_size, bits, rhs_idx, sorted_hint, y,
                 workspace, stream):
    torch = _torch()
    lib = load_library()
    for name, t in (("x", x), ("codes", codes), ("scales", scales), ("biases", biases),
                    ("rhs_idx", rhs_idx)):
        _contig(name, t)
    if rhs_idx.element_size() != 4:
        raise ValueError("rhs_idx must hold 32-bit ids")
    rows, l, k = x.shape
    e, n = scales.shape[0], scales.shape[1]
    if rhs_idx.numel() != rows:
        raise ValueError("rhs_idx must have one id per row")
    if y is None:
        y = _empty(stream, (rows, l, n), x.dtype, x.device)
    if workspace is None:
        need = lib.nq_gather_qmm_workspace_bytes(rows, l, k, e, n, group_size, bits, _dt(x),
                                                 _dt(scales), int(bool(sorted_hint)))
        if need:
            workspace = _empty(stream, need, torch.uint8, x.device)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(getattr(lib, entry)(_ptr(x), _dt(x), rows, l, k, _ptr(codes), _ptr(scales),
                               _ptr(biases), _dt(scales), e, n, group_size, bits, _ptr(rhs_idx),
                               int(bool(sorted_hint)), _ptr(y), _ptr(workspace), ws_bytes,
                               _stream(stream)))
    return y


def nq_gather_qmm(x, codes, scales, biases, group_size, bits, rhs_idx, sorted_hint=False, y=None,
                  workspace=None, stream=None):
    """x [rows, l, k]; codes [e, n, k*bits/32]; scales/biases [e, n, k/gs];
    rhs_idx [rows] (int32/uint32 bit patterns) -> y [rows, l, n] in x's dtype.
    A workspace is allocated when the call needs one and none is given."""
    return _gather_call("nq_gather_qmm", x, codes, scales, biases, group_size, bits, rhs_idx,
                        sorted_hint, y, workspace, stream)


def nq_gather_qmm_noalloc(x, codes, scales, biases, group_size, bits, rhs_idx, sorted_hint=False, y=None,
                          stream=None):
    """nq_gather_qmm with the grouping tables in the library's static device
    array: no workspace argument, and nothing allocated by the library (y is
    allocated here only when not given)."""
    lib = load_library()
    for name, t in (("x", x), ("codes", codes), ("scales", scales), ("biases", biases),
                    ("rhs_idx", rhs_idx)):
        _contig(name, t)
    if rhs_idx.element_size() != 4:
        raise ValueError("rhs_idx must hold 32-bit ids")
    rows, l, k = x.shape
    e, n = scales.shape[0], scales.shape[1]
    if rhs_idx.numel() != rows:
        raise ValueError("rhs_idx must have one id per row")
    if y is None:
        y = _empty(stream, (rows, l, n), x.dtype, x.device)
    _check(lib.nq_gather_qmm_noalloc(_ptr(x), _dt(x), rows, l, k, _ptr(codes), _ptr(scales), _ptr(biases),
                                     _dt(scales), e, n, group_size, bits, _ptr(rhs_idx), int(bool(sorted_hint)),
                                     _ptr(y), _stream(stream)))
    return y


def nq_gather_qmm_row_exact(x, codes, scales, biases, group_size, bits, rhs_idx, sorted_hint=False,
                            y=None, workspace=None, stream=None):
    """As nq_gather_qmm, every row bit-equal to its one-row product."""
    return _gather_call("nq_gather_qmm_row_exact", x, codes, scales, biases, group_size, bits,
                        rhs_idx, sorted_hint, y, workspace, stream)


def nq_gather_qmm_lhs(x, codes, scales, biases, group_size, bits, lhs_idx, rhs_idx,
                      sorted_hint=False, row_exact=False, y=None, workspace=None, stream=None):
    """x [x_items, l, k]; lhs_idx and rhs_idx [rows] (32-bit ids): row r of
    y [rows, l, n] is x[lhs_idx[r]] times expert rhs_idx[r]'s weights; an id
    past x_items or e gives a zero row."""
    torch = _torch()
    lib = load_library()
    for name, t in (("x", x), ("codes", codes), ("scales", scales), ("biases", biases),
                    ("lhs_idx", lhs_idx), ("rhs_idx", rhs_idx)):
        _contig(name, t)
    if lhs_idx.element_size() != 4 or rhs_idx.element_size() != 4:
        raise ValueError("lhs_idx and rhs_idx must hold 32-bit ids")
    x_items, l, k = x.shape
    e, n = scales.shape[0], scales.shape[1]
    rows = rhs_idx.numel()
    if lhs_idx.numel() != rows:
        raise ValueError("lhs_idx and rhs_idx must have one id per output row")
    if y is None:
        y = _empty(stream, (rows, l, n), x.dtype, x.device)
    if workspace is None:
        need = lib.nq_gather_qmm_workspace_bytes(rows, l, k, e, n, group_size, bits, _dt(x),
                                                 _dt(scales), int(bool(sorted_hint)))
        if need:
            workspace = _empty(stream, need, torch.uint8, x.device)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.nq_gather_qmm_lhs(_ptr(x), _dt(x), x_items, rows, l, k, _ptr(codes), _ptr(scales),
                                 _ptr(biases), _dt(scales), e, n, group_size, bits, _ptr(lhs_idx),
                                 _ptr(rhs_idx), int(bool(sorted_hint)), int(bool(row_exact)),
                                 _ptr(y), _ptr(workspace), ws_bytes, _stream(stream)))
    return y


# ---------------------------------------------------------------- floating-point modes
def _fp(mode):
    if mode not in FP_MODES:
        raise ValueError(f"unknown floating-point mode {mode!r} (one of {sorted(FP_MODES)})")
    return FP_MODES[mode]


def nq_fp_quantize(w, mode, codes=None, scales=None, stream=None):
    """w [..., k] (f32 or bf16) -> (codes uint32-as-int32 [..., k*bits/32],
    scales uint8 [..., k/group]) in mode "mxfp4", "mxfp8" or "nvfp4"."""
    torch = _torch()
    lib = load_library()
    mid, bits, gs = _fp(mode)
    _contig("w", w)
    k = w.shape[-1]
    n = w.numel() // k if k else 0
    lead = tuple(w.shape[:-1])
    if codes is None:
        codes = _empty(stream, lead + (words_per_row(k, bits),), torch.int32, w.device)
    if scales is None:
        scales = _empty(stream, lead + (k // gs,), torch.uint8, w.device)
    _check(lib.nq_fp_quantize(_ptr(w), _dt(w), n, k, mid, _ptr(codes), _ptr(scales), _stream(stream)))
    return codes, scales


def nq_fp_dequantize(codes, scales, mode, out_dtype=None, out=None, stream=None):
    """-> w_hat [..., k] in out_dtype (default bf16)."""
    torch = _torch()
    lib = load_library()
    mid, bits, gs = _fp(mode)
    for name, t in (("codes", codes), ("scales", scales)):
        _contig(name, t)
    k = scales.shape[-1] * gs
    n = scales.numel() // scales.shape[-1] if scales.shape[-1] else 0
    if out is None:
        out = _empty(stream, tuple(scales.shape[:-1]) + (k,), out_dtype or torch.bfloat16, scales.device)
    _check(lib.nq_fp_dequantize(_ptr(codes), _ptr(scales), n, k, mid, _ptr(out), _dt(out),
                                _stream(stream)))
    return out


def nq_fp_qmm(x, codes, scales, mode, global_scale=None, row_exact=False, y=None, stream=None):
    """y [m, n] = x [m, k] times the transposed weights (times the fp32 global
    scale, a one-element GPU tensor, NVFP4 only), in x's dtype."""
    torch = _torch()
    lib = load_library()
    mid, bits, gs = _fp(mode)
    for name, t in (("x", x), ("codes", codes), ("scales", scales)):
        _contig(name, t)
    m, k = x.shape
    n = scales.shape[0]
    if scales.shape[1] * gs != k or codes.shape != (n, words_per_row(k, bits)):
        raise ValueError("codes/scales shapes do not match x and the mode")
    if y is None:
        y = _empty(stream, (m, n), x.dtype, x.device)
    _check(lib.nq_fp_qmm(_ptr(x), _dt(x), m, k, _ptr(codes), _ptr(scales), _ptr(global_scale), n, mid,
                         int(bool(row_exact)), _ptr(y), _stream(stream)))
    return y


def nq_fp_gather_qmm_workspace_bytes(rows, l, k, e, n):
    return load_library().nq_fp_gather_qmm_workspace_bytes(rows, l, k, e, n)


def nq_fp_gather_qmm(x, codes, scales, mode, rhs_idx, global_scales=None, row_exact=False, y=None,
                     workspace=None, stream=None):
    """x [rows, l, k], stacked experts codes [e, n, words] and scales [e, n,
    groups], rhs_idx [rows] (uint32 as int32), optional per-expert fp32 global
    scales [e] (NVFP4) -> y [rows, l, n]; row_exact keeps every row's
    one-row bits.  The workspace (bytes from nq_fp_gather_qmm_workspace_bytes)
    is allocated here when not given."""
    torch = _torch()
    lib = load_library()
    mid, bits, gs = _fp(mode)
    for name, t in (("x", x), ("codes", codes), ("scales", scales), ("rhs_idx", rhs_idx)):
        _contig(name, t)
    rows, l, k = x.shape
    e, n = scales.shape[0], scales.shape[1]
    if scales.shape[2] * gs != k or codes.shape != (e, n, words_per_row(k, bits)):
        raise ValueError("codes/scales shapes do not match x and the mode")
    if rhs_idx.numel() != rows:
        raise ValueError("rhs_idx must hold one expert per row")
    if y is None:
        y = _empty(stream, (rows, l, n), x.dtype, x.device)
    if workspace is None:
        need = lib.nq_fp_gather_qmm_workspace_bytes(rows, l, k, e, n)
        workspace = _empty(stream, need, torch.uint8, x.device) if need else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.nq_fp_gather_qmm(_ptr(x), _dt(x), rows, l, k, _ptr(codes), _ptr(scales),
                                _ptr(global_scales), e, n, mid, _ptr(rhs_idx), int(bool(row_exact)), _ptr(y),
                                _ptr(workspace), ws_bytes, _stream(stream)))
    return y


def nq_fp_qmm_notrans_workspace_bytes(m, ni, nc, mode, x_dtype, row_exact=False):
    torch = _torch()
    xd = NQ_F32 if x_dtype == torch.float32 else NQ_BF16
    return load_library().nq_fp_qmm_notrans_workspace_bytes(m, ni, nc, _fp(mode)[0], xd,
                                                            int(bool(row_exact)))


def nq_fp_qmm_notrans(x, codes, scales, mode, global_scale=None, row_exact=False, y=None, workspace=None,
                      stream=None):
    """y [m, nc] = x [m, ni] times the quantized matrix [ni, nc] as stored
    (codes [ni, nc*bits/32], scales [ni, nc/group]); with the forward weights
    this is the derivative for the activations.  The workspace is allocated
    here when not given."""
    torch = _torch()
    lib = load_library()
    mid, bits, gs = _fp(mode)
    for name, t in (("x", x), ("codes", codes), ("scales", scales)):
        _contig(name, t)
    m, ni = x.shape
    nc = scales.shape[1] * gs
    if scales.shape[0] != ni or codes.shape != (ni, words_per_row(nc, bits)):
        raise ValueError("codes/scales shapes do not match x and the mode")
    if y is None:
        y = _empty(stream, (m, nc), x.dtype, x.device)
    if workspace is None:
        need = lib.nq_fp_qmm_notrans_workspace_bytes(m, ni, nc, mid, _dt(x), int(bool(row_exact)))
        workspace = _empty(stream, need, torch.uint8, x.device) if need else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.nq_fp_qmm_notrans(_ptr(x), _dt(x), m, ni, _ptr(codes), _ptr(scales), _ptr(global_scale), nc,
                                 mid, int(bool(row_exact)), _ptr(y), _ptr(workspace), ws_bytes,
                                 _stream(stream)))
    return y

