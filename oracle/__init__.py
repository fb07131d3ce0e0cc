"""CPU oracle for group-wise affine quantization -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The GPU library does not depend on it in any way.

Thin numpy wrappers around nq_oracle.c (see that file for the readings of the
"Quantization" page of the nuvec documentation that it follows).  The
floating-point modes (MXFP4, MXFP8, NVFP4) are in the numpy module fp.py.  bf16 arrays
are passed as numpy uint16 bit patterns.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# NQ_ORACLE_LIB selects another build of the same source (the sanitizer build)
_LIB_PATH = os.environ.get("NQ_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16 = 0, 1
_c_i64 = ctypes.c_int64
_c_int = ctypes.c_int
_c_p = ctypes.c_void_p


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(_LIB_PATH)
        L.oracle_quantize.argtypes = [_c_p, _c_int, _c_i64, _c_i64, _c_int, _c_int, _c_p, _c_p, _c_p]
        L.oracle_dequantize.argtypes = [_c_p, _c_p, _c_p, _c_int, _c_i64, _c_i64, _c_int, _c_int,
                                        _c_p, _c_int]
        L.oracle_dequantize_f64.argtypes = [_c_p, _c_p, _c_p, _c_int, _c_i64, _c_i64, _c_int,
                                            _c_int, _c_p]
        L.oracle_qmm_f64.argtypes = [_c_p, _c_int, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_int,
                                     _c_i64, _c_int, _c_int, _c_p]
        L.oracle_qmm_sample_f64.argtypes = [_c_p, _c_int, _c_i64, _c_p, _c_p, _c_p, _c_int, _c_int,
                                            _c_int, _c_p, _c_p, _c_i64, _c_p]
        L.oracle_gather_qmm_f64.argtypes = [_c_p, _c_int, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_p,
                                            _c_int, _c_i64, _c_i64, _c_int, _c_int, _c_p, _c_p]
        L.oracle_qmm_nt_f64.argtypes = [_c_p, _c_int, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_int,
                                        _c_i64, _c_int, _c_int, _c_p]
        L.oracle_qmm_grad_sb_f64.argtypes = [_c_p, _c_int, _c_p, _c_int, _c_i64, _c_i64, _c_p,
                                             _c_i64, _c_int, _c_int, _c_p, _c_p]
        L.oracle_gather_qmm_lhs_f64.argtypes = [_c_p, _c_int, _c_i64, _c_i64, _c_i64, _c_i64, _c_p,
                                                _c_p, _c_p, _c_int, _c_i64, _c_i64, _c_int, _c_int,
                                                _c_p, _c_p, _c_p]
        L.oracle_bf16_round.argtypes = [_c_p, _c_p, _c_i64]
        for f in ("oracle_quantize", "oracle_dequantize", "oracle_dequantize_f64",
                  "oracle_qmm_f64", "oracle_qmm_sample_f64", "oracle_gather_qmm_f64",
                  "oracle_qmm_nt_f64", "oracle_qmm_grad_sb_f64", "oracle_gather_qmm_lhs_f64",
                  "oracle_bits_supported", "oracle_group_supported", "oracle_threads"):
            getattr(L, f).restype = _c_int
        L.oracle_bf16_round.restype = None
        _lib = L
    return _lib


def _dt(a):
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"oracle takes float32 or uint16 (bf16 bits), got {a.dtype}")


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a):
    return np.ascontiguousarray(a)


def threads():
    """OpenMP threads the oracle's loops use."""
    return int(lib().oracle_threads())


def bf16_round(a):
    """float32 array -> uint16 bf16 bit patterns, round to nearest even."""
    a = _c(np.asarray(a, dtype=np.float32))
    out = np.empty(a.shape, dtype=np.uint16)
    lib().oracle_bf16_round(_ptr(a), _ptr(out), a.size)
    return out


def bf16_to_f32(h):
    """uint16 bf16 bit patterns -> float32 values (exact)."""
    h = np.asarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32)


def words_per_row(k, bits):
    return k * bits // 32


def quantize(w, group_size, bits):
    """w: [..., k] float32 or bf16 bits -> (codes uint32 [..., k*bits/32],
    scales [..., k/gs], biases [..., k/gs]) with scales and biases in w's dtype."""
    w = _c(w)
    k = w.shape[-1]
    n = w.size // k if k else 0
    if k % group_size:
        raise ValueError("k must be a multiple of group_size")
    codes = np.zeros(w.shape[:-1] + (words_per_row(k, bits),), dtype=np.uint32)
    scales = np.zeros(w.shape[:-1] + (k // group_size,), dtype=w.dtype)
    biases = np.zeros_like(scales)
    rc = lib().oracle_quantize(_ptr(w), _dt(w), n, k, group_size, bits, _ptr(codes),
                               _ptr(scales), _ptr(biases))
    if rc:
        raise ValueError(f"oracle_quantize rejected gs={group_size} bits={bits}")
    return codes, scales, biases


def dequantize(codes, scales, biases, group_size, bits, out_dtype=None):
    """The stand-alone dequantize contract; out_dtype defaults to the scales'."""
    codes, scales, biases = _c(codes), _c(scales), _c(biases)
    k = scales.shape[-1] * group_size
    n = scales.size // scales.shape[-1] if scales.shape[-1] else 0
    out_dtype = np.dtype(out_dtype or scales.dtype)
    out = np.zeros(scales.shape[:-1] + (k,), dtype=out_dtype)
    rc = lib().oracle_dequantize(_ptr(codes), _ptr(scales), _ptr(biases), _dt(scales), n, k,
                                 group_size, bits, _ptr(out), _dt(out))
    if rc:
        raise ValueError("oracle_dequantize rejected its arguments")
    return out


def dequantize_f64(codes, scales, biases, group_size, bits):
    codes, scales, biases = _c(codes), _c(scales), _c(biases)
    k = scales.shape[-1] * group_size
    n = scales.size // scales.shape[-1] if scales.shape[-1] else 0
    out = np.zeros(scales.shape[:-1] + (k,), dtype=np.float64)
    rc = lib().oracle_dequantize_f64(_ptr(codes), _ptr(scales), _ptr(biases), _dt(scales), n, k,
                                     group_size, bits, _ptr(out))
    if rc:
        raise ValueError("oracle_dequantize_f64 rejected its arguments")
    return out


def qmm_f64(x, codes, scales, biases, group_size, bits):
    """x [m, k] (float32 or bf16 bits) times the transposed dequantized
    weights [n, k] -> y [m, n] float64."""
    x, codes, scales, biases = _c(x), _c(codes), _c(scales), _c(biases)
    m, k = x.shape
    n = scales.shape[0]
    assert scales.shape[1] * group_size == k
    y = np.zeros((m, n), dtype=np.float64)
    rc = lib().oracle_qmm_f64(_ptr(x), _dt(x), m, k, _ptr(codes), _ptr(scales), _ptr(biases),
                              _dt(scales), n, group_size, bits, _ptr(y))
    if rc:
        raise ValueError(f"oracle_qmm_f64 failed ({rc})")
    return y


def qmm_sample_f64(x, codes, scales, biases, group_size, bits, ms, ns):
    """y[ms[i], ns[i]] of qmm_f64, computed one output at a time."""
    x, codes, scales, biases = _c(x), _c(codes), _c(scales), _c(biases)
    k = x.shape[-1]
    ms = _c(np.asarray(ms, dtype=np.int64))
    ns = _c(np.asarray(ns, dtype=np.int64))
    assert ms.shape == ns.shape
    out = np.zeros(ms.shape, dtype=np.float64)
    rc = lib().oracle_qmm_sample_f64(_ptr(x), _dt(x), k, _ptr(codes), _ptr(scales), _ptr(biases),
                                     _dt(scales), group_size, bits, _ptr(ms), _ptr(ns), ms.size,
                                     _ptr(out))
    if rc:
        raise ValueError("oracle_qmm_sample_f64 rejected its arguments")
    return out


def gather_qmm_f64(x, codes, scales, biases, group_size, bits, idx):
    """x [rows, l, k]; codes [e, n, k*bits/32]; scales/biases [e, n, k/gs];
    idx [rows] uint32 -> y [rows, l, n] float64 (zero rows for ids >= e)."""
    x, codes, scales, biases = _c(x), _c(codes), _c(scales), _c(biases)
    idx = _c(np.asarray(idx, dtype=np.uint32))
    rows, l, k = x.shape
    e, n = scales.shape[0], scales.shape[1]
    y = np.zeros((rows, l, n), dtype=np.float64)
    rc = lib().oracle_gather_qmm_f64(_ptr(x), _dt(x), rows, l, k, _ptr(codes), _ptr(scales),
                                     _ptr(biases), _dt(scales), e, n, group_size, bits,
                                     _ptr(idx), _ptr(y))
    if rc:
        raise ValueError("oracle_gather_qmm_f64 rejected its arguments")
    return y


def qmm_nt_f64(x, codes, scales, biases, group_size, bits):
    """x [m, ni] times the dequantized weights as stored, [ni, nc] (grouped
    along nc) -> y [m, nc] float64: the transpose = false product."""
    x, codes, scales, biases = _c(x), _c(codes), _c(scales), _c(biases)
    m, ni = x.shape
    assert scales.shape[0] == ni
    nc = scales.shape[1] * group_size
    y = np.zeros((m, nc), dtype=np.float64)
    rc = lib().oracle_qmm_nt_f64(_ptr(x), _dt(x), m, ni, _ptr(codes), _ptr(scales), _ptr(biases),
                                 _dt(scales), nc, group_size, bits, _ptr(y))
    if rc:
        raise ValueError("oracle_qmm_nt_f64 rejected its arguments")
    return y


def qmm_grad_sb_f64(x, dy, codes, group_size, bits):
    """Derivatives of sum(dy * qmm(x, w)) for the scales and biases of w:
    x [m, k], dy [m, n], codes [n, k*bits/32] -> (ds, db) [n, k/gs] float64."""
    x, dy, codes = _c(x), _c(dy), _c(codes)
    m, k = x.shape
    n = dy.shape[1]
    assert dy.shape[0] == m and codes.shape[0] == n
    ds = np.zeros((n, k // group_size), dtype=np.float64)
    db = np.zeros_like(ds)
    rc = lib().oracle_qmm_grad_sb_f64(_ptr(x), _dt(x), _ptr(dy), _dt(dy), m, k, _ptr(codes), n,
                                      group_size, bits, _ptr(ds), _ptr(db))
    if rc:
        raise ValueError("oracle_qmm_grad_sb_f64 rejected its arguments")
    return ds, db


def gather_qmm_lhs_f64(x, codes, scales, biases, group_size, bits, lhs, rhs):
    """x [b, l, k]; lhs [rows] (x item per output row, or None for the
    identity) and rhs [rows] (expert) -> y [rows, l, n] float64."""
    x, codes, scales, biases = _c(x), _c(codes), _c(scales), _c(biases)
    rhs = _c(np.asarray(rhs, dtype=np.uint32))
    lhs_p = None
    if lhs is not None:
        lhs = _c(np.asarray(lhs, dtype=np.uint32))
        assert lhs.shape == rhs.shape
        lhs_p = _ptr(lhs)
    b, l, k = x.shape
    rows = rhs.shape[0]
    e, n = scales.shape[0], scales.shape[1]
    y = np.zeros((rows, l, n), dtype=np.float64)
    rc = lib().oracle_gather_qmm_lhs_f64(_ptr(x), _dt(x), b, rows, l, k, _ptr(codes), _ptr(scales),
                                         _ptr(biases), _dt(scales), e, n, group_size, bits, lhs_p,
                                         _ptr(rhs), _ptr(y))
    if rc:
        raise ValueError("oracle_gather_qmm_lhs_f64 rejected its arguments")
    return y
