"""CPU oracle for the floating-point quantization modes MXFP4, MXFP8 and
NVFP4 -- TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and
the benchmark's CPU-baseline leg may import it; the GPU library does not
depend on it in any way.

What the "Quantization" page of the nuvec documentation fixes (sections
"Floating-point formats" and "Mixture of experts"): every weight is stored as
a small float, each group of a row shares one scale stored as a uint8 code,
there are no biases, the codes are packed into uint32 words like the affine
codes, dequantize gives bfloat16, a product comes out in x's dtype, and NVFP4
experts may carry one float32 global scale each.

The element and scale encodings are not on that page.  They are the public
definitions of the formats the mode names stand for:
  - MXFP4 and MXFP8 (OCP Microscaling Formats (MX) Specification v1.0,
    sections 5.1-5.3): blocks of 32 elements sharing one E8M0 scale, whose
    code s means 2^(s - 127) (s = 255: NaN); the elements are FP4 E2M1
    (MXFP4) or FP8 E4M3 (MXFP8; the OCP 8-bit float, "E4M3" with no
    infinities and NaN at S.1111.111).
  - NVFP4: blocks of 16 E2M1 elements sharing one FP8 E4M3 scale (an unsigned
    use of the E4M3 code), and optionally one fp32 scale per tensor, or per
    expert of a gathered product, multiplying every weight.

Quantize is a reading, not a pinned copy of the page's library:
  - MX (OCP MX v1.0 section 6.3): the shared exponent is
    floor(log2(max |w| of the block)) minus the largest exponent of the
    element format (2 for E2M1, 8 for E4M3), clamped to the E8M0 range
    (an all-zero block gets code 0); each element is w / 2^X rounded to the
    nearest element value, ties to the even code, saturating at the largest
    magnitude.
  - NVFP4: the scale code is fp32(max |w| / 6) rounded to the nearest E4M3
    value (ties to even, saturating at 448); each element is
    fp32(w / scale) rounded to E2M1 as above; a block whose scale rounds to
    zero stores zero codes.
  - A value's sign is kept, also when it rounds to zero (-0.0 stays -0).
  - Non-finite weights are outside the contract.
Every rounding decision is taken on fp32 numbers, as the GPU takes it.

Dequantize and the products are exact definitions: w_hat = g * S * E with
S the decoded scale, E the decoded element and g the global scale (1 when
absent); dequantize rounds w_hat (exact in fp64) to bfloat16 (round to
nearest even) or to fp32, and a NaN comes out as the canonical quiet NaN of
the output type (0x7fc0, 0x7fc00000) whatever the sign of the NaN element;
products are y = x . w_hat^T accumulated in fp64.
"""
import numpy as np

# mode name -> (C enum value, element format, bits per code, group size, scale format)
MODES = {
    "mxfp4": (1, "e2m1", 4, 32, "e8m0"),
    "mxfp8": (2, "e4m3", 8, 32, "e8m0"),
    "nvfp4": (3, "e2m1", 4, 16, "e4m3"),
}
MODE_IDS = {name: v[0] for name, v in MODES.items()}


def mode_info(mode):
    """(element format, bits, group size, scale format) of a mode name."""
    _, elem, bits, gs, scale = MODES[mode]
    return elem, bits, gs, scale


# ------------------------------------------------------------- the formats
def _minifloat_table(ebits, mbits, bias, e4m3_nan):
    """float64 value of every code of a sign / exponent / mantissa float with
    subnormals (exponent field 0 means 2^(1 - bias) * m / 2^mbits)."""
    n = 1 << (1 + ebits + mbits)
    out = np.empty(n, np.float64)
    for c in range(n):
        s = (c >> (ebits + mbits)) & 1
        e = (c >> mbits) & ((1 << ebits) - 1)
        m = c & ((1 << mbits) - 1)
        if e == 0:
            mag = np.ldexp(m / (1 << mbits), 1 - bias)
        else:
            mag = np.ldexp(1.0 + m / (1 << mbits), e - bias)
        if e4m3_nan and e == (1 << ebits) - 1 and m == (1 << mbits) - 1:
            mag = np.nan
        out[c] = -mag if s else mag
    return out


# FP4 E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit; no Inf or NaN.
E2M1 = _minifloat_table(2, 1, 1, False)
# FP8 E4M3: 1 sign, 4 exponent (bias 7), 3 mantissa bits; S.1111.111 is NaN.
E4M3 = _minifloat_table(4, 3, 7, True)
# E8M0: 8-bit exponent, bias 127, no sign and no zero; 0xff is NaN.
E8M0 = np.array([np.nan if c == 255 else np.ldexp(1.0, c - 127) for c in range(256)])

_TABLES = {"e2m1": (E2M1, 3), "e4m3": (E4M3, 7)}   # table, sign bit position
_EMAX = {"e2m1": 2, "e4m3": 8}                     # exponent of the largest value


def _magnitudes(fmt):
    """Non-negative finite values of a format, indexed by code (they increase
    with the code)."""
    table, sbit = _TABLES[fmt]
    mags = table[: 1 << sbit]
    return mags[np.isfinite(mags)]


def round_to_code(v, fmt):
    """Codes of the float32 values v in `fmt`: nearest magnitude, ties to the
    even code, saturating at the largest finite magnitude; the sign bit is
    v's sign bit."""
    v = np.asarray(v, np.float32)
    assert np.all(np.isfinite(v)), "non-finite values are outside the contract"
    mags = _magnitudes(fmt)
    _, sbit = _TABLES[fmt]
    a = np.abs(v).astype(np.float64)
    lo = np.searchsorted(mags, a, side="right") - 1          # mags[lo] <= a
    lo = np.minimum(lo, len(mags) - 1)
    hi = np.minimum(lo + 1, len(mags) - 1)
    mid = (mags[lo] + mags[hi]) / 2                          # exact in fp64
    code = np.where(a < mid, lo, np.where(a > mid, hi, np.where(lo % 2 == 0, lo, hi)))
    code = np.where(lo == len(mags) - 1, lo, code)            # saturation
    return (code | (np.signbit(v).astype(np.int64) << sbit)).astype(np.int64)


def decode(codes, fmt):
    """float64 values of element or scale codes."""
    table = {"e2m1": E2M1, "e4m3": E4M3, "e8m0": E8M0}[fmt]
    return table[np.asarray(codes, np.int64)]


# ------------------------------------------------------------- packing
def pack(codes, bits):
    """[rows, k] codes -> [rows, k * bits / 32] uint32, element j of a row in
    bits [j * bits, (j + 1) * bits) of the row's little-endian bit stream."""
    codes = np.asarray(codes, np.uint64)
    rows, k = codes.shape
    per = 32 // bits
    c = codes.reshape(rows, k // per, per)
    shifts = (np.arange(per, dtype=np.uint64) * np.uint64(bits))
    return np.bitwise_or.reduce(c << shifts, axis=2).astype(np.uint32)


def unpack(words, bits, k):
    """Inverse of pack."""
    words = np.asarray(words, np.uint64)
    per = 32 // bits
    shifts = (np.arange(per, dtype=np.uint64) * np.uint64(bits))
    c = (words[..., None] >> shifts) & np.uint64((1 << bits) - 1)
    return c.reshape(*words.shape[:-1], -1)[..., :k].astype(np.int64)


# ------------------------------------------------------------- bf16
def _as_f32(w):
    """float32 values of a float32 array or of bf16 bit patterns (uint16)."""
    w = np.asarray(w)
    if w.dtype == np.uint16:
        return (w.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return w.astype(np.float32)


def _round_bf16(v64):
    """fp64 values that are exact in fp32 (or overflow it) -> bf16 bit
    patterns, round to nearest even, NaN as 0x7fc0."""
    with np.errstate(over="ignore"):
        f = np.asarray(v64, np.float64).astype(np.float32)
    b = f.view(np.uint32).astype(np.uint64)
    r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)
    return np.where(np.isnan(f), np.uint16(0x7FC0), r)


# ------------------------------------------------------------- quantize
def quantize(w, mode):
    """w [rows, k] (float32, or bf16 bit patterns as uint16) -> (codes
    [rows, k * bits / 32] uint32, scales [rows, k / group] uint8)."""
    elem, bits, gs, scale_fmt = mode_info(mode)
    v = _as_f32(w)
    rows, k = v.shape
    assert k % gs == 0
    g = v.reshape(rows, k // gs, gs)
    amax = np.max(np.abs(g), axis=2)                        # fp32
    if scale_fmt == "e8m0":
        _, e = np.frexp(amax.astype(np.float64))             # amax = f 2^e, f in [0.5, 1)
        s = np.where(amax == 0, 0, np.clip(e - 1 - _EMAX[elem] + 127, 0, 254))
        x_exp = s - 127
        q = np.ldexp(g.astype(np.float64), -x_exp[..., None])   # exact: a power of two
        codes = round_to_code(q.astype(np.float32), elem)
    else:
        sf = (amax / np.float32(6.0)).astype(np.float32)     # IEEE fp32 division
        s = round_to_code(sf, "e4m3")
        S = decode(s, "e4m3").astype(np.float32)
        with np.errstate(divide="ignore", invalid="ignore"):
            q = (g / S[..., None]).astype(np.float32)         # IEEE fp32 division
        q = np.where(S[..., None] == 0, np.float32(0), q)
        codes = round_to_code(q, elem)
        codes = np.where(S[..., None] == 0, 0, codes)
    return pack(codes.reshape(rows, k), bits), s.astype(np.uint8)


# ------------------------------------------------------------- dequantize and products
def dequantize_f64(codes, scales, mode, k, global_scale=None):
    """Exact w_hat = g * S * E as fp64 [rows, k] (codes [.., rows, words],
    scales [.., rows, k / group])."""
    elem, bits, gs, scale_fmt = mode_info(mode)
    E = decode(unpack(codes, bits, k), elem)
    S = decode(scales, scale_fmt)
    w = E * np.repeat(S, gs, axis=-1)
    if global_scale is not None:
        w = w * np.float64(np.float32(global_scale))
    return w


def dequantize(codes, scales, mode, k, out_dtype="bf16"):
    """Stand-alone dequantize: S * E rounded to bf16 (bit patterns, uint16)
    or to float32."""
    w = dequantize_f64(codes, scales, mode, k)
    if out_dtype == "bf16":
        return _round_bf16(w)
    with np.errstate(over="ignore"):
        f = w.astype(np.float32)
    return np.where(np.isnan(f), np.uint32(0x7FC00000).view(np.float32), f)


def qmm_f64(x, codes, scales, mode, global_scale=None):
    """y = x . w_hat^T in fp64; x [m, k] float32 or bf16 bits."""
    xv = _as_f32(x).astype(np.float64)
    w = dequantize_f64(codes, scales, mode, xv.shape[-1], global_scale)
    return xv @ w.T


def gather_qmm_f64(x, codes, scales, mode, idx, global_scales=None):
    """Row r of x [rows, l, k] times the transposed weights of expert idx[r]
    (codes [e, n, words], scales [e, n, groups]); idx[r] >= e gives zeros."""
    xv = _as_f32(x).astype(np.float64)
    e, n = codes.shape[0], codes.shape[1]
    rows, l, k = xv.shape
    y = np.zeros((rows, l, n))
    for r in range(rows):
        ex = int(idx[r])
        if ex >= e:
            continue
        g = None if global_scales is None else global_scales[ex]
        y[r] = xv[r] @ dequantize_f64(codes[ex], scales[ex], mode, k, g).T
    return y


def qmm_nt_f64(x, codes, scales, mode, global_scale=None):
    """Product with the weights as stored ("transpose = false"): y = x .
    w_hat for a quantized matrix w_hat [ni, nc] whose groups run along nc
    (codes [ni, nc * bits / 32], scales [ni, nc / group]); x [m, ni].  With
    the forward weights this is the derivative for the activations."""
    xv = _as_f32(x).astype(np.float64)
    nc = scales.shape[-1] * mode_info(mode)[2]
    return xv @ dequantize_f64(codes, scales, mode, nc, global_scale)

