"""Pins of the floating-point-mode oracle (oracle/fp.py) against what the
format definitions and the mathematics fix: the published code values, an
independent library implementation of the 8-bit formats (torch's float8
types), brute-force nearest-value searches, exact round trips and invariants
of the quantize rules, and brute-force products on tiny inputs."""
import os

import numpy as np
import pytest
import torch

from oracle import fp as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_values():
    out = []
    for line in open(os.path.join(GOLDEN, "ocp_minifloats.txt")):
        if line.startswith("#") or not line.strip():
            continue
        fmt, code, val = (t.strip() for t in line.split("|"))
        out.append((fmt, int(code, 16), val))
    return out


@pytest.mark.parametrize("fmt,code,val", _golden_values())
def test_code_values_match_published_tables(fmt, code, val):
    got = F.decode(np.array([code]), fmt)[0]
    if val == "nan":
        assert np.isnan(got)
    elif val == "-0":
        assert got == 0 and np.signbit(got)
    else:
        assert got == float(val) and not np.signbit(got) or got == float(val) < 0


def test_e2m1_table_complete():
    # the 16 codes: the 8 published magnitudes, then their negatives
    mags = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert list(F.E2M1[:8]) == mags
    assert list(-F.E2M1[8:]) == mags and all(np.signbit(F.E2M1[8:]))


def test_e4m3_decode_matches_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = F.decode(np.arange(256), "e4m3")
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert np.array_equal(np.signbit(ref[ok]), np.signbit(got[ok]))


def test_e8m0_decode_matches_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = F.decode(np.arange(256), "e8m0")
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])


def _e4m3_probe_values():
    rng = np.random.default_rng(3)
    fin = F.E4M3[:127]
    mids = (fin[:-1] + fin[1:]) / 2                         # exact ties
    v = np.concatenate([fin, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
                        rng.uniform(0, 448, 4000), np.exp(rng.uniform(-14, 6, 4000))])
    v = v[v <= 448].astype(np.float32)
    return np.concatenate([v, -v])


def test_e4m3_rounding_matches_torch_in_range():
    # torch's float -> float8_e4m3fn cast rounds to nearest even; within the
    # finite range it must agree code for code (beyond 448 torch gives NaN,
    # where the oracle saturates: that case is pinned below)
    v = _e4m3_probe_values()
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy().astype(np.int64)
    got = F.round_to_code(v, "e4m3")
    assert np.array_equal(ref, got)


def test_rounding_saturates():
    assert list(F.round_to_code(np.array([449, 464, 500, 1e30, -1e30], np.float32), "e4m3")) == \
        [0x7E, 0x7E, 0x7E, 0x7E, 0xFE]
    assert list(F.round_to_code(np.array([6, 6.5, 7, 8, 1e30, -9], np.float32), "e2m1")) == \
        [7, 7, 7, 7, 7, 15]


@pytest.mark.parametrize("fmt", ["e2m1", "e4m3"])
def test_rounding_is_brute_force_nearest_ties_even(fmt):
    table = F.E2M1 if fmt == "e2m1" else F.E4M3
    sbit = 3 if fmt == "e2m1" else 7
    fin = [c for c in range(1 << sbit) if np.isfinite(table[c])]
    rng = np.random.default_rng(7)
    top = table[fin[-1]]
    mids = [(table[a] + table[b]) / 2 for a, b in zip(fin[:-1], fin[1:])]
    vals = np.concatenate([mids, rng.uniform(0, top, 2000), [0.0, top]]).astype(np.float32)
    got = F.round_to_code(vals, fmt)
    for v, c in zip(vals, got):
        d = [abs(float(v) - table[k]) for k in fin]
        best = min(d)
        cands = [k for k, dk in zip(fin, d) if dk == best]
        want = cands[0] if len(cands) == 1 else [k for k in cands if k % 2 == 0][0]
        assert c == want, (fmt, v, c, want)


def test_sign_kept_through_zero():
    c = F.round_to_code(np.array([-0.0, -1e-30, 1e-30, 0.0], np.float32), "e2m1")
    assert list(c) == [8, 8, 0, 0]


@pytest.mark.parametrize("bits", [4, 8])
def test_pack_matches_published_layout(bits):
    # the hand-worked packing fixture of the affine codes (same word layout)
    for line in open(os.path.join(GOLDEN, "pack_lsb_first.txt")):
        if line.startswith("#") or not line.strip():
            continue
        b, codes, words = (t.strip() for t in line.split("|"))
        if int(b) != bits:
            continue
        codes = [int(t) for t in codes.split()]
        per = 32 // bits
        padded = codes + [0] * (-len(codes) % per)
        got = F.pack(np.array([padded]), bits)[0]
        want = [int(w, 16) for w in words.split()]
        assert list(got[: len(want)]) == want
        assert list(F.unpack(got[None], bits, len(codes))[0]) == codes


@pytest.mark.parametrize("mode", ["mxfp4", "mxfp8"])
def test_mx_round_trip_of_representable_blocks(mode):
    # blocks built as 2^X * (element values) with an element in the top
    # binade come back with the same scale code and codes
    elem, bits, gs, _ = F.mode_info(mode)
    table = F.E2M1 if elem == "e2m1" else F.E4M3
    sbit = 3 if elem == "e2m1" else 7
    fin = np.array([c for c in range(1 << (sbit + 1)) if np.isfinite(table[c])])
    top = fin[table[fin] >= 2.0 ** F._EMAX[elem]]
    rng = np.random.default_rng(11)
    rows, k = 6, 4 * gs
    codes = rng.choice(fin, size=(rows, k))
    codes[:, ::gs] = rng.choice(top, size=(rows, k // gs))     # one top-binade value per block
    X = rng.integers(-20, 20, size=(rows, k // gs))
    w = table[codes] * np.ldexp(1.0, np.repeat(X, gs, axis=1))
    cq, sq = F.quantize(w.astype(np.float32), mode)
    assert np.array_equal(sq, (X + 127).astype(np.uint8))
    got = F.unpack(cq, bits, k)
    # equal values (a zero may come back as +0 or -0 only as given)
    assert np.array_equal(table[got], table[codes])
    assert np.array_equal(F.dequantize_f64(cq, sq, mode, k), w)


def _mx_clamp_rows():
    out = []
    for line in open(os.path.join(GOLDEN, "mx_scale_clamp.txt")):
        if line.startswith("#") or not line.strip():
            continue
        name, mode, vals, scode, ecodes = (t.strip() for t in line.split("|"))
        out.append(pytest.param(mode, vals, int(scode), [int(c, 16) for c in ecodes.split()], id=name))
    return out


def _parse_pow2_sum(tok):
    """'c*2^p' -> c * 2^p exactly; 'max' -> the largest finite fp32."""
    if tok == "max":
        return float(np.finfo(np.float32).max)
    c, p = tok.split("*2^")
    return float(np.ldexp(float(c), int(p)))


@pytest.mark.parametrize("mode,vals,scode,ecodes", _mx_clamp_rows())
def test_mx_scale_code_at_the_ends_of_the_range(mode, vals, scode, ecodes):
    """tests/golden/mx_scale_clamp.txt, worked out by hand: blocks whose
    shared exponent X + 127 falls below 0 take scale code 0 (2^-127) and
    elements w * 2^127; blocks holding the largest finite fp32 take code
    252 / 246 with saturated elements."""
    elem, bits, gs, _ = F.mode_info(mode)
    v = [_parse_pow2_sum(t) for t in vals.split()]
    w = np.zeros((1, gs), np.float64)
    w[0, : len(v)] = v
    w32 = w.astype(np.float32)
    assert np.array_equal(w32.astype(np.float64), w)                # exact in fp32
    cq, sq = F.quantize(w32, mode)
    assert sq.dtype == np.uint8 and int(sq[0, 0]) == scode
    b = np.unpackbits(cq[0].astype("<u4").view(np.uint8), bitorder="little")[: gs * bits]
    got = (b.reshape(gs, bits).astype(np.uint32) << np.arange(bits, dtype=np.uint32)).sum(axis=1)
    assert list(got[: len(ecodes)]) == ecodes
    assert not got[len(ecodes):].any()


@pytest.mark.parametrize("mode", ["mxfp4", "mxfp8"])
def test_mx_shared_exponent_rule(mode):
    # X = floor(log2 amax) - emax: amax / 2^X lies in [2^emax, 2^(emax + 1));
    # and every code is the nearest element of w / 2^X (brute force)
    elem, bits, gs, _ = F.mode_info(mode)
    table = F.E2M1 if elem == "e2m1" else F.E4M3
    emax = F._EMAX[elem]
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((4, 8 * gs)) * np.exp(rng.uniform(-8, 8, (4, 1)))).astype(np.float32)
    cq, sq = F.quantize(w, mode)
    X = sq.astype(np.int64) - 127
    amax = np.abs(w.reshape(4, -1, gs)).max(axis=2).astype(np.float64)
    r = amax / np.ldexp(1.0, X)
    assert np.all((r >= 2.0 ** emax) & (r < 2.0 ** (emax + 1)))
    codes = F.unpack(cq, bits, w.shape[1])
    fin = np.array([c for c in range(len(table)) if np.isfinite(table[c])])
    q = w.astype(np.float64) / np.ldexp(1.0, np.repeat(X, gs, axis=1))
    dist = np.abs(q[..., None] - table[fin][None, None, :])
    best = dist.min(axis=2)
    assert np.array_equal(np.abs(q - table[codes]), best)


def test_nvfp4_rules_brute_force():
    gs = 16
    rng = np.random.default_rng(9)
    w = (rng.standard_normal((3, 8 * gs)) * rng.uniform(0.5, 50, (3, 1))).astype(np.float32)
    cq, sq = F.quantize(w, "nvfp4")
    fin8 = np.array([c for c in range(127)])                 # non-negative finite E4M3
    amax = np.abs(w.reshape(3, -1, gs)).max(axis=2)
    target = (amax / np.float32(6)).astype(np.float64)
    d = np.abs(target[..., None] - F.E4M3[fin8])
    assert np.array_equal(np.abs(target - F.E4M3[sq]), d.min(axis=2))
    S = np.repeat(F.E4M3[sq].astype(np.float32), gs, axis=1)
    q = (w / S).astype(np.float64)
    codes = F.unpack(cq, 4, w.shape[1])
    d4 = np.abs(q[..., None] - F.E2M1[None, None, :])
    assert np.array_equal(np.abs(q - F.E2M1[codes]), d4.min(axis=2))


@pytest.mark.parametrize("mode", ["mxfp4", "mxfp8", "nvfp4"])
def test_zero_blocks(mode):
    _, bits, gs, _ = F.mode_info(mode)
    cq, sq = F.quantize(np.zeros((2, 2 * gs), np.float32), mode)
    assert not cq.any() and not sq.any()
    assert not F.dequantize(cq, sq, mode, 2 * gs).any()


@pytest.mark.parametrize("mode", ["mxfp4", "mxfp8", "nvfp4"])
def test_dequantize_bf16_matches_torch_rounding(mode):
    _, bits, gs, _ = F.mode_info(mode)
    rng = np.random.default_rng(1)
    w = (rng.standard_normal((8, 4 * gs)) * 3).astype(np.float32)
    cq, sq = F.quantize(w, mode)
    exact = F.dequantize_f64(cq, sq, mode, w.shape[1])
    ref = torch.from_numpy(exact).to(torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(F.dequantize(cq, sq, mode, w.shape[1]), ref)


def test_dequantize_nan_scale_and_element():
    # E8M0 0xff and E4M3 S.1111.111 decode to NaN; bf16 output is 0x7fc0
    cq = F.pack(np.array([[0x7F] + [0x38] * 31, [0x38] * 32]), 8)
    sq = np.array([[127], [255]], np.uint8)
    out = F.dequantize(cq, sq, "mxfp8", 32)
    assert out[0, 0] == 0x7FC0 and out[0, 1] == 0x3F80 and np.all(out[1] == 0x7FC0)


@pytest.mark.parametrize("mode", ["mxfp4", "mxfp8", "nvfp4"])
def test_products_brute_force(mode):
    elem, bits, gs, sfmt = F.mode_info(mode)
    rng = np.random.default_rng(2)
    n, k, m = 5, 2 * gs, 3
    w = rng.standard_normal((n, k)).astype(np.float32)
    x = rng.standard_normal((m, k)).astype(np.float32)
    cq, sq = F.quantize(w, mode)
    codes = F.unpack(cq, bits, k)
    # element and scale values from torch's float8 types and the published
    # E2M1 magnitudes, added one product at a time
    e2m1 = [0, 0.5, 1, 1.5, 2, 3, 4, 6]

    def elem_value(c):
        if elem == "e2m1":
            return (-1.0 if c & 8 else 1.0) * e2m1[c & 7]
        return float(torch.tensor([c], dtype=torch.uint8).view(torch.float8_e4m3fn).float())

    def scale_value(s):
        t = torch.tensor([s], dtype=torch.uint8)
        return float(t.view(torch.float8_e8m0fnu if sfmt == "e8m0" else torch.float8_e4m3fn).double())

    for g in (None, 0.37):
        y = F.qmm_f64(x, cq, sq, mode, g)
        for i in range(m):
            for j in range(n):
                acc = 0.0
                for t in range(k):
                    acc += float(x[i, t]) * scale_value(int(sq[j, t // gs])) * elem_value(int(codes[j, t]))
                if g is not None:
                    acc *= float(np.float32(g))
                assert abs(y[i, j] - acc) <= 1e-12 * max(1.0, abs(acc)), (mode, g, i, j)


def test_gather_rows_pick_their_expert():
    rng = np.random.default_rng(4)
    e, n, k = 3, 6, 64
    w = rng.standard_normal((e * n, k)).astype(np.float32)
    cq, sq = F.quantize(w, "nvfp4")
    cq, sq = cq.reshape(e, n, -1), sq.reshape(e, n, -1)
    x = rng.standard_normal((5, 2, k)).astype(np.float32)
    idx = np.array([2, 0, 7, 1, 2], np.uint32)
    gsc = np.array([0.5, 2.0, 0.25], np.float32)
    y = F.gather_qmm_f64(x, cq, sq, "nvfp4", idx, gsc)
    for r in range(5):
        if idx[r] >= e:
            assert not y[r].any()
        else:
            want = F.qmm_f64(x[r], cq[idx[r]], sq[idx[r]], "nvfp4") * float(gsc[idx[r]])
            assert np.allclose(y[r], want, rtol=1e-14, atol=0)


def test_dequantize_nan_is_canonical_in_both_outputs():
    # a negative NaN element (E4M3 0xff) and a NaN scale give the quiet NaN
    # of the output type, sign cleared
    cq = F.pack(np.array([[0xFF] + [0xB8] * 31]), 8)
    for s in (127, 255):
        f = F.dequantize(cq, np.array([[s]], np.uint8), "mxfp8", 32, "f32").view(np.uint32)
        assert f[0, 0] == 0x7FC00000
        b = F.dequantize(cq, np.array([[s]], np.uint8), "mxfp8", 32, "bf16")
        assert b[0, 0] == 0x7FC0
    f = F.dequantize(cq, np.array([[127]], np.uint8), "mxfp8", 32, "f32")
    assert f[0, 1] == -1.0


@pytest.mark.parametrize("mode", ["mxfp4", "mxfp8", "nvfp4"])
def test_weights_as_stored_adjoint_of_the_product(mode):
    # <dy, x . w_hat^T> = <dy . w_hat, x> for the same quantized matrix: a
    # transposed operand or a group axis along the wrong dimension fails it;
    # plus a brute-force entry
    _, bits, gs, _ = F.mode_info(mode)
    rng = np.random.default_rng(13)
    n, k, m = 6, 2 * gs, 3
    cq, sq = F.quantize(rng.standard_normal((n, k)).astype(np.float32), mode)
    x = rng.standard_normal((m, k)).astype(np.float32)
    dy = rng.standard_normal((m, n)).astype(np.float32)
    fwd = F.qmm_f64(x, cq, sq, mode, 0.5)
    dx = F.qmm_nt_f64(dy, cq, sq, mode, 0.5)
    assert dx.shape == (m, k)
    lhs = float(np.sum(dy.astype(np.float64) * fwd))
    rhs = float(np.sum(dx * x.astype(np.float64)))
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))
    E = F.decode(F.unpack(cq, bits, k), "e2m1" if bits == 4 else "e4m3")
    S = F.decode(sq, "e8m0" if mode != "nvfp4" else "e4m3")
    want = sum(float(dy[1, i]) * 0.5 * float(S[i, 5 // gs]) * float(E[i, 5]) for i in range(n))
    assert abs(dx[1, 5] - want) <= 1e-12 * max(1.0, abs(want))
