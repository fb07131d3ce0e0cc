"""Host-side checks of libnq.so that need no GPU.

- The library loads and exports every function include/nq.h declares.
- The planner is pure and its split of K never depends on the row count
  ("Determinism" section of the nuvec API index: routing is pure; rows of a
  row-exact product equal their one-row products).
- Every argument error is reported before anything is enqueued: each call
  below is invalid and returns its status without touching the device (the
  pointers are fake and never dereferenced).
"""
import ctypes
import os
import re

import pytest

from conftest import ROOT
from group_wise_affine_quantize_amd import _binding as B

HEADER = os.path.join(ROOT, "include", "nq.h")

NQ_OK, NQ_ERR_NULL, NQ_ERR_DTYPE, NQ_ERR_QUANT, NQ_ERR_SHAPE = 0, 1, 2, 3, 4
NQ_ERR_ALIGN, NQ_ERR_ALIAS, NQ_ERR_WORKSPACE, NQ_ERR_LAUNCH, NQ_ERR_PLAN = 5, 6, 7, 8, 9
F32, BF16 = 0, 1


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nq_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.library_path()):
        pytest.fail("libnq.so is not built (python -m group_wise_affine_quantize_amd.build)")
    return B.load_library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"nq_quantize", "nq_dequantize", "nq_qmm", "nq_qmm_row_exact", "nq_gather_qmm",
            "nq_qmm_plan", "nq_last_error", "nq_status_string"} <= set(names)
    for name in names:
        assert hasattr(lib, name), name
    # the binding wraps every declared entry point under the same name
    for name in names:
        assert name in B._SIGNATURES, name


def test_header_constants_match_binding():
    text = open(HEADER).read()
    assert re.search(r"#define NQ_ROW_INDEPENDENT_ROWS 8\b", text)
    assert B.NQ_ROW_INDEPENDENT_ROWS == 8
    assert re.search(r"NQ_F32 = 0, NQ_BF16 = 1", text)
    assert re.search(r"NQ_ROUTE_GEMV = 1, NQ_ROUTE_TILED = 2", text)
    assert ctypes.sizeof(B.Plan) == 32


def test_status_strings(lib):
    for st in range(10):
        assert lib.nq_status_string(st)
    assert lib.nq_status_string(0) == b"ok"
    assert lib.nq_version().count(b".") == 2


def plan(lib, m, n, k, gs=64, bits=4, x=BF16, sb=BF16, row_exact=0):
    p = B.Plan()
    st = lib.nq_qmm_plan(m, n, k, gs, bits, x, sb, row_exact, ctypes.byref(p))
    assert st == NQ_OK, lib.nq_last_error()
    return p


def test_plan_is_pure_and_row_independent(lib):
    shapes = [(14336, 4096), (4096, 4096), (1024, 14336), (1408, 2048), (256, 512), (7, 64)]
    for n, k in shapes:
        ref = plan(lib, 1, n, k)
        assert ref.route == B.NQ_ROUTE_GEMV
        for m in (1, 2, 3, 5, 8):
            p = plan(lib, m, n, k)
            assert (p.route, p.ksplit, p.rows_per_wave) == (ref.route, ref.ksplit,
                                                            ref.rows_per_wave)
        for m in (1, 9, 17, 100, 2048):
            p = plan(lib, m, n, k, row_exact=1)
            assert (p.route, p.ksplit, p.rows_per_wave) == (ref.route, ref.ksplit,
                                                            ref.rows_per_wave)
        again = plan(lib, 1, n, k)
        assert bytes(again) == bytes(ref)


def test_plan_routes(lib):
    assert plan(lib, 8, 14336, 4096).route == B.NQ_ROUTE_GEMV
    assert plan(lib, 9, 14336, 4096).route == B.NQ_ROUTE_TILED
    assert plan(lib, 9, 14336, 4096).tile_m == 128
    assert plan(lib, 2048, 14336, 4096).route == B.NQ_ROUTE_TILED
    assert plan(lib, 2048, 14336, 4096).tile_m == 256
    assert plan(lib, 2048, 14336, 4096, x=F32, sb=F32).route == B.NQ_ROUTE_GEMV
    # the 256 x 256 kernel loads scale rows as dwords: an odd number of bf16
    # groups per row (k = 192, group 64) takes 128 x 128 tiles; f32 scales
    # are always aligned
    assert plan(lib, 2048, 1024, 192).tile_m == 128
    assert plan(lib, 2048, 1024, 192, sb=F32).tile_m == 256
    assert plan(lib, 2048, 1024, 256).tile_m == 256
    # long inner dimension with a small output splits K
    assert plan(lib, 4, 1024, 14336).ksplit > 1
    assert plan(lib, 1, 14336, 4096).ksplit == 1
    # 8-bit codes with k in whole 1024-wide quarters up to 4096 below the
    # streaming shapes: the matrix-core family's four K quarters, for any m
    for m in (1, 8, 21):
        assert plan(lib, m, 4096, 4096, gs=128, bits=8, row_exact=1).ksplit == 4


FAKE = 0x10000          # 16-byte aligned, never dereferenced
FAKE2 = 0x40000000


def _qmm(lib, entry="nq_qmm", x=FAKE, x_dt=BF16, m=4, k=128, codes=FAKE2, scales=FAKE2 + 0x100000,
         biases=FAKE2 + 0x200000, sb_dt=BF16, n=64, gs=64, bits=4, y=FAKE2 + 0x300000, ws=0,
         ws_bytes=0):
    fn = getattr(lib, entry)
    return fn(x, x_dt, m, k, codes, scales, biases, sb_dt, n, gs, bits, y, ws, ws_bytes, None)


@pytest.mark.parametrize("entry", ["nq_qmm", "nq_qmm_row_exact"])
def test_qmm_argument_errors(lib, entry):
    cases = [
        (dict(x_dt=7), NQ_ERR_DTYPE, "dtype"),
        (dict(sb_dt=-1), NQ_ERR_DTYPE, "dtype"),
        (dict(bits=7), NQ_ERR_QUANT, "bits=7"),
        (dict(bits=16), NQ_ERR_QUANT, "bits=16"),
        (dict(gs=16), NQ_ERR_QUANT, "group_size=16"),
        (dict(k=100), NQ_ERR_SHAPE, "k=100 is not a multiple of group_size=64"),
        (dict(m=-1), NQ_ERR_SHAPE, "negative"),
        (dict(n=-2), NQ_ERR_SHAPE, "negative"),
        (dict(k=1 << 33), NQ_ERR_SHAPE, "too large"),
        (dict(y=0), NQ_ERR_NULL, "y is null"),
        (dict(x=0), NQ_ERR_NULL, "non-null"),
        (dict(codes=0), NQ_ERR_NULL, "non-null"),
        (dict(x=FAKE + 8), NQ_ERR_ALIGN, "aligned"),
        (dict(y=FAKE2 + 0x300004), NQ_ERR_ALIGN, "aligned"),
        (dict(scales=FAKE2 + 0x100001), NQ_ERR_ALIGN, "aligned"),
        (dict(y=FAKE), NQ_ERR_ALIAS, "y overlaps x"),
        (dict(y=FAKE2 + 0x100000), NQ_ERR_ALIAS, "y overlaps scales"),
        (dict(y=FAKE2 + 0x10), NQ_ERR_ALIAS, "y overlaps codes"),
    ]
    for kw, want, msg in cases:
        st = _qmm(lib, entry, **kw)
        assert st == want, (kw, st, lib.nq_last_error())
        err = lib.nq_last_error().decode()
        assert err.startswith(entry + ":") and msg in err, (kw, err)


def test_batched_argument_errors(lib):
    def q(**kw):
        a = dict(x=FAKE, x_dt=BF16, batch=3, l=4, k=128, codes=FAKE2, scales=FAKE2 + 0x100000,
                 biases=FAKE2 + 0x200000, sb_dt=BF16, n=64, gs=64, bits=4, y=FAKE2 + 0x300000)
        a.update(kw)
        return lib.nq_qmm_batched(a["x"], a["x_dt"], a["batch"], a["l"], a["k"], a["codes"],
                                  a["scales"], a["biases"], a["sb_dt"], a["n"], a["gs"], a["bits"],
                                  a["y"], 0, 0, None)
    assert q(batch=-1) == NQ_ERR_SHAPE
    assert q(l=-1) == NQ_ERR_SHAPE
    assert q(batch=1 << 20, l=1 << 20) == NQ_ERR_SHAPE
    assert q(k=100) == NQ_ERR_SHAPE
    assert q(bits=7) == NQ_ERR_QUANT
    assert q(y=0) == NQ_ERR_NULL
    # x spans batch * l rows of k
    assert q(y=FAKE + 3 * 4 * 128 * 2 - 16) == NQ_ERR_ALIAS
    assert b"nq_qmm_batched: y overlaps x" in lib.nq_last_error()
    assert q(batch=0, x=0, y=0) == NQ_OK
    assert q(l=0, x=0, y=0) == NQ_OK


def test_empty_products_enqueue_nothing(lib):
    # m == 0 or n == 0: OK without touching any pointer (all null here)
    assert _qmm(lib, m=0, x=0, codes=0, scales=0, biases=0, y=0) == NQ_OK
    assert lib.nq_last_error() == b""
    assert _qmm(lib, n=0, x=0, codes=0, scales=0, biases=0, y=0) == NQ_OK
    st = lib.nq_gather_qmm(0, BF16, 0, 1, 128, 0, 0, 0, BF16, 4, 64, 64, 4, 0, 0, 0, 0, 0, None)
    assert st == NQ_OK


@pytest.mark.parametrize("bits", [1, 2, 3, 5, 6])
def test_plan_routes_other_widths(lib, bits):
    """Every stored width has a product route: matrix-vector for few rows,
    128-row tiles for many (the 256-row tiles take 4 and 8 bits)."""
    assert plan(lib, 8, 4096, 4096, bits=bits).route == B.NQ_ROUTE_GEMV
    p = plan(lib, 2048, 4096, 4096, bits=bits)
    assert p.route == B.NQ_ROUTE_TILED and p.tile_m == 128 and p.tile_n == 128
    assert plan(lib, 2048, 4096, 4096, bits=bits, row_exact=1).route == B.NQ_ROUTE_GEMV
    forced = plan(lib, 2048, 256, 256, bits=4)
    assert forced.tile_m == 256
    st = lib.nq_qmm_with_plan(ctypes.byref(forced), FAKE, BF16, 2048, 256, FAKE2, FAKE2 + 0x100000,
                              FAKE2 + 0x200000, BF16, 256, 64, bits, FAKE2 + 0x300000, 0, 0, None)
    assert st == NQ_ERR_PLAN and b"not supported" in lib.nq_last_error()


def test_plan_errors(lib):
    p = B.Plan()
    p.route = 99
    st = lib.nq_qmm_with_plan(ctypes.byref(p), FAKE, BF16, 4, 128, FAKE2, FAKE2 + 0x100000,
                              FAKE2 + 0x200000, BF16, 64, 64, 4, FAKE2 + 0x300000, 0, 0, None)
    assert st == NQ_ERR_PLAN and b"unknown route" in lib.nq_last_error()
    p.route, p.ksplit, p.rows_per_wave = B.NQ_ROUTE_GEMV, 9, 4
    st = lib.nq_qmm_with_plan(ctypes.byref(p), FAKE, BF16, 4, 128, FAKE2, FAKE2 + 0x100000,
                              FAKE2 + 0x200000, BF16, 64, 64, 4, FAKE2 + 0x300000, 0, 0, None)
    assert st == NQ_ERR_PLAN
    # 4 rows take 4 weight rows per wave in the VALU kernels (8-bit codes, k = 128)
    p.route, p.ksplit, p.rows_per_wave = B.NQ_ROUTE_GEMV, 2, 2
    st = lib.nq_qmm_with_plan(ctypes.byref(p), FAKE, BF16, 4, 128, FAKE2, FAKE2 + 0x100000,
                              FAKE2 + 0x200000, BF16, 64, 64, 8, FAKE2 + 0x300000, 0, 0, None)
    assert st == NQ_ERR_PLAN and b"does not fit" in lib.nq_last_error()
    p.route, p.tile_m, p.tile_n = B.NQ_ROUTE_TILED, 128, 128
    st = lib.nq_qmm_with_plan(ctypes.byref(p), FAKE, F32, 4, 128, FAKE2, FAKE2 + 0x100000,
                              FAKE2 + 0x200000, BF16, 64, 64, 4, FAKE2 + 0x300000, 0, 0, None)
    assert st == NQ_ERR_PLAN and b"bf16" in lib.nq_last_error()
    p.tile_m, p.tile_n = 256, 256     # k = 96 is not a multiple of 64
    st = lib.nq_qmm_with_plan(ctypes.byref(p), FAKE, BF16, 4, 96, FAKE2, FAKE2 + 0x100000,
                              FAKE2 + 0x200000, BF16, 64, 32, 4, FAKE2 + 0x300000, 0, 0, None)
    assert st == NQ_ERR_PLAN and b"does not fit" in lib.nq_last_error()
    st = lib.nq_qmm_with_plan(None, FAKE, BF16, 4, 128, FAKE2, 0, 0, BF16, 64, 64, 4, 0, 0, 0,
                              None)
    assert st == NQ_ERR_NULL


def test_quantize_argument_errors(lib):
    q = lambda **kw: lib.nq_quantize(kw.get("w", FAKE), kw.get("dt", BF16), kw.get("n", 8),
                                     kw.get("k", 128), kw.get("gs", 64), kw.get("bits", 4),
                                     kw.get("codes", FAKE2), kw.get("scales", FAKE2 + 0x100000),
                                     kw.get("biases", FAKE2 + 0x200000), None)
    assert q(dt=3) == NQ_ERR_DTYPE
    assert q(bits=7) == NQ_ERR_QUANT
    assert q(bits=0) == NQ_ERR_QUANT
    assert q(gs=256) == NQ_ERR_QUANT
    assert q(k=96) == NQ_ERR_SHAPE
    assert q(w=0) == NQ_ERR_NULL
    assert q(w=FAKE + 4) == NQ_ERR_ALIGN
    assert q(codes=FAKE) == NQ_ERR_ALIAS
    assert q(scales=FAKE2 + 0x8) == NQ_ERR_ALIAS
    assert b"nq_quantize:" in lib.nq_last_error()
    assert q(n=0, w=0, codes=0, scales=0, biases=0) == NQ_OK
    d = lambda **kw: lib.nq_dequantize(kw.get("codes", FAKE2), kw.get("scales", FAKE2 + 0x100000),
                                       kw.get("biases", FAKE2 + 0x200000), kw.get("sb", BF16),
                                       kw.get("n", 8), kw.get("k", 128), kw.get("gs", 64),
                                       kw.get("bits", 4), kw.get("out", FAKE), kw.get("odt", F32),
                                       None)
    assert d(odt=5) == NQ_ERR_DTYPE
    assert d(bits=7) == NQ_ERR_QUANT
    assert d(k=33) == NQ_ERR_SHAPE
    assert d(out=0) == NQ_ERR_NULL
    assert d(out=FAKE2 + 0x100000) == NQ_ERR_ALIAS
    assert d(out=FAKE + 2) == NQ_ERR_ALIGN


def test_gather_argument_errors(lib):
    def g(**kw):
        a = dict(x=FAKE, x_dt=BF16, rows=4, l=1, k=128, codes=FAKE2, scales=FAKE2 + 0x100000,
                 biases=FAKE2 + 0x200000, sb_dt=BF16, e=8, n=64, gs=64, bits=4,
                 idx=FAKE2 + 0x300000, sorted_hint=0, y=FAKE2 + 0x400000)
        a.update(kw)
        return lib.nq_gather_qmm(a["x"], a["x_dt"], a["rows"], a["l"], a["k"], a["codes"],
                                 a["scales"], a["biases"], a["sb_dt"], a["e"], a["n"], a["gs"],
                                 a["bits"], a["idx"], a["sorted_hint"], a["y"], 0, 0, None)
    assert g(e=-1) == NQ_ERR_SHAPE
    assert g(k=100) == NQ_ERR_SHAPE
    assert g(idx=0) == NQ_ERR_NULL
    assert g(y=FAKE2 + 0x300000) == NQ_ERR_ALIAS
    assert b"rhs_idx" in lib.nq_last_error()
    assert g(idx=FAKE2 + 0x300002) == NQ_ERR_ALIGN
    assert g(bits=7) == NQ_ERR_QUANT
    assert b"nq_gather_qmm:" in lib.nq_last_error()


def test_gather_lhs_argument_errors(lib):
    def g(**kw):
        a = dict(x=FAKE, x_dt=BF16, x_items=2, rows=4, l=1, k=128, codes=FAKE2,
                 scales=FAKE2 + 0x100000, biases=FAKE2 + 0x200000, sb_dt=BF16, e=8, n=64, gs=64,
                 bits=4, lhs=FAKE2 + 0x500000, idx=FAKE2 + 0x300000, sorted_hint=0, row_exact=0,
                 y=FAKE2 + 0x400000)
        a.update(kw)
        return lib.nq_gather_qmm_lhs(a["x"], a["x_dt"], a["x_items"], a["rows"], a["l"], a["k"],
                                     a["codes"], a["scales"], a["biases"], a["sb_dt"], a["e"],
                                     a["n"], a["gs"], a["bits"], a["lhs"], a["idx"],
                                     a["sorted_hint"], a["row_exact"], a["y"], 0, 0, None)
    assert g(lhs=0) == NQ_ERR_NULL
    assert b"lhs_idx" in lib.nq_last_error()
    assert g(x_items=0) == NQ_ERR_SHAPE
    assert g(x_items=-3) == NQ_ERR_SHAPE
    assert b"x_items" in lib.nq_last_error()
    assert g(lhs=FAKE2 + 0x500002) == NQ_ERR_ALIGN
    assert g(y=FAKE2 + 0x500000) == NQ_ERR_ALIAS          # y overlaps lhs_idx
    assert b"lhs_idx" in lib.nq_last_error()
    # x spans x_items items of l * k elements
    assert g(y=FAKE + 2 * 128 * 2 - 16, x_items=2) == NQ_ERR_ALIAS
    assert b"y overlaps x" in lib.nq_last_error()
    assert g(idx=0, row_exact=1) == NQ_ERR_NULL
    assert g(bits=7) == NQ_ERR_QUANT
    assert b"nq_gather_qmm_lhs:" in lib.nq_last_error()
    # nothing to do: no rows
    assert g(rows=0, lhs=0) == NQ_OK


def test_gather_grouped_route_workspace(lib):
    """Many rows per expert take the grouped route, which needs a workspace;
    few rows per expert (or few rows) do not."""
    def need(rows, l, e, n=1408, k=2048):
        return lib.nq_gather_qmm_workspace_bytes(rows, l, k, e, n, 64, 4, BF16, BF16, 1)
    assert need(512, 1, 32) > 0                 # the mixture-of-experts workload
    assert need(512, 1, 32) % 16 == 0 or need(512, 1, 32) >= 512 * 4
    assert need(4, 1, 8) == 0                   # the page example: 4 rows, 8 experts
    assert need(100, 1, 32) == 0                # fewer than 4 vectors per expert
    assert need(8, 2, 2) > 0                    # 16 vectors over 2 experts
    assert need(512, 1, 32) == need(256, 2, 32)  # vectors = rows * l
    assert need(0, 1, 32) == 0 and need(512, 1, 0) == 0

    # codes of 32 experts take 46 MB: every array sits 64 MB from the next
    y = FAKE2 + 0x8000000
    def g(ws, ws_bytes, rows=512):
        return lib.nq_gather_qmm(FAKE, BF16, rows, 1, 2048, FAKE2, FAKE2 + 0x4000000,
                                 FAKE2 + 0x5000000, BF16, 32, 1408, 64, 4, FAKE2 + 0x6000000, 1,
                                 y, ws, ws_bytes, None)
    nb = need(512, 1, 32)
    ws = FAKE2 + 0x10000000
    assert g(0, 0) == NQ_ERR_WORKSPACE
    assert b"workspace" in lib.nq_last_error()
    assert g(ws, nb - 1) == NQ_ERR_WORKSPACE
    assert g(ws + 8, nb) == NQ_ERR_ALIGN
    assert g(y, nb) == NQ_ERR_ALIAS                       # workspace overlaps y
    assert g(FAKE2 + 0x6000000, nb) == NQ_ERR_ALIAS       # ... or the ids


def test_error_string_is_thread_local(lib):
    import threading
    _qmm(lib, k=100)
    seen = {}

    def other():
        seen["before"] = lib.nq_last_error()
        _qmm(lib, bits=7)
        seen["after"] = lib.nq_last_error()

    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen["before"] == b""
    assert b"bits=7" in seen["after"]
    assert b"k=100" in lib.nq_last_error()


def _nt(lib, entry="nq_qmm_notrans", x=FAKE, x_dt=BF16, m=4, ni=128, codes=FAKE2, scales=FAKE2 + 0x100000,
        biases=FAKE2 + 0x200000, sb_dt=BF16, nc=256, gs=64, bits=4, y=FAKE2 + 0x300000,
        ws=FAKE2 + 0x1000000, ws_bytes=1 << 24):
    fn = getattr(lib, entry)
    return fn(x, x_dt, m, ni, codes, scales, biases, sb_dt, nc, gs, bits, y, ws, ws_bytes, None)


@pytest.mark.parametrize("entry", ["nq_qmm_notrans", "nq_qmm_notrans_row_exact"])
def test_notrans_argument_errors(lib, entry):
    """The product with the weights as stored validates like nq_qmm; its
    groups run along the columns (nc), and its matrix-vector route needs a
    workspace fixed by (ni, nc)."""
    need = lib.nq_qmm_notrans_workspace_bytes(4, 128, 256, 64, 4, BF16, 0)
    assert need > 0 and need == lib.nq_qmm_notrans_workspace_bytes(1, 128, 256, 64, 4, BF16, 0)
    assert lib.nq_qmm_notrans_workspace_bytes(64, 128, 256, 64, 4, BF16, 0) == 0      # tiled
    assert lib.nq_qmm_notrans_workspace_bytes(64, 128, 256, 64, 4, BF16, 1) == need   # row-exact
    assert lib.nq_qmm_notrans_workspace_bytes(64, 100, 256, 64, 4, BF16, 0) > 0       # ni % 64
    assert lib.nq_qmm_notrans_workspace_bytes(64, 96, 256, 64, 4, BF16, 0) > 0        # ni % 64
    cases = [
        (dict(x_dt=7), NQ_ERR_DTYPE, "dtype"),
        (dict(bits=7), NQ_ERR_QUANT, "bits=7"),
        (dict(nc=100), NQ_ERR_SHAPE, "not a multiple of group_size=64"),
        (dict(m=-1), NQ_ERR_SHAPE, "negative"),
        (dict(y=0), NQ_ERR_NULL, "y is null"),
        (dict(codes=0), NQ_ERR_NULL, "non-null"),
        (dict(x=FAKE + 8), NQ_ERR_ALIGN, "aligned"),
        (dict(y=FAKE), NQ_ERR_ALIAS, "y overlaps x"),
        (dict(ws=0), NQ_ERR_WORKSPACE, "workspace"),
        (dict(ws_bytes=need - 1), NQ_ERR_WORKSPACE, "workspace"),
        (dict(ws=FAKE2 + 0x1000008), NQ_ERR_ALIGN, "workspace"),
        (dict(ws=FAKE2 + 0x300000), NQ_ERR_ALIAS, "workspace overlaps"),
    ]
    for kw, want, msg in cases:
        st = _nt(lib, entry, **kw)
        assert st == want, (kw, st, lib.nq_last_error())
        err = lib.nq_last_error().decode()
        assert err.startswith(entry + ":") and msg in err, (kw, err)
    assert _nt(lib, entry, m=0, x=0, codes=0, scales=0, biases=0, y=0, ws=0, ws_bytes=0) == NQ_OK


def _grad(lib, x=FAKE, dy=FAKE + 0x100000, x_dt=BF16, m=4, k=256, codes=FAKE2, n=64, gs=64, bits=4,
          ds=FAKE2 + 0x200000, db=FAKE2 + 0x300000, g_dt=F32):
    return lib.nq_qmm_grad_scales_biases(x, dy, x_dt, m, k, codes, n, gs, bits, ds, db, g_dt, None)


def test_grad_scales_biases_argument_errors(lib):
    op = "nq_qmm_grad_scales_biases"
    cases = [
        (dict(g_dt=3), NQ_ERR_DTYPE, "dtype"),
        (dict(bits=0), NQ_ERR_QUANT, "bits=0"),
        (dict(k=100), NQ_ERR_SHAPE, "multiple of group_size"),
        (dict(m=-3), NQ_ERR_SHAPE, "negative"),
        (dict(ds=0), NQ_ERR_NULL, "non-null"),
        (dict(codes=0), NQ_ERR_NULL, "non-null"),
        (dict(dy=0), NQ_ERR_NULL, "x and dy"),
        (dict(codes=FAKE2 + 2), NQ_ERR_ALIGN, "aligned"),
        (dict(ds=FAKE2 + 0x200002), NQ_ERR_ALIGN, "aligned"),
        (dict(db=FAKE2 + 0x200000), NQ_ERR_ALIAS, "dscales overlaps dbiases"),
        (dict(ds=FAKE), NQ_ERR_ALIAS, "dscales overlaps x"),
        (dict(db=FAKE2 + 0x10), NQ_ERR_ALIAS, "dbiases overlaps codes"),
    ]
    for kw, want, msg in cases:
        st = _grad(lib, **kw)
        assert st == want, (kw, st, lib.nq_last_error())
        err = lib.nq_last_error().decode()
        assert err.startswith(op + ":") and msg in err, (kw, err)
    assert _grad(lib, n=0, x=0, dy=0, codes=0, ds=0, db=0) == NQ_OK


def test_fp_mode_constants_match_binding():
    text = open(HEADER).read()
    assert re.search(r"NQ_MXFP4 = 1, NQ_MXFP8 = 2, NQ_NVFP4 = 3", text)
    assert (B.NQ_MXFP4, B.NQ_MXFP8, B.NQ_NVFP4) == (1, 2, 3)
    assert {m: v[1:] for m, v in B.FP_MODES.items()} == {"mxfp4": (4, 32), "mxfp8": (8, 32),
                                                         "nvfp4": (4, 16)}


def _fp_qmm(lib, x=FAKE, x_dt=BF16, m=4, k=128, codes=FAKE2, scales=FAKE2 + 0x100000, g=0, n=64,
            mode=1, row_exact=0, y=FAKE2 + 0x300000):
    return lib.nq_fp_qmm(x, x_dt, m, k, codes, scales, g, n, mode, row_exact, y, None)


def test_fp_qmm_argument_errors(lib):
    cases = [
        (dict(x_dt=5), NQ_ERR_DTYPE, "dtype"),
        (dict(mode=0), NQ_ERR_QUANT, "mode=0"),
        (dict(mode=4), NQ_ERR_QUANT, "mode=4"),
        (dict(g=FAKE2 + 0x400000), NQ_ERR_QUANT, "only defined for NQ_NVFP4"),
        (dict(mode=3, g=FAKE2 + 0x400002), NQ_ERR_ALIGN, "4-byte"),
        (dict(k=48), NQ_ERR_SHAPE, "multiple of 32"),
        (dict(m=-1), NQ_ERR_SHAPE, "negative"),
        (dict(n=-1), NQ_ERR_SHAPE, "negative"),
        (dict(k=1 << 33), NQ_ERR_SHAPE, "too large"),
        (dict(x=0), NQ_ERR_NULL, "non-null"),
        (dict(scales=0), NQ_ERR_NULL, "non-null"),
        (dict(y=0), NQ_ERR_NULL, "non-null"),
        (dict(x=FAKE + 8), NQ_ERR_ALIGN, "aligned"),
        (dict(y=FAKE), NQ_ERR_ALIAS, "y overlaps"),
        (dict(y=FAKE2 + 0x100000), NQ_ERR_ALIAS, "y overlaps"),
    ]
    for kw, want, msg in cases:
        st = _fp_qmm(lib, **kw)
        assert st == want, (kw, st, lib.nq_last_error())
        err = lib.nq_last_error().decode()
        assert err.startswith("nq_fp_qmm:") and msg in err, (kw, err)
    # empty products enqueue nothing and succeed, even with null pointers
    assert _fp_qmm(lib, m=0, x=0, y=0) == NQ_OK
    assert _fp_qmm(lib, n=0, x=0, y=0) == NQ_OK


def test_fp_storage_and_gather_argument_errors(lib):
    q = lambda **kw: lib.nq_fp_quantize(kw.get("w", FAKE), kw.get("dt", F32), kw.get("n", 4),
                                        kw.get("k", 64), kw.get("mode", 3), kw.get("codes", FAKE2),
                                        kw.get("scales", FAKE2 + 0x100000), None)
    assert q(mode=9) == NQ_ERR_QUANT
    assert q(k=16) == NQ_ERR_SHAPE
    assert q(codes=0) == NQ_ERR_NULL
    assert q(codes=FAKE2 + 4) == NQ_ERR_ALIGN
    assert q(scales=FAKE + 16) == NQ_ERR_ALIAS and b"overlaps w" in lib.nq_last_error()
    assert q(n=0, w=0) == NQ_OK
    d = lambda **kw: lib.nq_fp_dequantize(kw.get("codes", FAKE2), kw.get("scales", FAKE2 + 0x100000),
                                          4, 64, kw.get("mode", 2), kw.get("out", FAKE), kw.get("dt", BF16),
                                          None)
    assert d(dt=3) == NQ_ERR_DTYPE
    assert d(out=FAKE2) == NQ_ERR_ALIAS
    assert d(out=FAKE + 2) == NQ_ERR_ALIGN
    assert d(scales=0) == NQ_ERR_NULL
    gq = lambda **kw: lib.nq_fp_gather_qmm(FAKE, BF16, kw.get("rows", 4), 1, 64, FAKE2, FAKE2 + 0x100000,
                                           kw.get("g", 0), kw.get("e", 8), 32, kw.get("mode", 3),
                                           kw.get("idx", FAKE2 + 0x200000), 0, FAKE2 + 0x300000,
                                           kw.get("ws", 0), kw.get("ws_bytes", 0), None)
    assert gq(idx=0) == NQ_ERR_NULL and b"rhs_idx" in lib.nq_last_error()
    assert gq(idx=FAKE2 + 0x200002) == NQ_ERR_ALIGN
    assert gq(e=0) == NQ_ERR_SHAPE
    assert gq(mode=1, g=FAKE2 + 0x400000) == NQ_ERR_QUANT
    assert gq(g=FAKE2 + 0x300000) == NQ_ERR_ALIAS
    # shared experts are grouped on the device: a workspace is required
    need = lib.nq_fp_gather_qmm_workspace_bytes(64, 1, 64, 8, 32)
    assert need > 0 and lib.nq_fp_gather_qmm_workspace_bytes(4, 1, 64, 8, 32) == 0
    assert gq(rows=64) == NQ_ERR_WORKSPACE and b"workspace" in lib.nq_last_error()
    assert gq(rows=64, ws=FAKE2 + 0x800000, ws_bytes=need - 1) == NQ_ERR_WORKSPACE
    assert gq(rows=64, ws=FAKE2 + 0x800008, ws_bytes=need) == NQ_ERR_ALIGN
    assert gq(rows=64, ws=FAKE2 + 0x300000, ws_bytes=need) == NQ_ERR_ALIAS


def test_fp_notrans_argument_errors(lib):
    def q(**kw):
        return lib.nq_fp_qmm_notrans(kw.get("x", FAKE), kw.get("dt", BF16), kw.get("m", 2), kw.get("ni", 128),
                                     FAKE2, FAKE2 + 0x100000, kw.get("g", 0), kw.get("nc", 64), kw.get("mode", 1),
                                     kw.get("rx", 0), kw.get("y", FAKE2 + 0x300000), kw.get("ws", 0),
                                     kw.get("ws_bytes", 0), None)
    need = lib.nq_fp_qmm_notrans_workspace_bytes(2, 128, 64, 1, BF16, 0)
    assert need > 0 and lib.nq_fp_qmm_notrans_workspace_bytes(64, 128, 64, 1, BF16, 0) == 0
    assert lib.nq_fp_qmm_notrans_workspace_bytes(64, 128, 64, 1, BF16, 1) > 0
    assert q() == NQ_ERR_WORKSPACE and b"nq_fp_qmm_notrans:" in lib.nq_last_error()
    assert q(mode=7) == NQ_ERR_QUANT
    assert q(nc=48) == NQ_ERR_SHAPE
    assert q(m=-1) == NQ_ERR_SHAPE
    assert q(g=FAKE2 + 0x400000) == NQ_ERR_QUANT
    assert q(x=0) == NQ_ERR_NULL
    assert q(x=FAKE + 4) == NQ_ERR_ALIGN
    assert q(y=FAKE) == NQ_ERR_ALIAS
    assert q(ws=FAKE2 + 0x800008, ws_bytes=need) == NQ_ERR_ALIGN
    assert q(ws=FAKE2 + 0x300000, ws_bytes=need) == NQ_ERR_ALIAS
    assert q(m=0, x=0, y=0) == NQ_OK
