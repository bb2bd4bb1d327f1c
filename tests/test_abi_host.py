"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every function the header
declares, and rejects bad arguments with the documented status before launching anything."""
import ctypes
import os
import re

import pytest

from post_weight_quantization_05_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gptq_mi355x.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="library not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gptq_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = _lib.load()
    names = declared_functions()
    assert len(names) == 15, names
    for n in names:
        assert hasattr(lib, n), n
        assert n in _lib.SIGNATURES, n


def test_status_strings_and_version():
    for code, name in [(0, "GPTQ_OK"), (-1, "GPTQ_ERR_INVALID_ARG"), (-2, "GPTQ_ERR_UNSUPPORTED"),
                       (-3, "GPTQ_ERR_NOT_SPD"), (-4, "GPTQ_ERR_NONFINITE"), (-5, "GPTQ_ERR_WORKSPACE"),
                       (-6, "GPTQ_ERR_HIP")]:
        assert _lib.status_string(code) == name
    assert _lib.status_string(7) == "GPTQ_ERR_UNKNOWN"
    assert b"gfx950" in _lib.load().gptq_version()


def test_workspace_queries():
    lib = _lib.load()
    assert lib.gptq_hessian_workspace_bytes(0, 10, 1) == 0
    assert lib.gptq_hessian_workspace_bytes(10, 10, 7) == 0
    small = lib.gptq_hessian_workspace_bytes(512, 256, _lib.GPTQ_F32)
    big = lib.gptq_hessian_workspace_bytes(262144, 4096, _lib.GPTQ_BF16)
    assert 0 < small < big
    # fp32 partials of 136 lower-triangle 256x256 tiles per row slice + fp64 column sums
    assert big % (136 * 256 * 256 * 4) < 136 * 256 * 256 * 4 and big >= 136 * 256 * 256 * 4
    assert lib.gptq_prepare_workspace_bytes(4096) >= 4096 * 4096 * 8
    assert lib.gptq_quantize_workspace_bytes(4096, 4096) >= 4096 * 4096 * 8 + 4096 * 128 * 8
    assert lib.gptq_prepare_workspace_bytes(0) == 0
    assert lib.gptq_quantize_workspace_bytes(5, 0) == 0
    # the R route adds T (out x in doubles) to the same layout
    assert lib.gptq_quantize_r_workspace_bytes(4096, 4096) == lib.gptq_quantize_workspace_bytes(4096, 4096) + 4096 * 4096 * 8
    assert lib.gptq_quantize_r_workspace_bytes(5, 0) == 0


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


def test_hessian_argument_errors():
    lib = _lib.load()
    n = ctypes.c_int64(0)
    bad = _lib.GPTQ_ERR_INVALID_ARG

    def call(X=FAKE, dt=1, rows=8, d=4, ld=4, S=FAKE, cs=FAKE, nt=ctypes.byref(n), ws=FAKE, wsb=1 << 30):
        return lib.gptq_hessian_accumulate(X, dt, rows, d, ld, S, cs, nt, ws, wsb, None)

    assert call(X=None) == bad
    assert call(S=None) == bad
    assert call(cs=None) == bad
    assert call(nt=None) == bad
    assert call(rows=0) == bad
    assert call(d=0) == bad
    assert call(ld=3) == bad
    assert call(dt=2) == bad
    assert call(ws=None) == _lib.GPTQ_ERR_WORKSPACE
    assert call(wsb=16) == _lib.GPTQ_ERR_WORKSPACE
    assert n.value == 0  # untouched on error


def test_prepare_argument_errors():
    lib = _lib.load()
    bad = _lib.GPTQ_ERR_INVALID_ARG

    def call(S=FAKE, cs=FAKE, nt=10, d=4, damp=0.01, act=0, flags=0, U=FAKE, perm=FAKE, dead=FAKE, ws=FAKE,
             wsb=1 << 30):
        return lib.gptq_prepare_chol(S, cs, nt, d, damp, act, flags, U, perm, dead, ws, wsb, None)

    assert call(S=None) == bad
    assert call(U=None) == bad
    assert call(perm=None) == bad
    assert call(dead=None) == bad
    assert call(nt=0) == bad
    assert call(d=0) == bad
    assert call(damp=-1.0) == bad
    assert call(damp=float("nan")) == bad
    assert call(damp=float("inf")) == bad
    assert call(flags=3) == bad
    assert call(flags=4) == bad
    # the R form needs in % 64 == 0
    assert call(flags=_lib.GPTQ_FACTOR_R_FORM, d=100) == _lib.GPTQ_ERR_UNSUPPORTED
    assert call(ws=None) == _lib.GPTQ_ERR_WORKSPACE
    assert call(wsb=8) == _lib.GPTQ_ERR_WORKSPACE


def test_quantize_argument_errors():
    lib = _lib.load()
    bad = _lib.GPTQ_ERR_INVALID_ARG

    def call(W=FAKE, dt=1, out=8, d=256, ld=256, U=FAKE, perm=FAKE, dead=FAKE, bits=4, group=0, codes=FAKE,
             scales=FAKE, ws=FAKE, wsb=1 << 30):
        return lib.gptq_quantize_layer(W, dt, out, d, ld, U, perm, dead, bits, group, codes, scales, None, None,
                                       ws, wsb, None)

    assert call(W=None) == bad
    assert call(codes=None) == bad
    assert call(scales=None) == bad
    assert call(U=None) == bad
    assert call(out=0) == bad
    assert call(ld=255) == bad
    assert call(bits=1) == bad
    assert call(bits=9) == bad
    assert call(group=-1) == bad
    assert call(dt=5) == bad
    for g in (3, 48, 100, 200):
        assert call(group=g) == _lib.GPTQ_ERR_UNSUPPORTED
    assert call(ws=None) == _lib.GPTQ_ERR_WORKSPACE
    assert call(group=256, wsb=4) == _lib.GPTQ_ERR_WORKSPACE


def test_quantize_ex_argument_errors():
    """The grid-selecting entry point: unknown grid, or the asymmetric grid without a zeros buffer, are
    argument errors; the other checks are those of gptq_quantize_layer."""
    lib = _lib.load()
    bad = _lib.GPTQ_ERR_INVALID_ARG

    def call(grid=_lib.GPTQ_GRID_ASYMMETRIC, zeros=FAKE, W=FAKE, bits=4, group=0, ws=FAKE, wsb=1 << 30):
        return lib.gptq_quantize_layer_ex(W, 1, 8, 256, 256, FAKE, FAKE, FAKE, bits, group, grid, FAKE, FAKE, zeros,
                                          None, None, ws, wsb, None)

    assert call(grid=2) == bad
    assert call(grid=-1) == bad
    assert call(zeros=None) == bad
    assert call(W=None) == bad
    assert call(bits=9) == bad
    assert call(group=48) == _lib.GPTQ_ERR_UNSUPPORTED
    assert call(ws=None) == _lib.GPTQ_ERR_WORKSPACE
    assert call(grid=_lib.GPTQ_GRID_SYMMETRIC, zeros=None, ws=None) == _lib.GPTQ_ERR_WORKSPACE


def test_quantize_r_argument_errors():
    """The R-form loop: the checks of gptq_quantize_layer_ex, plus in % 64 == 0 and groups that divide 128
    (UNSUPPORTED otherwise)."""
    lib = _lib.load()
    bad = _lib.GPTQ_ERR_INVALID_ARG

    def call(W=FAKE, dt=1, out=8, d=256, ld=256, R=FAKE, perm=FAKE, dead=FAKE, bits=4, group=0, grid=0,
             codes=FAKE, scales=FAKE, zeros=None, ws=FAKE, wsb=1 << 30):
        return lib.gptq_quantize_layer_r(W, dt, out, d, ld, R, perm, dead, bits, group, grid, codes, scales, zeros,
                                         None, None, ws, wsb, None)

    assert call(R=None) == bad
    assert call(W=None) == bad
    assert call(grid=2) == bad
    assert call(grid=1) == bad  # asymmetric without zeros
    assert call(bits=9) == bad
    for g in (3, 48, 256, 1024):
        assert call(group=g) == _lib.GPTQ_ERR_UNSUPPORTED
    assert call(d=200, ld=200) == _lib.GPTQ_ERR_UNSUPPORTED
    assert call(ws=None) == _lib.GPTQ_ERR_WORKSPACE
    assert call(group=64, wsb=4) == _lib.GPTQ_ERR_WORKSPACE
    # the route through U's workspace lacks T
    assert call(wsb=lib.gptq_quantize_workspace_bytes(8, 256)) == _lib.GPTQ_ERR_WORKSPACE


def test_pack_and_dequant_argument_errors():
    lib = _lib.load()
    bad = _lib.GPTQ_ERR_INVALID_ARG
    assert lib.gptq_packed_words_per_row(256, 4) == 32
    assert lib.gptq_packed_words_per_row(300, 3) == 29   # ceil(900 / 32)
    assert lib.gptq_packed_words_per_row(1, 8) == 1
    assert lib.gptq_packed_words_per_row(0, 4) == 0
    assert lib.gptq_packed_words_per_row(16, 9) == 0
    assert lib.gptq_pack_codes(None, 4, 16, 4, 0, FAKE, None) == bad
    assert lib.gptq_pack_codes(FAKE, 4, 16, 4, 0, None, None) == bad
    assert lib.gptq_pack_codes(FAKE, 0, 16, 4, 0, FAKE, None) == bad
    assert lib.gptq_pack_codes(FAKE, 4, 16, 1, 0, FAKE, None) == bad
    assert lib.gptq_pack_codes(FAKE, 4, 16, 4, 3, FAKE, None) == bad

    def mm(X=FAKE, dt=1, n=8, d=16, ldx=16, P=FAKE, sc=FAKE, z=FAKE, gi=FAKE, out=4, bits=4, grid=1, group=0,
           relu=0, Y=FAKE, ldy=4):
        return lib.gptq_dequant_matmul(X, dt, n, d, ldx, P, sc, z, gi, out, bits, grid, group, None, relu, Y, ldy,
                                       None)

    assert mm(X=None) == bad
    assert mm(P=None) == bad
    assert mm(gi=None) == bad
    assert mm(z=None) == bad               # asymmetric grid needs zeros
    assert mm(grid=7) == bad
    assert mm(ldx=15) == bad
    assert mm(ldy=3) == bad
    assert mm(dt=9) == bad
    assert mm(bits=9) == bad
    assert mm(n=0) == bad
    assert mm(relu=2) == bad


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError, match="missing"):
        _lib.load(str(tmp_path / "nope.so"))


def test_factor_route_choice():
    """gptq_quantize's route when flags is None: the R form where the library takes it and it measured faster
    (one grid per row, or in >= 8192), else the route through U."""
    import post_weight_quantization_05_amd as G
    assert G.factor_route(4096, 0) == G.GPTQ_FACTOR_R_FORM
    assert G.factor_route(4096, None) == G.GPTQ_FACTOR_R_FORM
    assert G.factor_route(4096, 128) == G.GPTQ_FACTOR_REVERSED
    assert G.factor_route(11008, 128) == G.GPTQ_FACTOR_R_FORM
    assert G.factor_route(11008, 32) == G.GPTQ_FACTOR_R_FORM
    assert G.factor_route(11008, 256) == G.GPTQ_FACTOR_REVERSED  # wider than a panel: the R form does not take it
    assert G.factor_route(100, 0) == G.GPTQ_FACTOR_REVERSED      # not a multiple of 64
    assert G.factor_route(8200, 0) == G.GPTQ_FACTOR_REVERSED
