"""C ABI checks that need no GPU: the library loads, exports every symbol that
include/gptq.h declares, and rejects bad arguments on the host before any
launch (every call below returns before touching the device)."""
import ctypes
import os
import re

import pytest

import post_weight_quantization_02_amd as G

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gptq.h")

pytestmark = pytest.mark.skipif(not os.path.exists(G.lib_path()),
                                reason="libgptq.so not built (run __graft_entry__.build())")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gptq(?:2d)?_[a-z_]+)\s*\(", text)))


def _status(name):
    return {"GPTQ_OK": 0, "GPTQ_ERR_NULL_POINTER": 1, "GPTQ_ERR_BAD_SIZE": 2,
            "GPTQ_ERR_BAD_LEADING_DIM": 3, "GPTQ_ERR_BAD_DTYPE": 4, "GPTQ_ERR_BAD_BITS": 5,
            "GPTQ_ERR_BAD_BLOCK": 6, "GPTQ_ERR_BAD_GROUP": 7, "GPTQ_ERR_WORKSPACE": 8,
            "GPTQ_ERR_BAD_DAMP": 9, "GPTQ_ERR_LAUNCH": 10, "GPTQ_ERR_TOO_LARGE": 11, "GPTQ_ERR_SCRATCH": 12}[name]


def test_header_status_values_match():
    text = open(HEADER).read()
    for name, val in re.findall(r"(GPTQ_[A-Z_]+)\s*=\s*(\d+)", text):
        if name.startswith("GPTQ_ERR") or name == "GPTQ_OK":
            assert _status(name) == int(val)


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert "gptq_hessian_accumulate" in names and "gptq_quantize_layer" in names
    lib = ctypes.CDLL(G.lib_path())
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings():
    assert G.gptq_version().startswith("gptq-gfx950")
    for s in range(13):
        assert G.gptq_status_string(s) and G.gptq_status_string(s) != "unknown status"
    assert G.gptq_status_string(99) == "unknown status"


FAKE = 0x1000  # never dereferenced: validation fails first


def test_hessian_validation():
    lib = G.library()
    f = lib.gptq_hessian_accumulate
    assert f(FAKE, 0, FAKE, 0, 10, 10, FAKE, 1 << 30, None) == _status("GPTQ_ERR_BAD_SIZE")
    assert f(FAKE, 8, FAKE, 0, -1, 8, FAKE, 1 << 30, None) == _status("GPTQ_ERR_BAD_SIZE")
    assert f(FAKE, 8, FAKE, 7, 4, 8, FAKE, 1 << 30, None) == _status("GPTQ_ERR_BAD_DTYPE")
    assert f(None, 8, FAKE, 0, 4, 8, FAKE, 1 << 30, None) == _status("GPTQ_ERR_NULL_POINTER")
    assert f(FAKE, 8, None, 0, 4, 8, FAKE, 1 << 30, None) == _status("GPTQ_ERR_NULL_POINTER")
    assert f(FAKE, 8, FAKE, 0, 4, 7, FAKE, 1 << 30, None) == _status("GPTQ_ERR_BAD_LEADING_DIM")
    need = G.gptq_hessian_accumulate_workspace_size(8, 4, 0)
    assert need > 0
    assert f(FAKE, 8, FAKE, 0, 4, 8, FAKE, need - 1, None) == _status("GPTQ_ERR_WORKSPACE")
    assert f(FAKE, 8, FAKE, 0, 4, 8, None, need, None) == _status("GPTQ_ERR_WORKSPACE")
    assert f(FAKE, 8, None, 0, 0, 8, None, 0, None) == _status("GPTQ_OK")   # empty chunk
    assert f(FAKE, 1 << 21, FAKE, 0, 4, 1 << 21, FAKE, 1 << 30, None) == _status("GPTQ_ERR_TOO_LARGE")


def test_prepare_validation():
    f = G.library().gptq_prepare_hinv
    assert f(FAKE, 0, 0.01, FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == _status("GPTQ_ERR_BAD_SIZE")
    assert f(None, 8, 0.01, FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == _status("GPTQ_ERR_NULL_POINTER")
    assert f(FAKE, 8, 0.01, FAKE, FAKE, None, FAKE, 1 << 40, None) == _status("GPTQ_ERR_NULL_POINTER")
    assert f(FAKE, 8, -0.5, FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == _status("GPTQ_ERR_BAD_DAMP")
    assert f(FAKE, 8, float("nan"), FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == _status("GPTQ_ERR_BAD_DAMP")
    need = G.gptq_prepare_hinv_workspace_size(8)
    assert need >= 8 * 8 * 8
    assert f(FAKE, 8, 0.01, FAKE, FAKE, FAKE, FAKE, need - 1, None) == _status("GPTQ_ERR_WORKSPACE")


def test_quantize_validation():
    f = G.library().gptq_quantize_layer
    need = G.gptq_quantize_layer_workspace_size(4, 32, 16)
    ok = dict(W0=FAKE, w_dtype=0, d_row=4, d_col=32, ld_w=32, U=FAKE, lam=FAKE, bits=4,
              group=0, block=16, codes=FAKE, scales=FAKE, zeros=FAKE, err=FAKE, ws=FAKE,
              ws_bytes=need)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["W0"], a["w_dtype"], a["d_row"], a["d_col"], a["ld_w"], a["U"], a["lam"],
                 a["bits"], a["group"], a["block"], a["codes"], a["scales"], a["zeros"], a["err"],
                 a["ws"], a["ws_bytes"], None)

    assert call(d_row=0) == _status("GPTQ_ERR_BAD_SIZE")
    assert call(w_dtype=3) == _status("GPTQ_ERR_BAD_DTYPE")
    assert call(U=None) == _status("GPTQ_ERR_NULL_POINTER")
    assert call(err=None) == _status("GPTQ_ERR_NULL_POINTER")
    assert call(ld_w=31) == _status("GPTQ_ERR_BAD_LEADING_DIM")
    assert call(bits=1) == _status("GPTQ_ERR_BAD_BITS")
    assert call(bits=9) == _status("GPTQ_ERR_BAD_BITS")
    for b in (0, 8, 24, 256):
        assert call(block=b) == _status("GPTQ_ERR_BAD_BLOCK")
    assert call(group=24) == _status("GPTQ_ERR_BAD_GROUP")
    assert call(group=8) == _status("GPTQ_ERR_BAD_GROUP")
    assert call(group=-1) == _status("GPTQ_ERR_BAD_GROUP")
    assert call(ws_bytes=need - 1) == _status("GPTQ_ERR_WORKSPACE")
    assert G.gptq_quantize_layer_workspace_size(4, 32, 24) == 0


def test_workspace_sizes_are_monotone():
    a = G.gptq_quantize_layer_workspace_size(512, 512, 128)
    b = G.gptq_quantize_layer_workspace_size(4096, 4096, 128)
    assert 0 < a < b
    assert G.gptq_prepare_hinv_workspace_size(4096) > G.gptq_prepare_hinv_workspace_size(512)
    assert G.gptq_hessian_accumulate_workspace_size(4096, 262144, 1) > 0


def test_act_order_validation():
    lib = G.library()
    f = lib.gptq_act_order_perm
    assert f(FAKE, 0, FAKE, None) == _status("GPTQ_ERR_BAD_SIZE")
    assert f(None, 8, FAKE, None) == _status("GPTQ_ERR_NULL_POINTER")
    assert f(FAKE, 8, None, None) == _status("GPTQ_ERR_NULL_POINTER")
    assert f(FAKE, 1 << 21, FAKE, None) == _status("GPTQ_ERR_TOO_LARGE")
    p = lib.gptq_prepare_hinv_perm
    assert p(FAKE, 8, None, 0.01, FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == _status("GPTQ_ERR_NULL_POINTER")
    assert p(FAKE, 0, FAKE, 0.01, FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == _status("GPTQ_ERR_BAD_SIZE")
    assert p(FAKE, 8, FAKE, -1.0, FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == _status("GPTQ_ERR_BAD_DAMP")
    need = G.gptq_prepare_hinv_workspace_size(8)
    assert p(FAKE, 8, FAKE, 0.01, FAKE, FAKE, FAKE, FAKE, need - 1, None) == _status("GPTQ_ERR_WORKSPACE")
    q = lib.gptq_quantize_layer_perm
    needq = G.gptq_quantize_layer_workspace_size(4, 32, 16)
    args = [FAKE, 0, 4, 32, 32, FAKE, FAKE, FAKE, 4, 0, 16, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, needq, None]
    a = list(args); a[7] = None
    assert q(*a) == _status("GPTQ_ERR_NULL_POINTER")     # perm
    a = list(args); a[14] = None
    assert q(*a) == _status("GPTQ_ERR_NULL_POINTER")     # g_idx
    a = list(args); a[8] = 9
    assert q(*a) == _status("GPTQ_ERR_BAD_BITS")
    a = list(args); a[17] = needq - 1
    assert q(*a) == _status("GPTQ_ERR_WORKSPACE")


def test_packed_validation():
    lib = G.library()
    assert G.gptq_packed_words_per_row(100, 3) == 4 * 3
    assert G.gptq_packed_words_per_row(32, 4) == 4
    assert G.gptq_packed_words_per_row(100, 5) == 0
    f = lib.gptq_pack_codes
    assert f(FAKE, 0, 64, 64, 4, None, FAKE, 8, None) == _status("GPTQ_ERR_BAD_SIZE")
    assert f(None, 4, 64, 64, 4, None, FAKE, 8, None) == _status("GPTQ_ERR_NULL_POINTER")
    assert f(FAKE, 4, 64, 64, 5, None, FAKE, 8, None) == _status("GPTQ_ERR_BAD_BITS")
    assert f(FAKE, 4, 64, 63, 4, None, FAKE, 8, None) == _status("GPTQ_ERR_BAD_LEADING_DIM")
    assert f(FAKE, 4, 64, 64, 4, None, FAKE, 7, None) == _status("GPTQ_ERR_BAD_LEADING_DIM")
    d = lib.gptq_dequant_matmul
    ok = [FAKE, 8, 4, FAKE, FAKE, 16, None, 4, 64, FAKE, 1, 2, 64, FAKE, 4, None]
    a = list(ok); a[11] = 9
    assert d(*a) == _status("GPTQ_ERR_TOO_LARGE")      # m > 8
    a = list(ok); a[11] = 0
    assert d(*a) == _status("GPTQ_ERR_BAD_SIZE")
    a = list(ok); a[5] = 24
    assert d(*a) == _status("GPTQ_ERR_BAD_GROUP")
    a = list(ok); a[10] = 7
    assert d(*a) == _status("GPTQ_ERR_BAD_DTYPE")
    a = list(ok); a[14] = 3
    assert d(*a) == _status("GPTQ_ERR_BAD_LEADING_DIM")  # ld_y < d_row
    a = list(ok); a[3] = None
    assert d(*a) == _status("GPTQ_ERR_NULL_POINTER")


def test_dequantize_validation():
    f = G.library().gptq_dequantize
    ok = [FAKE, 4, 64, 64, FAKE, FAKE, 16, None, FAKE, 0, 64, None]
    a = list(ok); a[1] = 0
    assert f(*a) == _status("GPTQ_ERR_BAD_SIZE")
    a = list(ok); a[0] = None
    assert f(*a) == _status("GPTQ_ERR_NULL_POINTER")
    a = list(ok); a[8] = None
    assert f(*a) == _status("GPTQ_ERR_NULL_POINTER")
    a = list(ok); a[9] = 5
    assert f(*a) == _status("GPTQ_ERR_BAD_DTYPE")
    a = list(ok); a[6] = -1
    assert f(*a) == _status("GPTQ_ERR_BAD_GROUP")
    a = list(ok); a[3] = 63
    assert f(*a) == _status("GPTQ_ERR_BAD_LEADING_DIM")
    a = list(ok); a[10] = 10
    assert f(*a) == _status("GPTQ_ERR_BAD_LEADING_DIM")
    a = list(ok); a[2] = (1 << 20) + 1; a[3] = a[2]; a[10] = a[2]
    assert f(*a) == _status("GPTQ_ERR_TOO_LARGE")


def test_gptq2d_validation():
    assert "gptq2d_quantize" in _declared()
    f = G.library().gptq2d_quantize
    need = G.gptq2d_quantize_workspace_size(64, 48)
    assert need > 64 * 48 * 4 and G.gptq2d_quantize_workspace_size(0, 48) == 0
    ok = [FAKE, 0, 64, 48, 48, FAKE, FAKE, 4, FAKE, 48, FAKE, FAKE, FAKE, FAKE, need, None]
    a = list(ok); a[2] = 0
    assert f(*a) == _status("GPTQ_ERR_BAD_SIZE")
    a = list(ok); a[5] = None
    assert f(*a) == _status("GPTQ_ERR_NULL_POINTER")
    a = list(ok); a[1] = 3
    assert f(*a) == _status("GPTQ_ERR_BAD_DTYPE")
    a = list(ok); a[7] = 9
    assert f(*a) == _status("GPTQ_ERR_BAD_BITS")
    a = list(ok); a[4] = 47
    assert f(*a) == _status("GPTQ_ERR_BAD_LEADING_DIM")
    a = list(ok); a[9] = 40
    assert f(*a) == _status("GPTQ_ERR_BAD_LEADING_DIM")
    a = list(ok); a[14] = need - 1
    assert f(*a) == _status("GPTQ_ERR_WORKSPACE")
    a = list(ok); a[3] = (1 << 20) + 1; a[4] = a[3]; a[9] = a[3]
    assert f(*a) == _status("GPTQ_ERR_TOO_LARGE")


def test_noalloc_validation_and_scratch_limit():
    f = G.library().gptq_quantize_layer_noalloc
    assert G.GPTQ_NOALLOC_SCRATCH_BYTES == 96 << 20
    text = open(HEADER).read()
    assert "#define GPTQ_NOALLOC_SCRATCH_BYTES (96ull << 20)" in text
    # same argument checks as gptq_quantize_layer, all before any device call
    assert f(FAKE, 1, 0, 64, 64, FAKE, FAKE, 4, 0, 128, FAKE, FAKE, FAKE, FAKE, None) == _status("GPTQ_ERR_BAD_SIZE")
    assert f(None, 1, 8, 64, 64, FAKE, FAKE, 4, 0, 128, FAKE, FAKE, FAKE, FAKE, None) == _status("GPTQ_ERR_NULL_POINTER")
    assert f(FAKE, 1, 8, 64, 64, FAKE, FAKE, 9, 0, 128, FAKE, FAKE, FAKE, FAKE, None) == _status("GPTQ_ERR_BAD_BITS")
    assert f(FAKE, 1, 8, 64, 64, FAKE, FAKE, 4, 24, 128, FAKE, FAKE, FAKE, FAKE, None) == _status("GPTQ_ERR_BAD_GROUP")
    assert f(FAKE, 1, 8, 64, 32, FAKE, FAKE, 4, 0, 128, FAKE, FAKE, FAKE, FAKE, None) == _status("GPTQ_ERR_BAD_LEADING_DIM")
    # the limit is the workspace query against the fixed array
    fits = G.gptq_quantize_layer_workspace_size(4096, 4096, 128)
    assert 0 < fits <= G.GPTQ_NOALLOC_SCRATCH_BYTES
    big = G.gptq_quantize_layer_workspace_size(4096, 8192, 128)
    assert big > G.GPTQ_NOALLOC_SCRATCH_BYTES
    assert f(FAKE, 1, 4096, 8192, 8192, FAKE, FAKE, 4, 128, 128, FAKE, FAKE, FAKE, FAKE, None) == \
        _status("GPTQ_ERR_SCRATCH")
    assert "no-allocation" in G.gptq_status_string(12)


def test_launch_timing_host_side():
    G.gptq_launch_timing(True)
    assert G.gptq_launch_timing_read(G.TIMING_PANEL) == (0.0, 0, 0.0)   # nothing recorded yet
    G.gptq_launch_timing(False)
    f = G.library().gptq_launch_timing_read
    import ctypes
    ms, n, w = ctypes.c_double(), ctypes.c_int64(), ctypes.c_double()
    assert f(7, ctypes.byref(ms), ctypes.byref(n), ctypes.byref(w)) == _status("GPTQ_ERR_BAD_SIZE")
    assert f(0, None, ctypes.byref(n), ctypes.byref(w)) == _status("GPTQ_ERR_NULL_POINTER")
