"""The C ABI library: it loads, exports every symbol the header declares, and
rejects bad arguments on the host before touching the GPU (CPU only).

Only argument-checking paths are called here: each returns before any HIP
call, so no GPU is needed.
"""

import ctypes
import glob
import os
import re

import pytest

import dequant_gemv_rht_amd as dq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"^(?:wq_status|size_t|const char \*)\s*(\w+)\s*\(", text, flags=re.M))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dq.LIB_PATH):
        pytest.fail("libwq.so is not built: run python -m dequant_gemv_rht_amd.build")
    return dq.lib()


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ["wq_pack", "rht_apply", "wq_linear", "wq_quantize", "wq_unpack",
                     "wq_linear_workspace", "wq_linear_batch", "wq_packed_words", "wq_last_error",
                     "wq_stream_read"]:
        assert required in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in dq.SIGNATURES, f"binding lacks {name}"


def test_binding_names_match_abi():
    for name in ["wq_pack", "rht_apply", "wq_linear", "wq_quantize", "wq_unpack", "wq_linear_batch",
                 "wq_linear_workspace", "wq_packed_words"]:
        assert callable(getattr(dq, name)), name


def test_packed_words(lib):
    assert lib.wq_packed_words(4, 512, 1024, None) == 512 * 1024 // 8
    assert lib.wq_packed_words(3, 10, 128, None) == 10 * 12
    assert lib.wq_packed_words(6, 10, 128, None) == 10 * 24
    assert lib.wq_packed_words(8, 10, 128, None) == 10 * 32
    sel = (ctypes.c_uint8 * 3)(6, 8, 6)
    assert lib.wq_packed_words(0, 192, 128, sel) == 64 * 24 + 64 * 32 + 64 * 24
    assert lib.wq_packed_words(5, 10, 128, None) == 0
    assert "bits=5" in lib.wq_last_error().decode()
    assert lib.wq_packed_words(4, 10, 100, None) == 0
    bad = (ctypes.c_uint8 * 1)(7)
    assert lib.wq_packed_words(0, 64, 128, bad) == 0


def _weight(**kw):
    base = dict(bits=4, group=128, n=64, k=256, codes=16, scales=16, zeros=16, block_bits=None,
                block_off=None, rht_signs=None, rht_block=0)
    base.update(kw)
    return dq.WqWeight(**base)


@pytest.mark.parametrize("kw,status,text", [
    (dict(bits=5), dq.WQ_E_UNSUPPORTED, "bits=5"),
    (dict(group=64), dq.WQ_E_UNSUPPORTED, "group"),
    (dict(k=200), dq.WQ_E_ARG, "multiple of 128"),
    (dict(n=0), dq.WQ_E_ARG, "positive"),
    (dict(codes=None), dq.WQ_E_ARG, "non-NULL"),
    (dict(codes=8), dq.WQ_E_ALIGN, "aligned"),
    (dict(bits=0, n=96), dq.WQ_E_ARG, "n % 64"),
    (dict(bits=0), dq.WQ_E_ARG, "block_bits"),
    (dict(rht_signs=16, rht_block=64), dq.WQ_E_UNSUPPORTED, "rht_block"),
])
def test_linear_rejects_bad_weights(lib, kw, status, text):
    w = _weight(**kw)
    st = lib.wq_linear(ctypes.byref(w), 16, 1, 256, 16, dq.WQ_F16, 64, 0, 16, 1 << 20, None)
    assert st == status
    assert text in lib.wq_last_error().decode()


def test_linear_rejects_bad_host_widths(lib):
    # the optional host copy of a mixed layout's widths is read on the host
    # and refused (before anything is launched) unless every value is 6 or 8
    good = (ctypes.c_uint8 * 2)(6, 8)
    bad = (ctypes.c_uint8 * 2)(6, 7)
    for bh, text in ((bad, "block_bits_host[1]=7"), (good, "y_dtype")):
        # a good copy passes the weight checks and meets the next defect (the
        # output type), so nothing is launched either way
        w = _weight(bits=0, n=128, block_bits=16, block_off=16, block_bits_host=ctypes.addressof(bh))
        st = lib.wq_linear(ctypes.byref(w), 16, 1, 256, 16, 7, 128, 0, 16, 1 << 20, None)
        assert st == dq.WQ_E_ARG and text in lib.wq_last_error().decode()


@pytest.mark.parametrize("args,status,text", [
    (dict(m=0), dq.WQ_E_ARG, "m=0"),
    (dict(x=None), dq.WQ_E_ARG, "non-NULL"),
    (dict(x=24), dq.WQ_E_ALIGN, "aligned"),
    (dict(ldx=100), dq.WQ_E_ARG, "ldx"),
    (dict(ldx=260), dq.WQ_E_ALIGN, "multiple of 8"),
    (dict(ldy=10), dq.WQ_E_ARG, "ldy"),
    (dict(ydt=7), dq.WQ_E_ARG, "y_dtype"),
    (dict(flags=2), dq.WQ_E_ARG, "flags"),
    (dict(ws=0, m=64, signs=16, flags=1), dq.WQ_E_WORKSPACE, "workspace"),
    (dict(ws=64 * 256, m=64, signs=16, flags=1), dq.WQ_E_WORKSPACE, "workspace"),
])
def test_linear_rejects_bad_io(lib, args, status, text):
    a = dict(m=1, x=16, ldx=256, y=16, ydt=dq.WQ_F16, ldy=64, flags=0, ws=1 << 20, k=256, signs=None)
    a.update(args)
    w = _weight(k=a["k"], rht_signs=a["signs"], rht_block=128 if a["signs"] else 0)
    st = lib.wq_linear(ctypes.byref(w), a["x"], a["m"], a["ldx"], a["y"], a["ydt"], a["ldy"], a["flags"],
                       16, a["ws"], None)
    assert st == status, lib.wq_last_error()
    assert text in lib.wq_last_error().decode()


def _arranged(k, m):
    # the batch-tile GEMV's arranged activations: 80 bytes per 32 elements
    # and batch row, rounded up to 256 bytes
    return (m * (k // 32) * 80 + 255) // 256 * 256


def test_workspace_sizes(lib):
    # batch 1: the GEMV keeps everything in LDS, no workspace at any K
    assert lib.wq_linear_workspace(ctypes.byref(_weight()), 1) == 0
    w = _weight(n=4096, k=2560, rht_signs=16, rht_block=128)
    assert lib.wq_linear_workspace(ctypes.byref(w), 1) == 0
    # 2..16 rows: the arranged activations of all m rows
    for m in (2, 3, 4, 16):
        assert lib.wq_linear_workspace(ctypes.byref(w), m) == _arranged(2560, m)
    # without rotation the activations are still arranged (pair order, sums)
    w_plain = _weight(n=4096, k=2560)
    assert lib.wq_linear_workspace(ctypes.byref(w_plain), 4) == _arranged(2560, 4)
    # the mixed 6/8-bit layout runs the tiled GEMV, which needs none
    w_mixed = _weight(bits=0, n=128, k=256, block_bits=16, block_off=16)
    assert lib.wq_linear_workspace(ctypes.byref(w_mixed), 16) == 0
    # the matrix-core path (m >= 17) stages the rotated activations, fp16 [m][k]
    for m in (17, 63, 64):
        assert lib.wq_linear_workspace(ctypes.byref(w), m) >= m * 2560 * 2
    assert lib.wq_linear_workspace(ctypes.byref(w), 0) == ctypes.c_size_t(-1).value


def test_other_entry_points_reject(lib):
    assert lib.rht_apply(16, 16, 16, 1, 256, 256, 256, 64, None) == dq.WQ_E_UNSUPPORTED
    assert lib.rht_apply(16, 16, 16, 1, 100, 256, 256, 128, None) == dq.WQ_E_ARG
    assert lib.rht_apply(16, 16, 16, 1, 256, 264, 256, 128, None) == dq.WQ_E_ARG
    assert lib.wq_pack(7, 4, 128, 16, None, 16, None, None) == dq.WQ_E_UNSUPPORTED
    assert lib.wq_pack(0, 64, 128, 16, None, 16, None, None) == dq.WQ_E_ARG
    assert lib.wq_unpack(4, 4, 128, None, None, None, 16, None) == dq.WQ_E_ARG
    assert lib.wq_quantize(4, 4, 100, 16, None, None, 16, 16, 16, None) == dq.WQ_E_ARG
    assert lib.wq_quantize(4, 4, 128, 16, 8, None, 16, 16, 16, None) == dq.WQ_E_ALIGN
    arr = (dq.WqWeight * 2)(_weight(), _weight(bits=3))
    xs = (ctypes.c_void_p * 2)(16, 16)
    lds = (ctypes.c_int64 * 2)(256, 256)
    ys = (ctypes.c_void_p * 2)(16, 16)
    dts = (ctypes.c_int32 * 2)(dq.WQ_F16, dq.WQ_F16)
    ldy = (ctypes.c_int64 * 2)(64, 64)
    assert lib.wq_linear_batch(2, arr, xs, lds, 1, ys, dts, ldy, 0, 16, 1 << 20, None) == dq.WQ_E_UNSUPPORTED
    assert "one code width" in lib.wq_last_error().decode()
    assert lib.wq_linear_batch(9, arr, xs, lds, 1, ys, dts, ldy, 0, 16, 1 << 20, None) == dq.WQ_E_ARG
    assert lib.wq_linear_batch(2, arr, xs, lds, 0, ys, dts, ldy, 0, 16, 1 << 20, None) == dq.WQ_E_ARG


def test_batch_workspace_for_large_m(lib):
    # m = 1: no workspace; 2 <= m <= 16: every linear's arranged activations
    # side by side; m >= 17: one matrix-core launch over all the linears,
    # whose workspace holds every linear's rotated activations (fp16 [m][k])
    # and the fp32 partial sums of split K
    sg = dict(rht_signs=16, rht_block=128)
    arr = (dq.WqWeight * 2)(_weight(n=256, k=2560, **sg), _weight(n=128, k=9728, **sg))
    assert lib.wq_linear_batch_workspace(2, arr, 1) == 0
    assert lib.wq_linear_batch_workspace(2, arr, 16) == _arranged(2560, 16) + _arranged(9728, 16)
    assert lib.wq_linear_batch_workspace(2, arr, 5) == _arranged(2560, 5) + _arranged(9728, 5)
    assert lib.wq_linear_batch_workspace(2, arr, 40) >= 40 * (2560 + 9728) * 2
    need = lib.wq_linear_batch_workspace(2, arr, 512)
    assert need >= 512 * (2560 + 9728) * 2
    assert need >= lib.wq_linear_workspace(ctypes.byref(arr[0]), 512)
    xs = (ctypes.c_void_p * 2)(16, 16)
    lds = (ctypes.c_int64 * 2)(2560, 9728)
    ys = (ctypes.c_void_p * 2)(16, 16)
    dts = (ctypes.c_int32 * 2)(dq.WQ_F16, dq.WQ_F16)
    ldy = (ctypes.c_int64 * 2)(256, 128)
    st = lib.wq_linear_batch(2, arr, xs, lds, 512, ys, dts, ldy, dq.WQ_FUSE_RHT, 16, need - 256, None)
    assert st == dq.WQ_E_WORKSPACE


def test_matrix_core_path_workspace_covers_rotated_activations(lib):
    # the matrix-core path rotates the activations into the workspace first,
    # so the workspace must hold fp16 [m][k] and a smaller one is refused
    # before anything is launched.
    w = _weight(n=256, k=2560, rht_signs=16, rht_block=128)
    need = lib.wq_linear_workspace(ctypes.byref(w), 512)
    assert need >= 512 * 2560 * 2
    st = lib.wq_linear(ctypes.byref(w), 16, 512, 2560, 16, dq.WQ_F16, 256, dq.WQ_FUSE_RHT, 16, 16, None)
    assert st == dq.WQ_E_WORKSPACE
    assert "workspace" in lib.wq_last_error().decode()


def test_stream_read_rejects_bad_arguments(lib):
    assert lib.wq_stream_read(None, 16, 16, None) == dq.WQ_E_ARG
    assert lib.wq_stream_read(16, 0, 16, None) == dq.WQ_E_ARG
    assert lib.wq_stream_read(16, 24, 16, None) == dq.WQ_E_ARG
    assert lib.wq_stream_read(8, 16, 16, None) == dq.WQ_E_ALIGN


def test_embed_rejects_bad_arguments(lib):
    # every check runs before anything touches the device
    def call(w, ids=16, count=4, out=16, dt=dq.WQ_F16, ldo=2560):
        return lib.wq_embed(ctypes.byref(w), ids, count, out, dt, ldo, None)
    table = _weight(bits=8, n=151936, k=2560)
    assert call(table, count=0, ids=None, out=None) == dq.WQ_OK         # nothing to do
    assert call(table, ids=None) == dq.WQ_E_ARG
    assert call(table, out=None) == dq.WQ_E_ARG
    assert call(table, count=-1) == dq.WQ_E_ARG
    assert call(table, ldo=2559) == dq.WQ_E_ARG
    assert call(table, dt=7) == dq.WQ_E_ARG
    assert call(table, ldo=2564) == dq.WQ_E_ALIGN                       # fp16 rows need ldo % 8 == 0
    assert call(table, out=24) == dq.WQ_E_ALIGN
    assert call(table, ids=18) == dq.WQ_E_ALIGN
    assert call(table, count=1 << 31) == dq.WQ_E_UNSUPPORTED
    assert call(_weight(bits=8, n=64, k=2560, rht_signs=16, rht_block=128)) == dq.WQ_E_UNSUPPORTED
    assert call(_weight(bits=0, n=64, k=2560, block_bits=16, block_off=16)) == dq.WQ_E_UNSUPPORTED
    assert call(_weight(bits=5, n=64, k=2560)) == dq.WQ_E_UNSUPPORTED
    assert b"wq_embed" in lib.wq_last_error()


def test_gemv_batch_rejects_small_workspace(lib):
    # above one batch row the GEMV arranges the activations in the workspace;
    # a missing or short one is refused before anything is launched
    sg = dict(rht_signs=16, rht_block=128)
    w = _weight(n=256, k=2560, **sg)
    need = lib.wq_linear_workspace(ctypes.byref(w), 4)
    assert need == _arranged(2560, 4)
    st = lib.wq_linear(ctypes.byref(w), 16, 4, 2560, 16, dq.WQ_F16, 256, dq.WQ_FUSE_RHT, 16, need - 16, None)
    assert st == dq.WQ_E_WORKSPACE
    arr = (dq.WqWeight * 1)(w)
    xs = (ctypes.c_void_p * 1)(16)
    lds = (ctypes.c_int64 * 1)(2560)
    ys = (ctypes.c_void_p * 1)(16)
    dts = (ctypes.c_int32 * 1)(dq.WQ_F16)
    ldy = (ctypes.c_int64 * 1)(256)
    st = lib.wq_linear_batch(1, arr, xs, lds, 4, ys, dts, ldy, dq.WQ_FUSE_RHT, None, 0, None)
    assert st == dq.WQ_E_WORKSPACE


def test_noalloc_refuses_a_call_beyond_its_scratch(lib):
    # the size check runs on the host before the scratch or any kernel is
    # touched: 4096 rows of K = 9728 need ~80 MB of rotated activations
    w = _weight(n=256, k=9728, rht_signs=16, rht_block=128)
    need = lib.wq_linear_batch_workspace(1, ctypes.byref(w), 4096)
    assert need > dq.NOALLOC_SCRATCH_BYTES
    xs, lds, ys = (ctypes.c_void_p * 1)(16), (ctypes.c_int64 * 1)(9728), (ctypes.c_void_p * 1)(16)
    dts, ldys = (ctypes.c_int32 * 1)(dq.WQ_F16), (ctypes.c_int64 * 1)(256)
    st = lib.wq_linear_batch_noalloc(1, ctypes.byref(w), xs, lds, 4096, ys, dts, ldys, dq.WQ_FUSE_RHT, None)
    assert st == dq.WQ_E_WORKSPACE
    assert "static scratch" in lib.wq_last_error().decode()


@pytest.mark.parametrize("bits", [0, 4])
def test_grouped_workspace_matches_single_linear(lib, bits):
    # one linear through the grouped call takes the same path as wq_linear,
    # so it must reserve the same workspace, at every batch size (a grouped
    # workspace sized for the GEMV while the call ran the matrix-core path
    # would be written past its end)
    kw = dict(bits=bits, n=2560, k=9728, rht_signs=16, rht_block=128)
    if bits == 0:
        kw.update(block_bits=16, block_off=16)
    w = _weight(**kw)
    for m in (1, 2, 8, 16, 17, 31, 32, 33, 63, 64, 65, 128, 512):
        single = lib.wq_linear_workspace(ctypes.byref(w), m)
        group = lib.wq_linear_batch_workspace(1, ctypes.byref(w), m)
        assert single == group, (bits, m, single, group)


def test_sizes_beyond_32_bit_offsets_are_refused_before_launch(lib):
    # the kernels address activations, codes, scales and zeros with 32-bit
    # buffer offsets: larger requests are refused on the host, on the
    # batch-tile, batch-1 and matrix-core paths alike (nothing is launched:
    # no GPU here)
    for m, ldx, k in ((1, 1 << 30, 256), (4, 1 << 28, 256), (64, 1 << 24, 256), (512, 1 << 21, 256)):
        w = _weight(k=k, rht_signs=16, rht_block=128)
        st = lib.wq_linear(ctypes.byref(w), 16, m, ldx, 16, dq.WQ_F16, 64, dq.WQ_FUSE_RHT, 16, 1 << 50, None)
        assert st == dq.WQ_E_UNSUPPORTED, (m, ldx, lib.wq_last_error())
        assert "activations" in lib.wq_last_error().decode()
    w = _weight(k=1 << 27)
    st = lib.wq_linear(ctypes.byref(w), 16, 1, 1 << 27, 16, dq.WQ_F16, 64, 0, 16, 1 << 50, None)
    assert st == dq.WQ_E_UNSUPPORTED and "k=" in lib.wq_last_error().decode()
    w = _weight(bits=8, n=1 << 20, k=1 << 12)
    st = lib.wq_linear(ctypes.byref(w), 16, 64, 1 << 12, 16, dq.WQ_F16, 1 << 20, 0, 16, 1 << 50, None)
    assert st == dq.WQ_E_UNSUPPORTED and "4 GiB" in lib.wq_last_error().decode()
    arr = (dq.WqWeight * 2)(_weight(), _weight(k=1 << 27))
    xs = (ctypes.c_void_p * 2)(16, 16)
    lds = (ctypes.c_int64 * 2)(256, 1 << 27)
    ys = (ctypes.c_void_p * 2)(16, 16)
    dts = (ctypes.c_int32 * 2)(dq.WQ_F16, dq.WQ_F16)
    ldy = (ctypes.c_int64 * 2)(64, 64)
    assert lib.wq_linear_batch(2, arr, xs, lds, 1, ys, dts, ldy, 0, 16, 1 << 50, None) == dq.WQ_E_UNSUPPORTED
