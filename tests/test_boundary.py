"""The C-ABI library: it builds, loads, exports every symbol include/qlin.h
declares, and validates arguments on the host (no GPU needed: every error
except QLIN_ERR_HIP / QLIN_ERR_NO_DEVICE is raised before any HIP call)."""
import ctypes
import os
import re

import pytest
import torch

import oracle
from group_wise_bit_amd import qlin

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qlin.h")

OK, NULL, SHAPE, BITS, GROUP, ALIGN, FORMAT, ALIAS, WORKSPACE, NODEV, HIP = range(11)
FAKE = 0x7F0000000000        # a 16-byte aligned address that is never dereferenced


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qlin_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return qlin.library()


def test_exports_every_declared_symbol(lib):
    declared = header_functions()
    assert len(declared) == 21
    assert sorted(qlin.EXPORTS) == declared
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code, name in qlin.STATUS_NAMES.items():
        assert lib.qlin_status_string(code).decode().startswith(name)
    assert b"unknown" in lib.qlin_status_string(99)
    assert lib.qlin_abi_version() == 1


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("n,k", [(1, 64), (63, 128), (64, 64), (65, 896), (896, 896), (151936, 896)])
def test_size_queries_match_layout(lib, bits, n, k):
    assert lib.qlin_packed_bytes(n, k, bits) == 4 * oracle.packed_words(n, k, bits)
    t = oracle.n_tiles(n)
    assert lib.qlin_meta_entries(n, k, 64) == t * 64 * (k // 64)
    assert lib.qlin_meta_entries(n, k, k) == t * 64


def test_size_queries_reject(lib):
    assert lib.qlin_packed_bytes(0, 64, 4) == 0
    assert lib.qlin_packed_bytes(8, 100, 4) == 0
    assert lib.qlin_packed_bytes(8, 64, 1) == 0
    assert lib.qlin_packed_bytes(8, 64, 9) == 0
    assert lib.qlin_packed_bytes(8, 64, 16) == 0
    assert lib.qlin_meta_entries(8, 128, 32) == 0


def quant(lib, w=FAKE, ld=128, n=8, k=128, bits=4, group=64, codes=FAKE + (1 << 30),
          scale=FAKE + (2 << 30), zero=FAKE + (3 << 30)):
    return lib.qlin_quantize(w, ld, n, k, bits, group, codes, scale, zero, None)


def test_quantize_validation(lib):
    assert quant(lib, w=None) == NULL
    assert quant(lib, scale=None) == NULL
    assert quant(lib, zero=None) == NULL
    assert quant(lib, n=0) == SHAPE
    assert quant(lib, k=100) == SHAPE
    assert quant(lib, k=0) == SHAPE
    assert quant(lib, ld=64) == SHAPE
    assert quant(lib, ld=132) == ALIGN
    assert quant(lib, bits=1) == BITS
    assert quant(lib, bits=9) == BITS
    assert quant(lib, bits=16) == BITS
    assert quant(lib, group=32) == GROUP
    assert quant(lib, group=256) == GROUP
    assert quant(lib, w=FAKE + 8) == ALIGN
    assert quant(lib, codes=FAKE + 4) == ALIGN
    assert quant(lib, scale=FAKE) == ALIAS
    assert quant(lib, codes=FAKE + 256) == ALIAS
    assert quant(lib, zero=FAKE + (2 << 30) + 16) == ALIAS


def weight(**kw):
    d = dict(n=8, k=128, bits=4, group=64, format=0, reserved=0, data=FAKE, ld=0,
             scale=FAKE + (1 << 30), zero=FAKE + (2 << 30))
    d.update(kw)
    return qlin.QlinWeightC(d["n"], d["k"], d["bits"], d["group"], d["format"], d["reserved"],
                            d["data"], d["ld"], d["scale"], d["zero"])


def gemv(lib, w, x=FAKE + (3 << 30), y=FAKE + (4 << 30), ws=None, wsb=0):
    return lib.qlin_gemv(ctypes.byref(w), x, y, ws, wsb, None)


def gemm(lib, w, X=FAKE + (3 << 30), m=4, ldx=128, Y=FAKE + (4 << 30), ldy=8, ws=None, wsb=0):
    return lib.qlin_gemm(ctypes.byref(w), X, m, ldx, Y, ldy, ws, wsb, None)


def test_gemv_validation(lib):
    assert lib.qlin_gemv(None, FAKE, FAKE, None, 0, None) == NULL
    assert gemv(lib, weight(data=None)) == NULL
    assert gemv(lib, weight(scale=None)) == NULL
    assert gemv(lib, weight(), x=None) == NULL
    assert gemv(lib, weight(), y=None) == NULL
    assert gemv(lib, weight(n=0)) == SHAPE
    assert gemv(lib, weight(k=96)) == SHAPE
    assert gemv(lib, weight(ld=128)) == SHAPE           # packed weights take no pitch
    assert gemv(lib, weight(bits=16)) == BITS           # 16 only with fp16 masters
    assert gemv(lib, weight(bits=1)) == BITS
    assert gemv(lib, weight(bits=9)) == BITS            # packed: 2 .. 8
    assert gemv(lib, weight(format=1, ld=128, bits=9)) == BITS
    assert gemv(lib, weight(group=128 + 64, k=128)) == GROUP
    assert gemv(lib, weight(format=3)) == FORMAT
    assert gemv(lib, weight(reserved=1)) == FORMAT
    assert gemv(lib, weight(data=FAKE + 4)) == ALIGN
    assert gemv(lib, weight(), x=FAKE + (3 << 30) + 2) == ALIGN
    assert gemv(lib, weight(format=1, ld=64)) == SHAPE
    assert gemv(lib, weight(format=1, ld=132)) == ALIGN
    assert gemv(lib, weight(), y=FAKE + 64) == ALIAS    # y inside the codes
    assert gemv(lib, weight(), y=FAKE + (3 << 30) + 16) == ALIAS
    assert gemv(lib, weight(), ws=FAKE + (4 << 30), wsb=64) == ALIAS
    assert gemv(lib, weight(), ws=FAKE + (5 << 30), wsb=-1) == WORKSPACE


def test_gemm_validation(lib):
    assert gemm(lib, weight(), X=None) == NULL
    assert gemm(lib, weight(), m=0) == SHAPE
    assert gemm(lib, weight(), ldx=64) == SHAPE
    assert gemm(lib, weight(), ldy=4) == SHAPE
    assert gemm(lib, weight(), ldx=132) == ALIGN
    assert gemm(lib, weight(format=1, ld=128)) == FORMAT  # GEMM takes packed weights only
    assert gemm(lib, weight(), Y=FAKE + (3 << 30)) == ALIAS


def weights(*ws):
    return (qlin.QlinWeightC * len(ws))(*ws)


def ptrs(*ps):
    return (ctypes.c_void_p * len(ps))(*ps)


Y0, Y1, Y2 = FAKE + (4 << 30), FAKE + (5 << 30), FAKE + (6 << 30)


def multi(lib, ws, ys, x=FAKE + (3 << 30), count=None, ws_=None, wsb=0):
    count = len(ws) if count is None else count
    return lib.qlin_gemv_multi(weights(*ws), count, x, ptrs(*ys), ws_, wsb, None)


def swiglu(lib, g, u, x=FAKE + (3 << 30), h=Y0, h16=Y1, ws_=None, wsb=0):
    return lib.qlin_gemv_swiglu(ctypes.byref(g), ctypes.byref(u), x, h, h16, ws_, wsb, None)


def other_weight(i, **kw):
    # a second / third weight at its own addresses
    base = FAKE + ((8 + 4 * i) << 30)
    d = dict(data=base, scale=base + (1 << 30), zero=base + (2 << 30))
    d.update(kw)
    return weight(**d)


def test_gemv_multi_validation(lib):
    w0, w1, w2 = weight(), other_weight(0, n=200), other_weight(1, n=1)
    assert lib.qlin_gemv_multi(None, 1, FAKE, ptrs(Y0), None, 0, None) == NULL
    assert lib.qlin_gemv_multi(weights(w0), 1, FAKE + (3 << 30), None, None, 0, None) == NULL
    assert multi(lib, [w0], [None]) == NULL
    assert multi(lib, [w0], [Y0], x=None) == NULL
    assert multi(lib, [w0], [Y0], count=0) == SHAPE
    assert multi(lib, [w0, w1, w2, w0, w1], [Y0, Y1, Y2, Y0, Y1]) == SHAPE   # at most 4
    assert multi(lib, [w0, other_weight(0, k=256)], [Y0, Y1]) == SHAPE      # one k
    assert multi(lib, [w0, other_weight(0, bits=3)], [Y0, Y1]) == FORMAT
    assert multi(lib, [w0, other_weight(0, group=128)], [Y0, Y1]) == FORMAT
    assert multi(lib, [w0, other_weight(0, format=1, ld=128)], [Y0, Y1]) == FORMAT
    assert multi(lib, [w0, w1], [Y0, Y0 + 16]) == ALIAS                     # outputs overlap
    assert multi(lib, [w0, w1], [Y0, FAKE + (8 << 30) + 64]) == ALIAS       # y inside w1
    assert multi(lib, [w0, w1], [Y0, FAKE + (3 << 30)]) == ALIAS            # y on x
    assert multi(lib, [w0, w1], [Y0, Y1 + 4]) == ALIGN
    assert multi(lib, [w0, w1], [Y0, Y1], ws_=Y1, wsb=64) == ALIAS
    assert multi(lib, [w0, w1], [Y0, Y1], ws_=FAKE + (7 << 30), wsb=-1) == WORKSPACE


def test_gemv_swiglu_validation(lib):
    g, u = weight(), other_weight(0)
    assert lib.qlin_gemv_swiglu(None, ctypes.byref(u), FAKE, Y0, Y1, None, 0, None) == NULL
    assert swiglu(lib, g, u, h=None, h16=None) == NULL
    assert swiglu(lib, g, u, x=None) == NULL
    assert swiglu(lib, g, other_weight(0, n=16)) == SHAPE
    assert swiglu(lib, g, other_weight(0, k=256)) == SHAPE
    assert swiglu(lib, g, other_weight(0, bits=8)) == FORMAT
    assert swiglu(lib, g, other_weight(0, format=1, ld=128)) == FORMAT
    assert swiglu(lib, g, u, h16=Y0 + 16) == ALIAS                          # h16 inside h
    assert swiglu(lib, g, u, h=FAKE + 32) == ALIAS                           # h on gate codes
    assert swiglu(lib, g, u, h16=Y1 + 2) == ALIGN


def embed(lib, w, ids=FAKE + (3 << 30), count=4, o16=Y0, o32=Y1, ld=128):
    return lib.qlin_embed_rows(ctypes.byref(w), ids, count, o16, o32, ld, None)


def test_embed_rows_validation(lib):
    assert lib.qlin_embed_rows(None, FAKE, 1, Y0, None, 128, None) == NULL
    assert embed(lib, weight(), count=0) == OK                  # nothing to do, no device needed
    assert embed(lib, weight(), ids=None) == NULL
    assert embed(lib, weight(), o16=None, o32=None) == NULL
    assert embed(lib, weight(), count=-1) == SHAPE
    assert embed(lib, weight(), ld=64) == SHAPE
    assert embed(lib, weight(), ld=132) == ALIGN
    assert embed(lib, weight(), o16=Y0 + 2) == ALIGN
    assert embed(lib, weight(), ids=FAKE + (3 << 30) + 2) == ALIGN
    assert embed(lib, weight(format=1, ld=128)) == FORMAT
    assert embed(lib, weight(bits=16)) == BITS
    assert embed(lib, weight(), o32=Y0 + 64) == ALIAS            # outputs overlap
    assert embed(lib, weight(), o16=FAKE + 16) == ALIAS          # output on the codes
    assert embed(lib, weight(), o32=FAKE + (3 << 30)) == ALIAS   # output on the ids


def qjob(i, **kw):
    base = FAKE + ((20 + 4 * i) << 30)
    d = dict(w16=base, ld_w=128, n=8, k=128, codes=base + (1 << 30), scale=base + (2 << 30),
             zero=base + (3 << 30))
    d.update(kw)
    return qlin.QlinQuantJobC(d["w16"], d["ld_w"], d["n"], d["k"], d["codes"], d["scale"], d["zero"])


def qbatch(lib, jobs, bits=4, group=64, count=None):
    arr = (qlin.QlinQuantJobC * max(len(jobs), 1))(*jobs)
    return lib.qlin_quantize_batch(arr, len(jobs) if count is None else count, bits, group, None)


def test_quantize_batch_validation(lib):
    assert qbatch(lib, [], count=0) == OK
    assert lib.qlin_quantize_batch(None, 1, 4, 64, None) == NULL
    assert qbatch(lib, [qjob(0)], count=-1) == SHAPE
    assert qbatch(lib, [qjob(0)], group=128) == GROUP         # 64 or 0 (per row) only
    assert qbatch(lib, [qjob(0)], bits=9) == BITS
    assert qbatch(lib, [qjob(0), qjob(1, k=100)]) == SHAPE
    assert qbatch(lib, [qjob(0), qjob(1, scale=None)]) == NULL
    assert qbatch(lib, [qjob(0), qjob(1, ld_w=132)]) == ALIGN
    assert qbatch(lib, [qjob(0), qjob(1, zero=FAKE + (20 << 30))]) == ALIAS   # on job 0's master
    assert qbatch(lib, [qjob(0), qjob(1, codes=FAKE + (21 << 30) + 64)]) == ALIAS  # on job 0's codes


def gmulti(lib, ws, ys, lds, X=FAKE + (3 << 30), m=4, ldx=128, count=None, ws_=None, wsb=0):
    count = len(ws) if count is None else count
    return lib.qlin_gemm_multi(weights(*ws), count, X, m, ldx, ptrs(*ys),
                               (ctypes.c_int64 * len(lds))(*lds), ws_, wsb, None)


def test_gemm_multi_validation(lib):
    w0, w1 = weight(), other_weight(0, n=200)
    assert gmulti(lib, [w0, w1], [Y0, Y1], [8, 200], X=None) == NULL
    assert gmulti(lib, [w0, w1], [Y0, None], [8, 200]) == NULL
    assert gmulti(lib, [w0, w1], [Y0, Y1], [8, 200], count=5) == SHAPE
    assert gmulti(lib, [w0, w1], [Y0, Y1], [8, 100]) == SHAPE            # ld_y < n
    assert gmulti(lib, [w0, other_weight(0, k=256)], [Y0, Y1], [8, 8]) == SHAPE
    assert gmulti(lib, [w0, other_weight(0, bits=2)], [Y0, Y1], [8, 8]) == FORMAT
    assert gmulti(lib, [w0, w1], [Y0, Y0 + 64], [8, 200]) == ALIAS       # outputs overlap
    assert gmulti(lib, [w0, w1], [Y0, FAKE + 128], [8, 200]) == ALIAS    # output on w0 codes
    assert gmulti(lib, [w0, w1], [Y0, Y1 + 4], [8, 200]) == ALIGN
    assert gmulti(lib, [w0, w1], [Y0, Y1], [8, 200], m=0) == SHAPE
    assert lib.qlin_gemm_multi_workspace_bytes(weights(w0, w1), 2, 4) == 0
    big = weight(n=128, k=16384)
    assert lib.qlin_gemm_multi_workspace_bytes(weights(big, big), 2, 8) > 65536


def gswiglu(lib, g, u, X=FAKE + (3 << 30), m=4, ldx=128, H=Y0, H16=Y1, ldh=8, ws_=None, wsb=0):
    return lib.qlin_gemm_swiglu(ctypes.byref(g), ctypes.byref(u), X, m, ldx, H, H16, ldh, ws_,
                                wsb, None)


def test_gemm_swiglu_validation(lib):
    g, u = weight(), other_weight(0)
    assert lib.qlin_gemm_swiglu(None, ctypes.byref(u), FAKE, 4, 128, Y0, Y1, 8, None, 0,
                                None) == NULL
    assert gswiglu(lib, g, u, X=None) == NULL
    assert gswiglu(lib, g, u, H=None, H16=None) == NULL
    assert gswiglu(lib, g, other_weight(0, n=16)) == SHAPE                  # one n
    assert gswiglu(lib, g, other_weight(0, k=256)) == SHAPE                 # one k
    assert gswiglu(lib, g, other_weight(0, bits=8)) == FORMAT
    assert gswiglu(lib, g, other_weight(0, group=128)) == FORMAT
    assert gswiglu(lib, g, other_weight(0, format=1, ld=128)) == FORMAT     # packed only
    assert gswiglu(lib, g, u, m=0) == SHAPE
    assert gswiglu(lib, g, u, ldx=64) == SHAPE
    assert gswiglu(lib, g, u, ldh=4) == SHAPE
    assert gswiglu(lib, g, u, ldx=132) == ALIGN
    assert gswiglu(lib, g, u, H16=Y1 + 2) == ALIGN
    assert gswiglu(lib, g, u, H16=Y0 + 16) == ALIAS                         # H16 inside H
    assert gswiglu(lib, g, u, H=FAKE + 32) == ALIAS                         # H on gate codes
    assert gswiglu(lib, g, u, H16=FAKE + (8 << 30) + 64) == ALIAS           # H16 on up codes
    assert gswiglu(lib, g, u, H=FAKE + (3 << 30)) == ALIAS                  # H on X
    assert gswiglu(lib, g, u, ws_=Y0, wsb=64) == ALIAS
    assert gswiglu(lib, g, u, ws_=FAKE + (7 << 30), wsb=-1) == WORKSPACE
    assert lib.qlin_gemm_swiglu_workspace_bytes(ctypes.byref(g), 4) == 0
    big = weight(n=128, k=16384)               # two tiles, 256 K-blocks: split across groups
    assert lib.qlin_gemm_swiglu_workspace_bytes(ctypes.byref(big), 8) > 65536
    assert lib.qlin_gemm_swiglu_workspace_bytes(ctypes.byref(big), 0) == 0
    assert lib.qlin_gemm_swiglu_workspace_bytes(ctypes.byref(weight(bits=9)), 8) == 0


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-GPU path")
def test_no_device(lib):
    # calls that pass every host check (with fake addresses: never run on a GPU)
    assert quant(lib, bits=5, codes=None) == NODEV            # scale/zero only: any lever width
    assert gemv(lib, weight(format=1, ld=128, bits=6)) == NODEV
    assert qbatch(lib, [qjob(0, codes=None), qjob(1, codes=None)], group=0) == NODEV
    assert gmulti(lib, [weight(), other_weight(0, n=200)], [Y0, Y1], [8, 200]) == NODEV
    assert qbatch(lib, [qjob(0), qjob(1)]) == NODEV
    assert embed(lib, weight()) == NODEV
    assert quant(lib) == NODEV
    assert gemv(lib, weight()) == NODEV
    assert gemm(lib, weight()) == NODEV
    assert gemm(lib, weight(), m=64, ldy=64) == NODEV
    assert multi(lib, [weight(), other_weight(0)], [Y0, Y1]) == NODEV
    assert swiglu(lib, weight(), other_weight(0)) == NODEV
    assert swiglu(lib, weight(), other_weight(0), h=None) == NODEV
    assert gswiglu(lib, weight(), other_weight(0)) == NODEV
    assert gswiglu(lib, weight(), other_weight(0), H=None, m=300) == NODEV


def test_workspace_queries(lib):
    big = weight(n=128, k=16384)               # two tiles, 256 K-blocks: split across groups
    need = lib.qlin_gemv_workspace_bytes(ctypes.byref(big))
    assert need > 65536 and need % 4 == 0
    small = weight(n=151936, k=896)
    assert lib.qlin_gemv_workspace_bytes(ctypes.byref(small)) == 0
    assert lib.qlin_gemm_workspace_bytes(ctypes.byref(big), 8) > 65536
    assert lib.qlin_gemm_workspace_bytes(ctypes.byref(weight(bits=9)), 8) == 0
    # multi: the launch's tiles add up; swiglu: two partials per row
    pair = weights(big, big)
    assert lib.qlin_gemv_multi_workspace_bytes(pair, 2) >= need
    assert lib.qlin_gemv_multi_workspace_bytes(pair, 0) == 0
    assert lib.qlin_gemv_multi_workspace_bytes(weights(big, weight(k=256)), 2) == 0
    assert lib.qlin_gemv_swiglu_workspace_bytes(ctypes.byref(big)) > 65536


TUNE_HEADER = os.path.join(ROOT, "include", "qlin_tune.h")


def test_tune_header_exports(lib):
    text = re.sub(r"/\*.*?\*/", "", open(TUNE_HEADER).read(), flags=re.S)
    declared = sorted(set(re.findall(r"\b(qlin_[a-z0-9_]+)\s*\(", text)))
    assert declared == sorted(qlin.TUNE_EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_launch_override_validation(lib):
    """The sweep/test override is validated on the host; NULL clears it."""
    def ov(fam, vals):
        arr = None if vals is None else (ctypes.c_int32 * 3)(*vals)
        return lib.qlin_set_launch_override(fam, arr)
    assert ov(0, (16, 2, 64)) == OK
    assert ov(0, None) == OK
    assert ov(0, (12, 1, 64)) == SHAPE      # waves
    assert ov(0, (16, 0, 64)) == SHAPE      # splits
    assert ov(0, (16, 1, 32)) == SHAPE      # rows
    assert ov(1, (0, 1, 0)) == OK
    assert ov(1, (128, 3, 0)) == OK
    assert ov(1, (16, 1, 0)) == OK
    assert ov(1, (7, 1, 0)) == OK
    assert ov(1, (8, 1, 0)) == OK
    assert ov(1, (9, 1, 0)) == SHAPE
    assert ov(1, (96, 1, 0)) == SHAPE
    assert ov(1, None) == OK
    assert ov(2, (16, 1, 64)) == SHAPE
    qlin.set_launch_override("gemv", "8,2")     # rows default to whole tiles
    qlin.set_launch_override("gemv", None)
    with pytest.raises(qlin.QlinError):
        qlin.set_launch_override("gemm", (9, 1))


def _cpu_weight(n=128, k=128, bits=4):
    t = oracle.n_tiles(n) * 64
    return qlin.QWeight(n, k, bits, 64, qlin.FMT_PACKED,
                        torch.zeros(qlin.packed_bytes(n, k, bits) // 4, dtype=torch.int32),
                        torch.zeros(t * (k // 64), dtype=torch.float16),
                        torch.zeros(t * (k // 64), dtype=torch.uint8))


def test_binding_refuses_bad_outputs_before_any_launch():
    """The C ABI cannot see buffer sizes: the binding checks every output
    (dtype, device, unit-stride rows, room) and every x length first."""
    w = _cpu_weight()
    x = torch.zeros(128, dtype=torch.float16)
    with pytest.raises(TypeError):
        qlin.gemv(w, torch.zeros(64, dtype=torch.float16))
    with pytest.raises(TypeError):
        qlin.gemv(w, x, torch.zeros(128, dtype=torch.float16))
    with pytest.raises(ValueError):
        qlin.gemv(w, x, torch.zeros(127, dtype=torch.float32))
    with pytest.raises(ValueError):
        qlin.gemv(w, x, torch.zeros(128, dtype=torch.float32, device="meta"))
    with pytest.raises(ValueError):
        qlin.gemv(w, x, torch.zeros(256, dtype=torch.float32)[::2])
    X = torch.zeros(8, 128, dtype=torch.float16)
    with pytest.raises(ValueError):
        qlin.gemm(w, X, torch.zeros(8, 127, dtype=torch.float32))
    with pytest.raises(ValueError):
        qlin.gemm(w, X, torch.zeros(7, 128, dtype=torch.float32))
    with pytest.raises(TypeError):
        qlin.gemm(w, X, torch.zeros(8, 128, dtype=torch.float16))
    with pytest.raises(ValueError):
        qlin.gemm(w, X, torch.zeros(128, 8, dtype=torch.float32).t())
    with pytest.raises(TypeError):
        qlin.gemv_multi([w, w], torch.zeros(64, dtype=torch.float16))
    with pytest.raises(ValueError):
        qlin.gemv_multi([w, w], x, [torch.zeros(128), torch.zeros(100)])
    with pytest.raises(TypeError):
        qlin.gemv_swiglu(w, w, x, None, torch.zeros(128, dtype=torch.float32))
    with pytest.raises(ValueError):
        qlin.gemv_swiglu(w, w, x, torch.zeros(64, dtype=torch.float32), None)
    with pytest.raises(TypeError):
        qlin.gemv_swiglu(w, w, torch.zeros(127, dtype=torch.float16))
    with pytest.raises(ValueError):
        qlin.gemm_multi([w], X, [torch.zeros(8, 64, dtype=torch.float32)])
    with pytest.raises(ValueError):
        qlin.gemm_swiglu(w, w, X, None, torch.zeros(4, 128, dtype=torch.float16))
    with pytest.raises(TypeError):
        qlin.gemm_swiglu(w, w, X, torch.zeros(8, 128, dtype=torch.float16), None)


PEAKS_HEADER = os.path.join(ROOT, "include", "qlin_peaks.h")
PEAKS_LIB = os.path.join(ROOT, "group_wise_bit_amd", "libqlin_peaks.so")


def test_peaks_header_exports():
    """The measurement library loads and exports what its header declares;
    its host-side argument checks refuse bad reads before any launch."""
    if not os.path.exists(PEAKS_LIB):
        pytest.skip("libqlin_peaks.so not built")
    text = re.sub(r"/\*.*?\*/", "", open(PEAKS_HEADER).read(), flags=re.S)
    declared = sorted(set(re.findall(r"\b(qlin_[a-z0-9_]+)\s*\(", text)))
    assert declared == ["qlin_peak_mfma", "qlin_peak_mfma_waves", "qlin_peak_read_groups",
                        "qlin_peak_stream_read"]
    plib = ctypes.CDLL(PEAKS_LIB)
    for name in declared:
        assert hasattr(plib, name), name
    plib.qlin_peak_read_groups.restype = ctypes.c_int64
    plib.qlin_peak_mfma_waves.restype = ctypes.c_int64
    assert plib.qlin_peak_read_groups() == 16384
    assert plib.qlin_peak_mfma_waves() == 2048
    plib.qlin_peak_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                           ctypes.c_void_p]
    for src, nbytes in ((FAKE, 16 * 16384 + 8), (FAKE + 8, 16 * 16384), (FAKE, 16 * 100),
                        (None, 16 * 16384)):
        assert plib.qlin_peak_stream_read(src, nbytes, FAKE, None) != 0
