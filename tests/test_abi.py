"""The C-ABI library: it loads, exports everything include/dbf.h declares, and
validates arguments on the host before any HIP call.  No GPU is needed (and
no compute is attempted): on a host without a GPU a well-formed dbf_pack
returns DBF_ERR_HIP."""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import dbf_linear_fwd_amd as dbf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dbf.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dbf_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("dbf_pack", "dbf_linear_forward", "dbf_free"):
        assert required in names
    assert set(names) == set(dbf.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    L = dbf.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", dbf.library_path()], capture_output=True, text=True)
    exported = set(re.findall(r"\sT\s(dbf_[a-z_]+)$", out.stdout, flags=re.M))
    assert set(declared_functions()) <= exported


def test_header_compiles_as_c(tmp_path):
    """The header is plain C: it compiles in a C translation unit without HIP headers."""
    src = '#include "dbf.h"\nint main(void){ dbf_info_t i; (void)i; return (int)DBF_OK; }\n'
    c = os.path.join(str(tmp_path), "t.c")
    open(c, "w").write(src)
    res = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                          "-c", c, "-o", os.path.join(str(tmp_path), "t.o")], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr


def test_binding_constants_match_the_header(tmp_path):
    """Every status, path and flag value the binding uses is the header's:
    a C program built against dbf.h prints them."""
    names = ["DBF_OK", "DBF_ERR_INVALID_ARG", "DBF_ERR_SHAPE", "DBF_ERR_OOM", "DBF_ERR_HIP", "DBF_ERR_UNSUPPORTED",
             "DBF_PATH_AUTO", "DBF_PATH_DECODE", "DBF_PATH_PREFILL", "DBF_PATH_DECODE_TABLE", "DBF_PATH_DECODE_EXACT",
             "DBF_PACK_BACKWARD"]
    body = "".join(f'    printf("{n} %d\\n", (int){n});\n' for n in names)
    src = f'#include <stdio.h>\n#include "dbf.h"\nint main(void) {{\n{body}    return 0;\n}}\n'
    c = os.path.join(str(tmp_path), "consts.c")
    exe = os.path.join(str(tmp_path), "consts")
    open(c, "w").write(src)
    res = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), c, "-o", exe],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    out = subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split("\n")
    values = dict(line.split() for line in out if line)
    for n in names:
        assert int(values[n]) == getattr(dbf, n), n


def test_status_strings():
    for code in range(6):
        assert dbf.dbf_status_string(code)
    assert dbf.dbf_status_string(0) == "success"
    assert dbf.dbf_status_string(99) == "unknown status"


def _small():
    rng = np.random.default_rng(0)
    n, m, k = 8, 12, 4
    A = (1 - 2 * rng.integers(0, 2, size=(n, k))).astype(np.int8)
    B = (1 - 2 * rng.integers(0, 2, size=(k, m))).astype(np.int8)
    a = np.ones(n, np.float16).view(np.uint16)
    mid = np.ones(k, np.float16).view(np.uint16)
    b = np.ones(m, np.float16).view(np.uint16)
    return n, m, k, A, B, a, mid, b


def _raw_pack(n, m, k, A, B, a, mid, b, max_batch, out=True):
    L = dbf.lib()
    h = ctypes.c_void_p()
    p = lambda arr: None if arr is None else arr.ctypes.data
    return L.dbf_pack(n, m, k, p(A), p(B), p(a), p(mid), p(b), max_batch, ctypes.byref(h) if out else None), h


def test_pack_argument_validation_before_any_hip_call():
    n, m, k, A, B, a, mid, b = _small()
    E = dbf.DBF_ERR_INVALID_ARG
    assert _raw_pack(n, m, k, A, B, a, mid, b, 4, out=False)[0] == E
    assert _raw_pack(n, m, k, None, B, a, mid, b, 4)[0] == E
    assert _raw_pack(n, m, k, A, None, a, mid, b, 4)[0] == E
    assert _raw_pack(n, m, k, A, B, None, mid, b, 4)[0] == E
    assert _raw_pack(n, m, k, A, B, a, None, b, 4)[0] == E
    assert _raw_pack(n, m, k, A, B, a, mid, None, 4)[0] == E
    for bad in ((0, m, k), (n, 0, k), (n, m, 0), (-1, m, k)):
        assert _raw_pack(*bad, A, B, a, mid, b, 4)[0] == E
    assert _raw_pack(n, m, k, A, B, a, mid, b, 0)[0] == E
    A0 = A.copy()
    A0[3, 2] = 0
    st, h = _raw_pack(n, m, k, A0, B, a, mid, b, 4)
    assert st == E and h.value is None
    B0 = B.copy()
    B0[1, 5] = 3
    assert _raw_pack(n, m, k, A, B0, a, mid, b, 4)[0] == E
    # sizes whose byte counts overflow are a shape error
    big = 1 << 30
    assert _raw_pack(big + 1, m, k, A, B, a, mid, b, 4)[0] == dbf.DBF_ERR_SHAPE


def test_forward_and_info_validation():
    L = dbf.lib()
    assert L.dbf_linear_forward(None, None, None, 1, None) == dbf.DBF_ERR_INVALID_ARG
    assert L.dbf_linear_forward_ex(None, None, None, 1, 0, None) == dbf.DBF_ERR_INVALID_ARG
    assert L.dbf_get_info(None, None) == dbf.DBF_ERR_INVALID_ARG
    assert L.dbf_timing_enable(None, 1) == dbf.DBF_ERR_INVALID_ARG
    cnt = ctypes.c_int32()
    assert L.dbf_timing_read(None, None, 0, ctypes.byref(cnt)) == dbf.DBF_ERR_INVALID_ARG
    L.dbf_free(None)  # no-op


def _have_gpu():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.mark.skipif(_have_gpu(), reason="checks the no-GPU error path")
def test_pack_without_gpu_reports_hip_error():
    n, m, k, A, B, a, mid, b = _small()
    st, h = _raw_pack(n, m, k, A, B, a, mid, b, 4)
    assert st == dbf.DBF_ERR_HIP and h.value is None
    with pytest.raises(dbf.DbfError) as e:
        dbf.dbf_pack(n, m, k, A, B, a, mid, b, 4)
    assert e.value.status == dbf.DBF_ERR_HIP


def test_group_entry_validates_before_any_device_call():
    """Argument errors of dbf_linear_forward_group are reported without a GPU."""
    import ctypes
    L = dbf.lib()
    vp = ctypes.c_void_p
    null_hs = ctypes.POINTER(vp)()
    assert L.dbf_linear_forward_group(null_hs, 1, None, null_hs, 1, None) == dbf.DBF_ERR_INVALID_ARG
    hs = (vp * 1)(None)
    ys = (vp * 1)(None)
    assert L.dbf_linear_forward_group(hs, 0, None, ys, 1, None) == dbf.DBF_ERR_INVALID_ARG   # count 0
    assert L.dbf_linear_forward_group(hs, 9, None, ys, 1, None) == dbf.DBF_ERR_INVALID_ARG   # count > 8
    assert L.dbf_linear_forward_group(hs, 1, None, ys, 1, None) == dbf.DBF_ERR_INVALID_ARG   # null handle


def test_backward_entries_validate_before_any_device_call():
    import ctypes
    L = dbf.lib()
    A = np.ones((4, 3), np.int8)
    B = np.ones((3, 5), np.int8)
    a = np.ones(4, np.float16).view(np.uint16)
    mid = np.ones(3, np.float16).view(np.uint16)
    b = np.ones(5, np.float16).view(np.uint16)
    h = ctypes.c_void_p()
    p = lambda arr: arr.ctypes.data_as(ctypes.c_void_p)
    # unknown flag bits
    assert L.dbf_pack_ex(4, 5, 3, p(A), p(B), p(a), p(mid), p(b), 2, 6, ctypes.byref(h)) == dbf.DBF_ERR_INVALID_ARG
    assert h.value is None
    # null output pointer
    assert L.dbf_pack_ex(4, 5, 3, p(A), p(B), p(a), p(mid), p(b), 2, 1, None) == dbf.DBF_ERR_INVALID_ARG
    # null handles
    assert L.dbf_linear_backward_data(None, None, None, 1, None) == dbf.DBF_ERR_INVALID_ARG
    assert L.dbf_linear_backward(None, None, None, None, None, None, None, 1, None) == dbf.DBF_ERR_INVALID_ARG


def test_bqq_pack_validates_before_any_device_call():
    """dbf_bqq_pack reports argument errors (null pointers, sizes, entries
    other than 0/1) without touching a GPU; with valid arguments and no GPU
    it reports a HIP error and returns no handle."""
    L = dbf.lib()
    p, n, d, m = 2, 4, 3, 5
    Y = np.ones((p, n, d), np.uint8)
    Z = np.zeros((p, d, m), np.uint8)
    r = np.ones(p, np.float16).view(np.uint16)
    h = ctypes.c_void_p()
    P = lambda arr: arr.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
    E = dbf.DBF_ERR_INVALID_ARG
    assert L.dbf_bqq_pack(n, m, d, p, P(Y), P(Z), P(r), P(r), P(r), 0x3C00, 4, None) == E
    assert L.dbf_bqq_pack(n, m, d, p, None, P(Z), P(r), P(r), P(r), 0x3C00, 4, ctypes.byref(h)) == E
    assert L.dbf_bqq_pack(n, m, d, p, P(Y), P(Z), None, P(r), P(r), 0x3C00, 4, ctypes.byref(h)) == E
    for bad in ((0, m, d, p), (n, 0, d, p), (n, m, 0, p), (n, m, d, 0)):
        assert L.dbf_bqq_pack(*bad, P(Y), P(Z), P(r), P(r), P(r), 0x3C00, 4, ctypes.byref(h)) == E
    assert L.dbf_bqq_pack(n, m, d, p, P(Y), P(Z), P(r), P(r), P(r), 0x3C00, 0, ctypes.byref(h)) == E
    Y2 = Y.copy()
    Y2[1, 2, 0] = 2
    assert L.dbf_bqq_pack(n, m, d, p, P(Y2), P(Z), P(r), P(r), P(r), 0x3C00, 4, ctypes.byref(h)) == E
    Z2 = Z.copy()
    Z2[0, 1, 4] = 255
    assert L.dbf_bqq_pack(n, m, d, p, P(Y), P(Z2), P(r), P(r), P(r), 0x3C00, 4, ctypes.byref(h)) == E
    assert h.value is None
    if not _have_gpu():
        assert L.dbf_bqq_pack(n, m, d, p, P(Y), P(Z), P(r), P(r), P(r), 0x3C00, 4,
                              ctypes.byref(h)) == dbf.DBF_ERR_HIP
        assert h.value is None


def test_bqq_pack_grouped_validates_before_any_device_call():
    """dbf_bqq_pack_grouped reports argument and shape errors (null
    pointers, sizes, entries other than 0/1, d not a multiple of 64 or more
    than 8 terms with several groups) without touching a GPU."""
    L = dbf.lib()
    p, n, d, m, g = 2, 4, 64, 10, 4  # three groups
    ng = 3
    Y = np.ones((p, n, d), np.uint8)
    Z = np.zeros((p, d, m), np.uint8)
    r = np.ones(p * ng, np.float16).view(np.uint16)
    u = np.ones(ng, np.float16).view(np.uint16)
    h = ctypes.c_void_p()
    P = lambda arr: arr.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
    E = dbf.DBF_ERR_INVALID_ARG
    assert L.dbf_bqq_pack_grouped(n, m, d, p, g, P(Y), P(Z), P(r), P(r), P(r), P(u), 4, None) == E
    assert L.dbf_bqq_pack_grouped(n, m, d, p, g, P(Y), P(Z), P(r), P(r), P(r), None, 4, ctypes.byref(h)) == E
    assert L.dbf_bqq_pack_grouped(n, m, d, p, 0, P(Y), P(Z), P(r), P(r), P(r), P(u), 4, ctypes.byref(h)) == E
    for bad in ((0, m, d, p), (n, 0, d, p), (n, m, 0, p), (n, m, d, 0)):
        assert L.dbf_bqq_pack_grouped(*bad, g, P(Y), P(Z), P(r), P(r), P(r), P(u), 4, ctypes.byref(h)) == E
    Y2 = Y.copy()
    Y2[1, 2, 0] = 2
    assert L.dbf_bqq_pack_grouped(n, m, d, p, g, P(Y2), P(Z), P(r), P(r), P(r), P(u), 4, ctypes.byref(h)) == E
    # several groups: the term boundaries must fall on 64-row tiles, at most 8 terms
    Yb = np.ones((p, n, 96), np.uint8)
    Zb = np.zeros((p, 96, m), np.uint8)
    assert L.dbf_bqq_pack_grouped(n, m, 96, p, g, P(Yb), P(Zb), P(r), P(r), P(r), P(u),
                                  4, ctypes.byref(h)) == dbf.DBF_ERR_SHAPE
    Y9 = np.ones((9, n, d), np.uint8)
    Z9 = np.zeros((9, d, m), np.uint8)
    r9 = np.ones(9 * ng, np.float16).view(np.uint16)
    assert L.dbf_bqq_pack_grouped(n, m, d, 9, g, P(Y9), P(Z9), P(r9), P(r9), P(r9), P(u),
                                  4, ctypes.byref(h)) == dbf.DBF_ERR_SHAPE
    assert h.value is None
    if not _have_gpu():
        assert L.dbf_bqq_pack_grouped(n, m, d, p, g, P(Y), P(Z), P(r), P(r), P(r), P(u), 4,
                                      ctypes.byref(h)) == dbf.DBF_ERR_HIP
        assert h.value is None


def test_factorize_validates_before_any_device_call():
    L = dbf.lib()
    E = dbf.DBF_ERR_INVALID_ARG
    f = ctypes.c_float
    p = ctypes.c_void_p(16)  # never dereferenced: every call below fails validation first
    assert L.dbf_factorize(None, 4, 4, 2, p, p, None, None, f(1.0), 1, 1, 1, p, p, p, p, p, None, None) == E
    assert L.dbf_factorize(p, 4, 4, 2, p, p, None, None, f(1.0), 1, 1, 1, None, p, p, p, p, None, None) == E
    for n, m, k in ((0, 4, 2), (4, 0, 2), (4, 4, 0)):
        assert L.dbf_factorize(p, n, m, k, p, p, None, None, f(1.0), 1, 1, 1, p, p, p, p, p, None, None) == E
    for outer, inner, pw in ((0, 1, 1), (1, 0, 1), (1, 1, 0)):
        assert L.dbf_factorize(p, 4, 4, 2, p, p, None, None, f(1.0), outer, inner, pw, p, p, p, p, p, None,
                               None) == E
    assert L.dbf_factorize(p, 4, 4, 2, p, p, None, None, f(0.0), 1, 1, 1, p, p, p, p, p, None, None) == E
    assert L.dbf_factorize(p, 1 << 20, 1 << 20, 2, p, p, None, None, f(1.0), 1, 1, 1, p, p, p, p, p, None,
                           None) == dbf.DBF_ERR_SHAPE
