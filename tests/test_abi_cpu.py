"""The C ABI library loads and exports every entry point declared in
include/spgemm.h; argument checks that return before any device call work on
a machine without a GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "spgemm.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(spgemm_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = _declared()
    for must in ("spgemm_plan", "spgemm_symbolic", "spgemm_numeric", "spgemm_destroy",
                 "spgemm_get_stats", "spgemm_compute_params", "spgemm_status_string",
                 "spgemm_last_error", "spgemm_prune_colnorm_count", "spgemm_prune_colnorm_fill",
                 "spgemm_prune_destroy", "spgemm_mcl_inflate_count", "spgemm_mcl_inflate_fill",
                 "spgemm_transpose", "spgemm_row_estimates"):
        assert must in names


def test_library_exports_every_declared_symbol():
    import spgemm_symbolic_row_amd as sg
    L = sg.lib()
    for name in _declared():
        assert hasattr(L, name), name


def test_argument_validation_without_device():
    import spgemm_symbolic_row_amd as sg
    L = sg.lib()
    h = ctypes.c_void_p()
    dummy = ctypes.c_void_p(16)
    # NULL out-pointer
    assert L.spgemm_plan(None, 1, 1, 1, dummy, dummy, dummy, 1, dummy, dummy, dummy, 1, 1,
                         None, None) == -1
    # negative sizes
    assert L.spgemm_plan(ctypes.byref(h), -1, 1, 1, dummy, dummy, dummy, 1, dummy, dummy, dummy,
                         1, 1, None, None) == -1
    # bad dtype
    assert L.spgemm_plan(ctypes.byref(h), 1, 1, 1, dummy, dummy, dummy, 1, dummy, dummy, dummy,
                         1, 7, None, None) == -1
    # NULL device arrays with nnz > 0
    assert L.spgemm_plan(ctypes.byref(h), 1, 1, 1, dummy, None, dummy, 1, dummy, dummy, dummy,
                         1, 1, None, None) == -1
    # sizes beyond the int32 index range
    assert L.spgemm_plan(ctypes.byref(h), 1 << 31, 1, 1, dummy, dummy, dummy, 1, dummy, dummy,
                         dummy, 1, 1, None, None) == -3
    assert h.value is None
    assert b"int32" in L.spgemm_last_error(None)
    # calls on a NULL plan
    assert L.spgemm_symbolic(None, dummy, ctypes.byref(ctypes.c_int64())) == -1
    assert L.spgemm_numeric(None, dummy, dummy) == -1
    L.spgemm_destroy(None)
    # transpose: negative sizes, bad dtype, NULL outputs, int32 range
    t = L.spgemm_transpose
    assert t(-1, 1, 1, dummy, 0, dummy, dummy, 1, dummy, 0, dummy, dummy, None) == -1
    assert t(1, 1, 1, dummy, 0, dummy, dummy, 7, dummy, 0, dummy, dummy, None) == -1
    assert t(1, 1, 1, dummy, 0, dummy, dummy, 1, None, 0, dummy, dummy, None) == -1
    assert t(1, 1, 1, dummy, 0, dummy, dummy, 1, dummy, 0, None, dummy, None) == -1
    assert t(1, 1, 1, dummy, 0, dummy, dummy, 1, dummy, 0, dummy, None, None) == -1
    assert t(1 << 31, 1, 1, dummy, 0, dummy, dummy, 1, dummy, 0, dummy, dummy, None) == -3
    assert t(1, 1, 1 << 31, dummy, 0, dummy, dummy, 1, dummy, 0, dummy, dummy, None) == -3
    assert L.spgemm_row_estimates(None, None, None) == -1
    for s, word in ((0, b"ok"), (-2, b"canonical"), (-3, b"overflow"), (-6, b"order")):
        assert word in L.spgemm_status_string(s)


def test_binding_refuses_missing_library(tmp_path, monkeypatch):
    import spgemm_symbolic_row_amd as sg
    monkeypatch.setattr(sg, "_lib", None)
    monkeypatch.setattr(sg, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(RuntimeError, match="not built"):
        sg.lib()
