import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: takes more than a few seconds")


def assert_csr_equal_structure(rp, col, ref_rp, ref_col, what=""):
    rp = np.asarray(rp, dtype=np.int64)
    ref_rp = np.asarray(ref_rp, dtype=np.int64)
    assert rp.shape == ref_rp.shape, f"{what}: row_ptr length {rp.shape} vs {ref_rp.shape}"
    bad = np.nonzero(rp != ref_rp)[0]
    assert bad.size == 0, f"{what}: row_ptr differs first at {bad[0]}: {rp[bad[0]]} vs {ref_rp[bad[0]]}"
    col = np.asarray(col)
    ref_col = np.asarray(ref_col)
    assert col.shape == ref_col.shape
    badc = np.nonzero(col != ref_col)[0]
    assert badc.size == 0, f"{what}: col differs first at {badc[0]}: {col[badc[0]]} vs {ref_col[badc[0]]}"


def assert_values_close(val, ref_val, ref_mag, rtol, what=""):
    """|c - c_ref| <= rtol * sum_k |a_ik b_kj| per entry (equals rtol*|c_ref|
    when all terms share a sign)."""
    val = np.asarray(val, dtype=np.float64)
    err = np.abs(val - ref_val)
    lim = rtol * ref_mag
    bad = np.nonzero(~(err <= lim))[0]
    assert bad.size == 0, (f"{what}: {bad.size} values outside tolerance; first at {bad[0]}: "
                           f"{val[bad[0]]!r} vs {ref_val[bad[0]]!r} (mag {ref_mag[bad[0]]!r})")
    if val.size:
        with np.errstate(divide="ignore", invalid="ignore"):
            r = np.where(lim > 0, err / lim, 0.0)
        print(f"{what}: {val.size} values, largest error {float(r.max()):.3g} of the bound",
              flush=True)
