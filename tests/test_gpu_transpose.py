"""GPU parity for the CSR transpose (spgemm_transpose) and the rectangular
products built on it: A*A^T and A*R with an aggregation operator R.

The transpose moves indices and copies values, so it must match the oracle's
transpose bit for bit: row pointers, columns and values.  Products are
checked as in test_gpu_parity: exact structure, values within
rtol * sum |terms| (exact for integer-valued inputs).
"""
import numpy as np
import pytest

import oracle
import synth
from conftest import assert_csr_equal_structure, assert_values_close

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
sg = pytest.importorskip("spgemm_symbolic_row_amd")


def _np(t, dtype=None):
    a = t.detach().cpu().numpy()
    return a.astype(dtype) if dtype is not None else a


def _gpu_transpose(A, rowptr64_in=False, rowptr64_out=False, pattern_only=False):
    dA = sg.to_device(A)
    if rowptr64_in:
        dA = sg.CsrDevice(dA.row_ptr.to(torch.int64), dA.col, dA.val, A.m, A.n)
    dT = sg.transpose(dA, out_rowptr64=rowptr64_out, pattern_only=pattern_only)
    torch.cuda.synchronize()
    assert dT.row_ptr.dtype == (torch.int64 if rowptr64_out else torch.int32)
    assert (dT.m, dT.n) == (A.n, A.m)
    return dT


def _check_transpose(A, **kw):
    print(f"transpose m={A.m} n={A.n} nnz={A.col.shape[0]} {A.val.dtype} {kw}", flush=True)
    dT = _gpu_transpose(A, **kw)
    ref = oracle.transpose(A)
    np.testing.assert_array_equal(_np(dT.row_ptr, np.int64), ref.row_ptr)
    np.testing.assert_array_equal(_np(dT.col), ref.col)
    if kw.get("pattern_only"):
        assert dT.val is None
    else:
        v = _np(dT.val)
        assert v.dtype == A.val.dtype
        np.testing.assert_array_equal(v.view(np.uint8), ref.val.view(np.uint8))
    return dT


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
@pytest.mark.parametrize("m,n,per_row,seed", [
    (1, 1, 1.0, 0),            # a single entry
    (300, 500, 6.0, 1),        # one digit pass, one ragged tile
    (20000, 1024, 10.0, 2),    # 10-bit columns: still one pass, 25 tiles + tail
    (20000, 1025, 10.0, 3),    # 11 bits: two passes
    (5000, 70000, 30.0, 4),    # two passes of 9 bits, many tiles
])
def test_transpose_matches_oracle(m, n, per_row, seed, dtype):
    A = synth.sparse_uniform(m, n, per_row, seed, dtype=dtype)
    _check_transpose(A)


def test_transpose_three_passes_and_index_widths():
    # 2^21 columns: 21 bits in three passes of 7; int64 row pointers in and out.
    A = synth.sparse_uniform(3000, 1 << 21, 40.0, 5)
    _check_transpose(A)
    _check_transpose(A, rowptr64_in=True, rowptr64_out=True)
    _check_transpose(A, pattern_only=True)


def test_transpose_rmat_hot_columns():
    # power-law columns: some rows of A^T hold thousands of entries
    A = synth.rmat(15, 16, seed=4)
    T = _check_transpose(A)
    assert int(np.diff(_np(T.row_ptr, np.int64)).max()) > 1000


@pytest.mark.parametrize("case", ["no_entries", "no_rows", "no_cols", "empty_rows_and_cols"])
def test_transpose_degenerate(case):
    if case == "no_entries":
        A = synth.CSR(np.zeros(6, np.int32), np.zeros(0, np.int32), np.zeros(0), 5, 7)
    elif case == "no_rows":
        A = synth.CSR(np.zeros(1, np.int32), np.zeros(0, np.int32), np.zeros(0), 0, 7)
    elif case == "no_cols":
        A = synth.CSR(np.zeros(6, np.int32), np.zeros(0, np.int32), np.zeros(0), 5, 0)
    else:
        A = synth.random_csr(400, 900, 2.0, 6, values="uniform", empty_row_frac=0.5)
    _check_transpose(A)


def test_transpose_rejects_column_out_of_range():
    # The column check runs on the device over every entry; positions are
    # computed from the same digit counts, so the sort stays in bounds.
    A = synth.random_csr(50, 40, 3.0, 7, values="uniform")
    dA = sg.to_device(A)
    bad = dA.col.clone()
    bad[bad.numel() // 2] = 40
    with pytest.raises(sg.SpgemmError) as e:
        sg.transpose(sg.CsrDevice(dA.row_ptr, bad, dA.val, A.m, A.n))
    assert e.value.status == -2
    bad[bad.numel() // 2] = -1
    with pytest.raises(sg.SpgemmError):
        sg.transpose(sg.CsrDevice(dA.row_ptr, bad, dA.val, A.m, A.n))
    torch.cuda.synchronize()


def _check_product(dA, dB, A, B, exact=False, **opts):
    with sg.Plan(dA, dB, **opts) as p:
        rp, _ = p.symbolic()
        col, val = p.numeric()
        st = p.stats()
    torch.cuda.synchronize()
    ref = oracle.spgemm(A, B)
    assert_csr_equal_structure(_np(rp, np.int64), _np(col), ref.row_ptr, ref.col, "C")
    v = _np(val)
    if exact:
        np.testing.assert_array_equal(v, ref.val)
    else:
        rtol = 1e-12 if A.val.dtype == np.float64 else 1e-5
        assert_values_close(v, ref.val, ref.mag, rtol, "C")
    assert st["lds_hash_products"] + st["lds_dense_products"] == st["products"]
    return st, ref


def _oracle_t(A):
    T = oracle.transpose(A)
    return synth.CSR(T.row_ptr.astype(np.int32), T.col, T.val, T.m, T.n)


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
@pytest.mark.parametrize("rs,cs,per_row,seed", [(8, 11, 8, 1), (10, 13, 16, 2)])
def test_aat_rectangular_rmat(rs, cs, per_row, seed, dtype):
    A = synth.rmat_rect(rs, cs, per_row, seed=seed, dtype=dtype)
    print(f"A*A^T rmat_rect {rs} {cs} {per_row} {dtype}", flush=True)
    dA = sg.to_device(A)
    dT = sg.transpose(dA)
    _check_product(dA, dT, A, _oracle_t(A))


def test_aat_integer_exact_heavy_rows():
    # integer values: any summation order is exact; the heavy path is forced
    A = synth.random_csr(400, 3000, 60.0, 8, values="int")
    dA = sg.to_device(A)
    dT = sg.transpose(dA)
    st, ref = _check_product(dA, dT, A, _oracle_t(A), exact=True, heavy_threshold=256, dense_width=512,
                             max_chunks_per_level=4)
    assert st["heavy_rows"] > 0
    # A*A^T is symmetric, structure and values alike
    m = A.m
    rows = np.repeat(np.arange(m), np.diff(ref.row_ptr))
    D = np.full((m, m), np.nan)
    D[rows, ref.col] = ref.val
    np.testing.assert_array_equal(np.isnan(D), np.isnan(D.T))
    np.testing.assert_array_equal(np.nan_to_num(D), np.nan_to_num(D.T))


def test_restriction_product_laplacian():
    # C = A*R on the 27-point Laplacian with 2x2x2 aggregates (16^3 grid)
    A = synth.laplacian27(16)
    R = synth.grid_aggregation(16, 2)
    _check_product(sg.to_device(A), sg.to_device(R), A, R, exact=True)


def test_restriction_product_rmat_random_aggregates():
    A = synth.rmat(13, 16, seed=9)
    R = synth.aggregation(A.n, 8, seed=10)
    _check_product(sg.to_device(A), sg.to_device(R), A, R)
    # R^T A R, the coarse operator: transpose and both products on the GPU,
    # the same chain in the oracle alone
    dR = sg.to_device(R)
    rp, col, val = sg.matmul(sg.to_device(A), dR)
    dAR = sg.CsrDevice(rp, col, val, A.m, R.n)
    o = oracle.spgemm(A, R)
    ARo = synth.CSR(o.row_ptr.astype(np.int32), o.col, o.val, A.m, R.n)
    _check_product(sg.transpose(dR), dAR, _oracle_t(R), ARo)
