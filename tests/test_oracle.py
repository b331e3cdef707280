"""Pins for the CPU oracle, independent of the oracle's own code.

Each check compares the oracle against something fixed by the mathematics:
brute-force dense products on tiny integer inputs (exact), the closed form of
the squared 27-point Laplacian, identities, transposition, a sort-based set
union for the structure, row/column sums of stochastic matrices, and scipy as
a third implementation.  test_mutants_fail compiles deliberately broken
copies of the oracle and checks that these pins catch them.
"""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest
import scipy.sparse as sp

import oracle
import synth
from conftest import assert_csr_equal_structure, assert_values_close

from synth import CSR


def _dense_reference(A: CSR, B: CSR):
    """Brute force: structure from the 0/1 pattern product, values from the
    dense product.  With small-integer values both are exact in fp64."""
    Ad, Bd = A.to_dense(), B.to_dense()
    Ap = np.zeros_like(Ad)
    Bp = np.zeros_like(Bd)
    rowsA = np.repeat(np.arange(A.m), np.diff(A.row_ptr.astype(np.int64)))
    rowsB = np.repeat(np.arange(B.m), np.diff(B.row_ptr.astype(np.int64)))
    Ap[rowsA, A.col] = 1.0
    Bp[rowsB, B.col] = 1.0
    pattern = (Ap @ Bp) > 0
    vals = Ad @ Bd
    return pattern, vals


def _check_vs_bruteforce(A, B):
    r = oracle.spgemm(A, B)
    pattern, vals = _dense_reference(A, B)
    m = A.m
    exp_rp = np.zeros(m + 1, dtype=np.int64)
    np.cumsum(pattern.sum(axis=1), out=exp_rp[1:])
    exp_col = np.nonzero(pattern)[1].astype(np.int32)   # row-major, sorted columns
    assert_csr_equal_structure(r.row_ptr, r.col, exp_rp, exp_col, "bruteforce")
    rows = np.repeat(np.arange(m), np.diff(exp_rp))
    np.testing.assert_array_equal(r.val, vals[rows, exp_col])
    return r


@pytest.mark.parametrize("m,k,n,per_row,seed", [
    (1, 1, 1, 1.0, 0), (7, 5, 3, 2.0, 1), (40, 30, 50, 3.0, 2), (64, 64, 64, 4.0, 3),
    (128, 96, 80, 6.0, 4), (100, 1, 100, 0.5, 5), (50, 120, 7, 10.0, 6),
])
def test_bruteforce_integer_exact(m, k, n, per_row, seed):
    A = synth.random_csr(m, k, per_row, seed, values="int", empty_row_frac=0.2)
    B = synth.random_csr(k, n, per_row, seed + 100, values="int", empty_row_frac=0.2)
    _check_vs_bruteforce(A, B)


def test_bruteforce_keeps_exact_cancellation():
    # Row 0 of A = [1, 1], B rows [1] and [-1] on column 0: C[0,0] = 0 exactly,
    # and the entry stays (structural definition).
    A = CSR(np.array([0, 2], np.int32), np.array([0, 1], np.int32), np.array([1.0, 1.0]), 1, 2)
    B = CSR(np.array([0, 1, 2], np.int32), np.array([0, 0], np.int32), np.array([1.0, -1.0]), 2, 1)
    r = _check_vs_bruteforce(A, B)
    assert r.row_ptr.tolist() == [0, 1] and r.col.tolist() == [0] and r.val.tolist() == [0.0]


def test_compensated_sum_exact():
    """Terms whose exact sum is representable but lost by plain fp64
    summation: 1e16 + 1 - 1e16 + 0.5 + 1e-3 = 1.501 (nearest double).  The oracle
    must return the correctly rounded exact sum, which pins the compensation."""
    terms = np.array([1e16, 1.0, -1e16, 0.5, 1e-3])
    A = CSR(np.array([0, 5], np.int32), np.arange(5, dtype=np.int32), terms, 1, 5)
    B = CSR(np.arange(6, dtype=np.int32), np.zeros(5, np.int32), np.ones(5), 5, 1)
    r = oracle.spgemm(A, B)
    assert r.col.tolist() == [0]
    assert r.val[0] == 1.501
    assert r.terms[0] == 5


def test_empty_and_degenerate():
    # nnz(A) = 0
    A = CSR(np.zeros(6, np.int32), np.zeros(0, np.int32), np.zeros(0), 5, 4)
    B = synth.random_csr(4, 9, 2.0, 0)
    r = oracle.spgemm(A, B)
    assert r.row_ptr.tolist() == [0] * 6 and r.col.size == 0
    # B all empty rows
    A = synth.random_csr(5, 4, 2.0, 1)
    B = CSR(np.zeros(5, np.int32), np.zeros(0, np.int32), np.zeros(0), 4, 9)
    r = oracle.spgemm(A, B)
    assert r.col.size == 0
    # single dense row times dense matrix
    A = synth.random_csr(1, 30, 100.0, 2, values="int")
    B = synth.random_csr(30, 30, 100.0, 3, values="int")
    _check_vs_bruteforce(A, B)


def _laplacian_closed_form_check(nx):
    """A = 27 I - S with S = T (x) T (x) T, T the nx x nx tridiagonal of ones,
    so A^2 = 729 I - 54 S + T^2 (x) T^2 (x) T^2.  (T^2)_xx is 3 inside and 2
    at the ends, (T^2)_{x,x+-1} = 2, (T^2)_{x,x+-2} = 1."""
    A = synth.laplacian27(nx)
    r = oracle.spgemm(A, A)
    N = nx ** 3
    # nnz(C) = (5 nx - 6)^3: each 1D factor T^2 is pentadiagonal.
    assert int(r.row_ptr[-1]) == (5 * nx - 6) ** 3
    # products: sum_i P_i = (sum over 1D of deg^2)^3 = (2*2^2 + (nx-2)*3^2)^3
    P = oracle.row_products(A, A)
    assert int(P.sum()) == (2 * 4 + (nx - 2) * 9) ** 3
    rows = np.repeat(np.arange(N, dtype=np.int64), np.diff(r.row_ptr))
    cols = r.col.astype(np.int64)

    def coords(i):
        return i % nx, (i // nx) % nx, i // (nx * nx)

    xi, yi, zi = coords(rows)
    xj, yj, zj = coords(cols)

    def t2(a, b):
        d = np.abs(a - b)
        out = np.where(d == 2, 1, np.where(d == 1, 2, 0))
        diag = np.where((a == 0) | (a == nx - 1), 2, 3)
        return np.where(d == 0, diag, out)

    s = ((np.abs(xi - xj) <= 1) & (np.abs(yi - yj) <= 1) & (np.abs(zi - zj) <= 1)).astype(np.int64)
    expect = 729 * (rows == cols) - 54 * s + t2(xi, xj) * t2(yi, yj) * t2(zi, zj)
    # every entry of C is within the 5x5x5 box and is a nonzero integer
    assert np.all(np.abs(xi - xj) <= 2) and np.all(np.abs(yi - yj) <= 2) and np.all(np.abs(zi - zj) <= 2)
    np.testing.assert_array_equal(r.val, expect.astype(np.float64))
    assert np.all(expect != 0)


@pytest.mark.parametrize("nx", [3, 4, 8, 13])
def test_laplacian_closed_form_small(nx):
    _laplacian_closed_form_check(nx)


@pytest.mark.slow
def test_laplacian_closed_form_64():
    _laplacian_closed_form_check(64)


def test_identity():
    A = synth.rmat(10, 16, seed=3)
    I = synth.identity(A.m)
    for X, Y in ((A, I), (I, A)):
        r = oracle.spgemm(X, Y)
        assert_csr_equal_structure(r.row_ptr, r.col, A.row_ptr, A.col, "identity")
        np.testing.assert_array_equal(r.val, A.val)


def _transpose(M: CSR) -> CSR:
    rows = np.repeat(np.arange(M.m, dtype=np.int64), np.diff(M.row_ptr.astype(np.int64)))
    key = M.col.astype(np.int64) * M.m + rows
    o = np.argsort(key, kind="stable")
    cnt = np.bincount(M.col, minlength=M.n)
    rp = np.zeros(M.n + 1, dtype=np.int64)
    np.cumsum(cnt, out=rp[1:])
    return CSR(rp.astype(np.int32), rows[o].astype(np.int32), M.val[o], M.n, M.m)


@pytest.mark.parametrize("case", ["rmat", "rect"])
def test_transpose_identity(case):
    if case == "rmat":
        A = synth.rmat(11, 16, seed=1)
        B = synth.rmat(11, 8, seed=2)
    else:
        A = synth.random_csr(300, 200, 6.0, 7, values="uniform", empty_row_frac=0.1)
        B = synth.random_csr(200, 500, 5.0, 8, values="uniform", empty_row_frac=0.1)
    C = oracle.spgemm(A, B)
    Ct = oracle.spgemm(_transpose(B), _transpose(A))
    Cc = CSR(C.row_ptr, C.col, C.val, A.m, B.n)
    T = _transpose(Cc)
    assert_csr_equal_structure(Ct.row_ptr, Ct.col, T.row_ptr, T.col, "transpose")
    # compare values with the mag of the transposed product (same multiset of terms)
    assert_values_close(Ct.val, T.val, Ct.mag, 1e-14, "transpose")


def test_row_products_and_bound():
    A = synth.rmat(12, 16, seed=4)
    P = oracle.row_products(A, A)
    nb = np.diff(A.row_ptr.astype(np.int64))
    rows = np.repeat(np.arange(A.m), nb)
    expect = np.bincount(rows, weights=nb[A.col], minlength=A.m).astype(np.int64)
    np.testing.assert_array_equal(P, expect)
    r = oracle.spgemm(A, A)
    cnt = np.diff(r.row_ptr)
    assert np.all(cnt <= P)
    # terms per entry sum to the products of the row
    row_of = np.repeat(np.arange(A.m), cnt)
    np.testing.assert_array_equal(np.bincount(row_of, weights=r.terms, minlength=A.m), P)


def test_symbolic_matches_sort_union():
    A = synth.rmat(11, 16, seed=5)
    B = synth.rmat(11, 4, seed=6)
    cnt = oracle.symbolic(A, B)
    brp = B.row_ptr.astype(np.int64)
    for i in range(0, A.m, 7):
        ks = A.col[A.row_ptr[i]:A.row_ptr[i + 1]]
        cols = [B.col[brp[k]:brp[k + 1]] for k in ks]
        u = np.unique(np.concatenate(cols)) if cols else np.zeros(0)
        assert cnt[i] == u.size


def test_row_range_and_row_list_agree():
    A = synth.rmat(10, 16, seed=9)
    full = oracle.spgemm(A, A)
    part = oracle.spgemm(A, A, r0=100, r1=400)
    off = full.row_ptr[100]
    np.testing.assert_array_equal(part.row_ptr + off, full.row_ptr[100:401])
    sl = slice(int(full.row_ptr[100]), int(full.row_ptr[400]))
    np.testing.assert_array_equal(part.col, full.col[sl])
    np.testing.assert_array_equal(part.val, full.val[sl])
    rows = np.array([5, 900, 3, 3, 1023])
    lst = oracle.spgemm(A, A, rows=rows)
    for q, i in enumerate(rows):
        a, b = full.row_ptr[i], full.row_ptr[i + 1]
        c, d = lst.row_ptr[q], lst.row_ptr[q + 1]
        np.testing.assert_array_equal(lst.col[c:d], full.col[a:b])
        np.testing.assert_array_equal(lst.val[c:d], full.val[a:b])


def test_row_stochastic_row_sums():
    def stochastic(m, n, per_row, seed):
        M = synth.random_csr(m, n, per_row, seed, values="pos")
        rs = np.add.reduceat(M.val, M.row_ptr[:-1].astype(np.int64)) if M.nnz else np.zeros(m)
        nonempty = np.diff(M.row_ptr) > 0
        rows = np.repeat(np.arange(m), np.diff(M.row_ptr.astype(np.int64)))
        M.val = M.val / np.where(nonempty, rs, 1.0)[rows]
        return M, nonempty
    A, ne_a = stochastic(400, 300, 8.0, 10)
    B, ne_b = stochastic(300, 500, 8.0, 11)
    assert ne_b.all()
    r = oracle.spgemm(A, B)
    sums = np.zeros(A.m)
    rows = np.repeat(np.arange(A.m), np.diff(r.row_ptr))
    np.add.at(sums, rows, r.val)
    np.testing.assert_allclose(sums[ne_a], 1.0, rtol=0, atol=500 * np.finfo(float).eps)


def test_planted_partition_column_sums():
    A = synth.planted_partition(30, 100, 28, 4, seed=1)
    # A is column-stochastic (in fp32), so A^2 is column-stochastic.
    colsum_a = np.bincount(A.col, weights=A.val.astype(np.float64), minlength=A.n)
    np.testing.assert_allclose(colsum_a, 1.0, atol=1e-6)
    r = oracle.spgemm(A, A)
    colsum = np.bincount(r.col, weights=r.val, minlength=A.n)
    np.testing.assert_allclose(colsum, 1.0, atol=1e-5)
    assert np.all(np.bincount(A.col, minlength=A.n) == 33)


def test_scipy_cross_check():
    # positive values, so scipy's dropping of numerical zeros never triggers
    A = synth.rmat(11, 16, seed=12)
    B = synth.random_csr(A.n, 700, 9.0, 13, values="pos")
    r = oracle.spgemm(A, B)
    S = (sp.csr_matrix((A.val, A.col, A.row_ptr), shape=(A.m, A.n))
         @ sp.csr_matrix((B.val, B.col, B.row_ptr), shape=(B.m, B.n))).tocsr()
    S.sort_indices()
    assert_csr_equal_structure(r.row_ptr, r.col, S.indptr, S.indices, "scipy")
    np.testing.assert_allclose(r.val, S.data, rtol=1e-13, atol=0)


def test_fp32_inputs_accumulate_in_fp64():
    A = synth.random_csr(200, 200, 10.0, 14, values="uniform", dtype=np.float32)
    r = oracle.spgemm(A, A)
    Ad = A.to_dense()          # float64 copy of the fp32 values
    pattern, vals = _dense_reference(A, A)
    rows = np.repeat(np.arange(A.m), np.diff(r.row_ptr))
    # fp32*fp32 products are exact in fp64; only the sums round
    assert_values_close(r.val, vals[rows, r.col], r.mag, 1e-15, "fp32 inputs")
    assert Ad.dtype == np.float64


def _read_golden(name):
    out = {}
    for line in open(os.path.join(os.path.dirname(__file__), "golden", name)):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        k, *v = line.split()
        out[k] = np.array([float(x) for x in v])
    return out


def test_mcl_inflate_hand_example():
    # tests/golden/mcl_inflate_hand.txt: worked by hand from the step the
    # Trident page describes (normalise columns, prune, square).
    g = _read_golden("mcl_inflate_hand.txt")
    rp, col, val = g["row_ptr"].astype(np.int64), g["col"].astype(np.int32), g["val"]
    for single in (True, False):
        for thr, key in ((0.3, "t0.3"), (0.0, "t0")):
            orp, oc, ov = oracle.mcl_inflate(3, 3, rp, col, val, thr, single=single)
            np.testing.assert_array_equal(orp, g[key + "_row_ptr"].astype(np.int64))
            np.testing.assert_array_equal(oc, g[key + "_col"].astype(np.int32))
            np.testing.assert_array_equal(ov, g[key + "_val"])


def test_mcl_inflate_fixpoints():
    # The identity is a fixed point of the whole iteration (I*I = I, columns
    # already sum to 1, 1 >= any threshold below 1, 1^2 = 1).
    I = synth.identity(7, np.float32)
    C = oracle.spgemm(I, I)
    orp, oc, ov = oracle.mcl_inflate(7, 7, C.row_ptr, C.col, C.val, 0.5)
    np.testing.assert_array_equal(orp, I.row_ptr.astype(np.int64))
    np.testing.assert_array_equal(oc, I.col)
    np.testing.assert_array_equal(ov, np.ones(7))
    # The uniform 4x4 matrix J/4: (J/4)^2 = J/4, normalised 1/4 everywhere,
    # squared 1/16; pruned away entirely above 1/4.
    n = 4
    J = synth.CSR(np.arange(0, n * n + 1, n, dtype=np.int32),
                  np.tile(np.arange(n, dtype=np.int32), n), np.full(n * n, 0.25, np.float32), n, n)
    C = oracle.spgemm(J, J)
    np.testing.assert_array_equal(C.val, np.full(n * n, 0.25))
    orp, oc, ov = oracle.mcl_inflate(n, n, C.row_ptr, C.col, C.val, 0.25)
    np.testing.assert_array_equal(ov, np.full(n * n, 0.0625))
    orp, oc, ov = oracle.mcl_inflate(n, n, C.row_ptr, C.col, C.val, 0.26)
    assert orp[-1] == 0


def test_mcl_iterations_separate_clusters():
    # Markov clustering of two 30-node cliques joined by one edge: after a
    # few iterations no mass flows between the cliques, and every column
    # keeps at least one entry inside its own clique.
    n, h = 60, 30
    dense = np.zeros((n, n))
    dense[:h, :h] = 1.0
    dense[h:, h:] = 1.0
    dense[h - 1, h] = dense[h, h - 1] = 1.0
    dense /= dense.sum(axis=0, keepdims=True)
    X = sp.csr_matrix(dense.astype(np.float32))
    A = synth.CSR(X.indptr.astype(np.int32), X.indices.astype(np.int32), X.data, n, n)
    for _ in range(6):
        C = oracle.spgemm(A, A)
        rp, col, val = oracle.mcl_inflate(n, n, C.row_ptr, C.col, C.val, 0.002)
        A = synth.CSR(rp.astype(np.int32), col, val.astype(np.float32), n, n)
    rows = np.repeat(np.arange(n), np.diff(A.row_ptr))
    assert np.all((rows < h) == (A.col < h))
    assert set(A.col.tolist()) == set(range(n))


def test_prune_colnorm_small():
    # C (3x3) with entries straddling the threshold 1e-4
    rp = np.array([0, 2, 4, 5], np.int64)
    col = np.array([0, 2, 0, 1, 2], np.int32)
    val = np.array([0.5, 5e-5, 1e-4, 0.25, 0.75])
    orp, oc, ov = oracle.prune_colnorm(3, 3, rp, col, val, 1e-4)
    # 5e-5 dropped; 1e-4 (exactly the fp32 threshold after rounding) kept
    assert orp.tolist() == [0, 1, 3, 4]
    assert oc.tolist() == [0, 0, 1, 2]
    np.testing.assert_allclose(ov, [0.5 / (0.5 + 1e-4), 1e-4 / (0.5 + 1e-4), 1.0, 1.0], rtol=1e-15)
    # keep override drops an entry that passes and keeps one that does not
    keep = np.array([-1, 1, 0, -1, -1], np.int8)
    orp, oc, ov = oracle.prune_colnorm(3, 3, rp, col, val, 1e-4, keep=keep)
    assert orp.tolist() == [0, 2, 3, 4] and oc.tolist() == [0, 2, 1, 2]
    np.testing.assert_allclose(ov, [1.0, 5e-5 / (5e-5 + 0.75), 1.0, 0.75 / (5e-5 + 0.75)], rtol=1e-15)


def _golden_csr(g, p, m, n, dtype=np.float64):
    return CSR(g[p + "_row_ptr"].astype(np.int32), g[p + "_col"].astype(np.int32),
               g[p + "_val"].astype(dtype), m, n)


def test_transpose_hand_example():
    # tests/golden/transpose_hand.txt: transpose and A*A^T worked by hand.
    g = _read_golden("transpose_hand.txt")
    for dt in (np.float64, np.float32):
        A = _golden_csr(g, "a", 3, 4, dt)
        T = oracle.transpose(A)
        assert (T.m, T.n) == (4, 3) and T.val.dtype == dt
        np.testing.assert_array_equal(T.row_ptr, g["t_row_ptr"].astype(np.int64))
        np.testing.assert_array_equal(T.col, g["t_col"].astype(np.int32))
        np.testing.assert_array_equal(T.val, g["t_val"].astype(dt))
        C = oracle.spgemm(A, T)
        np.testing.assert_array_equal(C.row_ptr, g["aat_row_ptr"].astype(np.int64))
        np.testing.assert_array_equal(C.col, g["aat_col"].astype(np.int32))
        np.testing.assert_array_equal(C.val, g["aat_val"])
    P = oracle.transpose(CSR(A.row_ptr, A.col, None, 3, 4))
    assert P.val is None and P.col.tolist() == g["t_col"].astype(int).tolist()


@pytest.mark.parametrize("m,n,per_row,seed", [
    (0, 5, 1.0, 0), (5, 0, 0.0, 0), (1, 1, 1.0, 1), (40, 7, 3.0, 2), (7, 300, 20.0, 3),
    (500, 800, 6.0, 4), (300, 2000, 1.5, 5)])
def test_transpose_against_scipy_and_sort(m, n, per_row, seed):
    # Two independent transposes: scipy's, and a stable sort of the entries
    # by (column, row) in the test itself.
    for values in ("uniform", "int"):
        A = synth.random_csr(m, n, per_row, seed, values=values, empty_row_frac=0.2)
        for dt in (np.float64, np.float32):
            A = CSR(A.row_ptr, A.col, A.val.astype(dt), m, n)
            T = oracle.transpose(A)
            S = sp.csr_matrix((A.val, A.col, A.row_ptr), shape=(m, n)).T.tocsr()
            S.sort_indices()
            np.testing.assert_array_equal(T.row_ptr, S.indptr.astype(np.int64))
            np.testing.assert_array_equal(T.col, S.indices.astype(np.int32))
            np.testing.assert_array_equal(T.val, S.data)
            R = _transpose(A)
            np.testing.assert_array_equal(T.col, R.col)
            np.testing.assert_array_equal(T.val, R.val)
            # involution: (A^T)^T == A, bit for bit
            TT = oracle.transpose(T)
            np.testing.assert_array_equal(TT.row_ptr, A.row_ptr.astype(np.int64))
            np.testing.assert_array_equal(TT.col, A.col)
            np.testing.assert_array_equal(TT.val, A.val)


def test_transpose_rejects_bad_column():
    A = CSR(np.array([0, 2], np.int32), np.array([0, 3], np.int32), np.ones(2), 1, 3)
    with pytest.raises(ValueError):
        oracle.transpose(A)


@pytest.mark.parametrize("m,k,per_row,seed", [(30, 50, 3.0, 11), (64, 200, 8.0, 12),
                                              (100, 20, 2.0, 13)])
def test_aat_bruteforce(m, k, per_row, seed):
    # A*A^T from the oracle's transpose and product against dense brute force;
    # the result is symmetric, structure and values alike.
    A = synth.random_csr(m, k, per_row, seed, values="int", empty_row_frac=0.2)
    T = oracle.transpose(A)
    Tc = CSR(T.row_ptr.astype(np.int32), T.col, T.val, T.m, T.n)
    r = _check_vs_bruteforce(A, Tc)
    D = np.zeros((m, m))
    rows = np.repeat(np.arange(m), np.diff(r.row_ptr))
    D[rows, r.col] = r.val + 0.5   # stored zeros stay visible
    np.testing.assert_array_equal(D, D.T)


def _rows_of_sizes(sizes, n, seed):
    """B whose row r holds sizes[r] distinct uniform columns of [0, n)."""
    rng = np.random.default_rng(seed)
    cols = [np.sort(rng.choice(n, size=k, replace=False)) for k in sizes]
    rp = np.zeros(len(sizes) + 1, np.int64)
    np.cumsum(sizes, out=rp[1:])
    col = np.concatenate(cols).astype(np.int32) if len(cols) else np.zeros(0, np.int32)
    return CSR(rp.astype(np.int32), col, np.ones(col.shape[0]), len(sizes), n)


@pytest.mark.parametrize("M", [32, 64])
def test_hll_accuracy(M):
    # Ocean §3: relative error about 1.04 / sqrt(M).  With A = I the estimate
    # of row i is that of B's row i, whose exact distinct count is its length.
    rng = np.random.default_rng(M)
    large = rng.integers(300, 5000, size=1500)
    small = rng.integers(1, M // 2, size=1500)
    for sizes, kind in ((large, "large"), (small, "small")):
        B = _rows_of_sizes(sizes, 1 << 20, 3)
        I = synth.identity(B.m)
        r = oracle.hll_estimate(I, B, M) / sizes
        sd = 1.04 / np.sqrt(M)
        if kind == "large":
            assert abs(r.mean() - 1.0) < 0.03, r.mean()
            assert 0.7 * sd < r.std() < 1.3 * sd, (r.std(), sd)
        else:   # linear counting: small bias (about n / 2M), small spread
            assert abs(r.mean() - 1.0) < 0.05, r.mean()
            assert r.std() < 0.7 * sd, r.std()


def test_hll_special_cases():
    # empty row -> 0; one column -> M ln(M / (M - 1)); duplicates do not count;
    # the merged sketch of A's row equals the sketch of its products' columns.
    B = CSR(np.array([0, 0, 1, 4], np.int32), np.array([7, 7, 7, 7], np.int32)[:4],
            np.ones(4), 3, 10)
    B = CSR(np.array([0, 0, 1, 2], np.int32), np.array([7, 7], np.int32), np.ones(2), 3, 10)
    A = CSR(np.array([0, 1, 2, 4], np.int32), np.array([0, 1, 1, 2], np.int32), np.ones(4), 3, 3)
    for M in (32, 64):
        e = oracle.hll_estimate(A, B, M)
        assert e[0] == 0.0
        assert e[1] == M * np.log(M / (M - 1))
        assert e[2] == e[1]
    with pytest.raises(ValueError):
        oracle.hll_estimate(A, B, 16)


@pytest.mark.parametrize("M", [32, 64])
def test_hll_merge_equals_direct(M):
    A = synth.rmat(11, 8, seed=5)
    S = oracle.hll_sketch(A, M)
    est, regs = oracle.hll_estimate(A, A, M, with_regs=True)
    rp = A.row_ptr.astype(np.int64)
    for i in range(A.m):
        ks = A.col[rp[i]:rp[i + 1]]
        want = S[ks].max(axis=0) if ks.size else np.zeros(M, np.uint8)
        np.testing.assert_array_equal(regs[i], want)


def test_capacity_sample_and_workflow_rule():
    P = np.array([0, 5, 100, 100, 3])
    est = np.array([0.0, 9.2, 10.0, 80.0, 0.4])
    np.testing.assert_array_equal(oracle.capacity(P, None, 2.0), P)
    np.testing.assert_array_equal(oracle.capacity(P, est, 1.5), [0, 5, 15, 100, 1])
    np.testing.assert_array_equal(oracle.capacity(P, est, 2.0), [0, 5, 20, 100, 1])
    assert oracle.hll_registers(47 * 100, 100) == 32 and oracle.hll_registers(48 * 100, 100) == 64
    assert oracle.hll_coefficient(32) == 2.0 and oracle.hll_coefficient(64) == 1.5
    assert len(oracle.sample_rows(100)) == 100
    assert len(oracle.sample_rows(5000)) == 600
    assert len(oracle.sample_rows(100000)) == 3000
    assert len(oracle.sample_rows(10 ** 6)) == 10000
    s = oracle.sample_rows(12345)
    assert s[0] == 0 and np.all(np.diff(s) > 0) and s[-1] < 12345
    # Table 1: upper bound below 64 products per row; estimation when the
    # expansion ratio and the sampled compression ratio are both >= 8
    assert oracle.select_workflow(1000, 5000, 63999, 100.0) == 1
    assert oracle.select_workflow(1000, 5000, 64000, 8.0) == 2
    assert oracle.select_workflow(1000, 8000, 64000, 8.0) == 2
    assert oracle.select_workflow(1000, 8001, 64000, 8.0) == 0
    assert oracle.select_workflow(1000, 5000, 64000, 7.99) == 0


# --- planted mistakes -------------------------------------------------------

_MUTANTS = {
    "dropped_term": ("for (int64_t b = b_rp[k]; b < b_rp[k + 1]; ++b) {\n      int32_t c = b_col[b];\n      double p",
                     "for (int64_t b = b_rp[k]; b < b_rp[k + 1] - 1; ++b) {\n      int32_t c = b_col[b];\n      double p"),
    "wrong_sign": ("cmp[c] += (s - t) + p;", "cmp[c] -= (s - t) + p;"),
    "wrong_index": ("double p = a * (val_is_f32 ? (double)bf[b] : bd[b]);",
                    "double p = a * (val_is_f32 ? (double)bf[b_rp[k]] : bd[b_rp[k]]);"),
    "unsorted": ("qsort(touched, (size_t)nt, sizeof(int32_t), cmp_i32);", "(void)cmp_i32;"),
    "a_value_index": ("double a = val_is_f32 ? (double)af[j] : ad[j];",
                      "double a = val_is_f32 ? (double)af[a_rp[i]] : ad[a_rp[i]];"),
    "mcl_no_square": ("z = (double)(y * y);", "z = (double)y;"),
    "mcl_prune_raw": ("k = y >= (float)threshold;", "k = (float)c_val[e] >= (float)threshold;"),
    "mcl_count_not_sum": ("e < c_rp[i + 1]; ++e) colsum[c_col[e]] += c_val[e];",
                          "e < c_rp[i + 1]; ++e) colsum[c_col[e]] += 1.0;"),
    "transpose_rows_reversed": ("for (int64_t i = 0; i < m; ++i) {\n    for (int64_t e = a_rp[i]; e < a_rp[i + 1]; ++e) {\n      const int64_t q",
                                "for (int64_t i = m - 1; i >= 0; --i) {\n    for (int64_t e = a_rp[i]; e < a_rp[i + 1]; ++e) {\n      const int64_t q"),
    "transpose_value_index": ("((double *)t_val)[q] = ((const double *)a_val)[e];",
                              "((double *)t_val)[q] = ((const double *)a_val)[q];"),
    "transpose_row_index": ("t_col[q] = (int32_t)i;", "t_col[q] = a_col[e];"),
    "hll_rank_off_by_one": ("rank = (31 - lg) - b + 1;", "rank = (31 - lg) - b + 2;"),
    "hll_alpha": ("const double alpha = M == 32 ? 0.697 : 0.709;",
                  "const double alpha = M == 32 ? 0.797 : 0.809;"),
    "hll_no_linear_counting": ("if (e <= 2.5 * M && zeros > 0)", "if (e <= 0.0 && zeros > 0)"),
    "hll_unhashed": ("const uint32_t h = hll_hash((uint32_t)c);", "const uint32_t h = (uint32_t)c;"),
}


def _pins_pass(lib_path):
    """Run the brute-force, Laplacian and transpose pins against a given
    library; return True when all of them pass."""
    saved_lib, saved_path = oracle._lib, oracle._LIB
    try:
        oracle._lib, oracle._LIB = None, lib_path
        try:
            for (m, k, n, pr, seed) in [(40, 30, 50, 3.0, 2), (64, 64, 64, 4.0, 3)]:
                A = synth.random_csr(m, k, pr, seed, values="int", empty_row_frac=0.2)
                B = synth.random_csr(k, n, pr, seed + 100, values="int", empty_row_frac=0.2)
                _check_vs_bruteforce(A, B)
            _laplacian_closed_form_check(4)
            test_transpose_identity("rect")
            test_compensated_sum_exact()
            test_mcl_inflate_hand_example()
            test_mcl_inflate_fixpoints()
            test_transpose_hand_example()
            test_transpose_against_scipy_and_sort(500, 800, 6.0, 4)
            test_hll_accuracy(32)
            test_hll_accuracy(64)
            test_hll_special_cases()
        except (AssertionError, RuntimeError):
            return False
        return True
    finally:
        oracle._lib, oracle._LIB = saved_lib, saved_path


@pytest.mark.parametrize("name", sorted(_MUTANTS))
def test_mutants_fail(name):
    src = open(oracle._SRC).read()
    old, new = _MUTANTS[name]
    assert old in src, name
    d = tempfile.mkdtemp()
    try:
        shutil.copy(os.path.join(os.path.dirname(oracle._SRC), "oracle.h"), d)
        with open(os.path.join(d, "oracle.c"), "w") as f:
            f.write(src.replace(old, new))
        lib = os.path.join(d, "libmut.so")
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
                               "-o", lib, os.path.join(d, "oracle.c"), "-lm"])
        assert not _pins_pass(lib), f"mutant {name} passed the pins"
    finally:
        shutil.rmtree(d)


def test_unmutated_passes_pins():
    assert _pins_pass(oracle.build(force=False))


# --- the row-by-row checker used by the full-size GPU parity tests ----------

@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_check_rows_accepts_oracle_and_flags_planted_errors(dtype):
    # The checker recomputes each row as oracle_numeric does; it must accept
    # the oracle's own C (rounded to the value type) over any row block, and
    # flag a wrong row length, a wrong column and a value outside the bound.
    A = synth.random_csr(300, 250, 6.0, 71, values="uniform", empty_row_frac=0.2, dtype=dtype)
    B = synth.random_csr(250, 400, 7.0, 72, values="uniform", empty_row_frac=0.2, dtype=dtype)
    ref = oracle.spgemm(A, B)
    rtol = 1e-12 if dtype == np.float64 else 1e-5
    g = ref.val.astype(dtype)
    rep = oracle.check_rows(A, B, 0, A.m, ref.row_ptr, ref.col, g, rtol)
    assert rep.ok and rep.entries == ref.col.size and rep.max_terms == int(ref.terms.max())
    # a block in the middle, its entries given from their own offset
    r0, r1 = 40, 170
    a, b = int(ref.row_ptr[r0]), int(ref.row_ptr[r1])
    rep = oracle.check_rows(A, B, r0, r1, ref.row_ptr[r0:r1 + 1], ref.col[a:b], g[a:b], rtol)
    assert rep.ok and rep.entries == b - a
    # integer inputs must match exactly
    Ai = synth.random_csr(120, 90, 5.0, 73, values="int", dtype=dtype)
    Bi = synth.random_csr(90, 110, 5.0, 74, values="int", dtype=dtype)
    ri = oracle.spgemm(Ai, Bi)
    assert oracle.check_rows(Ai, Bi, 0, Ai.m, ri.row_ptr, ri.col, ri.val.astype(dtype), 0,
                             exact=True).ok
    # a value one tolerance step outside the bound
    e = int(np.argmax(ref.mag))
    bad = g.copy()
    bad[e] = dtype(ref.val[e] + 3 * rtol * ref.mag[e])
    rep = oracle.check_rows(A, B, 0, A.m, ref.row_ptr, ref.col, bad, rtol)
    assert rep.bad_values == 1 and rep.first_bad_value == e and rep.bad_rows == 0
    # a wrong column inside a row
    row = int(np.nonzero(np.diff(ref.row_ptr) >= 2)[0][3])
    cc = ref.col.copy()
    cc[ref.row_ptr[row]] = cc[ref.row_ptr[row] + 1]
    rep = oracle.check_rows(A, B, 0, A.m, ref.row_ptr, cc, g, rtol)
    assert rep.bad_rows == 1 and rep.first_bad_row == row
    # a row one entry short (the next row starts one earlier)
    rp = ref.row_ptr.copy()
    rp[row + 1] -= 1
    rep = oracle.check_rows(A, B, 0, A.m, rp, ref.col, g, rtol)
    assert rep.bad_rows == 2 and rep.first_bad_row == row
