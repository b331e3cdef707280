"""Python access to the CPU oracle (liboracle.so).  TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg may
import this package.  The HIP library neither imports nor links it.

The oracle computes C = A*B for CSR inputs by Gustavson's row-wise method
with a per-thread dense accumulator (gMAGNUS page, §II-B, Eq. 1, Algorithm 1)
and returns, per entry, the Neumaier-compensated fp64 value, the sum of the
absolute values of its terms and the number of terms.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

_i64p = ctypes.POINTER(ctypes.c_int64)


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (plain C, OpenMP, no FP contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC",
                               "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        vp = ctypes.c_void_p
        i64 = ctypes.c_int64
        lib.oracle_row_products.restype = i64
        lib.oracle_row_products.argtypes = [i64, i64, vp, vp, vp, vp]
        lib.oracle_symbolic.restype = ctypes.c_int
        lib.oracle_symbolic.argtypes = [i64, i64, i64, vp, vp, vp, vp, vp, ctypes.c_int]
        lib.oracle_numeric.restype = ctypes.c_int
        lib.oracle_numeric.argtypes = [i64, i64, i64, vp, vp, vp, vp, vp, vp, ctypes.c_int,
                                       vp, vp, vp, vp, vp, ctypes.c_int]
        lib.oracle_check_rows.restype = i64
        lib.oracle_check_rows.argtypes = [i64, i64, i64, vp, vp, vp, vp, vp, vp, ctypes.c_int,
                                          vp, i64, vp, vp, ctypes.c_int, ctypes.c_double,
                                          ctypes.c_int, vp, vp, ctypes.c_int]
        lib.oracle_prune_colnorm.restype = i64
        lib.oracle_prune_colnorm.argtypes = [i64, i64, vp, vp, vp, ctypes.c_float, vp,
                                             vp, vp, vp]
        lib.oracle_mcl_inflate.restype = i64
        lib.oracle_mcl_inflate.argtypes = [i64, i64, vp, vp, vp, ctypes.c_double, ctypes.c_int,
                                           vp, vp, vp, vp]
        lib.oracle_transpose.restype = ctypes.c_int
        lib.oracle_hll_sketch.restype = ctypes.c_int
        lib.oracle_hll_sketch.argtypes = [i64, vp, vp, ctypes.c_int, vp]
        lib.oracle_hll_estimate.restype = ctypes.c_int
        lib.oracle_hll_estimate.argtypes = [i64, i64, vp, vp, vp, vp, ctypes.c_int, vp, vp]
        lib.oracle_transpose.argtypes = [i64, i64, vp, vp, vp, ctypes.c_int, vp, vp, vp]
        _lib = lib
    return _lib


def _p(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


@dataclass
class OracleResult:
    row_ptr: np.ndarray   # int64, local to the row range (row_ptr[0] == 0)
    col: np.ndarray       # int32
    val: np.ndarray       # float64 (compensated sum)
    mag: np.ndarray       # float64, sum of |terms|
    terms: np.ndarray     # int32, number of products summed
    r0: int
    r1: int


def row_products(A, B, r0: int = 0, r1: int | None = None) -> np.ndarray:
    """Per-row intermediate-product counts P_i of A*B (int64)."""
    lib = _load()
    r1 = A.m if r1 is None else r1
    arp, acol, brp = _c(A.row_ptr, np.int32), _c(A.col, np.int32), _c(B.row_ptr, np.int32)
    out = np.zeros(r1 - r0, dtype=np.int64)
    lib.oracle_row_products(r0, r1, _p(arp), _p(acol), _p(brp), _p(out))
    return out


def symbolic(A, B, r0: int = 0, r1: int | None = None, nthreads: int = 0) -> np.ndarray:
    """nnz of each row of A*B in [r0, r1) (int64)."""
    lib = _load()
    r1 = A.m if r1 is None else r1
    assert A.n == B.m
    arp, acol = _c(A.row_ptr, np.int32), _c(A.col, np.int32)
    brp, bcol = _c(B.row_ptr, np.int32), _c(B.col, np.int32)
    cnt = np.zeros(r1 - r0, dtype=np.int64)
    rc = lib.oracle_symbolic(r0, r1, B.n, _p(arp), _p(acol), _p(brp), _p(bcol), _p(cnt), nthreads)
    if rc != 0:
        raise MemoryError("oracle_symbolic failed (%d)" % rc)
    return cnt


def spgemm(A, B, r0: int = 0, r1: int | None = None, nthreads: int = 0,
           rows: np.ndarray | None = None) -> OracleResult:
    """C = A*B on rows [r0, r1) of A (or on the listed rows, in that order)."""
    lib = _load()
    assert A.n == B.m
    f32 = A.val.dtype == np.float32
    assert B.val.dtype == A.val.dtype
    vdt = np.float32 if f32 else np.float64
    arp, acol, aval = _c(A.row_ptr, np.int32), _c(A.col, np.int32), _c(A.val, vdt)
    brp, bcol, bval = _c(B.row_ptr, np.int32), _c(B.col, np.int32), _c(B.val, vdt)
    if rows is not None:
        # Build a row-gathered copy of A so that the listed rows become rows
        # [0, len(rows)) of a smaller matrix; the arithmetic is unchanged.
        rows = np.asarray(rows, dtype=np.int64)
        starts = arp[rows].astype(np.int64)
        lens = arp[rows + 1].astype(np.int64) - starts
        rp = np.zeros(rows.shape[0] + 1, dtype=np.int64)
        np.cumsum(lens, out=rp[1:])
        idx = np.repeat(starts - rp[:-1], lens) + np.arange(int(rp[-1]), dtype=np.int64)
        arp, acol, aval = _c(rp, np.int32), _c(acol[idx], np.int32), _c(aval[idx], vdt)
        r0, r1 = 0, rows.shape[0]
    r1 = (arp.shape[0] - 1) if r1 is None else r1
    cnt = np.zeros(r1 - r0, dtype=np.int64)
    rc = lib.oracle_symbolic(r0, r1, B.n, _p(arp), _p(acol), _p(brp), _p(bcol), _p(cnt), nthreads)
    if rc != 0:
        raise MemoryError("oracle_symbolic failed (%d)" % rc)
    crp = np.zeros(r1 - r0 + 1, dtype=np.int64)
    np.cumsum(cnt, out=crp[1:])
    nnz = int(crp[-1])
    col = np.empty(nnz, dtype=np.int32)
    val = np.empty(nnz, dtype=np.float64)
    mag = np.empty(nnz, dtype=np.float64)
    terms = np.empty(nnz, dtype=np.int32)
    rc = lib.oracle_numeric(r0, r1, B.n, _p(arp), _p(acol), _p(aval), _p(brp), _p(bcol),
                            _p(bval), 1 if f32 else 0, _p(crp), _p(col), _p(val), _p(mag),
                            _p(terms), nthreads)
    if rc != 0:
        raise RuntimeError("oracle_numeric failed (%d)" % rc)
    return OracleResult(crp, col, val, mag, terms, r0, r1)


@dataclass
class CheckReport:
    bad_rows: int        # rows whose length or columns differ
    first_bad_row: int   # -1 when none
    bad_values: int      # entries outside the tolerance
    first_bad_value: int # offset in C of the first, -1 when none
    entries: int         # entries compared
    max_terms: int       # most products summed into one entry
    max_rel: float       # largest |g - c| / |c| over entries with c != 0

    @property
    def ok(self) -> bool:
        return self.bad_rows == 0 and self.bad_values == 0


def check_rows(A, B, r0: int, r1: int, g_rp, g_col, g_val, rtol: float, exact: bool = False,
               g_base: int | None = None, nthreads: int = 0) -> CheckReport:
    """Compare rows [r0, r1) of another implementation's C = A*B with the
    oracle, row by row, without forming the oracle's C.  g_rp: the r1-r0+1
    row offsets of those rows (absolute); g_col, g_val: their entries, the
    first at absolute offset g_base (default g_rp[0]).  A row must match in
    length and columns exactly; a value c' must satisfy |c' - c| <= rtol *
    sum of |terms| (exact: c' == c), c being the compensated oracle value."""
    lib = _load()
    assert A.n == B.m
    f32 = A.val.dtype == np.float32
    vdt = np.float32 if f32 else np.float64
    arp, acol, aval = _c(A.row_ptr, np.int32), _c(A.col, np.int32), _c(A.val, vdt)
    brp, bcol, bval = _c(B.row_ptr, np.int32), _c(B.col, np.int32), _c(B.val, vdt)
    grp = _c(g_rp, np.int64)
    assert grp.shape[0] == r1 - r0 + 1
    gcol = _c(g_col, np.int32)
    gf32 = np.asarray(g_val).dtype == np.float32
    gval = _c(g_val, np.float32 if gf32 else np.float64)
    base = int(grp[0]) if g_base is None else int(g_base)
    assert gcol.shape[0] >= int(grp[-1]) - base and gval.shape[0] == gcol.shape[0]
    rep = np.zeros(8, dtype=np.int64)
    mr = np.zeros(1, dtype=np.float64)
    rc = lib.oracle_check_rows(r0, r1, B.n, _p(arp), _p(acol), _p(aval), _p(brp), _p(bcol),
                               _p(bval), 1 if f32 else 0, _p(grp), base, _p(gcol), _p(gval),
                               1 if gf32 else 0, float(rtol), 1 if exact else 0, _p(rep),
                               _p(mr), nthreads)
    if rc < 0:
        raise MemoryError("oracle_check_rows failed")
    return CheckReport(int(rep[0]), int(rep[1]), int(rep[2]), int(rep[3]), int(rep[4]),
                       int(rep[5]), float(mr[0]))


def prune_colnorm(m: int, n: int, row_ptr, col, val, threshold: float = 1e-4,
                  keep: np.ndarray | None = None):
    """Markov-clustering prune (keep c >= threshold, compared in fp32) and
    column renormalisation (divide by the fp64 sum of the kept column).
    Returns (row_ptr int64, col int32, val float64)."""
    lib = _load()
    rp, cc, vv = _c(row_ptr, np.int64), _c(col, np.int32), _c(val, np.float64)
    kk = None if keep is None else _c(keep, np.int8)
    nnz = cc.shape[0]
    orp = np.zeros(m + 1, dtype=np.int64)
    oc = np.empty(nnz, dtype=np.int32)
    ov = np.empty(nnz, dtype=np.float64)
    w = lib.oracle_prune_colnorm(m, n, _p(rp), _p(cc), _p(vv), ctypes.c_float(threshold),
                                 _p(kk), _p(orp), _p(oc), _p(ov))
    if w < 0:
        raise MemoryError("oracle_prune_colnorm failed")
    return orp, oc[:w].copy(), ov[:w].copy()


def mcl_inflate(m: int, n: int, row_ptr, col, val, threshold: float = 0.002,
                single: bool = True, keep: np.ndarray | None = None):
    """The rest of one Markov-clustering iteration after the expansion:
    column normalisation (fp64 sums of every entry; each value divided in
    fp64 and rounded to fp32 when `single`), prune below `threshold`
    (compared in fp32 when `single`), square (in fp32 when `single`).
    Returns (row_ptr int64, col int32, val float64)."""
    lib = _load()
    rp, cc, vv = _c(row_ptr, np.int64), _c(col, np.int32), _c(val, np.float64)
    kk = None if keep is None else _c(keep, np.int8)
    nnz = cc.shape[0]
    orp = np.zeros(m + 1, dtype=np.int64)
    oc = np.empty(max(nnz, 1), dtype=np.int32)
    ov = np.empty(max(nnz, 1), dtype=np.float64)
    w = lib.oracle_mcl_inflate(m, n, _p(rp), _p(cc), _p(vv), float(threshold),
                               1 if single else 0, _p(kk), _p(orp), _p(oc), _p(ov))
    if w < 0:
        raise MemoryError("oracle_mcl_inflate failed")
    return orp, oc[:w].copy(), ov[:w].copy()


@dataclass
class CSRMatrix:
    """An m x n CSR matrix in host arrays (the attribute names spgemm reads)."""
    row_ptr: np.ndarray   # int64, m+1
    col: np.ndarray       # int32
    val: np.ndarray | None
    m: int
    n: int


def transpose(A) -> CSRMatrix:
    """A^T by the definition T[j, i] = A[i, j]; rows of T list their column
    indices in rising order, values are copied unchanged (A's dtype)."""
    lib = _load()
    rp, cc = _c(A.row_ptr, np.int64), _c(A.col, np.int32)
    vv = None
    if A.val is not None:
        vv = _c(A.val, np.float32 if A.val.dtype == np.float32 else np.float64)
    nnz = int(rp[A.m])
    trp = np.zeros(A.n + 1, dtype=np.int64)
    tc = np.empty(max(nnz, 1), dtype=np.int32)
    tv = None if vv is None else np.empty(max(nnz, 1), dtype=vv.dtype)
    rc = lib.oracle_transpose(A.m, A.n, _p(rp), _p(cc), _p(vv),
                              1 if (vv is not None and vv.dtype == np.float32) else 0,
                              _p(trp), _p(tc), _p(tv))
    if rc == -2:
        raise ValueError("column index out of range")
    if rc != 0:
        raise MemoryError("oracle_transpose failed")
    return CSRMatrix(trp, tc[:nnz].copy(), None if tv is None else tv[:nnz].copy(), A.n, A.m)


# --- Ocean's size-prediction workflows (Ocean page, §3 and its Table 1) ---

def hll_sketch(B, M: int) -> np.ndarray:
    """Per-row HyperLogLog registers of B: uint8 array (B.m, M)."""
    lib = _load()
    brp, bcol = _c(B.row_ptr, np.int32), _c(B.col, np.int32)
    regs = np.zeros((max(B.m, 1), M), dtype=np.uint8)
    if lib.oracle_hll_sketch(B.m, _p(brp), _p(bcol), M, _p(regs)) != 0:
        raise ValueError("M must be 32 or 64")
    return regs[:B.m]


def hll_estimate(A, B, M: int, r0: int = 0, r1: int | None = None, with_regs: bool = False):
    """HyperLogLog estimate of nnz(C_i) for rows [r0, r1) of C = A*B, from a
    sketch of each row's product columns (float64; registers on request)."""
    lib = _load()
    r1 = A.m if r1 is None else r1
    arp, acol = _c(A.row_ptr, np.int32), _c(A.col, np.int32)
    brp, bcol = _c(B.row_ptr, np.int32), _c(B.col, np.int32)
    est = np.zeros(max(r1 - r0, 1), dtype=np.float64)
    regs = np.zeros((max(r1 - r0, 1), M), dtype=np.uint8) if with_regs else None
    if lib.oracle_hll_estimate(r0, r1, _p(arp), _p(acol), _p(brp), _p(bcol), M, _p(est),
                               _p(regs)) != 0:
        raise ValueError("M must be 32 or 64")
    est = est[:r1 - r0]
    return (est, regs[:r1 - r0]) if with_regs else est


def hll_registers(products: int, nnz_a: int) -> int:
    """Sketch size: 32 registers when the input expansion ratio
    products / nnz(A) is below 48, else 64 (Ocean §4, parameters)."""
    return 32 if products < 48 * max(nnz_a, 1) else 64


def hll_coefficient(M: int) -> float:
    """Estimates are scaled by 1.5 (2.0 with 32 registers) before sizing
    (Ocean §5.3)."""
    return 2.0 if M == 32 else 1.5


def capacity(P: np.ndarray, est: np.ndarray | None, coef: float) -> np.ndarray:
    """Output slots reserved per row: the upper bound P_i, or with an estimate
    min(P_i, ceil(coef * est_i)) and at least 1 for a row with products."""
    P = np.asarray(P, dtype=np.int64)
    if est is None:
        return P.copy()
    c = np.ceil(coef * np.asarray(est, dtype=np.float64)).astype(np.int64)
    c = np.minimum(c, P)
    return np.where(P > 0, np.maximum(c, 1), 0)


def sample_rows(m: int) -> np.ndarray:
    """Rows sampled for the compression ratio: 3% of the rows, at least 600
    and at most 10,000 (all rows when fewer), evenly spaced."""
    s = min(m, min(10000, max(600, int(round(0.03 * m)))))
    return (np.arange(s, dtype=np.int64) * m) // max(s, 1)


def select_workflow(m: int, nnz_a: int, products: int, sampled_cr: float | None) -> int:
    """Ocean's Table 1: 1 = upper bound when the average products per row is
    below 64; else 2 = HyperLogLog estimation when the expansion ratio
    products / nnz(A) and the sampled compression ratio are both >= 8; else
    0 = symbolic."""
    if products < 64 * m:
        return 1
    if products >= 8 * nnz_a and sampled_cr is not None and sampled_cr >= 8.0:
        return 2
    return 0
