"""Seeded synthetic CSR matrices shaped like the workloads on the pages.

This module holds no SpGEMM arithmetic: it only draws sparsity patterns and
values.  The CPU oracle (tests) and the HIP path (tests, bench) both consume
the arrays it returns, so the two sides are compared on identical inputs.

Every generator is deterministic for a given seed (numpy PCG64).  All outputs
are canonical CSR: row_ptr[0] == 0, row_ptr monotone, column indices sorted
ascending and unique inside each row, 0 <= col < ncols.

Workload sources
----------------
* Erdos-Renyi rows (Poisson(8) entries per row, uniform columns): a small,
  general-purpose case.
* 27-point Laplacian on an nx^3 grid: the banded / well-behaved class the
  gMAGNUS page contrasts with power-law inputs (gMAGNUS, §I and §II-B).
* R-MAT with the Graph500 parameters a=0.57, b=c=0.19 (gMAGNUS, §IV-A), here
  squared at edge factor 16 with duplicates merged.
* Planted-partition, column-stochastic matrix for one Markov-clustering
  expansion (Trident page, §5.7).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

__all__ = [
    "CSR", "erdos_renyi", "laplacian27", "rmat", "planted_partition",
    "random_csr", "identity", "workload", "rmat_rect", "sparse_uniform", "aggregation",
    "grid_aggregation", "banded_outliers",
]


@dataclass
class CSR:
    """A CSR matrix held in host numpy arrays (int32 indices)."""
    row_ptr: np.ndarray   # int32 or int64, length m+1
    col: np.ndarray       # int32, length nnz
    val: np.ndarray       # float64 or float32, length nnz
    m: int                # rows
    n: int                # columns

    @property
    def nnz(self) -> int:
        return int(self.col.shape[0])

    def check_canonical(self) -> None:
        rp = self.row_ptr.astype(np.int64)
        assert rp.shape == (self.m + 1,)
        assert rp[0] == 0 and rp[-1] == self.nnz
        assert np.all(np.diff(rp) >= 0)
        if self.nnz:
            assert self.col.min() >= 0 and self.col.max() < self.n
            # strictly increasing inside each row
            d = np.diff(self.col.astype(np.int64))
            row_of = np.repeat(np.arange(self.m), np.diff(rp))
            same_row = row_of[1:] == row_of[:-1]
            assert np.all(d[same_row] > 0)

    def to_dense(self) -> np.ndarray:
        out = np.zeros((self.m, self.n), dtype=np.float64)
        rows = np.repeat(np.arange(self.m), np.diff(self.row_ptr.astype(np.int64)))
        out[rows, self.col] = self.val
        return out


def _from_sorted_keys(keys: np.ndarray, m: int, n: int, val: np.ndarray) -> CSR:
    """Build CSR from unique int64 keys row*n+col that are sorted ascending."""
    rows = keys // n
    cols = (keys - rows * n).astype(np.int32)
    counts = np.bincount(rows, minlength=m)
    rp = np.zeros(m + 1, dtype=np.int64)
    np.cumsum(counts, out=rp[1:])
    return CSR(rp.astype(np.int32), cols, val, m, n)


def _distinct_draws(rng: np.random.Generator, rows: int, k: int, universe: int) -> np.ndarray:
    """rows x k matrix whose rows are uniform random k-subsets of [0, universe).

    Draw with replacement, then redraw duplicated positions until every row is
    duplicate-free.  The procedure treats all elements of the universe alike,
    so each row's final set is a uniform k-subset.
    """
    assert k <= universe
    x = rng.integers(0, universe, size=(rows, k), dtype=np.int64)
    while True:
        s = np.sort(x, axis=1)
        dup_sorted = np.zeros_like(s, dtype=bool)
        dup_sorted[:, 1:] = s[:, 1:] == s[:, :-1]
        bad_rows = np.nonzero(dup_sorted.any(axis=1))[0]
        if bad_rows.size == 0:
            return s
        x = s
        sub = x[bad_rows]
        d = dup_sorted[bad_rows]
        sub[d] = rng.integers(0, universe, size=int(d.sum()), dtype=np.int64)
        x[bad_rows] = sub


def erdos_renyi(n: int = 4096, mean_per_row: float = 8.0, seed: int = 0,
                ncols: int | None = None, dtype=np.float64,
                lo: float = -1.0, hi: float = 1.0) -> CSR:
    """Rows with Poisson(mean) entries (clipped to ncols), distinct uniform
    sorted columns, values uniform in [lo, hi)."""
    ncols = n if ncols is None else ncols
    rng = np.random.default_rng(seed)
    k = np.minimum(rng.poisson(mean_per_row, size=n), ncols).astype(np.int64)
    cols = []
    for i in range(n):
        if k[i]:
            cols.append(np.sort(rng.choice(ncols, size=int(k[i]), replace=False)))
    col = (np.concatenate(cols) if cols else np.zeros(0, np.int64)).astype(np.int32)
    rp = np.zeros(n + 1, dtype=np.int64)
    np.cumsum(k, out=rp[1:])
    val = rng.uniform(lo, hi, size=col.shape[0]).astype(dtype)
    return CSR(rp.astype(np.int32), col, val, n, ncols)


def laplacian27(nx: int = 64, dtype=np.float64) -> CSR:
    """27-point stencil on an nx^3 grid, lexicographic index x + nx*(y + nx*z).

    Neighbours at max-norm distance <= 1, truncated at the boundary (no wrap);
    26 on the diagonal and -1 off it.
    """
    N = nx ** 3
    idx = np.arange(N, dtype=np.int64)
    x = idx % nx
    y = (idx // nx) % nx
    z = idx // (nx * nx)
    cols, vals, valid = [], [], []
    # (dz, dy, dx) in lexicographic order gives ascending column indices.
    for dz in (-1, 0, 1):
        for dy in (-1, 0, 1):
            for dx in (-1, 0, 1):
                ok = ((x + dx >= 0) & (x + dx < nx) & (y + dy >= 0) & (y + dy < nx)
                      & (z + dz >= 0) & (z + dz < nx))
                cols.append(idx + dx + nx * dy + nx * nx * dz)
                vals.append(26.0 if (dx, dy, dz) == (0, 0, 0) else -1.0)
                valid.append(ok)
    C = np.stack(cols, axis=1)
    V = np.broadcast_to(np.array(vals), C.shape)
    M = np.stack(valid, axis=1)
    counts = M.sum(axis=1)
    rp = np.zeros(N + 1, dtype=np.int64)
    np.cumsum(counts, out=rp[1:])
    return CSR(rp.astype(np.int32), C[M].astype(np.int32), V[M].astype(dtype), N, N)


def rmat(scale: int, edge_factor: int = 16, abcd=(0.57, 0.19, 0.19, 0.05),
         seed: int = 0, dtype=np.float64, block: int = 1 << 22) -> CSR:
    """R-MAT graph: edge_factor * 2^scale directed edges, each placed by a
    recursive quadrant choice per bit (no noise, no vertex permutation);
    self-loops kept, duplicates merged to one entry, then one uniform [0,1)
    value per merged entry."""
    a, b, c, _ = abcd
    n = 1 << scale
    E = edge_factor * n
    rng = np.random.default_rng(seed)
    keys = np.empty(E, dtype=np.int64)
    t_ab, t_abc = a + b, a + b + c
    for s in range(0, E, block):
        e = min(E, s + block) - s
        r = np.zeros(e, dtype=np.int64)
        q = np.zeros(e, dtype=np.int64)
        for _bit in range(scale):
            u = rng.random(e)
            row_bit = u >= t_ab                       # quadrants c, d
            col_bit = ((u >= a) & (u < t_ab)) | (u >= t_abc)   # quadrants b, d
            r = (r << 1) | row_bit
            q = (q << 1) | col_bit
        keys[s:s + e] = r * n + q
    keys = np.unique(keys)
    val = rng.random(keys.shape[0]).astype(dtype)
    return _from_sorted_keys(keys, n, n, val)


def planted_partition(n_clusters: int = 1000, cluster_size: int = 1000,
                      intra: int = 28, inter: int = 4, seed: int = 0,
                      dtype=np.float32) -> CSR:
    """Column-stochastic planted-partition matrix.

    Column j lies in cluster c = j // cluster_size.  It gets `intra` distinct
    rows drawn uniformly from its cluster without j, `inter` distinct rows
    drawn uniformly from outside the cluster, and the self-loop (j, j).
    Weights are uniform [0,1); each column is divided by its sum in float64
    and the result rounded once to `dtype`.
    """
    n = n_clusters * cluster_size
    rng = np.random.default_rng(seed)
    j = np.arange(n, dtype=np.int64)
    cbase = (j // cluster_size) * cluster_size
    jloc = j - cbase
    x = _distinct_draws(rng, n, intra, cluster_size - 1)
    rows_in = cbase[:, None] + x + (x >= jloc[:, None])
    y = _distinct_draws(rng, n, inter, n - cluster_size)
    rows_out = y + cluster_size * (y >= cbase[:, None])
    rows = np.concatenate([rows_in, rows_out, j[:, None]], axis=1)   # n x (intra+inter+1)
    w = rng.random(rows.shape)
    w = w / w.sum(axis=1, keepdims=True)
    cols = np.broadcast_to(j[:, None], rows.shape)
    keys = (rows * n + cols).ravel()
    order = np.argsort(keys, kind="stable")
    keys = keys[order]
    val = w.ravel()[order].astype(dtype)
    return _from_sorted_keys(keys, n, n, val)


def random_csr(m: int, n: int, per_row: float, seed: int, values: str = "int",
               empty_row_frac: float = 0.0, dtype=np.float64, banded: int | None = None) -> CSR:
    """Small general-purpose test matrices.

    values: "int" draws integers in [-3, 3] (so products and sums are exact in
    fp64), "uniform" draws U[-1, 1), "pos" draws U[0, 1).
    banded: if given, columns are restricted to |col - row * n / m| <= banded.
    """
    rng = np.random.default_rng(seed)
    k = rng.poisson(per_row, size=m)
    if empty_row_frac > 0:
        k[rng.random(m) < empty_row_frac] = 0
    rows_cols = []
    for i in range(m):
        if banded is None:
            lo_c, hi_c = 0, n
        else:
            ctr = (i * n) // max(m, 1)
            lo_c, hi_c = max(0, ctr - banded), min(n, ctr + banded + 1)
        kk = int(min(k[i], hi_c - lo_c))
        k[i] = kk
        if kk:
            rows_cols.append(np.sort(rng.choice(np.arange(lo_c, hi_c), size=kk, replace=False)))
    col = (np.concatenate(rows_cols) if rows_cols else np.zeros(0, np.int64)).astype(np.int32)
    rp = np.zeros(m + 1, dtype=np.int64)
    np.cumsum(k, out=rp[1:])
    nnz = col.shape[0]
    if values == "int":
        val = rng.integers(-3, 4, size=nnz).astype(dtype)
    elif values == "pos":
        val = rng.random(nnz).astype(dtype)
    else:
        val = rng.uniform(-1.0, 1.0, size=nnz).astype(dtype)
    return CSR(rp.astype(np.int32), col, val, m, n)


def banded_outliers(m: int, n: int, in_band: int, band: int, outliers: int, seed: int,
                    values: str = "int", dtype=np.float64) -> CSR:
    """Rows with `in_band` distinct columns drawn within `band` of the
    diagonal position row * n / m and Poisson(`outliers`) more drawn
    uniformly from the whole row (a clustered matrix with thin links between
    clusters, as the Markov-clustering iterates).  values as for random_csr."""
    rng = np.random.default_rng(seed)
    cols = []
    for i in range(m):
        ctr = (i * n) // max(m, 1)
        lo_c, hi_c = max(0, ctr - band), min(n, ctr + band + 1)
        a = rng.choice(np.arange(lo_c, hi_c), size=min(in_band, hi_c - lo_c), replace=False)
        b = rng.integers(0, n, size=rng.poisson(outliers))
        cols.append(np.unique(np.concatenate([a, b])))
    k = np.array([c.size for c in cols], dtype=np.int64)
    col = np.concatenate(cols).astype(np.int32)
    rp = np.zeros(m + 1, dtype=np.int64)
    np.cumsum(k, out=rp[1:])
    if values == "int":
        val = rng.integers(-3, 4, size=col.size).astype(dtype)
    else:
        val = rng.random(col.size).astype(dtype)
    return CSR(rp.astype(np.int32), col, val, m, n)


def identity(n: int, dtype=np.float64) -> CSR:
    return CSR(np.arange(n + 1, dtype=np.int32), np.arange(n, dtype=np.int32),
               np.ones(n, dtype=dtype), n, n)


def rmat_rect(row_scale: int, col_scale: int, edges_per_row: int = 16,
              abcd=(0.57, 0.19, 0.19, 0.05), seed: int = 0, dtype=np.float64) -> CSR:
    """Rectangular R-MAT: 2^row_scale x 2^col_scale, edges_per_row * 2^row_scale
    edges.  The first min(row_scale, col_scale) bits of both indices come from
    quadrant choices as in rmat(); the remaining bits of the longer index use
    that index's marginal (c + d for a row bit, b + d for a column bit).
    Duplicates merged, one uniform [0,1) value per entry."""
    a, b, c, d = abcd
    m, n = 1 << row_scale, 1 << col_scale
    E = edges_per_row * m
    rng = np.random.default_rng(seed)
    r = np.zeros(E, dtype=np.int64)
    q = np.zeros(E, dtype=np.int64)
    for lvl in range(max(row_scale, col_scale)):
        u = rng.random(E)
        if lvl < min(row_scale, col_scale):
            r = (r << 1) | (u >= a + b)
            q = (q << 1) | (((u >= a) & (u < a + b)) | (u >= a + b + c))
        elif row_scale > col_scale:
            r = (r << 1) | (u < c + d)
        else:
            q = (q << 1) | (u < b + d)
    keys = np.unique(r * n + q)
    val = rng.random(keys.shape[0]).astype(dtype)
    return _from_sorted_keys(keys, m, n, val)


def sparse_uniform(m: int, n: int, per_row: float, seed: int, dtype=np.float64,
                   values: str = "uniform") -> CSR:
    """About per_row * m entries at uniform random positions of an m x n
    matrix (duplicates merged); values U[-1,1) or small integers ("int")."""
    rng = np.random.default_rng(seed)
    E = int(per_row * m)
    keys = np.unique(rng.integers(0, m * n, size=E, dtype=np.int64)) if m * n else \
        np.zeros(0, np.int64)
    if values == "int":
        val = rng.integers(-3, 4, size=keys.shape[0]).astype(dtype)
    else:
        val = rng.uniform(-1.0, 1.0, size=keys.shape[0]).astype(dtype)
    return _from_sorted_keys(keys, m, n, val)


def aggregation(n_fine: int, agg_size: int, seed: int = 0, dtype=np.float64) -> CSR:
    """Piecewise-constant aggregation operator, n_fine x ceil(n_fine/agg_size):
    the fine points, in a random order, are cut into aggregates of agg_size
    (the last may be smaller); R[i, agg(i)] = 1, one entry per row."""
    rng = np.random.default_rng(seed)
    nc = (n_fine + agg_size - 1) // agg_size
    agg = np.empty(n_fine, dtype=np.int64)
    agg[rng.permutation(n_fine)] = np.arange(n_fine, dtype=np.int64) // agg_size
    return CSR(np.arange(n_fine + 1, dtype=np.int32), agg.astype(np.int32),
               np.ones(n_fine, dtype=dtype), n_fine, nc)


def grid_aggregation(nx: int, a: int, dtype=np.float64) -> CSR:
    """Aggregation of an nx^3 grid (index x + nx*(y + nx*z)) into a x a x a
    blocks: R[i, block(i)] = 1, nx^3 x ceil(nx/a)^3."""
    nb = (nx + a - 1) // a
    i = np.arange(nx ** 3, dtype=np.int64)
    x, y, z = i % nx, (i // nx) % nx, i // (nx * nx)
    blk = (x // a) + nb * ((y // a) + nb * (z // a))
    return CSR(np.arange(nx ** 3 + 1, dtype=np.int32), blk.astype(np.int32),
               np.ones(nx ** 3, dtype=dtype), nx ** 3, nb ** 3)


# Named workloads: C = A.A for each.
WORKLOADS = {
    "er4096": "Erdos-Renyi 4096x4096, Poisson(8) per row, fp64 U[-1,1], seed 0",
    "lap27_64": "27-point Laplacian on a 64^3 grid (262,144 rows), fp64",
    "rmat18": "R-MAT scale 18, edge factor 16, (0.57,0.19,0.19,0.05), fp64 U[0,1], seed 0",
    "rmat20": "R-MAT scale 20, edge factor 16, (0.57,0.19,0.19,0.05), fp64 U[0,1], seed 0",
    "mcl1m": "planted partition 1000x1000 clusters, 28 intra + 4 inter + self per column, fp32 column-stochastic, seed 0",
    "rmat_rect": "rectangular R-MAT 2^17 x 2^20, 16 edges per row, (0.57,0.19,0.19,0.05), fp64 U[0,1], seed 0 (operand of A*A^T)",
    "agg_rmat18": "aggregation operator 2^18 x 2^15, random aggregates of 8, fp64 ones, seed 1 (operand R of A*R with A = rmat18)",
}


def workload(name: str) -> CSR:
    if name == "er4096":
        return erdos_renyi(4096, 8.0, seed=0)
    if name == "lap27_64":
        return laplacian27(64)
    if name == "rmat18":
        return rmat(18, 16, seed=0)
    if name == "rmat20":
        return rmat(20, 16, seed=0)
    if name == "mcl1m":
        return planted_partition(1000, 1000, 28, 4, seed=0)
    if name == "mcl_iter":
        return planted_partition(100, 1000, 28, 4, seed=0)
    if name == "rmat_rect":
        return rmat_rect(17, 20, 16, seed=0)
    if name == "agg_rmat18":
        return aggregation(1 << 18, 8, seed=1)
    m = name.split("_")
    if m[0] == "rmat" and len(m) == 2:          # e.g. "rmat_12"
        return rmat(int(m[1]), 16, seed=0)
    raise KeyError(name)
