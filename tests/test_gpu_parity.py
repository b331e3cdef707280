"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Structure (row_ptr and sorted col) must match exactly.  Values: integer-valued
inputs must match exactly; otherwise |c - c_ref| <= rtol * sum_k |a_ik b_kj|
per entry with rtol = 1e-12 (fp64) or 1e-5 (fp32).  The sum of |terms| is the
scale that bounds the error of any summation order (for same-sign terms it
equals |c_ref|).  Full-size configurations are checked on every row, streamed
to the host in row blocks and compared with the oracle row by row.
"""
import numpy as np
import pytest

import oracle
import synth
from conftest import assert_csr_equal_structure, assert_values_close

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
sg = pytest.importorskip("spgemm_symbolic_row_amd")

RTOL = {np.float64: 1e-12, np.float32: 1e-5}


def _rtol(A, ref):
    return RTOL[A.val.dtype.type]


def _to_np(t, dtype=None):
    a = t.detach().cpu().numpy()
    return a.astype(dtype) if dtype is not None else a


def gpu_product(A, B, **opts):
    dA = sg.to_device(A)
    dB = dA if B is A else sg.to_device(B)
    with sg.Plan(dA, dB, **opts) as p:
        rp, nnz = p.symbolic()
        col, val = p.numeric()
        st = p.stats()
    torch.cuda.synchronize()
    return _to_np(rp, np.int64), _to_np(col), _to_np(val), st


def check_full(A, B, exact=False, **opts):
    rp, col, val, st = gpu_product(A, B, **opts)
    ref = oracle.spgemm(A, B)
    assert_csr_equal_structure(rp, col, ref.row_ptr, ref.col, "C")
    if exact:
        np.testing.assert_array_equal(val, ref.val)
    else:
        assert_values_close(val, ref.val, ref.mag, _rtol(A, ref), "C")
    assert st["lds_hash_products"] + st["lds_dense_products"] == st["products"]
    assert st["nnz_c"] == int(ref.row_ptr[-1])
    return st


# ------------------------------------------------------------ small shapes
@pytest.mark.parametrize("dtype", [np.float64, np.float32])
@pytest.mark.parametrize("m,k,n,per_row,seed", [
    (1, 1, 1, 1.0, 0), (7, 5, 3, 2.0, 1), (64, 64, 64, 4.0, 3), (300, 200, 500, 6.0, 4),
    (1000, 1, 1000, 0.7, 5), (50, 120, 7, 10.0, 6), (2000, 3000, 1500, 12.0, 7),
])
def test_small_random_exact(m, k, n, per_row, seed, dtype):
    A = synth.random_csr(m, k, per_row, seed, values="int", empty_row_frac=0.2, dtype=dtype)
    B = synth.random_csr(k, n, per_row, seed + 100, values="int", empty_row_frac=0.2, dtype=dtype)
    check_full(A, B, exact=True)


@pytest.mark.parametrize("opts", [{}, {"workflow": 1}, {"workflow": 2}, {"workflow": 3},
                                  {"light_no_esc": 1}], ids=["wf0", "wf1", "wf2", "wf3", "noesc"])
@pytest.mark.parametrize("case", ["m0", "k0", "nnz0", "single", "empty_b"])
def test_degenerate(case, opts):
    if case == "m0":
        A = synth.CSR(np.zeros(1, np.int32), np.zeros(0, np.int32), np.zeros(0), 0, 5)
        B = synth.random_csr(5, 6, 2.0, 1)
    elif case == "k0":
        A = synth.CSR(np.zeros(4, np.int32), np.zeros(0, np.int32), np.zeros(0), 3, 0)
        B = synth.CSR(np.zeros(1, np.int32), np.zeros(0, np.int32), np.zeros(0), 0, 6)
    elif case == "nnz0":
        A = synth.CSR(np.zeros(11, np.int32), np.zeros(0, np.int32), np.zeros(0), 10, 10)
        B = synth.random_csr(10, 10, 3.0, 2)
    elif case == "single":
        A = synth.CSR(np.array([0, 1], np.int32), np.array([0], np.int32), np.array([2.0]), 1, 1)
        B = synth.CSR(np.array([0, 1], np.int32), np.array([0], np.int32), np.array([3.0]), 1, 1)
    else:
        A = synth.random_csr(20, 30, 4.0, 3)
        B = synth.CSR(np.zeros(31, np.int32), np.zeros(0, np.int32), np.zeros(0), 30, 9)
    check_full(A, B, exact=True, **opts)


def test_er4096_config():
    A = synth.workload("er4096")
    st = check_full(A, A)
    assert st["heavy_rows"] == 0


def test_uniform_values_fp64_and_fp32():
    for dt in (np.float64, np.float32):
        A = synth.random_csr(3000, 2500, 20.0, 11, values="uniform", dtype=dt)
        B = synth.random_csr(2500, 4000, 30.0, 12, values="uniform", dtype=dt)
        check_full(A, B)


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_esc_short_rows_match_hash(dtype):
    # Rows of at most 32 products take the expand-sort-compact kernel: rows of
    # up to 60 entries whose B rows are mostly empty (more entries than
    # lanes), duplicate columns, empty rows; the hash kernels and the oracle
    # agree with it.
    B = synth.random_csr(3000, 400, 0.8, 41, values="int", empty_row_frac=0.8, dtype=dtype)
    A = synth.random_csr(2000, 3000, 25.0, 42, values="int", empty_row_frac=0.1, dtype=dtype)
    P = oracle.row_products(A, B)
    assert P.max() <= 32 and (np.diff(A.row_ptr) > 32).any()
    st = check_full(A, B, exact=True)
    st2 = check_full(A, B, exact=True, light_no_esc=1)
    assert st["nnz_c"] == st2["nnz_c"]
    C = synth.random_csr(4000, 4000, 3.0, 43, values="uniform", dtype=dtype)
    check_full(C, C)


def test_wide_light_rows_all_bins():
    # rows of 1..~6000 products exercise every light-row bin, with both hash
    # sizes and sorts near their capacity
    rng = np.random.default_rng(5)
    m, k, n = 4000, 3000, 200000
    A = synth.random_csr(m, k, 1.0, 13, values="int")
    lens = np.minimum((2.0 ** rng.uniform(0, 12.5, size=m)).astype(int), k)
    cols = [np.sort(rng.choice(k, size=int(c), replace=False)) for c in lens]
    rp = np.zeros(m + 1, np.int64)
    np.cumsum(lens, out=rp[1:])
    A = synth.CSR(rp.astype(np.int32), np.concatenate(cols).astype(np.int32),
                  rng.integers(-3, 4, size=int(rp[-1])).astype(np.float64), m, k)
    B = synth.random_csr(k, n, 1.5, 14, values="int")
    st = check_full(A, B, exact=True)
    assert st["heavy_rows"] == 0 or st["heavy_products"] > 0


# ------------------------------------------------ dense-window light rows
@pytest.mark.parametrize("dtype", [np.float64, np.float32])
@pytest.mark.parametrize("m,n,per_row,band,seed", [
    (3000, 3000, 3.0, 40, 21),      # small bins, narrow spans
    (2000, 2500, 14.0, 300, 22),    # middle bins
    (1500, 60000, 40.0, 1000, 23),  # large bins, spans up to a few thousand columns
    (2500, 200000, 10.0, None, 24), # unbanded: spans too wide, the hash path
])
def test_dense_window_rows_match_hash(m, n, per_row, band, seed, dtype):
    # Light rows whose products span a narrow window take the LDS bitmap +
    # rank accumulator; turning it off must give the same C, and both the
    # oracle's.
    A = synth.random_csr(m, m, per_row, seed, values="int", empty_row_frac=0.1, dtype=dtype,
                         banded=band)
    B = synth.random_csr(m, n, per_row, seed + 50, values="int", empty_row_frac=0.1,
                         dtype=dtype, banded=None if band is None else band * n // m)
    st = check_full(A, B, exact=True)
    rp, col, val, st_h = gpu_product(A, B, light_hash_only=1)
    rp_w, col_w, val_w, _ = gpu_product(A, B)
    np.testing.assert_array_equal(rp, rp_w)
    np.testing.assert_array_equal(col, col_w)
    np.testing.assert_array_equal(val, val_w)
    assert st_h["lds_dense_products"] == 0
    if band is not None:
        assert st["lds_dense_products"] > 0
    else:
        assert st["lds_dense_products"] == 0


# ------------------------------- diagonal window plus outlier table (hybrid)
@pytest.mark.parametrize("dtype", [np.float64, np.float32])
@pytest.mark.parametrize("m,k,n,in_band,band,outl,seed", [
    (100000, 100000, 100000, 26, 400, 5, 31),  # most rows hybrid; first and last rows
                                               # have windows clipped by the matrix edge
    (150000, 150000, 150000, 14, 300, 12, 32), # many outliers: some rows over the table
    (30000, 60000, 150000, 20, 150, 6, 33),    # rectangular (window centre row * n / m)
])
def test_hybrid_window_rows(m, k, n, in_band, band, outl, seed, dtype):
    # Light rows of at least 512 products whose span is too wide for the
    # dense window take a dense window around their diagonal position plus a
    # hash table for the other columns; the hash path alone
    # (light_hash_only) and the oracle must agree with it.
    A = synth.banded_outliers(m, k, in_band, band, outl, seed, dtype=dtype)
    B = synth.banded_outliers(k, n, in_band, band * n // k, outl, seed + 1, dtype=dtype)
    st = check_full(A, B, exact=True)
    rp_h, col_h, val_h, st_h = gpu_product(A, B, light_hash_only=1)
    rp, col, val, _ = gpu_product(A, B)
    np.testing.assert_array_equal(rp, rp_h)
    np.testing.assert_array_equal(col, col_h)
    np.testing.assert_array_equal(val, val_h)
    assert st_h["hybrid_rows"] == 0
    assert st["heavy_rows"] == 0
    assert st["hybrid_rows"] > 0
    if outl >= 10:
        assert st["hybrid_rows"] < st["light_rows"]


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_hybrid_window_rows_largest_bin(dtype):
    # Light rows of up to tau products (heavy_row_threshold = tau): rows of
    # more than 2,048 entries, nearly all of the window's columns set plus a
    # few hundred outliers, take the 1024-thread hybrid kernel; the few rows
    # above tau products take the heavy path.
    A = synth.banded_outliers(100000, 100000, 80, 500, 2, 41, dtype=dtype)
    B = synth.banded_outliers(100000, 100000, 80, 500, 2, 42, dtype=dtype)
    st = check_full(A, B, exact=True, heavy_row_threshold=6826)
    rp_h, col_h, val_h, st_h = gpu_product(A, B, light_hash_only=1, heavy_row_threshold=6826)
    rp, col, val, _ = gpu_product(A, B, heavy_row_threshold=6826)
    np.testing.assert_array_equal(rp, rp_h)
    np.testing.assert_array_equal(col, col_h)
    np.testing.assert_array_equal(val, val_h)
    nnz = np.diff(rp)
    assert st["hybrid_rows"] > 0 and st_h["hybrid_rows"] == 0
    assert (nnz > 2048).sum() > 10000


# -------------------------------------------------- heavy path, forced sizes
@pytest.mark.parametrize("scale,tau,W,nmax", [
    (10, 64, 256, 32),     # one level, 4 chunks
    (11, 64, 256, 4),      # two levels [4, 2]
    (12, 32, 128, 2),      # five levels of 2
    (12, 200, 1024, 64),   # one level, light and dense chunks
    (11, 64, 2048, 32),    # one W-wide chunk: no multisplit
    (13, 64, 4096, 2),     # wide chunks: small ones take the hash kernels
])
@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_heavy_path_forced(scale, tau, W, nmax, dtype):
    A = synth.rmat(scale, 16, seed=scale)
    A.val = A.val.astype(dtype)
    st = check_full(A, A, heavy_threshold=tau, dense_width=W, max_chunks_per_level=nmax)
    assert st["heavy_rows"] > 0
    nreq = max(1, 1 << int(np.ceil(np.log2(max(A.n / W, 1)))))
    assert st["params"]["chunks_required"] == nreq
    if nreq > 1:
        assert st["level_elems"][0] == st["heavy_products"]


def test_heavy_integer_exact_multilevel():
    A = synth.rmat(12, 16, seed=21)
    A.val = np.round(A.val * 6 - 3)   # small integers: any summation order is exact
    check_full(A, A, exact=True, heavy_threshold=48, dense_width=256, max_chunks_per_level=4)


def test_rectangular_heavy():
    A = synth.random_csr(600, 400, 60.0, 31, values="int")
    B = synth.random_csr(400, 5000, 80.0, 32, values="int")
    check_full(A, B, exact=True, heavy_threshold=256, dense_width=512, max_chunks_per_level=4)


def test_rmat14_default_parameters():
    A = synth.rmat(14, 16, seed=0)
    st = check_full(A, A)
    assert st["params"]["tau"] == 6826


@pytest.mark.parametrize("direct", [0, 1], ids=["expanded", "dense_direct"])
@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_default_width_dense_chunks(dtype, direct):
    # The default chunk width (16384 for fp64, 32768 for fp32) with chunks
    # above a lowered tau, so the dense chunk kernels run at full width:
    # fp64 marks columns with bytes, fp32 with bits (bytes would not fit
    # beside the 128 KiB accumulator).
    A = synth.rmat(15, 16, seed=12, dtype=dtype)
    st = check_full(A, A, heavy_threshold=512, dense_direct=direct)
    assert st["heavy_rows"] > 0
    assert st["params"]["dense_width"] == (16384 if dtype == np.float64 else 32768)


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_dense_chunks_with_negative_zero_products(dtype):
    # Columns whose products are all -0.0 are still entries of C: the 16
    # heaviest rows get only -0.0 values (every column of their dense chunks
    # sums to -0.0), the next 300 heavy rows -0.0 on half of their entries
    # (some columns of a chunk do, the others do not).
    A = synth.rmat(15, 16, seed=12, dtype=dtype)
    P = oracle.row_products(A, A)
    order = np.argsort(-P, kind="stable")
    rp = A.row_ptr.astype(np.int64)
    rng = np.random.default_rng(5)
    val = A.val.copy()
    for i in order[:16]:
        val[rp[i]:rp[i + 1]] = -0.0
    for i in order[16:316]:
        seg = np.arange(rp[i], rp[i + 1])
        val[seg[rng.random(seg.size) < 0.5]] = -0.0
    A.val = val
    st = check_full(A, A, heavy_threshold=512)
    assert st["dense_chunks"] > 0
    hv = P > st["heavy_row_threshold"]
    assert hv[order[:316]].all()


def test_options_do_not_change_the_result():
    A = synth.rmat(11, 16, seed=3)
    A.val = np.round(A.val * 4 - 2)
    ref = gpu_product(A, A, heavy_threshold=64, dense_width=256, max_chunks_per_level=4)
    for opts in (dict(heavy_threshold=64, dense_width=256, max_chunks_per_level=4, single_stream=1),
                 dict(heavy_threshold=64, dense_width=256, max_chunks_per_level=4, rowptr64=1),
                 dict(heavy_threshold=100, dense_width=512, max_chunks_per_level=2),
                 dict(heavy_threshold=100, heavy_row_threshold=20, dense_width=512),
                 dict(heavy_row_threshold=1),
                 dict(heavy_threshold=64, dense_width=256, max_chunks_per_level=4, dense_direct=1),
                 dict(heavy_threshold=64, dense_width=256, max_chunks_per_level=4, dense_direct=1,
                      mem_budget=100_000),
                 dict()):
        rp, col, val, _ = gpu_product(A, A, **opts)
        np.testing.assert_array_equal(rp, ref[0])
        np.testing.assert_array_equal(col, ref[1])
        np.testing.assert_array_equal(val, ref[2])


@pytest.mark.parametrize("direct", [0, 1], ids=["expanded", "dense_direct"])
@pytest.mark.parametrize("budget", [1, 200_000])
def test_heavy_rows_in_batches(budget, direct):
    # A memory budget far below the intermediate's size splits the heavy rows
    # into batches (one row each at budget 1); symbolic counts every heavy
    # row's slots from A and B and expands the first batch, numeric expands
    # the others (with dense_direct: their light chunks only, the dense ones
    # from run lists).
    A = synth.rmat(11 if budget == 1 else 12, 16, seed=5)
    A.val = np.round(A.val * 6 - 3)
    opts = dict(heavy_threshold=64, dense_width=256, max_chunks_per_level=4, dense_direct=direct)
    st = check_full(A, A, exact=True, mem_budget=budget, **opts)
    assert st["batches"] > 1
    if budget == 1:
        assert st["batches"] == st["heavy_rows"]
    one = gpu_product(A, A, **opts)
    assert one[3]["batches"] == 1
    for a, b in zip(gpu_product(A, A, mem_budget=budget, **opts)[:3], one[:3]):
        np.testing.assert_array_equal(a, b)
    assert st["level_elems"] == one[3]["level_elems"]
    assert st["final_chunks"] == one[3]["final_chunks"]


def _light_chunk_edges(dtype):
    # Every row is heavy; its first-level chunks (2048 columns wide) are
    # light and hold exactly E elements, E around the sizes where the chunk
    # kernels change (32, 64, 128, 256 elements sorted in registers, larger
    # ones by the bitmap rank): B row k has column k mod 7 (chunk 0: E
    # elements over at most 7 columns, so long runs of equal columns are
    # summed) and column 2048 + k (chunk 1: E distinct columns).
    sizes = [1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 300]
    K = max(sizes)
    rp = np.zeros(len(sizes) + 1, np.int64)
    rp[1:] = np.cumsum(sizes)
    acol = np.concatenate([np.arange(e) for e in sizes]).astype(np.int32)
    rng = np.random.default_rng(5)
    aval = rng.integers(-3, 4, acol.size).astype(dtype)
    A = synth.CSR(rp.astype(np.int32), acol, aval, len(sizes), K)
    bcol = np.stack([np.arange(K) % 7, 2048 + np.arange(K)], axis=1).reshape(-1).astype(np.int32)
    bval = rng.integers(-3, 4, bcol.size).astype(dtype)
    B = synth.CSR((2 * np.arange(K + 1)).astype(np.int32), bcol, bval, K, 4096)
    A.check_canonical()
    B.check_canonical()
    return A, B


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_light_chunks_at_kernel_boundaries(dtype):
    A, B = _light_chunk_edges(dtype)
    st = check_full(A, B, exact=True, heavy_threshold=512, heavy_row_threshold=1, dense_width=256,
                    max_chunks_per_level=2)
    assert st["heavy_rows"] == A.m
    assert st["dense_chunks"] == 0


@pytest.mark.parametrize("W,nmax,budget", [(256, 4, 0), (128, 2, 0), (256, 32, 0), (256, 4, 150_000)])
def test_chunk_counts_from_structure_match_data_pass(W, nmax, budget):
    # The level histograms derived from A's structure and B's chunk runs must
    # be the integers the pass over the expanded columns counts: same chunk
    # tree (level sizes, final chunks) and the same product.
    A = synth.rmat(12, 16, seed=13)
    A.val = np.round(A.val * 6 - 3)
    opts = dict(heavy_threshold=40, dense_width=W, max_chunks_per_level=nmax, mem_budget=budget)
    a = gpu_product(A, A, histogram_from_data=1, **opts)
    b = gpu_product(A, A, **opts)
    for x, y in zip(a[:3], b[:3]):
        np.testing.assert_array_equal(x, y)
    for key in ("level_elems", "final_chunks", "dense_chunks"):
        assert a[3][key] == b[3][key], key
    # batch cuts follow the (unordered) heavy-row list, so only their presence
    assert (a[3]["batches"] > 1) == (b[3]["batches"] > 1) == (budget > 0)
    ref = oracle.spgemm(A, A)
    assert_csr_equal_structure(b[0], b[1], ref.row_ptr, ref.col, "C")
    np.testing.assert_array_equal(b[2], ref.val)


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
@pytest.mark.parametrize("W,nmax,budget", [(256, 4, 0), (256, 32, 0), (128, 2, 0), (256, 4, 150_000)])
def test_expansion_modes_agree(W, nmax, budget, dtype):
    # The one-pass run scatter (default), the page's outer product followed by
    # one multisplit pass per level, and the first level fed from A and B
    # must give the same chunk tree and the same C.
    A = synth.rmat(12, 16, seed=17)
    A.val = np.round(A.val * 6 - 3).astype(dtype)
    opts = dict(heavy_threshold=40, dense_width=W, max_chunks_per_level=nmax, mem_budget=budget)
    runs = {m: gpu_product(A, A, expansion=m, profile=1, **opts) for m in (0, 1, 2)}
    win = {m: r[3]["phase_windows"] for m, r in runs.items()}
    assert win[0]["expand_final"] > 0 and win[0]["outer_product"] == 0 and win[0]["multisplit"] == 0
    assert win[1]["outer_product"] > 0 and win[1]["expand_final"] == 0 and win[1]["expand_split"] == 0
    assert win[2]["expand_split"] > 0 and win[2]["outer_product"] == 0 and win[2]["expand_final"] == 0
    for m in (1, 2):
        for x, y in zip(runs[m][:3], runs[0][:3]):
            np.testing.assert_array_equal(x, y)
        for key in ("level_elems", "final_chunks", "dense_chunks"):
            assert runs[m][3][key] == runs[0][3][key], key
    ref = oracle.spgemm(A, A)
    assert_csr_equal_structure(runs[0][0], runs[0][1], ref.row_ptr, ref.col, "C")
    np.testing.assert_array_equal(runs[0][2], ref.val.astype(dtype))


def test_batches_fp32_multilevel():
    A = synth.rmat(12, 16, seed=8, dtype=np.float32)
    st = check_full(A, A, mem_budget=300_000, heavy_threshold=48, dense_width=256,
                    max_chunks_per_level=2)
    assert st["batches"] > 1 and st["params"]["levels"] == 4   # 4096 / 256 = 2^4


def test_validate_rejects_non_canonical():
    A = synth.random_csr(50, 50, 4.0, 1)
    bad = synth.CSR(A.row_ptr.copy(), A.col.copy(), A.val.copy(), 50, 50)
    r = int(np.nonzero(np.diff(bad.row_ptr) >= 2)[0][0])
    a = bad.row_ptr[r]
    bad.col[a], bad.col[a + 1] = bad.col[a + 1], bad.col[a]   # unsorted row, in range
    with pytest.raises(sg.SpgemmError) as e:
        gpu_product(bad, A, validate=1)
    assert e.value.status == -2
    check_full(A, A, exact=True, validate=1)


# ------------------------------------------------------------ full configs
def test_laplacian_config_exact():
    A = synth.workload("lap27_64")
    st = check_full(A, A, exact=True)
    assert st["products"] == 566 ** 3 and st["nnz_c"] == 314 ** 3 and st["heavy_rows"] == 0
    # every row's products span at most 2 * (2 + 2*64 + 2*4096) + 1 columns:
    # all of them take the dense window
    assert st["lds_dense_products"] == st["products"]


def _full_product(A, **opts):
    dA = sg.to_device(A)
    with sg.Plan(dA, dA, **opts) as p:
        rp, nnz = p.symbolic()
        col, val = p.numeric()
        st = p.stats()
    torch.cuda.synchronize()
    del dA
    return rp, col, val, nnz, st


def _check_every_row(A, rp, col, val, block_entries=1 << 30):
    """Every row of the GPU's C = A*A against the oracle, streamed to the
    host in row blocks of at most `block_entries` entries: row lengths and
    columns exactly, values to the stated relative tolerance of the sum of
    |terms|.  Returns the host row pointers."""
    rp_h = _to_np(rp, np.int64)
    assert rp_h[0] == 0 and np.all(np.diff(rp_h) >= 0)
    rtol = RTOL[A.val.dtype.type]
    r0, worst, terms, entries = 0, 0.0, 0, 0
    while r0 < A.m:
        r1 = int(np.searchsorted(rp_h, rp_h[r0] + block_entries, side="right")) - 1
        r1 = min(max(r1, r0 + 1), A.m)
        a, b = int(rp_h[r0]), int(rp_h[r1])
        gcol, gval = _to_np(col[a:b]), _to_np(val[a:b])
        rep = oracle.check_rows(A, A, r0, r1, rp_h[r0:r1 + 1], gcol, gval, rtol)
        print(f"rows [{r0}, {r1}) entries {b - a}: bad rows {rep.bad_rows} "
              f"(first {rep.first_bad_row}), bad values {rep.bad_values} "
              f"(first {rep.first_bad_value}), max rel {rep.max_rel:.3g}, "
              f"max terms {rep.max_terms}", flush=True)
        assert rep.ok, f"rows [{r0}, {r1}): {rep}"
        worst, terms, entries = max(worst, rep.max_rel), max(terms, rep.max_terms), entries + rep.entries
        del gcol, gval
        r0 = r1
    assert entries == rp_h[-1]
    print(f"all {A.m} rows, {entries} entries: max rel {worst:.3g}, max terms {terms}", flush=True)
    return rp_h


def test_rmat18_config_every_row():
    A = synth.workload("rmat18")
    P = oracle.row_products(A, A)
    rp, col, val, nnz, st = _full_product(A)
    assert st["params"]["tau"] == 6826 and st["heavy_row_threshold"] == 6826 // 3
    assert st["heavy_rows"] == int((P > 6826 // 3).sum()) and st["params"]["v_chunks"] == [16]
    assert st["lds_dense_products"] > 0
    rp_h = _check_every_row(A, rp, col, val)
    assert rp_h[-1] == nnz
    del rp, col, val
    torch.cuda.empty_cache()


def test_planted_partition_small_with_prune():
    A = synth.planted_partition(100, 500, 28, 4, seed=3)
    check_full(A, A)
    dA = sg.to_device(A)
    rp, col, val = sg.matmul(dA, dA)
    orp, ocol, oval = sg.prune_colnorm(rp, col, val, A.m, A.n, 1e-4)
    ref = oracle.spgemm(A, A)
    # keep decisions in fp32 (the value type); entries within 1e-5 relative of
    # the threshold may go either way, so adopt the GPU's decision there.
    ref32 = ref.val.astype(np.float32)
    band = np.abs(ref.val - 1e-4) <= 1e-5 * 1e-4
    gval = _to_np(val).astype(np.float64)
    keep = np.where(band, gval >= np.float32(1e-4), -1).astype(np.int8)
    erp, ecol, evals = oracle.prune_colnorm(A.m, A.n, ref.row_ptr, ref.col, ref.val, 1e-4, keep=keep)
    assert_csr_equal_structure(_to_np(orp, np.int64), _to_np(ocol), erp, ecol, "pruned")
    np.testing.assert_allclose(_to_np(oval).astype(np.float64), evals, rtol=1e-5, atol=0)
    # outside the band the keep decision is the oracle's fp32 comparison
    assert np.array_equal(keep[~band] == -1, np.ones((~band).sum(), bool))
    assert ecol.size == int(((ref32 >= np.float32(1e-4)) & ~band).sum() + (keep[band] == 1).sum())


def _random_csr(m, n, per_row, col_hi, seed, dtype):
    """m x n CSR, per_row distinct columns per row drawn from [0, col_hi),
    values multiples of 1/64 in (0, 1] (no value meets a threshold of 0.3)."""
    rng = np.random.default_rng(seed)
    cols = [np.sort(rng.choice(col_hi, per_row, replace=False)) for _ in range(m)]
    col = np.concatenate(cols).astype(np.int32)
    val = (rng.integers(1, 65, col.size) / 64.0).astype(dtype)
    rp = np.arange(0, m * per_row + 1, per_row, dtype=np.int32)
    return synth.CSR(rp, col, val, m, n)


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
@pytest.mark.parametrize("case", ["one_bucket", "scattered"])
def test_prune_column_sums_past_their_buckets(case, dtype):
    # The prune's column sums go through column buckets sized for nnz(C)
    # spread evenly; entries that do not fit fall back to global adds.
    # one_bucket: every column lies in the first of four buckets, so three
    # quarters of its entries overflow.  scattered: a work group's 40 rows
    # hold 32,000 nearly distinct columns, past its LDS table and its list.
    if case == "one_bucket":
        C = _random_csr(3000, 8192, 50, 2048, 7, dtype)
    else:
        C = _random_csr(400, 200_000, 800, 200_000, 8, dtype)
    dC = sg.to_device(C)
    orp, ocol, oval = sg.prune_colnorm(dC.row_ptr, dC.col, dC.val, C.m, C.n, 0.3)
    erp, ecol, evals = oracle.prune_colnorm(C.m, C.n, C.row_ptr, C.col, C.val.astype(np.float64), 0.3)
    assert_csr_equal_structure(_to_np(orp, np.int64), _to_np(ocol), erp, ecol, "pruned")
    np.testing.assert_allclose(_to_np(oval).astype(np.float64), evals,
                               rtol=1e-5 if dtype == np.float32 else 1e-12, atol=0)


def _check_mcl_inflate(rp, col, val, m, n, thr, dtype):
    """GPU MCL inflation of C (device CSR) against the oracle on the same C;
    normalised values within 1e-6 relative of the threshold may go either
    way, so the GPU's decision is adopted there.  Returns the GPU result."""
    orp, ocol, oval = sg.mcl_inflate(rp, col, val, m, n, thr)
    crp, ccol = _to_np(rp, np.int64), _to_np(col)
    cval = _to_np(val).astype(np.float64)
    s = np.zeros(n)
    np.add.at(s, ccol, cval)
    y = np.where(s[ccol] != 0, cval / np.where(s[ccol] != 0, s[ccol], 1), 0.0)
    band = np.abs(y - thr) <= 1e-6 * thr
    grows = np.repeat(np.arange(m), np.diff(_to_np(orp, np.int64)))
    gkept = set(zip(grows.tolist(), _to_np(ocol).tolist()))
    crows = np.repeat(np.arange(m), np.diff(crp))
    keep = np.full(ccol.size, -1, np.int8)
    for e in np.nonzero(band)[0]:
        keep[e] = 1 if (int(crows[e]), int(ccol[e])) in gkept else 0
    erp, ecol, evals = oracle.mcl_inflate(m, n, crp, ccol, cval, thr,
                                          single=dtype == np.float32, keep=keep)
    assert_csr_equal_structure(_to_np(orp, np.int64), _to_np(ocol), erp, ecol, "mcl inflation")
    np.testing.assert_allclose(_to_np(oval).astype(np.float64), evals,
                               rtol=1e-5 if dtype == np.float32 else 1e-12, atol=0)
    return orp, ocol, oval


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_mcl_inflate_matches_oracle(dtype):
    A = synth.planted_partition(40, 200, 28, 4, seed=5, dtype=dtype)
    dA = sg.to_device(A)
    rp, col, val = sg.matmul(dA, dA)
    _check_mcl_inflate(rp, col, val, A.m, A.n, 0.002, dtype)
    # a threshold below every value keeps the whole structure
    orp, ocol, _ = sg.mcl_inflate(rp, col, val, A.m, A.n, 0.0)
    np.testing.assert_array_equal(_to_np(orp, np.int64), _to_np(rp, np.int64))
    np.testing.assert_array_equal(_to_np(ocol), _to_np(col))


def test_mcl_iterations_step_by_step():
    # Markov clustering as on the Trident page (10 iterations, threshold
    # 0.002), each step checked against the oracle on the GPU's own input:
    # the expansion against the oracle's product, the inflation against the
    # oracle's inflation of the GPU's C.
    A = synth.planted_partition(30, 150, 28, 4, seed=7)
    X = sg.to_device(A)
    Xh = A
    for it in range(10):
        st = check_full(Xh, Xh, rowptr64=1)
        rp, col, val = sg.matmul(X, X, rowptr64=1)
        orp, ocol, oval = _check_mcl_inflate(rp, col, val, A.m, A.n, 0.002, np.float32)
        orp = orp.to(torch.int32)
        X = sg.CsrDevice(orp, ocol, oval, A.m, A.n)
        Xh = synth.CSR(_to_np(orp, np.int32), _to_np(ocol), _to_np(oval), A.m, A.n)
    # the loop in the binding gives the same clustering (LDS atomics may add
    # in another order, so a value that lands on the threshold could flip)
    Y, products = sg.mcl(sg.to_device(A), iterations=10, threshold=0.002)
    assert len(products) == 10
    def entries(Z):
        r = np.repeat(np.arange(A.m), np.diff(_to_np(Z.row_ptr, np.int64)))
        return dict(zip(zip(r.tolist(), _to_np(Z.col).tolist()), _to_np(Z.val).tolist()))
    ey, ex = entries(Y), entries(X)
    assert len(set(ey) ^ set(ex)) <= max(1, len(ex) // 1000)
    common = sorted(set(ey) & set(ex))
    np.testing.assert_allclose([ey[k] for k in common], [ex[k] for k in common], rtol=1e-4)


def test_mcl_config_every_row_and_prune():
    # C = A*A for the 10^6-column planted partition, every row against the
    # oracle; then the prune and column renormalisation of the whole C against
    # the oracle's, with the GPU's keep decision adopted only for entries
    # within 1e-5 relative of the threshold.
    A = synth.workload("mcl1m")
    rp, col, val, nnz, st = _full_product(A)
    assert st["heavy_rows"] == 0
    _check_every_row(A, rp, col, val)
    orp, ocol, oval = sg.prune_colnorm(rp, col, val, A.m, A.n, 1e-4)
    torch.cuda.synchronize()
    gval = _to_np(val).astype(np.float64)
    del col, val
    torch.cuda.empty_cache()
    ref = oracle.spgemm(A, A)
    np.testing.assert_array_equal(_to_np(rp, np.int64), ref.row_ptr)
    band = np.abs(ref.val - 1e-4) <= 1e-5 * 1e-4
    keep = np.full(ref.val.size, -1, np.int8)
    keep[band] = gval[band] >= np.float32(1e-4)
    print(f"entries within the tie band: {int(band.sum())}", flush=True)
    erp, ecol, evals = oracle.prune_colnorm(A.m, A.n, ref.row_ptr, ref.col, ref.val, 1e-4,
                                            keep=keep)
    del ref, gval, keep
    assert_csr_equal_structure(_to_np(orp, np.int64), _to_np(ocol), erp, ecol, "pruned")
    g = _to_np(oval).astype(np.float64)
    np.testing.assert_allclose(g, evals, rtol=1e-5, atol=0)
    print(f"pruned: {ecol.size} of {int(nnz)} entries kept, max rel "
          f"{float(np.max(np.abs(g - evals) / evals)):.3g}", flush=True)
    del rp, orp, ocol, oval
    torch.cuda.empty_cache()


def test_rmat20_config_every_row_batched_rowptr64():
    A = synth.workload("rmat20")
    P = oracle.row_products(A, A)
    torch.cuda.empty_cache()
    rp, col, val, nnz, st = _full_product(A, rowptr64=1)
    assert st["params"]["v_chunks"] == [32, 2] and st["params"]["levels"] == 2
    hv = P > st["heavy_row_threshold"]
    assert st["heavy_rows"] == int(hv.sum()) and st["heavy_products"] == int(P[hv].sum())
    assert st["batches"] > 1 and nnz > 2 ** 31
    rp_h = _check_every_row(A, rp, col, val)
    assert rp_h[-1] == nnz
    del rp, col, val
    torch.cuda.empty_cache()
