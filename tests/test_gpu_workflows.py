"""GPU parity of the size-prediction workflows for light rows (Ocean page,
§3 and Table 1): upper bound (1), HyperLogLog estimate (2) and the automatic
choice (3).

C must match the oracle exactly in structure and within the usual value
tolerance in every workflow.  The integer steps are compared exactly with the
oracle: reserved slots (P_i, or min(P_i, ceil(coef * E_i))), the HyperLogLog
estimates themselves (sums of powers of two and one division: exact in
fp64), the number of rows that did not fit, and the workflow chosen.
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


def _run(A, B, exact=False, **opts):
    print(f"workflow {opts} m={A.m} k={A.n} n={B.n} {A.val.dtype}", flush=True)
    dA = sg.to_device(A)
    dB = dA if B is A else sg.to_device(B)
    with sg.Plan(dA, dB, **opts) as p:
        rp, _ = p.symbolic()
        st0 = p.stats()
        cap = est = None
        if st0["workflow"] != 0:
            cap, est = p.row_estimates(with_estimates=st0["workflow"] == 2)
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
    assert st["device_errors"] == 0
    return st, ref, (None if cap is None else _np(cap)), (None if est is None else _np(est))


def _light(A, B, st):
    P = oracle.row_products(A, B)
    return P, (P > 0) & (P <= st["heavy_row_threshold"])


CASES = {
    "int_small": lambda: (synth.random_csr(300, 200, 6.0, 1, values="int", empty_row_frac=0.2),
                          synth.random_csr(200, 400, 5.0, 2, values="int", empty_row_frac=0.2)),
    "rmat12": lambda: (synth.rmat(12, 8, seed=3),) * 2,
    "lap16": lambda: (synth.laplacian27(16),) * 2,
    "er4096": lambda: (synth.workload("er4096"),) * 2,
    "rect_fp32": lambda: (synth.random_csr(500, 300, 8.0, 4, values="uniform", dtype=np.float32),
                          synth.random_csr(300, 2000, 12.0, 5, values="uniform",
                                           dtype=np.float32)),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_upper_bound_workflow(case):
    A, B = CASES[case]()
    st, ref, cap, _ = _run(A, B, exact=(case in ("int_small", "lap16")), workflow=1)
    assert st["workflow"] == 1 and st["overflow_rows"] == 0
    P, light = _light(A, B, st)
    np.testing.assert_array_equal(cap, np.where(light, P, 0))
    assert st["light_capacity"] == int(P[light].sum())


@pytest.mark.parametrize("M", [32, 64])
@pytest.mark.parametrize("case", sorted(CASES))
def test_hll_workflow_estimates_exact(case, M):
    A, B = CASES[case]()
    st, ref, cap, est = _run(A, B, exact=(case in ("int_small", "lap16")), workflow=2,
                             hll_registers=M)
    assert st["workflow"] == 2 and st["hll_registers"] == M
    P, light = _light(A, B, st)
    e_ref = oracle.hll_estimate(A, B, M)
    np.testing.assert_array_equal(est[light], e_ref[light])
    assert np.all(est[~light] == 0)
    c_ref = oracle.capacity(P, e_ref, oracle.hll_coefficient(M))
    np.testing.assert_array_equal(cap, np.where(light, c_ref, 0))
    nnz = np.diff(ref.row_ptr)
    assert st["overflow_rows"] == int(np.sum(light & (nnz > c_ref)))


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_hll_overflow_rows_recomputed(dtype):
    # A quarter of the estimate: most rows do not fit and are computed again
    # with P_i slots; C is unchanged.
    A = synth.rmat(12, 8, seed=6, dtype=dtype)
    st, ref, cap, est = _run(A, A, workflow=2, hll_registers=64, hll_coef_pct=25)
    P, light = _light(A, A, st)
    c_ref = oracle.capacity(P, oracle.hll_estimate(A, A, 64), 0.25)
    nnz = np.diff(ref.row_ptr)
    want = int(np.sum(light & (nnz > c_ref)))
    assert want > 100
    assert st["overflow_rows"] == want


def test_workflows_with_heavy_rows():
    # Heavy rows keep the exact chunk path in every workflow.
    A = synth.rmat(12, 16, seed=7)
    A.val = np.round(A.val * 6 - 3)
    for wf in (1, 2):
        st, *_ = _run(A, A, exact=True, workflow=wf, heavy_threshold=256, dense_width=512,
                      max_chunks_per_level=4)
        assert st["heavy_rows"] > 0 and st["workflow"] == wf


def _oracle_choice(A, B, heavy_threshold):
    # Heavy rows (more than heavy_threshold products) keep the exact chunk
    # path and are left out of the sampled compression ratio.
    P = oracle.row_products(A, B)
    total = int(P.sum())
    cr = None
    if total >= 64 * A.m and total >= 8 * A.col.shape[0]:
        M = oracle.hll_registers(total, A.col.shape[0])
        rows = [int(r) for r in oracle.sample_rows(A.m) if P[r] <= heavy_threshold]
        e = np.concatenate([oracle.hll_estimate(A, B, M, r, r + 1) for r in rows])
        cr = float(P[rows].sum()) / float(e.sum())
    return oracle.select_workflow(A.m, A.col.shape[0], total, cr), cr


def _narrow(m, k, per_row, width, seed):
    """B whose rows all fall in one narrow column window: high compression."""
    rng = np.random.default_rng(seed)
    rows = [np.sort(rng.choice(width, size=per_row, replace=False)) for _ in range(k)]
    rp = np.arange(0, k * per_row + 1, per_row, dtype=np.int32)
    return synth.CSR(rp, np.concatenate(rows).astype(np.int32),
                     rng.uniform(-1, 1, k * per_row), k, m)


@pytest.mark.parametrize("case", ["er", "narrow", "rmat", "rmat_heavy"])
def test_auto_selection_follows_table_1(case):
    if case == "er":          # about 64 products per row or fewer: upper bound
        A = synth.erdos_renyi(2048, 6.0, seed=1)
        B = A
    elif case == "narrow":    # expansion 64, compression about 16: estimate
        A = synth.random_csr(3000, 2000, 16.0, 2, values="uniform")
        B = _narrow(4000, 2000, 64, 96, 3)
    else:                      # compression below 8: symbolic
        A = synth.rmat(12, 16, seed=8)
        B = A
    opts = {"heavy_threshold": 256} if case == "rmat_heavy" else {}
    st, *_ = _run(A, B, workflow=3, **opts)
    want, cr = _oracle_choice(A, B, st["heavy_row_threshold"])
    assert st["workflow"] == want
    if cr is not None:
        assert abs(st["sampled_cr"] - cr) <= 1e-12 * cr
    assert want == {"er": 1, "narrow": 2, "rmat": 0, "rmat_heavy": 0}[case]


def test_row_estimates_errors():
    A = synth.random_csr(50, 50, 3.0, 9, values="uniform")
    dA = sg.to_device(A)
    with sg.Plan(dA, dA) as p:
        with pytest.raises(sg.SpgemmError):      # before symbolic
            p.row_estimates()
        p.symbolic()
        with pytest.raises(sg.SpgemmError):      # workflow 0 has none
            p.row_estimates()
        p.numeric()
    with sg.Plan(dA, dA, workflow=1) as p:
        p.symbolic()
        with pytest.raises(sg.SpgemmError):      # estimates need workflow 2
            p.row_estimates(with_estimates=True)
        cap, _ = p.row_estimates(with_estimates=False)
        p.numeric()
    with pytest.raises(sg.SpgemmError):
        sg.Plan(dA, dA, workflow=4)
    with pytest.raises(sg.SpgemmError):
        sg.Plan(dA, dA, hll_registers=16)
    torch.cuda.synchronize()
