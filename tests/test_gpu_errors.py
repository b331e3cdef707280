"""Failure handling through the C ABI, every condition forced from the host:
an allocator callback that returns NULL, calls out of order, a lowered index
limit, and the device status word set through the test hook.  No kernel is
made to fault; every product here is small and valid.

The pages report out-of-memory, illegal-access and time-out failures of
other libraries (gMAGNUS page, §IV-A/§IV-B; Ocean page, evaluation); the
library's contract is a status code with C left untouched where stated.
"""
import ctypes

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
sg = pytest.importorskip("spgemm_symbolic_row_amd")

ALLOC = ctypes.CFUNCTYPE(ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p)
FREE = ctypes.CFUNCTYPE(None, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p)

OK, INVALID_ARG, INDEX_OVERFLOW, OOM, STATE, INTERNAL = 0, -1, -3, -4, -6, -7


class FailingAllocator:
    """Device memory from torch for the first `budget` requests, NULL after.
    Freed blocks are kept until release(), after a device synchronisation,
    so no block is reused while the library's streams may still read it."""

    def __init__(self, budget):
        self.budget, self.calls = budget, 0
        self.live, self.dead = {}, []
        self.c_alloc, self.c_free = ALLOC(self._alloc), FREE(self._free)

    def _alloc(self, nbytes, stream, ctx):
        self.calls += 1
        if self.calls > self.budget:
            return None
        t = torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device="cuda")
        self.live[t.data_ptr()] = t
        return t.data_ptr()

    def _free(self, ptr, stream, ctx):
        t = self.live.pop(ptr, None)
        if t is not None:
            self.dead.append(t)

    def options(self):
        return dict(alloc=ctypes.cast(self.c_alloc, ctypes.c_void_p).value,
                    free=ctypes.cast(self.c_free, ctypes.c_void_p).value)

    def release(self):
        torch.cuda.synchronize()
        self.dead.clear()
        assert not self.live, f"{len(self.live)} blocks never freed"


def _sentinel_outputs(m, nnz_guess, dtype, rp64=False):
    rp = torch.full((m + 1,), -7, dtype=torch.int64 if rp64 else torch.int32, device="cuda")
    col = torch.full((max(nnz_guess, 1),), -7, dtype=torch.int32, device="cuda")
    val = torch.full((max(nnz_guess, 1),), 12345.0, dtype=dtype, device="cuda")
    return rp, col, val


def _untouched(rp, col, val):
    torch.cuda.synchronize()
    return (bool((rp == -7).all()) and bool((col == -7).all())
            and bool((val == 12345.0).all()))


def _attempt(dA, budget, nnz, **opts):
    """plan -> symbolic -> numeric with an allocator that fails after
    `budget` requests; returns (stage reached or failed, status, allocator,
    outputs)."""
    fa = FailingAllocator(budget)
    rp, col, val = _sentinel_outputs(dA.m, nnz, dA.val.dtype)
    stage, status, msg = "done", OK, ""
    p = None
    try:
        stage = "plan"
        p = sg.Plan(dA, dA, **fa.options(), **opts)
        stage = "symbolic"
        p.symbolic(rp)
        stage = "numeric"
        p.numeric(col[:p.nnz], val[:p.nnz])
        stage = "wait"
        p.wait()
        stage = "done"
    except sg.SpgemmError as e:
        status, msg = e.status, str(e)
    finally:
        if p is not None:
            p.destroy()
        fa.release()
    if status != OK:
        print(f"  allocator budget {budget}: {stage} failed: {msg} (after {fa.calls} requests)",
              flush=True)
    return stage, status, fa, (rp, col, val)


@pytest.mark.parametrize("opts", [
    dict(heavy_threshold=64, dense_width=256, max_chunks_per_level=4),
    dict(heavy_threshold=64, dense_width=256, max_chunks_per_level=4, mem_budget=-3),
    dict(workflow=1),
], ids=["kept", "batched", "upper_bound"])
def test_failing_allocator_gives_oom_and_leaves_c_untouched(opts):
    A = synth.rmat(11, 16, seed=4)
    dA = sg.to_device(A)
    ref = oracle.spgemm(A, A)
    nnz = int(ref.row_ptr[-1])
    opts = dict(opts)
    if opts.get("mem_budget") == -3:
        # about three heavy-row batches: a third of the two-buffer intermediate
        st = sg.matmul(dA, dA, with_stats=True, **{k: v for k, v in opts.items()
                                                   if k != "mem_budget"})[3]
        opts["mem_budget"] = st["heavy_products"] * 2 * 12 // 3
    stage, status, fa, (rp, col, val) = _attempt(dA, 10 ** 9, nnz, **opts)
    assert stage == "done" and status == OK, (stage, status)
    n_alloc = fa.calls
    assert n_alloc > 5
    np.testing.assert_array_equal(rp.cpu().numpy().astype(np.int64), ref.row_ptr)
    np.testing.assert_array_equal(col[:nnz].cpu().numpy(), ref.col)
    batched = "mem_budget" in opts
    seen = set()
    # every allocation index when there are few, else 120 spread over them
    budgets = range(n_alloc) if n_alloc <= 120 else \
        sorted(set(np.linspace(0, n_alloc - 1, 120).astype(int).tolist()))
    print(f"{n_alloc} allocations in a full product; failing at {len(budgets)} of them",
          flush=True)
    for budget in budgets:
        stage, status, fa, out = _attempt(dA, budget, nnz, **opts)
        print(f"fail at allocation {budget}: stage {stage}, status {status}", flush=True)
        assert status == OOM, (budget, stage, status)
        seen.add(stage)
        if stage in ("plan", "symbolic"):
            assert _untouched(*out), (budget, stage)
        else:
            # only the batched schedule allocates in numeric
            assert stage == "numeric" and batched, (budget, stage)
            got = out[0].cpu().numpy().astype(np.int64)
            np.testing.assert_array_equal(got, ref.row_ptr)   # C.row_ptr stays valid
    assert "plan" in seen and "symbolic" in seen
    assert ("numeric" in seen) == batched


def test_call_order_is_enforced():
    A = synth.random_csr(200, 200, 5.0, 3, values="int")
    dA = sg.to_device(A)
    col0 = torch.empty(1, dtype=torch.int32, device="cuda")
    val0 = torch.empty(1, dtype=torch.float64, device="cuda")
    p = sg.Plan(dA, dA)
    try:
        with pytest.raises(sg.SpgemmError) as e:
            p.numeric(col0, val0)            # numeric before symbolic
        assert e.value.status == STATE
        rp, nnz = p.symbolic()
        with pytest.raises(sg.SpgemmError) as e:
            p.symbolic()                     # symbolic twice
        assert e.value.status == STATE
        col, val = p.numeric()
        with pytest.raises(sg.SpgemmError) as e:
            p.numeric(col, val)              # numeric twice
        assert e.value.status == STATE
        p.wait()
    finally:
        p.destroy()
    ref = oracle.spgemm(A, A)
    np.testing.assert_array_equal(col.cpu().numpy(), ref.col)
    # after a failed call the plan is in the error state
    nnz = int(ref.row_ptr[-1])
    p = sg.Plan(dA, dA, index_limit=nnz - 1)
    try:
        with pytest.raises(sg.SpgemmError) as e:
            p.symbolic()
        assert e.value.status == INDEX_OVERFLOW
        with pytest.raises(sg.SpgemmError) as e:
            p.numeric(col, val)
        assert e.value.status == STATE
    finally:
        p.destroy()


def test_index_limit_overflow():
    A = synth.rmat(10, 16, seed=2)
    dA = sg.to_device(A)
    ref = oracle.spgemm(A, A)
    nnz = int(ref.row_ptr[-1])
    P = oracle.row_products(A, A)
    # int32 C.row_ptr: nnz(C) one above the limit is rejected, C.row_ptr untouched
    rp, _, _ = _sentinel_outputs(A.m, 1, torch.float64)
    with sg.Plan(dA, dA, index_limit=nnz - 1) as p:
        with pytest.raises(sg.SpgemmError) as e:
            p.symbolic(rp)
        assert e.value.status == INDEX_OVERFLOW
    torch.cuda.synchronize()
    assert bool((rp == -7).all())
    # at the limit, or with int64 row pointers, the product goes through
    for opts in (dict(index_limit=nnz), dict(index_limit=nnz - 1, rowptr64=1)):
        with sg.Plan(dA, dA, **opts) as p:
            r, n = p.symbolic()
            c, v = p.numeric()
        assert n == nnz
        np.testing.assert_array_equal(c.cpu().numpy(), ref.col)
    # a row with more products than the limit is rejected by the plan
    with pytest.raises(sg.SpgemmError) as e:
        sg.Plan(dA, dA, index_limit=int(P.max()) - 1, rowptr64=1)
    assert e.value.status == INDEX_OVERFLOW
    sg.Plan(dA, dA, index_limit=int(P.max()), rowptr64=1).destroy()
    with pytest.raises(sg.SpgemmError) as e:
        sg.Plan(dA, dA, index_limit=-1)
    assert e.value.status == INVALID_ARG


def test_device_status_surfaces_without_stats():
    # The numeric phase is asynchronous: a tripped device check (here the
    # size-mismatch bit, stored by the test hook) must be reported by the
    # binding's own products and by spgemm_wait, without reading stats.
    A = synth.rmat(10, 16, seed=6)
    dA = sg.to_device(A)
    with pytest.raises(sg.SpgemmError) as e:
        sg.matmul(dA, dA, debug_device_error=8)
    assert e.value.status == INTERNAL and "disagree" in str(e.value)
    p = sg.Plan(dA, dA, debug_device_error=8, heavy_threshold=64, dense_width=256)
    try:
        p.symbolic()
        p.numeric()                          # returns: the check runs on the device
        with pytest.raises(sg.SpgemmError) as e:
            p.wait()
        assert e.value.status == INTERNAL
    finally:
        p.destroy()
    # spgemm_get_stats reports it too (on a plan that was not waited on)
    p = sg.Plan(dA, dA, debug_device_error=8)
    try:
        p.symbolic()
        p.numeric()
        with pytest.raises(sg.SpgemmError) as e:
            p.stats()
        assert e.value.status == INTERNAL
    finally:
        p.destroy()
    # the same product without the hook is clean
    rp, col, val = sg.matmul(dA, dA)
    ref = oracle.spgemm(A, A)
    np.testing.assert_array_equal(col.cpu().numpy(), ref.col)
