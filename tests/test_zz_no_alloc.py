"""spgemm_transpose_noalloc: the transpose whose temporaries live in the
library's fixed device scratch array, through the C ABI, against the
allocating spgemm_transpose (bit for bit: it is index work) and the oracle's
transpose, on calls in a row whose second input is smaller, and its
rejection of inputs whose temporaries exceed the array."""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
sg = pytest.importorskip("spgemm_symbolic_row_amd")


def _host(T):
    torch.cuda.synchronize()
    return (T.row_ptr.cpu().numpy().astype(np.int64), T.col.cpu().numpy(),
            None if T.val is None else T.val.cpu().numpy())


def _same(A, dA, **kw):
    print(f"transpose {A.m} x {A.n}, nnz {A.nnz}, {A.val.dtype}, {kw}", flush=True)
    ref = _host(sg.transpose(dA, **kw))
    got = _host(sg.transpose(dA, no_alloc=True, **kw))
    for x, y in zip(got, ref):
        if y is None:
            assert x is None
        else:
            assert x.dtype == y.dtype and np.array_equal(x.view(np.uint8), y.view(np.uint8))
    T = oracle.transpose(A)
    assert np.array_equal(got[0], T.row_ptr) and np.array_equal(got[1], T.col)
    if got[2] is not None:
        assert np.array_equal(got[2], T.val)
    return got


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_noalloc_transpose_matches_the_allocating_one(dtype):
    # A larger input with three digit passes, then a smaller one with one,
    # then a middle one: each call reuses the scratch the previous one left.
    big = synth.sparse_uniform(4000, 1 << 21, 150.0, seed=11, dtype=dtype)
    small = synth.sparse_uniform(700, 900, 5.0, seed=12, dtype=dtype)
    mid = synth.sparse_uniform(3000, 50000, 20.0, seed=13, dtype=dtype)
    for A, kw in ((big, {}), (small, {}), (mid, {"out_rowptr64": True}),
                  (small, {"pattern_only": True}), (big, {})):
        _same(A, sg.to_device(A), **kw)


def test_noalloc_transpose_degenerate_shapes():
    for A in (synth.CSR(np.zeros(1, np.int32), np.zeros(0, np.int32), np.zeros(0), 0, 5),
              synth.CSR(np.zeros(6, np.int32), np.zeros(0, np.int32), np.zeros(0), 5, 0),
              synth.CSR(np.array([0, 1], np.int32), np.array([3], np.int32),
                        np.array([2.5]), 1, 4)):
        _same(A, sg.to_device(A))


def test_noalloc_transpose_rejects_inputs_beyond_the_scratch():
    # fp64 with three digit passes takes about 32 bytes of temporaries per
    # entry; 2.5 million entries exceed the 64 MiB array.
    A = synth.sparse_uniform(2500, 1 << 21, 1000.0, seed=14)
    assert A.nnz > 2_400_000
    dA = sg.to_device(A)
    with pytest.raises(sg.SpgemmError) as e:
        sg.transpose(dA, no_alloc=True)
    assert e.value.status == -1 and "64 MiB" in str(e.value)
    # the allocating entry point still takes it, and a smaller call after
    # the rejection works
    sg.transpose(dA)
    small = synth.sparse_uniform(300, 400, 4.0, seed=15)
    _same(small, sg.to_device(small))
