"""Python binding of libspgemm.so: sparse C = A*B (CSR) on one MI355X.

Argument marshalling only: every step of the product runs in the HIP
library.  PyTorch supplies device memory and the current stream.  There is
no CPU fallback; without the built library every call raises.

    import spgemm_symbolic_row_amd as sg
    rp, col, val = sg.matmul(A, B)          # A, B: CsrDevice or torch sparse CSR
    stats = sg.last_stats()

The underlying C entry points (include/spgemm.h) are exposed with the same
names through `lib()`.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

__all__ = [
    "lib", "Options", "Params", "Stats", "CsrDevice", "Plan", "matmul", "compute_params",
    "prune_colnorm", "SpgemmError", "to_device", "last_stats",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspgemm.so")

c_i64, c_i32, c_vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p


class Options(ctypes.Structure):
    _fields_ = [
        ("lds_budget", c_i64), ("heavy_threshold", c_i64), ("dense_width", c_i64),
        ("mem_budget", c_i64), ("max_chunks_per_level", c_i32), ("rowptr64", c_i32),
        ("validate", c_i32), ("single_stream", c_i32), ("profile", c_i32),
        ("histogram_from_data", c_i32), ("alloc", c_vp), ("free", c_vp),
        ("alloc_ctx", c_vp), ("expansion", c_i32), ("heavy_row_threshold", c_i32),
        ("light_hash_only", c_i32), ("workflow", c_i32), ("hll_registers", c_i32),
        ("hll_coef_pct", c_i32), ("light_no_esc", c_i32), ("index_limit", c_i64),
        ("debug_device_error", c_i64), ("dense_direct", c_i64), ("reserved", c_i64 * 1),
    ]


class Params(ctypes.Structure):
    _fields_ = [
        ("tau", c_i64), ("n_dense", c_i64), ("dense_width", c_i64), ("chunks_required", c_i64),
        ("chunks_max", c_i32), ("levels", c_i32), ("v_chunks", c_i32 * 8),
        ("level_width", c_i64 * 8),
    ]

    def as_dict(self):
        L = self.levels
        return {"tau": self.tau, "n_dense": self.n_dense, "dense_width": self.dense_width,
                "chunks_required": self.chunks_required, "chunks_max": self.chunks_max,
                "levels": L, "v_chunks": list(self.v_chunks[:L]),
                "level_width": list(self.level_width[:L])}


class Stats(ctypes.Structure):
    _fields_ = [
        ("products", c_i64), ("max_row_products", c_i64), ("light_rows", c_i64),
        ("heavy_rows", c_i64), ("heavy_products", c_i64), ("heavy_a_nnz", c_i64),
        ("nnz_c", c_i64), ("params", Params), ("level_elems", c_i64 * 8),
        ("final_chunks", c_i64), ("dense_chunks", c_i64), ("lds_hash_products", c_i64),
        ("lds_dense_products", c_i64), ("global_products", c_i64), ("batches", c_i64),
        ("ms_plan", ctypes.c_double), ("ms_symbolic", ctypes.c_double),
        ("ms_numeric", ctypes.c_double), ("phase_ms", ctypes.c_double * 16),
        ("phase_windows", c_i32 * 16), ("device_errors", c_i64),
        ("heavy_row_threshold", c_i64), ("chunk_col_bytes", c_i64),
        ("workflow", c_i32), ("hll_registers", c_i32), ("light_capacity", c_i64),
        ("overflow_rows", c_i64), ("sampled_cr", ctypes.c_double),
        ("phase_min_ms", ctypes.c_double * 16), ("hybrid_rows", c_i64),
    ]

    def as_dict(self):
        d = {name: getattr(self, name) for name, _ in self._fields_
             if name not in ("params", "level_elems", "phase_ms", "phase_windows",
                             "phase_min_ms")}
        d["params"] = self.params.as_dict()
        d["level_elems"] = list(self.level_elems[:self.params.levels])
        d["phase_ms"] = {PHASES[i]: self.phase_ms[i] for i in range(len(PHASES))}
        d["phase_windows"] = {PHASES[i]: self.phase_windows[i] for i in range(len(PHASES))}
        d["phase_min_ms"] = {PHASES[i]: self.phase_min_ms[i] for i in range(len(PHASES))}
        return d


PHASES = ["row_info", "sym_light", "csc", "outer_product", "histogram", "multisplit",
          "sym_chunk_hash", "sym_chunk_dense", "rowptr", "num_light", "num_chunk_hash",
          "num_chunk_dense", "chunk_hist", "expand_split", "expand_final", "sym_heavy"]


SPGEMM_F32, SPGEMM_F64 = 0, 1
_lib = None


class SpgemmError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{msg} (status {status})")
        self.status = status


def lib():
    """The loaded libspgemm.so (ctypes), with argument types declared."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m spgemm_symbolic_row_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        st = ctypes.c_int
        L.spgemm_compute_params.restype = st
        L.spgemm_compute_params.argtypes = [c_i64, c_i64, c_i32, c_i32, c_i32, c_i64,
                                            ctypes.POINTER(Params)]
        L.spgemm_plan.restype = st
        L.spgemm_plan.argtypes = [ctypes.POINTER(c_vp), c_i64, c_i64, c_i64, c_vp, c_vp, c_vp,
                                  c_i64, c_vp, c_vp, c_vp, c_i64, ctypes.c_int,
                                  ctypes.POINTER(Options), c_vp]
        L.spgemm_symbolic.restype = st
        L.spgemm_symbolic.argtypes = [c_vp, c_vp, ctypes.POINTER(c_i64)]
        L.spgemm_numeric.restype = st
        L.spgemm_numeric.argtypes = [c_vp, c_vp, c_vp]
        L.spgemm_wait.restype = st
        L.spgemm_wait.argtypes = [c_vp]
        L.spgemm_get_stats.restype = st
        L.spgemm_get_stats.argtypes = [c_vp, ctypes.POINTER(Stats)]
        L.spgemm_destroy.restype = None
        L.spgemm_destroy.argtypes = [c_vp]
        L.spgemm_status_string.restype = ctypes.c_char_p
        L.spgemm_status_string.argtypes = [ctypes.c_int]
        L.spgemm_last_error.restype = ctypes.c_char_p
        L.spgemm_last_error.argtypes = [c_vp]
        L.spgemm_prune_colnorm_count.restype = st
        L.spgemm_prune_colnorm_count.argtypes = [ctypes.POINTER(c_vp), c_i64, c_i64, c_vp, c_i32,
                                                 c_vp, c_vp, ctypes.c_int, ctypes.c_double, c_vp,
                                                 c_i32, ctypes.POINTER(c_i64), c_vp]
        L.spgemm_prune_colnorm_fill.restype = st
        L.spgemm_prune_colnorm_fill.argtypes = [c_vp, c_vp, c_vp]
        L.spgemm_mcl_inflate_count.restype = st
        L.spgemm_mcl_inflate_count.argtypes = L.spgemm_prune_colnorm_count.argtypes
        L.spgemm_mcl_inflate_fill.restype = st
        L.spgemm_mcl_inflate_fill.argtypes = [c_vp, c_vp, c_vp]
        L.spgemm_prune_destroy.restype = None
        L.spgemm_prune_destroy.argtypes = [c_vp]
        L.spgemm_row_estimates.restype = st
        L.spgemm_row_estimates.argtypes = [c_vp, c_vp, c_vp]
        L.spgemm_transpose.restype = st
        L.spgemm_transpose.argtypes = [c_i64, c_i64, c_i64, c_vp, c_i32, c_vp, c_vp, ctypes.c_int,
                                       c_vp, c_i32, c_vp, c_vp, c_vp]
        L.spgemm_transpose_noalloc.restype = st
        L.spgemm_transpose_noalloc.argtypes = L.spgemm_transpose.argtypes
        _lib = L
    return _lib


def _check(status, plan=None):
    if status != 0:
        L = lib()
        msg = (L.spgemm_last_error(plan) or b"").decode()
        raise SpgemmError(status, f"{L.spgemm_status_string(status).decode()}: {msg}")


def compute_params(ncols, lds_bytes, val_bytes=8, col_bytes=4, max_chunks_per_level=0,
                   dense_width=0) -> dict:
    """GetMagnusParams on the host (no GPU needed)."""
    p = Params()
    _check(lib().spgemm_compute_params(ncols, lds_bytes, val_bytes, col_bytes,
                                       max_chunks_per_level, dense_width, ctypes.byref(p)))
    return p.as_dict()


@dataclass
class CsrDevice:
    """A CSR matrix in device memory (torch tensors): int32 row_ptr/col."""
    row_ptr: "object"
    col: "object"
    val: "object"
    m: int
    n: int

    @property
    def nnz(self) -> int:
        return int(self.col.numel())


def to_device(A, device="cuda"):
    """synth.CSR (numpy) -> CsrDevice."""
    import torch
    return CsrDevice(torch.from_numpy(A.row_ptr.astype("int32")).to(device),
                     torch.from_numpy(A.col.astype("int32")).to(device),
                     torch.from_numpy(A.val).to(device), A.m, A.n)


def _as_csr(X):
    if isinstance(X, CsrDevice):
        return X
    import torch
    if isinstance(X, torch.Tensor) and X.layout == torch.sparse_csr:
        return CsrDevice(X.crow_indices().to(torch.int32), X.col_indices().to(torch.int32),
                         X.values(), X.shape[0], X.shape[1])
    raise TypeError("expected CsrDevice or a torch sparse CSR tensor")


def _make_options(**kw) -> Options:
    o = Options()
    for k, v in kw.items():
        if v is None:
            continue
        if not hasattr(o, k):
            raise TypeError(f"unknown option {k}")
        setattr(o, k, int(v))
    return o


class Plan:
    """One C = A*B: plan -> symbolic -> numeric, then destroy (or `with`)."""

    def __init__(self, A, B, stream=None, **options):
        import torch
        A, B = _as_csr(A), _as_csr(B)
        if A.n != B.m:
            raise ValueError("inner dimensions differ")
        for X in (A, B):
            if X.row_ptr.dtype != torch.int32 or X.col.dtype != torch.int32:
                raise TypeError("row_ptr and col must be int32")
            if not (X.row_ptr.is_cuda and X.col.is_cuda and X.val.is_cuda):
                raise TypeError("CSR arrays must be device tensors")
            if not (X.row_ptr.is_contiguous() and X.col.is_contiguous() and X.val.is_contiguous()):
                raise TypeError("CSR arrays must be contiguous")
        if A.val.dtype != B.val.dtype or A.val.dtype not in (torch.float32, torch.float64):
            raise TypeError("values must be both float32 or both float64")
        self.A, self.B = A, B            # borrowed until destroy
        self.dtype = A.val.dtype
        self.rowptr64 = bool(options.get("rowptr64", 0))
        self.stream = torch.cuda.current_stream() if stream is None else stream
        self._opts = _make_options(**options)
        h = c_vp()
        dt = SPGEMM_F64 if self.dtype == torch.float64 else SPGEMM_F32
        _check(lib().spgemm_plan(ctypes.byref(h), A.m, A.n, B.n, A.row_ptr.data_ptr(),
                                 A.col.data_ptr(), A.val.data_ptr(), A.nnz, B.row_ptr.data_ptr(),
                                 B.col.data_ptr(), B.val.data_ptr(), B.nnz, dt,
                                 ctypes.byref(self._opts), c_vp(self.stream.cuda_stream)))
        self._h = h
        self.m, self.n = A.m, B.n

    def symbolic(self, row_ptr=None):
        import torch
        if row_ptr is None:
            row_ptr = torch.empty(self.m + 1, dtype=torch.int64 if self.rowptr64 else torch.int32,
                                  device=self.A.col.device)
        nnz = c_i64()
        _check(lib().spgemm_symbolic(self._h, row_ptr.data_ptr(), ctypes.byref(nnz)), self._h)
        self.row_ptr = row_ptr
        self.nnz = nnz.value
        return row_ptr, nnz.value

    def numeric(self, col=None, val=None):
        import torch
        dev = self.A.col.device
        if col is None:
            col = torch.empty(max(self.nnz, 1), dtype=torch.int32, device=dev)[:self.nnz]
        if val is None:
            val = torch.empty(max(self.nnz, 1), dtype=self.dtype, device=dev)[:self.nnz]
        _check(lib().spgemm_numeric(self._h, col.data_ptr(), val.data_ptr()), self._h)
        self._numeric_done = True
        return col, val

    def wait(self):
        """Block until the plan's work is done; raise SpgemmError when a
        device-side capacity check tripped (C must not be used then)."""
        _check(lib().spgemm_wait(self._h), self._h)

    def row_estimates(self, with_estimates=True):
        """Light rows' reserved output slots (int64) and, with the HyperLogLog
        workflow, their estimates (float64); other rows 0.  After symbolic."""
        import torch
        cap = torch.zeros(self.m, dtype=torch.int64, device=self.A.col.device)
        est = torch.zeros(self.m, dtype=torch.float64, device=self.A.col.device) \
            if with_estimates else None
        _check(lib().spgemm_row_estimates(self._h, cap.data_ptr(),
                                          None if est is None else est.data_ptr()), self._h)
        return cap, est

    def stats(self) -> dict:
        s = Stats()
        _check(lib().spgemm_get_stats(self._h, ctypes.byref(s)), self._h)
        return s.as_dict()

    def destroy(self):
        if getattr(self, "_h", None):
            lib().spgemm_destroy(self._h)
            self._h = None

    def __enter__(self):
        return self

    def __exit__(self, exc_type, exc, tb):
        # Device-side checks of the asynchronous numeric phase surface here
        # (unless an exception is already on its way).
        try:
            if exc_type is None and getattr(self, "_numeric_done", False) and self._h:
                self.wait()
        finally:
            self.destroy()

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


_last_stats = None


def last_stats():
    return _last_stats


def matmul(A, B, with_stats: bool = False, **options):
    """C = A*B.  Returns (row_ptr, col, val) device tensors (and stats)."""
    global _last_stats
    with Plan(A, B, **options) as p:
        rp, _ = p.symbolic()
        col, val = p.numeric()
        st = p.stats() if with_stats else None
    _last_stats = st
    return (rp, col, val, st) if with_stats else (rp, col, val)


def _two_call(count_fn, fill_fn, row_ptr, col, val, m, n, threshold, out_rowptr64):
    import torch
    L = lib()
    rp64 = 1 if row_ptr.dtype == torch.int64 else 0
    dt = SPGEMM_F64 if val.dtype == torch.float64 else SPGEMM_F32
    orp = torch.empty(m + 1, dtype=torch.int64 if out_rowptr64 else torch.int32,
                      device=col.device)
    h = c_vp()
    nnz = c_i64()
    stream = torch.cuda.current_stream().cuda_stream
    _check(count_fn(ctypes.byref(h), m, n, row_ptr.data_ptr(), rp64, col.data_ptr(),
                    val.data_ptr(), dt, float(threshold), orp.data_ptr(),
                    1 if out_rowptr64 else 0, ctypes.byref(nnz), c_vp(stream)))
    try:
        ocol = torch.empty(max(nnz.value, 1), dtype=torch.int32, device=col.device)[:nnz.value]
        oval = torch.empty(max(nnz.value, 1), dtype=val.dtype, device=col.device)[:nnz.value]
        _check(fill_fn(h, ocol.data_ptr(), oval.data_ptr()))
    finally:
        L.spgemm_prune_destroy(h)
    return orp, ocol, oval


def mcl_inflate(row_ptr, col, val, m, n, threshold=0.002, out_rowptr64=False):
    """The rest of one Markov-clustering iteration after the expansion:
    normalise the columns, drop entries below the threshold, square the rest."""
    L = lib()
    return _two_call(L.spgemm_mcl_inflate_count, L.spgemm_mcl_inflate_fill, row_ptr, col, val,
                     m, n, threshold, out_rowptr64)


def mcl(A, iterations=10, threshold=0.002, **options):
    """Markov clustering: `iterations` times, C = A*A (expansion), then
    normalise, prune and square (mcl_inflate); C becomes the next A.
    Returns the final CsrDevice and the products of every expansion."""
    X = _as_csr(A)
    options = dict(options)
    options.setdefault("rowptr64", 1)   # C may hold more than 2^31 entries
    products = []
    for _ in range(iterations):
        with Plan(X, X, **options) as p:
            rp, _ = p.symbolic()
            col, val = p.numeric()
            products.append(p.stats()["products"])
        # The kept matrix is the next input, whose indices are int32.
        rp, col, val = mcl_inflate(rp, col, val, X.m, X.n, threshold, out_rowptr64=False)
        X = CsrDevice(rp, col, val, X.m, X.n)
    return X, products


def prune_colnorm(row_ptr, col, val, m, n, threshold=1e-4, out_rowptr64=False):
    """Markov-clustering prune (keep >= threshold) and column renormalisation."""
    import torch
    L = lib()
    rp64 = 1 if row_ptr.dtype == torch.int64 else 0
    dt = SPGEMM_F64 if val.dtype == torch.float64 else SPGEMM_F32
    orp = torch.empty(m + 1, dtype=torch.int64 if out_rowptr64 else torch.int32,
                      device=col.device)
    h = c_vp()
    nnz = c_i64()
    stream = torch.cuda.current_stream().cuda_stream
    _check(L.spgemm_prune_colnorm_count(ctypes.byref(h), m, n, row_ptr.data_ptr(), rp64,
                                        col.data_ptr(), val.data_ptr(), dt, float(threshold),
                                        orp.data_ptr(), 1 if out_rowptr64 else 0,
                                        ctypes.byref(nnz), c_vp(stream)))
    try:
        ocol = torch.empty(max(nnz.value, 1), dtype=torch.int32, device=col.device)[:nnz.value]
        oval = torch.empty(max(nnz.value, 1), dtype=val.dtype, device=col.device)[:nnz.value]
        _check(L.spgemm_prune_colnorm_fill(h, ocol.data_ptr(), oval.data_ptr()))
    finally:
        L.spgemm_prune_destroy(h)
    return orp, ocol, oval


def transpose(A, out_rowptr64=False, pattern_only=False, no_alloc=False):
    """A^T as a CsrDevice (n x m): rows list their columns in rising order,
    values copied unchanged (spgemm_transpose; with no_alloc, the entry point
    whose temporaries live in the library's fixed scratch array,
    spgemm_transpose_noalloc)."""
    import torch
    X = _as_csr(A)
    dev = X.col.device
    nnz = X.nnz
    rp64 = 1 if X.row_ptr.dtype == torch.int64 else 0
    vals = None if (pattern_only or X.val is None) else X.val
    vdt = torch.float64 if (vals is None or vals.dtype == torch.float64) else torch.float32
    dt = SPGEMM_F64 if vdt == torch.float64 else SPGEMM_F32
    trp = torch.empty(X.n + 1, dtype=torch.int64 if out_rowptr64 else torch.int32, device=dev)
    tcol = torch.empty(max(nnz, 1), dtype=torch.int32, device=dev)[:nnz]
    tval = None if vals is None else torch.empty(max(nnz, 1), dtype=vdt, device=dev)[:nnz]
    stream = torch.cuda.current_stream().cuda_stream
    fn = lib().spgemm_transpose_noalloc if no_alloc else lib().spgemm_transpose
    _check(fn(X.m, X.n, nnz, X.row_ptr.data_ptr(), rp64, X.col.data_ptr(),
                                  None if vals is None else vals.data_ptr(), dt, trp.data_ptr(),
                                  1 if out_rowptr64 else 0, tcol.data_ptr(),
                                  None if tval is None else tval.data_ptr(), c_vp(stream)))
    return CsrDevice(trp, tcol, tval, X.n, X.m)
