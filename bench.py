"""Throughput of C = A*A on one MI355X, with the roofline of the dominant
kernel and the CPU oracle timed beside it.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config rmat20]

A step is one whole product: plan + symbolic + allocation of C + numeric
(+ prune/renormalise for the Markov-clustering workload), inputs resident in
HBM.  The metric is GFLOP/s with flops = 2 x intermediate products.  Prints
one JSON line on stdout; diagnostics go to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0

WORKLOADS = {
    "rmat18": "R-MAT scale 18 (262,144 rows), edge factor 16, (a,b,c,d)=(0.57,0.19,0.19,0.05), "
              "duplicates merged, fp64 U[0,1], seed 0; C = A*A",
    "rmat20": "R-MAT scale 20 (1,048,576 rows), edge factor 16, same (a,b,c,d), fp64; C = A*A",
    "lap27_64": "27-point Laplacian on a 64^3 grid, fp64; C = A*A",
    "er4096": "Erdos-Renyi 4096x4096, Poisson(8) per row, fp64 U[-1,1], seed 0; C = A*A",
    "mcl1m": "planted partition 1000x1000, 28 intra + 4 inter + self per column, fp32 "
             "column-stochastic; C = A*A, prune < 1e-4, renormalise columns",
    "mcl_iter": "planted partition 100x1000, 28 intra + 4 inter + self per column, fp32 "
                "column-stochastic; 10 Markov-clustering iterations (C = A*A, normalise "
                "columns, prune < 0.002, square; C is the next A)",
    "aat": "rectangular R-MAT 2^17 x 2^20, 16 edges per row, same (a,b,c,d), fp64 U[0,1], "
           "seed 0; C = A*A^T with A^T formed on the GPU inside the step",
    "restrict": "R-MAT scale 18 as rmat18 times an aggregation operator R (2^18 x 2^15, "
                "random aggregates of 8, ones, seed 1); C = A*R",
}

# matrices of each configuration: A, and B when it is not A (or A^T)
CONFIG_MATRICES = {"aat": ("rmat_rect", "transpose"), "restrict": ("rmat18", "agg_rmat18")}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(st, phase, sv, si=4):
    """Algorithmic bytes one step moves in the given phase, and the per-unit
    figure they are built from.  The units are the effective-byte model's:
    s_i + s_v per heavy product written by an expansion (a 4-byte column and
    the value, whatever width the build stores), s_i + s_v per element read by
    a chunk accumulator.  Only expansions that write values count; a
    columns-only pass is extra work of the build's batched schedule."""
    E = sum(st["level_elems"])
    if phase == "expand_split":
        return st["level_elems"][0] * (si + sv), f"{si + sv} B written per heavy product (first-level chunks)"
    if phase == "outer_product":
        return st["heavy_products"] * (si + sv), f"{si + sv} B written per heavy product"
    if phase == "expand_final":
        return (st["heavy_products"] * (si + sv),
                f"{si + sv} B (4 B column + {sv} B value) written per heavy product (final chunks)")
    if phase == "multisplit":
        return E * 2 * (si + sv), f"{2 * (si + sv)} B (read + write) per element per level"
    if phase == "histogram":
        return E * si, f"{si} B read per element per level"
    if phase == "num_chunk_dense":
        return st["lds_dense_products"] * (si + sv), f"{si + sv} B read per dense-chunk element"
    if phase == "num_chunk_hash":
        return ((st["heavy_products"] - st["lds_dense_products"]) * (si + sv),
                f"{si + sv} B read per light-chunk element")
    if phase == "sym_chunk_dense":
        return st["lds_dense_products"] * si, f"{si} B read per dense-chunk element"
    if phase == "num_light":
        return ((st["products"] - st["heavy_products"]) * (si + sv),
                f"{si + sv} B of B read per light-row product")
    return None, None


S_LM = 160 * 1024   # LDS per work group on gfx950 (the default s_LM)


def frozen_heavy(A, B, sv):
    """Heavy products P_h and the elements entering each multisplit level
    E_l at the default parameters (a row is heavy iff P_i > tau; a chunk
    recurses iff it holds more than tau elements), computed on the host from
    the structure of A and B alone, so that no option of the run can move
    the effective-byte denominator.  Counts per (row, chunk) are the rows of
    A's pattern times per-row chunk histograms of B."""
    import numpy as np
    import scipy.sparse as ssp

    import spgemm_symbolic_row_amd as sg

    prm = sg.compute_params(B.n, S_LM, sv)
    tau = prm["tau"]
    arp = A.row_ptr.astype(np.int64)
    lenB = np.diff(B.row_ptr.astype(np.int64))
    rowA = np.repeat(np.arange(A.m), np.diff(arp))
    P = np.bincount(rowA, weights=lenB[A.col].astype(np.float64), minlength=A.m)
    P = np.rint(P).astype(np.int64)
    heavy = np.nonzero(P > tau)[0]
    Ph = int(P[heavy].sum())
    E = []
    if prm["levels"] > 0 and heavy.size:
        E.append(Ph)
        lens = arp[heavy + 1] - arp[heavy]
        hrp = np.zeros(heavy.size + 1, np.int64)
        np.cumsum(lens, out=hrp[1:])
        idx = np.repeat(arp[heavy] - hrp[:-1], lens) + np.arange(int(hrp[-1]))
        Ah = ssp.csr_matrix((np.ones(idx.size, np.int64), A.col[idx], hrp),
                            shape=(heavy.size, B.m))
        rowB = np.repeat(np.arange(B.m), lenB)
        for w in prm["level_width"][:-1]:
            nch = (B.n + w - 1) // w
            H = ssp.csr_matrix((np.ones(B.nnz, np.int64), (rowB, B.col // w)),
                               shape=(B.m, nch))
            cnt = (Ah @ H).data
            E.append(int(cnt[cnt > tau].sum()))
    return {"tau": tau, "heavy_rows": int(heavy.size), "heavy_products": Ph,
            "level_elems": E, "v_chunks": prm["v_chunks"]}


def effective_bytes(A, fz, nnzC, sv, si=4, B=None, transposed=False, rp64=False,
                    prune_nnz=None):
    """Effective-byte denominator of one step: compulsory traffic (symbolic
    reads the structure of A and B and writes C.row_ptr; numeric reads A, B
    and C.row_ptr and writes C.col and C.val) plus what the method
    materialises when it expands once, with values: P_h (s_i + s_v) for the
    expansion, sum_l E_l (3 s_i + 2 s_v) for the histogram read and the
    multisplit read and write of every level, P_h (2 s_i + s_v) for the
    chunk symbolic read and the numeric read.  P_h and E_l come frozen from
    frozen_heavy().  B defaults to A; with `transposed`, B = A^T is formed
    inside the step (A read once, A^T written once).  prune_nnz: the Markov
    clustering step's kept entries; its prune reads C, writes the kept
    entries, reads them again and writes their renormalised values."""
    m, nnzA = A.m, A.nnz
    rp, rpc = 4, (8 if rp64 else 4)
    kB, nnzB = (A.n, A.nnz) if transposed else ((A.m, A.nnz) if B is None else (B.m, B.nnz))
    sym = (m + 1) * rp + nnzA * si + (kB + 1) * rp + nnzB * si + (m + 1) * rpc
    num = ((m + 1) * rp + nnzA * (si + sv) + (kB + 1) * rp + nnzB * (si + sv) + (m + 1) * rpc
           + nnzC * (si + sv))
    if transposed:
        num += (m + 1) * rp + (A.n + 1) * rp + 2 * nnzA * (si + sv)
    Ph, E = fz["heavy_products"], sum(fz["level_elems"])
    heavy = Ph * (si + sv) + E * (3 * si + 2 * sv) + Ph * (2 * si + sv)
    prune = 0
    if prune_nnz is not None:
        prune = ((m + 1) * rpc + nnzC * (si + sv) + (m + 1) * 4 + prune_nnz * (si + sv)
                 + prune_nnz * (si + sv) + prune_nnz * sv)
    return sym + num + heavy + prune


def copy_bandwidth(gib=4.0, reps=5):
    """Device-to-device copy rate on this GPU (bytes read + written per
    second, GB/s), the measured ceiling beside the nominal HBM peak."""
    import torch
    n = int(gib * 2 ** 30) // 8
    src = torch.ones(n, dtype=torch.float64, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    torch.cuda.empty_cache()
    return round(2 * n * 8 / (ms / 1e3) / 1e9, 1)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def traffic_for(kernel, workload):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current sources (the kernel's, and the host code that
    decides which elements it moves: the SHA-256 of their contents in the
    listed order); else None."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    srcs = rec.get("sources") or [rec["source"]]
    h = hashlib.sha256()
    for src in srcs:
        h.update(open(os.path.join(ROOT, src), "rb").read())
    if h.hexdigest() != rec["source_sha256"]:
        return None
    return rec["bytes_per_launch"]


MCL_ITERS, MCL_THRESHOLD = 10, 0.002


def run_mcl_iter(args, A, opts):
    """Markov clustering: a step is the whole run of MCL_ITERS iterations;
    GFLOP/s counts 2 x the products of every expansion."""
    import numpy as np
    import torch

    import spgemm_symbolic_row_amd as sg

    dA = sg.to_device(A)
    opts = {k: v for k, v in opts.items() if k != "profile"}

    def step():
        return sg.mcl(dA, iterations=MCL_ITERS, threshold=MCL_THRESHOLD, **opts)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        X, prods = step()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    K = args.steps
    P = int(sum(prods))
    value = 2.0 * P * K / dt / 1e9
    log(f"{dt / K * 1e3:.3f} ms/step, {value:.2f} GFLOP/s; products per iteration {prods}; "
        f"final nnz {int(X.col.numel())}")
    line = {
        "metric": "SpGEMM GFLOP/s (2x intermediate products) + % HBM roofline, 1 MI355X",
        "value": round(value, 3), "unit": "GFLOP/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(dt / K * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": WORKLOADS[args.config], "rows": A.m, "nnz_a": A.nnz,
                   "iterations": MCL_ITERS, "threshold": MCL_THRESHOLD,
                   "products_per_iteration": [int(x) for x in prods], "products": P,
                   "final_nnz": int(X.col.numel()), "parallelism": "single GPU"},
        "roofline": None,
        "cpu_baseline": None,
    }
    del dA, X
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        import oracle
        threads = int(os.environ.get("OMP_NUM_THREADS", 0)) or os.cpu_count()
        B = A
        t0 = time.perf_counter()
        Pc = 0
        for _ in range(MCL_ITERS):
            Pc += int(oracle.row_products(B, B).sum())
            C = oracle.spgemm(B, B)
            rp, col, val = oracle.mcl_inflate(B.m, B.n, C.row_ptr, C.col, C.val, MCL_THRESHOLD)
            B = synth_csr(rp, col, val.astype(np.float32), A.m, A.n)
        t = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": round(2 * Pc / t / 1e9, 4), "unit": "GFLOP/s",
                                "cores": threads, "kind": "oracle", "cpu_model": cpu_model(),
                                "sample": f"the whole {MCL_ITERS}-iteration run once, {t:.2f} s"}
        log(f"cpu baseline: {line['cpu_baseline']}")
    print(json.dumps(line), flush=True)


def synth_csr(rp, col, val, m, n):
    import numpy as np

    import synth
    return synth.CSR(rp.astype(np.int32), col.astype(np.int32), val, m, n)


def cpu_baseline(A, target_s=15.0, B=None, note=""):
    """The oracle (as it stands) on the same matrices (B defaults to A): a
    uniform random sample of rows of A sized to about target_s seconds, or,
    when the whole product takes less than that, the whole product repeated."""
    import numpy as np

    import oracle
    import synth

    rng = np.random.default_rng(0)

    def sub(frac):
        rows = np.sort(rng.choice(A.m, max(1, int(A.m * frac)), replace=False))
        rp = A.row_ptr.astype(np.int64)
        lens = rp[rows + 1] - rp[rows]
        nrp = np.zeros(rows.size + 1, np.int64)
        np.cumsum(lens, out=nrp[1:])
        idx = np.repeat(rp[rows] - nrp[:-1], lens) + np.arange(int(nrp[-1]))
        return synth.CSR(nrp.astype(np.int32), A.col[idx], A.val[idx], rows.size, A.n), rows.size

    B = A if B is None else B

    def timed(S):
        t0 = time.perf_counter()
        oracle.spgemm(S, B)
        return time.perf_counter() - t0

    P_all = int(oracle.row_products(A, B).sum())
    S, _ = sub(0.02)
    P0 = int(oracle.row_products(S, B).sum())
    rate = P0 / max(timed(S), 1e-6)
    est_full = P_all / max(rate, 1.0)
    threads = int(os.environ.get("OMP_NUM_THREADS", 0)) or os.cpu_count()
    if est_full >= target_s:
        S, nrows = sub(target_s / est_full)
        P = int(oracle.row_products(S, B).sum())
        t = timed(S)
        sample = (f"{nrows} of {A.m} rows chosen uniformly at random (seed 0), "
                  f"{P} intermediate products, {t:.2f} s")
    else:
        runs = max(1, min(10, int(np.ceil(target_s / max(est_full, 1e-3)))))
        t = sum(timed(A) for _ in range(runs))
        P = P_all * runs
        sample = f"the whole product (all {A.m} rows, {P_all} products) run {runs} times, {t:.2f} s"
    return {"value": round(2 * P / t / 1e9, 4), "unit": "GFLOP/s", "cores": threads,
            "kind": "oracle", "sample": sample + note, "cpu_model": cpu_model(),
            "host_threads": os.cpu_count()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="rmat20", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-copy-rate", action="store_true",
                    help="skip the device-copy bandwidth measurement")
    ap.add_argument("--no-profile", action="store_true",
                    help="do not time kernel phases with HIP events")
    ap.add_argument("--single-stream", action="store_true",
                    help="run light and heavy work on one stream (diagnostics)")
    ap.add_argument("--copy-calibration-gib", type=float, default=0.0,
                    help="first run one device-to-device copy of this many GiB, so "
                         "hardware byte counters can be scaled against a known size")
    ap.add_argument("--dense-width", type=int, default=0, help="override W (tuning)")
    ap.add_argument("--max-chunks", type=int, default=0,
                    help="override the chunks per multisplit level (tuning)")
    ap.add_argument("--lds-budget", type=int, default=0, help="override s_LM (tuning)")
    ap.add_argument("--heavy-threshold", type=int, default=0, help="override tau (tuning)")
    ap.add_argument("--heavy-row-threshold", type=int, default=0,
                    help="override the light/heavy row split (tuning)")
    ap.add_argument("--mem-budget", type=int, default=0,
                    help="bytes for the heavy intermediate (tuning; 0 = the library's)")
    ap.add_argument("--workflow", type=int, default=-1,
                    help="light-row size prediction: 0 symbolic, 1 upper bound, 2 HyperLogLog, "
                         "3 Table 1 choice (default: the library's)")
    ap.add_argument("--light-no-esc", action="store_true",
                    help="short rows by the LDS hash kernels instead of ESC (diagnostics)")
    ap.add_argument("--dense-direct", action="store_true",
                    help="dense chunks accumulated straight from A and B (diagnostics)")
    ap.add_argument("--light-hash-only", action="store_true",
                    help="no dense windows for light rows (diagnostics)")
    ap.add_argument("--expansion", type=int, default=-1,
                    help="heavy-row expansion: 0 straight into final chunks, 1 outer product + "
                         "multisplit, 2 first level fed from A and B (default: the library's)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library is a single-GPU SpGEMM; run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import spgemm_symbolic_row_amd as sg

    if not torch.cuda.is_available():
        raise RuntimeError("bench.py needs a GPU")
    torch.cuda.set_device(0)
    if args.copy_calibration_gib > 0:
        nbytes = int(args.copy_calibration_gib * 2 ** 30)
        src = torch.ones(nbytes // 8, dtype=torch.float64, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: {nbytes} bytes read and {nbytes} bytes written")
        del src, dst
    t = time.time()
    a_name, b_name = CONFIG_MATRICES.get(args.config, (args.config, None))
    A = synth.workload(a_name)
    transposed = b_name == "transpose"
    B = synth.workload(b_name) if b_name and not transposed else None
    log(f"generated {args.config}: {A.m} x {A.n}, nnz {A.nnz}"
        + (f"; B {B.m} x {B.n}, nnz {B.nnz}" if B is not None else "")
        + f" in {time.time() - t:.1f} s")
    dA = sg.to_device(A)
    dB = sg.to_device(B) if B is not None else None
    f64 = A.val.dtype == np.float64
    sv = 8 if f64 else 4
    opts = {} if args.no_profile else {"profile": 1}
    if args.single_stream:
        opts["single_stream"] = 1
    if args.dense_width:
        opts["dense_width"] = args.dense_width
    if args.max_chunks:
        opts["max_chunks_per_level"] = args.max_chunks
    if args.lds_budget:
        opts["lds_budget"] = args.lds_budget
    if args.heavy_threshold:
        opts["heavy_threshold"] = args.heavy_threshold
    if args.heavy_row_threshold:
        opts["heavy_row_threshold"] = args.heavy_row_threshold
    if args.mem_budget:
        opts["mem_budget"] = args.mem_budget
    if args.expansion >= 0:
        opts["expansion"] = args.expansion
    if args.light_hash_only:
        opts["light_hash_only"] = 1
    if args.dense_direct:
        opts["dense_direct"] = 1
    if args.workflow >= 0:
        opts["workflow"] = args.workflow
    if args.light_no_esc:
        opts["light_no_esc"] = 1
    if args.config == "rmat20":
        opts["rowptr64"] = 1   # nnz(C) is about 9.7e9
    if args.config == "mcl_iter":
        return run_mcl_iter(args, A, opts)
    mcl = args.config == "mcl1m"

    def step():
        dR = dB if dB is not None else (sg.transpose(dA) if transposed else dA)
        with sg.Plan(dA, dR, **opts) as p:
            rp, _ = p.symbolic()
            col, val = p.numeric()
            out = (rp, col, val)
            if mcl:
                out = sg.prune_colnorm(rp, col, val, A.m, A.n, 1e-4)
            st = p.stats()
        if mcl:
            st["pruned_nnz"] = int(out[1].numel())
        return out, st

    for _ in range(args.warmup):
        _, st = step()
    torch.cuda.synchronize()
    phase_tot, phase_min = {}, {}
    t0 = time.perf_counter()
    for _ in range(args.steps):
        _, st = step()
        for k, v in st["phase_ms"].items():
            phase_tot[k] = phase_tot.get(k, 0.0) + v
            w = st["phase_min_ms"][k]
            if w > 0:
                phase_min[k] = min(phase_min.get(k, w), w)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    K = args.steps
    P = st["products"]
    value = 2.0 * P * K / dt / 1e9
    ms = dt / K * 1e3
    t = time.time()
    if transposed:
        import scipy.sparse as ssp
        T = ssp.csr_matrix((A.val, A.col, A.row_ptr), shape=(A.m, A.n)).T.tocsr()
        T.sort_indices()
        Bh = synth.CSR(T.indptr.astype(np.int32), T.indices.astype(np.int32), T.data, A.n, A.m)
    else:
        Bh = B if B is not None else A
    fz = frozen_heavy(A, Bh, sv)
    log(f"frozen heavy figures at the default parameters: {fz} ({time.time() - t:.1f} s)")
    eff = effective_bytes(A, fz, st["nnz_c"], sv, B=B, transposed=transposed,
                          rp64=bool(opts.get("rowptr64")), prune_nnz=st.get("pruned_nnz"))
    log(f"{ms:.3f} ms/step, {value:.2f} GFLOP/s, effective {eff / (dt / K) / 1e9:.1f} GB/s")
    for k, v in sorted(phase_tot.items(), key=lambda kv: -kv[1]):
        if v > 0:
            log(f"  {k:18s} {v / K:9.3f} ms/step  windows/step {st['phase_windows'][k]}")

    roof = None
    if not args.no_profile:
        cands = [k for k in ("multisplit", "expand_split", "outer_product", "expand_final",
                             "num_chunk_dense", "histogram")
                 if phase_tot.get(k, 0) > 0]
        if not cands and phase_tot.get("num_light", 0) > 0:
            cands = ["num_light"]
        if cands:
            kern = max(cands, key=lambda k: phase_tot[k])
            windows = st["phase_windows"][kern]
            avg_ms = phase_tot[kern] / (windows * K)
            step_bytes, unit_desc = algorithmic_bytes(st, kern, sv)
            byt = step_bytes / windows
            achieved = byt / (avg_ms / 1e3) / 1e9
            roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                    "traffic": traffic_for(kern, args.config), "kernel": kern,
                    "avg_launch_ms": round(avg_ms, 4), "bytes_per_launch": int(byt),
                    "per_unit": unit_desc}
            if kern in phase_min:
                # The shortest launch (with several heavy batches the first
                # one runs beside the heavy-row slot counts and takes longer;
                # the batches differ in size, so no rate is derived from it).
                roof["min_launch_ms"] = round(phase_min[kern], 4)
            # The other heavy kernels with an algorithmic byte count, as the
            # pages report a fraction of speed of light per core kernel.
            others = []
            # (The histogram phase is left out: by default it derives the
            # level counts from the structure and reads no element.)
            for k in ("expand_final", "num_chunk_dense", "num_chunk_hash", "sym_chunk_dense",
                      "multisplit", "expand_split", "outer_product"):
                if k == kern or phase_tot.get(k, 0) <= 0:
                    continue
                kb, kunit = algorithmic_bytes(st, k, sv)
                if not kb:
                    continue
                kw = st["phase_windows"][k]
                kms = phase_tot[k] / (kw * K)
                others.append({"kernel": k, "avg_launch_ms": round(kms, 4),
                               "bytes_per_launch": int(kb / kw),
                               "frac": round(kb / kw / (kms / 1e3) / 1e9 / HBM_PEAK_GBPS, 4),
                               "per_unit": kunit})
            if others:
                roof["other_kernels"] = others
            if not args.no_copy_rate:
                roof["copy_gbps"] = copy_bandwidth()
                roof["frac_of_copy"] = round(achieved / roof["copy_gbps"], 4)
                log(f"device copy {roof['copy_gbps']} GB/s (read + write)")

    line = {
        "metric": "SpGEMM GFLOP/s (2x intermediate products) + % HBM roofline, 1 MI355X",
        "value": round(value, 3), "unit": "GFLOP/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f64" if f64 else "f32",
        "data": "synthetic",
        "config": {"workload": WORKLOADS[args.config], "rows": A.m, "cols": A.n, "nnz_a": A.nnz,
                   "products": P, "nnz_c": st["nnz_c"], "heavy_rows": st["heavy_rows"],
                   "heavy_products": st["heavy_products"],
                   "v_chunks": st["params"]["v_chunks"], "tau": st["params"]["tau"],
                   "batches": st["batches"],
                   "frozen_heavy_products": fz["heavy_products"],
                   "frozen_level_elems": fz["level_elems"],
                   "effective_bytes": int(eff),
                   "effective_gbps": round(eff / (dt / K) / 1e9, 1),
                   "effective_frac": round(eff / (dt / K) / 1e9 / HBM_PEAK_GBPS, 4),
                   "parallelism": "single GPU"},
        "roofline": roof,
        "cpu_baseline": None,
    }
    if transposed:
        # the transpose inside the step, timed on its own
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(5):
            sg.transpose(dA)
        torch.cuda.synchronize()
        line["config"]["transpose_ms"] = round((time.perf_counter() - t0) / 5 * 1e3, 4)
        log(f"transpose alone: {line['config']['transpose_ms']} ms")
    del dA, dB
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        note = ""
        if transposed:
            import oracle
            t0 = time.perf_counter()
            T = oracle.transpose(A)
            tt = time.perf_counter() - t0
            B = synth.CSR(T.row_ptr.astype(np.int32), T.col, T.val, T.m, T.n)
            note = f"; A^T formed by the oracle beforehand in {tt:.2f} s, not counted"
        line["cpu_baseline"] = cpu_baseline(A, B=B, note=note)
        log(f"cpu baseline: {line['cpu_baseline']}")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
