"""Host-side parameter selection (GetMagnusParams) against the gMAGNUS page.

The pins are the page's own printed chunk tuples (Tables V and VI, stored in
tests/golden/magnus_num_chunks.txt with their citation) and the closed-form
values that follow from the LDS size on gfx950.  No GPU is needed.
"""
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "magnus_num_chunks.txt")


@pytest.fixture(scope="module")
def sg():
    import spgemm_symbolic_row_amd as m
    m.lib()
    return m


def _parse(tok):
    if tok == "N/A":
        return None
    if ":" in tok:
        req, rest = tok.split(":")
        return int(req), [int(x) for x in rest.split(",")]
    return int(tok), [int(tok)]


def _rows():
    out = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        name, ncols, pvc, h200 = line.split()
        out.append((name, int(ncols), _parse(pvc), _parse(h200)))
    return out


@pytest.mark.parametrize("name,ncols,pvc,h200", _rows())
def test_tables_v_vi_chunk_tuples(sg, name, ncols, pvc, h200):
    """W = 4096 / n_chunksMax = 32 (PVC) and W = 8192 / 64 (H200) reproduce
    every printed tuple: ceiling to a power of two, quotient split."""
    for expect, W, nmax in ((pvc, 4096, 32), (h200, 8192, 64)):
        if expect is None:
            continue
        p = sg.compute_params(ncols, 65536, 8, 4, nmax, W)
        req, v = expect
        assert p["chunks_required"] == req, (name, W)
        assert p["v_chunks"] == v, (name, W)
        assert p["levels"] == len(v)
        assert int(np.prod(p["v_chunks"])) == req
        assert p["level_width"][-1] == W


def test_dense_width_from_lds(sg):
    # s_LM = 64 KiB and 114 KiB with 8-byte values give W = 4096 and 8192, the
    # widths that reproduce the tables on PVC and H200.
    assert sg.compute_params(1 << 20, 64 * 1024, 8)["dense_width"] == 4096
    assert sg.compute_params(1 << 20, 114 * 1024, 8)["dense_width"] == 8192


def test_gfx950_defaults(sg):
    lds = 160 * 1024
    p = sg.compute_params(262144, lds, 8)          # R-MAT scale 18, fp64
    assert p["tau"] == 6826 and p["n_dense"] == 20164 and p["dense_width"] == 16384
    assert p["chunks_required"] == 16 and p["v_chunks"] == [16] and p["level_width"] == [16384]
    p = sg.compute_params(1 << 20, lds, 8)         # R-MAT scale 20, fp64: two levels
    assert p["chunks_required"] == 64 and p["v_chunks"] == [32, 2]
    assert p["level_width"] == [32768, 16384]
    p = sg.compute_params(1000000, lds, 4)         # planted partition, fp32
    assert p["tau"] == 10240 and p["dense_width"] == 32768
    assert p["chunks_required"] == 32 and p["v_chunks"] == [32]
    p = sg.compute_params(4096, lds, 8)            # one W-wide chunk: no multisplit
    assert p["chunks_required"] == 1 and p["levels"] == 0
    p = sg.compute_params(1 << 20, 80 * 1024, 8)   # half the LDS per work group
    assert p["tau"] == 3413 and p["dense_width"] == 8192 and p["v_chunks"] == [32, 4]


def test_tau_eq4_reading(sg):
    # tau = s_LM / (alpha (s_col + s_val)), alpha = 2 (a hash of tau entries in
    # 2 tau slots fills the budget).
    for lds, vb in ((65536, 4), (116736, 4), (163840, 8), (163840, 4), (81920, 8)):
        assert sg.compute_params(1000, lds, vb)["tau"] == lds // (2 * (4 + vb))


def test_levels_eq7(sg):
    # n_levels = ceil(log2 n_req / log2 n_max); product of v = n_req; powers of 2
    for nreq_log in range(0, 16):
        for nmax_log in (1, 2, 3, 5, 6):
            ncols = (1 << nreq_log) * 1024
            L = -(-nreq_log // nmax_log)
            if L > 8:   # more levels than the parameter record holds
                with pytest.raises(sg.SpgemmError):
                    sg.compute_params(ncols, 65536, 8, 4, 1 << nmax_log, 1024)
                continue
            p = sg.compute_params(ncols, 65536, 8, 4, 1 << nmax_log, 1024)
            assert p["chunks_required"] == 1 << nreq_log
            if nreq_log == 0:
                assert p["levels"] == 0
                continue
            assert p["levels"] == L
            assert all(v & (v - 1) == 0 for v in p["v_chunks"])
            assert int(np.prod(p["v_chunks"])) == 1 << nreq_log
            assert all(v == 1 << nmax_log for v in p["v_chunks"][:-1])


def test_invalid_arguments(sg):
    with pytest.raises(sg.SpgemmError):
        sg.compute_params(100, 0, 8)
    with pytest.raises(sg.SpgemmError):
        sg.compute_params(100, 65536, 8, 4, 3)      # n_chunksMax not a power of two
    with pytest.raises(sg.SpgemmError):
        sg.compute_params(100, 65536, 8, 4, 32, 1000)  # W not a power of two
