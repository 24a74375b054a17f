"""Host-side checks of the integer logic the kernels rely on: the tile order
and persistent grid ("B200 GEMM Optimization Ladder", section E step 7),
the LDS swizzles against the fragment-read pattern ("B200 TMA Pipeline
Designer", section B: a swizzle that does not match the matrix-core read
pattern is a failure mode), the epilogue staging pitch and the rule that
spreads direct loads over matrix-core instructions.

The functions are the ones in csrc/sched.hpp, compiled for the host with
g++ into a throw-away shared library; no GPU is involved."""
import ctypes
import os
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SCHED = os.path.join(ROOT, "matrix_core_engineering_amd", "csrc", "sched.hpp")

SHIM = r'''
#include "%s"
extern "C" {
int h_xcd_major(int wg, int nwg) { return mce::xcd_major(wg, nwg); }
void h_grouped_tile(int id, int tm_, int tn_, int g, int *tm, int *tn)
{ mce::grouped_tile(id, tm_, tn_, g, *tm, *tn); }
int h_persistent_tile_id(int wg, int nwg, int r) { return mce::persistent_tile_id(wg, nwg, r); }
int h_swz8(int r) { return mce::swz8(r); }
int h_swz4(int r) { return mce::swz4(r); }
int h_swz4g(int r) { return mce::swz4g(r); }
int h_loads_after(int x, int n, int l) { return mce::loads_after(x, n, l) ? 1 : 0; }
}
'''


@pytest.fixture(scope="module")
def lib(tmp_path_factory):
    d = tmp_path_factory.mktemp("hostlogic")
    src = d / "shim.cpp"
    src.write_text(SHIM % SCHED)
    so = d / "libshim.so"
    subprocess.run(["g++", "-O1", "-std=c++17", "-shared", "-fPIC", str(src), "-o", str(so)],
                   check=True)
    lib = ctypes.CDLL(str(so))
    lib.h_grouped_tile.argtypes = [ctypes.c_int] * 4 + [ctypes.POINTER(ctypes.c_int)] * 2
    return lib


def grouped(lib, i, tm_, tn_, g):
    a, b = ctypes.c_int(), ctypes.c_int()
    lib.h_grouped_tile(i, tm_, tn_, g, ctypes.byref(a), ctypes.byref(b))
    return a.value, b.value


@pytest.mark.parametrize("nwg", [1, 7, 8, 9, 63, 64, 100, 255, 256, 257, 1000, 1024])
def test_xcd_major_bijection_and_xcd_blocks(lib, nwg):
    pos = [lib.h_xcd_major(w, nwg) for w in range(nwg)]
    assert sorted(pos) == list(range(nwg))
    # workgroups dispatched to one XCD (same id mod 8) get consecutive positions
    for x in range(8):
        mine = sorted(lib.h_xcd_major(w, nwg) for w in range(x, nwg, 8))
        assert mine == list(range(mine[0], mine[0] + len(mine))) if mine else True


@pytest.mark.parametrize("tm_,tn_,g", [(1, 1, 1), (32, 32, 8), (16, 16, 8), (17, 33, 8), (5, 3, 8),
                                       (9, 4, 4), (32, 24, 8), (3, 40, 3)])
def test_grouped_tile_bijection(lib, tm_, tn_, g):
    seen = set()
    for i in range(tm_ * tn_):
        a, b = grouped(lib, i, tm_, tn_, min(g, tm_))
        assert 0 <= a < tm_ and 0 <= b < tn_
        seen.add((a, b))
    assert len(seen) == tm_ * tn_


@pytest.mark.parametrize("ntiles,ncu", [(1024, 256), (256, 256), (561, 256), (17, 256), (1000, 255)])
def test_persistent_grid_covers_every_tile_once(lib, ntiles, ncu):
    """The kernels' own count: workgroup wg at position first = xcd_major(wg)
    runs tiles r*nwg + first for r < my_tiles."""
    nwg = min(ntiles, ncu)
    hits = np.zeros(ntiles, dtype=int)
    for wg in range(nwg):
        first = lib.h_xcd_major(wg, nwg)
        my = (ntiles - 1 - first) // nwg + 1 if first < ntiles else 0
        for r in range(my):
            t = lib.h_persistent_tile_id(wg, nwg, r)
            assert 0 <= t < ntiles
            hits[t] += 1
    assert (hits == 1).all()


def slots(rows, logical_chunk, swz, row_bytes):
    """16-byte bank slots (64 banks x 4 bytes = 16 slots) that a ds_read_b128
    of logical chunk `logical_chunk` touches for each row."""
    return [((r * row_bytes) // 16 + (logical_chunk ^ swz(r))) % 16 for r in rows]


@pytest.mark.parametrize("base", [0, 32, 64, 96, 128, 160, 192, 224])
def test_swz8_fragment_reads_conflict_free(lib, base):
    """128-byte rows: a 16-lane pass of a fragment read takes rows
    base + 16p .. +15 at one logical chunk; its 16 slots must differ."""
    for chunk in range(8):
        for p in range(2):
            rows = range(base + 16 * p, base + 16 * p + 16)
            s = slots(rows, chunk, lib.h_swz8, 128)
            assert len(set(s)) == 16, (chunk, p, s)


@pytest.mark.parametrize("base", [0, 32, 64, 96])
def test_swz4_fragment_reads_conflict_free(lib, base):
    """64-byte rows (level 7): four rows share the 16 slots, so a 16-lane
    pass over 16 rows needs each group of four rows that map to the same
    slots to use four different chunks."""
    for chunk in range(4):
        for p in range(2):
            rows = list(range(base + 16 * p, base + 16 * p + 16))
            s = slots(rows, chunk, lib.h_swz4, 64)
            counts = np.bincount(s, minlength=16)
            assert counts.max() == 1, (chunk, p, s)


@pytest.mark.parametrize("base", [0, 32, 64, 96])
def test_swz4g_fragment_reads_conflict_free(lib, base):
    """Register-staged kernel, 64-byte rows: same 16-lane read pattern."""
    for chunk in range(4):
        for p in range(2):
            rows = list(range(base + 16 * p, base + 16 * p + 16))
            counts = np.bincount(slots(rows, chunk, lib.h_swz4g, 64), minlength=16)
            assert counts.max() == 1, (chunk, p)


def test_swizzles_are_permutations_per_row(lib):
    for r in range(512):
        assert sorted(c ^ lib.h_swz8(r) for c in range(8)) == list(range(8))
        assert sorted(c ^ lib.h_swz4(r) for c in range(4)) == list(range(4))
        assert sorted(c ^ lib.h_swz4g(r) for c in range(4)) == list(range(4))


@pytest.mark.parametrize("e", range(8))
@pytest.mark.parametrize("kchunk", range(4))
def test_swz4g_spreads_transposed_write_rows(lib, e, kchunk):
    """MN-major operands are written transposed: the 16 lanes that share a
    K pair write rows 8c + e, c = 0..15, at one logical chunk; swz4g puts
    them in four different physical chunks (swz4 in only two)."""
    phys = {kchunk ^ lib.h_swz4g(8 * c + e) for c in range(16)}
    assert len(phys) == 4
    assert len({kchunk ^ lib.h_swz4(8 * c + e) for c in range(16)}) == 2


def test_epilogue_staging_pitch_spreads_banks():
    """Staged epilogue: lane (l32, h) writes 8 bytes at row l32, byte
    jj*64 + q*16 + 8h of a 144-byte-pitch buffer; for every (jj, q) the 64
    lanes' writes cover each 4-byte bank exactly twice."""
    pitch = 144
    for jj in range(2):
        for q in range(4):
            banks = np.zeros(64, dtype=int)
            for lane in range(64):
                l32, h = lane % 32, lane // 32
                addr = l32 * pitch + jj * 64 + q * 16 + h * 8
                for w in range(2):
                    banks[(addr // 4 + w) % 64] += 1
            assert (banks == 2).all(), (jj, q, banks)


@pytest.mark.parametrize("n,l", [(32, 16), (32, 11), (16, 4), (12, 12), (10, 8), (4, 2), (7, 0), (16, 9)])
def test_loads_after_spreads_evenly(lib, n, l):
    marks = [lib.h_loads_after(x, n, l) for x in range(n)]
    assert sum(marks) == l
    pos = [x for x in range(n) if marks[x]]
    if l > 1:
        gaps = np.diff(pos)
        assert gaps.min() >= n // l and gaps.max() <= -(-n // l)
